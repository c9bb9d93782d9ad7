// bench_ceilings.hip -- attainable ceilings on gfx950 for the bench line's
// two rooflines, measured on the same machine as the kernels they judge.
// Built in-tree into libfa_ceilings.so; only bench.py loads it.  Nothing here
// is part of the attention path.
//
// The roofline argument of marketmaker.cc "Atencion flash y la pregunta sobre
// la longitud de la secuencia", section "Por que la atencion esta ligada a la
// memoria": a kernel is bounded by bytes moved or by arithmetic.  The nominal
// peaks (8 TB/s HBM3E, 2.5 PFLOP/s dense bf16 at 2.4 GHz) are the primary
// denominators; these kernels measure what one launch on this chip actually
// reaches for the same access pattern or instruction mix:
//
//  * ceil_read_chunks: every workgroup sums one contiguous chunk with 16-byte
//    loads -- the split-KV decode's access pattern (one slice per workgroup).
//  * ceil_read_stride: grid-stride 16-byte loads over the whole buffer.
//  * ceil_mfma: back-to-back v_mfma_f32_32x32x16_bf16 on register operands
//    (4 independent accumulators), the dense-MFMA rate at the sustained clock.
//  * ceil_mfma_mix: the prefill's per-tile instruction mix with operands in
//    registers -- 16 MFMAs against 32 FMA, 32 exp2, 32 adds and 16 bf16 pair
//    conversions per wave, interleaved the way the prefill kernel does -- with
//    no LDS staging, barriers, masking or causal tail: what that mix allows;
//    its variants take VALU work out or move it to the MFMA pipe.
// Every kernel stores one value per thread (or per workgroup) derived from all
// of its work, so none of it is dead.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kReadThreads = 256;

// Workgroup g sums bytes [g * chunk, min((g + 1) * chunk, n)) of x; every
// thread keeps U loads of 16 bytes in flight per round.
template <int U>
__global__ void __launch_bounds__(kReadThreads)
ceil_read_chunks(const u32x4_t *__restrict__ x, long long n16, long long chunk16,
                 uint32_t *__restrict__ out)
{
    const long long beg = (long long)blockIdx.x * chunk16;
    const long long end = beg + chunk16 < n16 ? beg + chunk16 : n16;
    u32x4_t acc = {0u, 0u, 0u, 0u};
    long long i = beg + threadIdx.x;
    for (; i + (U - 1) * kReadThreads < end; i += U * kReadThreads) {
        u32x4_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(&x[i + u * kReadThreads]);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u] + (uint32_t)u;
    }
    for (; i < end; i += kReadThreads) acc += x[i];
    out[(size_t)blockIdx.x * kReadThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// Grid-stride sum of all of x, U loads in flight per thread and round.
template <int U>
__global__ void __launch_bounds__(kReadThreads)
ceil_read_stride(const u32x4_t *__restrict__ x, long long n16, uint32_t *__restrict__ out)
{
    const long long stride = (long long)gridDim.x * kReadThreads;
    u32x4_t acc = {0u, 0u, 0u, 0u};
    long long i = (long long)blockIdx.x * kReadThreads + threadIdx.x;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u32x4_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(&x[i + u * stride]);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u] + (uint32_t)u;
    }
    for (; i < n16; i += stride) acc += x[i];
    out[(size_t)blockIdx.x * kReadThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

__device__ __forceinline__ bf16x8_t seed_op(float s)
{
    bf16x8_t v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (__bf16)(s * (float)(e + 1) * 0.01f);
    return v;
}

// `iters` rounds of 16 MFMAs (32x32x16 bf16) per wave on 4 independent
// accumulators.  FLOP per wave per round: 16 * 2 * 32 * 32 * 16.
__global__ void __launch_bounds__(256)
ceil_mfma(int iters, float *__restrict__ out)
{
    const float s = (float)(threadIdx.x & 63) * 0.015625f;
    bf16x8_t a = seed_op(s), b = seed_op(1.f - s);
    f32x16_t acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x16_t{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 16; ++k)
            acc[k & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k & 3], 0, 0, 0);
        asm volatile("" : "+v"(a));  // keep the rounds from being folded together
    }
    float r = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) r += acc[i][e];
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = r;
}

// The prefill's per-tile mix, `iters` tiles per wave (rounded up to even):
// 8 MFMAs producing the next tile's scores and 8 accumulating P V of the
// previous tile, while the VALU turns the current scores (two 32x32 blocks,
// 32 values per lane) into exp2(s * c + m) with their row sums and packs them
// to bf16 pairs that feed the next tile's P V.  Unrolled by two so the score
// registers swap roles instead of being copied, as in the prefill kernel.
//
// The template flags give the trade-off variants (the default, all of FMA and
// ADD and neither extra, is the ceiling):
//   FMA  -- the scale-and-shift FMA before each exp2; without it the scores
//           arrive shifted (the accumulator starts from a per-lane -m) and
//           unscaled, i.e. the VALU work left if the scale were folded into Q;
//   ADD  -- the row sums as fp32 adds on the VALU;
//   XQK  -- 8 more score MFMAs: the cost of folding the scale into Q exactly,
//           as a bf16 hi/lo split of the scaled Q (twice the score products);
//   XSUM -- 4 more MFMAs that take the row sums from the packed P with an
//           all-ones operand, in place of the VALU adds.
template <bool FMA, bool ADD, bool XQK, bool XSUM>
__global__ void __launch_bounds__(256, 2)
ceil_mfma_mix(int iters, float c, float *__restrict__ out)
{
    const float s0 = (float)(threadIdx.x & 63) * 0.015625f;
    bf16x8_t kop = seed_op(s0);
    const bf16x8_t qop[2] = {seed_op(1.f - s0), seed_op(0.75f - s0)};  // two query blocks
    const bf16x8_t qlo[2] = {seed_op(0.01f - 0.001f * s0), seed_op(0.02f - 0.001f * s0)};
    const bf16x8_t vop = seed_op(0.5f * s0);
    const bf16x8_t ones = seed_op(100.f);
    f32x16_t sa[2], sb[2], acc[4], lsum[2];
    bf16x8_t p[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        sa[i] = f32x16_t{};
        lsum[i] = f32x16_t{};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x16_t{};
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t) p[i][t] = qop[i];
    float rowsum[2] = {0.f, 0.f};
    const float mneg = -0.25f;
    // score accumulator start: 0, or a per-lane -m when the FMA is left out
    f32x16_t cinit;
#pragma unroll
    for (int e = 0; e < 16; ++e) cinit[e] = FMA ? 0.f : mneg + 0.001f * s0;
    constexpr int NM = 16 + (XQK ? 8 : 0) + (XSUM ? 4 : 0);  // MFMAs per step
    constexpr int NV = (FMA ? 32 : 0) + 32 + (ADD ? 32 : 0) + 16;  // VALU per step
    auto step = [&](const f32x16_t (&sc)[2], f32x16_t (&sn)[2]) {
        asm volatile("" : "+v"(kop));  // a new K tile every step (not loop-invariant)
        // 8 MFMAs (16 with XQK): next scores (2 query blocks x 4 K-steps)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            sn[qb] = cinit;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                sn[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[qb], sn[qb], 0, 0, 0);
                if (XQK) sn[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qlo[qb], sn[qb], 0, 0, 0);
            }
        }
        // 8 MFMAs: P V of the previous tile (2 d-blocks x 2 K-steps x 2 query blocks)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
                    acc[2 * qb + mb] =
                        __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, p[qb][t], acc[2 * qb + mb], 0, 0, 0);
        if (XSUM) {  // 4 MFMAs: row sums of the previous tile's packed P
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
                    lsum[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, p[qb][t], lsum[qb], 0, 0, 0);
        }
        // softmax of the current scores: 32 FMA + 32 exp2 + 32 adds + 16 converts
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float a0 = sc[qb][8 * t + 2 * e], a1 = sc[qb][8 * t + 2 * e + 1];
                    if (FMA) {
                        a0 = fmaf(a0, c, mneg);
                        a1 = fmaf(a1, c, mneg);
                    }
                    const float x0 = __builtin_amdgcn_exp2f(a0);
                    const float x1 = __builtin_amdgcn_exp2f(a1);
                    if (ADD) rowsum[qb] = rowsum[qb] + x0 + x1;
                    const bf16x2_t pk = __builtin_convertvector((f32x2_t{x0, x1}), bf16x2_t);
                    w[e] = __builtin_bit_cast(uint32_t, pk);
                }
                p[qb][t] = __builtin_bit_cast(bf16x8_t, (u32x4_t{w[0], w[1], w[2], w[3]}));
            }
        __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
#pragma unroll
        for (int i = 0; i < NM - 1; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x0002, NV / (NM - 1), 0);
            __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
        }
    };
    for (int it = 0; it < iters; it += 2) {
        step(sa, sb);
        step(sb, sa);
    }
    float r = rowsum[0] + rowsum[1];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) r += acc[i][e] + sa[i & 1][e] + lsum[i & 1][e];
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = r;
}

}  // namespace

// Host entry points (ctypes; stream = hipStream_t as void*).  Return the
// hipError_t of the launch.  `out` needs grid * 256 elements; `unroll` is 8
// or 16 loads in flight per thread.
extern "C" {

int ceil_read_chunks_launch(const void *x, long long bytes, int grid, int unroll, void *out,
                            void *stream)
{
    const long long n16 = bytes / 16;
    const long long chunk16 = (n16 + grid - 1) / grid;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const u32x4_t *xp = static_cast<const u32x4_t *>(x);
    uint32_t *o = static_cast<uint32_t *>(out);
    if (unroll == 16)
        hipLaunchKernelGGL(ceil_read_chunks<16>, dim3(grid), dim3(kReadThreads), 0, st, xp, n16, chunk16, o);
    else
        hipLaunchKernelGGL(ceil_read_chunks<8>, dim3(grid), dim3(kReadThreads), 0, st, xp, n16, chunk16, o);
    return (int)hipGetLastError();
}

int ceil_read_stride_launch(const void *x, long long bytes, int grid, int unroll, void *out,
                            void *stream)
{
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const u32x4_t *xp = static_cast<const u32x4_t *>(x);
    uint32_t *o = static_cast<uint32_t *>(out);
    if (unroll == 16)
        hipLaunchKernelGGL(ceil_read_stride<16>, dim3(grid), dim3(kReadThreads), 0, st, xp, bytes / 16, o);
    else
        hipLaunchKernelGGL(ceil_read_stride<8>, dim3(grid), dim3(kReadThreads), 0, st, xp, bytes / 16, o);
    return (int)hipGetLastError();
}

int ceil_mfma_launch(int iters, int grid, void *out, void *stream)
{
    hipLaunchKernelGGL(ceil_mfma, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       iters, static_cast<float *>(out));
    return (int)hipGetLastError();
}

int ceil_mfma_mix_launch(int iters, int grid, void *out, void *stream)
{
    hipLaunchKernelGGL((ceil_mfma_mix<true, true, false, false>), dim3(grid), dim3(256), 0,
                       static_cast<hipStream_t>(stream), iters, 0.125f * 1.4426950408889634f,
                       static_cast<float *>(out));
    return (int)hipGetLastError();
}

// The trade-off variants of the mix (0 is the ceiling itself):
// 0 as the prefill; 1 no FMA; 2 no row-sum adds; 3 exp2 and converts only;
// 4 no FMA, scores from a hi/lo split of the scaled Q (24 MFMAs);
// 5 row sums on the MFMA pipe instead of the VALU (20 MFMAs).
// Returns hipErrorInvalidValue (1) for another variant.
int ceil_mfma_mix_variant_launch(int variant, int iters, int grid, void *out, void *stream)
{
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const float c = 0.125f * 1.4426950408889634f;
    float *o = static_cast<float *>(out);
    switch (variant) {
    case 0: hipLaunchKernelGGL((ceil_mfma_mix<true, true, false, false>), dim3(grid), dim3(256), 0, st, iters, c, o); break;
    case 1: hipLaunchKernelGGL((ceil_mfma_mix<false, true, false, false>), dim3(grid), dim3(256), 0, st, iters, c, o); break;
    case 2: hipLaunchKernelGGL((ceil_mfma_mix<true, false, false, false>), dim3(grid), dim3(256), 0, st, iters, c, o); break;
    case 3: hipLaunchKernelGGL((ceil_mfma_mix<false, false, false, false>), dim3(grid), dim3(256), 0, st, iters, c, o); break;
    case 4: hipLaunchKernelGGL((ceil_mfma_mix<false, true, true, false>), dim3(grid), dim3(256), 0, st, iters, c, o); break;
    case 5: hipLaunchKernelGGL((ceil_mfma_mix<true, false, false, true>), dim3(grid), dim3(256), 0, st, iters, c, o); break;
    default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

}  // extern "C"
