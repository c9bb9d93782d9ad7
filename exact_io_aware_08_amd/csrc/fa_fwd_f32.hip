// fa_fwd_f32.hip -- forward attention with fp32 inputs on fp32 MFMA (gfx950),
// and its E4M3 "P-cast" variant.
//
// Same tiling and online recurrence as the bf16/fp16 kernel (marketmaker.cc
// blog "Atencion flash y la pregunta sobre la longitud de la secuencia",
// sections "El algoritmo de atencion flash", "La recurrencia de softmax en
// linea", "FA2: paralelismo", "El enmascaramiento causal ..."), with
// v_mfma_f32_32x32x2f32.  That instruction takes one value per lane per
// operand, so both K and V are staged row-major in LDS and no transpose is
// needed: for S^T = K Q^T the K-slot of lane group g in step t is
// d = t + (D/2) g (contiguous per lane, so Q loads are vectorised); for
// O^T = V^T P^T the K-slot of lane group g in step (i, r) is key
// 8i + 4g + r, which is exactly the S^T accumulator register 4i + r.
//
// P-cast (gist.science "Resumen Tecnico: Precision de P-Cast en la Atencion
// FP8", sections "Planteamiento del Problema", "Optimizacion 1",
// "Optimizacion 2"): per tile, P = exp(s - m) relative to the running max m,
// the running sum l adds the uncast P, and P~ = E4M3_RNE(S * P) (hardware
// v_cvt_pk_fp8_f32, OCP E4M3FN on gfx950) is converted back exactly to fp32
// for the P~ V product; the epilogue divides by S * l (exact for S = 2^k).
// The KV tiles are visited in increasing or decreasing key order.  Q, K, V
// stay fp32 ("Contribuciones Clave", item 4), so the cast is the only
// reduced-precision step.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

constexpr int NW = 4;
constexpr int BR = NW * 32;

template <int D> struct F32Tile { static constexpr int BC = (D == 128) ? 32 : 64; };

__device__ __forceinline__ f32x16_t mma_f32(float a, float b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ unsigned wave_sum_u32(unsigned x)
{
    // integer sum over the wave: any order gives the same result
    const int i = wave_scan_i32((int)x);  // inclusive prefix sum, the total in lane 63
    return (unsigned)__builtin_amdgcn_readlane(i, 63);
}

// Input elements widen exactly to fp32 on load (TI = float or __bf16, the
// latter for the P-cast path on bf16 operands); O is written in TI.
template <typename TI> struct Wide;
template <> struct Wide<float> {
    static constexpr int PER = 4;  // elements per 16-byte load
    static __device__ __forceinline__ void get(const float *p, float (&x)[4])
    {
        const f32x4_t v = *reinterpret_cast<const f32x4_t *>(p);
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    }
};
template <> struct Wide<__bf16> {
    static constexpr int PER = 8;
    static __device__ __forceinline__ void get(const __bf16 *p, float (&x)[8])
    {
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // bf16 -> fp32 is a 16-bit shift, exact
            x[2 * i] = __uint_as_float(v[i] << 16);
            x[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
        }
    }
};

template <typename TI, int D, bool CAUSAL, bool PCAST>
__global__ void __launch_bounds__(256)
fwd_f32_kernel(const TI *__restrict__ Q, const TI *__restrict__ K,
               const TI *__restrict__ V, TI *__restrict__ O, float *__restrict__ LSE,
               int H, int Hkv, int Nq, int Nk, int n_bh, int n_qtiles, float scale,
               float scale_log2, float p_scale, int kv_flags, int n_sink,
               unsigned long long *__restrict__ counts)
{
    constexpr int BC = F32Tile<D>::BC;
    constexpr int NKB = BC / 32;          // 32-key blocks per tile
    constexpr int KSTR = D + 1;           // odd stride: column reads hit 32 banks
    constexpr int VSTR = D;
    constexpr int PER = Wide<TI>::PER;    // elements per 16-byte chunk
    constexpr int CPR = D / PER;          // chunks per row
    constexpr int CH = BC * CPR / 256;    // chunks per thread per tensor
    static_assert(CH * 256 == BC * CPR, "tile split");

    __shared__ float Ks[BC * KSTR];
    __shared__ __attribute__((aligned(16))) float Vs[BC * VSTR];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, c = lane & 31, hh = lane >> 5;

    const int qt = n_qtiles - 1 - (int)(blockIdx.x / (unsigned)n_bh);
    const int bh = (int)(blockIdx.x % (unsigned)n_bh);
    const int b = bh / H, h = bh - b * H;
    const int hk = h / (H / Hkv);
    const size_t qoff = (size_t)bh * Nq * D;
    const size_t kvoff = ((size_t)b * Hkv + hk) * Nk * D;
    const TI *Qb = Q + qoff;
    const TI *Kb = K + kvoff;
    const TI *Vb = V + kvoff;
    TI *Ob = O + qoff;

    const int q0 = qt * BR;
    const int q0w = q0 + w * 32;
    const int off = Nk - Nq;
    int nkt = (Nk + BC - 1) / BC;
    if (CAUSAL) {
        const int lim = min(q0 + BR, Nq) - 1 + off;
        nkt = lim < 0 ? 0 : min(nkt, lim / BC + 1);
    }
    const int row = q0w + c;
    const int row_lim = (row < Nq) ? (CAUSAL ? min(Nk, row + off + 1) : Nk) : 0;
    const int sink_end = ((n_sink + BC - 1) / BC) * BC;

    // Q operand: lane (c, hh) holds Q[row][t + (D/2) hh] for t = 0 .. D/2-1
    // (rows past Nq load the last row; their results are never stored).
    float qop[D / 2];
    const int qrow = min(row, Nq - 1);
#pragma unroll
    for (int t = 0; t < D / 2 / PER; ++t) {
        float x[PER];
        Wide<TI>::get(Qb + (size_t)qrow * D + (D / 2) * hh + PER * t, x);
#pragma unroll
        for (int e = 0; e < PER; ++e) qop[PER * t + e] = x[e];
    }

    f32x16_t acc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc[i] = f32x16_t{};
    float m_run = -INFINITY, l_run = 0.f;
    unsigned cnt[4] = {0u, 0u, 0u, 0u};

    // Keys past Nk load row Nk-1 (masked to weight 0).
    float kreg[CH][PER], vreg[CH][PER];
    auto load_tile = [&](int j) {
        const int j0 = j * BC;
#pragma unroll
        for (int r = 0; r < CH; ++r) {
            const int ci = tid + r * 256;
            const int key = min(j0 + ci / CPR, Nk - 1), cc = ci % CPR;
            Wide<TI>::get(Kb + (size_t)key * D + PER * cc, kreg[r]);
            Wide<TI>::get(Vb + (size_t)key * D + PER * cc, vreg[r]);
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int r = 0; r < CH; ++r) {
            const int ci = tid + r * 256;
            const int kl = ci / CPR, cc = ci % CPR;
            float *kp = &Ks[kl * KSTR + PER * cc];
#pragma unroll
            for (int e = 0; e < PER; ++e) kp[e] = kreg[r][e];
#pragma unroll
            for (int e = 0; e < PER; e += 4)
                *reinterpret_cast<f32x4_t *>(&Vs[kl * VSTR + PER * cc + e]) =
                    f32x4_t{vreg[r][e], vreg[r][e + 1], vreg[r][e + 2], vreg[r][e + 3]};
        }
    };

    const bool kv_reverse = (kv_flags & 1) != 0;  // bit 0: KV tiles in reverse order
    const bool tile_local = (kv_flags & 2) != 0;  // bit 1: tile-local max (P-cast ablation)
    auto tile_at = [&](int jj) { return kv_reverse ? (nkt - 1 - jj) : jj; };
    if (nkt > 0) load_tile(tile_at(0));
    for (int jj = 0; jj < nkt; ++jj) {
        const int j = tile_at(jj);
        __syncthreads();
        store_tile();
        __syncthreads();
        if (jj + 1 < nkt) load_tile(tile_at(jj + 1));
        const int j0 = j * BC;
        if (CAUSAL && j0 > q0w + 31 + off) continue;

        f32x16_t s[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            s[kb] = f32x16_t{};
#pragma unroll
            for (int t = 0; t < D / 2; ++t)
                s[kb] = mma_f32(Ks[(kb * 32 + c) * KSTR + t + (D / 2) * hh], qop[t], s[kb]);
        }

        const bool need_mask = (j0 + BC > Nk) || (CAUSAL && j0 + BC - 1 > q0w + off);
        if (need_mask) {
            const int lim = CAUSAL ? min(Nk, row + off + 1) : Nk;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = j0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if (key >= lim) s[kb][r] = -INFINITY;
                }
        }

        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = max_xor32(mx);
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2((m_run - m_use) * scale_log2);
        // P relative to the running max; in the tile-local ablation (P-cast
        // only) relative to this tile's own max, its weight restored by
        // beta = exp(m_tile - m_new) after the cast
        const bool local = PCAST && tile_local;
        const float m_ref = local ? ((mx == -INFINITY) ? 0.f : mx) : m_use;
        const float beta = local ? ((mx == -INFINITY) ? 0.f : fast_exp2((m_ref - m_use) * scale_log2)) : 1.f;
        const float mneg = -m_ref * scale_log2;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(fmaf(s[kb][r], scale_log2, mneg));
                s[kb][r] = p;
                rs += p;
            }
        l_run = l_run * alpha + (local ? rs * beta : rs);
        m_run = m_new;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) acc[i] *= alpha;

        if (PCAST) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const float p0 = s[kb][r], p1 = s[kb][r + 1];
                    const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(p0 * p_scale, p1 * p_scale, 0, false);
                    const float t0 = __builtin_amdgcn_cvt_f32_fp8(pk, 0);
                    const float t1 = __builtin_amdgcn_cvt_f32_fp8(pk, 1);
                    s[kb][r] = local ? t0 * beta : t0;
                    s[kb][r + 1] = local ? t1 * beta : t1;
                    const int key0 = j0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                    const int key1 = key0 + 1;
                    const unsigned f0 = (t0 == 0.f && p0 > 0.f), f1 = (t1 == 0.f && p1 > 0.f);
                    if (key0 < row_lim) {
                        if (key0 >= n_sink) { cnt[0] += 1; cnt[1] += f0; }
                        if (key0 >= sink_end) { cnt[2] += 1; cnt[3] += f0; }
                    }
                    if (key1 < row_lim) {
                        if (key1 >= n_sink) { cnt[0] += 1; cnt[1] += f1; }
                        if (key1 >= sink_end) { cnt[2] += 1; cnt[3] += f1; }
                    }
                }
        }

        // O^T += V^T P^T : K-slot of lane group hh in step (i, r) is key 8i + 4hh + r
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kl = kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                    acc[mb] = mma_f32(Vs[kl * VSTR + 32 * mb + c], s[kb][r], acc[mb]);
                }
    }

    const float l = sum_xor32(l_run);
    if (row < Nq) {
        const float den = PCAST ? p_scale * l : l;
        const float inv = l > 0.f ? 1.f / den : 0.f;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = 32 * mb + 8 * i + 4 * hh;
                typedef TI t4 __attribute__((ext_vector_type(4)));
                const t4 vals = t4{static_cast<TI>(acc[mb][4 * i] * inv), static_cast<TI>(acc[mb][4 * i + 1] * inv),
                                   static_cast<TI>(acc[mb][4 * i + 2] * inv), static_cast<TI>(acc[mb][4 * i + 3] * inv)};
                *reinterpret_cast<t4 *>(Ob + (size_t)row * D + d0) = vals;
            }
        if (LSE != nullptr && hh == 0)
            LSE[(size_t)bh * Nq + row] = l > 0.f ? m_run * scale + logf(l) : -INFINITY;
    }

    if (PCAST && counts != nullptr) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const unsigned tot = wave_sum_u32(cnt[i]);
            if (lane == 0 && tot) atomicAdd(counts + i, (unsigned long long)tot);
        }
    }
}

template <typename TI, int D, bool CAUSAL, bool PCAST>
hipError_t launch_t(const FwdProblem &p, hipStream_t st)
{
    const int n_qtiles = (p.Nq + BR - 1) / BR;
    const int n_bh = p.B * p.H;
    const dim3 grid((unsigned)n_qtiles * (unsigned)n_bh), block(256);
    hipLaunchKernelGGL((fwd_f32_kernel<TI, D, CAUSAL, PCAST>), grid, block, 0, st,
                       static_cast<const TI *>(p.q), static_cast<const TI *>(p.k),
                       static_cast<const TI *>(p.v), static_cast<TI *>(p.o), p.lse, p.H,
                       p.Hkv, p.Nq, p.Nk, n_bh, n_qtiles, p.scale, p.scale * kLog2e, p.p_scale,
                       p.kv_reverse, p.n_sink, p.counts);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdProblem &p, hipStream_t st)
{
    if (p.pcast && p.dtype == 2)  // P-cast on bf16 operands
        return p.causal ? launch_t<__bf16, D, true, true>(p, st) : launch_t<__bf16, D, false, true>(p, st);
    if (p.pcast)
        return p.causal ? launch_t<float, D, true, true>(p, st) : launch_t<float, D, false, true>(p, st);
    return p.causal ? launch_t<float, D, true, false>(p, st) : launch_t<float, D, false, false>(p, st);
}

__global__ void cast_e4m3_kernel(const float *__restrict__ x, uint8_t *__restrict__ codes,
                                 float *__restrict__ back, size_t n)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(x[i], 0.f, 0, false);
    if (codes) codes[i] = (uint8_t)(pk & 0xFF);
    if (back) back[i] = __builtin_amdgcn_cvt_f32_fp8(pk, 0);
}

}  // namespace

int fwd_f32_kv_tile(int d) { return d == 128 ? F32Tile<128>::BC : F32Tile<64>::BC; }

hipError_t launch_fwd_f32(const FwdProblem &p, hipStream_t st)
{
    return p.d == 64 ? launch_d<64>(p, st) : launch_d<128>(p, st);
}

hipError_t launch_cast_e4m3(const float *x, uint8_t *codes, float *back, size_t n,
                            hipStream_t st)
{
    if (n == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL(cast_e4m3_kernel, dim3(blocks), dim3(256), 0, st, x, codes, back, n);
    return hipGetLastError();
}

}  // namespace fa
