// fa_quant.hip -- E4M3 quantisation of Q, K or V for the FP8 attention path,
// with optional incoherent processing (a random-sign Hadamard rotation before
// the block-wise quantisation; "FA3: Mecanica de la tolva", item 3, of the
// flash-attention post on marketmaker.cc).
//
// Definition (the same the oracle states):
//   y     = H_d (s o x) when signs are given, else x; H_d is the Sylvester-
//           Hadamard matrix, formed by the fast transform in fp32 in stages
//           h = 1, 2, ..., d/2, each replacing (y_j, y_{j+h}) (j mod 2h < h)
//           by (y_j + y_{j+h}, y_j - y_{j+h});
//   group = 32 consecutive rows of one (b, h)          (layout 0), or
//           one column of one (b, h) over all rows      (layout 1), or
//           the whole tensor                            (whole != 0);
//   scale = 2^e, e the smallest integer >= -126 with amax(|y| over the
//           group) <= 448 * 2^e;
//   code  = E4M3_RNE(y * 2^-e), the hardware v_cvt_pk_fp8_f32 (OCP E4M3FN).
//
// One lane owns one row: it holds the row in fp32 registers, so the
// transform needs no data exchange and follows the stated order exactly.
// Row-block groups (layout 0, not whole) are reduced inside each 32-lane half
// of a wave, one pass.  The other groups need a maximum over rows: the
// scales array first collects the group maxima (as float bits, by atomic
// max), a second pass writes the codes, and a last pass turns the maxima into
// scales.  All passes read the input; HBM-bound.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

template <typename T> __device__ __forceinline__ float widen(T x) { return static_cast<float>(x); }

// Row i of slice bh into y[0..D) (fp32), with the sign flip and the transform.
template <typename T, int D>
__device__ __forceinline__ void load_row(const T *__restrict__ x, const float *__restrict__ signs,
                                         size_t row, float (&y)[D])
{
    constexpr int PER = 16 / sizeof(T);
    const u32x4_t *src = reinterpret_cast<const u32x4_t *>(x + row * D);
#pragma unroll
    for (int v = 0; v < D / PER; ++v) {
        const u32x4_t w = src[v];
        const T *e = reinterpret_cast<const T *>(&w);
#pragma unroll
        for (int t = 0; t < PER; ++t) y[v * PER + t] = widen(e[t]);
    }
    if (signs != nullptr) {
#pragma unroll
        for (int c = 0; c < D; ++c) y[c] *= signs[c];
#pragma unroll
        for (int h = 1; h < D; h *= 2)
#pragma unroll
            for (int j = 0; j < D; ++j)
                if ((j % (2 * h)) < h) {
                    const float a = y[j], b = y[j + h];
                    y[j] = a + b;
                    y[j + h] = a - b;
                }
    }
}

// Exponent of the group scale from the group maximum (see the definition).
__device__ __forceinline__ int scale_exp(float amax)
{
    const uint32_t u = __float_as_uint(amax);
    const int E = (int)(u >> 23) - 127;          // amax in [2^E, 2^(E+1)) for normal amax
    if (!(amax >= 0x1p-118f)) return -126;       // zero, subnormal or tiny: 2^-126 always fits
    const uint32_t mant = u & 0x7FFFFF;          // amax = (1 + mant/2^23) 2^E
    return (mant <= 0x600000u) ? E - 8 : E - 7;  // 1.75 * 2^8 = 448
}

__device__ __forceinline__ float pow2(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

template <int D>
__device__ __forceinline__ void store_codes(uint8_t *__restrict__ codes, size_t row, const float (&y)[D],
                                            const float (&inv)[D])
{
    u32x4_t *dst = reinterpret_cast<u32x4_t *>(codes + row * D);
#pragma unroll
    for (int v = 0; v < D / 16; ++v) {
        u32x4_t w;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = 16 * v + 4 * q;
            int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[c] * inv[c], y[c + 1] * inv[c + 1], 0, false);
            pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[c + 2] * inv[c + 2], y[c + 3] * inv[c + 3], pk, true);
            w[q] = (uint32_t)pk;
        }
        dst[v] = w;
    }
}

__device__ __forceinline__ float half_max(float v)
{
    // maximum over the 32-lane half of the wave this lane belongs to
    auto mx = [](float a, int b) { return fmaxf(a, __int_as_float(b)); };
    v = mx(v, dpp_mov<kDppXor1>(__float_as_int(v)));
    v = mx(v, dpp_mov<kDppXor2>(__float_as_int(v)));
    v = mx(v, dpp_mov<kDppHalfMirror>(__float_as_int(v)));
    v = mx(v, dpp_mov<kDppMirror>(__float_as_int(v)));
    return max_xor16(v);
}

// Grid (ceil(nblk / 8), B*H); each wave covers two 32-row blocks.
template <typename T, int D>
__global__ void __launch_bounds__(256)
quant_rows_kernel(const T *__restrict__ x, const float *__restrict__ signs, uint8_t *__restrict__ codes,
                  float *__restrict__ scales, int N, int nblk, int mode)
{
    // mode 0: block-local scales (written here); 1: read the group maximum
    // from scales (layout 0, whole tensor: slot 0 of the tensor); 2: read the
    // per-column maxima from scales [bh][D] (layout 1).
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int blk = 8 * blockIdx.x + 2 * w + (lane >> 5);
    const int bh = blockIdx.y;
    const int i = 32 * blk + (lane & 31);
    const bool live = blk < nblk && i < N;
    const size_t row = (size_t)bh * N + i;
    float y[D];
    if (live) load_row<T, D>(x, signs, row, y);
    else {
#pragma unroll
        for (int c = 0; c < D; ++c) y[c] = 0.f;
    }
    float inv[D];
    if (mode == 0) {
        float m = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) m = fmaxf(m, fabsf(y[c]));
        m = half_max(m);
        const int e = scale_exp(m);
#pragma unroll
        for (int c = 0; c < D; ++c) inv[c] = pow2(-e);
        if ((lane & 31) == 0 && blk < nblk) scales[(size_t)bh * nblk + blk] = pow2(e);
    } else if (mode == 1) {
        const int e = scale_exp(scales[0]);
#pragma unroll
        for (int c = 0; c < D; ++c) inv[c] = pow2(-e);
    } else {
#pragma unroll
        for (int c = 0; c < D; ++c) inv[c] = pow2(-scale_exp(scales[(size_t)bh * D + c]));
    }
    if (live) store_codes<D>(codes, row, y, inv);
}

// Group maxima by atomic max on the float bits (non-negative floats order as
// unsigned integers).  whole: one word (slot 0); else per column [bh][D].
template <typename T, int D>
__global__ void __launch_bounds__(256)
quant_amax_kernel(const T *__restrict__ x, const float *__restrict__ signs, float *__restrict__ amax,
                  int N, int nblk, int whole)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int blk = 8 * blockIdx.x + 2 * w + (lane >> 5);
    const int bh = blockIdx.y;
    const int i = 32 * blk + (lane & 31);
    float y[D];
    if (blk < nblk && i < N) load_row<T, D>(x, signs, (size_t)bh * N + i, y);
    else {
#pragma unroll
        for (int c = 0; c < D; ++c) y[c] = 0.f;
    }
    unsigned *bits = reinterpret_cast<unsigned *>(amax);
    if (whole) {
        float m = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) m = fmaxf(m, fabsf(y[c]));
        m = half_max(m);
        m = max_xor32(m);
        if (lane == 0) atomicMax(bits, __float_as_uint(m));
        return;
    }
    // per column: reduce each column over the wave, lane c (c < 64) keeps column c
    float mine[D / 64];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        float m = fabsf(y[c]);
        m = half_max(m);
        m = max_xor32(m);
        if ((c & 63) == lane) mine[c / 64] = m;
    }
#pragma unroll
    for (int t = 0; t < D / 64; ++t) atomicMax(bits + (size_t)bh * D + 64 * t + lane, __float_as_uint(mine[t]));
}

__global__ void zero_kernel(float *__restrict__ p, size_t n)
{
    for (size_t k = blockIdx.x * (size_t)blockDim.x + threadIdx.x; k < n; k += (size_t)gridDim.x * blockDim.x)
        p[k] = 0.f;
}

// Group maxima -> scales.  whole: one workgroup reads slot 0, then fills all
// n slots; per column: element-wise in place.
__global__ void finish_scales_kernel(float *__restrict__ s, size_t n, int whole)
{
    if (whole) {
        const float m = s[0];
        __syncthreads();
        const float sc = pow2(scale_exp(m));
        for (size_t k = threadIdx.x; k < n; k += blockDim.x) s[k] = sc;
        return;
    }
    for (size_t k = blockIdx.x * (size_t)blockDim.x + threadIdx.x; k < n; k += (size_t)gridDim.x * blockDim.x)
        s[k] = pow2(scale_exp(s[k]));
}

template <typename T, int D>
hipError_t launch_td(const QuantProblem &p, hipStream_t st)
{
    const T *x = static_cast<const T *>(p.x);
    const int nblk = (p.N + 31) / 32;
    const dim3 grid((unsigned)((nblk + 7) / 8), (unsigned)p.BH);
    if (p.layout == 0 && !p.whole) {
        hipLaunchKernelGGL((quant_rows_kernel<T, D>), grid, dim3(256), 0, st, x, p.signs, p.codes,
                           p.scales, p.N, nblk, 0);
        return hipGetLastError();
    }
    const size_t nsc = (size_t)p.BH * (p.layout == 0 ? nblk : D);
    const size_t nz = p.whole ? 1 : nsc;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((nz + 255) / 256 < 1024 ? (nz + 255) / 256 : 1024)),
                       dim3(256), 0, st, p.scales, nz);
    hipLaunchKernelGGL((quant_amax_kernel<T, D>), grid, dim3(256), 0, st, x, p.signs, p.scales, p.N,
                       nblk, p.whole);
    hipLaunchKernelGGL((quant_rows_kernel<T, D>), grid, dim3(256), 0, st, x, p.signs, p.codes,
                       p.scales, p.N, nblk, p.whole ? 1 : 2);
    if (p.whole)
        hipLaunchKernelGGL(finish_scales_kernel, dim3(1), dim3(1024), 0, st, p.scales, nsc, 1);
    else
        hipLaunchKernelGGL(finish_scales_kernel,
                           dim3((unsigned)((nsc + 255) / 256 < 1024 ? (nsc + 255) / 256 : 1024)),
                           dim3(256), 0, st, p.scales, nsc, 0);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const QuantProblem &p, hipStream_t st)
{
    return p.d == 64 ? launch_td<T, 64>(p, st) : launch_td<T, 128>(p, st);
}

}  // namespace

hipError_t launch_quant(const QuantProblem &p, hipStream_t st)
{
    if (p.dtype == 0) return launch_t<float>(p, st);
    if (p.dtype == 1) return launch_t<_Float16>(p, st);
    return launch_t<__bf16>(p, st);
}

}  // namespace fa
