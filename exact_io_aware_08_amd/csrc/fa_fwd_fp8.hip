// fa_fwd_fp8.hip -- forward attention with E4M3 Q, K, V and an E4M3 P, on the
// gfx950 FP8 matrix cores (v_mfma_f32_32x32x64_f8f6f4).
//
// Method: the online-softmax sweep of marketmaker.cc "El algoritmo de
// atencion flash" / "La recurrencia de softmax en linea" with FA2's deferred
// normalisation ("FA2: paralelismo"), run in FP8 as in "FA3: Mecanica de la
// tolva", item 3 (FP8 matrix products at twice the 16-bit rate; inputs
// quantised block-wise, optionally after a random rotation, by fa_quant).
// P is cast exactly as in gist.science "Resumen Tecnico: Precision de P-Cast
// en la Atencion FP8", "Planteamiento del Problema": P relative to the RUNNING
// maximum, multiplied by a static S, cast to E4M3, S divided out at the end;
// the row sum adds the uncast P; the KV tiles run forward or in reverse
// ("Optimizacion 1").
//
// Operands (all E4M3 codes with fp32 power-of-two scales):
//   q [B,H,Nq,d] with one scale per 32-row block, k [B,Hkv,Nk,d] likewise,
//   v [B,Hkv,Nk,d] with one scale per column.  A 32-row quantisation block
//   is exactly one MFMA row block, so the q and k scales fold into the
//   per-lane exponent factor (one multiply per tile); the v scales are
//   applied once per output element in the epilogue.
//
// gfx950 mapping (workgroup = 4 waves; a wave owns one block of 32 query
// rows; KV tiles of 64 keys, double-buffered in LDS, one barrier per tile):
//  * S^T = K Q^T on the FP8 MFMA: lane l, byte i of an operand carries
//    contraction index 32(l/32) + i (checked on the GPU), so K rows are read
//    from LDS as 32 contiguous bytes and Q stays in registers.
//  * The S^T accumulator of the two 32-key blocks gives lane (query l%32,
//    group g) the keys 32kb + 8(r/4) + 4g + r%4; converted to E4M3 in that
//    order it is directly the B operand of O^T = V^T P^T, with slot 8t + j
//    holding key 16t + 4g + j (j < 4) or 16t + 8 + 4g + (j - 4) (j >= 4).
//  * V is staged in LDS with bits 2 and 3 of the key index exchanged, so
//    those 8 keys are 8 consecutive rows, and the V^T operand comes from
//    four ds_read_b64_tr_b8 per 32 columns (within a 16-lane group, lane s
//    supplies row r0 + s/2, columns c0 + 8(s%2); lane i receives column
//    c0 + i of rows r0..r0+7; checked on the GPU).
//  * The running max is exact per tile (the cast depends on it); the
//    rescale of O^T is skipped when no row of the wave moved.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;

__device__ __forceinline__ f32x16_t mma_fp8(i32x8_t a, i32x8_t b, f32x16_t c)
{
    // zero scale operands select the unscaled instruction; formats 0/0 = E4M3 x E4M3
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ u32x2_t read_tr8(const uint8_t *p)
{
    return bitcast<u32x2_t>(__builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t *)(p)));
}

__device__ __forceinline__ i32x8_t join(u32x4_t lo, u32x4_t hi)
{
    return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <int D> struct Fp8Geo {
    // 32-row query blocks per wave: one.  The loop is VALU-bound, so at d = 64
    // the register budget goes to occupancy instead (about 125 VGPRs, three or
    // four waves per SIMD to hide exp and MFMA latency: 11% faster on the
    // trading-day prefill than two blocks at two waves); K and V operand reads
    // per MFMA double, which LDS absorbs at this rate.
    static constexpr int QB = 1;
    static constexpr int BR = 4 * 32 * QB;      // query rows per workgroup
    static constexpr int BC = 64;               // keys per KV tile
    static constexpr int RS = D + 16;           // LDS row stride in bytes (K and V)
    static constexpr int CPR = D / 16;          // 16-byte chunks per row
    static constexpr int CH = BC * CPR / 256;   // chunks per thread per tile
    static constexpr int KS = D / 64;           // 64-deep K-steps of the score product
    static constexpr int MB = D / 32;           // 32-row blocks of O^T
};

// LDS row of key k inside a V tile: bits 2 and 3 exchanged.
__device__ __forceinline__ int vrow(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

__device__ __forceinline__ float max_pair(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_pair(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <typename TO> struct Store4;
template <> struct Store4<float> {
    static __device__ __forceinline__ void put(float *p, float a, float b, float c, float d)
    {
        *reinterpret_cast<f32x4_t *>(p) = f32x4_t{a, b, c, d};
    }
};
template <> struct Store4<__bf16> {
    static __device__ __forceinline__ void put(__bf16 *p, float a, float b, float c, float d)
    {
        typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
        *reinterpret_cast<bf16x4_t *>(p) = bf16x4_t{(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
    }
};

template <int D, bool CAUSAL, typename TO>
__global__ void __launch_bounds__(256, D == 64 ? 3 : 2)
fwd_fp8_kernel(const uint8_t *__restrict__ Q, const uint8_t *__restrict__ K,
               const uint8_t *__restrict__ V, const float *__restrict__ qsc,
               const float *__restrict__ ksc, const float *__restrict__ vsc, TO *__restrict__ O,
               float *__restrict__ LSE, int H, int Hkv, int Nq, int Nk, int n_bh, int n_qtiles,
               float scale_log2, float log2S, int reverse)
{
    using G = Fp8Geo<D>;
    constexpr int QB = G::QB, BC = G::BC, RS = G::RS, KS = G::KS, MB = G::MB, CH = G::CH;

    __shared__ __attribute__((aligned(16))) uint8_t Kbuf[2][BC * RS];
    __shared__ __attribute__((aligned(16))) uint8_t Vbuf[2][BC * RS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, c = lane & 31, g = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

    const int qt = n_qtiles - 1 - (int)(blockIdx.x / (unsigned)n_bh);
    const int bh = (int)(blockIdx.x % (unsigned)n_bh);
    const int b = bh / H, h = bh - b * H;
    const int bhk = b * Hkv + h / (H / Hkv);
    const uint8_t *Qb = Q + (size_t)bh * Nq * D;
    const uint8_t *Kb = K + (size_t)bhk * Nk * D;
    const uint8_t *Vb = V + (size_t)bhk * Nk * D;
    const int nqb = (Nq + 31) / 32, nkb = (Nk + 31) / 32;

    const int q0 = qt * G::BR;
    const int q0w = q0 + w * 32 * QB;
    const int off = Nk - Nq;
    int nkt = (Nk + BC - 1) / BC;
    if (CAUSAL) {
        const int lim = min(q0 + G::BR, Nq) - 1 + off;
        nkt = lim < 0 ? 0 : min(nkt, lim / BC + 1);
    }

    // Q operand (B of S^T = K Q^T): lane (c, g), K-step ks holds bytes
    // [64ks + 32g, +32) of row q0w + 32qb + c; rows past Nq read as zero.
    i32x8_t qop[QB][KS];
    float cq[QB];
    {
        const __amdgpu_buffer_rsrc_t rq = rows_rsrc<uint8_t, D>(Qb, Nq, q0w);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int o = (32 * qb + c) * D + 64 * ks + 32 * g;
                qop[qb][ks] = join(__builtin_amdgcn_raw_buffer_load_b128(rq, o, 0, 0),
                                   __builtin_amdgcn_raw_buffer_load_b128(rq, o + 16, 0, 0));
            }
            cq[qb] = scale_log2 * qsc[(size_t)bh * nqb + min(q0w / 32 + qb, nqb - 1)];
        }
    }

    f32x16_t acc[QB][MB];
    float m_run[QB], l_run[QB];  // running max (log2 units, S-free), sum of S*p (this lane's keys)
    // E4M3 P operand of each query block.  A pair conversion writes half of a
    // register and keeps the other half, which the second conversion then
    // overwrites; starting from the previous tile's register (not from zero)
    // saves a move per register.
    i32x8_t pop[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[qb][mb] = f32x16_t{};
        m_run[qb] = -INFINITY;
        l_run[qb] = 0.f;
        pop[qb] = i32x8_t{};
    }

    // staging map: chunk ci = tid + 256 r is row ci / CPR, 16 bytes at (ci % CPR) * 16
    int goff[CH], kst[CH], vst[CH];
#pragma unroll
    for (int r = 0; r < CH; ++r) {
        const int ci = tid + 256 * r, row = ci / G::CPR, col = (ci % G::CPR) * 16;
        goff[r] = row * D + col;
        kst[r] = row * RS + col;
        vst[r] = vrow(row) * RS + col;
    }
    u32x4_t kreg[CH], vreg[CH];
    auto order = [&](int tt) { return reverse ? nkt - 1 - tt : tt; };
    auto load_tile = [&](int t) {
        const __amdgpu_buffer_rsrc_t rk = rows_rsrc<uint8_t, D>(Kb, Nk, BC * t);
        const __amdgpu_buffer_rsrc_t rv = rows_rsrc<uint8_t, D>(Vb, Nk, BC * t);
#pragma unroll
        for (int r = 0; r < CH; ++r) {
            kreg[r] = __builtin_amdgcn_raw_buffer_load_b128(rk, goff[r], 0, 0);
            vreg[r] = __builtin_amdgcn_raw_buffer_load_b128(rv, goff[r], 0, 0);
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int r = 0; r < CH; ++r) {
            *reinterpret_cast<u32x4_t *>(&Kbuf[buf][kst[r]]) = kreg[r];
            *reinterpret_cast<u32x4_t *>(&Vbuf[buf][vst[r]]) = vreg[r];
        }
    };

    // V^T transpose-read address of this lane (row r0 = 16t + 8g + (lane%16)/2,
    // column 16 (c/16) + 8 (lane%2), plus 32 mb)
    const int tr_off = (8 * g + ((lane & 15) >> 1)) * RS + 16 * (c >> 4) + 8 * (lane & 1);

    if (nkt > 0) {
        load_tile(order(0));
        store_tile(0);
        if (nkt > 1) load_tile(order(1));
    }
    for (int tt = 0; tt < nkt; ++tt) {
        lds_barrier();  // tile tt visible in buffer tt&1; buffer (tt+1)&1 free
        if (tt + 1 < nkt) {
            store_tile((tt + 1) & 1);
            if (tt + 2 < nkt) load_tile(order(tt + 2));
        }
        const int t = order(tt);
        const uint8_t *Ks = Kbuf[tt & 1];
        const uint8_t *Vs = Vbuf[tt & 1];

        i32x8_t kop[2][KS];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const uint8_t *p = &Ks[(32 * kb + c) * RS + 64 * ks + 32 * g];
                kop[kb][ks] = join(*reinterpret_cast<const u32x4_t *>(p),
                                   *reinterpret_cast<const u32x4_t *>(p + 16));
            }
        i32x8_t vop[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const u32x2_t x = read_tr8(Vs + tr_off + 16 * u * RS + 32 * mb);
                vop[mb][2 * u] = (int)x.x;
                vop[mb][2 * u + 1] = (int)x.y;
            }
        const float ks0 = ksc[(size_t)bhk * nkb + min(2 * t, nkb - 1)];
        const float ks1 = ksc[(size_t)bhk * nkb + min(2 * t + 1, nkb - 1)];
        const int k0 = BC * t;
        const bool need_mask = (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > q0w + off);

#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            f32x16_t s[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                s[kb] = f32x16_t{};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) s[kb] = mma_fp8(kop[kb][ks], qop[qb][ks], s[kb]);
            }
            if (need_mask) {
                const int qi = q0w + 32 * qb + c;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
                        if (key >= Nk || (CAUSAL && key > qi + off)) s[kb][r] = -INFINITY;
                    }
            }
            const float c0 = cq[qb] * ks0, c1 = cq[qb] * ks1;
            float t0 = s[0][0], t1 = s[1][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) {
                t0 = fmaxf(t0, s[0][r]);
                t1 = fmaxf(t1, s[1][r]);
            }
            const float tm = max_pair(fmaxf(t0 * c0, t1 * c1));
            const float mn = fmaxf(m_run[qb], tm);
            const float alpha = (mn == m_run[qb]) ? 1.f : fast_exp2(m_run[qb] - mn);
            if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
                l_run[qb] *= alpha;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[qb][mb][r] *= alpha;
            }
            m_run[qb] = mn;
            const float mref = (mn == -INFINITY) ? 0.f : mn - log2S;  // exp2(x c - mref) = S p
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const float ck = kb == 0 ? c0 : c1;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float p0 = fast_exp2(fmaf(s[kb][4 * u + 0], ck, -mref));
                    const float p1 = fast_exp2(fmaf(s[kb][4 * u + 1], ck, -mref));
                    const float p2 = fast_exp2(fmaf(s[kb][4 * u + 2], ck, -mref));
                    const float p3 = fast_exp2(fmaf(s[kb][4 * u + 3], ck, -mref));
                    l_run[qb] += p0;
                    l_run[qb] += p1;
                    l_run[qb] += p2;
                    l_run[qb] += p3;
                    int pk = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pop[qb][4 * kb + u], false);
                    pk = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, pk, true);
                    pop[qb][4 * kb + u] = pk;
                }
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[qb][mb] = mma_fp8(vop[mb], pop[qb], acc[qb][mb]);
        }
    }

    // epilogue: O = v_scale * acc / sum(S p),  LSE = ln 2 (m - log2 S) + ln(sum(S p))
    const float *vs = vsc + (size_t)bhk * D;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l = sum_pair(l_run[qb]);
        const int row = q0w + 32 * qb + c;
        if (row >= Nq) continue;
        TO *orow = O + ((size_t)bh * Nq + row) * D;
        if (l > 0.f) {
            const float inv = 1.f / l;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int d0 = 32 * mb + 8 * r4 + 4 * g;
                    const f32x4_t sc = *reinterpret_cast<const f32x4_t *>(vs + d0);
                    Store4<TO>::put(orow + d0, acc[qb][mb][4 * r4] * inv * sc.x,
                                    acc[qb][mb][4 * r4 + 1] * inv * sc.y,
                                    acc[qb][mb][4 * r4 + 2] * inv * sc.z,
                                    acc[qb][mb][4 * r4 + 3] * inv * sc.w);
                }
        } else {  // no visible key (v_scales may be absent when Nk = 0)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) Store4<TO>::put(orow + 32 * mb + 8 * r4 + 4 * g, 0.f, 0.f, 0.f, 0.f);
        }
        if (LSE != nullptr && g == 0)
            LSE[(size_t)bh * Nq + row] =
                (l > 0.f) ? (m_run[qb] - log2S) * 0.6931471805599453f + logf(l) : -INFINITY;
    }
}

template <int D, bool CAUSAL, typename TO>
hipError_t launch3(const Fp8Problem &p, hipStream_t st)
{
    using G = Fp8Geo<D>;
    const int n_bh = p.B * p.H;
    const int n_qtiles = (p.Nq + G::BR - 1) / G::BR;
    const unsigned blocks = (unsigned)n_qtiles * (unsigned)n_bh;
    hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, TO>), dim3(blocks), dim3(256), 0, st, p.q, p.k, p.v,
                       p.q_scales, p.k_scales, p.v_scales, static_cast<TO *>(p.o), p.lse, p.H, p.Hkv,
                       p.Nq, p.Nk, n_bh, n_qtiles, p.scale * kLog2e, log2f(p.p_scale), p.kv_reverse);
    return hipGetLastError();
}

template <int D, typename TO>
hipError_t launch2(const Fp8Problem &p, hipStream_t st)
{
    return p.causal ? launch3<D, true, TO>(p, st) : launch3<D, false, TO>(p, st);
}

template <typename TO>
hipError_t launch1(const Fp8Problem &p, hipStream_t st)
{
    return p.d == 64 ? launch2<64, TO>(p, st) : launch2<128, TO>(p, st);
}

}  // namespace

int fwd_fp8_kv_tile() { return 64; }

hipError_t launch_fwd_fp8(const Fp8Problem &p, hipStream_t st)
{
    return p.o_dtype == 0 ? launch1<float>(p, st) : launch1<__bf16>(p, st);
}

}  // namespace fa
