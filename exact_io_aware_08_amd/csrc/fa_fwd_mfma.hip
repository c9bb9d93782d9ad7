// fa_fwd_mfma.hip -- forward (prefill) attention on bf16/fp16 MFMA, gfx950.
//
// Method: marketmaker.cc blog "Atencion flash y la pregunta sobre la longitud
// de la secuencia", sections "El algoritmo de atencion flash" (Q split into
// row blocks, K/V into column blocks, each query block sweeps the KV blocks
// keeping a running max m, running sum l and an output accumulator) and
// "La recurrencia de softmax en linea" (accumulator rescaled by
// e^(m_old - m_new) whenever the max grows); "FA2: paralelismo" (the
// normalisation by l is deferred to the end; the grid also runs over query
// blocks; each wave owns whole query rows, so no cross-wave reduction);
// "El enmascaramiento causal ..." (KV tiles wholly in the future are never
// loaded or computed).  systems-analysis.info "FlashAttention (IT)",
// "Innovazioni chiave": QK^T, mask, softmax and xV fused in one kernel that
// writes only O (and the per-row LSE).
//
// gfx950 mapping (one workgroup = 4 waves = 128 query rows of one (b, h)):
//  * Each wave owns 32 query rows.  Scores are computed transposed,
//    S^T = K Q^T, on v_mfma_f32_32x32x16: the fp32 result then gives lane l
//    the 16 keys {8i + 4(l/32) + r} of query l%32, so a row's max needs one
//    exchange between lanes l and l^32 and its sum none until the epilogue.
//  * The S^T accumulator is directly the B operand of O^T = V^T P^T (after a
//    cvt to bf16/fp16): key-slot k of lane group g in K-step t is key
//    16t + 8(k/4) + 4g + k%4 of the 32-key block.  V^T is therefore staged
//    in LDS transposed ([d][key]) so the A operand is two 8-byte reads.
//  * K tiles are staged row-major in LDS ([key][d], padded), read as 16-byte
//    A-operand rows.  Q stays in registers for the whole sweep.
//  * Global loads of KV tile j+1 are issued before tile j is computed, so
//    HBM/L2 latency overlaps the MFMA and softmax work.
//  * Causal grids run the longest query tiles first.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

constexpr int NW = 4;
constexpr int BR = NW * 32;
constexpr int BC = kFwdKvTile;
static_assert(BR == kFwdQTile, "query tile");
static_assert(BC == 64, "the kernel body assumes two 32-key blocks per tile");

// Tile geometry of the KV staging (256 threads, 16-byte chunks).
template <int D> struct KvGeom {
    static constexpr int KSTR = D + 8;            // K tile row stride in LDS (elements)
    static constexpr int VSTR = BC + 4;           // V^T tile row stride in LDS (elements)
    static constexpr int CPR = D / 8;             // 16-byte chunks per K/V row
    static constexpr int KCH = BC * CPR / 256;    // K chunks per thread per tile
    static constexpr int PPR = 256 / CPR;         // V key pairs per round
    static constexpr int VROUNDS = (BC / 2) / PPR;
    static_assert(KCH * 256 == BC * CPR && VROUNDS * PPR * 2 == BC, "tile split");
};

// Global -> registers for KV tile starting at key j0.  Keys past Nk (ragged
// last tile) load row Nk-1 instead: their scores are masked to -inf, so they
// get weight 0 and the finite V row adds nothing.
template <typename T, int D>
__device__ __forceinline__ void load_kv_tile(const T *__restrict__ Kb, const T *__restrict__ Vb,
                                             int Nk, int j0, int tid,
                                             u32x4_t (&kreg)[KvGeom<D>::KCH],
                                             u32x4_t (&vreg)[2 * KvGeom<D>::VROUNDS])
{
    using G = KvGeom<D>;
#pragma unroll
    for (int r = 0; r < G::KCH; ++r) {
        const int ci = tid + r * 256;
        const int key = min(j0 + ci / G::CPR, Nk - 1), cc = ci % G::CPR;
        kreg[r] = *reinterpret_cast<const u32x4_t *>(Kb + (size_t)key * D + cc * 8);
    }
#pragma unroll
    for (int r = 0; r < G::VROUNDS; ++r) {
        const int kp = tid / G::CPR + r * G::PPR, cc = tid % G::CPR;
        const int k0 = min(j0 + 2 * kp, Nk - 1), k1 = min(j0 + 2 * kp + 1, Nk - 1);
        vreg[2 * r] = *reinterpret_cast<const u32x4_t *>(Vb + (size_t)k0 * D + cc * 8);
        vreg[2 * r + 1] = *reinterpret_cast<const u32x4_t *>(Vb + (size_t)k1 * D + cc * 8);
    }
}

// Registers -> LDS: K row-major [key][d]; V transposed [d][key], two keys
// packed per dword (key 2kp in the low half, 2kp+1 in the high half).
template <typename T, int D>
__device__ __forceinline__ void store_kv_tile(T *Ks, T *Vt, int tid,
                                              const u32x4_t (&kreg)[KvGeom<D>::KCH],
                                              const u32x4_t (&vreg)[2 * KvGeom<D>::VROUNDS])
{
    using G = KvGeom<D>;
#pragma unroll
    for (int r = 0; r < G::KCH; ++r) {
        const int ci = tid + r * 256;
        *reinterpret_cast<u32x4_t *>(&Ks[(ci / G::CPR) * G::KSTR + (ci % G::CPR) * 8]) = kreg[r];
    }
#pragma unroll
    for (int r = 0; r < G::VROUNDS; ++r) {
        const int kp = tid / G::CPR + r * G::PPR, cc = tid % G::CPR;
        const u32x4_t a = vreg[2 * r], bq = vreg[2 * r + 1];
        // element e of the chunk is d = 8cc + e
        uint32_t *base = reinterpret_cast<uint32_t *>(&Vt[(cc * 8) * G::VSTR + 2 * kp]);
        constexpr int RS = G::VSTR / 2;  // V^T row stride in dwords
        base[0 * RS] = pack_lo16(a.x, bq.x);
        base[1 * RS] = pack_hi16(a.x, bq.x);
        base[2 * RS] = pack_lo16(a.y, bq.y);
        base[3 * RS] = pack_hi16(a.y, bq.y);
        base[4 * RS] = pack_lo16(a.z, bq.z);
        base[5 * RS] = pack_hi16(a.z, bq.z);
        base[6 * RS] = pack_lo16(a.w, bq.w);
        base[7 * RS] = pack_hi16(a.w, bq.w);
    }
}

template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 2)
fwd_mfma_kernel(const T *__restrict__ Q, const T *__restrict__ K, const T *__restrict__ V,
                T *__restrict__ O, float *__restrict__ LSE, int H, int Hkv, int Nq, int Nk,
                int n_bh, int n_qtiles, float scale, float scale_log2)
{
    using M = Mma16<T>;
    using v8 = typename M::v8;
    constexpr int KSTR = KvGeom<D>::KSTR;
    constexpr int VSTR = KvGeom<D>::VSTR;
    constexpr int KCH = KvGeom<D>::KCH;
    constexpr int VROUNDS = KvGeom<D>::VROUNDS;

    __shared__ __attribute__((aligned(16))) T Ks[BC * KSTR];
    __shared__ __attribute__((aligned(16))) T Vt[D * VSTR];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, c = lane & 31, hh = lane >> 5;

    const int qt = n_qtiles - 1 - (int)(blockIdx.x / (unsigned)n_bh);
    const int bh = (int)(blockIdx.x % (unsigned)n_bh);
    const int b = bh / H, h = bh - b * H;
    const int hk = h / (H / Hkv);
    const size_t qoff = (size_t)bh * Nq * D;
    const size_t kvoff = ((size_t)b * Hkv + hk) * Nk * D;
    const T *Qb = Q + qoff;
    const T *Kb = K + kvoff;
    const T *Vb = V + kvoff;
    T *Ob = O + qoff;

    const int q0 = qt * BR;
    const int q0w = q0 + w * 32;
    const int off = Nk - Nq;
    int nkt = (Nk + BC - 1) / BC;
    if (CAUSAL) {
        const int lim = min(q0 + BR, Nq) - 1 + off;  // last key any row of the block sees
        nkt = lim < 0 ? 0 : min(nkt, lim / BC + 1);
    }

    // Q operand (B of S^T = K Q^T): lane (c, hh) holds Q[q0w + c][16t + 8hh + e].
    // Rows past Nq load the last row instead; their results are never stored.
    v8 qop[D / 16];
    {
        const int qrow = min(q0w + c, Nq - 1);
#pragma unroll
        for (int t = 0; t < D / 16; ++t)
            qop[t] = bitcast<v8>(*reinterpret_cast<const u32x4_t *>(Qb + (size_t)qrow * D + 16 * t + 8 * hh));
    }

    f32x16_t acc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc[i] = f32x16_t{};
    float m_run = -INFINITY, l_run = 0.f;

    u32x4_t kreg[KCH], vreg[2 * VROUNDS];
    if (nkt > 0) load_kv_tile<T, D>(Kb, Vb, Nk, 0, tid, kreg, vreg);
    for (int j = 0; j < nkt; ++j) {
        __syncthreads();  // every wave is done reading tile j-1
        store_kv_tile<T, D>(Ks, Vt, tid, kreg, vreg);
        __syncthreads();
        if (j + 1 < nkt) load_kv_tile<T, D>(Kb, Vb, Nk, (j + 1) * BC, tid, kreg, vreg);
        const int j0 = j * BC;
        if (CAUSAL && j0 > q0w + 31 + off) continue;  // no row of this wave sees tile j

        // ---- S^T = K_j Q^T (fp32) ----
        f32x16_t s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = f32x16_t{};
#pragma unroll
            for (int t = 0; t < D / 16; ++t) {
                const v8 kop = *reinterpret_cast<const v8 *>(&Ks[(kb * 32 + c) * KSTR + 16 * t + 8 * hh]);
                s[kb] = M::mma32(kop, qop[t], s[kb]);
            }
        }

        // ---- mask: ragged last tile, and the diagonal band when causal ----
        const bool need_mask = (j0 + BC > Nk) || (CAUSAL && j0 + BC - 1 > q0w + off);
        if (need_mask) {
            const int lim = CAUSAL ? min(Nk, q0w + c + off + 1) : Nk;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = j0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if (key >= lim) s[kb][r] = -INFINITY;
                }
        }

        // ---- online softmax (running max; normalisation deferred) ----
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2((m_run - m_use) * scale_log2);
        const float mneg = -m_use * scale_log2;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(fmaf(s[kb][r], scale_log2, mneg));
                s[kb][r] = p;
                rs += p;
            }
        l_run = l_run * alpha + rs;
        m_run = m_new;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) acc[i] *= alpha;

        // ---- O^T += V_j^T P^T ----
        v8 pop[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 8; ++e) pop[kb * 2 + t][e] = static_cast<T>(s[kb][8 * t + e]);
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const T *vp = &Vt[(32 * mb + c) * VSTR + kb * 32 + 16 * t + 4 * hh];
                    const u32x2_t lo = *reinterpret_cast<const u32x2_t *>(vp);
                    const u32x2_t hi = *reinterpret_cast<const u32x2_t *>(vp + 8);
                    const v8 vop = bitcast<v8>(u32x4_t{lo.x, lo.y, hi.x, hi.y});
                    acc[mb] = M::mma32(vop, pop[kb * 2 + t], acc[mb]);
                }
    }

    // ---- epilogue: O = acc / l, LSE = m*scale + ln l ----
    const float l = l_run + __shfl_xor(l_run, 32);
    const int row = q0w + c;
    if (row < Nq) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = 32 * mb + 8 * i + 4 * hh;
                typedef T t4 __attribute__((ext_vector_type(4)));
                t4 vals;
                vals[0] = static_cast<T>(acc[mb][4 * i + 0] * inv);
                vals[1] = static_cast<T>(acc[mb][4 * i + 1] * inv);
                vals[2] = static_cast<T>(acc[mb][4 * i + 2] * inv);
                vals[3] = static_cast<T>(acc[mb][4 * i + 3] * inv);
                *reinterpret_cast<t4 *>(Ob + (size_t)row * D + d0) = vals;
            }
        if (LSE != nullptr && hh == 0)
            LSE[(size_t)bh * Nq + row] = l > 0.f ? m_run * scale + logf(l) : -INFINITY;
    }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_t(const FwdProblem &p, hipStream_t st)
{
    const int n_qtiles = (p.Nq + BR - 1) / BR;
    const int n_bh = p.B * p.H;
    const dim3 grid((unsigned)n_qtiles * (unsigned)n_bh), block(256);
    hipLaunchKernelGGL((fwd_mfma_kernel<T, D, CAUSAL>), grid, block, 0, st,
                       static_cast<const T *>(p.q), static_cast<const T *>(p.k),
                       static_cast<const T *>(p.v), static_cast<T *>(p.o), p.lse, p.H, p.Hkv,
                       p.Nq, p.Nk, n_bh, n_qtiles, p.scale, p.scale * kLog2e);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_dt(const FwdProblem &p, hipStream_t st)
{
    if (p.d == 64) return p.causal ? launch_t<T, 64, true>(p, st) : launch_t<T, 64, false>(p, st);
    return p.causal ? launch_t<T, 128, true>(p, st) : launch_t<T, 128, false>(p, st);
}

}  // namespace

hipError_t launch_fwd_mfma(const FwdProblem &p, hipStream_t st)
{
    if (p.dtype == 2) return launch_dt<__bf16>(p, st);
    return launch_dt<_Float16>(p, st);
}

}  // namespace fa
