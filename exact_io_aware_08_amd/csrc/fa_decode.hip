// fa_decode.hip -- split-KV decode with a log-sum-exp merge, gfx950.
//
// One new query token per (batch, head) attends to a KV cache of Nk keys.
// The key axis is cut into `splits` slices; each workgroup runs the online
// softmax recurrence (marketmaker.cc blog "Atencion flash y la pregunta sobre
// la longitud de la secuencia", sections "El algoritmo de atencion flash" and
// "La recurrencia de softmax en linea") over one slice and writes a partial
// (O_s normalised, lse_s); a second kernel merges the partials.  Because the
// recurrence is a reassociation, merging partials of any key partition with
//   LSE = M + ln sum_s e^(lse_s - M),  O = sum_s e^(lse_s - LSE) O_s
// gives the same result as one sweep.
//
// GQA: a workgroup serves up to 16 query heads that share one KV head, so
// the KV slice is read once for all of them (gist.science "FlashAttention
// for Scalable Vector Architectures", section "Metodologia": load the shared
// KV head once and reuse it).  The work is a scan of the KV cache, bound by
// HBM bandwidth; the small products run on v_mfma_f32_16x16x32 with the
// query heads in the N dimension (padded to 16):
//   S^T (16 keys x 16 heads) = K_blk q^T: A = K rows loaded straight from
//     global memory in operand layout (lane l: key l%16, d = 32t + 8(l/16) + e);
//   O^T (d x 16 heads) += V^T P^T: P^T comes from the S^T accumulators
//     (lane group g, slot e -> key 4g + e, or 16 + 4g + e-4); V^T is staged
//     per wave in LDS, transposed, and read as two 8-byte runs.
// Each of the 4 waves takes its own 32 keys of every 128-key step, keeps its
// own (m, l, O), and the waves are merged through LDS at the end.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

constexpr int NW = 4;
constexpr int WK = 32;  // keys per wave per step
static_assert(NW * WK == kDecodeStep, "step");

template <typename T, int D>
__global__ void __launch_bounds__(256)
decode_split_kernel(const T *__restrict__ Qg, const T *__restrict__ K, const T *__restrict__ V,
                    float *__restrict__ part_o, float *__restrict__ part_lse, int H, int Hkv,
                    int Nk, int G, int n_qgroups, int splits, int chunk, float scale,
                    float scale_log2)
{
    using M = Mma16<T>;
    using v8 = typename M::v8;
    constexpr int VSTR = WK + 4;          // per-wave V^T row stride (elements)
    constexpr int CPR = D / 8;            // 16-byte chunks per row
    constexpr int VPAIRS = D / 32;        // key pairs loaded per lane per step
    constexpr int KT = D / 32;            // K-steps of the S^T product

    // The per-wave V^T slices and the end-of-sweep merge buffer are never live
    // together, so they share one LDS block (a barrier separates the uses).
    constexpr int VT_BYTES = NW * D * VSTR * (int)sizeof(T);
    constexpr int SO_BYTES = NW * 16 * (D + 1) * (int)sizeof(float);
    __shared__ __attribute__((aligned(16))) unsigned char smem[VT_BYTES > SO_BYTES ? VT_BYTES : SO_BYTES];
    __shared__ float sm_m[NW][16], sm_l[NW][16];
    T(*Vt)[D * VSTR] = reinterpret_cast<T(*)[D * VSTR]>(smem);
    float(*sm_o)[16][D + 1] = reinterpret_cast<float(*)[16][D + 1]>(smem);

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, c = lane & 15, g = lane >> 4;

    const int split = (int)(blockIdx.x % (unsigned)splits);
    int rest = (int)(blockIdx.x / (unsigned)splits);
    const int qg = rest % n_qgroups;
    rest /= n_qgroups;
    const int hk = rest % Hkv;
    const int b = rest / Hkv;
    const int h0 = hk * G + qg * 16;
    const int nq = min(16, G - qg * 16);  // real query heads in this group

    const int kbeg = split * chunk;
    const int kend = min(Nk, kbeg + chunk);
    const size_t kvoff = ((size_t)b * Hkv + hk) * Nk * D;
    const T *Kb = K + kvoff;
    const T *Vb = V + kvoff;

    // q operand (B of S^T): lane (c, g) holds q[h0 + c][32t + 8g + e]; padding
    // columns c >= nq repeat the last real head and are never written out.
    v8 qop[KT];
    const int qh = h0 + min(c, nq - 1);
#pragma unroll
    for (int t = 0; t < KT; ++t)
        qop[t] = bitcast<v8>(*reinterpret_cast<const u32x4_t *>(Qg + ((size_t)b * H + qh) * D + 32 * t + 8 * g));

    f32x4_t acc[D / 16];
#pragma unroll
    for (int i = 0; i < D / 16; ++i) acc[i] = f32x4_t{};
    float m_run = -INFINITY, l_run = 0.f;

    // Keys past kend load row kend-1 instead (masked to weight 0).
    u32x4_t kreg[2][KT], vreg[2 * VPAIRS];
    auto load_step = [&](int base) {  // base: first key of this wave's 32
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                const int key = min(base + 16 * kb + c, kend - 1);
                kreg[kb][t] = *reinterpret_cast<const u32x4_t *>(Kb + (size_t)key * D + 32 * t + 8 * g);
            }
#pragma unroll
        for (int u = 0; u < VPAIRS; ++u) {
            const int kp = lane / CPR + u * (64 / CPR), cc = lane % CPR;
            const int k0 = min(base + 2 * kp, kend - 1), k1 = min(base + 2 * kp + 1, kend - 1);
            vreg[2 * u] = *reinterpret_cast<const u32x4_t *>(Vb + (size_t)k0 * D + 8 * cc);
            vreg[2 * u + 1] = *reinterpret_cast<const u32x4_t *>(Vb + (size_t)k1 * D + 8 * cc);
        }
    };

    T *vt = Vt[w];
    const int nsteps = kend > kbeg ? (kend - kbeg + kDecodeStep - 1) / kDecodeStep : 0;
    if (nsteps > 0) load_step(kbeg + w * WK);
    for (int st = 0; st < nsteps; ++st) {
        const int base = kbeg + st * kDecodeStep + w * WK;
        // V^T into this wave's LDS slice (keys 2kp, 2kp+1 packed per dword)
#pragma unroll
        for (int u = 0; u < VPAIRS; ++u) {
            const int kp = lane / CPR + u * (64 / CPR), cc = lane % CPR;
            const uint32_t a[4] = {vreg[2 * u].x, vreg[2 * u].y, vreg[2 * u].z, vreg[2 * u].w};
            const uint32_t bq[4] = {vreg[2 * u + 1].x, vreg[2 * u + 1].y, vreg[2 * u + 1].z,
                                    vreg[2 * u + 1].w};
            uint32_t *dst = reinterpret_cast<uint32_t *>(&vt[(8 * cc) * VSTR + 2 * kp]);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                dst[(2 * m) * (VSTR / 2)] = pack_lo16(a[m], bq[m]);
                dst[(2 * m + 1) * (VSTR / 2)] = pack_hi16(a[m], bq[m]);
            }
        }
        u32x4_t kcur[2][KT];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int t = 0; t < KT; ++t) kcur[kb][t] = kreg[kb][t];
        if (st + 1 < nsteps) load_step(base + kDecodeStep);

        // S^T for this wave's 32 keys
        f32x4_t s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = f32x4_t{};
#pragma unroll
            for (int t = 0; t < KT; ++t) s[kb] = M::mma16(bitcast<v8>(kcur[kb][t]), qop[t], s[kb]);
        }
        if (base + WK > kend) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (base + 16 * kb + 4 * g + r >= kend) s[kb][r] = -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2((m_run - m_use) * scale_log2);
        const float mneg = -m_use * scale_log2;
        float rs = 0.f;
        v8 pop;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = fast_exp2(fmaf(s[kb][r], scale_log2, mneg));
                rs += p;
                pop[4 * kb + r] = static_cast<T>(p);
            }
        l_run = l_run * alpha + rs;
        m_run = m_new;
#pragma unroll
        for (int i = 0; i < D / 16; ++i) acc[i] *= alpha;

        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int mb = 0; mb < D / 16; ++mb) {
            const T *vp = &vt[(16 * mb + c) * VSTR + 4 * g];
            const u32x2_t lo = *reinterpret_cast<const u32x2_t *>(vp);
            const u32x2_t hi = *reinterpret_cast<const u32x2_t *>(vp + 16);
            acc[mb] = M::mma16(bitcast<v8>(u32x4_t{lo.x, lo.y, hi.x, hi.y}), pop, acc[mb]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // ---- merge the 4 waves of this workgroup ----
    float l = l_run + __shfl_xor(l_run, 16);
    l += __shfl_xor(l, 32);
    __syncthreads();  // every wave is done with its V^T slice (sm_o aliases it)
    if (g == 0) {
        sm_m[w][c] = m_run;
        sm_l[w][c] = l;
    }
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) sm_o[w][c][16 * mb + 4 * g + r] = acc[mb][r];
    __syncthreads();

    const int qi = tid >> 4;          // query head slot 0..15
    const int dl = tid & 15;          // this thread covers d = dl + 16 i
    if (qi < nq) {
        float M_ = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) M_ = fmaxf(M_, sm_m[ww][qi]);
        float wt[NW], L = 0.f;
        const float Mu = (M_ == -INFINITY) ? 0.f : M_;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            wt[ww] = fast_exp2((sm_m[ww][qi] - Mu) * scale_log2);
            L += wt[ww] * sm_l[ww][qi];
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
        const size_t prow = ((size_t)b * H + h0 + qi) * splits + split;
#pragma unroll
        for (int i = 0; i < D / 16; ++i) {
            const int d = dl + 16 * i;
            float o = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) o += wt[ww] * sm_o[ww][qi][d];
            part_o[prow * D + d] = o * inv;
        }
        if (dl == 0) part_lse[prow] = L > 0.f ? M_ * scale + logf(L) : -INFINITY;
    }
}

// One thread per (b, h, d); partials of all splits merged with log-sum-exp.
template <typename T, int D>
__global__ void __launch_bounds__(256)
decode_merge_kernel(const float *__restrict__ part_o, const float *__restrict__ part_lse,
                    T *__restrict__ O, float *__restrict__ LSE, int BH, int splits)
{
    const int idx = blockIdx.x * 256 + threadIdx.x;
    const int bh = idx / D, d = idx % D;
    if (bh >= BH) return;
    const float *pl = part_lse + (size_t)bh * splits;
    float M_ = -INFINITY;
    for (int s = 0; s < splits; ++s) M_ = fmaxf(M_, pl[s]);
    float o = 0.f, L = 0.f;
    if (M_ != -INFINITY) {
        const float *po = part_o + (size_t)bh * splits * D + d;
        for (int s = 0; s < splits; ++s) {
            const float wgt = __expf(pl[s] - M_);
            L += wgt;
            o += wgt * po[(size_t)s * D];
        }
        o /= L;
    }
    O[(size_t)bh * D + d] = static_cast<T>(o);
    if (LSE != nullptr && d == 0) LSE[bh] = (M_ == -INFINITY) ? -INFINITY : M_ + logf(L);
}

template <typename T, int D>
hipError_t launch_t(const DecodeProblem &p, hipStream_t st)
{
    const int G = p.H / p.Hkv;
    const int n_qgroups = (G + 15) / 16;
    const unsigned n_blocks = (unsigned)p.splits * (unsigned)(p.B * p.Hkv * n_qgroups);
    hipLaunchKernelGGL((decode_split_kernel<T, D>), dim3(n_blocks), dim3(256), 0, st,
                       static_cast<const T *>(p.q), static_cast<const T *>(p.k),
                       static_cast<const T *>(p.v), p.part_o, p.part_lse, p.H, p.Hkv, p.Nk, G,
                       n_qgroups, p.splits, p.chunk, p.scale, p.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int BH = p.B * p.H;
    const unsigned mblocks = (unsigned)(((size_t)BH * D + 255) / 256);
    hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(mblocks), dim3(256), 0, st, p.part_o,
                       p.part_lse, static_cast<T *>(p.o), p.lse, BH, p.splits);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_dt(const DecodeProblem &p, hipStream_t st)
{
    return p.d == 64 ? launch_t<T, 64>(p, st) : launch_t<T, 128>(p, st);
}

}  // namespace

hipError_t launch_decode(const DecodeProblem &p, hipStream_t st)
{
    return p.dtype == 2 ? launch_dt<__bf16>(p, st) : launch_dt<_Float16>(p, st);
}

}  // namespace fa
