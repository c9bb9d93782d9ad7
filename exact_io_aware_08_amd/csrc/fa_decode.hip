// fa_decode.hip -- split-KV decode with a log-sum-exp merge of the splits,
// gfx950.
//
// One new query token per (batch, head) attends to a KV cache of Nk keys.
// The key axis is cut into `splits` slices; each workgroup runs the online
// softmax recurrence (marketmaker.cc blog "Atencion flash y la pregunta sobre
// la longitud de la secuencia", sections "El algoritmo de atencion flash" and
// "La recurrencia de softmax en linea") over one slice and writes a partial
// (O_s normalised, lse_s).  Because the recurrence is a reassociation,
// merging the partials of any key partition with
//   LSE = M + ln sum_s e^(lse_s - M),  O = sum_s e^(lse_s - LSE) O_s
// gives the same result as one sweep.  A second, small kernel merges: one
// wave per (batch, head) loads its partials in wide batches.  (A merge
// inside the sweep kernel, by the last workgroup of each group to finish,
// costs more than the kernel boundary on this chip: with device-scope
// release/acquire fences, which write back and invalidate each XCD's whole
// L2, or with device-scope relaxed stores and loads and an arrival ticket,
// whose three dependent round trips to memory outlast a launch.)  With one
// split the sweep kernel writes O and LSE itself.
//
// GQA: a workgroup serves up to 16 query heads that share one KV head, so
// the KV slice is read once for all of them (gist.science "FlashAttention
// for Scalable Vector Architectures", section "Metodologia": load the shared
// KV head once and reuse it).  The work is a scan of the KV cache, bound by
// HBM bandwidth, so the kernel is built to keep many bytes in flight: each
// wave holds a ring of NP register stages and issues the loads of step
// st + NP as soon as step st is consumed.  K and V of at least kStreamBytes
// per call are read with the non-temporal cache policy (for a paged batch
// with automatic splits the kernel counts them from the lengths): measured on
// MI355X, that is 11% faster for the 134 MB TinyLlama-shaped cache read cold
// (10% for the same cache as 128-key pages) and 2% faster even when the same
// cache is read by every call, while a 33 MB cache read by every call is 10%
// faster with the default policy (its lines stay in the 256 MB last-level
// cache between calls), a 70 MB ragged paged batch read from four rotating
// pools 5% faster, and a 67 MB contiguous cache the same either way.  Loads go through buffer
// descriptors that cover exactly the workgroup's key slice, so the
// prefetches past its end read zero and touch no memory.
//
// The small products run on v_mfma_f32_16x16x32 with the query heads in the
// N dimension (padded to 16):
//   S^T (16 keys x 16 heads) = K_blk q^T: A = K rows loaded straight from
//     global memory in operand layout (lane l: key l%16, d = 32t + 8(l/16) + e);
//   O^T (d x 16 heads) += V^T P^T: P^T comes from the S^T accumulators
//     (lane group g, slot e -> key 4g + e, or 16 + 4g + e-4).  V is stored
//     row-major in a per-wave LDS slice and read back transposed with
//     ds_read_b64_tr_b16: within each 16-lane group, lane s supplies the
//     address of key kb + s/4, columns 4(s%4)..+3, and lane i receives
//     column i of keys kb..kb+3 -- exactly the A-operand slots.
// Each of the 4 waves takes its own 32 keys of every 128-key step, keeps its
// own (m, l, O), and the waves are merged through LDS at the end.
//
// The cache is either contiguous or paged with per-sequence lengths (a
// block table maps each sequence's logical pages to physical pages, the
// KV-cache management of serving systems the "FlashAttention (IT)" entry
// mentions under "Soluzioni specializzate"); only the address of each
// wave's 32-key block changes.  A paged batch can also be split from its
// lengths, which only the device knows: every workgroup reads them, takes
// one chunk size for the whole batch (about kPagedTargetItems workgroups in
// all) and finds its (sequence, split) pair with a prefix sum over the
// lanes, so a ragged or skewed batch fills the GPU instead of following its
// longest sequence.
#include <mutex>

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

constexpr int NW = 4;
constexpr int WK = 32;                    // keys per wave per step
constexpr double kStreamBytes = 96.0 * (1 << 20);  // K + V bytes per call from which loads stream
static_assert(NW * WK == kDecodeStep, "step");

template <int D> struct DecodeGeo {
    static constexpr int NP = D == 64 ? 4 : 2;  // register stages (steps in flight)
    static constexpr int KT = D / 32;           // K-steps of the S^T product
    static constexpr int CPR = D / 8;           // 16-byte chunks per row
    static constexpr int VCH = WK * CPR / 64;   // V chunks per lane per step
    static constexpr int VS = D + 8;            // V row stride in LDS (elements, 16-byte rows)
};

// Buffer resource over `bytes` bytes starting at `base`; loads past the end
// read as zero.  Wave-uniform arguments.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const void *base, long long bytes)
{
    // clamped to the 31-bit range (a wave reads 32 rows past `base` at most)
    const long long b = bytes < 0 ? 0 : (bytes < 0x7fffffffLL ? bytes : 0x7fffffffLL);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)b,
                                             kBufferFlags);
}

// Cache addressing.  Contiguous: [B, Hkv, Nk, D], every sequence Nk keys.
// Paged: K/V pages [num_pages, Hkv, page_size, D]; key t of sequence b lives
// in page block_table[b * max_pages + t / page_size] at row t % page_size,
// and the sequence has seq_lens[b] keys.  page_size is a multiple of 32, so
// the 32 keys a wave loads per step never straddle a page.  Lengths are
// clamped to [0, max_pages * page_size] and a page index outside
// [0, num_pages) reads nothing, so bad tables cannot make an access fault.
struct PagedCache {
    const int *block_table;
    const int *seq_lens;
    int page_size, max_pages, num_pages;
    int auto_split;     // splits follow the lengths (see paged_auto_pair)
    int B;              // sequences (entries of seq_lens)
    int *split_counts;  // automatic splits with a merge: [B], each sequence's split count
};

// Automatic splits of a paged batch, from the lengths on the device (every
// wave computes the same values).  The chunk: about kPagedTargetItems
// workgroups for the whole batch, at least kPagedMinChunk keys, a multiple of
// the split granularity `gran`, at most the clamp length rounded up (a
// sequence then has one split).  Sequence b gets
// min(smax, max(1, ceil(len_b / chunk))) splits, and the (sequence, split)
// pairs are numbered sequence-major.  Returns the chunk, and for pair p its
// sequence, split and the sequence's split count; false past the last pair.
// The first 64 lengths are read once and kept for the scan.
__device__ bool paged_auto_pair(const int *__restrict__ lens, int B, int cap, int hq, int gran,
                                int smax, int p, int &chunk, int &b_out, int &sp_out, int &n_out,
                                long long &tot_out)
{
    const int lane = threadIdx.x & 63;
    const int L0 = lane < B ? min(max(lens[lane], 0), cap) : 0;
    long long tot = L0;
    for (int b = lane + 64; b < B; b += 64) tot += min(max(lens[b], 0), cap);
    tot = wave_sum_i64(tot);
    tot_out = tot;
    long long ch = (tot * hq + kPagedTargetItems - 1) / kPagedTargetItems;
    const long long top = ((long long)cap + gran - 1) / gran * gran;
    ch = (ch + gran - 1) / gran * gran;
    ch = ch < top ? ch : top;
    chunk = (int)(ch > kPagedMinChunk ? ch : kPagedMinChunk);

    int acc = 0;
    for (int base = 0; base < B; base += 64) {
        const int b = base + lane;
        const int L = base == 0 ? L0 : (b < B ? min(max(lens[b], 0), cap) : 0);
        const int n = b < B ? min(smax, max(1, (L + chunk - 1) / chunk)) : 0;
        const int inc = wave_scan_i32(n);  // inclusive prefix sum over the lanes
        const int blk = __builtin_amdgcn_readlane(inc, 63);
        if (p < acc + blk) {
            const int j = __builtin_ctzll(__ballot(acc + inc > p));
            const int incj = __builtin_amdgcn_readlane(inc, j), nj = __builtin_amdgcn_readlane(n, j);
            b_out = base + j;
            sp_out = p - (acc + incj - nj);
            n_out = nj;
            return true;
        }
        acc += blk;
    }
    return false;
}

// (Two workgroups per CU as the register target: the kernel then fits in
// 256 VGPRs with no accumulation registers, where a one-workgroup target let
// the compiler park the MFMA results in AGPRs and copy them to and from the
// VGPRs every step.)
template <typename T, int D, bool PAGED, bool STREAM>
__global__ void __launch_bounds__(256, 2)
decode_kernel(const T *__restrict__ Qg, const T *__restrict__ K, const T *__restrict__ V,
              T *__restrict__ O, float *__restrict__ LSE, float *__restrict__ part_o,
              float *__restrict__ part_lse, int H, int Hkv, int Nk, int G, int n_qgroups,
              int splits, int chunk, float scale, float scale_log2, PagedCache pc)
{
    using M = Mma16<T>;
    using v8 = typename M::v8;
    using Geo = DecodeGeo<D>;
    constexpr int NP = Geo::NP, KT = Geo::KT, CPR = Geo::CPR, VCH = Geo::VCH, VS = Geo::VS;
    constexpr int kPolicy = STREAM ? kLoadStream : 0;  // cache policy of the K/V loads

    // Per-wave V slices and the end-of-sweep merge buffer are never live
    // together, so they share one LDS block (a barrier separates the uses).
    constexpr int VT_BYTES = NW * WK * VS * (int)sizeof(T);
    constexpr int SO_BYTES = NW * 16 * (D + 1) * (int)sizeof(float);
    __shared__ __attribute__((aligned(16))) unsigned char smem[VT_BYTES > SO_BYTES ? VT_BYTES : SO_BYTES];
    __shared__ float sm_m[NW][16], sm_l[NW][16];
    float(*sm_o)[16][D + 1] = reinterpret_cast<float(*)[16][D + 1]>(smem);

    const int tid = threadIdx.x;
    const int lane = tid & 63, c = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

    int split, qg, hk, b, nsp_b = splits;
    // paged, automatic splits: the batch's K and V bytes are known here, and a
    // large batch is streamed with the non-temporal policy like a large
    // contiguous cache (wave-uniform)
    bool stream_rt = false;
    if (PAGED && pc.auto_split) {
        // workgroup = (pair of the flattened (sequence, split) list, KV head,
        // query-head group); the chunk follows the batch's total length
        const int hq = Hkv * n_qgroups;
        const int cap = pc.max_pages * pc.page_size;
        long long tot = 0;
        const bool found = paged_auto_pair(pc.seq_lens, pc.B, cap, hq, kDecodeStep * Geo::NP, splits,
                                           (int)(blockIdx.x / (unsigned)hq), chunk, b, split, nsp_b, tot);
        stream_rt = __builtin_amdgcn_readfirstlane(
                        (int)(2.0 * (double)tot * Hkv * D * (double)sizeof(T) >= kStreamBytes)) != 0;
        // the same in every lane and wave: scalar values
        if (!__builtin_amdgcn_readfirstlane((int)found)) return;  // past the last pair (the grid is an upper bound)
        chunk = __builtin_amdgcn_readfirstlane(chunk);
        b = __builtin_amdgcn_readfirstlane(b);
        split = __builtin_amdgcn_readfirstlane(split);
        nsp_b = __builtin_amdgcn_readfirstlane(nsp_b);
        const int r = (int)(blockIdx.x % (unsigned)hq);
        hk = r / n_qgroups;
        qg = r - hk * n_qgroups;
        // one workgroup per sequence tells the merge how many splits it has
        if (pc.split_counts != nullptr && split == 0 && r == 0 && threadIdx.x == 0)
            pc.split_counts[b] = nsp_b;
    } else {
        split = (int)(blockIdx.x % (unsigned)splits);
        const int grp = (int)(blockIdx.x / (unsigned)splits);  // (b, hk, qg)
        qg = grp % n_qgroups;
        const int bk = grp / n_qgroups;                         // b * Hkv + hk
        hk = bk % Hkv;
        b = bk / Hkv;
    }
    const int h0 = hk * G + qg * 16;
    const int nq = min(16, G - qg * 16);  // real query heads in this group

    int nk_b = Nk;
    if (PAGED) nk_b = max(0, min(pc.seq_lens[b], pc.max_pages * pc.page_size));
    const int kbeg = split * chunk;
    // (automatic splits: the last split of a sequence takes what is left)
    const int kend = (PAGED && pc.auto_split && split == nsp_b - 1) ? nk_b : min(nk_b, kbeg + chunk);
    // Paged, split: a split wholly past this sequence's length writes nothing
    // (the merge reads only the splits that hold keys); split 0 always writes,
    // so an empty sequence still gets O = 0, LSE = -inf.  Uniform per workgroup.
    if (PAGED && splits > 1 && split > 0 && kbeg >= nk_b) return;
    const size_t kvoff = PAGED ? 0 : ((size_t)b * Hkv + hk) * Nk * D;
    const T *Kb = K + kvoff;
    const T *Vb = V + kvoff;

    // q operand (B of S^T): lane (c, g) holds q[h0 + c][32t + 8g + e]; padding
    // columns c >= nq repeat the last real head and are never written out.
    v8 qop[KT];
    const int qh = h0 + min(c, nq - 1);
#pragma unroll
    for (int t = 0; t < KT; ++t)
        qop[t] = bitcast<v8>(*reinterpret_cast<const u32x4_t *>(Qg + ((size_t)b * H + qh) * D + 32 * t + 8 * g));

    // Per-lane byte offsets within one wave's 32 keys of a step.
    int koff[2][KT], voff[VCH], vst[VCH];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int t = 0; t < KT; ++t)
            koff[kb][t] = ((16 * kb + c) * D + 32 * t + 8 * g) * (int)sizeof(T);
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
        const int ci = lane + 64 * u, key = ci / CPR, cc = ci % CPR;
        voff[u] = (key * D + 8 * cc) * (int)sizeof(T);
        vst[u] = key * VS + 8 * cc;
    }
    // ds_read_b64_tr_b16 addresses: 16-lane group g reads keys kb + (c / 4)
    // (kb = 4g, then 16 + 4g) and columns 16 mb + 4 (c % 4).
    T *vt = reinterpret_cast<T *>(smem) + w * WK * VS;
    const int tr0 = (4 * g + c / 4) * VS + 4 * (c % 4);

    u32x4_t kreg[NP][2][KT], vreg[NP][VCH];
    // Paged: a window of the block table in one register, lane l holding the
    // physical page of logical page tab_win + l of this sequence (read once,
    // refreshed every 64 pages), so a stage's addresses need no dependent
    // scalar load.  Entries past the table are clamped to its last one.
    int tab_win = 0, tab = 0;
    auto tab_load = [&](int first) {
        tab_win = first;
        tab = pc.block_table[(size_t)b * pc.max_pages + min(first + lane, pc.max_pages - 1)];
    };
    if (PAGED) tab_load(min(kbeg / pc.page_size, pc.max_pages - 1));
    const int nsteps = kend > kbeg ? (kend - kbeg + kDecodeStep - 1) / kDecodeStep : 0;
    auto load_step = [&](int sp, int st) {
        const int rel = st * kDecodeStep + w * WK;  // first key of this wave's 32, in the slice
        long long left = (long long)(kend - kbeg - rel) * D * (long long)sizeof(T);
        size_t row0 = (size_t)(kbeg + rel) * D;  // element offset of the block's first key
        if (PAGED) {
            // wave-uniform: one table entry per 32-key block, from the window
            const int t = kbeg + rel;
            const int pidx = min(t / pc.page_size, pc.max_pages - 1);
            if (pidx - tab_win >= 64) tab_load(pidx);
            const int phys = __builtin_amdgcn_readlane(tab, pidx - tab_win);
            const int in_page = t - pidx * pc.page_size;
            const bool ok = t < kend && (unsigned)phys < (unsigned)pc.num_pages;
            left = ok ? (long long)min(kend - t, pc.page_size - in_page) * D * (long long)sizeof(T) : 0;
            row0 = ok ? ((size_t)phys * Hkv + hk) * pc.page_size * D + (size_t)in_page * D : 0;
        }
        const __amdgpu_buffer_rsrc_t rk = span_rsrc(Kb + row0, left);
        const __amdgpu_buffer_rsrc_t rv = span_rsrc(Vb + row0, left);
        if (PAGED && stream_rt) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int t = 0; t < KT; ++t)
                    kreg[sp][kb][t] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff[kb][t], 0, kLoadStream);
#pragma unroll
            for (int u = 0; u < VCH; ++u)
                vreg[sp][u] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff[u], 0, kLoadStream);
        } else {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int t = 0; t < KT; ++t)
                    kreg[sp][kb][t] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff[kb][t], 0, kPolicy);
#pragma unroll
            for (int u = 0; u < VCH; ++u)
                vreg[sp][u] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff[u], 0, kPolicy);
        }
        // keep the stages' loads in issue order, so the wait for the oldest
        // stage leaves the younger ones in flight
        __builtin_amdgcn_sched_barrier(0);
    };

    f32x4_t acc[D / 16];
#pragma unroll
    for (int i = 0; i < D / 16; ++i) acc[i] = f32x4_t{};
    float m_run = -INFINITY, l_run = 0.f;

#pragma unroll
    for (int sp = 0; sp < NP; ++sp) load_step(sp, sp);
    // wait for q only now: the KV prefetches above are already in flight
    settle(qop);

    // At least one round, also for an empty slice (its keys are all masked):
    // with no guard around the loop the prologue loads stay where they are,
    // ahead of the wait for q.
    const int nround = max(1, (nsteps + NP - 1) / NP);
    int r = 0;
    do {
#pragma unroll
        for (int sp = 0; sp < NP; ++sp) {
            const int st = r * NP + sp;
            const int base = kbeg + st * kDecodeStep + w * WK;  // first key of this wave's 32

            // V rows into this wave's LDS slice, row-major
#pragma unroll
            for (int u = 0; u < VCH; ++u) *reinterpret_cast<u32x4_t *>(vt + vst[u]) = vreg[sp][u];

            // S^T for this wave's 32 keys
            f32x4_t s[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                s[kb] = f32x4_t{};
#pragma unroll
                for (int t = 0; t < KT; ++t)
                    s[kb] = M::mma16(bitcast<v8>(kreg[sp][kb][t]), qop[t], s[kb]);
            }
            // the stage's registers are consumed: prefetch step st + NP into them
            load_step(sp, st + NP);

            if (base + WK > kend) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (base + 16 * kb + 4 * g + q >= kend) s[kb][q] = -INFINITY;
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int q = 0; q < 4; ++q) mx = fmaxf(mx, s[kb][q]);
            mx = max_xor16(mx);
            mx = max_xor32(mx);
            const float m_new = fmaxf(m_run, mx);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float mneg = -m_use * scale_log2;
            // Rescale only when some row's max moved: otherwise alpha is
            // exactly 1, and after the first steps the max rarely moves.
            float alpha = 1.f;
            if (__builtin_amdgcn_ballot_w64(m_new != m_run) != 0) {
                alpha = fast_exp2((m_run - m_use) * scale_log2);
#pragma unroll
                for (int i = 0; i < D / 16; ++i) acc[i] *= alpha;
            }
            float rs = 0.f;
            v8 pop;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float p = fast_exp2(fmaf(s[kb][q], scale_log2, mneg));
                    rs += p;
                    pop[4 * kb + q] = static_cast<T>(p);
                }
            l_run = l_run * alpha + rs;
            m_run = m_new;

            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int mb = 0; mb < D / 16; ++mb) {
                const u32x2_t a = read_tr(vt + tr0 + 16 * mb);
                const u32x2_t bq = read_tr(vt + tr0 + 16 * VS + 16 * mb);
                acc[mb] = M::mma16(bitcast<v8>(u32x4_t{a.x, a.y, bq.x, bq.y}), pop, acc[mb]);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    } while (++r < nround);

    // ---- merge the 4 waves of this workgroup ----
    float l = sum_xor16(l_run);
    l = sum_xor32(l);
    __syncthreads();  // every wave is done with its V slice (sm_o aliases it)
    if (g == 0) {
        sm_m[w][c] = m_run;
        sm_l[w][c] = l;
    }
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb)
#pragma unroll
        for (int q = 0; q < 4; ++q) sm_o[w][c][16 * mb + 4 * g + q] = acc[mb][q];
    __syncthreads();

    const int qi = tid >> 4;          // query head slot 0..15
    const int dl = tid & 15;          // this thread covers d = dl + 16 i
    float ov[D / 16];
    float lse_wg = -INFINITY;
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
#pragma unroll
        for (int i = 0; i < D / 16; ++i) {
            float o = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) o += wt[ww] * sm_o[ww][qi][dl + 16 * i];
            ov[i] = o * inv;
        }
        lse_wg = L > 0.f ? M_ * scale + logf(L) : -INFINITY;
    }

    const size_t bh = (size_t)b * H + h0 + qi;
    if (splits == 1) {  // the workgroup saw every key: its result is final
        if (qi < nq) {
#pragma unroll
            for (int i = 0; i < D / 16; ++i) O[bh * D + dl + 16 * i] = static_cast<T>(ov[i]);
            if (LSE != nullptr && dl == 0) LSE[bh] = lse_wg;
        }
        return;
    }

    if (qi < nq) {
        const size_t prow = bh * splits + split;
#pragma unroll
        for (int i = 0; i < D / 16; ++i) part_o[prow * D + dl + 16 * i] = ov[i];
        if (dl == 0) part_lse[prow] = lse_wg;
    }
}

// One wave per (b, h); lane d accumulates output column d (and d + 64).
// The per-split LSEs are wave-uniform, so every lane reads all of them
// (scalar loads) and no cross-lane reduction is needed; the partial rows are
// loaded in batches of JB (addresses clamped to the last split read, surplus
// rows weighted 0), the first batch before the LSEs are even looked at.  For
// a paged cache only the splits that hold keys of the sequence are read (the
// sweep skips the others without writing).
template <typename T, int D>
__global__ void __launch_bounds__(256)
decode_merge_kernel(const float *__restrict__ part_o, const float *__restrict__ part_lse,
                    T *__restrict__ O, float *__restrict__ LSE, int BH, int splits,
                    const int *__restrict__ seq_lens, int H, int chunk, int cap,
                    const int *__restrict__ split_counts)
{
    constexpr int DPL = D / 64;  // output columns per lane
    constexpr int JB = 16;
    const int lane = threadIdx.x & 63;
    const int bh = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (bh >= BH) return;
    // paged: only the splits that hold keys of this sequence were written
    int nsp = splits;
    if (split_counts != nullptr) {  // automatic splits: as the sweep recorded them
        nsp = max(1, min(splits, split_counts[bh / H]));
    } else if (seq_lens != nullptr) {
        const int len = max(0, min(seq_lens[bh / H], cap));
        nsp = max(1, min(splits, (len + chunk - 1) / chunk));
    }
    const float *pl = part_lse + (size_t)bh * splits;
    const float *po = part_o + (size_t)bh * splits * D + lane;

    float vb[JB][DPL];
    auto load_batch = [&](int s1) {
#pragma unroll
        for (int j = 0; j < JB; ++j) {
            const int sj = min(s1 + j, nsp - 1);
#pragma unroll
            for (int i = 0; i < DPL; ++i) vb[j][i] = po[(size_t)sj * D + 64 * i];
        }
    };
    load_batch(0);
    float M_ = -INFINITY;
    for (int s = 0; s < nsp; s += 8) {
#pragma unroll
        for (int j = 0; j < 8; ++j) M_ = fmaxf(M_, pl[min(s + j, nsp - 1)]);
    }
    float acc[DPL], L = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
    if (M_ != -INFINITY) {
        for (int s0 = 0; s0 < nsp; s0 += JB) {
            if (s0 > 0) load_batch(s0);
#pragma unroll
            for (int j = 0; j < JB; ++j) {
                const int sj = s0 + j;
                const float wj = sj < nsp ? fast_exp2((pl[min(sj, nsp - 1)] - M_) * kLog2e) : 0.f;
                L += wj;
#pragma unroll
                for (int i = 0; i < DPL; ++i) acc[i] += wj * vb[j][i];
            }
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) O[(size_t)bh * D + lane + 64 * i] = static_cast<T>(acc[i] * inv);
    if (LSE != nullptr && lane == 0) LSE[bh] = (M_ == -INFINITY) ? -INFINITY : M_ + logf(L);
}

// Merge for many splits (more than kMergeNarrow): one round of vector loads
// per JB partials -- lane j reads the LSE of split s0 + j, and every lane
// reads its output columns of all JB partial rows -- instead of scalar loads
// that depend on each other.  The split weights reach every lane by readlane;
// a further round (more than JB splits) folds in with a running reference
// M_, rescaling what is already summed by e^(M_old - M_new).
constexpr int kMergeNarrow = 16;

template <typename T, int D>
__global__ void __launch_bounds__(256)
decode_merge_wide_kernel(const float *__restrict__ part_o, const float *__restrict__ part_lse,
                         T *__restrict__ O, float *__restrict__ LSE, int BH, int splits,
                         const int *__restrict__ seq_lens, int H, int chunk, int cap,
                         const int *__restrict__ split_counts)
{
    constexpr int DPL = D / 64;    // output columns per lane
    constexpr int JB = 64 / DPL;   // partial rows per round of loads
    const int lane = threadIdx.x & 63;
    const int bh = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (bh >= BH) return;
    int nsp = splits;
    if (split_counts != nullptr) {
        nsp = max(1, min(splits, split_counts[bh / H]));
    } else if (seq_lens != nullptr) {
        const int len = max(0, min(seq_lens[bh / H], cap));
        nsp = max(1, min(splits, (len + chunk - 1) / chunk));
    }
    const float *pl = part_lse + (size_t)bh * splits;
    const float *po = part_o + (size_t)bh * splits * D + lane;

    float M_ = -INFINITY, L = 0.f, acc[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
    for (int s0 = 0; s0 < nsp; s0 += JB) {
        const int n = min(JB, nsp - s0);
        const float lj = lane < n ? pl[s0 + lane] : -INFINITY;
        float vb[JB][DPL];
#pragma unroll
        for (int j = 0; j < JB; ++j) {
            const int sj = s0 + min(j, n - 1);
#pragma unroll
            for (int i = 0; i < DPL; ++i) vb[j][i] = po[(size_t)sj * D + 64 * i];
        }
        float mb = lj;
        mb = wave_max_f32(mb);
        const float Mn = fmaxf(M_, mb);
        if (Mn == -INFINITY) continue;  // every split so far empty (wave-uniform)
        const float a = fast_exp2((M_ - Mn) * kLog2e);  // 0 while M_ = -inf
        L *= a;
#pragma unroll
        for (int i = 0; i < DPL; ++i) acc[i] *= a;
        const float wl = lane < n ? fast_exp2((lj - Mn) * kLog2e) : 0.f;
        float ws = wl;
        ws = wave_sum_f32(ws);
        L += ws;
#pragma unroll
        for (int j = 0; j < JB; ++j) {
            const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j));
#pragma unroll
            for (int i = 0; i < DPL; ++i) acc[i] += wj * vb[j][i];
        }
        M_ = Mn;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) O[(size_t)bh * D + lane + 64 * i] = static_cast<T>(acc[i] * inv);
    if (LSE != nullptr && lane == 0) LSE[bh] = (M_ == -INFINITY) ? -INFINITY : M_ + logf(L);
}

template <typename T, int D>
hipError_t launch_t(const DecodeProblem &p, hipStream_t st)
{
    const int G = p.H / p.Hkv;
    const int n_qgroups = (G + 15) / 16;
    const int hq = p.Hkv * n_qgroups;
    const bool auto_split = p.block_table != nullptr && p.auto_split;
    const unsigned n_blocks = auto_split ? (unsigned)(paged_auto_pairs(p.B, hq, p.splits) * hq)
                                         : (unsigned)p.splits * (unsigned)(p.B * hq);
    const PagedCache pc{p.block_table, p.seq_lens, p.page_size, p.max_pages, p.num_pages,
                        auto_split ? 1 : 0, p.B, auto_split ? p.split_counts : nullptr};
    // stream a large contiguous cache past the caches (small ones keep the
    // default policy; a paged batch decides on the device from its lengths)
    const bool stream = p.block_table == nullptr &&
                        2.0 * p.B * p.Hkv * (double)p.Nk * D * sizeof(T) >= (double)kStreamBytes;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(n_blocks), dim3(256), 0, st, static_cast<const T *>(p.q),
                           static_cast<const T *>(p.k), static_cast<const T *>(p.v),
                           static_cast<T *>(p.o), p.lse, p.part_o, p.part_lse, p.H, p.Hkv, p.Nk, G,
                           n_qgroups, p.splits, p.chunk, p.scale, p.scale * kLog2e, pc);
    };
    if (p.block_table != nullptr) go(decode_kernel<T, D, true, false>);
    else if (stream) go(decode_kernel<T, D, false, true>);
    else go(decode_kernel<T, D, false, false>);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    const int BH = p.B * p.H;
    auto merge = p.splits > kMergeNarrow ? decode_merge_wide_kernel<T, D> : decode_merge_kernel<T, D>;
    hipLaunchKernelGGL(merge, dim3((unsigned)((BH + 3) / 4)), dim3(256), 0, st, p.part_o,
                       p.part_lse, static_cast<T *>(p.o), p.lse, BH, p.splits,
                       p.block_table != nullptr ? p.seq_lens : nullptr, p.H, p.chunk,
                       p.max_pages * p.page_size, auto_split ? p.split_counts : nullptr);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_dt(const DecodeProblem &p, hipStream_t st)
{
    return p.d == 64 ? launch_t<T, 64>(p, st) : launch_t<T, 128>(p, st);
}

// Scratch of fa_decode_noalloc: the per-split partials (the workspace of
// fa_decode) in a static device array, so that entry point allocates
// nothing.  Each GPU holds its own copy for the life of the process.  In host
// code the array's name is only a stand-in for the symbol: its device address
// comes from hipGetSymbolAddress, looked up once per device.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

}  // namespace

hipError_t decode_scratch(void **ptr)
{
    constexpr int kMaxDevices = 64;
    static std::once_flag once[kMaxDevices];
    static void *addr[kMaxDevices];
    static hipError_t err[kMaxDevices];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(once[dev], [dev]() {
        void *p = nullptr;
        err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        addr[dev] = err[dev] == hipSuccess ? p : nullptr;
    });
    *ptr = addr[dev];
    return err[dev];
}

int decode_chunk_keys(int d) { return kDecodeStep * (d == 64 ? DecodeGeo<64>::NP : DecodeGeo<128>::NP); }

hipError_t launch_decode(const DecodeProblem &p, hipStream_t st)
{
    return p.dtype == 2 ? launch_dt<__bf16>(p, st) : launch_dt<_Float16>(p, st);
}

}  // namespace fa
