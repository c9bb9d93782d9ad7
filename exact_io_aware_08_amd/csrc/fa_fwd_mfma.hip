// fa_fwd_mfma.hip -- forward (prefill) attention on bf16/fp16 MFMA, gfx950.
//
// Method: marketmaker.cc blog "Atencion flash y la pregunta sobre la longitud
// de la secuencia", sections "El algoritmo de atencion flash" (Q split into
// row blocks, K/V into column blocks, each query block sweeps the KV blocks
// keeping a running max m, running sum l and an output accumulator) and
// "La recurrencia de softmax en linea" (the accumulator is rescaled by
// e^(m_old - m_new) when the reference max grows; the result is a
// reassociation of the two-pass softmax); "FA2: paralelismo" (normalisation
// deferred to the end; the grid also runs over query blocks; each wave owns
// whole query rows); "FA3: Mecanica de la tolva", item 2 (the score matmul of
// one block runs while the softmax of the previous block runs on the other
// unit); "El enmascaramiento causal ..." (KV tiles wholly in the future are
// never loaded or computed).  systems-analysis.info "FlashAttention (IT)",
// "Innovazioni chiave": one fused kernel that writes only O (and the LSE).
//
// gfx950 mapping (one workgroup = 4 waves; each wave owns QB blocks of 32
// query rows of one (b, h); a KV tile has NKB blocks of 32 keys; QB*NKB = 2
// score blocks per wave at d = 64, one at d = 128, where a 32-key tile keeps
// the LDS of a workgroup at 48 KB and the registers under 256, so two waves
// share each SIMD; at d = 256 a workgroup has 8 waves and two waves share
// each query block, each holding the Q operand and O accumulator of one
// half of d and exchanging partial scores through LDS once per tile):
//  * Scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16:
//    the fp32 result gives lane l the 16 keys {8i + 4(l/32) + r} of query
//    l%32 per 32x32 block, so a row's max needs one v_permlane32_swap and
//    its sum no exchange until the epilogue.
//  * The S^T accumulator is directly the B operand of O^T = V^T P^T (after
//    v_cvt_pk to bf16/fp16): key-slot k of lane group g in K-step t is key
//    16t + 8(k/4) + 4g + k%4 of the 32-key block.  K and V are both staged
//    row-major ([key][d]) with one 16-byte store per chunk; K is read as
//    16-byte A-operand rows, and the V^T operand comes from two
//    ds_read_b64_tr_b16 (within a 16-lane group, lane s gives the address of
//    row r0 + s/4, columns c0 + 4(s%4)..+3, and lane i receives column
//    c0 + i of rows r0..r0+3 -- four consecutive keys of one d).  Q stays in
//    registers for the whole sweep.
//  * Every K and V^T operand read from LDS feeds all QB query blocks of the
//    wave, so LDS traffic per MFMA falls as QB grows (QB = 2 at d = 64,
//    where it is what bounds the loop; QB = 1 at d = 128 for registers).
//  * Pipeline with one barrier per KV tile: K is staged one tile ahead of V
//    (both double-buffered in LDS) and global loads run two tiles ahead, so
//    in iteration j the wave issues the S^T MFMAs of tile j+1 interleaved
//    with the softmax of tile j on the VALU, then the P V MFMAs of tile j
//    interleaved with staging the next tiles.
//  * Global loads are buffer loads with the descriptor rebased per tile:
//    rows past the end of a slice read as zero (hardware range check), so
//    ragged tails need no address clamping on the VALU.
//  * The reference max of each row is the exact max of its first tile; it
//    is moved (with the e^(m_old - m_new) rescale) only when a later tile's
//    exponentials leave a safe range, detected from that tile's row sums.
//    In exact arithmetic any reference value gives the same O and LSE, and
//    the per-tile row max and rescale stay off the common path.
//  * Causal grids run the longest query tiles first.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

// Row-sum accumulation of one converted pair of probabilities.  For fp16
// the sum is taken over the converted values with v_dot2 (an 11-bit
// mantissa keeps the normaliser within 2^-12 relative); bf16 keeps only 8
// bits, which would move the LSE by up to 2^-9, so its sum adds the fp32
// values.
template <typename T> struct Pack2;
template <> struct Pack2<__bf16> {
    typedef __bf16 v2 __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ float add(v2, float p0, float p1, float c) {
        return c + p0 + p1;
    }
    // the first pair of a sum (p0 >= 0, so this equals 0 + p0 + p1)
    static __device__ __forceinline__ float first(v2, float p0, float p1) { return p0 + p1; }
};
template <> struct Pack2<_Float16> {
    typedef _Float16 v2 __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ float add(v2 a, float, float, float c) {
        const v2 one = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(a, one, c, false);
    }
    static __device__ __forceinline__ float first(v2 a, float p0, float p1) {
        return add(a, p0, p1, 0.f);
    }
};

// Geometry for head dim D and QB query blocks per wave.
template <int D, int QB> struct Geo {
    // d = 256: two waves share each query block, each holding the Q operand
    // and the O accumulator of one half of d (DS = 2), so a wave fits in 256
    // registers and two waves share each SIMD.
    static constexpr int DS = D >= 256 ? 2 : 1;  // waves per query block
    static constexpr int DW = D / DS;            // head-dim columns per wave
    static constexpr int NW = 4 * DS;            // waves per workgroup
    static constexpr int NT = 64 * NW;           // threads per workgroup
    static constexpr int NKB = (QB >= 2 || D >= 128) ? 1 : 2;  // 32-key blocks per KV tile
    // (d = 128 with 64-key tiles needed 96 KB of LDS: one workgroup, one wave
    //  per SIMD, 1.5x slower than two waves with 32-key tiles)
    static constexpr int NSB = QB * NKB;         // 32x32 score blocks per wave
    static constexpr int BC = 32 * NKB;          // keys per KV tile
    static constexpr int BR = 4 * 32 * QB;       // queries per workgroup
    static constexpr int KSTR = D + 8;           // K tile row stride in LDS (elements)
    // V tile row stride in LDS (elements): 48 dwords at d = 64, 80 at d =
    // 128, 144 at d = 256, i.e. 16 (mod 32) banks apart per row, so the four
    // rows times four 8-byte column chunks that a half-wave's transpose read
    // touches fall in distinct banks.
    static constexpr int VS = D == 64 ? 96 : D == 128 ? 160 : 288;
    static constexpr int CPR = D / 8;            // 16-byte chunks per K/V row
    static constexpr int KCH = BC * CPR / NT;    // K (and V) chunks per thread per tile
    static_assert(KCH >= 1 && KCH * NT == BC * CPR, "staging split");
    static_assert(DS == 1 || NSB == 1, "d split with one score block per wave");
    static_assert(VS >= D && (VS * 2) % 16 == 0, "V row stride");
};

// Per-thread offsets of the staging loads and LDS stores within a tile:
// chunk ci = tid + NT r -> row ci / CPR, chunk ci % CPR (row-major,
// coalesced).  K and V use the same map, with their own LDS row strides.
template <int D, int QB> struct KvMap {
    using G = Geo<D, QB>;
    int off[G::KCH];  // byte offsets of the chunks in global memory
    int kst[G::KCH];  // LDS element offsets in the K tile
    int vst[G::KCH];  // LDS element offsets in the V tile
    __device__ __forceinline__ KvMap(int tid, int elem_bytes) {
#pragma unroll
        for (int r = 0; r < G::KCH; ++r) {
            const int ci = tid + r * G::NT;
            off[r] = ((ci / G::CPR) * D + (ci % G::CPR) * 8) * elem_bytes;
            kst[r] = (ci / G::CPR) * G::KSTR + (ci % G::CPR) * 8;
            vst[r] = (ci / G::CPR) * G::VS + (ci % G::CPR) * 8;
        }
    }
};

template <typename T, int D, int QB>
__device__ __forceinline__ void load_rows(__amdgpu_buffer_rsrc_t rs, const KvMap<D, QB> &mp,
                                          u32x4_t (&reg)[Geo<D, QB>::KCH])
{
#pragma unroll
    for (int r = 0; r < Geo<D, QB>::KCH; ++r)
        reg[r] = __builtin_amdgcn_raw_buffer_load_b128(rs, mp.off[r], 0, 0);
}

// Registers -> LDS, row-major [key][d] (K and V alike; V is read back
// transposed by ds_read_b64_tr_b16).
template <typename T, int D, int QB>
__device__ __forceinline__ void store_rows(T *buf, const int (&st)[Geo<D, QB>::KCH],
                                           const u32x4_t (&reg)[Geo<D, QB>::KCH])
{
#pragma unroll
    for (int r = 0; r < Geo<D, QB>::KCH; ++r) *reinterpret_cast<u32x4_t *>(&buf[st[r]]) = reg[r];
}

// S^T blocks (32 keys x 32 queries each) = K_tile Q_wave^T over the wave's
// head-dim columns [dbase, dbase + DW); block index qb * NKB + kb.  Each K
// operand read serves all QB query blocks.
template <typename T, int D, int QB>
__device__ __forceinline__ void scores(const T *Ks,
                                       const typename Mma16<T>::v8 (&qop)[QB][Geo<D, QB>::DW / 16],
                                       int c, int hh, int dbase, f32x16_t (&s)[Geo<D, QB>::NSB])
{
    using M = Mma16<T>;
    using v8 = typename M::v8;
    using G = Geo<D, QB>;
#pragma unroll
    for (int i = 0; i < G::NSB; ++i) s[i] = f32x16_t{};
#pragma unroll
    for (int kb = 0; kb < G::NKB; ++kb)
#pragma unroll
        for (int t = 0; t < G::DW / 16; ++t) {
            const v8 kop = *reinterpret_cast<const v8 *>(&Ks[(kb * 32 + c) * G::KSTR + dbase + 16 * t + 8 * hh]);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[qb * G::NKB + kb] = M::mma32(kop, qop[qb][t], s[qb * G::NKB + kb]);
        }
}

// Max / sum over the two lanes (l, l^32) that hold one query row.
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

template <typename T, int D, int QB, bool CAUSAL>
__global__ void __launch_bounds__((Geo<D, QB>::NT), (QB >= 3 ? 1 : 2))
fwd_mfma_kernel(const T *__restrict__ Q, const T *__restrict__ K, const T *__restrict__ V,
                T *__restrict__ O, float *__restrict__ LSE, int H, int Hkv, int Nq, int Nk,
                int n_bh, int n_qtiles, float scale, float scale_log2)
{
    using M = Mma16<T>;
    using v8 = typename M::v8;
    using P2 = Pack2<T>;
    using G = Geo<D, QB>;
    constexpr int BC = G::BC, NKB = G::NKB, VS = G::VS, NSB = G::NSB, DS = G::DS, DW = G::DW;

    __shared__ __attribute__((aligned(16))) T Kbuf[2][BC * G::KSTR];
    __shared__ __attribute__((aligned(16))) T Vbuf[3][BC * VS];  // tile i in Vbuf[i % 3]
    // d split: partial S^T exchange between the two waves of a query block,
    // [tile parity][wave][register quad][lane] (one float4 per lane each)
    __shared__ f32x4_t xbuf[DS > 1 ? 2 * G::NW * 4 * 64 : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63, c = lane & 31, hh = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    const int wq = w / DS;                                   // query block of this wave
    const int dbase = (w % DS) * DW;                         // its first head-dim column

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

    const int q0 = qt * G::BR;
    const int q0w = q0 + wq * 32 * QB;  // first row of this wave
    const int off = Nk - Nq;
    int nkt = (Nk + BC - 1) / BC;
    if (CAUSAL) {
        const int lim = min(q0 + G::BR, Nq) - 1 + off;  // last key any row of the block sees
        nkt = lim < 0 ? 0 : min(nkt, lim / BC + 1);
    }

    // Q operand (B of S^T = K Q^T): lane (c, hh) holds
    // Q[q0w + 32qb + c][dbase + 16t + 8hh + e].  Rows past Nq read as zeros
    // (buffer range check); they are never stored.
    v8 qop[QB][DW / 16];
    {
        const __amdgpu_buffer_rsrc_t rq = rows_rsrc<T, D>(Qb, Nq, q0w);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
            for (int t = 0; t < DW / 16; ++t)
                qop[qb][t] = bitcast<v8>(__builtin_amdgcn_raw_buffer_load_b128(
                    rq, ((32 * qb + c) * D + dbase + 16 * t + 8 * hh) * (int)sizeof(T), 0, 0));
            settle(qop[qb]);
        }
    }

    f32x16_t acc[QB][DW / 32];  // O^T rows dbase + 32 i + (register layout)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int i = 0; i < DW / 32; ++i) acc[qb][i] = f32x16_t{};
    float m_ref[QB], l_run[QB];  // reference max (raw units; same in lanes l, l^32), row-sum share
    float mneg[QB];              // -m_ref * scale * log2(e), 0 while m_ref = -inf
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_ref[qb] = -INFINITY;
        l_run[qb] = 0.f;
        mneg[qb] = 0.f;
    }
    auto set_mneg = [&](int qb) {
        mneg[qb] = (m_ref[qb] == -INFINITY) ? 0.f : -m_ref[qb] * scale_log2;
    };

    const KvMap<D, QB> mp(tid, (int)sizeof(T));
    // Transpose-read address of this lane within a V tile: 16-lane group
    // (hh, c / 16) reads rows 4hh + (lane % 16) / 4 (+ the K-step's first
    // key) and columns 16 (c / 16) + 4 (lane % 16 % 4) (+ 32 mb).
    const int tr_off = (4 * hh + ((lane & 15) >> 2)) * VS + 16 * (c >> 4) + 4 * (lane & 3);
    u32x4_t kreg[G::KCH], vreg[G::KCH];
    f32x16_t s_a[NSB], s_b[NSB];
    v8 p_a[NSB][2], p_b[NSB][2];  // P^T operands [score block][K-step] of two consecutive tiles
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int t = 0; t < 2; ++t) p_a[sb][t] = bitcast<v8>(u32x4_t{0u, 0u, 0u, 0u});
    auto tile = [&](int jj) { return min(jj, nkt - 1) * BC; };  // clamped first key of a tile

    // d split: publish this wave's partial S^T of a tile, and add the other
    // wave's (same lane layout; x + y == y + x, so both waves then hold the
    // same scores bit for bit and take the same softmax decisions).  Buffer
    // tile & 1 is written before the barrier that ends the previous step and
    // read after it; its next write comes after the following barrier.
    auto x_put = [&](int par, const f32x16_t (&sp)[NSB]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            xbuf[((par * G::NW + w) * 4 + i) * 64 + lane] =
                f32x4_t{sp[0][4 * i], sp[0][4 * i + 1], sp[0][4 * i + 2], sp[0][4 * i + 3]};
    };
    auto x_add = [&](int par, f32x16_t (&sp)[NSB]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4_t o = xbuf[((par * G::NW + (w ^ 1)) * 4 + i) * 64 + lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) sp[0][4 * i + e] += o[e];
        }
    };

    if (nkt > 0) {
        // prologue: K0 -> Kbuf[0], V0 -> Vbuf[0], K1 -> Kbuf[1]; registers
        // then hold K2 and V1.  Vbuf[2] stands for tile -1, whose (zero) P
        // is multiplied in the first step: it must hold finite values.
        load_rows<T, D, QB>(rows_rsrc<T, D>(Kb, Nk, 0), mp, kreg);
        load_rows<T, D, QB>(rows_rsrc<T, D>(Vb, Nk, 0), mp, vreg);
        for (int i = tid; i < BC * VS / 8; i += G::NT)
            reinterpret_cast<u32x4_t *>(Vbuf[2])[i] = u32x4_t{0u, 0u, 0u, 0u};
        store_rows<T, D, QB>(Kbuf[0], mp.kst, kreg);
        store_rows<T, D, QB>(Vbuf[0], mp.vst, vreg);
        load_rows<T, D, QB>(rows_rsrc<T, D>(Kb, Nk, tile(1)), mp, kreg);
        load_rows<T, D, QB>(rows_rsrc<T, D>(Vb, Nk, tile(1)), mp, vreg);
        store_rows<T, D, QB>(Kbuf[1], mp.kst, kreg);
        load_rows<T, D, QB>(rows_rsrc<T, D>(Kb, Nk, tile(2)), mp, kreg);
        lds_barrier();
        scores<T, D, QB>(Kbuf[0], qop, c, hh, dbase, s_a);
        if (DS > 1) x_put(0, s_a);
        lds_barrier();  // Kbuf[0] is overwritten in iteration 0
    }

    // O^T += V^T P^T for one tile whose V is in Vs (transpose reads).
    auto pv = [&](const T *Vs, const v8 (&pp)[NSB][2]) {
        Vs += tr_off;
#pragma unroll
        for (int mb = 0; mb < DW / 32; ++mb)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    // K-slots 0-3: keys 16t + 4hh + 0..3, slots 4-7: 16t + 8 + 4hh + 0..3
                    // (of block kb), column d = dbase + 32 mb + c: the S^T register order.
                    const T *vp = Vs + (kb * 32 + 16 * t) * VS + dbase + 32 * mb;
                    const u32x2_t lo = read_tr(vp);
                    const u32x2_t hi = read_tr(vp + 8 * VS);
                    const v8 vop = bitcast<v8>(u32x4_t{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        acc[qb][mb] = M::mma32(vop, pp[qb * NKB + kb][t], acc[qb][mb]);
                }
    };

    // One KV tile.  Invariant on entry: sc = S^T of tile j; pp = P of tile
    // j-1 (zero for j = 0); Kbuf[(j+1)&1] = K_{j+1}; Vbuf[(j-1)%3] = V_{j-1},
    // Vbuf[j%3] = V_j; kreg = K_{j+2}; vreg = V_{j+1} (tile indices past the
    // last tile are clamped to it; those copies go to buffers that are never
    // read again).  The product with V of tile j is deferred to step j+1, so
    // every step interleaves 16 MFMAs (S^T of tile j+1 and P V of tile j-1)
    // with the softmax of tile j on the VALU.  The staging is branch-free,
    // so the only waits on global loads are for data requested a full tile
    // earlier.  Tiles past a wave's causal limit are processed fully masked
    // (weight 0), which keeps the hot block free of branches.
    // The three V buffers rotate through element offsets held in scalar
    // registers: vo_prev = V_{j-1}, vo_cur = V_j, vo_next = V_{j+1} at step j.
    constexpr int VSZ = BC * VS;
    int vo_prev = 2 * VSZ, vo_cur = 0, vo_next = VSZ;
    T *const Vb0 = &Vbuf[0][0];
    auto step = [&](int j, f32x16_t (&sc)[NSB], f32x16_t (&sn)[NSB], const v8 (&pp)[NSB][2],
                    v8 (&pc)[NSB][2]) {
        const int j0 = j * BC;
        if (DS > 1) x_add(j & 1, sc);  // full S^T of tile j
        // ---- mask: ragged last tile, the diagonal band and beyond (causal) ----
        const bool need_mask = (j0 + BC > Nk) || (CAUSAL && j0 + BC - 1 > q0w + off);
        if (need_mask) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int lim = CAUSAL ? min(Nk, q0w + 32 * qb + c + off + 1) : Nk;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = j0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                        if (key >= lim) sc[qb * NKB + kb][r] = -INFINITY;
                    }
            }
        }

        // ---- reference max ----
        // A row takes the exact max of its first tile with a visible key as
        // its reference.  Afterwards the reference only moves when a tile's
        // exponentials leave the safe range, which the row sums below
        // detect; the per-tile row max is then never computed on the common
        // path.  Any finite reference gives the same O and LSE.
        auto tile_max = [&](int qb) {
            float m = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) m = fmaxf(m, sc[qb * NKB + kb][r]);
            return max_pair(m);
        };
        // Rows without a reference yet have no weight in acc or l, so setting
        // theirs needs no rescale (and commutes with the deferred P V).
        bool fresh = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) fresh |= (m_ref[qb] == -INFINITY);
        if (__builtin_amdgcn_ballot_w64(fresh) != 0) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float m = tile_max(qb);
                m_ref[qb] = m_ref[qb] == -INFINITY ? m : m_ref[qb];
                set_mneg(qb);
            }
        }
        // Any row: raise the reference to this tile's max, rescaling what
        // acc and l hold (everything up to tile j-1 -- the P V of tile j-1
        // is already in acc when this runs).
        auto rebase = [&]() {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float m = tile_max(qb);
                const bool raise = m > m_ref[qb];
                const float alpha = raise ? fast_exp2((m_ref[qb] - m) * scale_log2) : 1.f;
                m_ref[qb] = raise ? m : m_ref[qb];
                set_mneg(qb);
                l_run[qb] *= alpha;
#pragma unroll
                for (int i = 0; i < DW / 32; ++i) acc[qb][i] *= alpha;
            }
        };

        // P = exp2(s*c - m*c) packed to 16-bit, with this tile's row sums.
        float ts[QB];
        auto make_p = [&]() {
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int qb = sb / NKB;
                    typename P2::v2 pk[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float p0 = fast_exp2(fmaf(sc[sb][8 * t + 2 * e], scale_log2, mneg[qb]));
                        const float p1 = fast_exp2(fmaf(sc[sb][8 * t + 2 * e + 1], scale_log2, mneg[qb]));
                        pk[e] = __builtin_convertvector((f32x2_t{p0, p1}), typename P2::v2);
                        // keep each conversion here: without this the compiler
                        // sinks all of them past the range-check branch below,
                        // out of the MFMA-interleaved block
                        asm volatile("" : "+v"(pk[e]));
                        if (sb % NKB == 0 && t == 0 && e == 0) ts[qb] = P2::first(pk[e], p0, p1);
                        else ts[qb] = P2::add(pk[e], p0, p1, ts[qb]);
                    }
                    pc[sb][t] = bitcast<v8>(u32x4_t{bitcast<uint32_t>(pk[0]), bitcast<uint32_t>(pk[1]),
                                                    bitcast<uint32_t>(pk[2]), bitcast<uint32_t>(pk[3])});
                }
        };

        // ---- hot block: S^T of tile j+1 and P V of tile j-1 on the MFMA
        //      pipe while the VALU turns tile j into P.  It runs at raised
        //      wave priority, so the other wave on the SIMD (another
        //      workgroup) issues its staging, masking and barrier work in the
        //      hot block's gaps rather than ahead of it (about 1.5% faster on
        //      the trading-day prefill) ----
        __builtin_amdgcn_s_setprio(1);
        scores<T, D, QB>(Kbuf[(j + 1) & 1], qop, c, hh, dbase, sn);
        pv(Vb0 + vo_prev, pp);
        make_p();
        constexpr int N_MFMA = NSB * DW / 8;
        __builtin_amdgcn_sched_group_barrier(0x0100, NKB * (DW / 16) + 2 * (DW / 32) * NKB * 2, 0);  // LDS reads
#pragma unroll
        for (int i = 0; i < N_MFMA; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);             // 1 MFMA
            __builtin_amdgcn_sched_group_barrier(0x0002, 56 * NSB / N_MFMA, 0);  // VALU
        }
        __builtin_amdgcn_s_setprio(0);

        // Range check: exponentials above 2^64 per tile (or inf/NaN) mean the
        // reference is far below this tile's scores; rebase and redo the tile.
        bool out_of_range = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) out_of_range |= !(ts[qb] < 0x1p64f);
        if (__builtin_amdgcn_ballot_w64(out_of_range) != 0) {
            rebase();
            make_p();
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) l_run[qb] += ts[qb];
        if (DS > 1) x_put((j + 1) & 1, sn);  // partial S^T of tile j+1

        // ---- staging of the next tiles into buffers not read in this step ----
        store_rows<T, D, QB>(Kbuf[j & 1], mp.kst, kreg);
        load_rows<T, D, QB>(rows_rsrc<T, D>(Kb, Nk, tile(j + 3)), mp, kreg);
        store_rows<T, D, QB>(Vb0 + vo_next, mp.vst, vreg);
        load_rows<T, D, QB>(rows_rsrc<T, D>(Vb, Nk, tile(j + 2)), mp, vreg);
        lds_barrier();
    };

    // Unrolled by two so the score and P registers swap roles instead of
    // being copied.
    auto rotate = [&]() {
        const int t = vo_prev;
        vo_prev = vo_cur;
        vo_cur = vo_next;
        vo_next = t;
    };
    for (int j = 0; j < nkt; j += 2) {
        step(j, s_a, s_b, p_a, p_b);
        rotate();
        if (j + 1 < nkt) {
            step(j + 1, s_b, s_a, p_b, p_a);
            rotate();
        }
    }
    // the deferred P V of the last tile (after the last rotation vo_prev
    // holds V of tile nkt-1)
    if (nkt > 0) {
        if (nkt & 1) pv(Vb0 + vo_prev, p_b);
        else pv(Vb0 + vo_prev, p_a);
    }

    // ---- epilogue: O = acc / l, LSE = m*scale + ln l ----
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l = sum_pair(l_run[qb]);
        const int row = q0w + 32 * qb + c;
        if (row < Nq) {
            const float inv = l > 0.f ? 1.f / l : 0.f;
            typedef T t4 __attribute__((ext_vector_type(4)));
#pragma unroll
            for (int mb = 0; mb < DW / 32; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int d0 = dbase + 32 * mb + 8 * i + 4 * hh;
                    t4 vals;
                    vals[0] = static_cast<T>(acc[qb][mb][4 * i + 0] * inv);
                    vals[1] = static_cast<T>(acc[qb][mb][4 * i + 1] * inv);
                    vals[2] = static_cast<T>(acc[qb][mb][4 * i + 2] * inv);
                    vals[3] = static_cast<T>(acc[qb][mb][4 * i + 3] * inv);
                    *reinterpret_cast<t4 *>(Ob + (size_t)row * D + d0) = vals;
                }
            if (LSE != nullptr && hh == 0 && dbase == 0)
                LSE[(size_t)bh * Nq + row] = l > 0.f ? m_ref[qb] * scale + logf(l) : -INFINITY;
        }
    }
}

// Query blocks per wave.  d = 64: two (halves the LDS operand reads per MFMA
// and is faster on large grids), or one when fewer than kSmallGrid
// workgroups of 256 rows would exist -- 128-row workgroups then fill the
// 256 CUs better (measured on MI355X: B=4, H=12, N=2048 runs 20% faster).
// d = 128: one (register budget).
constexpr long long kSmallGrid = 1024;

int qb_for(int d, long long B, long long H, long long Nq)
{
    if (d != 64) return 1;
    const long long wg2 = (Nq + Geo<64, 2>::BR - 1) / Geo<64, 2>::BR * B * H;
    return wg2 < kSmallGrid ? 1 : 2;
}

template <typename T, int D, int QB, bool CAUSAL>
hipError_t launch_t(const FwdProblem &p, hipStream_t st)
{
    using G = Geo<D, QB>;
    const int n_qtiles = (p.Nq + G::BR - 1) / G::BR;
    const int n_bh = p.B * p.H;
    const dim3 grid((unsigned)n_qtiles * (unsigned)n_bh), block(G::NT);
    hipLaunchKernelGGL((fwd_mfma_kernel<T, D, QB, CAUSAL>), grid, block, 0, st,
                       static_cast<const T *>(p.q), static_cast<const T *>(p.k),
                       static_cast<const T *>(p.v), static_cast<T *>(p.o), p.lse, p.H, p.Hkv,
                       p.Nq, p.Nk, n_bh, n_qtiles, p.scale, p.scale * kLog2e);
    return hipGetLastError();
}

template <typename T, bool CAUSAL>
hipError_t launch_c(const FwdProblem &p, hipStream_t st)
{
    if (p.d == 256) return launch_t<T, 256, 1, CAUSAL>(p, st);
    if (p.d == 128) return launch_t<T, 128, 1, CAUSAL>(p, st);
    return qb_for(64, p.B, p.H, p.Nq) == 2 ? launch_t<T, 64, 2, CAUSAL>(p, st)
                                            : launch_t<T, 64, 1, CAUSAL>(p, st);
}

template <typename T>
hipError_t launch_dt(const FwdProblem &p, hipStream_t st)
{
    return p.causal ? launch_c<T, true>(p, st) : launch_c<T, false>(p, st);
}

}  // namespace

int fwd_mfma_kv_tile(int d, long long B, long long H, long long Nq)
{
    if (d == 256) return Geo<256, 1>::BC;
    if (d == 128) return Geo<128, 1>::BC;
    return qb_for(64, B, H, Nq) == 2 ? Geo<64, 2>::BC : Geo<64, 1>::BC;
}

hipError_t launch_fwd_mfma(const FwdProblem &p, hipStream_t st)
{
    if (p.dtype == 2) return launch_dt<__bf16>(p, st);
    return launch_dt<_Float16>(p, st);
}

}  // namespace fa
