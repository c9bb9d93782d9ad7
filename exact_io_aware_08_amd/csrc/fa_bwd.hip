// fa_bwd.hip -- attention backward by recomputation, gfx950.
//
// Method: marketmaker.cc blog "Atencion flash y la pregunta sobre la
// longitud de la secuencia", section "Pase hacia atras: volver a calcular en
// lugar de almacenar": the forward keeps only O and the per-row statistics
// (here LSE = m + ln l); the backward recomputes the probabilities tile by
// tile from them instead of storing the N x N matrix.  With dO = dL/dO:
//   P_ij  = exp(scale q_i.k_j - LSE_i)
//   dP_ij = dO_i . v_j,    D_i = dO_i . O_i  (= sum_j P_ij dP_ij)
//   dS_ij = P_ij (dP_ij - D_i)
//   dQ_i  = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,
//   dV_j  = sum_i P_ij dO_i          (GQA: dK, dV sum over the group).
//
// Three kernels, all deterministic (no floating-point atomics):
//  * bwd_dot_kernel: D_i in fp32, one 16-lane group per row.
//  * bwd_dq_kernel (query-parallel, the forward's layout): S^T = K Q^T and
//    dP^T = V dO^T on v_mfma_f32_32x32x16 put one query per lane (so LSE_i
//    and D_i are one value per lane); dS^T, packed to 16 bits, is directly
//    the B operand of dQ^T += K^T dS^T, whose K^T operand comes from
//    ds_read_b64_tr_b16 on the row-major K tile in LDS.
//  * bwd_dkdv_kernel (key-parallel): S = Q K^T and dP = dO V^T put one key
//    per lane; P and dS, packed, are the B operands of dV^T += dO^T P and
//    dK^T += Q^T dS, with dO^T and Q^T from transpose reads of the staged
//    query tile.  A workgroup owns 128 keys of one KV head and sweeps every
//    query tile of every query head of its group that sees those keys; the
//    sweep is software-pipelined (the S/dP products of the next query tile
//    and the dV/dK products of the previous one overlap the P/dS work).
// Scores, dP and all accumulators are fp32; P and dS are rounded to the
// input type only as MFMA operands.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

constexpr int NW = 4;
constexpr int TK = 32;  // rows per MFMA block (keys or queries)

// ---------------------------------------------------------------------------
// D_i = dO_i . O_i
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256)
bwd_dot_kernel(const T *__restrict__ O, const T *__restrict__ dO, float *__restrict__ Dv,
               long long rows)
{
    constexpr int PER = D / 16;  // elements per lane
    typedef T tv __attribute__((ext_vector_type(PER)));
    const long long r = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int l = threadIdx.x & 15;
    float acc = 0.f;
    if (r < rows) {
        const tv o = *reinterpret_cast<const tv *>(O + r * D + l * PER);
        const tv g = *reinterpret_cast<const tv *>(dO + r * D + l * PER);
#pragma unroll
        for (int e = 0; e < PER; ++e) acc = fmaf(static_cast<float>(o[e]), static_cast<float>(g[e]), acc);
    }
    acc += __shfl_xor(acc, 8);
    acc += __shfl_xor(acc, 4);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 1);
    if (r < rows && l == 0) Dv[r] = acc;
}

// Staging map of a 32-row tile of D-element rows: chunk ci = tid + 256 r.
template <int D> struct TileMap {
    static constexpr int CPR = D / 8;
    static constexpr int CH = TK * CPR / 256;  // 16-byte chunks per thread
    // LDS row stride (elements).  Each staged tile is read both as 16-byte
    // rows and by transpose reads; D + 40 (20 mod 32 dwords) measured best of
    // D + 8 ... D + 48 for the two together (LDS bank conflicts of D + 8
    // cost 1-6%).
    static constexpr int ST = D + 40;
    static_assert(CH >= 1 && CH * 256 == TK * CPR, "tile staging split");
    int off[CH], lds[CH];
    __device__ __forceinline__ TileMap(int tid, int elem_bytes) {
#pragma unroll
        for (int r = 0; r < CH; ++r) {
            const int ci = tid + 256 * r;
            off[r] = ((ci / CPR) * D + (ci % CPR) * 8) * elem_bytes;
            lds[r] = (ci / CPR) * ST + (ci % CPR) * 8;
        }
    }
};

template <int D>
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t rs, const TileMap<D> &mp,
                                          u32x4_t (&reg)[TileMap<D>::CH])
{
#pragma unroll
    for (int r = 0; r < TileMap<D>::CH; ++r) reg[r] = __builtin_amdgcn_raw_buffer_load_b128(rs, mp.off[r], 0, 0);
}

template <typename T, int D>
__device__ __forceinline__ void store_tile(T *buf, const TileMap<D> &mp, const u32x4_t (&reg)[TileMap<D>::CH])
{
#pragma unroll
    for (int r = 0; r < TileMap<D>::CH; ++r) *reinterpret_cast<u32x4_t *>(buf + mp.lds[r]) = reg[r];
}

// Pack registers 8t..8t+7 of a 32x32 fp32 block into the 16-bit MFMA operand
// of K-step t (slot k <-> row 16t + 8(k/4) + 4(l/32) + k%4 of the block).
template <typename T>
__device__ __forceinline__ typename Mma16<T>::v8 pack_block(const f32x16_t &x, int t)
{
    typedef T v2 __attribute__((ext_vector_type(2)));
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const v2 pk = __builtin_convertvector((f32x2_t{x[8 * t + 2 * e], x[8 * t + 2 * e + 1]}), v2);
        w[e] = bitcast<uint32_t>(pk);
    }
    return bitcast<typename Mma16<T>::v8>(u32x4_t{w[0], w[1], w[2], w[3]});
}

// A operand of a transposed product from a row-major 32-row tile in LDS:
// lane (c, hh) gets column 32 mb + c of rows 16t + 4hh + 0..3 (slots 0-3)
// and 16t + 8 + 4hh + 0..3 (slots 4-7).
template <typename T, int ST>
__device__ __forceinline__ typename Mma16<T>::v8 tr_operand(const T *tile, int tr_off, int mb, int t)
{
    const T *p = tile + tr_off + 16 * t * ST + 32 * mb;
    const u32x2_t lo = read_tr(p);
    const u32x2_t hi = read_tr(p + 8 * ST);
    return bitcast<typename Mma16<T>::v8>(u32x4_t{lo.x, lo.y, hi.x, hi.y});
}

// ---------------------------------------------------------------------------
// dQ (query-parallel).  Workgroup: 4 waves x 32 query rows of one (b, h).
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 2)
bwd_dq_kernel(const T *__restrict__ Q, const T *__restrict__ K, const T *__restrict__ V,
              const T *__restrict__ dO, const float *__restrict__ LSE,
              const float *__restrict__ Dv, T *__restrict__ dQ, int H, int Hkv, int Nq, int Nk,
              int n_bh, int n_qtiles, float scale, float scale_log2)
{
    using M = Mma16<T>;
    using v8 = typename M::v8;
    using TM = TileMap<D>;
    constexpr int ST = TM::ST, BR = NW * TK;

    __shared__ __attribute__((aligned(16))) T Kbuf[2][TK * ST];
    __shared__ __attribute__((aligned(16))) T Vbuf[2][TK * ST];

    const int tid = threadIdx.x;
    const int lane = tid & 63, c = lane & 31, hh = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

    const int qt = n_qtiles - 1 - (int)(blockIdx.x / (unsigned)n_bh);
    const int bh = (int)(blockIdx.x % (unsigned)n_bh);
    const int b = bh / H, h = bh - b * H;
    const int hk = h / (H / Hkv);
    const size_t qoff = (size_t)bh * Nq * D;
    const size_t kvoff = ((size_t)b * Hkv + hk) * Nk * D;
    const T *Kb = K + kvoff;
    const T *Vb = V + kvoff;

    const int q0 = qt * BR;
    const int q0w = q0 + w * TK;
    const int off = Nk - Nq;
    int nkt = (Nk + TK - 1) / TK;
    if (CAUSAL) {
        const int lim = min(q0 + BR, Nq) - 1 + off;
        nkt = lim < 0 ? 0 : min(nkt, lim / TK + 1);
    }

    // Q and dO operands (B of S^T = K Q^T and of dP^T = V dO^T): lane (c, hh)
    // holds row q0w + c, elements 16t + 8hh + 0..7.  Rows past Nq read zero.
    v8 qop[D / 16], gop[D / 16];
    {
        const __amdgpu_buffer_rsrc_t rq = rows_rsrc<T, D>(Q + qoff, Nq, q0w);
        const __amdgpu_buffer_rsrc_t rg = rows_rsrc<T, D>(dO + qoff, Nq, q0w);
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
            const int o = (c * D + 16 * t + 8 * hh) * (int)sizeof(T);
            qop[t] = bitcast<v8>(__builtin_amdgcn_raw_buffer_load_b128(rq, o, 0, 0));
            gop[t] = bitcast<v8>(__builtin_amdgcn_raw_buffer_load_b128(rg, o, 0, 0));
        }
        settle(qop);
        settle(gop);
    }
    const int row = q0w + c;
    const bool row_ok = row < Nq;
    float lse2 = 0.f, drow = 0.f;
    if (row_ok) {
        const float l = LSE[(size_t)bh * Nq + row];
        lse2 = l == -INFINITY ? 0.f : l * kLog2e;  // rows without keys: every P is masked
        drow = Dv[(size_t)bh * Nq + row];
    }
    const int lim = CAUSAL ? min(Nk, row + off + 1) : Nk;  // keys [0, lim) visible to this row

    f32x16_t acc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc[i] = f32x16_t{};

    const TM mp(tid, (int)sizeof(T));
    const int tr_off = (4 * hh + ((lane & 15) >> 2)) * ST + 16 * (c >> 4) + 4 * (lane & 3);
    u32x4_t kreg[TM::CH], vreg[TM::CH];
    auto tile = [&](int jj) { return min(jj, nkt - 1) * TK; };

    if (nkt > 0) {
        load_tile<D>(rows_rsrc<T, D>(Kb, Nk, 0), mp, kreg);
        load_tile<D>(rows_rsrc<T, D>(Vb, Nk, 0), mp, vreg);
        store_tile<T, D>(Kbuf[0], mp, kreg);
        store_tile<T, D>(Vbuf[0], mp, vreg);
        load_tile<D>(rows_rsrc<T, D>(Kb, Nk, tile(1)), mp, kreg);
        load_tile<D>(rows_rsrc<T, D>(Vb, Nk, tile(1)), mp, vreg);
        lds_barrier();
    }

    for (int j = 0; j < nkt; ++j) {
        const T *Ks = Kbuf[j & 1];
        const T *Vs = Vbuf[j & 1];
        // tile j+1 into the other buffers (free since the last barrier), then prefetch j+2
        store_tile<T, D>(Kbuf[(j + 1) & 1], mp, kreg);
        store_tile<T, D>(Vbuf[(j + 1) & 1], mp, vreg);
        load_tile<D>(rows_rsrc<T, D>(Kb, Nk, tile(j + 2)), mp, kreg);
        load_tile<D>(rows_rsrc<T, D>(Vb, Nk, tile(j + 2)), mp, vreg);

        f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
            const v8 kop = *reinterpret_cast<const v8 *>(&Ks[c * ST + 16 * t + 8 * hh]);
            const v8 vop = *reinterpret_cast<const v8 *>(&Vs[c * ST + 16 * t + 8 * hh]);
            s = M::mma32(kop, qop[t], s);
            dp = M::mma32(vop, gop[t], dp);
        }
        // P and dS for this tile (register r: key j*32 + 8(r/4) + 4hh + r%4).
        // Tiles whose every key every row of the wave sees (uniform test)
        // skip the per-element mask; rows past Nq are never stored.
        const int j0 = j * TK;
        f32x16_t ds;
        if (j0 + TK <= Nk && (!CAUSAL || j0 + TK - 1 <= q0w + off)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(fmaf(s[r], scale_log2, -lse2));
                ds[r] = p * (dp[r] - drow);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = j0 + 8 * (r >> 2) + 4 * hh + (r & 3);
                const float p = (key < lim) ? fast_exp2(fmaf(s[r], scale_log2, -lse2)) : 0.f;
                ds[r] = p * (dp[r] - drow);
            }
        }
        // dQ^T += K^T dS^T
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const v8 dsop = pack_block<T>(ds, t);
#pragma unroll
            for (int mb = 0; mb < D / 32; ++mb)
                acc[mb] = M::mma32(tr_operand<T, ST>(Ks, tr_off, mb, t), dsop, acc[mb]);
        }
        lds_barrier();
    }

    if (row_ok) {
        T *dq = dQ + qoff + (size_t)row * D;
        typedef T t4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                t4 vals;
#pragma unroll
                for (int e = 0; e < 4; ++e) vals[e] = static_cast<T>(acc[mb][4 * i + e] * scale);
                *reinterpret_cast<t4 *>(dq + 32 * mb + 8 * i + 4 * hh) = vals;
            }
    }
}

// ---------------------------------------------------------------------------
// dK, dV (key-parallel).  Workgroup: 4 waves x 32 keys of one (b, KV head);
// it sweeps the query tiles of all G query heads of the group.
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(256, D >= 128 ? 1 : 2)
bwd_dkdv_kernel(const T *__restrict__ Q, const T *__restrict__ K, const T *__restrict__ V,
                const T *__restrict__ dO, const float *__restrict__ LSE,
                const float *__restrict__ Dv, T *__restrict__ dK, T *__restrict__ dV, int H,
                int Hkv, int Nq, int Nk, int n_bkv, int n_ktiles, float scale, float scale_log2)
{
    using M = Mma16<T>;
    using v8 = typename M::v8;
    using TM = TileMap<D>;
    constexpr int ST = TM::ST, BKEYS = NW * TK;

    __shared__ __attribute__((aligned(16))) T Qbuf[4][TK * ST];      // iteration i in buffer i % 4
    __shared__ __attribute__((aligned(16))) T Gbuf[4][TK * ST];      // dO
    __shared__ __attribute__((aligned(16))) float Lbuf[4][TK];       // LSE * log2(e), 0 for rows without keys
    __shared__ __attribute__((aligned(16))) float Dbuf[4][TK];

    const int tid = threadIdx.x;
    const int lane = tid & 63, c = lane & 31, hh = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

    // Key tiles near the start are seen by the most queries under a causal
    // mask: launch them first.
    const int kt = (int)(blockIdx.x / (unsigned)n_bkv);
    const int bkv = (int)(blockIdx.x % (unsigned)n_bkv);
    const int b = bkv / Hkv, hk = bkv - b * Hkv;
    const int G = H / Hkv;
    const size_t kvoff = (size_t)bkv * Nk * D;
    const int k0 = kt * BKEYS;
    const int k0w = k0 + w * TK;
    const int key = k0w + c;  // this lane's key
    const int off = Nk - Nq;

    // K and V operands (B of S = Q K^T and of dP = dO V^T): lane (c, hh) holds
    // key k0w + c, elements 16t + 8hh + 0..7.  Keys past Nk read zero.
    v8 kop[D / 16], vop[D / 16];
    {
        const __amdgpu_buffer_rsrc_t rk = rows_rsrc<T, D>(K + kvoff, Nk, k0w);
        const __amdgpu_buffer_rsrc_t rv = rows_rsrc<T, D>(V + kvoff, Nk, k0w);
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
            const int o = (c * D + 16 * t + 8 * hh) * (int)sizeof(T);
            kop[t] = bitcast<v8>(__builtin_amdgcn_raw_buffer_load_b128(rk, o, 0, 0));
            vop[t] = bitcast<v8>(__builtin_amdgcn_raw_buffer_load_b128(rv, o, 0, 0));
        }
        settle(kop);
        settle(vop);
    }

    // Query tiles that see any key of this workgroup: q >= k0 - off (causal).
    const int nqt_all = (Nq + TK - 1) / TK;
    int qt0 = 0;
    if (CAUSAL) {
        const int first_q = k0 - off;
        qt0 = first_q <= 0 ? 0 : min(nqt_all, first_q / TK);
    }
    const int nqt = nqt_all - qt0;      // tiles per head
    const int n_it = nqt * G;           // iterations: (head in group, query tile)
    // Iteration it covers query head hk * G + it / nqt and query tile
    // qt0 + it % nqt.  The loads and the P/dS work each walk the iterations
    // in order, so each keeps its own (head, tile) position and advances it
    // by one (no integer division in the loop).
    struct ItPos {
        int it, h, qt;
    };
    auto advance = [&](ItPos &ps) {
        ++ps.it;
        if (++ps.qt == nqt_all) {
            ps.qt = qt0;
            ++ps.h;
        }
    };

    f32x16_t acck[D / 32], accv[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
        acck[i] = f32x16_t{};
        accv[i] = f32x16_t{};
    }

    const TM mp(tid, (int)sizeof(T));
    const int tr_off = (4 * hh + ((lane & 15) >> 2)) * ST + 16 * (c >> 4) + 4 * (lane & 3);
    u32x4_t qreg[2][TM::CH], greg[2][TM::CH];
    float lreg[2] = {0.f, 0.f};  // threads 0..31: LSE of row tid; 32..63: D of row tid-32
    // Global -> registers, iterations in order (it stays at the last
    // iteration once reached), into two register sets: iteration i goes to
    // set i & 1 two steps before it is staged, so each load has two steps to
    // arrive (with one set, one step: 2% slower on the trading day,
    // bit-identical).  The LSE is kept raw here and converted when staged:
    // using it at once would make the wave wait for these loads in the same
    // step.
    ItPos fp{0, 0, qt0};
    auto fetch = [&](int rs) {
        const int hq = hk * G + fp.h, q0 = fp.qt * TK;
        const size_t qoff = ((size_t)b * H + hq) * Nq * D;
        load_tile<D>(rows_rsrc<T, D>(Q + qoff, Nq, q0), mp, qreg[rs]);
        load_tile<D>(rows_rsrc<T, D>(dO + qoff, Nq, q0), mp, greg[rs]);
        if (tid < 2 * TK) {
            const int r = q0 + (tid & (TK - 1));
            const size_t ro = ((size_t)b * H + hq) * Nq + r;
            lreg[rs] = 0.f;
            if (r < Nq) lreg[rs] = tid < TK ? LSE[ro] : Dv[ro];
        }
        if (fp.it < n_it - 1) advance(fp);
    };
    auto stage = [&](int buf, int rs) {
        store_tile<T, D>(Qbuf[buf], mp, qreg[rs]);
        store_tile<T, D>(Gbuf[buf], mp, greg[rs]);
        if (tid < TK) Lbuf[buf][tid] = lreg[rs] == -INFINITY ? 0.f : lreg[rs] * kLog2e;
        else if (tid < 2 * TK) Dbuf[buf][tid - TK] = lreg[rs];
    };

    // Software pipeline over the iterations, as in the forward: step `it`
    // issues the S/dP products of iteration it+1 and the dV/dK products of
    // iteration it-1 on the MFMA pipe while the VALU turns S/dP of iteration
    // it into P and dS.  Iteration i's query and dO tile, LSE and D live in
    // buffer i % 4 from step i-2 (staging) to step i+1 (its dV/dK products);
    // buffer 3 stands for iteration -1, whose operands are zero, and holds
    // zeros so that its products stay finite.
    if (n_it > 0) {
        fetch(0);  // iteration 0
        stage(0, 0);
        fetch(0);  // 1
        stage(1, 0);
        fetch(0);  // 2, register set 0
        fetch(1);  // 3, register set 1
        for (int i = tid; i < TK * ST / 8; i += 256) {
            reinterpret_cast<u32x4_t *>(Qbuf[3])[i] = u32x4_t{0u, 0u, 0u, 0u};
            reinterpret_cast<u32x4_t *>(Gbuf[3])[i] = u32x4_t{0u, 0u, 0u, 0u};
        }
        lds_barrier();
    }

    // S = Q K^T and dP = dO V^T of the tile in buffer `bf` (register r:
    // query q0 + 8(r/4) + 4hh + r%4, key `key`)
    auto sdp = [&](int bf, f32x16_t &s, f32x16_t &dp) {
        const T *Qs = Qbuf[bf];
        const T *Gs = Gbuf[bf];
        s = f32x16_t{};
        dp = f32x16_t{};
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
            const v8 qa = *reinterpret_cast<const v8 *>(&Qs[c * ST + 16 * t + 8 * hh]);
            const v8 ga = *reinterpret_cast<const v8 *>(&Gs[c * ST + 16 * t + 8 * hh]);
            s = M::mma32(qa, kop[t], s);
            dp = M::mma32(ga, vop[t], dp);
        }
    };
    // dV^T += dO^T P,  dK^T += Q^T dS  with the tile in buffer `bf`
    auto dkdv = [&](int bf, const v8 (&pop)[2], const v8 (&dsop)[2]) {
        const T *Qs = Qbuf[bf];
        const T *Gs = Gbuf[bf];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int mb = 0; mb < D / 32; ++mb) {
                accv[mb] = M::mma32(tr_operand<T, ST>(Gs, tr_off, mb, t), pop[t], accv[mb]);
                acck[mb] = M::mma32(tr_operand<T, ST>(Qs, tr_off, mb, t), dsop[t], acck[mb]);
            }
    };
    // P and dS of iteration it from its S and dP, packed as MFMA operands
    ItPos pq{0, 0, qt0};  // the iteration whose P and dS the next step forms
    auto pds = [&](int it, const f32x16_t &s, const f32x16_t &dp, v8 (&pop)[2], v8 (&dsop)[2]) {
        const int bf = it & 3;
        const int q0 = pq.qt * TK;
        advance(pq);
        f32x16_t p, ds;
        // Tiles where every query sees every key of the wave (uniform test)
        // skip the per-element mask.
        const bool full = q0 + TK <= Nq && k0w + TK <= Nk && (!CAUSAL || k0w + TK - 1 <= q0 + off);
        if (full) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4_t l4 = *reinterpret_cast<const f32x4_t *>(&Lbuf[bf][8 * i + 4 * hh]);
                const f32x4_t d4 = *reinterpret_cast<const f32x4_t *>(&Dbuf[bf][8 * i + 4 * hh]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * i + e;
                    const float pv = fast_exp2(fmaf(s[r], scale_log2, -l4[e]));
                    p[r] = pv;
                    ds[r] = pv * (dp[r] - d4[e]);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4_t l4 = *reinterpret_cast<const f32x4_t *>(&Lbuf[bf][8 * i + 4 * hh]);
                const f32x4_t d4 = *reinterpret_cast<const f32x4_t *>(&Dbuf[bf][8 * i + 4 * hh]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * i + e;
                    const int q = q0 + 8 * i + 4 * hh + e;
                    const bool vis = q < Nq && key < Nk && (!CAUSAL || key <= q + off);
                    const float pv = vis ? fast_exp2(fmaf(s[r], scale_log2, -l4[e])) : 0.f;
                    p[r] = pv;
                    ds[r] = pv * (dp[r] - d4[e]);
                }
            }
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            pop[t] = pack_block<T>(p, t);
            dsop[t] = pack_block<T>(ds, t);
        }
    };

    f32x16_t s_a, dp_a, s_b, dp_b;
    v8 p_a[2], ds_a[2], p_b[2], ds_b[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        p_a[t] = bitcast<v8>(u32x4_t{0u, 0u, 0u, 0u});
        ds_a[t] = p_a[t];
    }
    if (n_it > 0) sdp(0, s_a, dp_a);

    // One step.  On entry: (sc, dpc) = S, dP of iteration it; (pp, dsp) =
    // operands of iteration it-1; buffers (it-1..it+1) % 4 staged; register
    // set it & 1 holds iteration it+2 and the other set iteration it+3.
    auto step = [&](int it, int rs, f32x16_t &sc, f32x16_t &dpc, f32x16_t &sn, f32x16_t &dpn,
                    const v8 (&pp)[2], const v8 (&dsp)[2], v8 (&pc)[2], v8 (&dsc)[2]) {
        stage((it + 2) & 3, rs);  // last read (iteration it-2's dV/dK) before the previous barrier
        fetch(rs);                // iteration it+4 into the set just staged (rs = it & 1)
        sdp((it + 1) & 3, sn, dpn);
        dkdv((it + 3) & 3, pp, dsp);  // iteration it-1
        pds(it, sc, dpc, pc, dsc);
        lds_barrier();
    };
    int it = 0;
    for (; it + 1 < n_it; it += 2) {
        step(it, 0, s_a, dp_a, s_b, dp_b, p_a, ds_a, p_b, ds_b);
        step(it + 1, 1, s_b, dp_b, s_a, dp_a, p_b, ds_b, p_a, ds_a);
    }
    if (it < n_it) {
        step(it, 0, s_a, dp_a, s_b, dp_b, p_a, ds_a, p_b, ds_b);
        dkdv(it & 3, p_b, ds_b);  // the last iteration's deferred products
    } else if (n_it > 0) {
        dkdv((n_it - 1) & 3, p_a, ds_a);
    }

    if (key < Nk) {
        T *dk = dK + kvoff + (size_t)key * D;
        T *dv = dV + kvoff + (size_t)key * D;
        typedef T t4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                t4 kv, vv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kv[e] = static_cast<T>(acck[mb][4 * i + e] * scale);
                    vv[e] = static_cast<T>(accv[mb][4 * i + e]);
                }
                *reinterpret_cast<t4 *>(dk + 32 * mb + 8 * i + 4 * hh) = kv;
                *reinterpret_cast<t4 *>(dv + 32 * mb + 8 * i + 4 * hh) = vv;
            }
    }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_t(const BwdProblem &p, hipStream_t st)
{
    const long long rows = (long long)p.B * p.H * p.Nq;
    if (rows > 0) {
        hipLaunchKernelGGL((bwd_dot_kernel<T, D>), dim3((unsigned)((rows + 15) / 16)), dim3(256), 0,
                           st, static_cast<const T *>(p.o), static_cast<const T *>(p.dout), p.dvec,
                           rows);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int n_qtiles = (p.Nq + NW * TK - 1) / (NW * TK);
        const int n_bh = p.B * p.H;
        hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL>), dim3((unsigned)n_qtiles * (unsigned)n_bh),
                           dim3(256), 0, st, static_cast<const T *>(p.q),
                           static_cast<const T *>(p.k), static_cast<const T *>(p.v),
                           static_cast<const T *>(p.dout), p.lse, p.dvec, static_cast<T *>(p.dq),
                           p.H, p.Hkv, p.Nq, p.Nk, n_bh, n_qtiles, p.scale, p.scale * kLog2e);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if ((long long)p.B * p.Hkv * p.Nk > 0) {
        const int n_ktiles = (p.Nk + NW * TK - 1) / (NW * TK);
        const int n_bkv = p.B * p.Hkv;
        hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL>),
                           dim3((unsigned)n_ktiles * (unsigned)n_bkv), dim3(256), 0, st,
                           static_cast<const T *>(p.q), static_cast<const T *>(p.k),
                           static_cast<const T *>(p.v), static_cast<const T *>(p.dout), p.lse,
                           p.dvec, static_cast<T *>(p.dk), static_cast<T *>(p.dv), p.H, p.Hkv,
                           p.Nq, p.Nk, n_bkv, n_ktiles, p.scale, p.scale * kLog2e);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <typename T>
hipError_t launch_dt(const BwdProblem &p, hipStream_t st)
{
    if (p.d == 64) return p.causal ? launch_t<T, 64, true>(p, st) : launch_t<T, 64, false>(p, st);
    return p.causal ? launch_t<T, 128, true>(p, st) : launch_t<T, 128, false>(p, st);
}

}  // namespace

hipError_t launch_bwd(const BwdProblem &p, hipStream_t st)
{
    return p.dtype == 2 ? launch_dt<__bf16>(p, st) : launch_dt<_Float16>(p, st);
}

}  // namespace fa
