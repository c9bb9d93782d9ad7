/*
 * fa.h -- C ABI of libfa: exact, IO-aware attention for AMD Instinct MI355X
 * (gfx950).
 *
 * What is computed.  O = softmax(Q K^T * scale) V, exactly (the result of the
 * definition, up to floating-point rounding), tile by tile with the online
 * softmax recurrence so the N x N score matrix never reaches device memory:
 *   - marketmaker.cc blog "Atencion flash y la pregunta sobre la longitud de la
 *     secuencia", sections "El algoritmo de atencion flash" (tiling, running
 *     max m, running sum l, rescaled output accumulator), "La recurrencia de
 *     softmax en linea" (a reassociation, not an approximation), "FA2:
 *     paralelismo" (deferred normalisation, query-block parallelism, no
 *     cross-wave row reductions) and "El enmascaramiento causal ..." (tiles
 *     wholly in the future are neither loaded nor computed);
 *   - systems-analysis.info "FlashAttention (IT)", section "Innovazioni chiave"
 *     (tiling, online softmax, one fused kernel that writes only the output).
 *
 * Conventions shared by every entry point.
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library allocates nothing and keeps no pointer after a call returns.
 *   - Layout is contiguous row-major [batch, heads, seq, head_dim]:
 *     q, o: [B, H, Nq, d];  k, v: [B, Hkv, Nk, d];  lse: [B, H, Nq] fp32.
 *     o has the input dtype.  Tensor pointers must be 16-byte aligned.
 *   - GQA/MQA: H must be a multiple of Hkv; query head h reads KV head
 *     h / (H / Hkv) (shared KV heads as in gist.science "FlashAttention for
 *     Scalable Vector Architectures", section "Metodologia").
 *   - Causal masking is bottom-right aligned: key j is visible to query i
 *     iff j <= i + (Nk - Nq).  A query with no visible key gets O = 0 and
 *     LSE = -inf.
 *   - lse holds the natural-log log-sum-exp of each score row,
 *     LSE = m + ln(l), the O(N) statistics the backward pass keeps
 *     (marketmaker.cc, section "Pase hacia atras").
 *   - Calls are asynchronous and ordered on `stream` (a hipStream_t passed as
 *     void*; NULL is the default stream).  No host synchronisation.
 *   - Errors: arguments are validated on the host before any launch; on an
 *     error nothing is launched and nothing is written.  There is never a
 *     silent fallback to another algorithm (the warning of marketmaker.cc,
 *     section "La integracion es de ocho lineas").  Launch failures return
 *     FA_ERR_HIP.  A current device that is not gfx950 returns
 *     FA_ERR_DEVICE.
 *   - Empty work: B == 0 or Nq == 0 returns FA_OK without a launch.  The
 *     pointer of an empty tensor may be NULL (q/o/lse when B*Nq == 0, k/v
 *     when B*Nk == 0).  Nk == 0 with Nq > 0 writes O = 0 and LSE = -inf.
 *   - Sizes: every tensor's element count per (batch, head) slice must be
 *     below 2^31.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype;

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = 1,      /* a required pointer is NULL                          */
    FA_ERR_SHAPE = 2,     /* negative size, H or Hkv < 1, or a slice too large   */
    FA_ERR_HEADDIM = 3,   /* d is not 64 or 128 (fa_fwd bf16/fp16: or 256)       */
    FA_ERR_GQA = 4,       /* H is not a multiple of Hkv                          */
    FA_ERR_DTYPE = 5,     /* dtype not supported by this entry point            */
    FA_ERR_ALIGN = 6,     /* a tensor pointer is not 16-byte aligned             */
    FA_ERR_SCALE = 7,     /* scale or p_scale is not finite and > 0              */
    FA_ERR_WORKSPACE = 8, /* decode workspace NULL or too small                  */
    FA_ERR_DEVICE = 9,    /* current device is not gfx950 (or cannot be queried) */
    FA_ERR_HIP = 10,      /* a kernel launch failed                              */
    FA_ERR_ARG = 11,      /* another argument out of range                       */
    FA_ERR_SCRATCH = 12   /* fa_decode_noalloc: partials exceed the static scratch */
} fa_status;

/*
 * Prefill / forward attention.
 *   q, k, v : device inputs, layout above, element type `dtype`
 *             (FA_BF16 and FA_F16 run on bf16/fp16 MFMA with fp32
 *             accumulation; FA_F32 runs on fp32 MFMA).
 *   d       : 64 or 128 for every dtype; also 256 for FA_BF16 and FA_F16
 *             (the head size FlashAttention-2 added, systems-analysis.info
 *             "FlashAttention (IT)", section "Evoluzione e sviluppi
 *             successivi").  Other values return FA_ERR_HEADDIM.
 *   o       : device output [B, H, Nq, d], same dtype as the inputs.
 *   lse     : device output [B, H, Nq] fp32, or NULL to skip it.
 *   causal  : 0 = full attention, 1 = bottom-right causal mask.
 *   scale   : multiplier of Q K^T (normally 1/sqrt(d)); finite and > 0.
 */
fa_status fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                 int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                 fa_dtype dtype, void *stream);

/*
 * Forward attention with the softmax probabilities cast to E4M3 before the
 * P*V product (gist.science "Resumen Tecnico: Precision de P-Cast en la
 * Atencion FP8", sections "Planteamiento del Problema", "Optimizacion 1" and
 * "Optimizacion 2"): per KV tile, P = exp(s - m) relative to the RUNNING max
 * m, then P~ = E4M3_RNE(p_scale * P) (OCP E4M3FN), O accumulates P~ V in
 * fp32, the running sum l uses the uncast P, and the epilogue divides by
 * p_scale * l.  The page keeps Q, K, V in fp32 (section "Contribuciones
 * Clave", item 4); bf16 operands are also accepted and are widened exactly
 * to fp32 on load, so the arithmetic after the load is the same.
 *   dtype      : FA_F32 or FA_BF16 (q, k, v and o all in that type).
 *   p_scale    : the static scale S (256 recommended); finite, > 0, <= 448.
 *   kv_reverse : bit 0: 0 = KV tiles in increasing key order, 1 = decreasing
 *                (the sink block last).  Bit 1 (an ablation, FA1's form in
 *                marketmaker.cc "El algoritmo de atencion flash"): P is taken
 *                relative to each tile's own max and its weight restored by
 *                exp(m_tile - m) after the cast, so every tile's largest P
 *                casts from exactly p_scale.  Other bits must be 0.
 *   n_sink     : keys [0, n_sink) are sink keys, excluded from counts[0..1].
 *   counts     : NULL, or a device array of 4 uint64 to which the call ADDS
 *                (the caller initialises it):
 *                [0] casts of non-sink keys (key >= n_sink),
 *                [1] of those, values flushed to zero (P~ == 0 while P > 0),
 *                [2] casts of keys outside the KV tiles that hold a sink key,
 *                [3] of those, values flushed to zero.
 *                Only visible (query, key) pairs with query < Nq count.
 * The KV tile width that fixes the tile boundaries is fa_kv_tile(dtype, d, 1)
 * (the same for both types).
 */
fa_status fa_fwd_pcast(const void *q, const void *k, const void *v, void *o, float *lse,
                       int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                       fa_dtype dtype, float p_scale, int kv_reverse, int n_sink,
                       unsigned long long *counts, void *stream);

/* Keys per KV tile used by the forward kernels for (dtype, d, pcast), or -1
 * for an unsupported combination.  Tile t covers keys [t*B_c, (t+1)*B_c).
 * The fp32 / P-cast value is exact (the P-cast result depends on it: a cast
 * sees the running max of the tiles before it).  For the 16-bit kernels at
 * d = 64 the width also depends on the grid -- 32 keys when at least 1024
 * workgroups of 256 query rows exist (ceil(Nq/256)*B*H >= 1024), else 64 --
 * and this returns the large-grid value; their results depend on it only
 * through rounding order.  At d = 128 and 256 (16-bit only) it is 32. */
int fa_kv_tile(fa_dtype dtype, int d, int pcast);

/*
 * Split-KV decode of one new query token per (batch, head) against a KV
 * cache, merged with log-sum-exp.  The online recurrence is associative, so
 * each split produces (O_s, lse_s) over its slice of keys and the merge is
 *   LSE = M + ln sum_s exp(lse_s - M),  M = max_s lse_s,
 *   O   = sum_s exp(lse_s - LSE) * O_s.
 * Each workgroup serves every query head of one KV head from one read of
 * its K/V slice (GQA: load the shared KV head once, gist.science
 * "FlashAttention for Scalable Vector Architectures", section "Metodologia").
 *   q        : device [B, H, 1, d];  k_cache, v_cache: device [B, Hkv, Nk, d].
 *   o        : device [B, H, 1, d] (dtype);  lse: device [B, H, 1] fp32 or NULL.
 *   No mask: the new token's K/V are already in the cache.
 *   dtype    : FA_BF16 or FA_F16.
 *   num_splits: 0 = automatic (fa_decode_splits), else 1..4096.  Splits are
 *              whole multiples of 512 keys (d = 64) or 256 keys (d = 128);
 *              splits past the end of the cache are empty and harmless.
 *   workspace: device memory of at least
 *              fa_decode_workspace_bytes(B, H, Hkv, Nk, d, num_splits) bytes,
 *              16-byte aligned, owned by the caller; it holds the per-split
 *              partial results (LSE, then O on a 256-byte boundary).  Its
 *              contents on entry do not matter.  The size is 0 when the call
 *              has one split; workspace may then be NULL.  Calls that share a
 *              workspace must be ordered (one stream): overlapping calls on
 *              one workspace race.
 *   With more than one split a second small kernel merges the partials on
 *   the same stream; with one split the sweep writes O and LSE itself.
 */
int fa_decode_splits(int B, int H, int Hkv, int Nk, int num_splits);
size_t fa_decode_workspace_bytes(int B, int H, int Hkv, int Nk, int d, int num_splits);
fa_status fa_decode(const void *q, const void *k_cache, const void *v_cache, void *o,
                    float *lse, int B, int H, int Hkv, int Nk, int d, float scale,
                    fa_dtype dtype, int num_splits, void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * fa_decode without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops and harnesses
 * that forbid allocation.  Same arguments, kernels and results as fa_decode
 * (bit for bit, for the same num_splits), except that the per-split partials
 * live in the library's own static device scratch of 8 MiB per GPU (a
 * file-scope device array, held by each GPU the library runs on until the
 * process ends).  The call allocates nothing; the caller passes inputs and
 * outputs.
 *   Limit: fa_decode_workspace_bytes(B, H, Hkv, Nk, d, num_splits) must be at
 *   most 8 MiB (8,388,608 bytes), else FA_ERR_SCRATCH and nothing is
 *   launched (the TinyLlama-shaped B=16, H=32, Hkv=4, Nk=8192 decode needs
 *   0.53 MB).  A call with one split uses no scratch.
 *   The scratch keeps whatever the last call wrote; each call's merge reads
 *   only partials its own sweep wrote on the same stream, so nothing needs
 *   clearing.  Every call on a GPU shares that GPU's scratch: calls that
 *   overlap on one GPU (other streams, other host threads) race.
 */
fa_status fa_decode_noalloc(const void *q, const void *k_cache, const void *v_cache, void *o,
                            float *lse, int B, int H, int Hkv, int Nk, int d, float scale,
                            fa_dtype dtype, int num_splits, void *stream);

/*
 * Split-KV decode against a paged KV cache with per-sequence lengths (the
 * KV-cache management of serving systems, systems-analysis.info
 * "FlashAttention (IT)", section "Soluzioni specializzate").  Same
 * computation and merge as fa_decode, sequence b attending to its own
 * seq_lens[b] keys.
 *   k_pages, v_pages: device [num_pages, Hkv, page_size, d] (dtype).
 *   block_table: device int32 [B, max_pages]; key t of sequence b is row
 *     t % page_size of page block_table[b][t / page_size].
 *   seq_lens: device int32 [B], each in [0, max_pages * page_size]; a
 *     sequence of length 0 gets O = 0 and LSE = -inf.
 *   page_size: a multiple of 32, at least 32.  max_pages >= 1.
 *   The device tables are not read on the host: lengths outside the range
 *   are clamped and page indices outside [0, num_pages) read nothing, so a
 *   bad table gives wrong numbers but no out-of-bounds access.
 *   num_splits > 0: every sequence is cut into that many chunks of
 *     ceil(max_pages * page_size / num_splits) keys (rounded up to the split
 *     granularity), as fa_decode with Nk = max_pages * page_size; the chunks
 *     past a sequence's end do no work.
 *   num_splits = 0 (automatic), B <= 256: the kernels read the lengths on
 *     the device and size one chunk for the whole batch, about 256
 *     workgroups' worth of keys in all (at least 512 keys, a multiple of the
 *     split granularity); sequence b gets max(1, ceil(seq_lens[b] / chunk))
 *     splits.  A ragged batch is then spread over the whole GPU instead of
 *     following its longest sequence.  No host synchronisation.  B > 256:
 *     the split count fa_decode would choose for Nk = max_pages * page_size.
 *   workspace: device memory of at least fa_decode_paged_workspace_bytes(B,
 *     H, Hkv, max_pages, page_size, d, num_splits) bytes (none when that is
 *     0), 16-byte aligned; contents on entry do not matter.
 */
size_t fa_decode_paged_workspace_bytes(int B, int H, int Hkv, int max_pages, int page_size, int d,
                                       int num_splits);
fa_status fa_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                          const int *block_table, const int *seq_lens, void *o, float *lse,
                          int B, int H, int Hkv, int num_pages, int page_size, int max_pages,
                          int d, float scale, fa_dtype dtype, int num_splits, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * Backward pass by recomputation (marketmaker.cc, section "Pase hacia atras:
 * volver a calcular en lugar de almacenar"): from the forward's O and LSE
 * and the output gradient dout = dL/dO, the gradients
 *   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dout,
 * with P = exp(scale Q K^T - LSE), dS = P (dout V^T - D), D = rowsum(dout * O),
 * recomputing P tile by tile.  GQA: dk, dv sum over the query heads of a group.
 *   q, o, dout, dq: device [B, H, Nq, d];  k, v, dk, dv: device [B, Hkv, Nk, d];
 *   lse: device [B, H, Nq] fp32 as written by fa_fwd (natural log; -inf for a
 *   row without visible keys).  Gradients are written in `dtype`; every
 *   element of dq, dk and dv is written (zeros where no key/query is visible).
 *   dtype: FA_BF16 or FA_F16.  Same causal convention as fa_fwd.
 *   workspace: device memory of at least fa_bwd_workspace_bytes(B, H, Nq)
 *   bytes (holds D), 16-byte aligned; contents on entry do not matter.
 *   Results are deterministic (no floating-point atomics).
 */
size_t fa_bwd_workspace_bytes(int B, int H, int Nq);
fa_status fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
                 const float *lse, void *dq, void *dk, void *dv, int B, int H, int Hkv, int Nq,
                 int Nk, int d, int causal, float scale, fa_dtype dtype, void *workspace,
                 size_t workspace_bytes, void *stream);

/*
 * E4M3 quantisation for the FP8 forward, with optional incoherent processing
 * (marketmaker.cc flash-attention post, "FA3: Mecanica de la tolva", item 3:
 * rotate at random before block-wise quantisation, so outliers spread over
 * all coordinates).
 *   y     = H_d (s o x) if signs != NULL, else x.  H_d: Sylvester-Hadamard
 *           matrix (entries +-1, H_d^T H_d = d I), applied by the fast
 *           transform in fp32 in stages h = 1, 2, ..., d/2, each replacing
 *           (y_j, y_{j+h}) (j mod 2h < h) by (y_j + y_{j+h}, y_j - y_{j+h}).
 *           Rotating q and k with the same signs multiplies q.k by d exactly:
 *           pass scale / d to fa_fwd_fp8.
 *   group = layout 0: 32 consecutive rows of one (b, h) -> scales [B,H,ceil(N/32)];
 *           layout 1: one column of one (b, h)          -> scales [B,H,d];
 *           whole = 1: one group for the whole tensor, its scale repeated in
 *           every slot of the layout.
 *   scale = 2^e, e the smallest integer >= -126 with max|y| over the group
 *           <= 448 * 2^e (448: the largest finite E4M3 value).
 *   code  = E4M3_RNE(y * 2^-e) (OCP E4M3FN); the value is decode(code) * 2^e.
 *   x: device [B,H,N,d] in dtype (FA_F32 / FA_F16 / FA_BF16), 16-byte aligned;
 *   codes: device [B,H,N,d] bytes, 16-byte aligned; scales: device fp32 as
 *   above (also used as scratch by layout 1 and whole = 1; contents on entry
 *   do not matter); signs: NULL or device fp32 [d] of +1/-1.  d: 64 or 128;
 *   B*H <= 65535.  Inputs must be finite.
 */
fa_status fa_quant_e4m3(const void *x, uint8_t *codes, float *scales, const float *signs, int B,
                        int H, int N, int d, fa_dtype dtype, int layout, int whole, void *stream);

/*
 * FP8 forward (prefill): attention over dequantised E4M3 operands with the P
 * cast of gist.science "Resumen Tecnico: Precision de P-Cast en la Atencion
 * FP8" ("Planteamiento del Problema", "Optimizacion 1"), on the FP8 matrix
 * cores ("FA3: Mecanica de la tolva", item 3).  With qh, kh, vh the
 * dequantised values (code value times its group scale) the result is, per
 * query row, in KV tiles of fa_fp8_kv_tile() keys taken forward (or in
 * reverse if kv_reverse):
 *   s_j = scale * qh.kh_j;  m' = max(m, max_j s_j);  p_j = exp(s_j - m');
 *   l = e^(m - m') l + sum_j p_j;  acc = e^(m - m') acc + sum_j E4M3(p_scale p_j) vh_j;
 *   O = acc / (p_scale l),  LSE = m + ln l.
 *   q: [B,H,Nq,d] codes, q_scales [B,H,ceil(Nq/32)] (fa_quant_e4m3 layout 0);
 *   k: [B,Hkv,Nk,d] codes, k_scales [B,Hkv,ceil(Nk/32)] (layout 0);
 *   v: [B,Hkv,Nk,d] codes, v_scales [B,Hkv,d] (layout 1, 16-byte aligned).
 *   Scales are expected to be powers of two (as fa_quant_e4m3 writes them);
 *   the product q_scale * k_scale * scale is formed in fp32.
 *   o: [B,H,Nq,d] in o_dtype (FA_BF16 or FA_F32); lse: nullable [B,H,Nq].
 *   p_scale: a power of two in [1, 256].  Causal convention as fa_fwd.
 */
int fa_fp8_kv_tile(void);
fa_status fa_fwd_fp8(const uint8_t *q, const uint8_t *k, const uint8_t *v, const float *q_scales,
                     const float *k_scales, const float *v_scales, void *o, float *lse, int B, int H,
                     int Hkv, int Nq, int Nk, int d, int causal, float scale, float p_scale,
                     int kv_reverse, fa_dtype o_dtype, void *stream);

/*
 * The device E4M3 round trip that fa_fwd_pcast applies to p_scale * P, on n
 * fp32 values: codes[i] = E4M3_RNE(x[i]) (OCP E4M3FN bit pattern),
 * back[i] = the value of that code.  x, codes, back are device pointers
 * (codes and back may each be NULL).  Exposed so the conversion can be
 * checked against a reference codec.
 */
fa_status fa_cast_e4m3(const float *x, uint8_t *codes, float *back, size_t n, void *stream);

const char *fa_status_str(fa_status s);

/* Library version, major*10000 + minor*100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
