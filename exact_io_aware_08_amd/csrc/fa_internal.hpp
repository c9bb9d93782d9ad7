// fa_internal.hpp -- launcher interface between the C ABI (fa_api.cpp) and the
// gfx950 kernels.  Arguments are validated by the caller before any launcher
// runs; launchers only compute grids and enqueue kernels on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Forward (prefill) problem.  dtype: 0 = fp32, 1 = fp16, 2 = bf16.
struct FwdProblem {
    const void *q, *k, *v;
    void *o;
    float *lse;  // nullable
    int B, H, Hkv, Nq, Nk, d;
    int causal;
    float scale;
    int dtype;
    // E4M3 P-cast variant (fp32 kernel only)
    int pcast;
    float p_scale;
    int kv_reverse;  // bit 0: reverse KV order; bit 1: tile-local max (ablation)
    int n_sink;
    unsigned long long *counts;  // nullable, 4 entries
};

struct DecodeProblem {
    const void *q, *k, *v;
    void *o;
    float *lse;  // nullable
    int B, H, Hkv, Nk, d;
    float scale;
    int dtype;
    int splits;  // resolved (>= 1); with auto_split, the most splits a sequence can get
    int chunk;   // keys per split, multiple of decode_chunk_keys(d) (not used with auto_split)
    int auto_split;  // paged cache, automatic splits: the chunk follows the batch's total length
    float *part_o;    // [B, H, splits, d]  (splits > 1)
    float *part_lse;  // [B, H, splits]     (splits > 1)
    int *split_counts;  // [B] (automatic paged splits with splits > 1)
    // paged cache (block_table == nullptr: contiguous [B, Hkv, Nk, d])
    const int *block_table;  // [B, max_pages]
    const int *seq_lens;     // [B]
    int page_size, max_pages, num_pages;
};

// Backward problem (16-bit types).  dvec: [B, H, Nq] fp32 scratch for D.
struct BwdProblem {
    const void *q, *k, *v, *o, *dout;
    const float *lse;
    void *dq, *dk, *dv;
    float *dvec;
    int B, H, Hkv, Nq, Nk, d;
    int causal;
    float scale;
    int dtype;
};

// E4M3 quantisation of one [BH, N, d] tensor.  dtype: 0 = fp32, 1 = fp16,
// 2 = bf16.  layout 0: scales [BH, ceil(N/32)]; 1: scales [BH, d].
struct QuantProblem {
    const void *x;
    uint8_t *codes;
    float *scales;
    const float *signs;  // nullable: no rotation
    int BH, N, d;
    int dtype, layout, whole;
};

// FP8 forward: E4M3 codes with fp32 scales.  o_dtype: 0 = fp32, 2 = bf16.
struct Fp8Problem {
    const uint8_t *q, *k, *v;
    const float *q_scales, *k_scales, *v_scales;
    void *o;
    float *lse;  // nullable
    int B, H, Hkv, Nq, Nk, d;
    int causal;
    float scale, p_scale;
    int kv_reverse;
    int o_dtype;
};

// Tile constants shared by the launchers and fa_kv_tile().
constexpr int kFwdQTile = 128;     // fewest queries per forward workgroup (grid-size bound)
constexpr int kDecodeStep = 128;   // keys per decode workgroup step (4 waves x 32)

// Paged decode with automatic splits.  The kernels read the sequence lengths
// on the device and cut every sequence into chunks of
//   chunk = max(kPagedMinChunk, ceil(total_keys * hq / kPagedTargetItems)),
// rounded up to decode_chunk_keys(d), where hq is the number of workgroups
// per (sequence, split) pair (KV heads x query-head groups): about
// kPagedTargetItems workgroups in all, whatever the lengths.  Sequence b gets
// max(1, ceil(len_b / chunk)) splits, never more than paged_auto_max_splits()
// (chunk >= kPagedMinChunk and chunk >= len_b * hq / kPagedTargetItems), and
// the pairs never number more than ceil(kPagedTargetItems / hq) + B.
constexpr int kPagedTargetItems = 256;
constexpr int kPagedMinChunk = 512;
// Every workgroup scans the lengths 64 at a time (one dependent load per 64
// sequences), so automatic splits serve batches of up to this many
// sequences; larger batches take the uniform split, which already yields
// enough workgroups.
constexpr int kPagedAutoMaxBatch = 256;
inline int paged_auto_max_splits(long long max_seq, int hq)
{
    const long long by_len = (max_seq + kPagedMinChunk - 1) / kPagedMinChunk;
    const long long by_items = (kPagedTargetItems + hq - 1) / hq;
    const long long s = by_len < by_items ? by_len : by_items;
    return s < 1 ? 1 : (int)s;
}
inline long long paged_auto_pairs(int B, int hq, int smax)
{
    const long long a = (long long)smax * B;
    const long long b = (kPagedTargetItems + hq - 1) / hq + (long long)B;
    return a < b ? a : b;
}

// Static device scratch of fa_decode_noalloc (the split partials), per GPU.
constexpr size_t kDecodeScratchBytes = (size_t)8 << 20;
// Device address of the current device's scratch (looked up once per device).
hipError_t decode_scratch(void **ptr);

int fwd_f32_kv_tile(int d);   // keys per KV tile, fp32 / P-cast kernel
int fwd_mfma_kv_tile(int d, long long B, long long H, long long Nq);  // keys per KV tile, bf16 / fp16 kernel
int decode_chunk_keys(int d); // granularity of a decode split (keys)
hipError_t launch_fwd_mfma(const FwdProblem &p, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdProblem &p, hipStream_t stream);
hipError_t launch_decode(const DecodeProblem &p, hipStream_t stream);
hipError_t launch_bwd(const BwdProblem &p, hipStream_t stream);
hipError_t launch_quant(const QuantProblem &p, hipStream_t stream);
int fwd_fp8_kv_tile();        // keys per KV tile of the FP8 kernel (the P-cast tile)
hipError_t launch_fwd_fp8(const Fp8Problem &p, hipStream_t stream);
hipError_t launch_cast_e4m3(const float *x, uint8_t *codes, float *back, size_t n,
                            hipStream_t stream);

}  // namespace fa
