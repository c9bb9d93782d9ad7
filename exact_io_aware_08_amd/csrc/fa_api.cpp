// fa_api.cpp -- the C ABI of libfa (declared in include/fa.h): host-side
// validation, device check, and dispatch to the gfx950 kernels.
//
// Every argument is checked before anything is launched; on an error the
// call returns a status and writes nothing.  There is no fallback path: an
// unsupported combination is an error (the risk of silent fallback is the
// point made in marketmaker.cc, "La integracion es de ocho lineas").
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>

#include "fa.h"
#include "fa_internal.hpp"

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
int g_dev_ok[kMaxDevices];

// 1 if the current device is gfx950, 0 if not, -1 if it cannot be queried.
int current_device_ok()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
    std::call_once(g_dev_once[dev], [dev]() {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            g_dev_ok[dev] = -1;
            return;
        }
        g_dev_ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
    });
    return g_dev_ok[dev];
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

fa_status device_status()
{
    const int ok = current_device_ok();
    return ok == 1 ? FA_OK : FA_ERR_DEVICE;
}

fa_status hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

constexpr long long kMaxSlice = (1LL << 31) - 1;

// Shape checks common to the forward entry points (pointers checked apart).
// Every entry point takes d = 64 and 128; `allow256` admits d = 256 (the
// bf16/fp16 forward only).
fa_status check_fwd_shape(int B, int H, int Hkv, int Nq, int Nk, int d, float scale,
                          bool allow256 = false)
{
    if (B < 0 || H < 1 || Hkv < 1 || Nq < 0 || Nk < 0) return FA_ERR_SHAPE;
    if (d != 64 && d != 128 && !(allow256 && d == 256)) return FA_ERR_HEADDIM;
    if (H % Hkv != 0) return FA_ERR_GQA;
    if ((long long)Nq * d > kMaxSlice || (long long)Nk * d > kMaxSlice) return FA_ERR_SHAPE;
    const long long qtiles = ((long long)Nq + fa::kFwdQTile - 1) / fa::kFwdQTile;
    if (qtiles * B * H > kMaxSlice) return FA_ERR_SHAPE;
    if (!(std::isfinite(scale) && scale > 0.f)) return FA_ERR_SCALE;
    return FA_OK;
}

// Pointers of empty tensors may be NULL: q, o, lse are only needed when
// B*Nq > 0, and k, v when B*Nk > 0.
fa_status check_fwd_ptrs(const void *q, const void *k, const void *v, const void *o,
                         const void *lse, int B, int Nq, int Nk)
{
    const bool need_q = B > 0 && Nq > 0, need_kv = B > 0 && Nk > 0;
    if ((need_q && (!q || !o)) || (need_kv && (!k || !v))) return FA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_ALIGN;
    if (lse && !aligned16(lse)) return FA_ERR_ALIGN;
    return FA_OK;
}

int auto_splits(int B, int H, int Hkv, int Nk)
{
    const int G = H / Hkv;
    const long long base = (long long)B * Hkv * ((G + 15) / 16);
    if (base <= 0 || Nk <= 0) return 1;
    // about one workgroup per CU (256), no split shorter than 512 keys: the
    // sweep streams at the same rate with fewer, longer slices, and fewer
    // splits leave less to merge
    long long s = (256 + base - 1) / base;
    const long long max_s = ((long long)Nk + 511) / 512;
    if (s > max_s) s = max_s;
    if (s < 1) s = 1;
    if (s > 4096) s = 4096;
    return (int)s;
}

int decode_chunk(int Nk, int splits, int d)
{
    const long long gran = fa::decode_chunk_keys(d);
    long long ch = ((long long)Nk + splits - 1) / splits;
    ch = ((ch + gran - 1) / gran) * gran;
    return ch < gran ? (int)gran : (int)ch;
}

// Decode workspace: [per-split LSE | per-split O | per-sequence split
// counts (automatic paged splits only)], each part starting on a 256-byte
// boundary.  No workspace without a split.
struct DecodeLayout {
    size_t lse_off, o_off, cnt_off, total;
};

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

DecodeLayout decode_layout(int B, int H, int Hkv, int d, int splits, bool counts = false)
{
    DecodeLayout L{0, 0, 0, 0};
    if (splits <= 1) return L;
    const size_t rows = (size_t)B * H * splits;
    L.lse_off = 0;
    L.o_off = round256(rows * sizeof(float));
    L.total = L.o_off + rows * (size_t)d * sizeof(float);
    if (counts) {
        L.cnt_off = round256(L.total);
        L.total = L.cnt_off + (size_t)B * sizeof(int);
    }
    return L;
}

}  // namespace

extern "C" {

fa_status fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                 int Hkv, int Nq, int Nk, int d, int causal, float scale, fa_dtype dtype,
                 void *stream)
{
    fa_status s = check_fwd_shape(B, H, Hkv, Nq, Nk, d, scale, dtype == FA_F16 || dtype == FA_BF16);
    if (s != FA_OK) return s;
    if ((s = check_fwd_ptrs(q, k, v, o, lse, B, Nq, Nk)) != FA_OK) return s;
    if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
    if (causal != 0 && causal != 1) return FA_ERR_ARG;
    if (B == 0 || Nq == 0) return FA_OK;
    if ((s = device_status()) != FA_OK) return s;
    fa::FwdProblem p{};
    p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
    p.B = B; p.H = H; p.Hkv = Hkv; p.Nq = Nq; p.Nk = Nk; p.d = d;
    p.causal = causal; p.scale = scale; p.dtype = (int)dtype;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == FA_F32) return hip_status(fa::launch_fwd_f32(p, st));
    return hip_status(fa::launch_fwd_mfma(p, st));
}

fa_status fa_fwd_pcast(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                       int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                       fa_dtype dtype, float p_scale, int kv_reverse, int n_sink,
                       unsigned long long *counts, void *stream)
{
    fa_status s = check_fwd_shape(B, H, Hkv, Nq, Nk, d, scale);
    if (s != FA_OK) return s;
    if ((s = check_fwd_ptrs(q, k, v, o, lse, B, Nq, Nk)) != FA_OK) return s;
    if (counts && (reinterpret_cast<uintptr_t>(counts) & 7u)) return FA_ERR_ALIGN;
    if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_DTYPE;
    if (!(std::isfinite(p_scale) && p_scale > 0.f && p_scale <= 448.f)) return FA_ERR_SCALE;
    if ((causal != 0 && causal != 1) || (kv_reverse & ~3) != 0 || n_sink < 0) return FA_ERR_ARG;
    if (B == 0 || Nq == 0) return FA_OK;
    if ((s = device_status()) != FA_OK) return s;
    fa::FwdProblem p{};
    p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
    p.B = B; p.H = H; p.Hkv = Hkv; p.Nq = Nq; p.Nk = Nk; p.d = d;
    p.causal = causal; p.scale = scale; p.dtype = (int)dtype;
    p.pcast = 1; p.p_scale = p_scale; p.kv_reverse = kv_reverse; p.n_sink = n_sink;
    p.counts = counts;
    return hip_status(fa::launch_fwd_f32(p, static_cast<hipStream_t>(stream)));
}

int fa_kv_tile(fa_dtype dtype, int d, int pcast)
{
    if (d == 256 && !pcast && (dtype == FA_F16 || dtype == FA_BF16))
        return fa::fwd_mfma_kv_tile(d, 1, 1, 1LL << 30);
    if (d != 64 && d != 128) return -1;
    if (dtype == FA_F32 || (pcast && dtype == FA_BF16)) return fa::fwd_f32_kv_tile(d);
    if (pcast) return -1;
    if (dtype == FA_F16 || dtype == FA_BF16) return fa::fwd_mfma_kv_tile(d, 1, 1, 1LL << 30);
    return -1;
}

int fa_decode_splits(int B, int H, int Hkv, int Nk, int num_splits)
{
    if (B < 0 || H < 1 || Hkv < 1 || H % Hkv || Nk < 0 || num_splits < 0 || num_splits > 4096)
        return -1;
    return num_splits > 0 ? num_splits : auto_splits(B, H, Hkv, Nk);
}

size_t fa_decode_workspace_bytes(int B, int H, int Hkv, int Nk, int d, int num_splits)
{
    const int s = fa_decode_splits(B, H, Hkv, Nk, num_splits);
    if (s < 0 || (d != 64 && d != 128)) return 0;
    return decode_layout(B, H, Hkv, d, s).total;
}

fa_status fa_decode(const void *q, const void *k_cache, const void *v_cache, void *o, float *lse,
                    int B, int H, int Hkv, int Nk, int d, float scale, fa_dtype dtype,
                    int num_splits, void *workspace, size_t workspace_bytes, void *stream)
{
    fa_status s = check_fwd_shape(B, H, Hkv, 1, Nk, d, scale);
    if (s != FA_OK) return s;
    if ((s = check_fwd_ptrs(q, k_cache, v_cache, o, lse, B, 1, Nk)) != FA_OK) return s;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
    if (num_splits < 0 || num_splits > 4096) return FA_ERR_ARG;
    const int splits = fa_decode_splits(B, H, Hkv, Nk, num_splits);
    const DecodeLayout lay = decode_layout(B, H, Hkv, d, splits);
    if (lay.total > 0 && (!workspace || workspace_bytes < lay.total)) return FA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA_ERR_ALIGN;
    const long long blocks = (long long)splits * B * Hkv * ((H / Hkv + 15) / 16);
    if (blocks > kMaxSlice) return FA_ERR_SHAPE;
    if (B == 0) return FA_OK;
    if ((s = device_status()) != FA_OK) return s;
    fa::DecodeProblem p{};
    p.q = q; p.k = k_cache; p.v = v_cache; p.o = o; p.lse = lse;
    p.B = B; p.H = H; p.Hkv = Hkv; p.Nk = Nk; p.d = d; p.scale = scale; p.dtype = (int)dtype;
    p.splits = splits;
    p.chunk = decode_chunk(Nk, splits, d);
    if (lay.total > 0) {
        char *ws = static_cast<char *>(workspace);
        p.part_lse = reinterpret_cast<float *>(ws + lay.lse_off);
        p.part_o = reinterpret_cast<float *>(ws + lay.o_off);
    }
    return hip_status(fa::launch_decode(p, static_cast<hipStream_t>(stream)));
}

fa_status fa_decode_noalloc(const void *q, const void *k_cache, const void *v_cache, void *o,
                            float *lse, int B, int H, int Hkv, int Nk, int d, float scale,
                            fa_dtype dtype, int num_splits, void *stream)
{
    fa_status s = check_fwd_shape(B, H, Hkv, 1, Nk, d, scale);
    if (s != FA_OK) return s;
    if ((s = check_fwd_ptrs(q, k_cache, v_cache, o, lse, B, 1, Nk)) != FA_OK) return s;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
    if (num_splits < 0 || num_splits > 4096) return FA_ERR_ARG;
    const int splits = fa_decode_splits(B, H, Hkv, Nk, num_splits);
    const DecodeLayout lay = decode_layout(B, H, Hkv, d, splits);
    if (lay.total > fa::kDecodeScratchBytes) return FA_ERR_SCRATCH;
    const long long blocks = (long long)splits * B * Hkv * ((H / Hkv + 15) / 16);
    if (blocks > kMaxSlice) return FA_ERR_SHAPE;
    if (B == 0) return FA_OK;
    if ((s = device_status()) != FA_OK) return s;
    fa::DecodeProblem p{};
    p.q = q; p.k = k_cache; p.v = v_cache; p.o = o; p.lse = lse;
    p.B = B; p.H = H; p.Hkv = Hkv; p.Nk = Nk; p.d = d; p.scale = scale; p.dtype = (int)dtype;
    p.splits = splits;
    p.chunk = decode_chunk(Nk, splits, d);
    if (lay.total > 0) {
        void *ws = nullptr;
        if (fa::decode_scratch(&ws) != hipSuccess || ws == nullptr) return FA_ERR_HIP;
        char *base = static_cast<char *>(ws);
        p.part_lse = reinterpret_cast<float *>(base + lay.lse_off);
        p.part_o = reinterpret_cast<float *>(base + lay.o_off);
    }
    return hip_status(fa::launch_decode(p, static_cast<hipStream_t>(stream)));
}

fa_status fa_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                          const int *block_table, const int *seq_lens, void *o, float *lse,
                          int B, int H, int Hkv, int num_pages, int page_size, int max_pages,
                          int d, float scale, fa_dtype dtype, int num_splits, void *workspace,
                          size_t workspace_bytes, void *stream)
{
    if (B < 0 || num_pages < 0 || max_pages < 1 || page_size < 32 || page_size % 32 != 0)
        return B < 0 ? FA_ERR_SHAPE : FA_ERR_ARG;
    const long long max_seq = (long long)max_pages * page_size;
    if (max_seq > kMaxSlice / 128) return FA_ERR_SHAPE;
    if ((long long)num_pages * Hkv * page_size * d > (1LL << 40)) return FA_ERR_SHAPE;
    fa_status s = check_fwd_shape(B, H, Hkv, 1, (int)max_seq, d, scale);
    if (s != FA_OK) return s;
    if (B > 0 && (!q || !o || !block_table || !seq_lens)) return FA_ERR_NULL;
    if (B > 0 && num_pages > 0 && (!k_pages || !v_pages)) return FA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o) ||
        (lse && !aligned16(lse)))
        return FA_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
        return FA_ERR_ALIGN;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
    if (num_splits < 0 || num_splits > 4096) return FA_ERR_ARG;
    const int hq = Hkv * ((H / Hkv + 15) / 16);  // workgroups per (sequence, split)
    const bool auto_split = num_splits == 0 && B <= fa::kPagedAutoMaxBatch;
    const int splits = auto_split ? fa::paged_auto_max_splits(max_seq, hq)
                                  : fa_decode_splits(B, H, Hkv, (int)max_seq, num_splits);
    const DecodeLayout lay = decode_layout(B, H, Hkv, d, splits, auto_split);
    if (lay.total > 0 && (!workspace || workspace_bytes < lay.total)) return FA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA_ERR_ALIGN;
    const long long blocks = (auto_split ? fa::paged_auto_pairs(B, hq, splits) : (long long)splits * B) * hq;
    if (blocks > kMaxSlice) return FA_ERR_SHAPE;
    if (B == 0) return FA_OK;
    if ((s = device_status()) != FA_OK) return s;
    fa::DecodeProblem p{};
    p.q = q; p.k = k_pages; p.v = v_pages; p.o = o; p.lse = lse;
    p.B = B; p.H = H; p.Hkv = Hkv; p.Nk = (int)max_seq; p.d = d; p.scale = scale;
    p.dtype = (int)dtype;
    p.splits = splits;
    p.chunk = decode_chunk((int)max_seq, splits, d);
    p.auto_split = auto_split ? 1 : 0;
    if (lay.total > 0) {
        char *ws = static_cast<char *>(workspace);
        p.part_lse = reinterpret_cast<float *>(ws + lay.lse_off);
        p.part_o = reinterpret_cast<float *>(ws + lay.o_off);
        if (auto_split) p.split_counts = reinterpret_cast<int *>(ws + lay.cnt_off);
    }
    p.block_table = block_table; p.seq_lens = seq_lens;
    p.page_size = page_size; p.max_pages = max_pages; p.num_pages = num_pages;
    return hip_status(fa::launch_decode(p, static_cast<hipStream_t>(stream)));
}

size_t fa_decode_paged_workspace_bytes(int B, int H, int Hkv, int max_pages, int page_size, int d,
                                       int num_splits)
{
    if (B < 0 || H < 1 || Hkv < 1 || H % Hkv || max_pages < 1 || page_size < 32 ||
        num_splits < 0 || num_splits > 4096 || (d != 64 && d != 128))
        return 0;
    const long long max_seq = (long long)max_pages * page_size;
    if (max_seq > kMaxSlice / 128) return 0;
    if (num_splits > 0 || B > fa::kPagedAutoMaxBatch)
        return fa_decode_workspace_bytes(B, H, Hkv, (int)max_seq, d, num_splits);
    const int hq = Hkv * ((H / Hkv + 15) / 16);
    return decode_layout(B, H, Hkv, d, fa::paged_auto_max_splits(max_seq, hq), true).total;
}

size_t fa_bwd_workspace_bytes(int B, int H, int Nq)
{
    if (B < 0 || H < 1 || Nq < 0) return 0;
    return round256((size_t)B * (size_t)H * (size_t)Nq * sizeof(float));
}

fa_status fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
                 const float *lse, void *dq, void *dk, void *dv, int B, int H, int Hkv, int Nq,
                 int Nk, int d, int causal, float scale, fa_dtype dtype, void *workspace,
                 size_t workspace_bytes, void *stream)
{
    fa_status s = check_fwd_shape(B, H, Hkv, Nq, Nk, d, scale);
    if (s != FA_OK) return s;
    // q-side tensors are needed when B*Nq > 0, k-side ones when B*Nk > 0
    if ((s = check_fwd_ptrs(q, k, v, dq, lse, B, Nq, Nk)) != FA_OK) return s;
    const bool need_q = B > 0 && Nq > 0, need_kv = B > 0 && Nk > 0;
    if (need_q && (!o || !dout || !lse)) return FA_ERR_NULL;
    if (need_kv && (!dk || !dv)) return FA_ERR_NULL;
    if (!aligned16(o) || !aligned16(dout) || !aligned16(dk) || !aligned16(dv)) return FA_ERR_ALIGN;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
    if (causal != 0 && causal != 1) return FA_ERR_ARG;
    const size_t need = fa_bwd_workspace_bytes(B, H, Nq);
    if (need > 0 && (!workspace || workspace_bytes < need)) return FA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA_ERR_ALIGN;
    if ((long long)((Nk + 127) / 128) * B * Hkv > kMaxSlice) return FA_ERR_SHAPE;
    if (B == 0 || (Nq == 0 && Nk == 0)) return FA_OK;
    if ((s = device_status()) != FA_OK) return s;
    fa::BwdProblem p{};
    p.q = q; p.k = k; p.v = v; p.o = o; p.dout = dout; p.lse = lse;
    p.dq = dq; p.dk = dk; p.dv = dv; p.dvec = static_cast<float *>(workspace);
    p.B = B; p.H = H; p.Hkv = Hkv; p.Nq = Nq; p.Nk = Nk; p.d = d;
    p.causal = causal; p.scale = scale; p.dtype = (int)dtype;
    return hip_status(fa::launch_bwd(p, static_cast<hipStream_t>(stream)));
}

fa_status fa_quant_e4m3(const void *x, uint8_t *codes, float *scales, const float *signs, int B,
                        int H, int N, int d, fa_dtype dtype, int layout, int whole, void *stream)
{
    if (B < 0 || H < 1 || N < 0) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEADDIM;
    if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
    if ((layout != 0 && layout != 1) || (whole != 0 && whole != 1)) return FA_ERR_ARG;
    if ((long long)N * d > kMaxSlice || (long long)B * H > 65535) return FA_ERR_SHAPE;
    if (B == 0 || N == 0) return FA_OK;
    if (!x || !codes || !scales) return FA_ERR_NULL;
    if (!aligned16(x) || !aligned16(codes) || (reinterpret_cast<uintptr_t>(scales) & 3u) ||
        (reinterpret_cast<uintptr_t>(signs) & 3u))
        return FA_ERR_ALIGN;
    fa_status s = device_status();
    if (s != FA_OK) return s;
    fa::QuantProblem p{x, codes, scales, signs, B * H, N, d, (int)dtype, layout, whole};
    return hip_status(fa::launch_quant(p, static_cast<hipStream_t>(stream)));
}

int fa_fp8_kv_tile(void) { return fa::fwd_fp8_kv_tile(); }

fa_status fa_fwd_fp8(const uint8_t *q, const uint8_t *k, const uint8_t *v, const float *q_scales,
                     const float *k_scales, const float *v_scales, void *o, float *lse, int B, int H,
                     int Hkv, int Nq, int Nk, int d, int causal, float scale, float p_scale,
                     int kv_reverse, fa_dtype o_dtype, void *stream)
{
    fa_status s = check_fwd_shape(B, H, Hkv, Nq, Nk, d, scale);
    if (s != FA_OK) return s;
    if ((s = check_fwd_ptrs(q, k, v, o, lse, B, Nq, Nk)) != FA_OK) return s;
    const bool need_q = B > 0 && Nq > 0, need_kv = B > 0 && Nk > 0;
    if ((need_q && !q_scales) || (need_kv && (!k_scales || !v_scales))) return FA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(q_scales) & 3u) || (reinterpret_cast<uintptr_t>(k_scales) & 3u) ||
        !aligned16(v_scales))
        return FA_ERR_ALIGN;
    // S: a power of two in [1, 256], so S * p <= 256 < 448 and S divides out exactly
    int e2 = 0;
    if (!(std::isfinite(p_scale) && p_scale >= 1.f && p_scale <= 256.f) ||
        std::frexp(p_scale, &e2) != 0.5f)
        return FA_ERR_SCALE;
    if (o_dtype != FA_F32 && o_dtype != FA_BF16) return FA_ERR_DTYPE;
    if ((causal != 0 && causal != 1) || (kv_reverse != 0 && kv_reverse != 1)) return FA_ERR_ARG;
    if (!need_q) return FA_OK;
    if ((s = device_status()) != FA_OK) return s;
    fa::Fp8Problem p{q, k, v, q_scales, k_scales, v_scales, o, lse, B, H, Hkv, Nq, Nk, d,
                     causal, scale, p_scale, kv_reverse, o_dtype == FA_F32 ? 0 : 2};
    return hip_status(fa::launch_fwd_fp8(p, static_cast<hipStream_t>(stream)));
}

fa_status fa_cast_e4m3(const float *x, uint8_t *codes, float *back, size_t n, void *stream)
{
    if (n == 0) return FA_OK;
    if (!x) return FA_ERR_NULL;
    if (n > (size_t)kMaxSlice * 256) return FA_ERR_SHAPE;
    fa_status s = device_status();
    if (s != FA_OK) return s;
    return hip_status(fa::launch_cast_e4m3(x, codes, back, n, static_cast<hipStream_t>(stream)));
}

const char *fa_status_str(fa_status s)
{
    switch (s) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: negative size, H/Hkv < 1, or a tensor slice too large";
    case FA_ERR_HEADDIM: return "FA_ERR_HEADDIM: head dimension must be 64 or 128 (256: bf16/fp16 forward only)";
    case FA_ERR_GQA: return "FA_ERR_GQA: H must be a multiple of Hkv";
    case FA_ERR_DTYPE: return "FA_ERR_DTYPE: dtype not supported by this entry point";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: a pointer is not 16-byte aligned";
    case FA_ERR_SCALE: return "FA_ERR_SCALE: scale must be finite and > 0 (p_scale also <= 448)";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: decode workspace is NULL or too small";
    case FA_ERR_DEVICE: return "FA_ERR_DEVICE: the current device is not gfx950";
    case FA_ERR_HIP: return "FA_ERR_HIP: a HIP kernel launch failed";
    case FA_ERR_ARG: return "FA_ERR_ARG: an argument is out of range";
    case FA_ERR_SCRATCH:
        return "FA_ERR_SCRATCH: the partial results need more than the library's 8 MiB static "
               "decode scratch (fa_decode_noalloc); use fa_decode with a workspace";
    }
    return "unknown fa_status";
}

int fa_version(void) { return 100; }

}  // extern "C"
