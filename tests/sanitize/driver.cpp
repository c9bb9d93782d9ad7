// Host-only sanitizer run (AddressSanitizer + UndefinedBehaviorSanitizer) of
// libfa's C ABI argument validation (fa_api.cpp, linked with stub launchers
// that report no device) and of the fp64 CPU oracle on tiny inputs.  Every
// error code is forced from the host, every call that passes validation must
// stop at FA_ERR_DEVICE, and the size helpers run on extreme arguments.
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "fa.h"

typedef long long i64;
typedef unsigned long long u64;
extern "C" {
int orc_attention(const float *q, const float *k, const float *v, i64 B, i64 H, i64 Hkv, i64 Nq,
                  i64 Nk, i64 d, int causal, double scale, const i64 *rows, i64 nrows, double *o,
                  double *lse, int nthreads);
int orc_attention_bwd(const float *q, const float *k, const float *v, const float *dout, i64 B,
                      i64 H, i64 Hkv, i64 Nq, i64 Nk, i64 d, int causal, double scale, double *dq,
                      double *dk, double *dv, double *adq, double *adk, double *adv, int nthreads);
int orc_pcast(const float *q, const float *k, const float *v, i64 B, i64 H, i64 Hkv, i64 Nq, i64 Nk,
              i64 d, int causal, float scale, int kv_tile, float p_scale, int reverse, i64 n_sink,
              const i64 *rows, i64 nrows, double *o, double *lse, u64 *counts, int nthreads);
int orc_quant_e4m3(const float *x, i64 B, i64 H, i64 N, i64 d, const float *signs, int layout,
                   int whole, unsigned char *codes, float *scales);
float orc_e4m3_decode(unsigned code);
unsigned orc_e4m3_encode(float x);
}

static int failures = 0;
#define CHECK(cond)                                                       \
    do {                                                                  \
        if (!(cond)) {                                                    \
            std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

int main()
{
    // Device pointers are never dereferenced on the host: aligned stand-ins.
    void *P = reinterpret_cast<void *>(0x10000);
    void *PM = reinterpret_cast<void *>(0x10004);  // not 16-byte aligned
    float *PF = static_cast<float *>(P);
    const uint8_t *P8 = static_cast<const uint8_t *>(P);

    // ---- fa_fwd ----
    CHECK(fa_fwd(P, P, P, P, PF, 1, 2, 1, 8, 8, 64, 1, 0.125f, FA_BF16, nullptr) == FA_ERR_DEVICE);
    CHECK(fa_fwd(nullptr, P, P, P, PF, 1, 2, 1, 8, 8, 64, 1, 0.125f, FA_BF16, nullptr) == FA_ERR_NULL);
    CHECK(fa_fwd(P, PM, P, P, PF, 1, 2, 1, 8, 8, 64, 1, 0.125f, FA_BF16, nullptr) == FA_ERR_ALIGN);
    CHECK(fa_fwd(P, P, P, P, PF, 1, 2, 1, 8, 8, 96, 1, 0.125f, FA_BF16, nullptr) == FA_ERR_HEADDIM);
    CHECK(fa_fwd(P, P, P, P, PF, 1, 2, 1, 8, 8, 256, 1, 0.125f, FA_F32, nullptr) == FA_ERR_HEADDIM);
    CHECK(fa_fwd(P, P, P, P, PF, 1, 2, 1, 8, 8, 256, 1, 0.125f, FA_F16, nullptr) == FA_ERR_DEVICE);
    CHECK(fa_fwd(P, P, P, P, PF, 1, 3, 2, 8, 8, 64, 1, 0.125f, FA_BF16, nullptr) == FA_ERR_GQA);
    CHECK(fa_fwd(P, P, P, P, PF, 1, 2, 1, 8, 8, 64, 1, 0.125f, (fa_dtype)7, nullptr) == FA_ERR_DTYPE);
    CHECK(fa_fwd(P, P, P, P, PF, 1, 2, 1, 8, 8, 64, 1, NAN, FA_BF16, nullptr) == FA_ERR_SCALE);
    CHECK(fa_fwd(P, P, P, P, PF, 1, 2, 1, 8, 8, 64, 2, 0.125f, FA_BF16, nullptr) == FA_ERR_ARG);
    CHECK(fa_fwd(P, P, P, P, PF, 0, 2, 1, 8, 8, 64, 1, 0.125f, FA_BF16, nullptr) == FA_OK);
    CHECK(fa_fwd(P, P, P, P, PF, INT_MAX, INT_MAX, 1, INT_MAX, INT_MAX, 64, 1, 0.125f, FA_BF16,
                 nullptr) == FA_ERR_SHAPE);
    CHECK(fa_fwd(P, P, P, P, PF, -1, 2, 1, 8, 8, 64, 1, 0.125f, FA_BF16, nullptr) == FA_ERR_SHAPE);

    // ---- fa_fwd_pcast ----
    CHECK(fa_fwd_pcast(P, P, P, P, PF, 1, 2, 2, 8, 8, 128, 1, 0.088f, FA_F32, 256.f, 1, 4,
                       static_cast<unsigned long long *>(P), nullptr) == FA_ERR_DEVICE);
    CHECK(fa_fwd_pcast(P, P, P, P, PF, 1, 2, 2, 8, 8, 128, 1, 0.088f, FA_F32, 512.f, 1, 4, nullptr,
                       nullptr) == FA_ERR_SCALE);
    CHECK(fa_fwd_pcast(P, P, P, P, PF, 1, 2, 2, 8, 8, 128, 1, 0.088f, FA_F32, 256.f, 4, 4, nullptr,
                       nullptr) == FA_ERR_ARG);
    CHECK(fa_fwd_pcast(P, P, P, P, PF, 1, 2, 2, 8, 8, 128, 1, 0.088f, FA_F16, 256.f, 1, 4, nullptr,
                       nullptr) == FA_ERR_DTYPE);

    // ---- decode ----
    const size_t ws = fa_decode_workspace_bytes(2, 8, 2, 100, 64, 3);
    CHECK(ws > 0);
    CHECK(fa_decode(P, P, P, P, PF, 2, 8, 2, 100, 64, 0.125f, FA_BF16, 3, P, ws, nullptr) == FA_ERR_DEVICE);
    CHECK(fa_decode(P, P, P, P, PF, 2, 8, 2, 100, 64, 0.125f, FA_BF16, 3, P, 16, nullptr) ==
          FA_ERR_WORKSPACE);
    CHECK(fa_decode(P, P, P, P, PF, 2, 8, 2, 100, 64, 0.125f, FA_BF16, 5000, P, ws, nullptr) ==
          FA_ERR_ARG);
    CHECK(fa_decode(P, P, P, P, PF, 2, 8, 2, 100, 64, 0.125f, FA_F32, 3, P, ws, nullptr) ==
          FA_ERR_DTYPE);
    // no-alloc decode: validation as fa_decode, then the static-scratch limit
    CHECK(fa_decode_noalloc(P, P, P, P, PF, 16, 32, 4, 8192, 64, 0.125f, FA_BF16, 0, nullptr) ==
          FA_ERR_DEVICE);
    CHECK(fa_decode_noalloc(P, P, P, P, PF, 64, 64, 8, 1 << 20, 128, 0.125f, FA_BF16, 64, nullptr) ==
          FA_ERR_SCRATCH);
    CHECK(fa_decode_noalloc(P, P, P, P, PF, 2, 8, 3, 100, 64, 0.125f, FA_BF16, 0, nullptr) == FA_ERR_GQA);
    CHECK(fa_decode_noalloc(nullptr, P, P, P, PF, 2, 8, 2, 100, 64, 0.125f, FA_BF16, 0, nullptr) ==
          FA_ERR_NULL);
    CHECK(fa_decode_noalloc(P, P, P, P, PF, 0, 8, 2, 100, 64, 0.125f, FA_BF16, 0, nullptr) == FA_OK);
    const int *PI = static_cast<const int *>(P);
    CHECK(fa_decode_paged(P, P, P, PI, PI, P, PF, 2, 8, 2, 16, 128, 8, 64, 0.125f, FA_BF16, 0, P,
                          fa_decode_paged_workspace_bytes(2, 8, 2, 8, 128, 64, 0), nullptr) == FA_ERR_DEVICE);
    // automatic splits need room for more splits than the contiguous default
    CHECK(fa_decode_paged(P, P, P, PI, PI, P, PF, 2, 8, 2, 16, 128, 8, 64, 0.125f, FA_BF16, 0, P,
                          fa_decode_workspace_bytes(2, 8, 2, 1024, 64, 0), nullptr) == FA_ERR_WORKSPACE);
    CHECK(fa_decode_paged(P, P, P, PI, PI, P, PF, 2, 8, 2, 16, 128, 8, 64, 0.125f, FA_BF16, 4, P,
                          fa_decode_paged_workspace_bytes(2, 8, 2, 8, 128, 64, 4), nullptr) == FA_ERR_DEVICE);
    CHECK(fa_decode_paged(P, P, P, nullptr, PI, P, PF, 2, 8, 2, 16, 128, 8, 64, 0.125f, FA_BF16, 0, P,
                          1 << 20, nullptr) == FA_ERR_NULL);

    // ---- backward, FP8, casts ----
    const size_t bws = fa_bwd_workspace_bytes(1, 2, 8);
    CHECK(fa_bwd(P, P, P, P, P, PF, P, P, P, 1, 2, 1, 8, 8, 64, 1, 0.125f, FA_BF16, P, bws, nullptr) ==
          FA_ERR_DEVICE);
    CHECK(fa_bwd(P, P, P, P, P, PF, P, P, P, 1, 2, 1, 8, 8, 64, 1, 0.125f, FA_F32, P, bws, nullptr) ==
          FA_ERR_DTYPE);
    CHECK(fa_bwd(P, P, P, P, P, PF, P, P, P, 1, 2, 1, 8, 8, 256, 1, 0.125f, FA_BF16, P, bws, nullptr) ==
          FA_ERR_HEADDIM);
    CHECK(fa_quant_e4m3(P, static_cast<uint8_t *>(P), PF, nullptr, 1, 2, 64, 64, FA_BF16, 2, 0,
                        nullptr) == FA_ERR_ARG);
    CHECK(fa_fwd_fp8(P8, P8, P8, PF, PF, PF, P, PF, 1, 2, 2, 64, 64, 64, 1, 0.002f, 3.f, 0, FA_BF16,
                     nullptr) == FA_ERR_SCALE);
    CHECK(fa_fwd_fp8(P8, P8, P8, PF, PF, PF, P, PF, 1, 2, 2, 64, 64, 64, 1, 0.002f, 256.f, 0, FA_BF16,
                     nullptr) == FA_ERR_DEVICE);
    CHECK(fa_cast_e4m3(nullptr, nullptr, nullptr, 4, nullptr) == FA_ERR_NULL);
    CHECK(fa_cast_e4m3(nullptr, nullptr, nullptr, 0, nullptr) == FA_OK);

    // ---- helpers on extreme arguments (no overflow, no out-of-range reads) ----
    for (int s = -2; s <= 13; ++s) CHECK(fa_status_str(static_cast<fa_status>(s)) != nullptr);
    const int big[] = {0, 1, 7, 4096, INT_MAX};
    for (int b : big)
        for (int n : big) {
            (void)fa_decode_splits(b, 32, 4, n, 0);
            (void)fa_decode_workspace_bytes(b, 32, 4, n, 64, 0);
            (void)fa_decode_paged_workspace_bytes(b, 32, 4, n, 32, 64, 0);
            (void)fa_decode_paged_workspace_bytes(b, 32, 4, n, 1 << 20, 128, 0);
            (void)fa_bwd_workspace_bytes(b, 32, n);
        }
    CHECK(fa_decode_splits(-1, 8, 2, 100, 0) == -1 && fa_decode_splits(1, 8, 3, 100, 0) == -1);
    CHECK(fa_kv_tile(FA_F32, 48, 0) == -1 && fa_version() == 100);

    // ---- oracle on tiny inputs ----
    const i64 B = 1, H = 2, Hkv = 1, N = 5, d = 8;
    std::vector<float> q(B * H * N * d), k(B * Hkv * N * d), v(B * Hkv * N * d), g(q.size());
    for (size_t i = 0; i < q.size(); ++i) q[i] = std::sin(0.37f * i) * 1.5f, g[i] = std::cos(0.11f * i);
    for (size_t i = 0; i < k.size(); ++i) k[i] = std::cos(0.23f * i), v[i] = std::sin(0.71f * i + 1.f);
    std::vector<double> o(q.size()), lse(B * H * N);
    CHECK(orc_attention(q.data(), k.data(), v.data(), B, H, Hkv, N, N, d, 1, 0.35, nullptr, 0,
                        o.data(), lse.data(), 2) == 0);
    for (i64 h = 0; h < H; ++h)  // causal row 0 sees key 0 only: O = V[0]
        for (i64 c = 0; c < d; ++c) CHECK(o[(h * N) * d + c] == static_cast<double>(v[c]));
    std::vector<float> vc(v.size(), 0.75f);  // constant values: every row's output is that value
    CHECK(orc_attention(q.data(), k.data(), vc.data(), B, H, Hkv, N, N, d, 0, 0.35, nullptr, 0,
                        o.data(), lse.data(), 2) == 0);
    for (double x : o) CHECK(std::fabs(x - 0.75) < 1e-12);
    std::vector<double> dq(q.size()), dk(k.size()), dv(v.size()), aq(q.size()), ak(k.size()),
        av(v.size());
    CHECK(orc_attention_bwd(q.data(), k.data(), v.data(), g.data(), B, H, Hkv, N, N, d, 1, 0.35,
                            dq.data(), dk.data(), dv.data(), aq.data(), ak.data(), av.data(), 2) == 0);
    for (double x : dk) CHECK(std::isfinite(x));
    u64 counts[4] = {0, 0, 0, 0};
    CHECK(orc_pcast(q.data(), k.data(), v.data(), B, H, Hkv, N, N, d, 1, 0.35f, 2, 256.f, 1, 1,
                    nullptr, 0, o.data(), lse.data(), counts, 2) == 0);
    CHECK(counts[0] > 0 && counts[1] <= counts[0]);
    std::vector<float> x(B * H * 64 * 64), signs(64), scales(2 * 64);
    for (size_t i = 0; i < x.size(); ++i) x[i] = std::sin(0.013f * i) * 3.f;
    for (int i = 0; i < 64; ++i) signs[i] = (i * 7 % 3) ? 1.f : -1.f;
    std::vector<unsigned char> codes(x.size());
    CHECK(orc_quant_e4m3(x.data(), B, H, 64, 64, signs.data(), 0, 0, codes.data(), scales.data()) == 0);
    CHECK(orc_quant_e4m3(x.data(), B, H, 64, 64, nullptr, 1, 0, codes.data(), scales.data()) == 0);
    for (unsigned code = 0; code < 256; ++code) {
        if ((code & 0x7f) == 0x7f) continue;  // NaN encodings
        const float f = orc_e4m3_decode(code);
        if (f == 0.f) continue;               // +0 and -0 encode alike
        CHECK(orc_e4m3_encode(f) == code);
    }

    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
