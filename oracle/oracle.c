/*
 * oracle.c -- plain, slow, obviously-correct CPU reference for exact attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg load this library.  It shares no code, header, table or
 * helper with the GPU library; both sides only consume the same seeded input
 * buffers.  Build: gcc -O2 -ffp-contract=off (no -ffast-math), so every
 * floating-point step below is one plain IEEE double operation.
 *
 * Pages cited (title, then section):
 *  [MM] marketmaker.cc, "Atencion flash y la pregunta sobre la longitud de la
 *       secuencia" (Spanish blog post on flash attention for trading models)
 *  [SA] systems-analysis.info, "FlashAttention (IT)" (encyclopedia entry)
 *  [PC] gist.science, "Resumen Tecnico: Precision de P-Cast en la Atencion FP8"
 *  [FV] gist.science, "FlashAttention for Scalable Vector Architectures"
 *
 * Parity status of each function (what pins it is in tests/test_oracle_*.py):
 *  orc_attention ....... pinned (brute force at 50 digits, torch fp64 SDPA,
 *                         closed forms, invariants, online recurrence)
 *  orc_attention_probs . pinned (rows sum to 1, same pins as above)
 *  orc_pcast ........... pinned (identity case vs orc_attention, underflow
 *                         fraction vs the closed form F, reverse-order zero
 *                         count, brute-force tiny case)
 *  orc_e4m3_* .......... pinned (OCP constants printed on [PC], torch float8)
 *  orc_F, orc_delta_c .. pinned (printed constants and thresholds of [PC],
 *                         Monte Carlo of the model)
 *  orc_expected_max_gauss pinned (k=1 -> 0, k=2 -> 1/sqrt(pi), Monte Carlo)
 *  orc_dp .............. pinned (the two facts printed on [PC] "Optimizacion 2")
 *  orc_attention_bwd ... pinned (torch fp64 autograd of SDPA, central finite
 *                         differences of orc_attention, the sum rules
 *                         sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i)
 *  orc_quant_e4m3 ...... pinned (the explicit Sylvester-Hadamard matrix on
 *                         exactly representable inputs, brute-force search
 *                         of the minimal scale exponent, half-ulp round trip,
 *                         exact codes on the E4M3 grid, group layouts)
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef long long i64;
typedef unsigned long long u64;

/* ------------------------------------------------------------------------ */
/* Exact attention by its definition.                                       */
/*                                                                          */
/* [MM] "Por que la atencion esta ligada a la memoria" and [SA]             */
/* "Problematica dell'attention standard" define                            */
/*     O = softmax(Q K^T * scale) V,   scale = 1/sqrt(d_k),                 */
/* with the score matrix S = Q K^T * scale formed in full.  Here each score */
/* row is formed completely before its softmax (two passes over the row:    */
/* max, then exponentials and their sum), which is the plain definition.    */
/*                                                                          */
/* Readings where the pages are silent:                                     */
/*  - causal masking ([MM] "El enmascaramiento causal..."): key j is        */
/*    visible to query i iff j <= i + (Nk - Nq) (bottom-right alignment;    */
/*    equals the usual j <= i when Nq == Nk);                               */
/*  - GQA ([FV] "Metodologia": shared KV heads): query head h reads KV head */
/*    h / (H / Hkv);                                                        */
/*  - the per-row statistics (m, l) ([MM] "Pase hacia atras") are reported  */
/*    as LSE = m + ln(l) in natural log; a row with no visible key has      */
/*    O = 0 and LSE = -inf.                                                 */
/* ------------------------------------------------------------------------ */

typedef struct {
    const float *q, *k, *v;
    i64 B, H, Hkv, Nq, Nk, d;
    int causal;
    double scale;
    const i64 *rows;   /* [B*H][nrows] or NULL (all rows) */
    i64 nrows;
    double *o, *lse;
    /* p-cast emulation */
    int pcast;
    int kv_tile;
    float p_scale;
    float scale_f;
    int reverse;
    int tile_local;    /* ablation: P relative to each tile's own max */
    i64 n_sink;
    /* work distribution */
    i64 n_items;
    i64 next;          /* atomic */
    u64 cnt[4];        /* atomic */
} job_t;

static i64 visible_count(const job_t *J, i64 i)
{
    if (!J->causal) return J->Nk;
    i64 lim = i + (J->Nk - J->Nq) + 1;
    if (lim < 0) lim = 0;
    if (lim > J->Nk) lim = J->Nk;
    return lim;
}

static double dot(const float *a, const float *b, i64 d)
{
    double acc = 0.0;
    for (i64 c = 0; c < d; ++c) acc += (double)a[c] * (double)b[c];
    return acc;
}

/* One row of the definition: fills s[0..lim) with the scores, then p. */
static void exact_row(const job_t *J, i64 b, i64 h, i64 i, double *s, double *o_row,
                      double *lse_out)
{
    const i64 d = J->d, g = J->H / J->Hkv, hk = h / g;
    const float *qi = J->q + ((b * J->H + h) * J->Nq + i) * d;
    const float *kb = J->k + (b * J->Hkv + hk) * J->Nk * d;
    const float *vb = J->v + (b * J->Hkv + hk) * J->Nk * d;
    const i64 lim = visible_count(J, i);
    for (i64 c = 0; c < d; ++c) o_row[c] = 0.0;
    if (lim == 0) { *lse_out = -INFINITY; return; }
    double m = -INFINITY;
    for (i64 j = 0; j < lim; ++j) {
        s[j] = J->scale * dot(qi, kb + j * d, d);
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (i64 j = 0; j < lim; ++j) { s[j] = exp(s[j] - m); l += s[j]; }
    for (i64 j = 0; j < lim; ++j) {
        const double p = s[j] / l;
        const float *vj = vb + j * d;
        for (i64 c = 0; c < d; ++c) o_row[c] += p * (double)vj[c];
    }
    *lse_out = m + log(l);
}

/* ------------------------------------------------------------------------ */
/* E4M3 (OCP 8-bit floating point, "E4M3FN" variant): 1 sign bit, 4        */
/* exponent bits with bias 7, 3 mantissa bits, no infinities, the all-ones  */
/* magnitude 0x7F is NaN.  Largest finite 448, smallest normal 2^-6,        */
/* subnormals m * 2^-9.  [PC] "Planteamiento del Problema" names the format */
/* (3-bit mantissa); [PC] "Marco Teorico" gives the round-to-zero threshold */
/* 2^-10 and "Optimizacion 2" the bound S <= 448 and 2^-6.                  */
/* Encoding rounds to nearest, ties to even; magnitudes at or above 464     */
/* (the midpoint above 448) saturate to 448.                                */
/* ------------------------------------------------------------------------ */

float orc_e4m3_decode(unsigned code)
{
    code &= 0xFF;
    const int sgn = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double a;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) a = ldexp((double)m, -9);
    else a = ldexp(1.0 + m / 8.0, e - 7);
    return (float)(sgn ? -a : a);
}

unsigned orc_e4m3_encode(float x)
{
    if (isnan(x)) return 0x7F;
    const unsigned sgn = signbit(x) ? 0x80u : 0u;
    const double a = fabs((double)x);
    if (a >= 464.0) return sgn | 0x7Eu;
    if (a < ldexp(1.0, -6)) {
        /* subnormal grid m * 2^-9; the product is exact, nearbyint is RNE */
        const double qv = nearbyint(a * 512.0);
        return sgn | (unsigned)qv;           /* qv == 8 is the code of 2^-6 */
    }
    int e2;
    frexp(a, &e2);
    int E = e2 - 1;                          /* a in [2^E, 2^(E+1)) */
    double qv = nearbyint(ldexp(a, 3 - E));  /* in [8, 16] */
    if (qv == 16.0) { qv = 8.0; E += 1; }
    return sgn | ((unsigned)(E + 7) << 3) | (unsigned)(qv - 8.0);
}

/* ------------------------------------------------------------------------ */
/* P-cast emulation.  [PC] "Planteamiento del Problema": the softmax        */
/* probabilities P are cast to E4M3 before the P*V product, after being     */
/* multiplied by a static scale S that is divided back out at the end; the  */
/* KV blocks of the online softmax run forward (0 -> N) or in reverse       */
/* (N -> 0) ("Optimizacion 1").  P is taken relative to the RUNNING maximum */
/* m, which is what lets early sink logits push later non-sink P under the  */
/* E4M3 range (the P-collapse described there).  [PC] "Contribuciones      */
/* Clave" item 4: Q, K, V stay in FP32, so the cast is the only reduced-    */
/* precision step.                                                          */
/*                                                                          */
/* Steps per query row (online recurrence of [MM] "La recurrencia de        */
/* softmax en linea": running max, running sum, accumulator rescaled by     */
/* e^(m_old - m_new)):                                                      */
/*   for each KV tile t of width kv_tile meeting the visible keys, in order:*/
/*     s_j  = fp32(scale * q.k_j)                   (fp32 logit)            */
/*     m'   = max(m, max_j s_j)                     (fp32)                  */
/*     a    = exp(m - m')                                                   */
/*     p_j  = fp32(exp(s_j - m'))                   (fp32, kernel precision)*/
/*     l    = a*l + sum_j p_j                       (sum of the uncast p)   */
/*     pt_j = E4M3(fp32(S * p_j))                   (the cast decision, fp32)*/
/*     acc  = a*acc + sum_j pt_j * v_j;  m = m'                             */
/*   O = acc / (S * l),  LSE = m + ln l                                     */
/* Counters: casts, and zeros (pt == 0 while p > 0), over two key sets:    */
/*   [0],[1] keys j >= n_sink (every non-sink key);                         */
/*   [2],[3] keys outside the KV tiles that hold a sink key (j >= the first */
/*           tile boundary at or after n_sink).  Non-sink keys that share a */
/*           tile with a sink are cast after the running max has absorbed   */
/*           the sink logits in either order; [PC] "Optimizacion 1" claims  */
/*           zero underflow for the values cast BEFORE the sink block.      */
/* ------------------------------------------------------------------------ */

static void pcast_row(job_t *J, i64 b, i64 h, i64 i, double *o_row, double *lse_out,
                      u64 *cnt)
{
    const i64 d = J->d, g = J->H / J->Hkv, hk = h / g, Bc = J->kv_tile;
    const float *qi = J->q + ((b * J->H + h) * J->Nq + i) * d;
    const float *kb = J->k + (b * J->Hkv + hk) * J->Nk * d;
    const float *vb = J->v + (b * J->Hkv + hk) * J->Nk * d;
    const i64 lim = visible_count(J, i);
    for (i64 c = 0; c < d; ++c) o_row[c] = 0.0;
    if (lim == 0) { *lse_out = -INFINITY; return; }
    const i64 ntiles = (lim + Bc - 1) / Bc;
    const i64 sink_end = ((J->n_sink + Bc - 1) / Bc) * Bc;
    float s[1024];
    float m = -INFINITY;
    double l = 0.0;
    for (i64 tt = 0; tt < ntiles; ++tt) {
        const i64 t = J->reverse ? (ntiles - 1 - tt) : tt;
        const i64 j0 = t * Bc;
        const i64 j1 = (j0 + Bc < lim) ? j0 + Bc : lim;
        float mn = m;
        for (i64 j = j0; j < j1; ++j) {
            s[j - j0] = (float)((double)J->scale_f * dot(qi, kb + j * d, d));
            if (s[j - j0] > mn) mn = s[j - j0];
        }
        /* The tile-local ablation (FA1's form in [MM] "El algoritmo de atencion
         * flash"): P relative to this tile's own maximum mt, so its largest
         * value casts from exactly S; its weight is restored by
         * beta = exp(mt - mn).  Default: P relative to the running max, beta = 1. */
        float mt = -INFINITY;
        for (i64 j = j0; j < j1; ++j)
            if (s[j - j0] > mt) mt = s[j - j0];
        const float pref = J->tile_local ? mt : mn;
        const double beta = J->tile_local ? exp((double)mt - (double)mn) : 1.0;
        const double a = (m == -INFINITY) ? 0.0 : exp((double)m - (double)mn);
        l *= a;
        for (i64 c = 0; c < d; ++c) o_row[c] *= a;
        for (i64 j = j0; j < j1; ++j) {
            const float p = (float)exp((double)s[j - j0] - (double)pref);
            l += (double)p * beta;
            const float x = p * J->p_scale;
            const float pt = orc_e4m3_decode(orc_e4m3_encode(x));
            const int flushed = (pt == 0.0f && p > 0.0f);
            if (j >= J->n_sink) { cnt[0] += 1; cnt[1] += flushed; }
            if (j >= sink_end) { cnt[2] += 1; cnt[3] += flushed; }
            const float *vj = vb + j * d;
            for (i64 c = 0; c < d; ++c) o_row[c] += beta * (double)pt * (double)vj[c];
        }
        m = mn;
    }
    const double den = (double)J->p_scale * l;
    for (i64 c = 0; c < d; ++c) o_row[c] /= den;
    *lse_out = (double)m + log(l);
}

/* ------------------------------------------------------------------------ */
/* Threading: items are (b, h, row) in row-major order, handed out in small */
/* chunks from an atomic counter.  Each item writes only its own outputs.   */
/* ------------------------------------------------------------------------ */

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    const i64 per_bh = J->rows ? J->nrows : J->Nq;
    double *s = J->pcast ? NULL : (double *)malloc(sizeof(double) * (size_t)(J->Nk > 0 ? J->Nk : 1));
    u64 cnt[4] = {0, 0, 0, 0};
    for (;;) {
        const i64 start = __atomic_fetch_add(&J->next, 8, __ATOMIC_RELAXED);
        if (start >= J->n_items) break;
        const i64 end = start + 8 < J->n_items ? start + 8 : J->n_items;
        for (i64 it = start; it < end; ++it) {
            const i64 bh = it / per_bh, r = it % per_bh;
            const i64 b = bh / J->H, h = bh % J->H;
            const i64 i = J->rows ? J->rows[bh * J->nrows + r] : r;
            double *o_row = J->o + it * J->d;
            if (J->pcast) pcast_row(J, b, h, i, o_row, J->lse + it, cnt);
            else exact_row(J, b, h, i, s, o_row, J->lse + it);
        }
    }
    for (int c = 0; c < 4; ++c) __atomic_fetch_add(&J->cnt[c], cnt[c], __ATOMIC_RELAXED);
    free(s);
    return NULL;
}

static int run(job_t *J, int nthreads)
{
    if (J->B < 0 || J->H < 1 || J->Hkv < 1 || J->H % J->Hkv || J->Nq < 0 || J->Nk < 0 || J->d < 1)
        return -1;
    if (J->rows) {
        for (i64 x = 0; x < J->B * J->H * J->nrows; ++x)
            if (J->rows[x] < 0 || J->rows[x] >= J->Nq) return -2;
    }
    if (J->pcast && (J->kv_tile < 1 || J->kv_tile > 1024)) return -3;
    J->n_items = J->B * J->H * (J->rows ? J->nrows : J->Nq);
    J->next = 0;
    J->cnt[0] = J->cnt[1] = J->cnt[2] = J->cnt[3] = 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int started = 0;
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&th[started], NULL, worker, J) == 0) ++started;
    worker(J);
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    return 0;
}

/* o: [B,H,R,d], lse: [B,H,R] where R = nrows (rows != NULL) or Nq. */
int orc_attention(const float *q, const float *k, const float *v, i64 B, i64 H, i64 Hkv,
                  i64 Nq, i64 Nk, i64 d, int causal, double scale, const i64 *rows,
                  i64 nrows, double *o, double *lse, int nthreads)
{
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.B = B; J.H = H; J.Hkv = Hkv; J.Nq = Nq; J.Nk = Nk; J.d = d;
    J.causal = causal; J.scale = scale; J.rows = rows; J.nrows = nrows; J.o = o; J.lse = lse;
    return run(&J, nthreads);
}

/* The full probability row p[0..Nk) of query (b,h,i); invisible keys get 0. */
int orc_attention_probs(const float *q, const float *k, i64 B, i64 H, i64 Hkv, i64 Nq,
                        i64 Nk, i64 d, int causal, double scale, i64 b, i64 h, i64 i,
                        double *p)
{
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = k; J.B = B; J.H = H; J.Hkv = Hkv; J.Nq = Nq; J.Nk = Nk; J.d = d;
    J.causal = causal; J.scale = scale;
    if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= Nq || H % Hkv) return -1;
    const i64 g = H / Hkv, hk = h / g;
    const float *qi = q + ((b * H + h) * Nq + i) * d;
    const float *kb = k + (b * Hkv + hk) * Nk * d;
    const i64 lim = visible_count(&J, i);
    for (i64 j = 0; j < Nk; ++j) p[j] = 0.0;
    if (lim == 0) return 0;
    double m = -INFINITY, l = 0.0;
    for (i64 j = 0; j < lim; ++j) {
        p[j] = scale * dot(qi, kb + j * d, d);
        if (p[j] > m) m = p[j];
    }
    for (i64 j = 0; j < lim; ++j) { p[j] = exp(p[j] - m); l += p[j]; }
    for (i64 j = 0; j < lim; ++j) p[j] /= l;
    return 0;
}

int orc_pcast(const float *q, const float *k, const float *v, i64 B, i64 H, i64 Hkv, i64 Nq,
              i64 Nk, i64 d, int causal, float scale, int kv_tile, float p_scale, int reverse,
              i64 n_sink, const i64 *rows, i64 nrows, double *o, double *lse,
              u64 *counts /* [4], see pcast_row */, int nthreads)
{
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.B = B; J.H = H; J.Hkv = Hkv; J.Nq = Nq; J.Nk = Nk; J.d = d;
    J.causal = causal; J.scale = (double)scale; J.scale_f = scale; J.rows = rows;
    J.nrows = nrows; J.o = o; J.lse = lse;
    /* reverse: bit 0 = KV tiles in reverse order, bit 1 = tile-local max */
    J.pcast = 1; J.kv_tile = kv_tile; J.p_scale = p_scale; J.reverse = reverse & 1;
    J.tile_local = (reverse >> 1) & 1;
    J.n_sink = n_sink;
    const int rc = run(&J, nthreads);
    if (counts) for (int c = 0; c < 4; ++c) counts[c] = J.cnt[c];
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Closed forms of [PC] "Marco Teorico" and "Optimizacion 2".               */
/* ------------------------------------------------------------------------ */

/* Standard normal CDF. */
double orc_Phi(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

/* Fraction of non-sink P values flushed to zero under forward KV order:
 * F(Delta, S) = Phi(Delta + delta_k - 10 ln 2 - ln S).  The page writes the
 * constant as 6.93 and identifies it with 10 ln 2, the log of the E4M3
 * round-to-zero threshold 2^-10. */
double orc_F(double delta, double S, double delta_k)
{
    return orc_Phi(delta + delta_k - 10.0 * log(2.0) - log(S));
}

/* Collapse threshold Delta_c = 10 ln 2 + ln S - delta_k (where F = 1/2). */
double orc_delta_c(double S, double delta_k) { return 10.0 * log(2.0) + log(S) - delta_k; }

/* delta_k = E[max of k iid N(0,1)] = int x * k phi(x) Phi(x)^(k-1) dx,
 * composite Simpson rule on [-12, 12] (the integrand is below 1e-30 outside). */
double orc_expected_max_gauss(int k)
{
    const int n = 48000;
    const double a = -12.0, b = 12.0, hstep = (b - a) / n;
    double acc = 0.0;
    for (int i = 0; i <= n; ++i) {
        const double x = a + i * hstep;
        const double f = x * k * exp(-0.5 * x * x) / sqrt(2.0 * M_PI) * pow(orc_Phi(x), k - 1);
        const double w = (i == 0 || i == n) ? 1.0 : ((i & 1) ? 4.0 : 2.0);
        acc += w * f;
    }
    return acc * hstep / 3.0;
}

/* d_p(S): the E4M3 quantisation step just below S, divided by S.  For S in
 * (2^(k-1), 2^k] the values just below S lie in the binade [2^(k-1), 2^k)
 * whose spacing is 2^(k-1-3). */
double orc_dp(double S)
{
    const double k = ceil(log2(S));
    return ldexp(1.0, (int)k - 4) / S;
}


/* ------------------------------------------------------------------------ */
/* Backward pass by its definition.  [MM] "Pase hacia atras: volver a      */
/* calcular en lugar de almacenar": the forward keeps only O and the row    */
/* statistics; the gradient is formed from the softmax probabilities again. */
/* With L a scalar loss and dO = dL/dO given, for each query row i and each */
/* visible key j (scores s_ij = scale * q_i.k_j, p from the complete row):  */
/*   dp_ij = dO_i . v_j                       (dL/dp_ij)                    */
/*   D_i   = sum_j p_ij dp_ij                                               */
/*   dS_ij = p_ij (dp_ij - D_i)               (softmax Jacobian applied)    */
/*   dQ_i  = scale * sum_j dS_ij k_j                                        */
/*   dK_j += scale * dS_ij q_i,   dV_j += p_ij dO_i                         */
/* With GQA the key/value gradients sum over the query heads of a group.    */
/* Optional absolute sums (for error bounds of reduced-precision results):  */
/*   adq = scale sum_j |dS_ij||k_j|, adk = scale sum_i |dS_ij||q_i|,        */
/*   adv = sum_i p_ij |dO_i|   (elementwise in the head dimension).         */
/* Work is split over (b, KV head): one thread owns every output row of     */
/* that KV head and of its query heads, so nothing is shared.               */
/* ------------------------------------------------------------------------ */

typedef struct {
    const float *q, *k, *v, *dout;
    i64 B, H, Hkv, Nq, Nk, d;
    int causal;
    double scale;
    double *dq, *dk, *dv, *adq, *adk, *adv;
    i64 next;  /* atomic */
} bjob_t;

static void *bwd_worker(void *arg)
{
    bjob_t *J = (bjob_t *)arg;
    const i64 d = J->d, g = J->H / J->Hkv;
    double *p = (double *)malloc(sizeof(double) * (size_t)(J->Nk > 0 ? J->Nk : 1));
    double *dp = (double *)malloc(sizeof(double) * (size_t)(J->Nk > 0 ? J->Nk : 1));
    job_t F;  /* for visible_count */
    memset(&F, 0, sizeof F);
    F.causal = J->causal; F.Nq = J->Nq; F.Nk = J->Nk;
    for (;;) {
        const i64 it = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
        if (it >= J->B * J->Hkv) break;
        const i64 b = it / J->Hkv, hk = it % J->Hkv;
        const float *kb = J->k + (b * J->Hkv + hk) * J->Nk * d;
        const float *vb = J->v + (b * J->Hkv + hk) * J->Nk * d;
        double *dkb = J->dk + (b * J->Hkv + hk) * J->Nk * d;
        double *dvb = J->dv + (b * J->Hkv + hk) * J->Nk * d;
        double *adkb = J->adk ? J->adk + (b * J->Hkv + hk) * J->Nk * d : NULL;
        double *advb = J->adv ? J->adv + (b * J->Hkv + hk) * J->Nk * d : NULL;
        for (i64 x = 0; x < J->Nk * d; ++x) {
            dkb[x] = 0.0; dvb[x] = 0.0;
            if (adkb) adkb[x] = 0.0;
            if (advb) advb[x] = 0.0;
        }
        for (i64 h = hk * g; h < (hk + 1) * g; ++h) {
            for (i64 i = 0; i < J->Nq; ++i) {
                const i64 row = (b * J->H + h) * J->Nq + i;
                const float *qi = J->q + row * d;
                const float *doi = J->dout + row * d;
                double *dqi = J->dq + row * d;
                double *adqi = J->adq ? J->adq + row * d : NULL;
                for (i64 c = 0; c < d; ++c) {
                    dqi[c] = 0.0;
                    if (adqi) adqi[c] = 0.0;
                }
                const i64 lim = visible_count(&F, i);
                if (lim == 0) continue;
                /* probabilities of the complete row (two passes) */
                double m = -INFINITY, l = 0.0;
                for (i64 j = 0; j < lim; ++j) {
                    p[j] = J->scale * dot(qi, kb + j * d, d);
                    if (p[j] > m) m = p[j];
                }
                for (i64 j = 0; j < lim; ++j) { p[j] = exp(p[j] - m); l += p[j]; }
                for (i64 j = 0; j < lim; ++j) p[j] /= l;
                /* dp and D */
                double D = 0.0;
                for (i64 j = 0; j < lim; ++j) {
                    dp[j] = dot(doi, vb + j * d, d);
                    D += p[j] * dp[j];
                }
                for (i64 j = 0; j < lim; ++j) {
                    const double ds = p[j] * (dp[j] - D);
                    const float *kj = kb + j * d;
                    for (i64 c = 0; c < d; ++c) {
                        dqi[c] += J->scale * ds * (double)kj[c];
                        dkb[j * d + c] += J->scale * ds * (double)qi[c];
                        dvb[j * d + c] += p[j] * (double)doi[c];
                        if (adqi) adqi[c] += J->scale * fabs(ds) * fabs((double)kj[c]);
                        if (adkb) adkb[j * d + c] += J->scale * fabs(ds) * fabs((double)qi[c]);
                        if (advb) advb[j * d + c] += p[j] * fabs((double)doi[c]);
                    }
                }
            }
        }
    }
    free(p);
    free(dp);
    return NULL;
}

/* dq: [B,H,Nq,d]; dk, dv: [B,Hkv,Nk,d] (float64).  adq/adk/adv: the same
 * shapes, or NULL. */
int orc_attention_bwd(const float *q, const float *k, const float *v, const float *dout, i64 B,
                      i64 H, i64 Hkv, i64 Nq, i64 Nk, i64 d, int causal, double scale,
                      double *dq, double *dk, double *dv, double *adq, double *adk,
                      double *adv, int nthreads)
{
    if (B < 0 || H < 1 || Hkv < 1 || H % Hkv || Nq < 0 || Nk < 0 || d < 1) return -1;
    bjob_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.dout = dout; J.B = B; J.H = H; J.Hkv = Hkv; J.Nq = Nq;
    J.Nk = Nk; J.d = d; J.causal = causal; J.scale = scale; J.dq = dq; J.dk = dk; J.dv = dv;
    J.adq = adq; J.adk = adk; J.adv = adv;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int started = 0;
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&th[started], NULL, bwd_worker, &J) == 0) ++started;
    bwd_worker(&J);
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* FP8 (E4M3) quantisation with incoherent processing.                      */
/*                                                                          */
/* [MM] "FA3: Mecanica de la tolva", item 3: FP8 attention loses accuracy   */
/* to outliers; the remedy is to rotate the vectors at random before the    */
/* block-wise quantisation, so an outlier's magnitude is spread over all    */
/* coordinates.  The pages give no rotation, block shape or scale rule;     */
/* the readings taken here:                                                 */
/*  - rotation: y = H_d (s o x), H_d the Sylvester-Hadamard matrix          */
/*    (H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]) and s a vector of       */
/*    random signs (+-1).  H_d^T H_d = d I, so applying the same rotation   */
/*    to q and k multiplies every dot product by exactly d (the attention   */
/*    scale is divided by d).  H_d x is formed by the fast transform in     */
/*    fp32, in stages h = 1, 2, 4, ..., d/2, each replacing the pair        */
/*    (y_j, y_{j+h}) (j mod 2h < h) by (y_j + y_{j+h}, y_j - y_{j+h});      */
/*    the codes depend on this fp32 rounding, so its order is part of the   */
/*    definition.                                                           */
/*  - groups: layout 0 = 32 consecutive rows of one (b, h) (all d columns), */
/*    scales [B, H, ceil(N/32)]; layout 1 = one column c of one (b, h) over */
/*    all N rows, scales [B, H, d]; whole != 0 = one group for the entire   */
/*    tensor, its scale written into every slot of the chosen layout.      */
/*  - scale: the power of two 2^e with e the smallest integer >= -126 such  */
/*    that amax <= 448 * 2^e (448 = the largest finite E4M3 value, [PC]    */
/*    "Optimizacion 2"); a zero group gets e = -126.                        */
/*  - code = E4M3_RNE(y * 2^-e) (the codec above); dequantised value        */
/*    decode(code) * 2^e.  Inputs are finite.                               */
/* ------------------------------------------------------------------------ */

static void fwht_f32(float *y, i64 d)
{
    for (i64 h = 1; h < d; h *= 2)
        for (i64 j = 0; j < d; ++j)
            if ((j % (2 * h)) < h) {
                const float a = y[j], b = y[j + h];
                y[j] = a + b;
                y[j + h] = a - b;
            }
}

static int scale_exponent(float amax)
{
    if (!(amax > 0.0f)) return -126;
    int E2;
    const double f = frexp((double)amax, &E2);   /* amax = f * 2^E2, f in [0.5, 1) */
    /* amax <= 448 * 2^e  <=>  f * 2^E2 <= 0.875 * 2^(9 + e) */
    int e = (f <= 0.875) ? E2 - 9 : E2 - 8;
    return e < -126 ? -126 : e;
}

int orc_quant_e4m3(const float *x, i64 B, i64 H, i64 N, i64 d, const float *signs, int layout,
                   int whole, unsigned char *codes, float *scales)
{
    if (B < 0 || H < 1 || N < 0 || d < 1 || (layout != 0 && layout != 1)) return 1;
    if (signs && (d & (d - 1))) return 2;               /* the transform needs d = 2^n */
    const i64 rows = B * H * N, nblk = (N + 31) / 32;
    float *y = (float *)malloc((size_t)(rows > 0 ? rows : 1) * (size_t)d * sizeof(float));
    if (!y) return 3;
    for (i64 r = 0; r < rows; ++r) {
        for (i64 c = 0; c < d; ++c) y[r * d + c] = signs ? signs[c] * x[r * d + c] : x[r * d + c];
        if (signs) fwht_f32(y + r * d, d);
    }
    const i64 nsc = B * H * (layout == 0 ? nblk : d);
    float *amax = (float *)calloc((size_t)(nsc > 0 ? nsc : 1), sizeof(float));
    if (!amax) { free(y); return 3; }
    for (i64 bh = 0; bh < B * H; ++bh)
        for (i64 i = 0; i < N; ++i)
            for (i64 c = 0; c < d; ++c) {
                const float a = fabsf(y[(bh * N + i) * d + c]);
                const i64 g = layout == 0 ? bh * nblk + i / 32 : bh * d + c;
                if (a > amax[g]) amax[g] = a;
            }
    if (whole) {
        float t = 0.0f;
        for (i64 g = 0; g < nsc; ++g) if (amax[g] > t) t = amax[g];
        for (i64 g = 0; g < nsc; ++g) amax[g] = t;
    }
    for (i64 g = 0; g < nsc; ++g) scales[g] = (float)ldexp(1.0, scale_exponent(amax[g]));
    for (i64 bh = 0; bh < B * H; ++bh)
        for (i64 i = 0; i < N; ++i)
            for (i64 c = 0; c < d; ++c) {
                const i64 g = layout == 0 ? bh * nblk + i / 32 : bh * d + c;
                const float inv = (float)ldexp(1.0, -scale_exponent(amax[g]));
                codes[(bh * N + i) * d + c] = (unsigned char)orc_e4m3_encode(y[(bh * N + i) * d + c] * inv);
            }
    free(amax);
    free(y);
    return 0;
}
