/*
 * rtp_oracle.c -- plain, slow CPU oracle for RTPurbo's head-split sparse
 * attention (test infrastructure only).
 *
 * Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library.  The GPU library shares no code with it:
 * no headers, no helpers, no tables.  Every function below is the plainest
 * reading of the method as the pages describe it, written for a reader to
 * check by eye, not for speed (apart from being compiled C).
 *
 * What the pages fix (all of them restate the same abstract):
 *  - "Full Attention Strikes Back: Transferring Full Attention into Sparse
 *    within Hundred Training Steps" (arXiv 2605.16928), abstract,
 *    observations (1)-(3): a few retrieval heads keep the whole KV cache and
 *    find their tokens with a 16-dimensional indexer; the useful token
 *    budget is chosen per query by top-p rather than a fixed top-k; the
 *    remaining heads only look at a restricted local window.
 *  - zhichai.net forum post "RTPurbo: Turning Dense LLMs into Sparse
 *    Attention Models with Just a Few Hundred Training Steps", section
 *    "Three Key Insights" items 1-3 (local heads keep only a local window;
 *    the 16-dim projection is built on the low-frequency RoPE dimensions;
 *    cumulative top-p replaces fixed top-k).
 *
 * Readings taken where the pages are silent (each is listed with its reason
 * in the design notes of the repository):
 *  - the projection is an fp32 fused-multiply-add chain over d = 0..D-1
 *    starting from +0, rounded once to bf16 (round to nearest even);
 *  - the indexer score is the fp32 chain over c = 0..15 from +0 of the
 *    exact bf16 x bf16 products;
 *  - indexer softmax: w_j = exp(s (d_j - m)), m = max_j d_j, s = idx_scale;
 *  - top-p: rank keys by (score descending, index ascending), keep the
 *    shortest prefix whose cumulative mass / Z reaches p (>=); p >= 1 keeps
 *    every key;
 *  - attention over a selected set renormalises softmax over that set only;
 *  - the local-head window is the last W positions including the query's
 *    own, united with the first N_s positions (sink tokens), clipped to
 *    [0, pos].
 *
 * Build:  gcc -O2 -std=c11 -ffp-contract=off -mfma -fPIC -shared -lm
 * (-ffp-contract=off: no implicit contraction; every fused operation is an
 * explicit fmaf call, so the rounding sequence is the one written here.)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* bf16 <-> fp32 (input/output conversion; bf16 is the top half of fp32) */
/* ------------------------------------------------------------------ */

float orc_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round a finite fp32 value to bf16, nearest-even. */
uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lower = u & 0xFFFFu;
    uint32_t upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u;
    return (uint16_t)upper;
}

/*
 * FP8 E4M3 (OCP "e4m3fn": 1 sign bit, 4 exponent bits with bias 7, 3
 * mantissa bits, no infinities, S.1111.111 is NaN) to fp32, exact.  K and V
 * stored in this format carry one fp32 scale each; a stored code c stands for
 * fl32(f32(c) * scale), the product rounded once to nearest even.
 */
float orc_fp8e4m3_to_f32(uint8_t c)
{
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 15;
    int m = c & 7;
    float v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexpf((float)m, -9);                 /* subnormal: m/8 * 2^-6 */
    else
        v = ldexpf((float)(8 + m), e - 10);        /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

void orc_fp8_dequant(const uint8_t *c, int64_t n, float scale, float *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_fp8e4m3_to_f32(c[i]) * scale;
}

/* ------------------------------------------------------------------ */
/* Step 1/2: low-rank indexer projection of keys (on append) and queries */
/* ------------------------------------------------------------------ */

/*
 * out[i][c] = bf16( sum_{d=0}^{D-1} x[i][d] * W[d][c] ), where the sum is
 * the fp32 chain acc = fmaf(x[i][d], W[d][c], acc), d ascending, acc = +0.
 * x has row stride ld (in elements); W is [D][16] row-major.
 * Follows the abstract's "16-dimensional indexer" and the forum post's
 * "low-dimensional projection" (Three Key Insights, item 2).
 */
void orc_project(const float *x, int64_t rows, int64_t ld, int32_t D,
                 const float *W, uint16_t *out)
{
    for (int64_t i = 0; i < rows; i++) {
        const float *xi = x + i * ld;
        for (int c = 0; c < 16; c++) {
            float acc = 0.0f;
            for (int d = 0; d < D; d++)
                acc = fmaf(xi[d], W[(int64_t)d * 16 + c], acc);
            out[i * 16 + c] = orc_f32_to_bf16(acc);
        }
    }
}

/* ------------------------------------------------------------------ */
/* Step 3: indexer scores                                              */
/* ------------------------------------------------------------------ */

/*
 * d[j] = fp32 chain over c = 0..15 of q_low[c] * k_low[j][c], from +0.
 * Inputs are bf16, so each product is exact in fp32 and fmaf equals
 * "add the exact product"; only the order c ascending matters.
 * Returns 0, or -1 if some product is not exact in fp32 (it then leaves the
 * scores written but the caller must not trust them as the documented
 * definition).
 */
int orc_scores(const uint16_t *q_low, const uint16_t *k_low, int64_t L,
               float *d)
{
    int exact = 1;
    float q[16];
    for (int c = 0; c < 16; c++)
        q[c] = orc_bf16_to_f32(q_low[c]);
    for (int64_t j = 0; j < L; j++) {
        float acc = 0.0f;
        for (int c = 0; c < 16; c++) {
            float k = orc_bf16_to_f32(k_low[j * 16 + c]);
            double pd = (double)q[c] * (double)k;   /* exact in double */
            if ((double)(float)pd != pd)
                exact = 0;
            acc = fmaf(q[c], k, acc);
        }
        d[j] = acc;
    }
    return exact ? 0 : -1;
}

/* ------------------------------------------------------------------ */
/* Steps 4/5: indexer softmax mass and dynamic top-p                   */
/* ------------------------------------------------------------------ */

typedef struct { float d; int64_t j; } ranked;

/* rank order: score descending, then index ascending (-0 equals +0) */
static int rank_cmp(const void *a, const void *b)
{
    const ranked *x = (const ranked *)a, *y = (const ranked *)b;
    if (x->d > y->d) return -1;
    if (x->d < y->d) return 1;
    return (x->j < y->j) ? -1 : (x->j > y->j ? 1 : 0);
}

/*
 * Top-p selection over the scores d[0..L-1] (cumulative top-p of the forum
 * post, Three Key Insights item 3; "dynamic top-p" of the abstract).
 *   m = max_j d_j;  w_j = exp(s * (d_j - m)) in double;  Z = sum_j w_j
 *   (j ascending);  sigma = ranks by (d desc, j asc);
 *   C_k = (w_sigma(1) + ... + w_sigma(k)) / Z;
 *   k* = L if p >= 1, else min{k >= 1 : C_k >= p} (L if rounding leaves
 *   none).
 * Writes the selected indices ascending into sel[0..k*-1] and returns k*.
 * If order != NULL it receives sigma (0-based, length L); if cum != NULL it
 * receives C_1..C_L (cum[k-1] = C_k).  Returns -1 for L < 1, p <= 0 or NaN.
 * Re-entrant: independent rows may run on separate threads.
 */
int64_t orc_topp(const float *d, int64_t L, double s, float p,
                 int32_t *sel, int64_t *order, double *cum)
{
    if (L < 1 || !(p > 0.0f))
        return -1;
    float m = d[0];
    for (int64_t j = 1; j < L; j++)
        if (d[j] > m) m = d[j];
    double *w = (double *)malloc(sizeof(double) * (size_t)L);
    ranked *sig = (ranked *)malloc(sizeof(ranked) * (size_t)L);
    double Z = 0.0;
    for (int64_t j = 0; j < L; j++) {
        w[j] = exp(s * ((double)d[j] - (double)m));
        Z += w[j];
        sig[j].d = d[j];
        sig[j].j = j;
    }
    qsort(sig, (size_t)L, sizeof(ranked), rank_cmp);

    int64_t kstar = L;
    double run = 0.0;
    int found = 0;
    for (int64_t k = 1; k <= L; k++) {
        run += w[sig[k - 1].j];
        double Ck = run / Z;
        if (cum) cum[k - 1] = Ck;
        if (!found && (double)p < 1.0 && Ck >= (double)p) {
            kstar = k;
            found = 1;
        }
    }
    /* emit sigma(1..k*) in ascending index order */
    char *take = (char *)calloc((size_t)L, 1);
    for (int64_t k = 0; k < kstar; k++)
        take[sig[k].j] = 1;
    int64_t n = 0;
    for (int64_t j = 0; j < L; j++)
        if (take[j]) sel[n++] = (int32_t)j;
    if (order)
        for (int64_t k = 0; k < L; k++)
            order[k] = sig[k].j;
    free(take);
    free(sig);
    free(w);
    return kstar;
}

/*
 * Fixed top-k selection over the scores d[0..L-1]: the fixed-budget rule
 * that the method's dynamic top-p replaces (abstract, observation (3); forum
 * post, "Three Key Insights" item 3), also used to cap a top-p set at a
 * budget of k keys.  The selected set is the first min(k, L) keys of the rank
 * order (d descending, then j ascending; -0 equals +0), written ascending
 * into sel.  Returns its size, or -1 for L < 1 or k < 1.
 */
int64_t orc_topk(const float *d, int64_t L, int64_t k, int32_t *sel)
{
    if (L < 1 || k < 1)
        return -1;
    ranked *sig = (ranked *)malloc(sizeof(ranked) * (size_t)L);
    for (int64_t j = 0; j < L; j++) {
        sig[j].d = d[j];
        sig[j].j = j;
    }
    qsort(sig, (size_t)L, sizeof(ranked), rank_cmp);
    int64_t n = k < L ? k : L;
    char *take = (char *)calloc((size_t)L, 1);
    for (int64_t i = 0; i < n; i++)
        take[sig[i].j] = 1;
    int64_t c = 0;
    for (int64_t j = 0; j < L; j++)
        if (take[j]) sel[c++] = (int32_t)j;
    free(take);
    free(sig);
    return n;
}

/* ------------------------------------------------------------------ */
/* Steps 6-8: exact softmax attention over an index set                */
/* ------------------------------------------------------------------ */

/*
 * out[0..D-1] = sum_{j in idx} softmax_j(scale * q . k_j) v_j, in double,
 * softmax renormalised over idx only (retrieval heads: the selected set;
 * local heads: the window set; dense: 0..pos).  K and V rows have stride ld.
 * Sums run in the order idx is given (the callers pass ascending sets).
 */
void orc_attend(const float *q, const float *K, const float *V, int64_t ld,
                int32_t D, const int32_t *idx, int64_t n, double scale,
                double *out)
{
    double *lg = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double mx = -INFINITY;
    for (int64_t t = 0; t < n; t++) {
        const float *k = K + (int64_t)idx[t] * ld;
        double dot = 0.0;
        for (int e = 0; e < D; e++)
            dot += (double)q[e] * (double)k[e];
        lg[t] = scale * dot;
        if (lg[t] > mx) mx = lg[t];
    }
    double den = 0.0;
    for (int e = 0; e < D; e++) out[e] = 0.0;
    for (int64_t t = 0; t < n; t++) {
        double pw = exp(lg[t] - mx);
        den += pw;
        const float *v = V + (int64_t)idx[t] * ld;
        for (int e = 0; e < D; e++)
            out[e] += pw * (double)v[e];
    }
    for (int e = 0; e < D; e++)
        out[e] = (n > 0) ? out[e] / den : 0.0;
    free(lg);
}

/*
 * Window set of a local head for a query at position pos: the first Ns
 * positions (sinks) united with the last W positions up to and including
 * pos, clipped to [0, pos], ascending, no duplicates.  Returns its size.
 */
int64_t orc_window_set(int64_t pos, int64_t W, int64_t Ns, int32_t *out)
{
    int64_t n = 0;
    int64_t lo = pos - W + 1;
    for (int64_t j = 0; j <= pos; j++)
        if (j < Ns || j >= lo)
            out[n++] = (int32_t)j;
    return n;
}
