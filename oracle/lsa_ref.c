/*
 * lsa_ref.c -- CPU oracle for the LongCat Sparse Attention (LSA) token-selection path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the GPU library is
 * checked against.  Only the test suite, the smoke check and the CPU-baseline leg of the bench
 * may load it; the product path (the HIP library and its Python binding) never does, and the two
 * share no code: no kernels, headers, helpers, tables or constants.
 *
 * Arithmetic is fp64 unless a step's own definition fixes another precision (the page-key mean,
 * which is defined in fp32 with a fixed summation order, and the selection decisions, which are
 * taken on fp32 scores because that is the precision the GPU path decides in).
 *
 * Sources (the pages this method is described on):
 *   [LSA]  "LongCat Sparse Attention: Taming the Lightning via Streaming-aware Hierarchical
 *          Cross-Layer Indexing" (paper summary page, aipaper.jasonlin.tech): abstract, key
 *          contributions (Cross-Layer Indexing 1/N; Hierarchical Indexing O(L) -> O(L/P + MP)),
 *          limitations (Streaming-Aware Indexing gives 50% of the budget to fixed regions).
 *   [CARD] "LongCat-Flash-Lite-Sparse" model card (ai-top.pl): the SI / CLI / HI bullet list.
 *   [DSA]  Baidu Cloud article on DeepSeek's Lightning Indexer (intl.cloud.baidu.com),
 *          "Core Architecture Analysis": 1. Lightweight Scoring Module, 2. Dynamic Token
 *          Selector, 3. Sparse Attention Calculator.
 *
 * Every function handles ONE sequence; callers loop over the batch.
 *
 * Parity pins: every function here is pinned by tests (library routines on special cases,
 * closed forms, invariants, brute force on tiny inputs); no function is "parity unpinned".
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define REF_KEY_BF16 1
#define REF_KEY_E4M3 2

/* Threads the parallel loops below use (for reporting CPU timings). */
int lsa_ref_num_threads(void) { return omp_get_max_threads(); }

/* Set the thread count of the parallel loops (timing runs on one core, or on all of them). */
void lsa_ref_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

/* ------------------------------------------------------------------------------------------ */
/* Number formats.                                                                             */
/* ------------------------------------------------------------------------------------------ */

/* bfloat16: the upper 16 bits of an IEEE-754 binary32. */
double lsa_ref_bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP 8-bit floating point, E4M3 "fn" variant (the format gfx950 and torch.float8_e4m3fn use):
 * 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; no infinities; exponent 15 with
 * mantissa 7 is NaN; exponent 0 encodes subnormals m * 2^-9. */
double lsa_ref_e4m3fn_to_double(uint8_t code)
{
    int s = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* binary32 -> bfloat16, round to nearest, ties to even (NaN kept quiet). */
uint16_t lsa_ref_f32_to_bf16_rne(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu))
        return (uint16_t)((u >> 16) | 0x40u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

/* The dequantised key element k[s][i], exactly (bf16 and e4m3 values and their products with a
 * binary32 scale are all representable in binary64). */
static double key_elem(const void *keys, int key_dtype, const float *scale, int d, int64_t s, int i)
{
    if (key_dtype == REF_KEY_BF16)
        return lsa_ref_bf16_to_double(((const uint16_t *)keys)[s * d + i]);
    return (double)scale[s] * lsa_ref_e4m3fn_to_double(((const uint8_t *)keys)[s * d + i]);
}

/* ------------------------------------------------------------------------------------------ */
/* a1. Lightning-Indexer scores.                                                               */
/* ------------------------------------------------------------------------------------------ */

/*
 * [DSA] 1. Lightweight Scoring Module: relevance of a past key to a query is ReLU of their dot
 * product.  The indexer of DeepSeek Sparse Attention ([LSA] abstract: "Lightning Indexer") uses
 * H indexer heads with per-query head weights:
 *
 *     I[t,s] = sum_h w[t,h] * ReLU( q[t,h] . k[s] ),   for s < V_t,   V_t = min(L, pos_t + 1)
 *
 * No 1/sqrt(d) factor: any positive factor folds into w and, ReLU being positively homogeneous,
 * changes no selection.  For e4m3 keys k[s] = scale[s] * kq[s].  Keys at s >= V_t (the future)
 * get -inf.
 *
 * Outputs (row-major [n_rows][L], any may be NULL):
 *   I  the score;
 *   A  sum_h |w[t,h]| * ReLU(q[t,h] . k[s])          (magnitude of the terms that were summed)
 *   E  sum_h |w[t,h]| * sum_i |q[t,h,i] * k[s,i]|     (magnitude before cancellation)
 * A and E are the error scales the tolerance on I is stated against.
 */
/* The formula above for one query row t whose H x d query values are qd (as doubles). */
static void index_scores_row(int64_t t, int H, int d, int64_t L, int64_t pos, const double *qd,
                             const float *w, const void *keys, int key_dtype, const float *scale,
                             double *I, double *A, double *E);

void lsa_ref_index_scores(int64_t n_rows, int H, int d, int64_t L, const int64_t *pos,
                          const uint16_t *q, const float *w, const void *keys, int key_dtype,
                          const float *scale, double *I, double *A, double *E)
{
    double *qd = (double *)malloc(sizeof(double) * (size_t)H * (size_t)d);
    for (int64_t t = 0; t < n_rows; ++t) {
        for (int64_t j = 0; j < (int64_t)H * d; ++j)
            qd[j] = lsa_ref_bf16_to_double(q[t * H * d + j]);
        index_scores_row(t, H, d, L, pos[t], qd, w, keys, key_dtype, scale, I, A, E);
    }
    free(qd);
}

static void index_scores_row(int64_t t, int H, int d, int64_t L, int64_t pos, const double *qd,
                             const float *w, const void *keys, int key_dtype, const float *scale,
                             double *I, double *A, double *E)
{
    {
        int64_t V = pos + 1 < L ? pos + 1 : L;
#pragma omp parallel for schedule(static)
        for (int64_t s = 0; s < L; ++s) {
            double score = 0.0, amag = 0.0, emag = 0.0;
            if (s >= V) {
                if (I) I[t * L + s] = -INFINITY;
                if (A) A[t * L + s] = 0.0;
                if (E) E[t * L + s] = 0.0;
                continue;
            }
            for (int h = 0; h < H; ++h) {
                double dot = 0.0, dabs = 0.0;
                for (int i = 0; i < d; ++i) {
                    double p = qd[h * d + i] * key_elem(keys, key_dtype, scale, d, s, i);
                    dot += p;
                    dabs += fabs(p);
                }
                double wh = (double)w[t * H + h];
                double relu = dot > 0.0 ? dot : 0.0;
                score += wh * relu;
                amag += fabs(wh) * relu;
                emag += fabs(wh) * dabs;
            }
            if (I) I[t * L + s] = score;
            if (A) A[t * L + s] = amag;
            if (E) E[t * L + s] = emag;
        }
    }
}

/* ------------------------------------------------------------------------------------------ */
/* fp8 queries: per-(query, head) e4m3 quantisation, then the scores of the quantised queries. */
/* ------------------------------------------------------------------------------------------ */

/*
 * [DSA] 1. Lightweight Scoring Module, "Quantized computation": the indexer may run its
 * products in 8-bit floating point.  Here a query row q[t,h,:] (bf16) is quantised the way the
 * fp8 key rows are:
 *     s      = max_i |q[t,h,i]| / 448           (binary32 division; 1 for an all-zero row)
 *     code_i = e4m3fn( q[t,h,i] / s )           (binary32 division, then round to nearest with
 *                                                ties to even, saturating at +-448)
 * and the scores are the formula of lsa_ref_index_scores with q[t,h,i] replaced by
 * s * e4m3(code_i) (exact in binary64).
 */

/* binary32 -> e4m3fn code: the nearest of the 127 non-negative finite values (magnitudes at or
 * beyond the largest, 448, give 448), ties to the even code; the sign is copied (+-0 keep their
 * sign).  NaN gives the NaN code 0x7F. */
uint8_t lsa_ref_f32_to_e4m3fn_sat(float x)
{
    if (x != x) return 0x7F;
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs((double)x);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    int best = 0;
    double best_err = a;
    for (int c = 1; c <= 0x7E; ++c) {
        double err = fabs(a - lsa_ref_e4m3fn_to_double((uint8_t)c));
        if (err < best_err || (err == best_err && (c & 1) == 0)) {
            best = c;
            best_err = err;
        }
    }
    return (uint8_t)(sign | best);
}

void lsa_ref_quantize_rows(int64_t n_rows, int d, const uint16_t *x, uint8_t *codes,
                           float *scale)
{
    for (int64_t r = 0; r < n_rows; ++r) {
        float amax = 0.0f;
        for (int i = 0; i < d; ++i) {
            float v = fabsf((float)lsa_ref_bf16_to_double(x[r * d + i]));
            if (v > amax) amax = v;
        }
        volatile float s = amax > 0.0f ? amax / 448.0f : 1.0f; /* one binary32 division */
        scale[r] = s;
        for (int i = 0; i < d; ++i) {
            volatile float y = (float)lsa_ref_bf16_to_double(x[r * d + i]) / s;
            codes[r * d + i] = lsa_ref_f32_to_e4m3fn_sat(y);
        }
    }
}

void lsa_ref_index_scores_q8(int64_t n_rows, int H, int d, int64_t L, const int64_t *pos,
                             const uint8_t *q8, const float *q_scale, const float *w,
                             const void *keys, int key_dtype, const float *scale, double *I,
                             double *A, double *E)
{
    double *qd = (double *)malloc(sizeof(double) * (size_t)H * (size_t)d);
    for (int64_t t = 0; t < n_rows; ++t) {
        for (int h = 0; h < H; ++h)
            for (int i = 0; i < d; ++i)
                qd[h * d + i] = (double)q_scale[t * H + h] *
                                lsa_ref_e4m3fn_to_double(q8[(t * H + h) * d + i]);
        index_scores_row(t, H, d, L, pos[t], qd, w, keys, key_dtype, scale, I, A, E);
    }
    free(qd);
}

/* ------------------------------------------------------------------------------------------ */
/* a2. Streaming-Aware selection: sink + local window + dynamic top-k.                         */
/* ------------------------------------------------------------------------------------------ */

typedef struct {
    float score;
    int32_t id;
} cand_t;

/* Order of the dynamic top-k: higher score first, lower token index on equal scores.  Compared
 * as binary32 values, so -0 and +0 are equal. */
static int by_score_desc_id_asc(const void *pa, const void *pb)
{
    const cand_t *a = (const cand_t *)pa, *b = (const cand_t *)pb;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    return (a->id > b->id) - (a->id < b->id);
}

static int by_id_asc(const void *pa, const void *pb)
{
    const cand_t *a = (const cand_t *)pa, *b = (const cand_t *)pb;
    return (a->id > b->id) - (a->id < b->id);
}

/*
 * [DSA] 2. Dynamic Token Selector keeps the k best-scoring past tokens of each query.
 * [CARD] Streaming-Aware Indexing and [LSA] abstract strategy (1): part of the budget goes to a
 * fixed attention sink and a local sliding window, the rest to dynamic top-k.
 *
 * Per row with valid length V (tokens [0, V) exist for this query):
 *   V <= k : every token [0, V), ascending, then -1.
 *   else   : sink [0, S) ascending, then window [V-W, V) ascending, then the top k-S-W of the
 *            middle [S, V-W) by (score desc, index asc), listed ascending.  (V > k >= S+W makes
 *            the middle non-empty and larger than k-S-W, so no padding.)
 *
 * Flat mode (cand_ids == NULL): scores[t][s] is the score of token s, n_cand == L.
 * Candidate mode: scores[t][j] belongs to token cand_ids[t][j]; ids of -1 are empty slots and
 * only ids inside the middle [S, V-W) compete; if fewer than k-S-W compete, all are taken and
 * the tail is -1.
 */
void lsa_ref_select(int64_t n_rows, int64_t n_cand, const float *scores, const int32_t *cand_ids,
                    const int64_t *Vrow, int k, int S, int W, int32_t *idx)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < n_rows; ++t) {
        int64_t V = Vrow[t];
        int32_t *out = idx + t * k;
        int o = 0;
        if (V <= k) {
            for (int64_t s = 0; s < V; ++s) out[o++] = (int32_t)s;
            while (o < k) out[o++] = -1;
            continue;
        }
        for (int s = 0; s < S; ++s) out[o++] = s;
        for (int64_t s = V - W; s < V; ++s) out[o++] = (int32_t)s;
        int need = k - S - W;
        cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)(n_cand > 0 ? n_cand : 1));
        int64_t nc = 0;
        for (int64_t j = 0; j < n_cand; ++j) {
            int64_t id = cand_ids ? cand_ids[t * n_cand + j] : j;
            if (id < S || id >= V - W) continue; /* also drops -1 */
            c[nc].score = scores[t * n_cand + j];
            c[nc].id = (int32_t)id;
            ++nc;
        }
        qsort(c, (size_t)nc, sizeof(cand_t), by_score_desc_id_asc);
        int take = nc < need ? (int)nc : need;
        qsort(c, (size_t)take, sizeof(cand_t), by_id_asc);
        for (int j = 0; j < take; ++j) out[o++] = c[j].id;
        while (o < k) out[o++] = -1;
        free(c);
    }
}

/* ------------------------------------------------------------------------------------------ */
/* a3. Page keys for Hierarchical Indexing.                                                    */
/* ------------------------------------------------------------------------------------------ */

/* Pairwise sum of n (a power of two) binary32 values: the two halves are summed separately and
 * then added, recursively.  This fixes the rounding of the sum completely. */
static float tree_sum_f32(const float *v, int n)
{
    if (n == 1) return v[0];
    float lo = tree_sum_f32(v, n / 2);
    float hi = tree_sum_f32(v + n / 2, n / 2);
    return lo + hi;
}

/*
 * [CARD] Hierarchical Indexing first recalls candidate blocks from coarse scores.  The pages do
 * not say what a block's coarse representation is; this library defines the page key as the mean
 * of the page's dequantised indexer keys, fixed to the bit:
 *
 *   v[j]   = binary32( scale[s] * kq[s][i] )  (e4m3 keys)  or  the bf16 value (bf16 keys),
 *            for slot j = s - p*P of page p, and +0.0 for slots past the end of the sequence;
 *   sum    = the pairwise tree sum of v[0..P) in binary32;
 *   pk     = bf16_rne( sum / n_p )  (binary32 division, n_p = tokens present in the page).
 *
 * P must be a power of two.  Output pk[ceil(L/P)][d] as bf16 bits.
 */
void lsa_ref_page_keys(int64_t L, int d, int P, const void *keys, int key_dtype,
                       const float *scale, uint16_t *pk)
{
    int64_t n_pages = (L + P - 1) / P;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < n_pages; ++p) {
        float *v = (float *)malloc(sizeof(float) * (size_t)P);
        int64_t n_p = L - p * P < P ? L - p * P : P;
        for (int i = 0; i < d; ++i) {
            for (int j = 0; j < P; ++j) {
                int64_t s = p * P + j;
                if (j >= n_p) { v[j] = 0.0f; continue; }
                if (key_dtype == REF_KEY_BF16) {
                    v[j] = (float)lsa_ref_bf16_to_double(((const uint16_t *)keys)[s * d + i]);
                } else {
                    float kq = (float)lsa_ref_e4m3fn_to_double(((const uint8_t *)keys)[s * d + i]);
                    v[j] = scale[s] * kq;
                }
            }
            float mean = tree_sum_f32(v, P) / (float)n_p;
            pk[p * d + i] = lsa_ref_f32_to_bf16_rne(mean);
        }
        free(v);
    }
}

/* ------------------------------------------------------------------------------------------ */
/* a4 + a5. Hierarchical Indexing: coarse page recall, then fine scoring inside the pages.     */
/* ------------------------------------------------------------------------------------------ */

/*
 * [CARD] Hierarchical Indexing works in two stages: it recalls candidate blocks by coarse scores,
 * then selects tokens finely inside those blocks.  [LSA] key contribution 3: per-query selection
 * cost falls from O(L) to O(L/P + MP) for pages of P tokens and M recalled pages.
 *
 * For each row with valid length V (only when V > k; otherwise nothing is recalled and every
 * output of the row is -1 / -inf, because the selector then takes all V tokens):
 *   1. eligible pages: those overlapping the middle [S, V-W), i.e. floor(S/P) ..
 *      floor((V-W-1)/P);
 *   2. coarse score of page p: the indexer formula on the page key,
 *      Ic[t,p] = sum_h w[t,h] ReLU(q[t,h] . pk[p])  (fp64, then rounded to binary32 -- the
 *      precision in which the GPU path ranks pages);
 *   3. recall the M best eligible pages by (coarse desc, page asc), all of them if fewer;
 *      page_ids lists them ascending, -1 padded;
 *   4. candidates: for the i-th recalled page p (ascending), slot i*P + j holds token p*P + j if
 *      it lies in the middle [S, V-W), with its fine score from the indexer formula on the
 *      token's own key (fp64); other slots hold id -1 and score -inf.
 *
 * Arrays: q [n_rows][H][d] bf16 bits, w [n_rows][H], pos [n_rows]; pk [ceil(L/P)][d] bf16 bits;
 * keys [L][d] (+ scale [L]).  Outputs page_ids [n_rows][M], cand_ids / cand_scores
 * [n_rows][M*P]; coarse [n_rows][ceil(L/P)] (may be NULL; -inf for ineligible pages, binary32
 * values otherwise); n_scored [n_rows] (may be NULL): vectors scored = eligible pages + fine
 * candidate tokens.
 */
void lsa_ref_page_recall(int64_t n_rows, int H, int d, int64_t L, const int64_t *pos,
                         const uint16_t *q, const float *w, const uint16_t *pk, const void *keys,
                         int key_dtype, const float *scale, int k, int S, int W, int P, int M,
                         int32_t *page_ids, int32_t *cand_ids, double *cand_scores,
                         double *coarse, int64_t *n_scored)
{
    int64_t n_pages = (L + P - 1) / P;
    int64_t slots = (int64_t)M * P;
    for (int64_t t = 0; t < n_rows; ++t) {
        int64_t V = pos[t] + 1 < L ? pos[t] + 1 : L;
        int32_t *pid = page_ids + t * M;
        int32_t *cid = cand_ids + t * slots;
        double *csc = cand_scores + t * slots;
        for (int j = 0; j < M; ++j) pid[j] = -1;
        for (int64_t j = 0; j < slots; ++j) { cid[j] = -1; csc[j] = -INFINITY; }
        if (coarse)
            for (int64_t p = 0; p < n_pages; ++p) coarse[t * n_pages + p] = -INFINITY;
        if (n_scored) n_scored[t] = 0;
        if (V <= k) continue;

        int64_t lo = V - W; /* middle is [S, lo) */
        int64_t p_first = S / P, p_last = (lo - 1) / P;
        int64_t n_elig = p_last - p_first + 1;

        /* coarse scores: the page key dequantises to bf16 values; reuse the score definition
         * with a unit scale and bf16 "keys". */
        double *Ic = (double *)malloc(sizeof(double) * (size_t)n_elig);
        int64_t one_pos = n_pages; /* every page is "in the past" of this pseudo-query */
#pragma omp parallel for schedule(static)
        for (int64_t p = p_first; p <= p_last; ++p) {
            double v;
            lsa_ref_index_scores(1, H, d, 1, &one_pos, q + t * H * d, w + t * H,
                                 pk + p * d, REF_KEY_BF16, NULL, &v, NULL, NULL);
            Ic[p - p_first] = v;
        }
        cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)n_elig);
        for (int64_t p = p_first; p <= p_last; ++p) {
            c[p - p_first].score = (float)Ic[p - p_first];
            c[p - p_first].id = (int32_t)p;
            if (coarse) coarse[t * n_pages + p] = (double)(float)Ic[p - p_first];
        }
        qsort(c, (size_t)n_elig, sizeof(cand_t), by_score_desc_id_asc);
        int take = n_elig < M ? (int)n_elig : M;
        qsort(c, (size_t)take, sizeof(cand_t), by_id_asc);
        int64_t n_fine = 0;
#pragma omp parallel for schedule(static) reduction(+ : n_fine)
        for (int i = 0; i < take; ++i) {
            int64_t p = c[i].id;
            pid[i] = (int32_t)p;
            for (int j = 0; j < P; ++j) {
                int64_t s = p * P + j;
                if (s < S || s >= lo) continue;
                double v;
                int64_t spos = L; /* the token is in the past of the query: score it */
                lsa_ref_index_scores(1, H, d, 1, &spos, q + t * H * d, w + t * H,
                                     key_dtype == REF_KEY_BF16
                                         ? (const void *)((const uint16_t *)keys + s * d)
                                         : (const void *)((const uint8_t *)keys + s * d),
                                     key_dtype, scale ? scale + s : NULL, &v, NULL, NULL);
                cid[(int64_t)i * P + j] = (int32_t)s;
                csc[(int64_t)i * P + j] = v;
                ++n_fine;
            }
        }
        if (n_scored) n_scored[t] = n_elig + n_fine;
        free(c);
        free(Ic);
    }
}

/* ------------------------------------------------------------------------------------------ */
/* a6 + a7. Sparse attention over the selected tokens (reused across layers).                  */
/* ------------------------------------------------------------------------------------------ */

/*
 * [DSA] 3. Sparse Attention Calculator: ordinary softmax attention restricted to the selected
 * tokens.  For query row t and head h, over the entries j of idx[t] that are not -1:
 *
 *   logit_j = tau * q[t,h] . K[idx_j]          (first d_qk columns of the K rows)
 *   o[t,h]  = sum_j softmax(logit)_j V[idx_j]  (first d_v columns of the V rows)
 *   lse     = log sum_j exp(logit_j)           (natural log)
 *
 * With MLA's latent cache the K and V rows are the same rows (V = the first d_v columns).
 * No valid entry: o = 0, lse = -inf.  Everything in fp64.
 * [LSA] Cross-Layer Indexing reuses one idx for N consecutive layers: callers run this once
 * per layer with that layer's q and cache and the same idx.
 */
void lsa_ref_sparse_attn(int64_t n_rows, int Hq, int d_qk, int d_v, int k, const uint16_t *q,
                         const uint16_t *kbase, int64_t k_stride, const uint16_t *vbase,
                         int64_t v_stride, const int32_t *idx, double tau, double *o,
                         double *lse)
{
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t t = 0; t < n_rows; ++t) {
        for (int h = 0; h < Hq; ++h) {
            const int32_t *sel = idx + t * k;
            const uint16_t *qh = q + (t * Hq + h) * d_qk;
            double *oh = o + (t * Hq + h) * d_v;
            double *logit = (double *)malloc(sizeof(double) * (size_t)k);
            double mx = -INFINITY;
            for (int j = 0; j < k; ++j) {
                if (sel[j] < 0) continue;
                const uint16_t *kr = kbase + (int64_t)sel[j] * k_stride;
                double dot = 0.0;
                for (int i = 0; i < d_qk; ++i)
                    dot += lsa_ref_bf16_to_double(qh[i]) * lsa_ref_bf16_to_double(kr[i]);
                logit[j] = tau * dot;
                if (logit[j] > mx) mx = logit[j];
            }
            for (int c = 0; c < d_v; ++c) oh[c] = 0.0;
            if (mx == -INFINITY) {
                if (lse) lse[t * Hq + h] = -INFINITY;
                free(logit);
                continue;
            }
            double den = 0.0;
            for (int j = 0; j < k; ++j) {
                if (sel[j] < 0) continue;
                double e = exp(logit[j] - mx);
                den += e;
                const uint16_t *vr = vbase + (int64_t)sel[j] * v_stride;
                for (int c = 0; c < d_v; ++c) oh[c] += e * lsa_ref_bf16_to_double(vr[c]);
            }
            for (int c = 0; c < d_v; ++c) oh[c] /= den;
            if (lse) lse[t * Hq + h] = mx + log(den);
            free(logit);
        }
    }
}

/* ------------------------------------------------------------------------------------------ */
/* f4. Backward of the sparse attention and of the indexer scores (the training path).         */
/* ------------------------------------------------------------------------------------------ */

/*
 * [LSA] abstract: LSA trains natively (to one million tokens), so the attention over the
 * selected tokens and the indexer's scores both carry gradients.  The pages print no backward
 * pass; the functions below are the derivatives of the forward definitions above, written out,
 * on binary64 inputs (bf16 and e4m3 values convert exactly; callers pass the converted arrays).
 * Their pins are central finite differences of the forward functions on binary64 inputs
 * (lsa_ref_sparse_attn_f64, lsa_ref_index_scores_sel_f64), so that they are checked against the
 * forward definitions and not against a second copy of themselves.
 */

/* For every key row r in [0, n_keys), the entries (t, j) of an index list with idx[t][j] == r,
 * in increasing (t, j) order: CSR arrays start[n_keys + 1] and ent[] (ent = t * k + j). */
static void invert_idx(int64_t n_rows, int k, const int32_t *idx, int64_t n_keys, int64_t **start,
                       int64_t **ent)
{
    int64_t *st = (int64_t *)calloc((size_t)n_keys + 1, sizeof(int64_t));
    for (int64_t e = 0; e < n_rows * k; ++e)
        if (idx[e] >= 0 && idx[e] < n_keys) ++st[idx[e] + 1];
    for (int64_t r = 0; r < n_keys; ++r) st[r + 1] += st[r];
    int64_t *fill = (int64_t *)malloc(sizeof(int64_t) * ((size_t)n_keys + 1));
    memcpy(fill, st, sizeof(int64_t) * ((size_t)n_keys + 1));
    int64_t *en = (int64_t *)malloc(sizeof(int64_t) * ((size_t)st[n_keys] + 1));
    for (int64_t e = 0; e < n_rows * k; ++e)
        if (idx[e] >= 0 && idx[e] < n_keys) en[fill[idx[e]]++] = e;
    free(fill);
    *start = st;
    *ent = en;
}

/*
 * The sparse attention of lsa_ref_sparse_attn on binary64 inputs, with entries outside
 * [0, n_keys) skipped: q [n_rows][Hq][d_qk], K rows k_stride apart, V rows v_stride apart.
 */
void lsa_ref_sparse_attn_f64(int64_t n_rows, int Hq, int d_qk, int d_v, int k, const double *q,
                             const double *K, int64_t k_stride, const double *V, int64_t v_stride,
                             const int32_t *idx, int64_t n_keys, double tau, double *o,
                             double *lse)
{
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t t = 0; t < n_rows; ++t) {
        for (int h = 0; h < Hq; ++h) {
            const int32_t *sel = idx + t * k;
            const double *qh = q + (t * Hq + h) * d_qk;
            double *oh = o + (t * Hq + h) * d_v;
            double *logit = (double *)malloc(sizeof(double) * (size_t)k);
            double mx = -INFINITY;
            for (int j = 0; j < k; ++j) {
                if (sel[j] < 0 || sel[j] >= n_keys) continue;
                const double *kr = K + (int64_t)sel[j] * k_stride;
                double dot = 0.0;
                for (int i = 0; i < d_qk; ++i) dot += qh[i] * kr[i];
                logit[j] = tau * dot;
                if (logit[j] > mx) mx = logit[j];
            }
            for (int c = 0; c < d_v; ++c) oh[c] = 0.0;
            if (mx == -INFINITY) {
                if (lse) lse[t * Hq + h] = -INFINITY;
                free(logit);
                continue;
            }
            double den = 0.0;
            for (int j = 0; j < k; ++j) {
                if (sel[j] < 0 || sel[j] >= n_keys) continue;
                const double e = exp(logit[j] - mx);
                den += e;
                const double *vr = V + (int64_t)sel[j] * v_stride;
                for (int c = 0; c < d_v; ++c) oh[c] += e * vr[c];
            }
            for (int c = 0; c < d_v; ++c) oh[c] /= den;
            if (lse) lse[t * Hq + h] = mx + log(den);
            free(logit);
        }
    }
}

/*
 * Gradients of the sparse attention.  With P_j = softmax(logit)_j over the valid entries j of
 * idx[t] (logit_j = tau q[t,h] . K[idx_j]) and the output gradient g = dLoss/do[t,h]:
 *   dP_j = g . V[idx_j]
 *   dS_j = P_j (dP_j - sum_i P_i dP_i)           (the softmax Jacobian applied to dP)
 *   dq[t,h]      = tau sum_j dS_j K[idx_j]
 *   dK[idx_j]   += tau dS_j q[t,h]               (over every row t and head h that selected it)
 *   dV[idx_j]   += P_j g
 * dq [n_rows][Hq][d_qk] is written; dK [n_keys][d_qk] and dV [n_keys][d_v] are written too
 * (rows nobody selected get 0).  A latent cache, whose rows serve as K and as V, has the
 * gradient dK[r][c] + (c < d_v ? dV[r][c] : 0) on row r.  The forward is recomputed in fp64.
 * Pass 1 handles one (t, h) at a time (dq); pass 2 one key row at a time, over the entries
 * that selected it in increasing order (dK, dV).
 */
void lsa_ref_sparse_attn_backward(int64_t n_rows, int Hq, int d_qk, int d_v, int k,
                                  const double *q, const double *K, int64_t k_stride,
                                  const double *V, int64_t v_stride, const int32_t *idx,
                                  int64_t n_keys, double tau, const double *g, double *dq,
                                  double *dK, double *dV)
{
    double *lse = (double *)malloc(sizeof(double) * (size_t)(n_rows * Hq + 1));
    double *D = (double *)malloc(sizeof(double) * (size_t)(n_rows * Hq + 1));
    /* pass 1: lse, D = sum_j P_j dP_j, dq */
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t t = 0; t < n_rows; ++t) {
        for (int h = 0; h < Hq; ++h) {
            const int32_t *sel = idx + t * k;
            const double *qh = q + (t * Hq + h) * d_qk;
            const double *gh = g + (t * Hq + h) * d_v;
            double *dqh = dq + (t * Hq + h) * d_qk;
            double *logit = (double *)malloc(sizeof(double) * (size_t)k);
            double *dP = (double *)malloc(sizeof(double) * (size_t)k);
            double mx = -INFINITY;
            for (int j = 0; j < k; ++j) {
                if (sel[j] < 0 || sel[j] >= n_keys) continue;
                const double *kr = K + (int64_t)sel[j] * k_stride;
                const double *vr = V + (int64_t)sel[j] * v_stride;
                double dot = 0.0, gv = 0.0;
                for (int i = 0; i < d_qk; ++i) dot += qh[i] * kr[i];
                for (int c = 0; c < d_v; ++c) gv += gh[c] * vr[c];
                logit[j] = tau * dot;
                dP[j] = gv;
                if (logit[j] > mx) mx = logit[j];
            }
            for (int i = 0; i < d_qk; ++i) dqh[i] = 0.0;
            double den = 0.0, pdp = 0.0;
            if (mx != -INFINITY) {
                for (int j = 0; j < k; ++j)
                    if (sel[j] >= 0 && sel[j] < n_keys) den += exp(logit[j] - mx);
                const double ls = mx + log(den);
                for (int j = 0; j < k; ++j)
                    if (sel[j] >= 0 && sel[j] < n_keys) pdp += exp(logit[j] - ls) * dP[j];
                for (int j = 0; j < k; ++j) {
                    if (sel[j] < 0 || sel[j] >= n_keys) continue;
                    const double dS = exp(logit[j] - ls) * (dP[j] - pdp);
                    const double *kr = K + (int64_t)sel[j] * k_stride;
                    for (int i = 0; i < d_qk; ++i) dqh[i] += tau * dS * kr[i];
                }
                lse[t * Hq + h] = ls;
            } else {
                lse[t * Hq + h] = -INFINITY;
            }
            D[t * Hq + h] = pdp;
            free(logit);
            free(dP);
        }
    }
    /* pass 2: dK, dV per key row */
    int64_t *start, *ent;
    invert_idx(n_rows, k, idx, n_keys, &start, &ent);
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t r = 0; r < n_keys; ++r) {
        double *dk = dK + r * d_qk;
        double *dv = dV + r * d_v;
        for (int i = 0; i < d_qk; ++i) dk[i] = 0.0;
        for (int c = 0; c < d_v; ++c) dv[c] = 0.0;
        const double *kr = K + r * k_stride;
        const double *vr = V + r * v_stride;
        for (int64_t e = start[r]; e < start[r + 1]; ++e) {
            const int64_t t = ent[e] / k;
            for (int h = 0; h < Hq; ++h) {
                const double *qh = q + (t * Hq + h) * d_qk;
                const double *gh = g + (t * Hq + h) * d_v;
                double dot = 0.0, gv = 0.0;
                for (int i = 0; i < d_qk; ++i) dot += qh[i] * kr[i];
                for (int c = 0; c < d_v; ++c) gv += gh[c] * vr[c];
                const double P = exp(tau * dot - lse[t * Hq + h]);
                const double dS = P * (gv - D[t * Hq + h]);
                for (int i = 0; i < d_qk; ++i) dk[i] += tau * dS * qh[i];
                for (int c = 0; c < d_v; ++c) dv[c] += P * gh[c];
            }
        }
    }
    free(start);
    free(ent);
    free(lse);
    free(D);
}

/*
 * The indexer scores of lsa_ref_index_scores at the selected entries only, on binary64 inputs:
 *   I[t][j] = sum_h w[t,h] ReLU(q[t,h] . keys[idx[t][j]])   for 0 <= idx[t][j] < V_t,
 * V_t = min(n_keys, pos_t + 1); other entries get 0 (they carry no score).
 */
void lsa_ref_index_scores_sel_f64(int64_t n_rows, int H, int d, int k, const int64_t *pos,
                                  const double *q, const double *w, const double *keys,
                                  const int32_t *idx, int64_t n_keys, double *I)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < n_rows; ++t) {
        const int64_t V = pos[t] + 1 < n_keys ? pos[t] + 1 : n_keys;
        for (int j = 0; j < k; ++j) {
            const int32_t s = idx[t * k + j];
            double acc = 0.0;
            if (s >= 0 && s < V) {
                for (int h = 0; h < H; ++h) {
                    double dot = 0.0;
                    for (int i = 0; i < d; ++i) dot += q[(t * H + h) * d + i] * keys[(int64_t)s * d + i];
                    acc += w[t * H + h] * (dot > 0.0 ? dot : 0.0);
                }
            }
            I[t * k + j] = acc;
        }
    }
}

/*
 * Gradients of the indexer scores at the selected entries, given gI[t][j] = dLoss/dI[t][j]
 * (entries outside [0, V_t) carry none), with ReLU'(0) taken as 0:
 *   dw[t,h]   = sum_j gI[t,j] ReLU(q[t,h] . keys[s_j])
 *   dq[t,h]   = sum_j gI[t,j] w[t,h] [q[t,h] . keys[s_j] > 0] keys[s_j]
 *   dk[s]     = sum over entries (t, j) with s_j = s of sum_h gI[t,j] w[t,h] [q[t,h] . keys[s] > 0] q[t,h]
 * dq [n_rows][H][d], dw [n_rows][H] and dk [n_keys][d] are written (rows nobody selected get 0).
 */
void lsa_ref_index_scores_backward(int64_t n_rows, int H, int d, int k, const int64_t *pos,
                                   const double *q, const double *w, const double *keys,
                                   const int32_t *idx, int64_t n_keys, const double *gI,
                                   double *dq, double *dw, double *dk)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < n_rows; ++t) {
        const int64_t V = pos[t] + 1 < n_keys ? pos[t] + 1 : n_keys;
        for (int h = 0; h < H; ++h) {
            const double *qh = q + (t * H + h) * d;
            double *dqh = dq + (t * H + h) * d;
            double dwh = 0.0;
            for (int i = 0; i < d; ++i) dqh[i] = 0.0;
            for (int j = 0; j < k; ++j) {
                const int32_t s = idx[t * k + j];
                if (s < 0 || s >= V) continue;
                const double *kr = keys + (int64_t)s * d;
                double dot = 0.0;
                for (int i = 0; i < d; ++i) dot += qh[i] * kr[i];
                if (dot > 0.0) {
                    dwh += gI[t * k + j] * dot;
                    for (int i = 0; i < d; ++i) dqh[i] += gI[t * k + j] * w[t * H + h] * kr[i];
                }
            }
            dw[t * H + h] = dwh;
        }
    }
    /* the entries outside [0, V_t) are dropped before the inversion */
    int32_t *vidx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n_rows * k + 1));
    for (int64_t t = 0; t < n_rows; ++t) {
        const int64_t V = pos[t] + 1 < n_keys ? pos[t] + 1 : n_keys;
        for (int j = 0; j < k; ++j) {
            const int32_t s = idx[t * k + j];
            vidx[t * k + j] = (s >= 0 && s < V) ? s : -1;
        }
    }
    int64_t *start, *ent;
    invert_idx(n_rows, k, vidx, n_keys, &start, &ent);
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t r = 0; r < n_keys; ++r) {
        double *dkr = dk + r * d;
        for (int i = 0; i < d; ++i) dkr[i] = 0.0;
        const double *kr = keys + r * d;
        for (int64_t e = start[r]; e < start[r + 1]; ++e) {
            const int64_t t = ent[e] / k;
            for (int h = 0; h < H; ++h) {
                const double *qh = q + (t * H + h) * d;
                double dot = 0.0;
                for (int i = 0; i < d; ++i) dot += qh[i] * kr[i];
                if (dot > 0.0)
                    for (int i = 0; i < d; ++i) dkr[i] += gI[ent[e]] * w[t * H + h] * qh[i];
            }
        }
    }
    free(start);
    free(ent);
    free(vidx);
}
