/*
 * lsa.h -- C ABI of the MI355X (gfx950) LongCat Sparse Attention token-selection library.
 *
 * The library computes, for every query of every sequence in a batch:
 *   1. lsa_index_scores  -- Lightning-Indexer scores I[t,s] = sum_h w[t,h] ReLU(q[t,h] . k[s])
 *   2. lsa_topk_select   -- Streaming-Aware selection: sink + local window + dynamic top-k
 *   3. lsa_page_summary  -- page keys for Hierarchical Indexing (mean of a page's keys)
 *   4. lsa_page_recall   -- Hierarchical Indexing: coarse page recall, fine scores in the pages
 *   5. lsa_sparse_attn   -- attention over the selected tokens (MLA latent cache or MHA),
 *                           reusable by several layers with one index list (Cross-Layer Indexing)
 *
 * Sources.  "LongCat Sparse Attention: Taming the Lightning via Streaming-aware Hierarchical
 * Cross-Layer Indexing" (paper summary page: abstract, key contributions, limitations); the
 * "LongCat-Flash-Lite-Sparse" model card (SI / CLI / HI bullet list); the Baidu Cloud article on
 * DeepSeek's Lightning Indexer ("Core Architecture Analysis": scoring module, token selector,
 * sparse attention calculator).
 *
 * Conventions shared by every entry point.
 *   Memory     Every tensor pointer is a caller-owned DEVICE pointer on the current HIP device,
 *              row-major and contiguous in the layout given at the argument.  The library
 *              allocates nothing, keeps no pointer after it returns and has no mutable global
 *              state; it is reentrant.  Workspaces (`ws`) are caller-owned device buffers of at
 *              least lsa_workspace_bytes() bytes, 256-byte aligned; their contents on entry do
 *              not matter.
 *   Streams    `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every call
 *              only enqueues kernels on it and never synchronises.
 *   Errors     Every argument is checked on the host before anything is enqueued: on any error
 *              nothing is enqueued and no output is written.  A failed launch returns
 *              LSA_ERR_DEVICE.  The library never aborts, prints or throws across the ABI.
 *   Numbers    bf16 = bfloat16; fp8 = OCP e4m3fn (no infinities, S.1111.111 is NaN) with one
 *              fp32 scale per key token.  Inputs must be finite.  Scores accumulate in fp32.
 *   Validity   Query i of a sequence sits at absolute position q_pos0 + i and sees the keys
 *              [0, V_i), V_i = min(kv_len, q_pos0 + i + 1).  Decode: n_q = 1, q_pos0 = kv_len-1.
 *   Order      Selections are deterministic: ties in score go to the lower token index (-0 and
 *              +0 are equal).  Identical calls give bitwise-identical outputs.
 */
#ifndef LSA_H
#define LSA_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define LSA_API __attribute__((visibility("default")))
#else
#define LSA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LSA_OK = 0,
    LSA_ERR_NULL_POINTER = 1,        /* a required pointer is NULL */
    LSA_ERR_BAD_SHAPE = 2,           /* a size or budget is out of range or inconsistent */
    LSA_ERR_BAD_DTYPE = 3,           /* unknown key dtype, or scale given/missing wrongly */
    LSA_ERR_UNSUPPORTED = 4,         /* valid, but outside what the kernels are built for */
    LSA_ERR_WORKSPACE_TOO_SMALL = 5, /* ws_bytes < lsa_workspace_bytes(...) or ws misaligned */
    LSA_ERR_DEVICE = 6               /* a HIP call or kernel launch failed */
} lsa_status;

typedef enum {
    LSA_KEY_BF16 = 1,     /* keys [B, L, d] bf16; key_scale must be NULL */
    LSA_KEY_FP8_E4M3 = 2  /* keys [B, L, d] e4m3fn codes; key_scale [B, L] fp32 required */
} lsa_key_dtype;

/* Shape of an indexing problem.  head_dim in {64, 128}; n_heads in {4, 8, 16, 32, 64};
 * 1 <= kv_len < 2^31; q_pos0 >= 0. */
typedef struct {
    int32_t batch, n_q, n_heads, head_dim;
    int64_t kv_len, q_pos0;
} lsa_index_shape;

/* Selection budget per query: k tokens = sink [0,S) + window (the W latest valid tokens) +
 * k - S - W dynamic picks.  0 <= S, 0 <= W, S + W <= k. */
typedef struct {
    int32_t k, sink, window;
} lsa_budget;

/* Attention shape.  latent = 1: MLA latent cache -- `v` must equal `k`, V is the first d_v
 * columns of the K rows and every query head shares the one latent head.  Row strides are in
 * elements (bf16), multiples of 8, >= d_qk (K) and >= d_v (V). */
typedef struct {
    int32_t n_heads, d_qk, d_v, latent;
    int64_t k_row_stride, v_row_stride;
    float scale; /* softmax temperature applied to q . k */
} lsa_attn_shape;

/*
 * lsa_index_scores -- Lightning-Indexer scores (Baidu Cloud article, "1. Lightweight Scoring
 * Module": ReLU of query-key dot products; DeepSeek Sparse Attention's indexer weights its H
 * heads per query):
 *     scores[b,i,s] = sum_h w[b,i,h] * ReLU( q[b,i,h,:] . k[b,s,:] )      for s <  V_i
 *     scores[b,i,s] = -inf                                                for s >= V_i
 * For fp8 keys k[b,s,:] = key_scale[b,s] * e4m3(keys[b,s,:]) (the scale is applied once after
 * the head sum; ReLU commutes with a positive scale).  No 1/sqrt(d): fold it into w.
 *   q          [B, n_q, H, d] bf16
 *   w          [B, n_q, H]    fp32
 *   keys       [B, L, d]      bf16 or e4m3 codes (see lsa_key_dtype)
 *   key_scale  [B, L] fp32 (fp8 keys; each scale > 0) or NULL (bf16 keys)
 *   scores     [B, n_q, L]    fp32, written completely
 */
LSA_API lsa_status lsa_index_scores(const lsa_index_shape *shape, const void *q, const float *w,
                            const void *keys, lsa_key_dtype key_dtype, const float *key_scale,
                            float *scores, void *stream);

/*
 * lsa_topk_select -- Streaming-Aware Indexing selection (model card, SI bullet; paper summary
 * page, abstract strategy (1) and the limitation that fixed regions take part of the budget)
 * on top of the Lightning Indexer's top-k (Baidu Cloud article, "2. Dynamic Token Selector").
 * For each query with valid length V:
 *   V <= k : idx = 0, 1, ..., V-1, then -1 up to k.
 *   V >  k : idx = [sink 0..S-1] [window V-W..V-1] [dynamic: the k-S-W best tokens of the
 *            middle [S, V-W) by (score desc, index asc), listed in ascending index order].
 * Flat mode (cand_ids == NULL): scores is [B, n_q, n_cand] with n_cand == kv_len, scores[..., s]
 *   belongs to token s (only the middle region is read).
 * Candidate mode: scores and cand_ids are [B, n_q, n_cand]; cand_ids rows are ascending with -1
 *   for empty slots (the output of lsa_page_recall).  Only ids in the middle [S, V-W) compete;
 *   with fewer than k-S-W of them all are taken and the tail of idx is -1.
 *   idx        [B, n_q, k] int32, written completely
 *   ws         workspace of lsa_workspace_bytes(LSA_OP_TOPK_SELECT, shape, budget, 0, 0, n_cand,
 *              NULL) bytes (0 for many short rows; few long rows are split over workgroups)
 * Limits: k - S - W <= 65536.
 */
LSA_API lsa_status lsa_topk_select(const lsa_index_shape *shape, lsa_budget budget, const float *scores,
                           int64_t n_cand, const int32_t *cand_ids, int32_t *idx, void *ws,
                           size_t ws_bytes, void *stream);

/*
 * lsa_page_summary -- page keys for Hierarchical Indexing.  The model card's HI bullet recalls
 * blocks of tokens by coarse scores but does not define a block's coarse key; this library
 * defines it as the mean of the block's dequantised keys, fixed to the bit:
 *     v[j] = fp32(key_scale[s] * e4m3(keys[s,:]))  (bf16 keys: the bf16 value), j = s - p*P,
 *            and +0 for slots past kv_len;
 *     page_keys[b,p,:] = bf16_rne( pairwise_fp32_tree_sum(v[0..P)) / n_p ),
 * n_p = number of tokens of page p that exist.  Pages [page_lo, page_hi) are (re)written, so a
 * decode loop can extend the table one completed page at a time.
 *   page_size  P, a power of two in [1, 256]
 *   page_keys  [B, ceil(L/P), d] bf16
 */
LSA_API lsa_status lsa_page_summary(const lsa_index_shape *shape, int32_t page_size, const void *keys,
                            lsa_key_dtype key_dtype, const float *key_scale, int64_t page_lo,
                            int64_t page_hi, void *page_keys, void *stream);

/*
 * lsa_page_recall -- Hierarchical Indexing's two stages (model card, HI bullet: recall candidate
 * blocks by coarse scores, then select tokens finely inside them; paper summary page, key
 * contribution 3: per-query cost O(L/P + M P) instead of O(L)).  For each query with V > k:
 *   eligible pages  the pages overlapping the middle [S, V-W): floor(S/P) .. floor((V-W-1)/P)
 *   coarse score    sum_h w ReLU(q . page_keys[p])                    (fp32)
 *   recall          the m_pages best eligible pages by (coarse desc, page asc), all if fewer;
 *                   page_ids lists them ascending, -1 padded
 *   candidates      slot i*P + j of the i-th recalled page p holds token p*P + j when it lies
 *                   in [S, V-W): cand_ids = the token, cand_scores = its indexer score (as
 *                   lsa_index_scores computes it); other slots: id -1, score -inf.
 * For V <= k nothing is recalled (all -1 / -inf): the selector then takes every valid token.
 * Feed (cand_scores, cand_ids, n_cand = m_pages * P) to lsa_topk_select.
 *   page_keys    [B, ceil(L/P), d] bf16 from lsa_page_summary
 *   page_ids     [B, n_q, m_pages] int32
 *   cand_scores  [B, n_q, m_pages * P] fp32;  cand_ids  [B, n_q, m_pages * P] int32
 *   ws           lsa_workspace_bytes(LSA_OP_PAGE_RECALL, ...) bytes
 * Limits: page_size a power of two in [32, 256] with head_dim 128 or [32, 256] with 64;
 *         1 <= m_pages <= 65536.
 */
LSA_API lsa_status lsa_page_recall(const lsa_index_shape *shape, lsa_budget budget, int32_t page_size,
                           int32_t m_pages, const void *q, const float *w, const void *page_keys,
                           const void *keys, lsa_key_dtype key_dtype, const float *key_scale,
                           int32_t *page_ids, float *cand_scores, int32_t *cand_ids, void *ws,
                           size_t ws_bytes, void *stream);

/*
 * lsa_sparse_attn -- attention over the selected tokens only (Baidu Cloud article, "3. Sparse
 * Attention Calculator"); with an MLA latent cache (the model card: LSA replaces dense MLA).
 * For each query i, head h, over the entries j of idx[b,i,:] that are in [0, kv_len):
 *     logit_j = scale * q[b,i,h,:] . K[b, idx_j, 0:d_qk]
 *     out[b,i,h,:] = sum_j softmax(logit)_j V[b, idx_j, 0:d_v]     (bf16, round to nearest)
 *     lse[b,i,h]   = log sum_j exp(logit_j)                          (natural log; optional)
 * Entries of -1 (or outside [0, kv_len)) are skipped; a row with none gives out = 0,
 * lse = -inf.  Cross-Layer Indexing (paper summary page, strategy (2)): call once per layer with
 * that layer's q / cache and the same idx.
 *   shape   uses batch, n_q and kv_len
 *   budget  sink/window say idx[.., 0:S] and idx[.., S:S+W] are contiguous runs (the layout
 *           lsa_topk_select writes when V > k); rows whose first entry is not 0 or whose
 *           runs are not contiguous fall back to a plain gather.  {0,0,0} = always gather.
 *   q       [B, n_q, Hq, d_qk] bf16
 *   k, v    [B, L, row_stride] bf16 (latent: v == k)
 *   idx     [B, n_q, k] int32
 *   out     [B, n_q, Hq, d_v] bf16;  lse  [B, n_q, Hq] fp32 or NULL
 *   ws      lsa_workspace_bytes(LSA_OP_SPARSE_ATTN, ...) bytes
 * Limits: latent: Hq a multiple of 16 (n_q * Hq / 16 <= 65535), d_qk = 576, d_v = 512 (the
 *         MLA shape: 512 latent + 64 rope columns); otherwise (per-head kernel): d_qk, d_v
 *         multiples of 8, <= 256.
 */
LSA_API lsa_status lsa_sparse_attn(const lsa_index_shape *shape, const lsa_attn_shape *attn,
                           lsa_budget budget, const void *q, const void *k, const void *v,
                           const int32_t *idx, void *out, float *lse, void *ws, size_t ws_bytes,
                           void *stream);

enum { LSA_OP_TOPK_SELECT = 1, LSA_OP_PAGE_RECALL = 2, LSA_OP_SPARSE_ATTN = 3 };

/* Workspace bytes needed by `op` for these arguments (0 if none).  Arguments an op does not
 * use may be NULL / 0 (LSA_OP_TOPK_SELECT reads n_cand; 0 means flat, n_cand = kv_len).
 * Returns (size_t)-1 for invalid arguments. */
LSA_API size_t lsa_workspace_bytes(int op, const lsa_index_shape *shape, lsa_budget budget,
                           int32_t page_size, int32_t m_pages, int64_t n_cand,
                           const lsa_attn_shape *attn);

/* A static, human-readable name of a status code. */
LSA_API const char *lsa_status_string(lsa_status status);

#ifdef __cplusplus
}
#endif

#endif /* LSA_H */
