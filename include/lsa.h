/*
 * lsa.h -- C ABI of the MI355X (gfx950) LongCat Sparse Attention token-selection library.
 *
 * The library computes, for every query of every sequence in a batch:
 *   1. lsa_index_scores  -- Lightning-Indexer scores I[t,s] = sum_h w[t,h] ReLU(q[t,h] . k[s])
 *   2. lsa_topk_select   -- Streaming-Aware selection: sink + local window + dynamic top-k
 *   3. lsa_page_summary  -- page keys for Hierarchical Indexing (mean of a page's keys)
 *   4. lsa_page_recall   -- Hierarchical Indexing: coarse page recall, fine scores in the pages
 *   5. lsa_sparse_attn   -- attention over the selected tokens (MLA latent cache or MHA),
 *                           reusable by several layers with one index list (Cross-Layer Indexing);
 *                           lsa_sparse_attn_layers runs such a group of layers in one call
 *   6. lsa_sparse_attn_backward, lsa_index_scores_backward -- the gradients of 5 and of the
 *                           indexer scores at the selected entries (the training path)
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
 *              +0 are equal).  Identical calls give bitwise-identical outputs, except the
 *              gradients of the backward entry points (fp32 atomic sums).
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
 * 1 <= kv_len < 2^31; q_pos0 >= 0.
 * Ragged batches (model card, HI bullet: sequences of different lengths share a batch): every
 * key / latent cache is laid out [B, kv_len, ...] with kv_len the capacity, and two optional
 * DEVICE arrays of B int32 (4-byte aligned, read by the kernels) give each sequence its own
 *   seq_len[b]   keys of sequence b (rows [0, seq_len[b]) of its cache; the rest is never read
 *                as a key: scores -inf, page keys of pages wholly past it 0, attention skips
 *                ids >= seq_len[b]); clamped into [0, kv_len].  NULL: kv_len for every b.
 *   seq_pos0[b]  position of sequence b's first query (query i sees keys
 *                [0, min(seq_len[b], seq_pos0[b] + i + 1))); negative values count as 0.
 *                NULL: q_pos0 for every b.  Ragged decode: seq_pos0[b] = seq_len[b] - 1.
 * With either array set, q_pos0 only serves where an array is NULL. */
typedef struct {
    int32_t batch, n_q, n_heads, head_dim;
    int64_t kv_len, q_pos0;
    const int32_t *seq_len;
    const int32_t *seq_pos0;
    /* Paged indexer keys (optional; block_table NULL = dense keys [B, kv_len, d]).  The keys
     * (and the fp8 keys' scales) are then pools of n_blocks blocks of block_size rows,
     * [n_blocks * block_size, d] (and [n_blocks * block_size]), and key s of sequence b is pool
     * row  block_table[b * blocks_per_seq + s / block_size] * block_size + s % block_size.
     * A table entry outside [0, n_blocks) gives that block's keys the score -inf.
     * block_size a power of two in [32, 2^20]; blocks_per_seq * block_size >= kv_len;
     * n_blocks * block_size < 2^31.  Only the calls that read indexer keys look at these
     * fields: lsa_index_scores and lsa_index_select take them at decode shapes (see there);
     * lsa_page_summary and lsa_page_recall with 32 <= page_size <= block_size (a page inside
     * one table block; a page whose entry lies outside the pool gets the zero page key);
     * lsa_index_scores_q8 and lsa_index_scores_backward return LSA_ERR_UNSUPPORTED for them. */
    const int32_t *block_table; /* [B, blocks_per_seq] int32, device */
    int32_t block_size, blocks_per_seq;
    int64_t n_blocks;
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
    /* Paged latent cache (optional; block_table NULL = dense caches [B, L, row]).  The cache
     * k (== v) is then a pool of n_blocks blocks of block_size rows, [n_blocks * block_size,
     * row], and token s of sequence b is pool row
     *     block_table[b * blocks_per_seq + s / block_size] * block_size + s % block_size.
     * A table entry outside [0, n_blocks) makes the tokens of that block skipped entries.
     * block_size a power of two; blocks_per_seq * block_size >= kv_len;
     * n_blocks * block_size < 2^31.  lsa_sparse_attn and lsa_sparse_attn_layers (latent
     * caches) take it; the per-head cache and the backward do not. */
    const int32_t *block_table; /* [B, blocks_per_seq] int32, device */
    int32_t block_size, blocks_per_seq;
    int64_t n_blocks;
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
 * Paged keys (shape->block_table): keys and key_scale are the pools; scores stay [B, n_q, L]
 *   by token position.  Taken at decode shapes (n_q at most 2 for H of 32 or 64, 4 for 16, 8
 *   for 8, 16 for 4) where a scoring workgroup's key range spans at most 510 table blocks;
 *   other shapes return LSA_ERR_UNSUPPORTED.
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
 * lsa_quantize_queries -- fp8 queries for the quantised indexer (Baidu Cloud article, "1.
 * Lightweight Scoring Module": the indexer's products may run in 8-bit floating point).  Each
 * query row q[b,i,h,:] is quantised the way fp8 key rows are:
 *     q_scale[b,i,h] = max_j |q[b,i,h,j]| / 448      (binary32 division; 1 for an all-zero row)
 *     q8[b,i,h,j]    = e4m3fn( q[b,i,h,j] / q_scale[b,i,h] )   (binary32 division, round to
 *                                                      nearest even, saturating at +-448)
 *   q        [B, n_q, H, d] bf16 (4-byte aligned); uses batch, n_q, n_heads, head_dim of shape
 *   q8       [B, n_q, H, d] e4m3 codes (2-byte aligned);  q_scale  [B, n_q, H] fp32
 * Limits: head_dim 64 or 128.
 */
LSA_API lsa_status lsa_quantize_queries(const lsa_index_shape *shape, const void *q, uint8_t *q8,
                                        float *q_scale, void *stream);

/*
 * lsa_index_scores_q8 -- lsa_index_scores with fp8 queries (from lsa_quantize_queries) against
 * fp8 keys, the contraction on gfx950's 8-bit MFMA (v_mfma_f32_32x32x64_f8f6f4, fp32
 * accumulation; twice the bf16 rate):
 *     scores[b,i,s] = key_scale[b,s] * sum_h w[b,i,h] q_scale[b,i,h] ReLU( e4m3(q8[b,i,h,:]) .
 *                     e4m3(keys[b,s,:]) )                     for s < V_i, -inf beyond
 * i.e. the indexer scores of the dequantised queries.  These differ from the bf16-query scores
 * by the query quantisation (relative error up to 2^-4 per element); the selection they give is
 * an approximation of the bf16-query selection, not the same set.
 *   key_dtype  must be LSA_KEY_FP8_E4M3 (else LSA_ERR_BAD_DTYPE);  q8 16-byte aligned
 *   other arguments as for lsa_index_scores (ragged arrays included)
 */
LSA_API lsa_status lsa_index_scores_q8(const lsa_index_shape *shape, const uint8_t *q8,
                                       const float *q_scale, const float *w, const void *keys,
                                       lsa_key_dtype key_dtype, const float *key_scale,
                                       float *scores, void *stream);

/*
 * lsa_index_select -- lsa_index_scores followed by lsa_topk_select (flat mode), fused for decode
 * (Baidu Cloud article, "Engineering Implementation Breakthroughs: 1. Operator Fusion
 * Optimization": scoring and selection as one operator, so the selection does not start from a
 * cold pass over the score rows).  Outputs are bitwise those of the two calls with the same
 * arguments: `scores` as lsa_index_scores writes it, `idx` as lsa_topk_select selects from it.
 * For few long flat rows (decode: n_q <= 2, heads 32 or 64, enough keys for the long scoring
 * launch, and rows long enough for the chunked selection) the scoring workgroups also histogram
 * their middle-region scores while the scores are in registers, and the selection reads each
 * row's exact threshold bin from those histograms instead of sampling the row before it
 * compacts what lies at or above it.  Where a row has at most 16 scoring workgroups of at most
 * 8192 keys each (32 sequences of up to 128K keys, for one), each workgroup also keeps its own
 * best scores (the histogram bins holding about twice its share of the row's picks) in a slice
 * of `ws`, and a single selection launch gathers the slices instead of passing over the score
 * rows again.  Other shapes run the two ordinary paths.
 *   q, w, keys, key_scale, scores   as for lsa_index_scores (scores 16-byte aligned; paged
 *           keys as there)
 *   idx     [B, n_q, k] int32 as for lsa_topk_select
 *   ws      lsa_workspace_bytes(LSA_OP_INDEX_SELECT, shape, budget, 0, 0, 0, NULL) bytes,
 *           256-byte aligned; its contents on entry do not matter
 * Limits: those of lsa_index_scores and lsa_topk_select.
 */
LSA_API lsa_status lsa_index_select(const lsa_index_shape *shape, lsa_budget budget, const void *q,
                                    const float *w, const void *keys, lsa_key_dtype key_dtype,
                                    const float *key_scale, float *scores, int32_t *idx, void *ws,
                                    size_t ws_bytes, void *stream);

/*
 * lsa_topk_select_noalloc -- lsa_topk_select without a caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  The selection and its result are those of lsa_topk_select with the
 * same arguments; the chunked path (few long rows) uses a scratch array the library holds on
 * each GPU instead of `ws`.  It calls no allocator.
 *   Scratch   16 MiB per GPU, part of the library's code object, held until the process ends.
 *             Calls whose chunked path would need more (lsa_workspace_bytes(LSA_OP_TOPK_SELECT,
 *             ...) > 16 MiB) return LSA_ERR_UNSUPPORTED and enqueue nothing.
 *   Races     Every call on one GPU shares that GPU's scratch: calls that may overlap on the
 *             same GPU (different streams, or concurrent host threads) race and must be
 *             serialised by the caller.  Calls on one stream are ordered and safe.
 *   Set-up    The first call on a device looks up that device's address of the scratch (a HIP
 *             runtime query, no allocation); a failure there returns LSA_ERR_DEVICE.
 */
LSA_API lsa_status lsa_topk_select_noalloc(const lsa_index_shape *shape, lsa_budget budget,
                                           const float *scores, int64_t n_cand,
                                           const int32_t *cand_ids, int32_t *idx, void *stream);

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
 *   page_keys  [B, ceil(L/P), d] bf16, 16-byte aligned (keys too)
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
 * Causality: a query with V < kv_len (a causal prefill chunk) may only recall pages that end
 *   before V, or a page key (a mean over the whole page) would carry later tokens into its
 *   coarse score.  The last eligible page ends before V exactly when window >= page_size - 1,
 *   so a call with q_pos0 + 1 < kv_len, or with per-sequence arrays (whose positions the host
 *   does not see), and window < page_size - 1 returns LSA_ERR_UNSUPPORTED.
 * Limits: page_size a power of two in [32, 256]; 1 <= m_pages <= 65536.
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
 *   shape   uses batch, n_q, kv_len and seq_len (ids at or past a sequence's length are skipped),
 *           and q_pos0 / seq_pos0 (the queries' positions) as a layout hint, below
 *   budget  k = entries per idx row.  sink / window, with the query positions, describe the
 *           layout lsa_topk_select writes: with V = min(length, position + 1), a query with
 *           V <= k lists rows 0 .. V-1 then -1, otherwise idx[.., 0:S] = rows 0 .. S-1 and
 *           idx[.., S:S+W] = rows V-W .. V-1.  The latent kernel loads the first rows it
 *           processes from that layout while the list itself is still arriving, and compares
 *           them with the list; where they differ it loads the listed rows instead.  The layout
 *           is a hint: every result is that of the list as given, whatever sink, window and
 *           the positions say.  Checked: 0 <= sink, 0 <= window, sink + window <= k.
 *   q       [B, n_q, Hq, d_qk] bf16
 *   k, v    [B, L, row_stride] bf16 (latent: v == k), or with attn->block_table a pool of
 *           blocks (see lsa_attn_shape): the ids stay token positions, the table finds the rows
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

/*
 * lsa_sparse_attn_layers -- lsa_sparse_attn for n_layers consecutive layers that share one index
 * list (paper summary page, strategy (2): Cross-Layer Indexing computes the index once for a
 * group of layers; model card, CLI bullet).  Layer l computes what
 * lsa_sparse_attn(shape, attn, budget, q[l], k[l], v[l], idx, out[l], lse[l], ...) computes.
 * With a latent cache every layer's gathers run in one launch and every layer's split partials
 * are merged in one more, instead of two launches per layer; the number of parts the list is
 * cut into for that merge is chosen for the whole launch (as for one layer of a batch n_layers
 * times larger), so a layer's result can differ from the single call's in the last bits of the
 * merge (it is bit-identical where both cut the list alike, and identical calls give identical
 * bits).
 *   n_layers   1 .. 8
 *   q, k, v, out   host arrays of n_layers device pointers, each as for lsa_sparse_attn (the
 *              arrays are read during the call only; the caller keeps ownership)
 *   lse        NULL, or a host array of n_layers device pointers (each may be NULL)
 *   shape, attn, budget, idx   shared by every layer, as for lsa_sparse_attn
 *   ws         n_layers * lsa_workspace_bytes(LSA_OP_SPARSE_ATTN, ...) bytes (rounded up to a
 *              multiple of 256), 256-byte aligned
 * Errors as lsa_sparse_attn; n_layers outside [1, 8] is LSA_ERR_BAD_SHAPE, a NULL array or
 * entry LSA_ERR_NULL_POINTER; batch * n_layers > 65535 is LSA_ERR_UNSUPPORTED.
 */
LSA_API lsa_status lsa_sparse_attn_layers(const lsa_index_shape *shape, const lsa_attn_shape *attn,
                                          lsa_budget budget, int32_t n_layers,
                                          const void *const *q, const void *const *k,
                                          const void *const *v, const int32_t *idx,
                                          void *const *out, float *const *lse, void *ws,
                                          size_t ws_bytes, void *stream);

/*
 * lsa_sparse_attn_backward -- gradients of lsa_sparse_attn (the training path: the paper summary
 * page's abstract reports native training to one million tokens).  For query i, head h and the
 * valid entries j of idx[b,i,:] (the entries lsa_sparse_attn uses), with
 * P_j = exp(scale q . K_j - lse) the forward's attention weights:
 *     dP_j = d_out[b,i,h,:] . V_j,   D = d_out[b,i,h,:] . out[b,i,h,:],   dS_j = P_j (dP_j - D)
 *     d_q[b,i,h,:]      += scale sum_j dS_j K_j
 *     d_k[b, idx_j, :]  += scale dS_j q[b,i,h,:]      (d_qk columns)
 *     d_v[b, idx_j, :]  += P_j d_out[b,i,h,:]         (d_v columns)
 * D uses the forward output (the P-weighted sum of dP equals d_out . out in exact arithmetic).
 * The gradients are ADDED into (fp32; zero them first for plain gradients): layers that share
 * a cache, or the chunks of a chunked prefill, accumulate.  A latent cache (attn->latent) has
 * one gradient array: pass d_v == d_k; its rows get dK + dV (dV on the first d_v columns).  A
 * non-latent call needs d_v != d_k.  The additions are fp32 atomics, so the order of the
 * partial sums (and the last bits) can differ between runs.
 *   shape, attn, budget, q, k, v, idx   as for lsa_sparse_attn (budget: k entries per row)
 *   budget.sink / budget.window, shape->q_pos0: the Streaming-Aware layout the lists were
 *           selected with (lsa_topk_select: entries [0, S) the sink rows 0..S-1, entries
 *           [S, S+W) the window rows V_i-W .. V_i-1, V_i = min(kv_len, q_pos0 + i + 1)).  Where
 *           an entry holds the row its position names and the query's sink and window are
 *           disjoint, its cache-gradient share is summed over the queries that share the row
 *           before it is added (one update per row column for many queries: the prefill
 *           chunks' sink and window rows); every other entry is added as described above.  The
 *           sum is the same, in another order.  Uniform batches only (no seq_len / seq_pos0);
 *           sink = window = 0 adds every entry per query.
 *   out     [B, n_q, Hq, d_v] bf16, 16-byte aligned;  lse  [B, n_q, Hq] fp32 (required)
 *   d_out   [B, n_q, Hq, d_v] bf16, 16-byte aligned
 *   d_q     [B, n_q, Hq, d_qk] fp32
 *   d_k     [B, L, d_qk] fp32 (dense rows);  d_v  [B, L, d_v] fp32 (latent: == d_k)
 * Limits: as lsa_sparse_attn, with dense caches only (attn->block_table must be NULL, else
 *         LSA_ERR_UNSUPPORTED).  No workspace.
 */
LSA_API lsa_status lsa_sparse_attn_backward(const lsa_index_shape *shape, const lsa_attn_shape *attn,
                                            lsa_budget budget, const void *q, const void *k,
                                            const void *v, const int32_t *idx, const void *out,
                                            const float *lse, const void *d_out, float *d_q,
                                            float *d_k, float *d_v, void *stream);

/*
 * lsa_index_scores_backward -- gradients of the indexer scores at the selected entries (the
 * training path of the Lightning Indexer, Baidu Cloud article, "1. Lightweight Scoring
 * Module").  Given d_scores[b,t,j], the gradient of the score of query t at its entry
 * s_j = idx[b,t,j] (entries outside [0, V_t) carry none), with ReLU'(0) = 0 and
 * G_jh = d_scores[b,t,j] w[b,t,h] [q[b,t,h] . keys[b,s_j] > 0]:
 *     d_w[b,t,h]      += sum_j d_scores[b,t,j] ReLU(q[b,t,h] . keys[b,s_j])
 *     d_q[b,t,h,:]    += sum_j G_jh keys[b,s_j,:]
 *     d_keys[b,s_j,:] += sum_h G_jh q[b,t,h,:]
 * (the dot products in fp32 from the bf16 inputs).  bf16 keys only: the 8-bit key format is an
 * inference-side encoding.  The gradients are ADDED into (fp32; zero them first), with fp32
 * atomics (summation order, and the last bits, can differ between runs).
 *   shape     as for lsa_index_scores (n_heads H <= 64, head_dim 64 or 128, ragged arrays allowed)
 *   budget    k = entries per idx row.  sink / window with shape->q_pos0: the Streaming-Aware
 *             layout the lists were selected with, as for lsa_sparse_attn_backward.  Where an
 *             entry holds the row its position names and the query's sink and window are
 *             disjoint, its d_keys share is summed over the queries that share the row before it
 *             is added (uniform batches, head_dim 128); every other entry is added per query.
 *             The sum is the same, in another order.  sink = window = 0 adds every entry per
 *             query.  Checked: 0 <= sink, 0 <= window, sink + window <= k.
 *   q [B, n_q, H, d] bf16, 16-byte aligned;  w [B, n_q, H] fp32;  keys [B, L, d] bf16, 16-byte aligned
 *   idx [B, n_q, k] int32;  d_scores [B, n_q, k] fp32
 *   d_q [B, n_q, H, d] fp32;  d_w [B, n_q, H] fp32;  d_keys [B, L, d] fp32
 */
LSA_API lsa_status lsa_index_scores_backward(const lsa_index_shape *shape, lsa_budget budget,
                                             const void *q, const float *w, const void *keys,
                                             const int32_t *idx, const float *d_scores, float *d_q,
                                             float *d_w, float *d_keys, void *stream);

enum { LSA_OP_TOPK_SELECT = 1, LSA_OP_PAGE_RECALL = 2, LSA_OP_SPARSE_ATTN = 3,
       LSA_OP_INDEX_SELECT = 4 };

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
