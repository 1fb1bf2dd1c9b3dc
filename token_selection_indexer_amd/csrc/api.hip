// api.hip -- the C ABI of include/lsa.h: argument validation, workspace sizing and kernel
// dispatch on the caller's stream.  Every check runs on the host before anything is enqueued.
#include "lsa.h"

#include <hip/hip_runtime.h>

#include "internal.hpp"

namespace {

constexpr int64_t kMaxGridYZ = 65535;

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

lsa_status check_index_shape(const lsa_index_shape *s)
{
    if (!s) return LSA_ERR_NULL_POINTER;
    if (s->batch < 0 || s->n_q < 0 || s->kv_len < 1 || s->kv_len >= (int64_t(1) << 31) ||
        s->q_pos0 < 0 || s->batch > kMaxGridYZ)
        return LSA_ERR_BAD_SHAPE;
    if (s->n_heads < 1 || s->head_dim < 1) return LSA_ERR_BAD_SHAPE;
    if (!lsa::scores_supported(s->n_heads, s->head_dim)) return LSA_ERR_UNSUPPORTED;
    return LSA_OK;
}

lsa_status check_keys(lsa_key_dtype kd, const void *keys, const float *scale)
{
    if (kd != LSA_KEY_BF16 && kd != LSA_KEY_FP8_E4M3) return LSA_ERR_BAD_DTYPE;
    if (!keys) return LSA_ERR_NULL_POINTER;
    if (kd == LSA_KEY_FP8_E4M3 && !scale) return LSA_ERR_BAD_DTYPE;
    if (kd == LSA_KEY_BF16 && scale) return LSA_ERR_BAD_DTYPE;
    if (!aligned(keys, 16) || (scale && !aligned(scale, 4))) return LSA_ERR_BAD_SHAPE;
    return LSA_OK;
}

lsa_status check_budget(lsa_budget b)
{
    if (b.k < 1 || b.sink < 0 || b.window < 0 || (int64_t)b.sink + b.window > b.k)
        return LSA_ERR_BAD_SHAPE;
    return LSA_OK;
}

lsa_status device_status(hipError_t e) { return e == hipSuccess ? LSA_OK : LSA_ERR_DEVICE; }

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

size_t recall_ws(const lsa_index_shape *s, int32_t page_size)
{
    const int64_t n_pages = (s->kv_len + page_size - 1) / page_size;
    return round256((size_t)s->batch * s->n_q * n_pages * sizeof(float));
}

lsa_status check_attn(const lsa_index_shape *s, const lsa_attn_shape *a, lsa_budget b)
{
    if (!s || !a) return LSA_ERR_NULL_POINTER;
    if (s->batch < 0 || s->n_q < 0 || s->kv_len < 1 || s->kv_len >= (int64_t(1) << 31) ||
        s->batch > kMaxGridYZ)
        return LSA_ERR_BAD_SHAPE;
    if (b.k < 1) return LSA_ERR_BAD_SHAPE;
    if (a->n_heads < 1 || a->d_qk < 1 || a->d_v < 1 || !(a->scale == a->scale))
        return LSA_ERR_BAD_SHAPE;
    if (a->k_row_stride < a->d_qk || a->v_row_stride < a->d_v || a->k_row_stride % 8 ||
        a->v_row_stride % 8)
        return LSA_ERR_BAD_SHAPE;
    if (a->latent != 0 && a->latent != 1) return LSA_ERR_BAD_SHAPE;
    if (a->latent && a->k_row_stride != a->v_row_stride) return LSA_ERR_BAD_SHAPE;
    if (!lsa::attn_supported(a->n_heads, a->d_qk, a->d_v, a->latent)) return LSA_ERR_UNSUPPORTED;
    if (a->latent && (int64_t)s->n_q * (a->n_heads / 16) > kMaxGridYZ) return LSA_ERR_UNSUPPORTED;
    return LSA_OK;
}

} // namespace

extern "C" {

const char *lsa_status_string(lsa_status st)
{
    switch (st) {
    case LSA_OK: return "LSA_OK";
    case LSA_ERR_NULL_POINTER: return "LSA_ERR_NULL_POINTER";
    case LSA_ERR_BAD_SHAPE: return "LSA_ERR_BAD_SHAPE";
    case LSA_ERR_BAD_DTYPE: return "LSA_ERR_BAD_DTYPE";
    case LSA_ERR_UNSUPPORTED: return "LSA_ERR_UNSUPPORTED";
    case LSA_ERR_WORKSPACE_TOO_SMALL: return "LSA_ERR_WORKSPACE_TOO_SMALL";
    case LSA_ERR_DEVICE: return "LSA_ERR_DEVICE";
    }
    return "LSA_ERR_UNKNOWN";
}

size_t lsa_workspace_bytes(int op, const lsa_index_shape *shape, lsa_budget budget,
                           int32_t page_size, int32_t m_pages, int64_t n_cand,
                           const lsa_attn_shape *attn)
{
    (void)n_cand;
    switch (op) {
    case LSA_OP_TOPK_SELECT: {
        if (!shape || shape->batch < 0 || shape->n_q < 0 || shape->kv_len < 1 ||
            check_budget(budget) != LSA_OK || n_cand < 0)
            return (size_t)-1;
        const int64_t n = n_cand == 0 ? shape->kv_len : n_cand;
        return lsa::select_workspace_bytes((int64_t)shape->batch * shape->n_q, n, lsa::SELECT_SI);
    }
    case LSA_OP_PAGE_RECALL:
        if (check_index_shape(shape) != LSA_OK || !pow2(page_size) || page_size < 32 ||
            page_size > 256 || m_pages < 1)
            return (size_t)-1;
        return recall_ws(shape, page_size);
    case LSA_OP_SPARSE_ATTN:
        if (check_attn(shape, attn, budget) != LSA_OK) return (size_t)-1;
        return round256(lsa::attn_workspace_bytes(shape->batch, shape->n_q, attn->n_heads, attn->d_v,
                                                  budget.k, attn->latent));
    default: return (size_t)-1;
    }
}

lsa_status lsa_index_scores(const lsa_index_shape *shape, const void *q, const float *w,
                            const void *keys, lsa_key_dtype key_dtype, const float *key_scale,
                            float *scores, void *stream)
{
    lsa_status st = check_index_shape(shape);
    if (st != LSA_OK) return st;
    if ((st = check_keys(key_dtype, keys, key_scale)) != LSA_OK) return st;
    if (!q || !w || !scores) return LSA_ERR_NULL_POINTER;
    if (!aligned(q, 16) || !aligned(w, 4) || !aligned(scores, 4)) return LSA_ERR_BAD_SHAPE;
    if (shape->n_q > kMaxGridYZ * 64) return LSA_ERR_UNSUPPORTED;
    if ((int64_t)shape->batch * shape->n_q == 0) return LSA_OK;
    lsa::ScoreArgs a{};
    a.q = static_cast<const uint16_t *>(q);
    a.w = w;
    a.keys = keys;
    a.kscale = key_scale;
    a.out = scores;
    a.batch = shape->batch;
    a.n_q = shape->n_q;
    a.heads = shape->n_heads;
    a.dim = shape->head_dim;
    a.n_keys = shape->kv_len;
    a.n_out = shape->kv_len;
    a.kv_len = shape->kv_len;
    a.q_pos0 = shape->q_pos0;
    a.mask = lsa::MASK_CAUSAL;
    a.fp8 = key_dtype == LSA_KEY_FP8_E4M3;
    return device_status(lsa::launch_scores(a, static_cast<hipStream_t>(stream)));
}

lsa_status lsa_topk_select(const lsa_index_shape *shape, lsa_budget budget, const float *scores,
                           int64_t n_cand, const int32_t *cand_ids, int32_t *idx, void *ws,
                           size_t ws_bytes, void *stream)
{
    if (!shape) return LSA_ERR_NULL_POINTER;
    if (shape->batch < 0 || shape->n_q < 0 || shape->kv_len < 1 ||
        shape->kv_len >= (int64_t(1) << 31) || shape->q_pos0 < 0)
        return LSA_ERR_BAD_SHAPE;
    lsa_status st = check_budget(budget);
    if (st != LSA_OK) return st;
    if (budget.k - budget.sink - budget.window > 65536) return LSA_ERR_UNSUPPORTED;
    if (!scores || !idx) return LSA_ERR_NULL_POINTER;
    if (!cand_ids && n_cand != shape->kv_len) return LSA_ERR_BAD_SHAPE;
    if (cand_ids && (n_cand < 1 || n_cand >= (int64_t(1) << 31))) return LSA_ERR_BAD_SHAPE;
    if (!aligned(scores, 16) || (cand_ids && !aligned(cand_ids, 16)) || !aligned(idx, 4))
        return LSA_ERR_BAD_SHAPE;
    const int64_t rows = (int64_t)shape->batch * shape->n_q;
    if (rows >= (int64_t(1) << 31)) return LSA_ERR_UNSUPPORTED;
    if (rows == 0) return LSA_OK;
    const size_t need = lsa::select_workspace_bytes(rows, n_cand, lsa::SELECT_SI);
    if (need && (!ws || ws_bytes < need || !aligned(ws, 256))) return LSA_ERR_WORKSPACE_TOO_SMALL;
    lsa::SelectArgs a{};
    a.scores = scores;
    a.cand_ids = cand_ids;
    a.out = idx;
    a.batch = shape->batch;
    a.n_q = shape->n_q;
    a.n_in = n_cand;
    a.kv_len = shape->kv_len;
    a.q_pos0 = shape->q_pos0;
    a.k = budget.k;
    a.sink = budget.sink;
    a.window = budget.window;
    a.mode = lsa::SELECT_SI;
    a.out_stride = budget.k;
    return device_status(lsa::launch_select(a, ws, static_cast<hipStream_t>(stream)));
}

lsa_status lsa_page_summary(const lsa_index_shape *shape, int32_t page_size, const void *keys,
                            lsa_key_dtype key_dtype, const float *key_scale, int64_t page_lo,
                            int64_t page_hi, void *page_keys, void *stream)
{
    if (!shape) return LSA_ERR_NULL_POINTER;
    if (shape->batch < 0 || shape->kv_len < 1 || shape->kv_len >= (int64_t(1) << 31) ||
        shape->batch > kMaxGridYZ)
        return LSA_ERR_BAD_SHAPE;
    if (shape->head_dim != 64 && shape->head_dim != 128) return LSA_ERR_UNSUPPORTED;
    if (!pow2(page_size) || page_size > 256) return LSA_ERR_BAD_SHAPE;
    lsa_status st = check_keys(key_dtype, keys, key_scale);
    if (st != LSA_OK) return st;
    if (!page_keys) return LSA_ERR_NULL_POINTER;
    if (!aligned(page_keys, 4)) return LSA_ERR_BAD_SHAPE;
    const int64_t n_pages = (shape->kv_len + page_size - 1) / page_size;
    if (page_lo < 0 || page_hi < page_lo || page_hi > n_pages) return LSA_ERR_BAD_SHAPE;
    if (shape->batch == 0 || page_hi == page_lo) return LSA_OK;
    return device_status(lsa::launch_page_summary(keys, key_dtype == LSA_KEY_FP8_E4M3, key_scale,
                                                  shape->batch, shape->kv_len, shape->head_dim,
                                                  page_size, page_lo, page_hi,
                                                  static_cast<uint16_t *>(page_keys),
                                                  static_cast<hipStream_t>(stream)));
}

lsa_status lsa_page_recall(const lsa_index_shape *shape, lsa_budget budget, int32_t page_size,
                           int32_t m_pages, const void *q, const float *w, const void *page_keys,
                           const void *keys, lsa_key_dtype key_dtype, const float *key_scale,
                           int32_t *page_ids, float *cand_scores, int32_t *cand_ids, void *ws,
                           size_t ws_bytes, void *stream)
{
    lsa_status st = check_index_shape(shape);
    if (st != LSA_OK) return st;
    if ((st = check_budget(budget)) != LSA_OK) return st;
    if (!pow2(page_size) || page_size < 32 || page_size > 256) return LSA_ERR_BAD_SHAPE;
    if (m_pages < 1 || m_pages > 65536) return LSA_ERR_BAD_SHAPE;
    if ((st = check_keys(key_dtype, keys, key_scale)) != LSA_OK) return st;
    if (!q || !w || !page_keys || !page_ids || !cand_scores || !cand_ids) return LSA_ERR_NULL_POINTER;
    if (!aligned(q, 16) || !aligned(page_keys, 16) || !aligned(w, 4) || !aligned(page_ids, 4) ||
        !aligned(cand_scores, 4) || !aligned(cand_ids, 4))
        return LSA_ERR_BAD_SHAPE;
    const int64_t rows = (int64_t)shape->batch * shape->n_q;
    if (rows >= (int64_t(1) << 31) || shape->n_q > kMaxGridYZ) return LSA_ERR_UNSUPPORTED;
    const size_t need = recall_ws(shape, page_size);
    if (rows == 0) return LSA_OK;
    if (!ws || ws_bytes < need) return LSA_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned(ws, 256)) return LSA_ERR_WORKSPACE_TOO_SMALL;

    const hipStream_t sm = static_cast<hipStream_t>(stream);
    const int64_t n_pages = (shape->kv_len + page_size - 1) / page_size;
    float *coarse = static_cast<float *>(ws);

    // stage 1a: coarse scores of the eligible pages
    lsa::ScoreArgs c{};
    c.q = static_cast<const uint16_t *>(q);
    c.w = w;
    c.keys = page_keys;
    c.kscale = nullptr;
    c.out = coarse;
    c.batch = shape->batch;
    c.n_q = shape->n_q;
    c.heads = shape->n_heads;
    c.dim = shape->head_dim;
    c.n_keys = n_pages;
    c.n_out = n_pages;
    c.kv_len = shape->kv_len;
    c.q_pos0 = shape->q_pos0;
    c.mask = lsa::MASK_PAGES;
    c.k = budget.k;
    c.sink = budget.sink;
    c.window = budget.window;
    c.page = page_size;
    c.fp8 = 0;
    if ((st = device_status(lsa::launch_scores(c, sm))) != LSA_OK) return st;

    // stage 1b: recall the best m_pages pages
    lsa::SelectArgs s{};
    s.scores = coarse;
    s.cand_ids = nullptr;
    s.out = page_ids;
    s.batch = shape->batch;
    s.n_q = shape->n_q;
    s.n_in = n_pages;
    s.kv_len = shape->kv_len;
    s.q_pos0 = shape->q_pos0;
    s.k = budget.k;
    s.sink = budget.sink;
    s.window = budget.window;
    s.mode = lsa::SELECT_PAGES;
    s.page = page_size;
    s.m_pages = m_pages;
    s.out_stride = m_pages;
    if ((st = device_status(lsa::launch_select(s, nullptr, sm))) != LSA_OK) return st;

    // stage 2: fine scores of the tokens of the recalled pages
    lsa::ScoreArgs f{};
    f.q = static_cast<const uint16_t *>(q);
    f.w = w;
    f.keys = keys;
    f.kscale = key_scale;
    f.out = cand_scores;
    f.out_ids = cand_ids;
    f.pages = page_ids;
    f.batch = shape->batch;
    f.n_q = shape->n_q;
    f.heads = shape->n_heads;
    f.dim = shape->head_dim;
    f.n_keys = shape->kv_len;
    f.n_out = (int64_t)m_pages * page_size;
    f.kv_len = shape->kv_len;
    f.q_pos0 = shape->q_pos0;
    f.k = budget.k;
    f.sink = budget.sink;
    f.window = budget.window;
    f.page = page_size;
    f.m_pages = m_pages;
    f.fp8 = key_dtype == LSA_KEY_FP8_E4M3;
    return device_status(lsa::launch_fine_scores(f, sm));
}

lsa_status lsa_sparse_attn(const lsa_index_shape *shape, const lsa_attn_shape *attn,
                           lsa_budget budget, const void *q, const void *k, const void *v,
                           const int32_t *idx, void *out, float *lse, void *ws, size_t ws_bytes,
                           void *stream)
{
    lsa_status st = check_attn(shape, attn, budget);
    if (st != LSA_OK) return st;
    if (!q || !k || !v || !idx || !out) return LSA_ERR_NULL_POINTER;
    if (attn->latent && v != k) return LSA_ERR_BAD_SHAPE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(idx, 4) ||
        !aligned(out, 4) || (lse && !aligned(lse, 4)))
        return LSA_ERR_BAD_SHAPE;
    if (budget.sink < 0 || budget.window < 0 || (int64_t)budget.sink + budget.window > budget.k)
        return LSA_ERR_BAD_SHAPE;
    const int64_t rows = (int64_t)shape->batch * shape->n_q;
    if (rows == 0) return LSA_OK;
    if (rows * attn->n_heads >= (int64_t(1) << 31) * 4) return LSA_ERR_UNSUPPORTED;
    const size_t need = round256(lsa::attn_workspace_bytes(shape->batch, shape->n_q, attn->n_heads,
                                                           attn->d_v, budget.k, attn->latent));
    if (need && (!ws || ws_bytes < need || !aligned(ws, 256))) return LSA_ERR_WORKSPACE_TOO_SMALL;
    lsa::AttnArgs a{};
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.idx = idx;
    a.out = static_cast<uint16_t *>(out);
    a.lse = lse;
    a.ws = static_cast<float *>(ws);
    a.batch = shape->batch;
    a.n_q = shape->n_q;
    a.heads = attn->n_heads;
    a.d_qk = attn->d_qk;
    a.d_v = attn->d_v;
    a.n_idx = budget.k;
    a.latent = attn->latent;
    a.kv_len = shape->kv_len;
    a.k_stride = attn->k_row_stride;
    a.v_stride = attn->v_row_stride;
    a.sink = budget.sink;
    a.window = budget.window;
    a.scale = attn->scale;
    a.n_split = lsa::attn_splits(shape->batch, shape->n_q, attn->n_heads, budget.k, attn->latent);
    return device_status(lsa::launch_sparse_attn(a, static_cast<hipStream_t>(stream)));
}

} // extern "C"
