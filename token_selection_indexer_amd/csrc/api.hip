// api.hip -- the C ABI of include/lsa.h: argument validation, workspace sizing and kernel
// dispatch on the caller's stream.  Every check runs on the host before anything is enqueued.
#include "lsa.h"

#include <hip/hip_runtime.h>

#include <algorithm>

#include "internal.hpp"

namespace {

constexpr int64_t kMaxGridYZ = 65535;

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

bool ragged(const lsa_index_shape *s) { return s->seq_len || s->seq_pos0; }

lsa_status check_ragged(const lsa_index_shape *s)
{
    if (!aligned(s->seq_len, 4) || !aligned(s->seq_pos0, 4)) return LSA_ERR_BAD_SHAPE;
    return LSA_OK;
}

lsa_status check_index_shape(const lsa_index_shape *s)
{
    if (!s) return LSA_ERR_NULL_POINTER;
    if (s->batch < 0 || s->n_q < 0 || s->kv_len < 1 || s->kv_len >= (int64_t(1) << 31) ||
        s->q_pos0 < 0 || s->batch > kMaxGridYZ)
        return LSA_ERR_BAD_SHAPE;
    if (s->n_heads < 1 || s->head_dim < 1) return LSA_ERR_BAD_SHAPE;
    if (!lsa::scores_supported(s->n_heads, s->head_dim)) return LSA_ERR_UNSUPPORTED;
    if (s->block_table) { // paged indexer keys
        const int64_t bs = s->block_size;
        if (!pow2(bs) || bs < 32 || bs > (1 << 20) || s->blocks_per_seq < 1 || s->n_blocks < 1 ||
            (int64_t)s->blocks_per_seq * bs < s->kv_len || s->n_blocks * bs >= (int64_t(1) << 31) ||
            !aligned(s->block_table, 4))
            return LSA_ERR_BAD_SHAPE;
    }
    return check_ragged(s);
}

// The indexer-key calls that take dense keys only.
lsa_status dense_keys_only(const lsa_index_shape *s)
{
    return s && s->block_table ? LSA_ERR_UNSUPPORTED : LSA_OK;
}

// The block table of paged indexer keys (shape checked), for pages of page_size keys: a page
// must lie inside one table block.  LSA_ERR_UNSUPPORTED otherwise.
lsa_status paged_pages(const lsa_index_shape *s, int32_t page_size, lsa::PagedTab &pt)
{
    pt = lsa::PagedTab{};
    if (!s->block_table) return LSA_OK;
    if (page_size < 32 || page_size > s->block_size) return LSA_ERR_UNSUPPORTED;
    while ((int64_t(1) << pt.lbs) < s->block_size) ++pt.lbs;
    pt.btab = s->block_table;
    pt.bps = s->blocks_per_seq;
    pt.n_blocks = s->n_blocks;
    return LSA_OK;
}

// Paged indexer keys (shape checked): the table fields of the scoring arguments, and whether
// the scoring launch that `a` asks for takes them.
lsa_status set_paged_keys(const lsa_index_shape *s, lsa::ScoreArgs &a)
{
    if (!s->block_table) return LSA_OK;
    int lbs = 0;
    while ((int64_t(1) << lbs) < s->block_size) ++lbs;
    a.btab = s->block_table;
    a.lbs = lbs;
    a.bps = s->blocks_per_seq;
    a.n_blocks = s->n_blocks;
    return lsa::scores_paged_ok(a) ? LSA_OK : LSA_ERR_UNSUPPORTED;
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

// The fused score + select plan for a shape: histogram groups per row (0: not fused) and the
// workspace layout.  With slices (each scoring workgroup owns at most kSliceSpan keys and the
// selection has a wave per scoring workgroup of the row): histograms, slice headers and entries,
// and one selection launch.  Else histograms, then the chunked selection's workspace.
struct FusedPlan {
    int groups = 0;
    bool slices = false;
    size_t hist_fine = 0, hist_coarse = 0, slice_hdr = 0, slice_ent = 0, select = 0, total = 0;
};

lsa::ScoreArgs score_args(const lsa_index_shape *shape, lsa_budget budget)
{
    lsa::ScoreArgs a{};
    a.batch = shape->batch;
    a.n_q = shape->n_q;
    a.heads = shape->n_heads;
    a.dim = shape->head_dim;
    a.n_keys = shape->kv_len;
    a.n_out = shape->kv_len;
    a.kv_len = shape->kv_len;
    a.q_pos0 = shape->q_pos0;
    a.seq_len = shape->seq_len;
    a.seq_pos0 = shape->seq_pos0;
    a.mask = lsa::MASK_CAUSAL;
    a.k = budget.k;
    a.sink = budget.sink;
    a.window = budget.window;
    return a;
}

lsa::SelectArgs select_args(const lsa_index_shape *shape, lsa_budget budget)
{
    lsa::SelectArgs a{};
    a.batch = shape->batch;
    a.n_q = shape->n_q;
    a.n_in = shape->kv_len;
    a.kv_len = shape->kv_len;
    a.q_pos0 = shape->q_pos0;
    a.seq_len = shape->seq_len;
    a.seq_pos0 = shape->seq_pos0;
    a.k = budget.k;
    a.sink = budget.sink;
    a.window = budget.window;
    a.mode = lsa::SELECT_SI;
    a.out_stride = budget.k;
    return a;
}

FusedPlan fused_plan(const lsa_index_shape *shape, lsa_budget budget)
{
    FusedPlan p;
    const int64_t rows = (int64_t)shape->batch * shape->n_q;
    p.select = lsa::select_workspace_bytes(rows, shape->kv_len, lsa::SELECT_SI);
    p.total = p.select;
    // fused only where the selection alone would take its chunked path (few long rows)
    if (rows == 0 || p.select == 0) return p;
    const lsa::ScoreArgs sa = score_args(shape, budget);
    const int groups = lsa::score_hist_groups(sa);
    if (groups == 0) return p;
    p.groups = groups;
    p.hist_fine = round256((size_t)rows * groups * 2048 * 4);
    p.hist_coarse = round256((size_t)rows * groups * 32 * 4);
    p.slices = groups <= lsa::select_slice_groups_max() &&
               lsa::score_hist_span(sa, groups) <= lsa::kSliceSpan;
    if (p.slices) {
        p.select = 0;
        p.slice_hdr = round256((size_t)rows * groups * 16);
        p.slice_ent = round256((size_t)rows * groups * lsa::kSliceCap * 8);
    }
    p.total = p.hist_fine + p.hist_coarse + p.slice_hdr + p.slice_ent + p.select;
    return p;
}

size_t index_select_ws(const lsa_index_shape *shape, lsa_budget budget)
{
    return fused_plan(shape, budget).total;
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
    case LSA_OP_INDEX_SELECT: {
        if (check_index_shape(shape) != LSA_OK || check_budget(budget) != LSA_OK)
            return (size_t)-1;
        return index_select_ws(shape, budget);
    }
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
    a.seq_len = shape->seq_len;
    a.seq_pos0 = shape->seq_pos0;
    a.mask = lsa::MASK_CAUSAL;
    a.fp8 = key_dtype == LSA_KEY_FP8_E4M3;
    if ((st = set_paged_keys(shape, a)) != LSA_OK) return st;
    return device_status(lsa::launch_scores(a, static_cast<hipStream_t>(stream)));
}

namespace {

// Validation and argument block shared by the two selection entry points.
lsa_status prepare_select(const lsa_index_shape *shape, lsa_budget budget, const float *scores,
                          int64_t n_cand, const int32_t *cand_ids, int32_t *idx,
                          lsa::SelectArgs &a, int64_t &rows)
{
    if (!shape) return LSA_ERR_NULL_POINTER;
    if (shape->batch < 0 || shape->n_q < 0 || shape->kv_len < 1 ||
        shape->kv_len >= (int64_t(1) << 31) || shape->q_pos0 < 0)
        return LSA_ERR_BAD_SHAPE;
    lsa_status st = check_budget(budget);
    if (st != LSA_OK) return st;
    if ((st = check_ragged(shape)) != LSA_OK) return st;
    if (budget.k - budget.sink - budget.window > 65536) return LSA_ERR_UNSUPPORTED;
    if (!scores || !idx) return LSA_ERR_NULL_POINTER;
    if (!cand_ids && n_cand != shape->kv_len) return LSA_ERR_BAD_SHAPE;
    if (cand_ids && (n_cand < 1 || n_cand >= (int64_t(1) << 31))) return LSA_ERR_BAD_SHAPE;
    if (!aligned(scores, 16) || (cand_ids && !aligned(cand_ids, 16)) || !aligned(idx, 4))
        return LSA_ERR_BAD_SHAPE;
    rows = (int64_t)shape->batch * shape->n_q;
    if (rows >= (int64_t(1) << 31)) return LSA_ERR_UNSUPPORTED;
    a = lsa::SelectArgs{};
    a.scores = scores;
    a.cand_ids = cand_ids;
    a.out = idx;
    a.batch = shape->batch;
    a.n_q = shape->n_q;
    a.n_in = n_cand;
    a.kv_len = shape->kv_len;
    a.q_pos0 = shape->q_pos0;
    a.seq_len = shape->seq_len;
    a.seq_pos0 = shape->seq_pos0;
    a.k = budget.k;
    a.sink = budget.sink;
    a.window = budget.window;
    a.mode = lsa::SELECT_SI;
    a.out_stride = budget.k;
    return LSA_OK;
}

} // namespace

lsa_status lsa_quantize_queries(const lsa_index_shape *shape, const void *q, uint8_t *q8,
                                float *q_scale, void *stream)
{
    if (!shape) return LSA_ERR_NULL_POINTER;
    if (shape->batch < 0 || shape->n_q < 0 || shape->n_heads < 1) return LSA_ERR_BAD_SHAPE;
    if (shape->head_dim != 64 && shape->head_dim != 128) return LSA_ERR_UNSUPPORTED;
    if (!q || !q8 || !q_scale) return LSA_ERR_NULL_POINTER;
    if (!aligned(q, 4) || !aligned(q8, 2) || !aligned(q_scale, 4)) return LSA_ERR_BAD_SHAPE;
    const int64_t rows = (int64_t)shape->batch * shape->n_q * shape->n_heads;
    if (rows == 0) return LSA_OK;
    if ((rows + 3) / 4 >= (int64_t(1) << 31)) return LSA_ERR_UNSUPPORTED;
    return device_status(lsa::launch_quantize_rows(static_cast<const uint16_t *>(q), rows,
                                                   shape->head_dim, q8, q_scale,
                                                   static_cast<hipStream_t>(stream)));
}

lsa_status lsa_index_scores_q8(const lsa_index_shape *shape, const uint8_t *q8,
                               const float *q_scale, const float *w, const void *keys,
                               lsa_key_dtype key_dtype, const float *key_scale, float *scores,
                               void *stream)
{
    lsa_status st = check_index_shape(shape);
    if (st != LSA_OK) return st;
    if ((st = dense_keys_only(shape)) != LSA_OK) return st;
    if ((st = check_keys(key_dtype, keys, key_scale)) != LSA_OK) return st;
    if (key_dtype != LSA_KEY_FP8_E4M3) return LSA_ERR_BAD_DTYPE; // 8-bit x 8-bit products
    if (!q8 || !q_scale || !w || !scores) return LSA_ERR_NULL_POINTER;
    if (!aligned(q8, 16) || !aligned(q_scale, 4) || !aligned(w, 4) || !aligned(scores, 4))
        return LSA_ERR_BAD_SHAPE;
    if ((int64_t)shape->n_q > kMaxGridYZ * 8) return LSA_ERR_UNSUPPORTED;
    if ((int64_t)shape->batch * shape->n_q == 0) return LSA_OK;
    lsa::ScoreArgs a{};
    a.q8 = q8;
    a.q_scale = q_scale;
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
    a.seq_len = shape->seq_len;
    a.seq_pos0 = shape->seq_pos0;
    a.mask = lsa::MASK_CAUSAL;
    a.fp8 = 1;
    return device_status(lsa::launch_scores(a, static_cast<hipStream_t>(stream)));
}

lsa_status lsa_index_select(const lsa_index_shape *shape, lsa_budget budget, const void *q,
                            const float *w, const void *keys, lsa_key_dtype key_dtype,
                            const float *key_scale, float *scores, int32_t *idx, void *ws,
                            size_t ws_bytes, void *stream)
{
    lsa_status st = check_index_shape(shape);
    if (st != LSA_OK) return st;
    if ((st = check_budget(budget)) != LSA_OK) return st;
    if (budget.k - budget.sink - budget.window > 65536) return LSA_ERR_UNSUPPORTED;
    if ((st = check_keys(key_dtype, keys, key_scale)) != LSA_OK) return st;
    if (!q || !w || !scores || !idx) return LSA_ERR_NULL_POINTER;
    if (!aligned(q, 16) || !aligned(w, 4) || !aligned(scores, 16) || !aligned(idx, 4))
        return LSA_ERR_BAD_SHAPE;
    if (shape->n_q > kMaxGridYZ * 64) return LSA_ERR_UNSUPPORTED;
    const int64_t rows = (int64_t)shape->batch * shape->n_q;
    if (rows >= (int64_t(1) << 31)) return LSA_ERR_UNSUPPORTED;
    if (rows == 0) return LSA_OK;
    const size_t need = index_select_ws(shape, budget);
    if (need && (!ws || ws_bytes < need || !aligned(ws, 256))) return LSA_ERR_WORKSPACE_TOO_SMALL;
    const hipStream_t sm = static_cast<hipStream_t>(stream);
    lsa::ScoreArgs a = score_args(shape, budget);
    a.q = static_cast<const uint16_t *>(q);
    a.w = w;
    a.keys = keys;
    a.kscale = key_scale;
    a.out = scores;
    a.fp8 = key_dtype == LSA_KEY_FP8_E4M3;
    if ((st = set_paged_keys(shape, a)) != LSA_OK) return st;
    lsa::SelectArgs s = select_args(shape, budget);
    s.scores = scores;
    s.out = idx;
    const FusedPlan p = fused_plan(shape, budget);
    if (!p.groups) { // not the decode shape: the two ordinary paths
        if ((st = device_status(lsa::launch_scores(a, sm))) != LSA_OK) return st;
        return device_status(lsa::launch_select(s, ws, sm));
    }
    uint8_t *base = static_cast<uint8_t *>(ws);
    a.hist_fine = reinterpret_cast<uint32_t *>(base);
    base += p.hist_fine;
    a.hist_coarse = reinterpret_cast<uint32_t *>(base);
    base += p.hist_coarse;
    if (!p.slices) {
        if ((st = device_status(lsa::launch_scores(a, sm))) != LSA_OK) return st;
        return device_status(
            lsa::launch_select_hist(s, base, a.hist_fine, a.hist_coarse, p.groups, sm));
    }
    a.slice_hdr = reinterpret_cast<int4 *>(base);
    a.slice_ent = reinterpret_cast<uint2 *>(base + p.slice_hdr);
    // a slice keeps the bins holding about twice its workgroup's expected share of the row's
    // `need` best: enough that the slices' keys at or above their highest bin almost always
    // number at least `need`, few enough to keep the selection's buffer small
    const int need_dyn = budget.k - budget.sink - budget.window;
    const int share = (need_dyn + p.groups - 1) / p.groups;
    a.slice_target = std::max(1, std::min({need_dyn, 2 * share + 32, lsa::kSliceCap}));
    if ((st = device_status(lsa::launch_scores(a, sm))) != LSA_OK) return st;
    return device_status(lsa::launch_select_slices(s, a.hist_fine, a.hist_coarse, a.slice_hdr,
                                                   a.slice_ent, p.groups, sm));
}

lsa_status lsa_topk_select(const lsa_index_shape *shape, lsa_budget budget, const float *scores,
                           int64_t n_cand, const int32_t *cand_ids, int32_t *idx, void *ws,
                           size_t ws_bytes, void *stream)
{
    lsa::SelectArgs a;
    int64_t rows = 0;
    lsa_status st = prepare_select(shape, budget, scores, n_cand, cand_ids, idx, a, rows);
    if (st != LSA_OK) return st;
    if (rows == 0) return LSA_OK;
    const size_t need = lsa::select_workspace_bytes(rows, n_cand, lsa::SELECT_SI);
    if (need && (!ws || ws_bytes < need || !aligned(ws, 256))) return LSA_ERR_WORKSPACE_TOO_SMALL;
    return device_status(lsa::launch_select(a, ws, static_cast<hipStream_t>(stream)));
}

lsa_status lsa_topk_select_noalloc(const lsa_index_shape *shape, lsa_budget budget,
                                   const float *scores, int64_t n_cand, const int32_t *cand_ids,
                                   int32_t *idx, void *stream)
{
    lsa::SelectArgs a;
    int64_t rows = 0;
    lsa_status st = prepare_select(shape, budget, scores, n_cand, cand_ids, idx, a, rows);
    if (st != LSA_OK) return st;
    if (rows == 0) return LSA_OK;
    const size_t need = lsa::select_workspace_bytes(rows, n_cand, lsa::SELECT_SI);
    if (need > lsa::select_scratch_bytes()) return LSA_ERR_UNSUPPORTED;
    void *ws = nullptr;
    if (need && lsa::select_scratch(&ws) != hipSuccess) return LSA_ERR_DEVICE;
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
    lsa::PagedTab pt;
    if (shape->block_table) { // paged keys: the table checks of the scoring calls
        lsa_index_shape chk = *shape;
        chk.n_q = 1;
        chk.n_heads = 64;
        chk.q_pos0 = 0;
        const lsa_status sc = check_index_shape(&chk);
        if (sc != LSA_OK) return sc;
        if (paged_pages(shape, page_size, pt) != LSA_OK) return LSA_ERR_UNSUPPORTED;
    }
    lsa_status st = check_keys(key_dtype, keys, key_scale);
    if (st != LSA_OK) return st;
    if ((st = check_ragged(shape)) != LSA_OK) return st;
    if (!page_keys) return LSA_ERR_NULL_POINTER;
    if (!aligned(page_keys, 16)) return LSA_ERR_BAD_SHAPE;
    const int64_t n_pages = (shape->kv_len + page_size - 1) / page_size;
    if (page_lo < 0 || page_hi < page_lo || page_hi > n_pages) return LSA_ERR_BAD_SHAPE;
    if (shape->batch == 0 || page_hi == page_lo) return LSA_OK;
    return device_status(lsa::launch_page_summary(keys, key_dtype == LSA_KEY_FP8_E4M3, key_scale,
                                                  shape->batch, shape->kv_len, shape->seq_len,
                                                  shape->head_dim, page_size, page_lo, page_hi,
                                                  static_cast<uint16_t *>(page_keys),
                                                  static_cast<hipStream_t>(stream), pt));
}

lsa_status lsa_page_recall(const lsa_index_shape *shape, lsa_budget budget, int32_t page_size,
                           int32_t m_pages, const void *q, const float *w, const void *page_keys,
                           const void *keys, lsa_key_dtype key_dtype, const float *key_scale,
                           int32_t *page_ids, float *cand_scores, int32_t *cand_ids, void *ws,
                           size_t ws_bytes, void *stream)
{
    lsa_status st = check_index_shape(shape);
    if (st != LSA_OK) return st;
    lsa::PagedTab pt;
    if ((st = paged_pages(shape, page_size, pt)) != LSA_OK) return st;
    if ((st = check_budget(budget)) != LSA_OK) return st;
    if (!pow2(page_size) || page_size < 32 || page_size > 256) return LSA_ERR_BAD_SHAPE;
    if (m_pages < 1 || m_pages > 65536) return LSA_ERR_BAD_SHAPE;
    // A query that sees fewer than kv_len keys (causal prefill) must not recall a page that
    // extends past its last valid key: that page's key is a mean over later tokens.  The last
    // eligible page ends before V when the window covers at least P - 1 tokens.
    // (With per-sequence arrays the host cannot see the positions: the window must cover it.)
    if ((ragged(shape) || shape->q_pos0 + 1 < shape->kv_len) && budget.window < page_size - 1)
        return LSA_ERR_UNSUPPORTED;
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
    c.seq_len = shape->seq_len;
    c.seq_pos0 = shape->seq_pos0;
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
    s.seq_len = shape->seq_len;
    s.seq_pos0 = shape->seq_pos0;
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
    f.seq_len = shape->seq_len;
    f.seq_pos0 = shape->seq_pos0;
    f.k = budget.k;
    f.sink = budget.sink;
    f.window = budget.window;
    f.page = page_size;
    f.m_pages = m_pages;
    f.fp8 = key_dtype == LSA_KEY_FP8_E4M3;
    f.btab = pt.btab; // paged keys (the page keys of stage 1 are a dense array)
    f.lbs = pt.lbs;
    f.bps = pt.bps;
    f.n_blocks = pt.n_blocks;
    return device_status(lsa::launch_fine_scores(f, sm));
}

} // extern "C"

namespace {

// lsa_sparse_attn over n_layers layers that share one index list (n_layers == 1: the
// single-layer call).  The pointer arrays are host arrays of device pointers.
lsa_status sparse_attn_layers(const lsa_index_shape *shape, const lsa_attn_shape *attn,
                              lsa_budget budget, int32_t n_layers, const void *const *q,
                              const void *const *k, const void *const *v, const int32_t *idx,
                              void *const *out, float *const *lse, void *ws, size_t ws_bytes,
                              void *stream)
{
    lsa_status st = check_attn(shape, attn, budget);
    if (st != LSA_OK) return st;
    if (n_layers < 1 || n_layers > lsa::kMaxAttnLayers) return LSA_ERR_BAD_SHAPE;
    if (!q || !k || !v || !idx || !out) return LSA_ERR_NULL_POINTER;
    for (int l = 0; l < n_layers; ++l) {
        if (!q[l] || !k[l] || !v[l] || !out[l]) return LSA_ERR_NULL_POINTER;
        if (attn->latent && v[l] != k[l]) return LSA_ERR_BAD_SHAPE;
        if (!aligned(q[l], 16) || !aligned(k[l], 16) || !aligned(v[l], 16) || !aligned(out[l], 4) ||
            (lse && lse[l] && !aligned(lse[l], 4)))
            return LSA_ERR_BAD_SHAPE;
    }
    if ((st = check_ragged(shape)) != LSA_OK) return st;
    if (!aligned(idx, 4)) return LSA_ERR_BAD_SHAPE;
    if (budget.sink < 0 || budget.window < 0 || (int64_t)budget.sink + budget.window > budget.k)
        return LSA_ERR_BAD_SHAPE;
    int lbs = 0;
    if (attn->block_table) { // a paged latent cache
        if (!attn->latent) return LSA_ERR_UNSUPPORTED;
        const int64_t bs = attn->block_size;
        if (!pow2(attn->block_size) || bs > (1 << 20) || attn->blocks_per_seq < 1 ||
            attn->n_blocks < 1 || (int64_t)attn->blocks_per_seq * bs < shape->kv_len ||
            attn->n_blocks * bs >= (int64_t(1) << 31) || !aligned(attn->block_table, 4))
            return LSA_ERR_BAD_SHAPE;
        while ((int64_t(1) << lbs) < bs) ++lbs;
    }
    const int64_t rows = (int64_t)shape->batch * shape->n_q;
    if (rows == 0) return LSA_OK;
    if (rows * attn->n_heads * n_layers >= (int64_t(1) << 31) * 4) return LSA_ERR_UNSUPPORTED;
    if ((int64_t)shape->batch * n_layers > kMaxGridYZ) return LSA_ERR_UNSUPPORTED;
    // the splits are chosen for the whole grid (every layer's workgroups), so a group of layers
    // needs no more partials than one layer of a batch n_layers times larger
    const size_t all_layers = lsa::attn_workspace_bytes(shape->batch * n_layers, shape->n_q,
                                                        attn->n_heads, attn->d_v, budget.k,
                                                        attn->latent);
    const size_t need = round256(all_layers);
    if (need && (!ws || ws_bytes < need || !aligned(ws, 256))) return LSA_ERR_WORKSPACE_TOO_SMALL;
    lsa::AttnArgs a{};
    a.q = static_cast<const uint16_t *>(q[0]);
    a.k = static_cast<const uint16_t *>(k[0]);
    a.v = static_cast<const uint16_t *>(v[0]);
    a.idx = idx;
    a.out = static_cast<uint16_t *>(out[0]);
    a.lse = lse ? lse[0] : nullptr;
    a.ws = static_cast<float *>(ws);
    a.batch = shape->batch;
    a.n_q = shape->n_q;
    a.heads = attn->n_heads;
    a.d_qk = attn->d_qk;
    a.d_v = attn->d_v;
    a.n_idx = budget.k;
    a.latent = attn->latent;
    a.kv_len = shape->kv_len;
    a.seq_len = shape->seq_len;
    a.k_stride = attn->k_row_stride;
    a.v_stride = attn->v_row_stride;
    a.sink = budget.sink;
    a.window = budget.window;
    a.q_pos0 = shape->q_pos0;
    a.seq_pos0 = shape->seq_pos0;
    a.scale = attn->scale;
    a.n_split = lsa::attn_splits(shape->batch * n_layers, shape->n_q, attn->n_heads, budget.k,
                                 attn->latent);
    a.layers = n_layers;
    a.ws_layer = (int64_t)(all_layers / n_layers / sizeof(float));
    a.btab = attn->block_table;
    a.lbs = lbs;
    a.bps = attn->block_table ? attn->blocks_per_seq : 0;
    a.n_blocks = attn->block_table ? attn->n_blocks : 0;
    for (int l = 0; l < n_layers; ++l) {
        a.lq[l] = static_cast<const uint16_t *>(q[l]);
        a.lk[l] = static_cast<const uint16_t *>(k[l]);
        a.lv[l] = static_cast<const uint16_t *>(v[l]);
        a.lout[l] = static_cast<uint16_t *>(out[l]);
        a.llse[l] = lse ? lse[l] : nullptr;
    }
    return device_status(lsa::launch_sparse_attn(a, static_cast<hipStream_t>(stream)));
}

} // namespace

extern "C" {

lsa_status lsa_sparse_attn(const lsa_index_shape *shape, const lsa_attn_shape *attn,
                           lsa_budget budget, const void *q, const void *k, const void *v,
                           const int32_t *idx, void *out, float *lse, void *ws, size_t ws_bytes,
                           void *stream)
{
    float *lse1[1] = {lse};
    return sparse_attn_layers(shape, attn, budget, 1, &q, &k, &v, idx, &out, lse1, ws, ws_bytes,
                              stream);
}

lsa_status lsa_sparse_attn_layers(const lsa_index_shape *shape, const lsa_attn_shape *attn,
                                  lsa_budget budget, int32_t n_layers, const void *const *q,
                                  const void *const *k, const void *const *v, const int32_t *idx,
                                  void *const *out, float *const *lse, void *ws, size_t ws_bytes,
                                  void *stream)
{
    return sparse_attn_layers(shape, attn, budget, n_layers, q, k, v, idx, out, lse, ws, ws_bytes,
                              stream);
}


lsa_status lsa_sparse_attn_backward(const lsa_index_shape *shape, const lsa_attn_shape *attn,
                                    lsa_budget budget, const void *q, const void *k, const void *v,
                                    const int32_t *idx, const void *out, const float *lse,
                                    const void *d_out, float *d_q, float *d_k, float *d_v,
                                    void *stream)
{
    lsa_status st = check_attn(shape, attn, budget);
    if (st != LSA_OK) return st;
    if (!q || !k || !v || !idx || !out || !lse || !d_out || !d_q || !d_k || !d_v)
        return LSA_ERR_NULL_POINTER;
    if (attn->latent && (v != k || d_v != d_k)) return LSA_ERR_BAD_SHAPE;
    if (!attn->latent && d_v == d_k) return LSA_ERR_BAD_SHAPE;
    if (attn->block_table) return LSA_ERR_UNSUPPORTED; // the gradients are dense
    if ((st = check_ragged(shape)) != LSA_OK) return st;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(idx, 4) ||
        !aligned(out, 16) || !aligned(lse, 4) || !aligned(d_out, 16) || !aligned(d_q, 4) ||
        !aligned(d_k, 4) || !aligned(d_v, 4))
        return LSA_ERR_BAD_SHAPE;
    if (budget.sink < 0 || budget.window < 0 || (int64_t)budget.sink + budget.window > budget.k)
        return LSA_ERR_BAD_SHAPE;
    const int64_t rows = (int64_t)shape->batch * shape->n_q;
    if (rows == 0) return LSA_OK;
    if (rows * attn->n_heads >= (int64_t(1) << 31) * 4) return LSA_ERR_UNSUPPORTED;
    lsa::AttnBwdArgs a{};
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.idx = idx;
    a.out = static_cast<const uint16_t *>(out);
    a.lse = lse;
    a.dout = static_cast<const uint16_t *>(d_out);
    a.dq = d_q;
    a.dk = d_k;
    a.dv = d_v;
    a.batch = shape->batch;
    a.n_q = shape->n_q;
    a.heads = attn->n_heads;
    a.d_qk = attn->d_qk;
    a.d_v = attn->d_v;
    a.n_idx = budget.k;
    a.latent = attn->latent;
    a.kv_len = shape->kv_len;
    a.seq_len = shape->seq_len;
    a.k_stride = attn->k_row_stride;
    a.v_stride = attn->v_row_stride;
    a.scale = attn->scale;
    a.n_split = lsa::attn_bwd_splits(shape->batch, shape->n_q, attn->n_heads, budget.k, attn->latent);
    a.sink = budget.sink;
    a.window = budget.window;
    a.q_pos0 = shape->seq_pos0 ? -1 : shape->q_pos0; // the key-major pass: uniform batches only
    a.si = 0;
    return device_status(lsa::launch_sparse_attn_backward(a, static_cast<hipStream_t>(stream)));
}

lsa_status lsa_index_scores_backward(const lsa_index_shape *shape, lsa_budget budget,
                                     const void *q, const float *w, const void *keys,
                                     const int32_t *idx, const float *d_scores, float *d_q,
                                     float *d_w, float *d_keys, void *stream)
{
    if (!shape) return LSA_ERR_NULL_POINTER;
    const int32_t k = budget.k;
    if (shape->batch < 0 || shape->n_q < 0 || shape->kv_len < 1 ||
        shape->kv_len >= (int64_t(1) << 31) || shape->q_pos0 < 0 || shape->batch > kMaxGridYZ ||
        shape->n_heads < 1 || shape->head_dim < 1 || k < 1)
        return LSA_ERR_BAD_SHAPE;
    if (budget.sink < 0 || budget.window < 0 || (int64_t)budget.sink + budget.window > k)
        return LSA_ERR_BAD_SHAPE;
    if (!lsa::index_bwd_supported(shape->n_heads, shape->head_dim)) return LSA_ERR_UNSUPPORTED;
    if (shape->n_q > kMaxGridYZ || dense_keys_only(shape) != LSA_OK) return LSA_ERR_UNSUPPORTED;
    lsa_status st = check_ragged(shape);
    if (st != LSA_OK) return st;
    if (!q || !w || !keys || !idx || !d_scores || !d_q || !d_w || !d_keys) return LSA_ERR_NULL_POINTER;
    if (!aligned(q, 16) || !aligned(w, 4) || !aligned(keys, 16) || !aligned(idx, 4) ||
        !aligned(d_scores, 4) || !aligned(d_q, 4) || !aligned(d_w, 4) || !aligned(d_keys, 4))
        return LSA_ERR_BAD_SHAPE;
    if ((int64_t)shape->batch * shape->n_q == 0) return LSA_OK;
    lsa::IndexBwdArgs a{};
    a.q = static_cast<const uint16_t *>(q);
    a.w = w;
    a.keys = static_cast<const uint16_t *>(keys);
    a.idx = idx;
    a.dscore = d_scores;
    a.dq = d_q;
    a.dw = d_w;
    a.dkeys = d_keys;
    a.batch = shape->batch;
    a.n_q = shape->n_q;
    a.heads = shape->n_heads;
    a.dim = shape->head_dim;
    a.n_idx = k;
    a.kv_len = shape->kv_len;
    a.q_pos0 = shape->q_pos0;
    a.seq_len = shape->seq_len;
    a.seq_pos0 = shape->seq_pos0;
    a.n_split = lsa::index_bwd_splits(shape->batch, shape->n_q, k);
    a.sink = budget.sink;
    a.window = budget.window;
    a.si = 0; // decided at launch
    return device_status(lsa::launch_index_scores_backward(a, static_cast<hipStream_t>(stream)));
}

} // extern "C"
