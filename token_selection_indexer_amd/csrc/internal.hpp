// internal.hpp -- argument blocks and kernel launchers shared by the host library's translation
// units.  Not part of the public ABI (include/lsa.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsa {

// Which keys a query row may score.
enum RowMask : int {
    MASK_CAUSAL = 0, // token keys: [0, V_t)
    MASK_PAGES = 1,  // page keys: pages overlapping the middle [S, V_t - W), none when V_t <= k
};

// Entries per workgroup slice of the fused decode selection (ScoreArgs::slice_ent), and the
// most keys a scoring workgroup may own for it (its scores are staged in LDS).
constexpr int kSliceCap = 1024;
constexpr int kSliceSpan = 8192;

struct ScoreArgs {
    const uint16_t *q;    // [B, n_q, H, d] bf16
    const float *w;       // [B, n_q, H]
    const void *keys;     // [B, n_keys, d] bf16 or e4m3
    const float *kscale;  // [B, n_keys] (fp8) or nullptr
    float *out;           // [B, n_q, n_out]
    int32_t *out_ids;     // fine mode: [B, n_q, n_out] token ids, else nullptr
    const int32_t *pages; // fine mode: [B, n_q, m_pages] recalled pages (ascending, -1 pad)
    int batch, n_q, heads, dim;
    int64_t n_keys;       // key rows per sequence
    int64_t n_out;        // outputs per query row
    int64_t kv_len, q_pos0;
    const int32_t *seq_len, *seq_pos0; // [B] ragged batch (device) or nullptr
    int mask;             // RowMask (flat / coarse modes)
    int k, sink, window;  // budget (coarse and fine modes)
    int page;             // P (coarse and fine modes)
    int m_pages;          // fine mode
    int fp8;              // keys are e4m3 with per-row scales
    // Decode selection fused into scoring (flat rows, one query per workgroup): each workgroup
    // also writes the 2048-bin histogram (key bits 31..21) of its middle-region scores, as 32
    // coarse sums of 64 bins each and the 64 fine bins of every non-empty group, to slice
    // [row][blockIdx.x].
    uint32_t *hist_fine;  // [rows][groups][2048] or nullptr
    uint32_t *hist_coarse; // [rows][groups][32]
    // With the histograms, each workgroup also keeps its middle-region scores in bins at or above
    // a local threshold bin (the bin of its slice_target-th best, one bin higher when more than
    // kSliceCap would be kept) in position order: slice [row][blockIdx.x] of slice_ent, entries
    // {score bits, position}, with header {bin, count, first position, end position} of the
    // workgroup's middle-region range.
    int4 *slice_hdr;      // [rows][groups]
    uint2 *slice_ent;     // [rows][groups][kSliceCap]
    int slice_target;
    // fp8 queries (q8 != nullptr): e4m3 codes [B, n_q, H, d] with one fp32 scale per (query,
    // head); `q` is then unused and the keys must be e4m3 too
    const uint8_t *q8;
    const float *q_scale; // [B, n_q, H]
    // Paged keys (btab != nullptr): keys and kscale are pools of n_blocks blocks of 2^lbs rows,
    // and key row s of sequence b is pool row btab[b * bps + (s >> lbs)] << lbs | s & (2^lbs - 1)
    // (a table entry outside [0, n_blocks): that block's scores are -inf).  Flat stream path.
    const int32_t *btab;
    int lbs, bps;
    int64_t n_blocks;
};

// A block table over pooled keys (btab == nullptr: dense keys): key row s of sequence b is pool
// row btab[b * bps + (s >> lbs)] << lbs | s & (2^lbs - 1); entries outside [0, n_blocks) mark
// blocks without keys.
struct PagedTab {
    const int32_t *btab = nullptr;
    int lbs = 0, bps = 0;
    int64_t n_blocks = 0;
};

// Block-table entries a paged scoring workgroup caches in LDS (its key range's blocks).
constexpr int kPagedTab = 512;
// Whether the paged form of the scoring launch takes this shape (the flat stream path, with a
// workgroup's key range covering at most kPagedTab table entries).
bool scores_paged_ok(const ScoreArgs &a);

// Per-row e4m3 quantisation: scale[r] = amax / 448 (1 for a zero row), codes = round to
// nearest even e4m3fn of x / scale, saturating.  x bf16 [rows, d], d in {64, 128}.
hipError_t launch_quantize_rows(const uint16_t *x, int64_t rows, int d, uint8_t *codes,
                                float *scale, hipStream_t stream);

// Flat or coarse scores: out[b,t,s] for s < n_out == n_keys, -inf outside the row's range.
hipError_t launch_scores(const ScoreArgs &a, hipStream_t stream);
// Fine scores over recalled pages: out / out_ids [b,t, i*P + j].
hipError_t launch_fine_scores(const ScoreArgs &a, hipStream_t stream);
bool scores_supported(int heads, int dim);
// Workgroups per query row ("groups") of the flat launch when it can emit the selection
// histograms (the long decode launch, one query per workgroup); 0 when it cannot.
int score_hist_groups(const ScoreArgs &a);
// Keys each workgroup of that launch owns (slices need at most kSliceSpan).
int64_t score_hist_span(const ScoreArgs &a, int groups);

struct SelectArgs {
    const float *scores;     // [rows, n_in]
    const int32_t *cand_ids; // [rows, n_in] or nullptr (position = id)
    int32_t *out;            // [rows, out_stride]
    int batch, n_q;
    int64_t n_in;
    int64_t kv_len, q_pos0;
    const int32_t *seq_len, *seq_pos0; // [B] ragged batch (device) or nullptr
    int k, sink, window;     // SI budget
    int mode;                // SelectMode
    int page;                // MODE_PAGES: P
    int m_pages;             // MODE_PAGES: how many pages to keep
    int out_stride;
};

enum SelectMode : int {
    SELECT_SI = 0,    // sink | window | dynamic top-(k-S-W) over the middle (flat or candidates)
    SELECT_PAGES = 1, // top-m_pages of the eligible pages of a coarse-score row, ids ascending
};

// Workspace of the selection (0 when one workgroup per row is used).
size_t select_workspace_bytes(int64_t rows, int64_t n_in, int mode);
hipError_t launch_select(const SelectArgs &a, void *ws, hipStream_t stream);
// The same, with the scoring launch's row histograms (ScoreArgs::hist_*) for flat rows: the
// chunked path reads each row's threshold bin from them instead of sampling the row.
hipError_t launch_select_hist(const SelectArgs &a, void *ws, const uint32_t *hist_fine,
                              const uint32_t *hist_coarse, int groups, hipStream_t stream);
// The fused decode path with slices: one launch, one workgroup per row, that gathers the
// scoring workgroups' slices (ScoreArgs::slice_*) at or above their highest local bin -- or,
// when those hold fewer than the row needs, takes the row's threshold bin from the histograms --
// and selects exactly.  No workspace of its own; at most select_slice_groups_max() scoring
// workgroups per row.
int select_slice_groups_max();
hipError_t launch_select_slices(const SelectArgs &a, const uint32_t *hist_fine,
                                const uint32_t *hist_coarse, const int4 *slice_hdr,
                                const uint2 *slice_ent, int groups, hipStream_t stream);
// The library's own per-device scratch for callers that cannot allocate: its size, and the
// current device's address of it (looked up on the first call on each device).
size_t select_scratch_bytes();
hipError_t select_scratch(void **ptr);

hipError_t launch_page_summary(const void *keys, int fp8, const float *kscale, int batch,
                               int64_t kv_len, const int32_t *seq_len, int dim, int page,
                               int64_t page_lo, int64_t page_hi, uint16_t *page_keys,
                               hipStream_t stream,
                               const PagedTab &paged = PagedTab{});

constexpr int kMaxAttnLayers = 8;

struct AttnArgs {
    const uint16_t *q;    // [B, n_q, Hq, d_qk]
    const uint16_t *k;    // [B, L, k_stride]
    const uint16_t *v;    // [B, L, v_stride]
    const int32_t *idx;   // [B, n_q, n_idx]
    uint16_t *out;        // [B, n_q, Hq, d_v]
    float *lse;           // [B, n_q, Hq] or nullptr
    float *ws;            // split partials
    int batch, n_q, heads, d_qk, d_v, n_idx, latent;
    int64_t kv_len, k_stride, v_stride;
    const int32_t *seq_len; // [B] valid rows per sequence (device) or nullptr
    int sink, window;
    int64_t q_pos0;         // query positions (with seq_pos0): where the layout puts the window
    const int32_t *seq_pos0;
    float scale;
    int n_split;          // workgroups per (query, head group); rounds are dealt to them in turn
    // Latent kernel: `layers` layers over the one index list (grid z = layer * batch + b), each
    // with its own q, cache, out and lse; the split partials of layer l start at ws + l * ws_layer
    int layers;
    int64_t ws_layer;
    // paged latent cache (btab != nullptr): k / lk are pools of n_blocks blocks of 2^lbs rows,
    // token s of sequence b at pool row btab[b * bps + (s >> lbs)] << lbs | (s & mask)
    const int32_t *btab;
    int lbs, bps;
    int64_t n_blocks;
    const uint16_t *lq[kMaxAttnLayers];
    const uint16_t *lk[kMaxAttnLayers];
    const uint16_t *lv[kMaxAttnLayers];
    uint16_t *lout[kMaxAttnLayers];
    float *llse[kMaxAttnLayers];
};

int attn_splits(int batch, int n_q, int heads, int n_idx, int latent);

// Backward of the sparse attention: the forward's operands plus its output and lse, the output
// gradient, and three fp32 gradients that are added into (d_k == d_v for a latent cache).
struct AttnBwdArgs {
    const uint16_t *q;    // [B, n_q, Hq, d_qk]
    const uint16_t *k;    // [B, L, k_stride]
    const uint16_t *v;    // [B, L, v_stride]
    const int32_t *idx;   // [B, n_q, n_idx]
    const uint16_t *out;  // [B, n_q, Hq, d_v] forward output
    const float *lse;     // [B, n_q, Hq] forward log-sum-exp (natural log)
    const uint16_t *dout; // [B, n_q, Hq, d_v]
    float *dq;            // [B, n_q, Hq, d_qk]
    float *dk;            // [B, L, d_qk]
    float *dv;            // [B, L, d_v] (latent: == dk)
    int batch, n_q, heads, d_qk, d_v, n_idx, latent;
    int64_t kv_len, k_stride, v_stride;
    const int32_t *seq_len; // [B] valid rows per sequence (device) or nullptr
    float scale;
    int n_split;          // chunks of the index list per (query, head group)
    // Streaming-Aware entries (sink [0, S) and window [S, S + W) of each list, as the selection
    // lays them out for V_t = min(kv_len, q_pos0 + t + 1)) taken by the key-major pass: si != 0
    int sink, window, si;
    int64_t q_pos0;
};

int attn_bwd_splits(int batch, int n_q, int heads, int n_idx, int latent);
hipError_t launch_sparse_attn_backward(const AttnBwdArgs &a, hipStream_t stream);

// Backward of the indexer scores at the selected entries (bf16 keys): gradients added into.
struct IndexBwdArgs {
    const uint16_t *q;        // [B, n_q, H, d]
    const float *w;           // [B, n_q, H]
    const uint16_t *keys;     // [B, L, d] bf16
    const int32_t *idx;       // [B, n_q, n_idx]
    const float *dscore;      // [B, n_q, n_idx]
    float *dq;                // [B, n_q, H, d]
    float *dw;                // [B, n_q, H]
    float *dkeys;             // [B, L, d]
    int batch, n_q, heads, dim, n_idx;
    int64_t kv_len, q_pos0;
    const int32_t *seq_len, *seq_pos0; // [B] ragged batch (device) or nullptr
    int n_split;              // chunks of the index list per query
    // Streaming-Aware entries (sink [0, S) and window [S, S + W) of each list, as the selection
    // lays them out) whose key gradient the key-major pass adds: si != 0
    int sink, window, si;
};

bool index_bwd_supported(int heads, int dim);
int index_bwd_splits(int batch, int n_q, int n_idx);
hipError_t launch_index_scores_backward(const IndexBwdArgs &a, hipStream_t stream);
size_t attn_workspace_bytes(int batch, int n_q, int heads, int d_v, int n_idx, int latent);
hipError_t launch_sparse_attn(const AttnArgs &a, hipStream_t stream);
bool attn_supported(int heads, int d_qk, int d_v, int latent);

} // namespace lsa
