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
    int mask;             // RowMask (flat / coarse modes)
    int k, sink, window;  // budget (coarse and fine modes)
    int page;             // P (coarse and fine modes)
    int m_pages;          // fine mode
    int fp8;              // keys are e4m3 with per-row scales
};

// Flat or coarse scores: out[b,t,s] for s < n_out == n_keys, -inf outside the row's range.
hipError_t launch_scores(const ScoreArgs &a, hipStream_t stream);
// Fine scores over recalled pages: out / out_ids [b,t, i*P + j].
hipError_t launch_fine_scores(const ScoreArgs &a, hipStream_t stream);
bool scores_supported(int heads, int dim);

struct SelectArgs {
    const float *scores;     // [rows, n_in]
    const int32_t *cand_ids; // [rows, n_in] or nullptr (position = id)
    int32_t *out;            // [rows, out_stride]
    int batch, n_q;
    int64_t n_in;
    int64_t kv_len, q_pos0;
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

hipError_t launch_page_summary(const void *keys, int fp8, const float *kscale, int batch,
                               int64_t kv_len, int dim, int page, int64_t page_lo,
                               int64_t page_hi, uint16_t *page_keys, hipStream_t stream);

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
    int sink, window;
    float scale;
    int n_split;          // chunks of the index list per (query, head group)
};

int attn_splits(int batch, int n_q, int heads, int n_idx, int latent);
size_t attn_workspace_bytes(int batch, int n_q, int heads, int d_v, int n_idx, int latent);
hipError_t launch_sparse_attn(const AttnArgs &a, hipStream_t stream);
bool attn_supported(int heads, int d_qk, int d_v, int latent);

} // namespace lsa
