// si_layout.hpp -- the Streaming-Aware entries of prefill index lists, for the key-major passes
// of the backward kernels.
//
// (Model card, SI bullet: a fixed share of every list is a sink of leading tokens and a local
// window of the latest ones.)  lsa_topk_select lays a list of a query with valid length
// V_t = min(kv_len, q_pos0 + t + 1) > k out as the sink rows 0 .. S-1 in entries [0, S), the
// window rows V_t - W .. V_t - 1 in entries [S, S + W), then the dynamic picks.  Neighbouring
// queries of a prefill chunk therefore share their sink rows and most of their window rows.  A
// key-major pass owns blocks of SRB consecutive key rows (the sink's, and those of the band the
// windows cover) with the queries whose sink or window reach them, sums those queries' gradient
// shares of each row and adds each row column once; the query-major kernel skips exactly the
// entries the pass takes.  Uniform batches only (one q_pos0, no per-sequence arrays).
//
// Args: any argument struct with kv_len, q_pos0 (int64), sink, window and n_q (int).
#pragma once

#include <cstdint>

namespace lsa {
namespace si {

constexpr int SRB = 64;  // key rows per key-major workgroup
constexpr int SQC = 128; // queries per key-major workgroup

struct Plan {
    int nsb;      // sink blocks: rows [SRB i, min(S, SRB (i + 1)))
    int64_t wlo;  // window blocks follow: rows [wlo + SRB j, + SRB)
    int64_t t_si; // first query whose sink and window are disjoint
    int cs, cw;   // query chunks per sink block and per window block
};

__host__ __device__ inline int64_t imin(int64_t x, int64_t y) { return x < y ? x : y; }
__host__ __device__ inline int64_t imax(int64_t x, int64_t y) { return x > y ? x : y; }

// V_t, the valid length the selection gives query t
template <class A>
__host__ __device__ inline int64_t valid_len(const A &a, int64_t t)
{
    return imin(a.kv_len, a.q_pos0 + t + 1);
}

// Entry j (holding id) of the list of a query of valid length V: the key-major pass takes it
// when the query's sink and window are disjoint and the entry holds the row the layout puts
// there (sink row j, or window row V - W + j - S).
template <class A>
__device__ inline bool taken(const A &a, int64_t V, int j, int32_t id)
{
    if (V - a.window < a.sink) return false;
    if (j < a.sink) return id == j;
    if (j < a.sink + a.window) return (int64_t)id == V - a.window + (j - a.sink);
    return false;
}

// Rows [r0, r1) of key-major block blk and the queries [t_lo, t_hi) whose sink or window can
// reach them (V_t > r0 and V_t - W < r1 for a window block).
template <class A>
__host__ __device__ inline void block(const A &a, const Plan &p, int blk, int64_t &r0, int64_t &r1,
                                      int64_t &t_lo, int64_t &t_hi)
{
    if (blk < p.nsb) {
        r0 = (int64_t)SRB * blk;
        r1 = imin(a.sink, r0 + SRB);
        t_lo = p.t_si;
        t_hi = a.n_q;
        return;
    }
    r0 = p.wlo + (int64_t)SRB * (blk - p.nsb);
    r1 = imin(r0 + SRB, a.kv_len);
    t_lo = imax(p.t_si, r0 - a.q_pos0);
    t_hi = a.kv_len < r1 + a.window ? a.n_q : imin(a.n_q, r1 + a.window - a.q_pos0 - 1);
}

// The key-major pass's blocks and query chunks (nchunk workgroups per sequence and head group),
// or false where it does not apply (no sink or window, no query whose sink and window are
// disjoint, a negative position) or would not pay: it pays when each row update it makes
// stands for at least 8 query entries (prefill chunks), not when every row is reached by one
// query or few (decode).  The caller checks its own further conditions (uniform batch, ...).
template <class A>
inline bool plan(const A &a, Plan &p, int &nblk, int &nchunk, int64_t grid_yz)
{
    const int64_t S = a.sink, W = a.window;
    if (a.q_pos0 < 0 || S < 0 || W < 0 || S + W == 0 || a.n_q < 1 || a.kv_len < S + W)
        return false;
    p.t_si = imax(0, S + W - a.q_pos0 - 1);
    if (p.t_si >= a.n_q) return false;
    p.nsb = (int)((S + SRB - 1) / SRB);
    const int64_t vmin = valid_len(a, p.t_si), vmax = valid_len(a, a.n_q - 1);
    p.wlo = S + SRB * ((vmin - W - S) / SRB); // vmin >= S + W
    const int64_t nwb = W > 0 ? (vmax - p.wlo + SRB - 1) / SRB : 0;
    if (p.nsb + nwb > (int64_t(1) << 30)) return false;
    nblk = (int)(p.nsb + nwb);
    int64_t span_s = 0, span_w = 0;
    for (int blk = 0; blk < nblk; ++blk) {
        int64_t r0, r1, t_lo, t_hi;
        block(a, p, blk, r0, r1, t_lo, t_hi);
        if (r0 < r1) (blk < p.nsb ? span_s : span_w) = imax(blk < p.nsb ? span_s : span_w, t_hi - t_lo);
    }
    p.cs = (int)((span_s + SQC - 1) / SQC);
    p.cw = (int)((span_w + SQC - 1) / SQC);
    if (p.nsb > 0 && p.cs < 1) p.cs = 1;
    if (nwb > 0 && p.cw < 1) p.cw = 1;
    const int64_t groups = (int64_t)p.nsb * p.cs + nwb * p.cw;
    if (groups < 1 || groups >= (int64_t(1) << 31) || grid_yz > 65535) return false;
    nchunk = (int)groups;
    const int64_t entries = (int64_t)(a.n_q - p.t_si) * (S + W); // entries the pass takes
    const int64_t own = groups * SRB;                             // row updates it makes
    return entries >= 8 * own;
}

// Workgroup g of a key-major launch -> its block and query chunk (the sink blocks' chunks
// first, then the window blocks').
__device__ inline void workgroup(const Plan &p, int g, int &blk, int &chunk)
{
    const int gs = p.nsb * p.cs;
    blk = g < gs ? g / p.cs : p.nsb + (g - gs) / p.cw;
    chunk = g < gs ? g % p.cs : (g - gs) % p.cw;
}

} // namespace si
} // namespace lsa
