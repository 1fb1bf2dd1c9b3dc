// topk.hip -- per-query selection: Streaming-Aware Indexing (sink + local window + dynamic
// top-k) and the page-recall top-M of Hierarchical Indexing.
//
// (Model card, SI bullet: part of the budget goes to a fixed sink and a local sliding window, the
// rest to dynamic sparse selection; Baidu Cloud article, "2. Dynamic Token Selector": top-k of
// the score row.  Model card, HI bullet: candidate blocks are recalled by coarse scores.)
//
// One workgroup of 1024 threads owns one query row.  The selection is an exact radix select on
// an order-preserving uint32 image of the fp32 scores (larger key = larger score, -0 == +0), with
// ties going to the lower position -- which is the lower token index, because rows are in token
// order and candidate lists are ascending:
//   1. histogram of key bits 31..21 (2048 bins in LDS) over the row;
//   2. the bin holding the k-th key; everything above it is selected;
//   3. if the elements of that bin and above fit in LDS, one ordered pass compacts them there and
//      the remaining digits (bits 20..10, 9..0) are resolved in LDS; otherwise the next digit is
//      histogrammed from the row again (heavy ties), until the threshold key T is exact;
//   4. one ordered pass emits keys > T plus the first (k - #greater) keys == T in position order,
//      so the picks come out ascending without a sort.
// Sink [0,S) and window [V-W,V) are written arithmetically, never scored or compared.
#include "device.hpp"
#include "internal.hpp"

namespace lsa {
namespace {

constexpr int NT = 1024;
constexpr int NW = NT / kWave;
constexpr int ITEMS = 4;            // contiguous elements per thread per round
constexpr int ROUND = NT * ITEMS;
constexpr int CAP = 8192;           // LDS candidate buffer (key, id) entries

struct Smem {
    int hist[2048];
    int scan[NW + 1];
    int misc[8];
    uint32_t buf_key[CAP];
    int32_t buf_id[CAP];
};

// A row's competing elements: positions [lo, hi) of `sc` (and `ids` in candidate mode); an
// element competes iff its id lies in [id_lo, id_hi).  Position order is id order.
struct Row {
    const float *sc;
    const int32_t *ids; // nullptr: id = position
    int64_t lo, hi;
    int64_t id_lo, id_hi;
    bool vec;           // 16-byte aligned rows: vector loads
};

__device__ __forceinline__ void load_items(const Row &r, int64_t base, uint32_t (&key)[ITEMS],
                                           int32_t (&id)[ITEMS])
{
    const int64_t p0 = base + (int64_t)threadIdx.x * ITEMS;
    float s[ITEMS];
    int32_t c[ITEMS];
    if (r.vec && p0 + ITEMS <= r.hi && p0 >= r.lo) {
        const float4 v = *reinterpret_cast<const float4 *>(r.sc + p0);
        s[0] = v.x; s[1] = v.y; s[2] = v.z; s[3] = v.w;
        if (r.ids) {
            const int4 iv = *reinterpret_cast<const int4 *>(r.ids + p0);
            c[0] = iv.x; c[1] = iv.y; c[2] = iv.z; c[3] = iv.w;
        } else {
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) c[j] = (int32_t)(p0 + j);
        }
    } else {
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const int64_t p = p0 + j;
            const bool in = p >= r.lo && p < r.hi;
            s[j] = in ? r.sc[p] : 0.0f;
            c[j] = in ? (r.ids ? r.ids[p] : (int32_t)p) : -1;
        }
    }
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const int64_t p = p0 + j;
        const bool ok = p >= r.lo && p < r.hi && c[j] >= r.id_lo && c[j] < r.id_hi;
        key[j] = ok ? order_key(s[j]) : 0u;
        id[j] = c[j];
    }
}

__device__ __forceinline__ int64_t round_begin(const Row &r) { return (r.lo / ITEMS) * ITEMS; }

// Histogram of digit (key >> shift) & (nbins-1) over the row's elements whose bits above the
// digit equal `prefix` (all elements when pbits == 0).
__device__ void hist_row(Smem &sm, const Row &r, int shift, int nbins, int pbits, uint32_t prefix)
{
    for (int i = threadIdx.x; i < 2048; i += NT) sm.hist[i] = 0;
    __syncthreads();
    const int hs = shift + __builtin_ctz((unsigned)nbins);
    for (int64_t base = round_begin(r); base < r.hi; base += ROUND) {
        uint32_t key[ITEMS];
        int32_t id[ITEMS];
        load_items(r, base, key, id);
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            if (!key[j]) continue;
            if (pbits && (hs >= 32 ? 0u : (key[j] >> hs)) != prefix) continue;
            atomicAdd(&sm.hist[(key[j] >> shift) & (uint32_t)(nbins - 1)], 1);
        }
    }
    __syncthreads();
}

__device__ void hist_buf(Smem &sm, int nbuf, int shift, int nbins, uint32_t prefix)
{
    for (int i = threadIdx.x; i < 2048; i += NT) sm.hist[i] = 0;
    __syncthreads();
    const int hs = shift + __builtin_ctz((unsigned)nbins);
    for (int i = threadIdx.x; i < nbuf; i += NT) {
        const uint32_t key = sm.buf_key[i];
        if ((key >> hs) != prefix) continue;
        atomicAdd(&sm.hist[(key >> shift) & (uint32_t)(nbins - 1)], 1);
    }
    __syncthreads();
}

// From the top bin down: the bin d where the running count first reaches `need`.  Returns d;
// *above = elements in bins > d, *at = elements in bin d, *total = all counted elements.
__device__ int find_digit(Smem &sm, int nbins, int need, int *above, int *at, int *total)
{
    // thread i owns bins (nbins-1 - 2i) and (nbins-2 - 2i): descending order over threads
    const int per = nbins / NT; // 2 or 1
    int mine = 0;
    int b0 = nbins - 1 - per * (int)threadIdx.x;
    for (int j = 0; j < per; ++j) mine += sm.hist[b0 - j];
    int tot;
    const int ex = block_exclusive_scan<NW>(mine, sm.scan, &tot);
    if (threadIdx.x == 0) {
        sm.misc[0] = -1;
        sm.misc[3] = tot;
    }
    __syncthreads();
    if (ex < need && ex + mine >= need) {
        int cum = ex;
        for (int j = 0; j < per; ++j) {
            const int c = sm.hist[b0 - j];
            if (cum + c >= need) {
                sm.misc[0] = b0 - j;
                sm.misc[1] = cum;
                sm.misc[2] = c;
                break;
            }
            cum += c;
        }
    }
    __syncthreads();
    const int d = sm.misc[0];
    *above = sm.misc[1];
    *at = sm.misc[2];
    *total = sm.misc[3];
    __syncthreads();
    return d;
}

// Ordered selection pass over the row: an element is taken iff key > T, or key == T and fewer
// than `eq_take` earlier elements had key == T (T == 0: every competing element).  Taken ids go
// to dst[0..) in position order, or into the LDS buffer when to_buf.  Returns the count taken.
__device__ int select_row(Smem &sm, const Row &r, uint32_t T, int eq_take, int32_t *dst,
                          bool to_buf, int limit)
{
    int taken = 0, eq_seen = 0;
    for (int64_t base = round_begin(r); base < r.hi && taken < limit; base += ROUND) {
        uint32_t key[ITEMS];
        int32_t id[ITEMS];
        load_items(r, base, key, id);
        int n_eq = 0;
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) n_eq += (key[j] && key[j] == T) ? 1 : 0;
        int eq_tot;
        const int eq_ex = block_exclusive_scan<NW>(n_eq, sm.scan, &eq_tot);
        bool take[ITEMS];
        int n_take = 0, eq_rank = eq_seen + eq_ex;
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            take[j] = false;
            if (!key[j]) continue;
            if (key[j] > T) take[j] = true;
            else if (key[j] == T) take[j] = (eq_rank++ < eq_take);
            n_take += take[j] ? 1 : 0;
        }
        int tot;
        int pos = taken + block_exclusive_scan<NW>(n_take, sm.scan, &tot);
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            if (!take[j]) continue;
            if (pos < limit) {
                if (to_buf) {
                    sm.buf_key[pos] = key[j];
                    sm.buf_id[pos] = id[j];
                } else {
                    dst[pos] = id[j];
                }
            }
            ++pos;
        }
        taken += tot;
        eq_seen += eq_tot;
    }
    return taken < limit ? taken : limit;
}

// The same over the LDS buffer (already in position order).
__device__ int select_buf(Smem &sm, int nbuf, uint32_t T, int eq_take, int32_t *dst, int limit)
{
    int taken = 0, eq_seen = 0;
    for (int base = 0; base < nbuf; base += NT) {
        const int i = base + threadIdx.x;
        const uint32_t key = i < nbuf ? sm.buf_key[i] : 0u;
        const int is_eq = (key && key == T) ? 1 : 0;
        int eq_tot;
        const int eq_ex = block_exclusive_scan<NW>(is_eq, sm.scan, &eq_tot);
        const bool take = key && (key > T || (is_eq && eq_seen + eq_ex < eq_take));
        int tot;
        const int pos = taken + block_exclusive_scan<NW>(take ? 1 : 0, sm.scan, &tot);
        if (take && pos < limit) dst[pos] = sm.buf_id[i];
        taken += tot;
        eq_seen += eq_tot;
    }
    return taken;
}

// Select `need` elements of the row by (key desc, position asc) into dst, ascending; pad -1.
__device__ void select_top(Smem &sm, const Row &r, int need, int32_t *dst)
{
    if (need <= 0) return;
    // level 0 over the row
    hist_row(sm, r, 21, 2048, 0, 0u);
    int above, at, total;
    int d = find_digit(sm, 2048, need, &above, &at, &total);
    if (total <= need) { // everything competes: take all, pad
        const int got = select_row(sm, r, 0u, 0, dst, false, need);
        for (int i = got + (int)threadIdx.x; i < need; i += NT) dst[i] = -1;
        return;
    }
    uint32_t prefix = (uint32_t)d;
    int pbits = 11;
    int need_rem = need - above;
    int taken_above = above;
    // Further digits: (shift, bits) = (10, 11), (0, 10).
    const int shifts[2] = {10, 0};
    const int bitsv[2] = {11, 10};
    bool in_buf = false;
    int nbuf = 0;
    for (int lvl = 0; lvl < 2; ++lvl) {
        if (!in_buf && taken_above + at <= CAP) {
            // compact every element with (key >> (32 - pbits)) >= prefix into LDS, in order
            const uint32_t lowest = prefix << (32 - pbits);
            nbuf = select_row(sm, r, lowest, INT32_MAX, nullptr, true, CAP);
            __syncthreads();
            in_buf = true;
        }
        const int sh = shifts[lvl], nb = 1 << bitsv[lvl];
        if (in_buf) hist_buf(sm, nbuf, sh, nb, prefix);
        else hist_row(sm, r, sh, nb, pbits, prefix);
        int a2, at2, tot2;
        d = find_digit(sm, nb, need_rem, &a2, &at2, &tot2);
        prefix = (prefix << bitsv[lvl]) | (uint32_t)d;
        pbits += bitsv[lvl];
        need_rem -= a2;
        taken_above += a2;
        at = at2;
    }
    // prefix is now the exact threshold key T; need_rem elements equal to T are taken.
    if (in_buf) select_buf(sm, nbuf, prefix, need_rem, dst, need);
    else select_row(sm, r, prefix, need_rem, dst, false, need);
}

__global__ __launch_bounds__(NT) void select_kernel(SelectArgs a)
{
    __shared__ Smem sm;
    const int64_t row = blockIdx.x;
    const int64_t t = row % a.n_q;
    int64_t V = a.q_pos0 + t + 1;
    if (V > a.kv_len) V = a.kv_len;
    int32_t *out = a.out + row * a.out_stride;
    Row r;
    r.sc = a.scores + row * a.n_in;
    r.ids = a.cand_ids ? a.cand_ids + row * a.n_in : nullptr;
    r.vec = (a.n_in % 4) == 0;

    if (a.mode == SELECT_SI) {
        if (V <= a.k) {
            for (int i = threadIdx.x; i < a.k; i += NT) out[i] = i < V ? i : -1;
            return;
        }
        for (int i = threadIdx.x; i < a.sink; i += NT) out[i] = i;
        for (int i = threadIdx.x; i < a.window; i += NT) out[a.sink + i] = (int32_t)(V - a.window + i);
        r.id_lo = a.sink;
        r.id_hi = V - a.window;
        if (r.ids) {
            r.lo = 0;
            r.hi = a.n_in;
        } else {
            r.lo = r.id_lo;
            r.hi = r.id_hi;
        }
        select_top(sm, r, a.k - a.sink - a.window, out + a.sink + a.window);
    } else { // SELECT_PAGES
        if (V <= a.k) {
            for (int i = threadIdx.x; i < a.m_pages; i += NT) out[i] = -1;
            return;
        }
        r.lo = r.id_lo = a.sink / a.page;
        r.hi = r.id_hi = (V - a.window - 1) / a.page + 1;
        select_top(sm, r, a.m_pages, out);
    }
}

} // namespace

hipError_t launch_select(const SelectArgs &a, hipStream_t stream)
{
    const int64_t rows = (int64_t)a.batch * a.n_q;
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(select_kernel, dim3((unsigned)rows), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

} // namespace lsa
