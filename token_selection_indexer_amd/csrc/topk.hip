// topk.hip -- per-query selection: Streaming-Aware Indexing (sink + local window + dynamic
// top-k) and the page-recall top-M of Hierarchical Indexing.
//
// (Model card, SI bullet: part of the budget goes to a fixed sink and a local sliding window, the
// rest to dynamic sparse selection; Baidu Cloud article, "2. Dynamic Token Selector": top-k of
// the score row.  Model card, HI bullet: candidate blocks are recalled by coarse scores.)
//
// Exact radix select on an order-preserving uint32 image of the fp32 scores (larger key = larger
// score, -0 == +0).  Ties go to the lower position, which is the lower token index because rows
// are in token order and candidate lists are ascending.  Picks are emitted by ordered compaction,
// so they come out ascending without a sort.  Sink [0,S) and window [V-W,V) are written
// arithmetically, never scored or compared.
//
// A sampled threshold makes the common case one pass over long rows: 64-element blocks spread
// over the row give T (from the sampled key of a rank that puts about twice the needed count of
// the row at or above T); every element >= T is compacted (in position order) into LDS, and the
// exact selection runs there -- the buffer then holds every element that can be picked, ties at
// the boundary included.  When fewer than the needed count, or more than the buffer holds, reach
// T, the exact histogram path below runs instead, so T affects speed only.
//
// Two paths:
//  * one workgroup per row (many rows: prefill, page recall):
//      rows of 32K and more: the sampled threshold as above; otherwise, or if it fails,
//      1. histogram of key bits 31..21 (2048 bins in LDS) over the row;
//      2. the bin b* holding the k-th key; bins above are taken outright;
//      3. if bins >= b* fit in LDS, one ordered pass compacts them there and bits 20..10, 9..0
//         are resolved in LDS; otherwise the next digit is histogrammed from the row again;
//      4. keys > T, then the first (k - #greater) keys == T, in position order.
//  * chunked (few long rows: decode): the row is cut into 4096-element chunks, one workgroup
//    each, so a handful of rows still fills the chip:
//      collect   every chunk derives the row's sampled threshold (the same in every chunk) and
//                compacts its elements >= T (in order) into its own slice of the workspace
//      finish    one workgroup per row concatenates the slices (chunk order = position order)
//                into LDS and selects exactly there; a row whose slices overflowed, or hold
//                fewer than the needed count, falls back to the one-workgroup path over the row.
#include "device.hpp"
#include "internal.hpp"

namespace lsa {
namespace {

constexpr int NBIN = 2048;          // 11-bit digits
constexpr int CAP = 8192;           // LDS candidate buffer entries (key, id)
constexpr int CHUNK = 4096;         // chunked path: elements per workgroup
constexpr int CHUNK_CAP = 512;      // chunked path: candidates kept per chunk
constexpr int CNT_THREADS = 256;    // chunked path: threads per chunk workgroup
constexpr int64_t SAMPLE_MIN = 32768; // one-workgroup rows at least this long use the sample

// ------------------------------------------------------------------------------------------
// Row access
// ------------------------------------------------------------------------------------------

// A row's competing elements: positions [lo, hi) of `sc` (and `ids` in candidate mode); an
// element competes iff its id lies in [id_lo, id_hi).  Position order is id order.
struct Row {
    const float *sc;
    const int32_t *ids; // nullptr: id = position
    int64_t lo, hi;
    int64_t id_lo, id_hi;
    bool vec;           // rows start 16-byte aligned: 4-element vector loads
};

// Elements p .. p+3 (p a multiple of 4) below `hi` (<= r.hi): keys (0 = does not compete) and
// ids.
__device__ __forceinline__ void elem4(const Row &r, int64_t p, uint32_t (&key)[4], int32_t (&id)[4],
                                      int64_t hi)
{
    if (r.vec && p >= r.lo && p + 4 <= hi) {
        const float4 v = *reinterpret_cast<const float4 *>(r.sc + p);
        const float f[4] = {v.x, v.y, v.z, v.w};
        int32_t c[4];
        if (r.ids) {
            const int4 iv = *reinterpret_cast<const int4 *>(r.ids + p);
            c[0] = iv.x; c[1] = iv.y; c[2] = iv.z; c[3] = iv.w;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) c[j] = (int32_t)(p + j);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            id[j] = c[j];
            key[j] = (c[j] >= r.id_lo && c[j] < r.id_hi) ? order_key(f[j]) : 0u;
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t q = p + j;
        if (q < r.lo || q >= hi) {
            id[j] = -1;
            key[j] = 0u;
            continue;
        }
        const int32_t c = r.ids ? r.ids[q] : (int32_t)q;
        id[j] = c;
        key[j] = (c >= r.id_lo && c < r.id_hi) ? order_key(r.sc[q]) : 0u;
    }
}

// Elements p .. p+3 (p a multiple of 4) below `hi` (<= r.hi) as raw scores, -inf for elements
// that do not compete, plus (candidate rows) their ids.  For a finite threshold t,
// "key(f) >= T" is "f >= t" (order_key is monotone and equates -0 with +0, as float comparison
// does), so a pass against a threshold needs no key per element.
__device__ __forceinline__ void elem4f(const Row &r, int64_t p, float (&f)[4], int32_t (&id)[4],
                                       int64_t hi)
{
    if (r.vec && p >= r.lo && p + 4 <= hi) {
        const float4 v = *reinterpret_cast<const float4 *>(r.sc + p);
        f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
        if (r.ids) {
            const int4 iv = *reinterpret_cast<const int4 *>(r.ids + p);
            id[0] = iv.x; id[1] = iv.y; id[2] = iv.z; id[3] = iv.w;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (!(id[j] >= r.id_lo && id[j] < r.id_hi)) f[j] = -INFINITY;
        }
        return; // flat rows: every position in [lo, hi) competes, id = position
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t q = p + j;
        f[j] = -INFINITY;
        id[j] = -1;
        if (q < r.lo || q >= hi) continue;
        const int32_t c = r.ids ? r.ids[q] : (int32_t)q;
        id[j] = c;
        if (c >= r.id_lo && c < r.id_hi) f[j] = r.sc[q];
    }
}

// The float whose order key is T (the smallest float f with key(f) >= T).
__device__ __forceinline__ float key_to_float(uint32_t T)
{
    return __uint_as_float((T & 0x80000000u) ? (T & 0x7fffffffu) : ~T);
}

// Element at position p: (key, id); key 0 = does not compete.
__device__ __forceinline__ uint32_t elem(const Row &r, int64_t p, int32_t &id)
{
    if (p < r.lo || p >= r.hi) {
        id = -1;
        return 0u;
    }
    const int32_t c = r.ids ? r.ids[p] : (int32_t)p;
    id = c;
    if (c < r.id_lo || c >= r.id_hi) return 0u;
    return order_key(r.sc[p]);
}

// Exclusive position of flagged items in (item, wave, lane) order -- which is position order
// when item j of thread t sits at base + j*NT + t.  cnt holds ITEMS*NT/64 ints of LDS.
// Barriers inside: every thread of the block must call it.
template <int NT, int ITEMS>
__device__ __forceinline__ void ordered_slots(const bool (&flag)[ITEMS], int (&slot)[ITEMS],
                                              int *cnt, int &total)
{
    constexpr int NW = NT / kWave;
    static_assert(ITEMS * NW <= kWave, "one wave scans the per-(item, wave) counts");
    const int lane = lane_id(), w = wave_id();
    uint64_t m[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        m[j] = __ballot(flag[j]);
        if (lane == 0) cnt[j * NW + w] = __popcll(m[j]);
    }
    __syncthreads();
    const int c = lane < ITEMS * NW ? cnt[lane] : 0;
    const int inc = wave_inclusive_scan(c);
    total = __shfl(inc, ITEMS * NW - 1, kWave);
    const int ex = inc - c;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const int base = __shfl(ex, j * NW + w, kWave);
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m[j] >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m[j], 0u));
        slot[j] = flag[j] ? base + below : -1;
    }
    __syncthreads();
}

// From the top bin down: the bin where the running count first reaches `need`.
struct Digit {
    int d, above, at, total;
};

template <int NT>
__device__ __forceinline__ Digit find_digit(const int *hist, int nbins, int need, int *scratch)
{
    // thread i owns bins [nbins - (i+1)*per, nbins - i*per), scanned top-down (with fewer bins
    // than threads, threads past the last bin own none)
    const int per = nbins >= NT ? nbins / NT : 1;
    const bool owner = (int)threadIdx.x * per < nbins;
    const int top = nbins - 1 - per * (int)threadIdx.x;
    int mine = 0;
    if (owner)
        for (int j = 0; j < per; ++j) mine += hist[top - j];
    int tot;
    const int ex = block_exclusive_scan<NT / kWave>(mine, scratch, &tot);
    if (threadIdx.x == 0) scratch[NT / kWave + 1] = -1;
    __syncthreads();
    if (owner && ex < need && ex + mine >= need) {
        int cum = ex;
        for (int j = 0; j < per; ++j) {
            const int c = hist[top - j];
            if (cum + c >= need) {
                scratch[NT / kWave + 1] = top - j;
                scratch[NT / kWave + 2] = cum;
                scratch[NT / kWave + 3] = c;
                break;
            }
            cum += c;
        }
    }
    __syncthreads();
    Digit r;
    r.d = scratch[NT / kWave + 1];
    r.above = scratch[NT / kWave + 2];
    r.at = scratch[NT / kWave + 3];
    r.total = tot;
    __syncthreads();
    return r;
}

// Threshold from a sample of the row.  NTH/64 * KPT blocks of 64 consecutive positions, evenly
// spread over [lo, hi) (len = hi - lo > 64 * blocks), are read; T is the lower edge of the
// 22-bit key prefix holding the rr-th largest sampled key, rr = 2 * need * (sampled / len) + 8,
// so about twice `need` elements of the row are expected at or above T.  Returns 0 when the
// sample has fewer than rr competing keys.  The caller checks what it collects against T (at
// least `need`, within capacity) and falls back to the exact histogram path otherwise, so T
// only ever affects speed, never the result.  Every workgroup computing T for the same row
// gets the same T.  `hist` holds NBIN ints.
template <int NTH, int KPT>
__device__ __forceinline__ uint32_t sample_threshold(int *hist, int *scratch, const Row &r, int need,
                                                     int64_t len)
{
    constexpr int NWV = NTH / kWave;
    constexpr int NSB = NWV * KPT; // sample blocks
    const int l = lane_id(), wv = wave_id();
    uint32_t key[KPT];
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const int sb = j * NWV + wv;
        const int64_t start = r.lo + (len - kWave) * sb / (NSB - 1);
        int32_t id;
        key[j] = elem(r, start + l, id);
        cnt += key[j] != 0u;
    }
    int m;
    block_exclusive_scan<NWV>(cnt, scratch, &m);
    const int64_t ns = (int64_t)NSB * kWave;
    const int64_t want = (2 * (int64_t)need * ns + len - 1) / len + 8;
    if (want > m) return 0u;
    int rem = (int)want;
    uint32_t prefix = 0u;
    // two 11-bit digits (key bits 31..21, then 20..10)
    for (int lvl = 0; lvl < 2; ++lvl) {
        const int shift = 21 - 11 * lvl;
        for (int i = threadIdx.x; i < NBIN; i += NTH) hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < KPT; ++j)
            if (key[j] && (lvl == 0 || (key[j] >> 21) == prefix))
                atomicAdd(&hist[(key[j] >> shift) & (NBIN - 1)], 1);
        __syncthreads();
        const Digit g = find_digit<NTH>(hist, NBIN, rem, scratch);
        prefix = (prefix << 11) | (uint32_t)g.d;
        rem -= g.above;
    }
    // passes compare floats against T: keep it above the key of -inf (always so for finite
    // sampled scores; a -inf threshold would also admit elements that do not compete)
    const uint32_t T = prefix << 10;
    return T > order_key(-INFINITY) ? T : 0u;
}

// ------------------------------------------------------------------------------------------
// One workgroup per row
// ------------------------------------------------------------------------------------------

constexpr int NT = 1024;
constexpr int NW = NT / kWave;
constexpr int ITEMS = 4;
constexpr int ROUND = NT * ITEMS;

struct Smem {
    int hist[NBIN];
    int scratch[NW + 8];
    int cnt[ITEMS * NW];
    uint32_t buf_key[CAP];
    int32_t buf_id[CAP];
};

__device__ __forceinline__ int64_t round_begin(const Row &r) { return r.lo; }

__device__ __forceinline__ void clear_hist(Smem &sm)
{
    for (int i = threadIdx.x; i < NBIN; i += NT) sm.hist[i] = 0;
    __syncthreads();
}

// Histogram of digit (key >> shift) & (nbins-1) over the row's elements whose bits above the
// digit equal `prefix` (all elements when pbits == 0).
__device__ __forceinline__ void hist_row(Smem &sm, const Row &r, int shift, int nbins, int pbits,
                                         uint32_t prefix)
{
    clear_hist(sm);
    const int hs = shift + __builtin_ctz((unsigned)nbins);
    for (int64_t base = round_begin(r); base < r.hi; base += ROUND) {
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            int32_t id;
            const uint32_t key = elem(r, base + (int64_t)j * NT + threadIdx.x, id);
            if (!key) continue;
            if (pbits && (hs >= 32 ? 0u : (key >> hs)) != prefix) continue;
            atomicAdd(&sm.hist[(key >> shift) & (uint32_t)(nbins - 1)], 1);
        }
    }
    __syncthreads();
}

// pbits == 0: every buffered key counts (the level-0 digit).
__device__ __forceinline__ void hist_buf(Smem &sm, int nbuf, int shift, int nbins, uint32_t prefix,
                                         int pbits = 1)
{
    clear_hist(sm);
    const int hs = shift + __builtin_ctz((unsigned)nbins);
    for (int i = threadIdx.x; i < nbuf; i += NT) {
        const uint32_t key = sm.buf_key[i];
        if (pbits && (key >> hs) != prefix) continue;
        atomicAdd(&sm.hist[(key >> shift) & (uint32_t)(nbins - 1)], 1);
    }
    __syncthreads();
}

// Ordered pass over the row: take key > T, or key == T while fewer than eq_take earlier
// elements had key == T.  Taken ids go to dst (or into the LDS buffer).  Returns the count.
__device__ __forceinline__ int select_row(Smem &sm, const Row &r, uint32_t T, int eq_take, int32_t *dst,
                          bool to_buf, int limit)
{
    int taken = 0, eq_seen = 0;
    for (int64_t base = round_begin(r); base < r.hi && taken < limit; base += ROUND) {
        uint32_t key[ITEMS];
        int32_t id[ITEMS];
        bool is_eq[ITEMS], take[ITEMS];
        int eq_slot[ITEMS], slot[ITEMS];
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            key[j] = elem(r, base + (int64_t)j * NT + threadIdx.x, id[j]);
            is_eq[j] = key[j] && key[j] == T;
        }
        int eq_tot;
        ordered_slots<NT, ITEMS>(is_eq, eq_slot, sm.cnt, eq_tot);
#pragma unroll
        for (int j = 0; j < ITEMS; ++j)
            take[j] = key[j] && (key[j] > T || (is_eq[j] && eq_seen + eq_slot[j] < eq_take));
        int tot;
        ordered_slots<NT, ITEMS>(take, slot, sm.cnt, tot);
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const int pos = taken + slot[j];
            if (!take[j] || pos >= limit) continue;
            if (to_buf) {
                sm.buf_key[pos] = key[j];
                sm.buf_id[pos] = id[j];
            } else {
                dst[pos] = id[j];
            }
        }
        taken += tot;
        eq_seen += eq_tot;
    }
    return taken; // may exceed limit: only the first `limit` were written
}

// The same over the LDS buffer (already in position order).
__device__ __forceinline__ int select_buf(Smem &sm, int nbuf, uint32_t T, int eq_take, int32_t *dst,
                                          int limit)
{
    int taken = 0, eq_seen = 0;
    for (int base = 0; base < nbuf; base += ROUND) {
        uint32_t key[ITEMS];
        bool is_eq[ITEMS], take[ITEMS];
        int eq_slot[ITEMS], slot[ITEMS];
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const int i = base + j * NT + threadIdx.x;
            key[j] = i < nbuf ? sm.buf_key[i] : 0u;
            is_eq[j] = key[j] && key[j] == T;
        }
        int eq_tot;
        ordered_slots<NT, ITEMS>(is_eq, eq_slot, sm.cnt, eq_tot);
#pragma unroll
        for (int j = 0; j < ITEMS; ++j)
            take[j] = key[j] && (key[j] > T || (is_eq[j] && eq_seen + eq_slot[j] < eq_take));
        int tot;
        ordered_slots<NT, ITEMS>(take, slot, sm.cnt, tot);
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const int pos = taken + slot[j];
            if (take[j] && pos < limit) dst[pos] = sm.buf_id[base + j * NT + threadIdx.x];
        }
        taken += tot;
        eq_seen += eq_tot;
    }
    return taken;
}

// The buffer holds, in position order, every element whose top `pbits` key bits are >= prefix
// (pbits == 11).  Resolve the remaining digits and emit `need` picks.
__device__ __forceinline__ void finish_in_buf(Smem &sm, int nbuf, uint32_t prefix, int need_rem,
                                              int32_t *dst,
                              int need)
{
    const int shifts[2] = {10, 0};
    const int bitsv[2] = {11, 10};
    for (int lvl = 0; lvl < 2; ++lvl) {
        hist_buf(sm, nbuf, shifts[lvl], 1 << bitsv[lvl], prefix);
        const Digit g = find_digit<NT>(sm.hist, 1 << bitsv[lvl], need_rem, sm.scratch);
        prefix = (prefix << bitsv[lvl]) | (uint32_t)g.d;
        need_rem -= g.above;
    }
    select_buf(sm, nbuf, prefix, need_rem, dst, need);
}

// The buffer holds, in position order, a set of elements that contains the row's `need` best.
// Emit exactly those (all of them, padded with -1, if there are at most `need`).
__device__ __forceinline__ void select_in_buf(Smem &sm, int nbuf, int need, int32_t *dst)
{
    if (nbuf <= need) {
        const int got = select_buf(sm, nbuf, 0u, 0, dst, need);
        for (int i = got + (int)threadIdx.x; i < need; i += NT) dst[i] = -1;
        return;
    }
    hist_buf(sm, nbuf, 21, NBIN, 0u, 0);
    const Digit g = find_digit<NT>(sm.hist, NBIN, need, sm.scratch);
    finish_in_buf(sm, nbuf, (uint32_t)g.d, need - g.above, dst, need);
}

// ---- streaming passes: each wave owns a contiguous segment of the row (no block barriers) ----

constexpr int WCAP = CAP / NW; // candidate list entries per wave

struct Seg {
    int64_t b0, b1; // [b0, b1): multiples of 4, covering the wave's part of [lo, hi)
};

__device__ __forceinline__ Seg wave_segment(const Row &r)
{
    const int64_t a0 = r.lo & ~int64_t(3);
    const int64_t n = r.hi - a0;
    const int64_t seg = ((n + NW - 1) / NW + 255) / 256 * 256;
    Seg s;
    s.b0 = a0 + (int64_t)wave_id() * seg;
    s.b1 = min(s.b0 + seg, r.hi);
    return s;
}

// Level-0 histogram (key bits 31..21) of the row.
__device__ __forceinline__ void hist_row_seg(Smem &sm, const Row &r)
{
    clear_hist(sm);
    const Seg sg = wave_segment(r);
    const int64_t whi = min(r.hi, sg.b1); // this wave's part of the row ends here
    constexpr int U = 4; // 4 x 1 KB of the segment in flight per wave
    for (int64_t p0 = sg.b0; p0 < sg.b1; p0 += U * 4 * kWave) {
        uint32_t key[U][4];
        int32_t id[U][4];
        static_for<0, U>([&](auto UI) {
            constexpr int u = decltype(UI)::value;
            elem4(r, p0 + u * 4 * kWave + 4 * lane_id(), key[u], id[u], whi);
        });
        static_for<0, U>([&](auto UI) {
            constexpr int u = decltype(UI)::value;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (key[u][j]) atomicAdd(&sm.hist[key[u][j] >> 21], 1);
        });
    }
    __syncthreads();
}

// Every element with key >= lowest, into the LDS buffer in position order.  Each wave appends
// its segment's elements to its own list (order kept by a wave prefix sum), then the lists are
// concatenated in wave order.  Returns false if a wave's list overflowed (caller falls back).
__device__ __forceinline__ bool collect_row_seg(Smem &sm, const Row &r, uint32_t lowest, int &nbuf,
                                                int &total_out)
{
    const int w = wave_id(), lane = lane_id();
    const Seg sg = wave_segment(r);
    const int64_t whi = min(r.hi, sg.b1); // this wave's part ends here; later positions read as
                                          // "does not compete"
    const int base = w * WCAP;
    const float tf = key_to_float(lowest);
    if (!(tf > -INFINITY)) { // threshold at or below -inf (only with -inf scores): the caller's
        total_out = 0;        // key-based ordered pass collects instead
        return false;
    }
    int cnt = 0;
    // The trip count is uniform over the wave (the scan below needs every lane).  U steps of
    // 4 x 64 elements are loaded before any is appended, so 4 KB per wave are in flight; the
    // steps are then appended in position order.  Elements are compared as floats; keys are
    // formed only for the few that are kept.
    constexpr int U = 4;
    for (int64_t p0 = sg.b0; p0 < sg.b1; p0 += U * 4 * kWave) {
        float fv[U][4];
        int32_t id[U][4];
        static_for<0, U>([&](auto UI) {
            constexpr int u = decltype(UI)::value;
            elem4f(r, p0 + u * 4 * kWave + 4 * lane, fv[u], id[u], whi);
        });
        // (static_for: the compiler does not unroll loops holding wave scans, and a rolled loop
        // would index the key arrays dynamically, i.e. from scratch memory)
        static_for<0, U>([&](auto UI) {
            constexpr int u = decltype(UI)::value;
            // position among the wave's kept elements in (lane, j) order: one ballot per j
            // (flags of lanes below this one via mbcnt), no scan
            bool fl[4];
            uint64_t m[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                fl[j] = fv[u][j] >= tf;
                m[j] = __ballot(fl[j]);
            }
            if ((m[0] | m[1] | m[2] | m[3]) == 0) return;
            int below = 0, tot = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                below += __builtin_amdgcn_mbcnt_hi((uint32_t)(m[j] >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m[j], 0u));
                tot += __popcll(m[j]);
            }
            int pos = cnt + below;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (!fl[j]) continue;
                if (pos < WCAP) {
                    sm.buf_key[base + pos] = order_key(fv[u][j]);
                    sm.buf_id[base + pos] =
                        r.ids ? id[u][j] : (int32_t)(p0 + u * 4 * kWave + 4 * lane + j);
                }
                ++pos;
            }
            cnt += tot;
        });
    }
    if (lane == 0) sm.cnt[w] = cnt;
    __syncthreads();
    int off = 0, total = 0, over = 0;
    for (int u = 0; u < NW; ++u) {
        const int c = sm.cnt[u];
        if (u < w) off += c;
        total += c;
        over |= c > WCAP;
    }
    total_out = total;
    if (over || total > CAP) {
        __syncthreads();
        return false;
    }
    // concatenate: lists are read into registers first, so no list is overwritten unread
    constexpr int PER = WCAP / kWave;
    uint32_t k[PER];
    int32_t id[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + i * kWave;
        k[i] = e < cnt ? sm.buf_key[base + e] : 0u;
        id[i] = e < cnt ? sm.buf_id[base + e] : 0;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + i * kWave;
        if (e < cnt) {
            sm.buf_key[off + e] = k[i];
            sm.buf_id[off + e] = id[i];
        }
    }
    __syncthreads();
    nbuf = total;
    return true;
}

// Select `need` elements of the row by (key desc, position asc) into dst, ascending; pad -1.
__device__ __forceinline__ void select_top(Smem &sm, const Row &r, int need, int32_t *dst)
{
    if (need <= 0) return;
    const int64_t len = r.hi - r.lo;
    // long rows: a sampled threshold lets one pass collect everything at or above it
    const uint32_t T =
        len >= SAMPLE_MIN ? sample_threshold<NT, 4>(sm.hist, sm.scratch, r, need, len) : 0u;
    if (T != 0u) {
        int nbuf = 0, total = 0;
        bool ok = collect_row_seg(sm, r, T, nbuf, total);
        if (!ok && total <= CAP) { // a wave's list overflowed, the buffer would not: ordered pass
            nbuf = select_row(sm, r, T, INT32_MAX, nullptr, true, CAP);
            __syncthreads();
            ok = true;
        }
        if (ok && nbuf >= need) {
            select_in_buf(sm, nbuf, need, dst);
            return;
        }
    }
    // exact histogram path
    hist_row_seg(sm, r);
    Digit g = find_digit<NT>(sm.hist, NBIN, need, sm.scratch);
    if (g.total <= need) { // everything competes: take all, pad
        const int got = min(select_row(sm, r, 0u, 0, dst, false, need), need);
        for (int i = got + (int)threadIdx.x; i < need; i += NT) dst[i] = -1;
        return;
    }
    uint32_t prefix = (uint32_t)g.d;
    int pbits = 11;
    int need_rem = need - g.above;
    int taken_above = g.above, at = g.at;
    if (taken_above + at <= CAP) {
        int nbuf, total;
        if (!collect_row_seg(sm, r, prefix << 21, nbuf, total)) { // uneven segments: ordered pass
            nbuf = select_row(sm, r, prefix << 21, INT32_MAX, nullptr, true, CAP);
            __syncthreads();
        }
        finish_in_buf(sm, nbuf, prefix, need_rem, dst, need);
        return;
    }
    // heavy ties: refine the threshold from the row itself
    const int shifts[2] = {10, 0};
    const int bitsv[2] = {11, 10};
    for (int lvl = 0; lvl < 2; ++lvl) {
        hist_row(sm, r, shifts[lvl], 1 << bitsv[lvl], pbits, prefix);
        const Digit h = find_digit<NT>(sm.hist, 1 << bitsv[lvl], need_rem, sm.scratch);
        prefix = (prefix << bitsv[lvl]) | (uint32_t)h.d;
        pbits += bitsv[lvl];
        need_rem -= h.above;
        taken_above += h.above;
    }
    select_row(sm, r, prefix, need_rem, dst, false, need);
}

// Row setup shared by both paths.  Returns false when the row needs no selection (all of it
// written already).
__device__ __forceinline__ bool setup_row(const SelectArgs &a, int64_t row, Row &r, int32_t *&dst,
                                          int &need,
                          bool write_fixed)
{
    const int64_t t = row % a.n_q;
    int64_t V = a.q_pos0 + t + 1;
    if (V > a.kv_len) V = a.kv_len;
    int32_t *out = a.out + row * a.out_stride;
    r.sc = a.scores + row * a.n_in;
    r.ids = a.cand_ids ? a.cand_ids + row * a.n_in : nullptr;
    r.vec = (a.n_in % 4) == 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0 &&
            (!a.cand_ids || (reinterpret_cast<uintptr_t>(a.cand_ids) & 15) == 0);
    if (a.mode == SELECT_SI) {
        if (V <= a.k) {
            if (write_fixed)
                for (int i = threadIdx.x; i < a.k; i += blockDim.x) out[i] = i < V ? i : -1;
            return false;
        }
        if (write_fixed) {
            for (int i = threadIdx.x; i < a.sink; i += blockDim.x) out[i] = i;
            for (int i = threadIdx.x; i < a.window; i += blockDim.x)
                out[a.sink + i] = (int32_t)(V - a.window + i);
        }
        r.id_lo = a.sink;
        r.id_hi = V - a.window;
        if (r.ids) {
            r.lo = 0;
            r.hi = a.n_in;
        } else {
            r.lo = r.id_lo;
            r.hi = r.id_hi;
        }
        dst = out + a.sink + a.window;
        need = a.k - a.sink - a.window;
    } else { // SELECT_PAGES
        if (V <= a.k) {
            if (write_fixed)
                for (int i = threadIdx.x; i < a.m_pages; i += blockDim.x) out[i] = -1;
            return false;
        }
        r.lo = r.id_lo = a.sink / a.page;
        r.hi = r.id_hi = (V - a.window - 1) / a.page + 1;
        dst = out;
        need = a.m_pages;
    }
    return need > 0;
}

__global__ __launch_bounds__(NT) void select_kernel(SelectArgs a)
{
    __shared__ Smem sm;
    Row r;
    int32_t *dst;
    int need;
    if (!setup_row(a, blockIdx.x, r, dst, need, true)) return;
    select_top(sm, r, need, dst);
}

// ------------------------------------------------------------------------------------------
// Chunked path
// ------------------------------------------------------------------------------------------

struct ChunkWs {
    int *count;      // [rows][n_chunks]  (CHUNK_CAP + 1 = overflow or no threshold)
    uint32_t *ckey;  // [rows][n_chunks][CHUNK_CAP]
    int32_t *cid;    // [rows][n_chunks][CHUNK_CAP]
    int n_chunks;
};

// Every chunk of a row derives the row's sampled threshold T (the same T in every workgroup)
// and compacts its elements with key >= T, in position order, into its slice of the workspace.
__global__ __launch_bounds__(CNT_THREADS) void chunk_collect_kernel(SelectArgs a, ChunkWs ws)
{
    constexpr int CI = CHUNK / CNT_THREADS; // items per thread
    __shared__ int hist[NBIN];
    __shared__ int scratch[CNT_THREADS / kWave + 8];
    __shared__ int cnt[kWave];
    const int64_t row = blockIdx.y;
    const int chunk = blockIdx.x;
    Row r;
    int32_t *dst;
    int need;
    if (!setup_row(a, row, r, dst, need, false)) return;
    int *cntp = ws.count + row * ws.n_chunks + chunk;
    // 1024 samples up to 256K positions, 4096 beyond (the expected sampled rank stays >= 16)
    const int64_t len = r.hi - r.lo;
    const uint32_t T = len <= (int64_t)1 << 18
                           ? sample_threshold<CNT_THREADS, 4>(hist, scratch, r, need, len)
                           : sample_threshold<CNT_THREADS, 16>(hist, scratch, r, need, len);
    if (T == 0u) { // no usable threshold: the finish kernel falls back to the exact path
        if (threadIdx.x == 0) *cntp = CHUNK_CAP + 1;
        return;
    }
    const int64_t c0 = (int64_t)chunk * CHUNK;
    if (c0 + CHUNK <= r.lo || c0 >= r.hi) {
        if (threadIdx.x == 0) *cntp = 0;
        return;
    }
    uint32_t *okey = ws.ckey + (row * ws.n_chunks + chunk) * CHUNK_CAP;
    int32_t *oid = ws.cid + (row * ws.n_chunks + chunk) * CHUNK_CAP;
    // CI items per thread: item j of thread t is element c0 + j*CNT_THREADS + t
    uint32_t key[CI];
    int32_t id[CI];
    bool take[CI];
    int slot[CI];
    const float tf = key_to_float(T);
#pragma unroll
    for (int j = 0; j < CI; ++j) {
        const int64_t p = c0 + (int64_t)j * CNT_THREADS + threadIdx.x;
        float f = -INFINITY;
        id[j] = -1;
        if (p >= r.lo && p < r.hi) {
            id[j] = r.ids ? r.ids[p] : (int32_t)p;
            if (id[j] >= r.id_lo && id[j] < r.id_hi) f = r.sc[p];
        }
        take[j] = f >= tf;
        key[j] = take[j] ? order_key(f) : 0u;
    }
    int taken;
    ordered_slots<CNT_THREADS, CI>(take, slot, cnt, taken);
#pragma unroll
    for (int j = 0; j < CI; ++j) {
        if (take[j] && slot[j] < CHUNK_CAP) {
            okey[slot[j]] = key[j];
            oid[slot[j]] = id[j];
        }
    }
    if (threadIdx.x == 0) *cntp = taken > CHUNK_CAP ? CHUNK_CAP + 1 : taken;
}

__global__ __launch_bounds__(NT) void chunk_finish_kernel(SelectArgs a, ChunkWs ws)
{
    __shared__ Smem sm;
    const int64_t row = blockIdx.x;
    Row r;
    int32_t *dst;
    int need;
    if (!setup_row(a, row, r, dst, need, true)) return;
    // slice offsets (exclusive scan of the counts) into sm.hist, which is free until the end
    const int *counts = ws.count + row * ws.n_chunks;
    int overflow = 0, total = 0;
    for (int base = 0; base < ws.n_chunks; base += NT) {
        const int i = base + threadIdx.x;
        const int c = i < ws.n_chunks ? counts[i] : 0;
        overflow |= c > CHUNK_CAP;
        int tot;
        const int ex = block_exclusive_scan<NW>(c > CHUNK_CAP ? 0 : c, sm.scratch, &tot);
        if (i < ws.n_chunks) sm.hist[i] = total + ex;
        total += tot;
    }
    __syncthreads();
    // copy the slices in chunk order: one wave per slice, coalesced
    if (total <= CAP) {
        for (int i = wave_id(); i < ws.n_chunks; i += NW) {
            const int c = counts[i];
            if (c > CHUNK_CAP) continue;
            const int off = sm.hist[i];
            const uint32_t *ck = ws.ckey + (row * ws.n_chunks + i) * CHUNK_CAP;
            const int32_t *ci = ws.cid + (row * ws.n_chunks + i) * CHUNK_CAP;
            for (int e = lane_id(); e < c; e += kWave) {
                sm.buf_key[off + e] = ck[e];
                sm.buf_id[off + e] = ci[e];
            }
        }
    }
    overflow = __syncthreads_or(overflow);
    // the slices hold every element >= T of the row; enough of them contain the `need` best
    if (overflow || total > CAP || total < need) { // fall back to the one-workgroup path
        select_top(sm, r, need, dst);
        return;
    }
    select_in_buf(sm, total, need, dst);
}

bool use_chunked(const SelectArgs &a)
{
    const int64_t rows = (int64_t)a.batch * a.n_q;
    return a.mode == SELECT_SI && rows < 1024 && a.n_in >= 8 * CHUNK &&
           (a.n_in + CHUNK - 1) / CHUNK <= NBIN;
}

} // namespace

size_t select_workspace_bytes(int64_t rows, int64_t n_in, int mode)
{
    SelectArgs a{};
    a.batch = (int)rows;
    a.n_q = 1;
    a.n_in = n_in;
    a.mode = mode;
    if (!use_chunked(a)) return 0;
    const int64_t nc = (n_in + CHUNK - 1) / CHUNK;
    auto r256 = [](size_t x) { return (x + 255) / 256 * 256; };
    return r256(rows * nc * 4) + 2 * r256(rows * nc * CHUNK_CAP * 4);
}

hipError_t launch_select(const SelectArgs &a, void *ws, hipStream_t stream)
{
    const int64_t rows = (int64_t)a.batch * a.n_q;
    if (rows == 0) return hipSuccess;
    if (!use_chunked(a)) {
        hipLaunchKernelGGL(select_kernel, dim3((unsigned)rows), dim3(NT), 0, stream, a);
        return hipGetLastError();
    }
    const int64_t nc = (a.n_in + CHUNK - 1) / CHUNK;
    auto r256 = [](size_t x) { return (x + 255) / 256 * 256; };
    uint8_t *p = static_cast<uint8_t *>(ws);
    ChunkWs w;
    w.count = reinterpret_cast<int *>(p);
    p += r256(rows * nc * 4);
    w.ckey = reinterpret_cast<uint32_t *>(p);
    p += r256(rows * nc * CHUNK_CAP * 4);
    w.cid = reinterpret_cast<int32_t *>(p);
    w.n_chunks = (int)nc;
    hipLaunchKernelGGL(chunk_collect_kernel, dim3((unsigned)nc, (unsigned)rows), dim3(CNT_THREADS),
                       0, stream, a, w);
    hipLaunchKernelGGL(chunk_finish_kernel, dim3((unsigned)rows), dim3(NT), 0, stream, a, w);
    return hipGetLastError();
}

} // namespace lsa
