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
// Every path ends the same way: a position-ordered set of the row's elements that contains its
// best lies in an LDS buffer (8192 entries), and the exact selection runs there.  Bins over the
// buffer's own range are refined (first linear in the score when the keys span many binades,
// then 11-bit digits of the key offset from the least key) until the bin holding the k-th key
// has at most 64 keys; one wave ranks those exactly, which fixes the threshold key T and how many
// copies of T are taken; one ordered emission writes the picks.
//
// Getting the buffer:
//  * one workgroup per row (many rows: prefill, page recall; also a fallback of the chunked
//    path):
//      rows that fit the buffer are copied into it as they are;
//      rows of 16K and more: a sampled threshold T (64-element blocks spread over the row; T is
//      the sampled key of a rank that puts about twice the needed count of the row at or above
//      it) lets one ordered pass compact every element >= T, ties at the boundary included;
//      otherwise, or when fewer than the needed count or more than the buffer holds reach T, a
//      histogram of key bits 31..21 over the row finds the bin of the k-th key and one ordered
//      pass compacts the bins at and above it (with heavy ties beyond the buffer, further digits
//      are histogrammed from the row and the picks written directly).
//  * chunked (few long rows: decode): the row is cut into 4096-element chunks, one workgroup
//    each, so a handful of rows still fills the chip:
//      collect   every chunk derives the row's sampled threshold (the same in every chunk) and
//                compacts its elements >= T (in order) into its own slice of the workspace
//      finish    one workgroup per row concatenates the slices (chunk order = position order)
//                into the buffer; a row whose slices overflowed, or hold fewer than the needed
//                count, falls back to the one-workgroup path over the row.
// A threshold only ever decides what reaches the buffer, never the result.
#include "device.hpp"
#include "internal.hpp"

#include <mutex>

namespace lsa {
namespace {

constexpr int NBIN = 2048;          // 11-bit digits
constexpr int CAP = 8192;           // LDS candidate buffer entries (key, id)
constexpr int CHUNK = 4096;         // chunked path: elements per workgroup
constexpr int CHUNK_CAP = 512;      // chunked path: candidates kept per chunk
constexpr int CNT_THREADS = 256;    // chunked path: threads per chunk workgroup
constexpr int64_t SAMPLE_MIN = 8192;  // one-workgroup rows longer than the buffer use the sample

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
        const uint4 v = ld16_nt(r.sc + p); // streaming pass: read once
        f[0] = __uint_as_float(v.x);
        f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z);
        f[3] = __uint_as_float(v.w);
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

// Wave-level exact rank among n <= 64 nonzero keys held in LDS (16-byte aligned, zero from
// entry n up to the next multiple of 4), 1 <= rem <= n: writes out[0] = the
// rem-th largest key, out[1] = how many of the keys equal to it fall within the top rem
// (rem - #greater), out[2] = whether that is all of them.  Lanes holding equal keys write equal
// values.  Call from one whole wave.
__device__ __forceinline__ void rank_small(const uint32_t *small, int n, int rem, int *out)
{
    const int l = lane_id();
    const uint32_t v = l < n ? small[l] : 0u;
    int gt = 0, ge = 0;
    // small[n .. 4*ceil(n/4)) are zero: no key of the n is below 1, so they count nowhere
    const uint4 *s4 = reinterpret_cast<const uint4 *>(small);
    for (int j = 0; j < (n + 3) / 4; ++j) {
        const uint4 u = s4[j];
        gt += (u.x > v) + (u.y > v) + (u.z > v) + (u.w > v);
        ge += (u.x >= v) + (u.y >= v) + (u.z >= v) + (u.w >= v);
    }
    if (l < n && gt < rem && rem <= ge) {
        out[0] = (int)v;
        out[1] = rem - gt;
        out[2] = rem == ge;
    }
}

// find_digit for NBIN = 2048 bins, scanned by wave 0 alone, so it costs one barrier: lane l
// sums bins [2048 - 32(l+1), 2048 - 32l) (lanes in top-down order); the first lane whose
// inclusive sum reaches `need` holds the digit, and 32 lanes then scan its 32 bins from the top.
// The histogram must be complete (a barrier after its last update).  Uses
// scratch[NTH/64 .. NTH/64 + 3]; the values read back stay valid until the caller's next
// barrier-separated write to those slots.
template <int NTH>
__device__ __forceinline__ Digit find_digit_w0(const int *hist, int need, int *scratch)
{
    constexpr int NWV = NTH / kWave;
    static_assert(NBIN == 32 * kWave, "32 bins per lane");
    if (threadIdx.x < kWave) {
        const int l = (int)threadIdx.x;
        const int4 *h4 = reinterpret_cast<const int4 *>(hist + NBIN - 32 * (l + 1));
        int mine = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int4 v = h4[i];
            mine += v.x + v.y + v.z + v.w;
        }
        const int inc = wave_inclusive_scan(mine);
        const int total = __builtin_amdgcn_readlane(inc, kWave - 1);
        const uint64_t ge = __ballot(inc >= need);
        if (ge != 0u) {
            const int L = (int)__builtin_ctzll(ge);
            const int exL = __builtin_amdgcn_readlane(inc, L) - __builtin_amdgcn_readlane(mine, L);
            const int top = NBIN - 32 * L - 1; // lane i < 32 takes bin top - i
            const int c = l < 32 ? hist[top - (l & 31)] : 0;
            const int inc2 = exL + wave_inclusive_scan(c);
            const uint64_t ge2 = __ballot(l < 32 && inc2 >= need);
            const int i = (int)__builtin_ctzll(ge2); // exists: exL + (sum of the 32) >= need
            if (l == i) {
                scratch[NWV] = total;
                scratch[NWV + 1] = top - i;
                scratch[NWV + 2] = inc2 - c;
                scratch[NWV + 3] = c;
            }
        } else if (l == 0) {
            scratch[NWV] = total;
            scratch[NWV + 1] = -1;
        }
    }
    __syncthreads();
    Digit r;
    r.total = scratch[NWV];
    r.d = scratch[NWV + 1];
    r.above = scratch[NWV + 2];
    r.at = scratch[NWV + 3];
    return r;
}

// Threshold from a sample of the row.  NTH/64 * KPT blocks of 64 consecutive positions, evenly
// spread over [lo, hi), are read; T is the rr-th largest sampled key (or, when the 11-bit bin
// holding it has more than 64 sampled keys, the lower edge of its 22-bit key prefix),
// rr = 2 * need * (sampled / len) + 8, so about twice `need` elements of the row are expected
// at or above T.  Returns 0 when the row is shorter than the sample or the sample has fewer
// than rr competing keys.  The caller checks what it collects against T (at least `need`,
// within capacity) and falls back to the exact histogram path otherwise, so T only ever affects
// speed, never the result.  Every workgroup computing T for the same row gets the same T.
// `hist` holds NBIN ints, `small` 64 (16-byte aligned), `scratch` NTH/64 + 8.
template <int NTH, int KPT>
__device__ __forceinline__ uint32_t sample_threshold(int *hist, int *scratch, uint32_t *small,
                                                     const Row &r, int need, int64_t len)
{
    constexpr int NWV = NTH / kWave;
    constexpr int NSB = NWV * KPT; // sample blocks
    if (len < (int64_t)kWave * NSB) return 0u;
    const int l = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(wave_id());
    // block sb = j*NWV + wv starts at lo + (len - 64) * sb / (NSB - 1): wave-uniform, and its 64
    // positions lie in [lo, hi)
    uint32_t key[KPT];
    float f[KPT];
    int32_t c[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const int64_t start = r.lo + (len - kWave) * (j * NWV + wv) / (NSB - 1);
        f[j] = r.sc[start + l];
        if (r.ids) c[j] = r.ids[start + l];
    }
    {
        int4 *h4 = reinterpret_cast<int4 *>(hist);
        for (int i = threadIdx.x; i < NBIN / 4; i += NTH) h4[i] = make_int4(0, 0, 0, 0);
    }
    if (threadIdx.x < kWave) small[threadIdx.x] = 0u;
    if (threadIdx.x == 0) scratch[NWV + 4] = 0;
    const int32_t id_lo = (int32_t)r.id_lo, id_hi = (int32_t)r.id_hi;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const bool in = !r.ids || (c[j] >= id_lo && c[j] < id_hi);
        key[j] = in ? order_key(f[j]) : 0u;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KPT; ++j)
        if (key[j]) atomicAdd(&hist[key[j] >> 21], 1);
    __syncthreads();
    const int64_t ns = (int64_t)NSB * kWave;
    const int64_t want = (2 * (int64_t)need * ns + len - 1) / len + 8;
    if (want > ns) return 0u;
    const Digit g = find_digit_w0<NTH>(hist, (int)want, scratch);
    if (want > g.total) return 0u;
    const int rem = (int)want - g.above;
    uint32_t T;
    if (g.at <= kWave) { // rank the crossing bin's sampled keys exactly
#pragma unroll
        for (int j = 0; j < KPT; ++j)
            if (key[j] && (key[j] >> 21) == (uint32_t)g.d)
                small[atomicAdd(&scratch[NWV + 4], 1)] = key[j];
        __syncthreads();
        if (threadIdx.x < kWave) rank_small(small, g.at, rem, scratch + NWV + 5);
        __syncthreads();
        T = (uint32_t)scratch[NWV + 5];
    } else { // second 11-bit digit (key bits 20..10)
        {
            int4 *h4 = reinterpret_cast<int4 *>(hist);
            for (int i = threadIdx.x; i < NBIN / 4; i += NTH) h4[i] = make_int4(0, 0, 0, 0);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < KPT; ++j)
            if (key[j] && (key[j] >> 21) == (uint32_t)g.d)
                atomicAdd(&hist[(key[j] >> 10) & (NBIN - 1)], 1);
        __syncthreads();
        const Digit h = find_digit_w0<NTH>(hist, rem, scratch);
        T = (((uint32_t)g.d << 11) | (uint32_t)h.d) << 10;
    }
    // passes compare floats against T: keep it above the key of -inf (always so for finite
    // sampled scores; a -inf threshold would also admit elements that do not compete)
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
    alignas(16) int hist[NBIN];
    int scratch[NW + 8];
    int cnt[ITEMS * NW];
    alignas(16) uint32_t small[kWave];
    alignas(16) uint32_t buf_key[CAP];
    alignas(16) int32_t buf_id[CAP];
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

// The LDS buffer is worked on from registers: with span = 64 * ceil(nbuf / (64 NW)), thread
// (wave w, lane l) holds entries span*w + 64u + l for u < span/64 (<= BI), so every wave has a
// like share and position order is (wave, u, lane).  Items past span/64 hold key 0.
constexpr int BI = CAP / NT;
__device__ __forceinline__ int buf_items(int nbuf) { return (nbuf + NW * kWave - 1) / (NW * kWave); }
__device__ __forceinline__ int buf_index(int nu, int u) { return (wave_id() * nu + u) * kWave + lane_id(); }

__device__ __forceinline__ void load_keys(const Smem &sm, int nbuf, uint32_t (&k)[BI])
{
    const int nu = buf_items(nbuf);
#pragma unroll
    for (int u = 0; u < BI; ++u) {
        const int i = buf_index(nu, u);
        k[u] = u < nu && i < nbuf ? sm.buf_key[i] : 0u;
    }
}

// Ordered emission from the buffer (keys k as load_keys gives them): key > T, then the first
// eq_take keys == T in position order, into dst[0, limit).  Key 0 never competes.  eq_all: every
// key == T is taken (eq_take is their count), i.e. simply key >= T.  One exchange of per-wave
// counts orders the picks.  Returns the number taken (which may exceed limit).
template <int NI>
__device__ __forceinline__ int select_buf(Smem &sm, int nbuf, uint32_t T, int eq_take, int32_t *dst,
                                          int limit, bool eq_all, const uint32_t (&k)[NI],
                                          const int32_t *ids)
{
    const int lane = lane_id(), w = wave_id();
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int nu = buf_items(nbuf);
    int32_t idv[NI];
#pragma unroll
    for (int u = 0; u < NI; ++u) {
        const int i = buf_index(nu, u);
        idv[u] = u < nu && i < nbuf ? ids[i] : 0;
    }
    auto put = [&](uint32_t slot, int32_t v) { // 32-bit offset from the uniform base
        if (slot < (uint32_t)limit) *reinterpret_cast<int32_t *>(reinterpret_cast<char *>(dst) + slot * 4u) = v;
    };
    auto below = [](uint64_t m) {
        return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    };
    // the masks are taken twice (count, then place) rather than kept: NI of them per kind would
    // hold 2 NI scalar registers each
    if (eq_all) {
        int cg = 0;
#pragma unroll
        for (int u = 0; u < NI; ++u) cg += (int)__popcll(__ballot(k[u] != 0u && k[u] >= T));
        if (lane == 0) sm.cnt[w] = cg;
        __syncthreads();
        // lane q < NW holds wave q's count; the prefix sum gives this wave's base
        const int ck = lane < NW ? sm.cnt[lane] : 0;
        const int ick = wave_inclusive_scan(ck);
        uint32_t pos = (uint32_t)(__builtin_amdgcn_readlane(ick, wu) - __builtin_amdgcn_readlane(ck, wu));
#pragma unroll
        for (int u = 0; u < NI; ++u) {
            if (u >= nu) break;
            const bool tk = k[u] != 0u && k[u] >= T;
            const uint64_t mg = __ballot(tk);
            if (tk) put(pos + below(mg), idv[u]);
            pos += (uint32_t)__popcll(mg);
        }
        return __builtin_amdgcn_readlane(ick, NW - 1);
    }
    int cg = 0, ce = 0;
#pragma unroll
    for (int u = 0; u < NI; ++u) {
        cg += (int)__popcll(__ballot(k[u] > T));
        ce += (int)__popcll(__ballot(k[u] != 0u && k[u] == T));
    }
    if (lane == 0) {
        sm.cnt[w] = cg;
        sm.cnt[NW + w] = ce;
    }
    __syncthreads();
    const int ck = lane < NW ? sm.cnt[lane] : 0, ek = lane < NW ? sm.cnt[NW + lane] : 0;
    const int ick = wave_inclusive_scan(ck), iek = wave_inclusive_scan(ek);
    const int bg = __builtin_amdgcn_readlane(ick, wu) - __builtin_amdgcn_readlane(ck, wu);
    const int be = __builtin_amdgcn_readlane(iek, wu) - __builtin_amdgcn_readlane(ek, wu);
    const int tg = __builtin_amdgcn_readlane(ick, NW - 1);
    const int te = __builtin_amdgcn_readlane(iek, NW - 1);
    // equal keys of earlier waves that are taken: equal ranks [0, be)
    int pos = bg + max(0, min(eq_take, be));
    int er = be; // equal rank of the wave's next equal key
#pragma unroll
    for (int u = 0; u < NI; ++u) {
        if (u >= nu) break;
        uint64_t mt = __ballot(k[u] > T);
        const uint64_t me = __ballot(k[u] != 0u && k[u] == T);
        if (me) {
            const int r = er + (int)below(me);
            mt |= __ballot(((me >> lane) & 1u) && r < eq_take);
            er += (int)__popcll(me);
        }
        if ((mt >> lane) & 1u) put((uint32_t)pos + below(mt), idv[u]);
        pos += (int)__popcll(mt);
    }
    return tg + max(0, min(eq_take, te));
}

// Wave-wide unsigned min / max in the DPP steps of wave_inclusive_scan (lane 63 ends with the
// whole wave's result; out-of-row sources and masked rows contribute the identity).
template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce_u(uint32_t x)
{
    const int id = MAX ? 0 : -1;
    auto op = [](uint32_t a, uint32_t b) { return MAX ? max(a, b) : min(a, b); };
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x111, 0xf, 0xf, false));
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x112, 0xf, 0xf, false));
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x114, 0xf, 0xf, false));
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x118, 0xf, 0xf, false));
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x142, 0xa, 0xf, false));
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x143, 0xc, 0xf, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)x, kWave - 1);
}

// The buffer holds nbuf entries in position order; its competing elements (key != 0; entries
// with key 0 do not compete) include the row's `need` best.  kmin / kmax: the least and greatest
// nonzero key (kmin > kmax when there is none).  Emit exactly the `need` best (all competing
// ones, padded with -1, if there are at most `need`).  On entry sm.hist, sm.small and
// sm.scratch[NW + 4] are zero and a barrier has passed since.
//
// Bins are refined until the bin holding the need-th key has at most 64 keys, which one wave
// then ranks exactly.  The first level is linear in the score over [min, max] when the keys
// span more than a few binades and both ends and the span are finite (a monotone digit, so bins
// stay small even where a whole score distribution crowds a few exponents).  Further levels take digits of rel = key - kmin:
// rel >> s0 with the smallest s0 that fits 2048 bins, then the next (up to) 11 bits below, each
// among the keys of the bins chosen so far -- down to a single key value if need be, of which
// the needed count of copies is taken.
template <int NI>
__device__ __forceinline__ void select_in_buf_range(Smem &sm, int nbuf, int need, int32_t *dst,
                                                    uint32_t kmin, uint32_t kmax,
                                                    const uint32_t (&k)[NI], const int32_t *ids)
{
    const float fmin = key_to_float(kmin), fmax = key_to_float(kmax);
    const float span = fmax - fmin;
    // (over at most a few binades, 11-bit digits of the key are as fine as linear bins)
    const bool lin = kmin < kmax && (kmax - kmin) >= (1u << 24) && fmin > -INFINITY &&
                     fmax < INFINITY && span > 0.0f && span < INFINITY;
    const float scale = lin ? (float)NBIN / span : 0.0f;
    auto fdigit = [&](uint32_t k) {
        return (uint32_t)min(NBIN - 1, (int)((key_to_float(k) - fmin) * scale));
    };
    const uint32_t range = kmin <= kmax ? kmax - kmin : 0u;
    const int nu = buf_items(nbuf); // items held per thread (the rest are key 0)
    bool lin_done = false;          // the linear level has chosen bin fd
    uint32_t fd = 0u;
    int key_lvls = 0, sh = 0;       // key levels applied; the last one's shift
    uint32_t pref = 0u;             // ... and the chosen rel >> sh
    int next_sh = range ? max(0, 32 - (int)__builtin_clz(range) - 11) : 0, next_hi = 32;
    auto in_bin = [&](uint32_t k) {
        return (!lin_done || fdigit(k) == fd) && (key_lvls == 0 || ((k - kmin) >> sh) == pref);
    };
    int rem = need;
    bool take_all = false;
    Digit g;
    for (bool first = true;; first = false) {
        const bool use_lin = lin && !lin_done;
        const uint32_t dmask = next_hi == 32 ? ~0u : (1u << (next_hi - next_sh)) - 1u;
#pragma unroll
        for (int u = 0; u < NI; ++u)
            if (u < nu && k[u] != 0u && in_bin(k[u]))
                atomicAdd(&sm.hist[use_lin ? fdigit(k[u]) : ((k[u] - kmin) >> next_sh) & dmask], 1);
        __syncthreads();
        g = find_digit_w0<NT>(sm.hist, rem, sm.scratch);
        if (first && g.total <= need) { // at most `need` compete: all of them, then -1
            take_all = true;
            break;
        }
        rem -= g.above;
        if (use_lin) {
            lin_done = true;
            fd = (uint32_t)g.d;
        } else {
            pref = key_lvls == 0 ? (uint32_t)g.d : (pref << (next_hi - next_sh)) | (uint32_t)g.d;
            sh = next_sh;
            ++key_lvls;
            next_hi = next_sh;
            next_sh = max(0, next_sh - 11);
        }
        if (g.at <= kWave || (key_lvls > 0 && sh == 0)) break;
        int4 *h4 = reinterpret_cast<int4 *>(sm.hist);
        for (int i = threadIdx.x; i < NBIN / 4; i += NT) h4[i] = make_int4(0, 0, 0, 0);
        __syncthreads();
    }
    uint32_t T;
    int eq_take;
    bool eq_all;
    if (take_all) {
        T = 1u;
        eq_take = 0;
        eq_all = true;
    } else if (g.at <= kWave) { // rank the bin's keys: the rem-th largest is the need-th
        uint32_t *small = sm.small;
#pragma unroll
        for (int u = 0; u < NI; ++u)
            if (u < nu && k[u] != 0u && in_bin(k[u])) small[atomicAdd(&sm.scratch[NW + 4], 1)] = k[u];
        __syncthreads();
        if (threadIdx.x < kWave) rank_small(small, g.at, rem, sm.scratch + NW + 5);
        __syncthreads();
        T = (uint32_t)sm.scratch[NW + 5];
        eq_take = sm.scratch[NW + 6];
        eq_all = sm.scratch[NW + 7] != 0;
    } else { // the bin is one key value (sh == 0): rem of its g.at copies are taken
        T = kmin + pref;
        eq_take = rem;
        eq_all = rem == g.at;
    }
    const int got = select_buf<NI>(sm, nbuf, T, eq_take, dst, need, eq_all, k, ids);
    if (take_all)
        for (int i = min(got, need) + (int)threadIdx.x; i < need; i += NT) dst[i] = -1;
}

// Per-wave extremes -> LDS (the caller's next barrier publishes them); read back with
// block_extremes after that barrier.  Uses sm.cnt[0 .. 2*NW).
__device__ __forceinline__ void wave_extremes(Smem &sm, uint32_t kmin, uint32_t kmax)
{
    kmin = wave_reduce_u<false>(kmin);
    kmax = wave_reduce_u<true>(kmax);
    uint32_t *mm = reinterpret_cast<uint32_t *>(sm.cnt);
    if (lane_id() == 0) {
        mm[wave_id()] = kmin;
        mm[NW + wave_id()] = kmax;
    }
}

__device__ __forceinline__ void block_extremes(const Smem &sm, uint32_t &kmin, uint32_t &kmax)
{
    const uint32_t *mm = reinterpret_cast<const uint32_t *>(sm.cnt);
    const int l = lane_id();
    kmin = wave_reduce_u<false>(l < NW ? mm[l] : ~0u);
    kmax = wave_reduce_u<true>(l < NW ? mm[NW + l] : 0u);
}

__device__ __forceinline__ void clear_hist_nobar(Smem &sm)
{
    int4 *h4 = reinterpret_cast<int4 *>(sm.hist);
    for (int i = threadIdx.x; i < NBIN / 4; i += NT) h4[i] = make_int4(0, 0, 0, 0);
    if (threadIdx.x < kWave) sm.small[threadIdx.x] = 0u;
    if (threadIdx.x == 0) sm.scratch[NW + 4] = 0;
}

// The buffer holds nbuf entries in position order whose competing elements (key != 0) include
// the row's `need` best, and a barrier has passed since its last write.  Emit exactly those (all
// competing ones, padded with -1, if there are at most `need`).
__device__ __forceinline__ void select_from_buf(Smem &sm, int nbuf, int need, int32_t *dst)
{
    uint32_t k[BI];
    load_keys(sm, nbuf, k);
    uint32_t kmin = ~0u, kmax = 0u;
#pragma unroll
    for (int u = 0; u < BI; ++u)
        if (k[u] != 0u) {
            kmin = min(kmin, k[u]);
            kmax = max(kmax, k[u]);
        }
    wave_extremes(sm, kmin, kmax);
    clear_hist_nobar(sm);
    __syncthreads();
    block_extremes(sm, kmin, kmax);
    select_in_buf_range<BI>(sm, nbuf, need, dst, kmin, kmax, k, sm.buf_id);
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

// Gathers into the LDS buffer a position-ordered set of the row's elements that contains its
// `need` best (need > 0) and returns its size, with a barrier passed after the last write -- or
// completes the row itself (everything competing taken, or heavy ties) and returns -1.
// Flat rows of at most NT * RI elements past the buffer (Hierarchical Indexing's page rows, for
// one) are read once, into registers: thread t holds positions a0 + RI t + [0, RI) (16-byte
// loads; thread order is position order).  An LDS histogram of every element's top 11 key bits
// gives the row's exact threshold bin (refined by the next 11 bits when the bin would overflow
// the buffer), and what lies at or above it is compacted into the buffer straight from the
// registers (the streaming paths pass over the row twice: a sample, then a collection).
constexpr int RI = 16;
constexpr int REGS_FALLBACK = -2;

// The buffer count, -1 when every competing element was written to dst (at most `need`), or
// REGS_FALLBACK when even the second digit leaves too many to fit the buffer.  Rows with 16-byte
// vector access and hi - (lo & ~3) <= NT * RI only.
__device__ __forceinline__ int prepare_buf_regs(Smem &sm, const Row &r, int need, int32_t *dst)
{
    const int64_t a0 = r.lo & ~int64_t(3);
    const int64_t last = (r.hi - 1) & ~int64_t(3); // the last quad holding an element
    const int64_t p0 = a0 + (int64_t)threadIdx.x * RI;
    float f[RI];
    // every quad is loaded (clamped to the last one) before any is used, masked afterwards
#pragma unroll
    for (int q = 0; q < RI / 4; ++q) {
        const float4 v = *reinterpret_cast<const float4 *>(r.sc + min(p0 + 4 * q, last));
        f[4 * q] = v.x;
        f[4 * q + 1] = v.y;
        f[4 * q + 2] = v.z;
        f[4 * q + 3] = v.w;
    }
    clear_hist(sm);
    uint32_t key[RI];
#pragma unroll
    for (int j = 0; j < RI; ++j) {
        const int64_t p = p0 + j;
        key[j] = p >= r.lo && p < r.hi ? order_key(f[j]) : 0u;
        if (key[j]) atomicAdd(&sm.hist[key[j] >> 21], 1);
    }
    __syncthreads();
    const Digit g = find_digit_w0<NT>(sm.hist, need, sm.scratch);
    const bool all = g.total <= need;
    uint32_t T = all ? 0u : (uint32_t)g.d << 21;
    if (!all && g.above + g.at > CAP) { // uniform: refine within bin d by key bits 20..10
        clear_hist(sm);
#pragma unroll
        for (int j = 0; j < RI; ++j)
            if (key[j] && (key[j] >> 21) == (uint32_t)g.d) atomicAdd(&sm.hist[(key[j] >> 10) & (NBIN - 1)], 1);
        __syncthreads();
        const Digit g2 = find_digit_w0<NT>(sm.hist, need - g.above, sm.scratch);
        if (g.above + g2.above + g2.at > CAP) return REGS_FALLBACK; // heavy ties
        T |= (uint32_t)g2.d << 10;
    }
    uint32_t take = 0; // bit j: element j competes and lies at or above the threshold
#pragma unroll
    for (int j = 0; j < RI; ++j) take |= (uint32_t)(key[j] != 0u && key[j] >= T) << j;
    int total;
    int slot = block_exclusive_scan<NW>(__popc(take), sm.scratch, &total);
#pragma unroll
    for (int j = 0; j < RI; ++j) {
        if (!((take >> j) & 1u)) continue;
        if (all) {
            dst[slot] = (int32_t)(p0 + j);
        } else {
            sm.buf_key[slot] = key[j];
            sm.buf_id[slot] = (int32_t)(p0 + j);
        }
        ++slot;
    }
    if (all) {
        for (int i = total + (int)threadIdx.x; i < need; i += NT) dst[i] = -1;
        return -1;
    }
    __syncthreads();
    return total;
}

template <bool REGS = false>
__device__ __forceinline__ int prepare_buf(Smem &sm, const Row &r, int need, int32_t *dst)
{
    const int64_t len = r.hi - r.lo;
    // rows that fit the buffer are copied there as they are (key 0 where an element does not
    // compete): entry i holds position a0 + i
    const int64_t a0 = r.lo & ~int64_t(3);
    if (r.hi - a0 <= CAP) {
        const int n4 = (int)((r.hi - a0 + 3) & ~int64_t(3));
#pragma unroll
        for (int u = 0; u < CAP / (4 * NT); ++u) {
            const int i = 4 * ((int)threadIdx.x + u * NT);
            if (i < n4) {
                uint32_t key[4];
                int32_t id[4];
                elem4(r, a0 + i, key, id, r.hi);
                *reinterpret_cast<uint4 *>(&sm.buf_key[i]) = make_uint4(key[0], key[1], key[2], key[3]);
                *reinterpret_cast<int4 *>(&sm.buf_id[i]) = make_int4(id[0], id[1], id[2], id[3]);
            }
        }
        __syncthreads();
        return n4;
    }
    if constexpr (REGS) {
        if (!r.ids && r.vec && r.hi - a0 <= (int64_t)NT * RI) {
            const int n = prepare_buf_regs(sm, r, need, dst);
            if (n != REGS_FALLBACK) return n;
        }
    }
    // long rows: a sampled threshold lets one pass collect everything at or above it
    const uint32_t T = len >= SAMPLE_MIN
                           ? sample_threshold<NT, 4>(sm.hist, sm.scratch, sm.small, r, need, len)
                           : 0u;
    if (T != 0u) {
        int nbuf = 0, total = 0;
        bool ok = collect_row_seg(sm, r, T, nbuf, total);
        if (!ok && total <= CAP) { // a wave's list overflowed, the buffer would not: ordered pass
            nbuf = select_row(sm, r, T, INT32_MAX, nullptr, true, CAP);
            __syncthreads();
            ok = true;
        }
        if (ok && nbuf >= need) return nbuf;
    }
    // exact histogram path
    hist_row_seg(sm, r);
    Digit g = find_digit_w0<NT>(sm.hist, need, sm.scratch);
    if (g.total <= need) { // everything competes: take all, pad
        const int got = min(select_row(sm, r, 0u, 0, dst, false, need), need);
        for (int i = got + (int)threadIdx.x; i < need; i += NT) dst[i] = -1;
        return -1;
    }
    uint32_t prefix = (uint32_t)g.d;
    int pbits = 11;
    int need_rem = need - g.above;
    if (g.above + g.at <= CAP) { // the buffer takes bins >= d: the need best
        int nbuf, total;
        if (!collect_row_seg(sm, r, prefix << 21, nbuf, total)) { // uneven segments: ordered pass
            nbuf = select_row(sm, r, prefix << 21, INT32_MAX, nullptr, true, CAP);
            __syncthreads();
        }
        return nbuf;
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
    }
    select_row(sm, r, prefix, need_rem, dst, false, need);
    return -1;
}

// Row setup shared by both paths.  Returns false when the row needs no selection (all of it
// written already).
__device__ __forceinline__ bool setup_row(const SelectArgs &a, int64_t row, Row &r, int32_t *&dst,
                                          int &need,
                          bool write_fixed)
{
    const int64_t t = row % a.n_q;
    const int64_t V = valid_len(a.seq_len, a.seq_pos0, (int)(row / a.n_q), t, a.kv_len, a.q_pos0);
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

// CAND: candidate rows (ids from the list); flat rows get a null id pointer the compiler can see,
// so the flat kernel carries no id loads.
template <bool CAND, bool REGS = false>
__device__ __forceinline__ void select_one_row(const SelectArgs &a)
{
    __shared__ Smem sm;
    Row r;
    int32_t *dst;
    int need;
    if (!setup_row(a, blockIdx.x, r, dst, need, true)) return;
    if (!CAND) r.ids = nullptr;
    const int nbuf = prepare_buf<REGS>(sm, r, need, dst);
    if (nbuf >= 0) select_from_buf(sm, nbuf, need, dst);
}

// Flat rows (prefill, page recall): at most 64 VGPRs and 96 SGPRs, so two workgroups share a CU
// (with one, the CU's memory path idles through each row's sampling and in-buffer selection).
__global__ __launch_bounds__(NT, 8) void select_kernel_flat(SelectArgs a) { select_one_row<false>(a); }

__global__ __launch_bounds__(NT) void select_kernel_cand(SelectArgs a) { select_one_row<true>(a); }

// Flat rows of CAP < n_in <= NT * RI elements: the register-resident path (one pass over the
// row).  Few such rows run at once (page recall), so the kernel may use more registers.
__global__ __launch_bounds__(NT) void select_kernel_regs(SelectArgs a) { select_one_row<false, true>(a); }

constexpr int HGROUPS = 32; // coarse sums of 64 bins each in the scoring launch's histograms

// The row's threshold bin from the scoring workgroups' histograms: the 11-bit bin d (key bits
// 31..21) holding the need-th largest middle-region key, how many keys lie above it and in it,
// and the row's middle-region total.  First the 32 coarse sums (64 bins each) locate the 64-bin
// group, then that group's 64 bins locate d; at each level the block's threads share the
// groups x bins loads (all in flight at once) and one wave finishes the sums from LDS.  d = -1
// when fewer than `need` keys compete.  Every thread of the NTH-thread block calls it; the
// result is the same in every thread.  `part` holds 2 * NTH ints of LDS, `scratch` 6.
template <int NTH>
__device__ __forceinline__ Digit hist_threshold(int *part, int *scratch, const uint32_t *hist_fine,
                                                const uint32_t *hist_coarse, int groups,
                                                int64_t row, int need)
{
    static_assert(NTH % 64 == 0 && NTH >= 64, "whole waves");
    constexpr int XC = NTH / HGROUPS, XF = NTH / 64; // slice strides per level
    const int l = lane_id(), t = (int)threadIdx.x;
    const uint32_t *hc = hist_coarse + row * groups * HGROUPS;
    const uint32_t *hf = hist_fine + row * groups * NBIN;
    {
        const int bin = t % HGROUPS, x0 = t / HGROUPS;
        int c = 0;
        for (int x = x0; x < groups; x += XC) c += (int)hc[x * HGROUPS + bin];
        part[t] = c;
    }
    __syncthreads();
    if (t < kWave) {
        // lane l < 32 holds coarse group 31 - l (top-down)
        int mine = 0;
        if (l < HGROUPS)
#pragma unroll
            for (int i = 0; i < XC; ++i) mine += part[i * HGROUPS + (HGROUPS - 1 - l)];
        const int inc = wave_inclusive_scan(mine);
        const uint64_t ge = __ballot(l < HGROUPS && inc >= need);
        const int L = ge ? (int)__builtin_ctzll(ge) : 0;
        const int exL = __builtin_amdgcn_readlane(inc, L) - __builtin_amdgcn_readlane(mine, L);
        if (l == 0) {
            scratch[0] = __builtin_amdgcn_readlane(inc, kWave - 1);
            scratch[1] = ge ? L : -1;
            scratch[2] = exL;
        }
    }
    __syncthreads();
    Digit r;
    r.total = scratch[0];
    r.d = -1;
    r.above = 0;
    r.at = 0;
    const int L = scratch[1];
    if (L < 0) return r; // uniform
    const int exL = scratch[2];
    const int top = 64 * (HGROUPS - 1 - L) + 63; // bin top - i is the i-th from the top
    {
        // a slice's fine bins are written only for the groups that hold keys: a group whose
        // coarse sum is 0 contributes 0 (its fine bins are left from earlier calls)
        const int i = t & 63, x0 = t >> 6, G = HGROUPS - 1 - L;
        int c = 0;
        for (int x = x0; x < groups; x += XF) {
            const int cg = (int)hc[x * HGROUPS + G];
            const int f = (int)hf[x * NBIN + top - i];
            c += cg ? f : 0;
        }
        part[NTH + t] = c;
    }
    __syncthreads();
    if (t < kWave) {
        int c = 0;
#pragma unroll
        for (int k = 0; k < XF; ++k) c += part[NTH + k * 64 + l];
        const int inc2 = exL + wave_inclusive_scan(c);
        const uint64_t ge2 = __ballot(inc2 >= need);
        const int i = (int)__builtin_ctzll(ge2); // exists: the group's keys reach `need`
        const int ab = __builtin_amdgcn_readlane(inc2, i) - __builtin_amdgcn_readlane(c, i);
        const int at = __builtin_amdgcn_readlane(c, i);
        if (l == 0) {
            scratch[3] = top - i;
            scratch[4] = ab;
            scratch[5] = at;
        }
    }
    __syncthreads();
    r.d = scratch[3];
    r.above = scratch[4];
    r.at = scratch[5];
    return r;
}

// ------------------------------------------------------------------------------------------
// Chunked path
// ------------------------------------------------------------------------------------------

constexpr int CNT_WAVES = CNT_THREADS / kWave;
constexpr int WSEG = CHUNK / CNT_WAVES; // positions per wave (contiguous)
constexpr int CI = WSEG / kWave;        // items per lane

struct ChunkWs {
    int *count;     // [rows][n_chunks]  (CHUNK_CAP + 1 = overflow or no threshold)
    float *cval;    // [rows][n_chunks][CHUNK_CAP] scores of the collected elements
    int32_t *cid;   // [rows][n_chunks][CHUNK_CAP] their ids
    int n_chunks;
    // the scoring launch's histograms of the rows (flat decode rows), or nullptr: then the
    // threshold is sampled from the row
    const uint32_t *hist_fine, *hist_coarse;
    int groups;
};

// Every chunk of a row derives the row's sampled threshold T (the same T in every workgroup)
// and compacts its elements with key >= T, in position order, into its slice of the workspace.
// Wave w owns positions [c0 + w*WSEG, c0 + (w+1)*WSEG); item j of lane l is position
// c0 + w*WSEG + j*64 + l.  CAND: candidate rows (ids read from the list).
template <bool CAND>
__global__ __launch_bounds__(CNT_THREADS) void chunk_collect_kernel(SelectArgs a, ChunkWs ws)
{
    __shared__ __align__(16) int hist[NBIN];
    __shared__ int scratch[CNT_WAVES + 8];
    static_assert(2 * CNT_THREADS <= NBIN, "histogram partial sums fit");
    __shared__ __align__(16) uint32_t small[kWave];
    __shared__ int wcnt[CNT_WAVES];
    const int64_t row = blockIdx.y;
    const int chunk = blockIdx.x;
    Row r;
    int32_t *dst;
    int need;
    if (!setup_row(a, row, r, dst, need, false)) return;
    int *cntp = ws.count + row * ws.n_chunks + chunk;
    const int64_t c0 = (int64_t)chunk * CHUNK;
    // a chunk outside the row collects nothing; the row's other chunks report its threshold
    if (c0 + CHUNK <= r.lo || c0 >= r.hi) {
        if (threadIdx.x == 0) *cntp = 0;
        return;
    }
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(wave_id());
    const int64_t wb = c0 + (int64_t)w * WSEG;
    const bool inner = wb >= r.lo && wb + WSEG <= r.hi; // wave-uniform
    // the chunk's loads go out first, so their latency overlaps the sample's
    float f[CI];
    int32_t id[CI];
    if (inner) {
        const float *ps = r.sc + wb + lane;
#pragma unroll
        for (int j = 0; j < CI; ++j) f[j] = __builtin_nontemporal_load(ps + j * kWave); // read once
        if (CAND) {
            const int32_t *pi = r.ids + wb + lane;
#pragma unroll
            for (int j = 0; j < CI; ++j) id[j] = pi[j * kWave];
        }
    } else { // positions clamped into the row (non-empty), used only when inside it
#pragma unroll
        for (int j = 0; j < CI; ++j) {
            const int64_t p = wb + j * kWave + lane;
            const int64_t pc = p < r.lo ? r.lo : (p >= r.hi ? r.hi - 1 : p);
            f[j] = r.sc[pc];
            if (CAND) id[j] = r.ids[pc];
        }
    }
    const int64_t len = r.hi - r.lo;
    uint32_t T;
    if (ws.hist_fine) {
        // the row's exact threshold bin, from the scoring launch's histograms: every element in
        // a bin at or above it is collected (the row's best above + at, at least `need`)
        const Digit g = hist_threshold<CNT_THREADS>(hist, scratch, ws.hist_fine, ws.hist_coarse,
                                                    ws.groups, row, need);
        const uint32_t Tg = g.d >= 0 ? (uint32_t)g.d << 21 : 0u;
        T = (g.d >= 0 && g.above + g.at <= CAP && Tg > order_key(-INFINITY)) ? Tg : 0u;
    } else {
        // 1024 samples up to 256K positions, 4096 beyond (the expected sampled rank stays >= 16)
        T = len <= (int64_t)1 << 18
                ? sample_threshold<CNT_THREADS, 4>(hist, scratch, small, r, need, len)
                : sample_threshold<CNT_THREADS, 16>(hist, scratch, small, r, need, len);
    }
    if (T == 0u) { // no usable threshold: the finish kernel falls back to the exact path
        if (threadIdx.x == 0) *cntp = CHUNK_CAP + 1;
        return;
    }
    const float tf = key_to_float(T);
    const int32_t id_lo = (int32_t)r.id_lo, id_hi = (int32_t)r.id_hi;
    uint64_t m[CI];
    if (inner) {
#pragma unroll
        for (int j = 0; j < CI; ++j) {
            bool take = f[j] >= tf;
            if (CAND) take = take && id[j] >= id_lo && id[j] < id_hi;
            m[j] = __ballot(take);
        }
    } else { // row-relative positions, compared unsigned against the row length
        const int32_t q0 = (int32_t)(wb - r.lo) + lane;
        const uint32_t ulen = (uint32_t)len;
#pragma unroll
        for (int j = 0; j < CI; ++j) {
            bool take = f[j] >= tf && (uint32_t)(q0 + j * kWave) < ulen;
            if (CAND) take = take && id[j] >= id_lo && id[j] < id_hi;
            m[j] = __ballot(take);
        }
    }
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < CI; ++j) cnt += (int)__popcll(m[j]);
    if (lane == 0) wcnt[w] = cnt;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int i = 0; i < CNT_WAVES; ++i) {
        const int c = wcnt[i];
        base += i < w ? c : 0;
        total += c;
    }
    if (total > CHUNK_CAP) {
        if (threadIdx.x == 0) *cntp = CHUNK_CAP + 1;
        return;
    }
    float *ov = ws.cval + (row * ws.n_chunks + chunk) * CHUNK_CAP;
    int32_t *oi = ws.cid + (row * ws.n_chunks + chunk) * CHUNK_CAP;
    const uint64_t lanebit = 1ull << lane;
    const int32_t id0 = (int32_t)wb + lane; // flat rows: id = position
    uint32_t pos = (uint32_t)base;
#pragma unroll
    for (int j = 0; j < CI; ++j) {
        const uint64_t mj = m[j];
        if (mj == 0u) continue;
        if (mj & lanebit) {
            const uint32_t slot = pos + __builtin_amdgcn_mbcnt_hi(
                                            (uint32_t)(mj >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mj, 0u));
            // 32-bit byte offsets from a wave-uniform base: scalar-base stores
            *reinterpret_cast<float *>(reinterpret_cast<char *>(ov) + slot * 4u) = f[j];
            *reinterpret_cast<int32_t *>(reinterpret_cast<char *>(oi) + slot * 4u) =
                CAND ? id[j] : id0 + j * kWave;
        }
        pos += (uint32_t)__popcll(mj);
    }
    if (threadIdx.x == 0) *cntp = total;
}

// Concatenates a row's slices (chunk order = position order) into the LDS buffer and selects
// exactly there.  counts[c] > CAPC marks a chunk that overflowed or found no threshold; then, or
// when the slices hold fewer than `need` or more than the buffer, the row is done by the
// one-workgroup path.  Every thread of the (NT-thread) block calls it.
template <int CAPC>
__device__ __forceinline__ void finish_row(Smem &sm, const Row &r, int need, int32_t *dst,
                                           const int *counts, const float *cval,
                                           const int32_t *cid, int nc)
{
    const int lane = lane_id(), w = wave_id();
    // every wave scans the counts itself (no block barrier); the first 64 stay in registers
    const int cfirst = lane < nc ? counts[lane] : 0;
    bool bad = cfirst > CAPC;
    int total = 0;
    {
        const int c = cfirst > CAPC ? 0 : cfirst;
        total = __shfl(wave_inclusive_scan(c), kWave - 1, kWave);
        for (int g = kWave; g < nc; g += kWave) {
            const int i = g + lane;
            int cg = i < nc ? counts[i] : 0;
            bad |= cg > CAPC;
            cg = cg > CAPC ? 0 : cg;
            total += __shfl(wave_inclusive_scan(cg), kWave - 1, kWave);
        }
    }
    // the same in every wave: every element >= T of the row sits in the slices, which hold at
    // least `need` elements and fit the buffer -- else the one-workgroup path over the row
    int nbuf = total;
    if (__ballot(bad) != 0 || total > CAP || total < need) {
        nbuf = prepare_buf(sm, r, need, dst);
    } else {
        int run = 0;
        for (int g = 0; g < nc; g += kWave) {
            const int cg = g == 0 ? cfirst : (g + lane < nc ? counts[g + lane] : 0);
            const int inc = wave_inclusive_scan(cg);
            const int off = run + inc - cg;
            run += __shfl(inc, kWave - 1, kWave);
            // this wave copies slices g + s, s = w, w + NW, ..., two at a time, two rounds of 64
            // entries each per pass: all of a pass's loads are issued (clamped to the slice's first
            // entry, or to slice g + w) before any is written
            const int ng = min(kWave, nc - g);
            for (int s0 = w; s0 < ng; s0 += 2 * NW) {
                int cs[2], os[2];
                const float *sv[2];
                const int32_t *si[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int sl = s0 + t * NW;
                    const bool ok = sl < ng;
                    cs[t] = ok ? __shfl(cg, sl, kWave) : 0;
                    os[t] = __shfl(off, ok ? sl : s0, kWave);
                    const int64_t slice = (int64_t)(g + (ok ? sl : s0)) * CAPC;
                    sv[t] = cval + slice;
                    si[t] = cid + slice;
                }
                const int cmax = max(cs[0], cs[1]);
                for (int e0 = 0; e0 < cmax; e0 += 2 * kWave) {
                    float v[2][2];
                    int32_t d[2][2];
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            const int e = e0 + u * kWave + lane;
                            const int ec = e < cs[t] ? e : 0;
                            v[t][u] = sv[t][ec];
                            d[t][u] = si[t][ec];
                        }
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            const int e = e0 + u * kWave + lane;
                            if (e < cs[t]) {
                                sm.buf_key[os[t] + e] = order_key(v[t][u]);
                                sm.buf_id[os[t] + e] = d[t][u];
                            }
                        }
                }
            }
        }
        __syncthreads();
    }
    if (nbuf >= 0) select_from_buf(sm, nbuf, need, dst);
}

// One workgroup per row: concatenates the row's slices into LDS and selects exactly there.
__global__ __launch_bounds__(NT) void chunk_finish_kernel(SelectArgs a, ChunkWs ws)
{
    __shared__ Smem sm;
    const int64_t row = blockIdx.x;
    Row r;
    int32_t *dst;
    int need;
    if (!setup_row(a, row, r, dst, need, true)) return;
    const int64_t base = row * ws.n_chunks;
    finish_row<CHUNK_CAP>(sm, r, need, dst, ws.count + base, ws.cval + base * CHUNK_CAP,
                          ws.cid + base * CHUNK_CAP, ws.n_chunks);
}

// The fused decode path where the row's scoring workgroups number at most one per wave of this
// block, one workgroup per row.  Scoring workgroup x kept, in its slice, every middle-region key
// of its range in bins >= its local bin L_x, in position order.  With Lmax the largest L_x, every
// slice holds all of its range's keys in bins >= Lmax, so the slices' entries in bins >= Lmax are
// exactly the row's keys there.  When they number at least `need` (and fit the buffer) the row's
// `need` best are among them: wave x counts its slice's entries in bins >= Lmax, a block scan of
// the counts places them (position order = workgroup order), and the buffer is selected exactly.
// Otherwise the row's threshold bin G comes from the scoring launch's histograms: a slice with
// L_x <= G provides its range's keys in bins >= G, any other range is read from the score row.
// A row whose bins >= G exceed the buffer takes the one-workgroup path.
struct SliceWs {
    const uint32_t *hist_fine, *hist_coarse;
    const int4 *hdr; // per scoring workgroup: {L, count, range begin, range end}
    const uint2 *ent; // per scoring workgroup: kSliceCap x {score bits, position}
    int groups;
};

constexpr int SLE = kSliceCap / kWave; // slice entries per lane
constexpr int SLE_FIRST = SLE / 2;     // loaded before the count is known

__global__ __launch_bounds__(NT) void slice_finish_kernel(SelectArgs a, SliceWs ws)
{
    __shared__ Smem sm;
    const int64_t row = blockIdx.x;
    Row r;
    int32_t *dst;
    int need;
    if (!setup_row(a, row, r, dst, need, true)) return;
    const int l = lane_id(), x = wave_id();
    const bool has = x < ws.groups; // wave-uniform
    const int64_t sx = row * ws.groups + x;
    // the first half of the slots is loaded with the header (slots past the count hold stale
    // values and are ignored); the rest only for a slice that holds more
    int4 h = make_int4(0, 0, 0, 0);
    uint2 e[SLE];
    const uint2 *pe = ws.ent + sx * kSliceCap;
    if (has) {
        h = ws.hdr[sx];
#pragma unroll
        for (int u = 0; u < SLE_FIRST; ++u) e[u] = pe[u * kWave + l];
    }
    const bool valid = !has || (h.y >= 0 && h.y <= kSliceCap); // wave-uniform
    if (has && h.y > SLE_FIRST * kWave) {
#pragma unroll
        for (int u = SLE_FIRST; u < SLE; ++u) e[u] = pe[u * kWave + l];
    }
    int *cnt = sm.cnt, *lbin = sm.cnt + NW; // NW counts, NW bins (sm.cnt holds ITEMS * NW)
    if (l == 0) lbin[x] = has ? (valid ? h.x : NBIN) : 0;
    __syncthreads();
    // lane i < groups reads slice i's entry (here and for the counts below)
    const uint32_t lmax = wave_reduce_u<true>(l < ws.groups ? (uint32_t)lbin[l] : 0u);
    // a slice's entries in bins >= T, in slot order, as (take, key, id) to `emit`
    auto slice = [&](uint32_t T, auto &&emit) {
#pragma unroll
        for (int u = 0; u < SLE; ++u) {
            if (u >= SLE_FIRST && h.y <= SLE_FIRST * kWave) break; // wave-uniform
            const uint32_t key = order_key(__uint_as_float(e[u].x));
            emit(u * kWave + l < h.y && (key >> 21) >= T, key, (int32_t)e[u].y);
        }
    };
    // the range's keys in bins >= T from the score row, four rounds of 64 positions in flight
    // (the range is clamped into the row's middle region, which it always lies in)
    const int64_t zlo = max((int64_t)h.z, r.lo), zhi = min((int64_t)h.w, r.hi);
    auto scan = [&](uint32_t T, auto &&emit) {
        for (int64_t p0 = zlo; p0 < zhi; p0 += 4 * kWave) {
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t p = p0 + u * kWave + l;
                v[u] = p < zhi ? r.sc[p] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t p = p0 + u * kWave + l;
                const uint32_t key = order_key(v[u]);
                emit(p < zhi && (key >> 21) >= T, key, (int32_t)p);
            }
        }
    };
    int c = 0;
    auto count = [&](bool tk, uint32_t, int32_t) { c += (int)__popcll(__ballot(tk)); };
    uint32_t pos = 0;
    auto put = [&](bool tk, uint32_t key, int32_t id) {
        const uint64_t m = __ballot(tk);
        if (tk) {
            const uint32_t slot = pos + __builtin_amdgcn_mbcnt_hi(
                                            (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (slot < (uint32_t)CAP) {
                sm.buf_key[slot] = key;
                sm.buf_id[slot] = id;
            }
        }
        pos += (uint32_t)__popcll(m);
    };
    // counts of every wave -> this wave's offset and the total (one barrier)
    auto place = [&](int &total) {
        if (l == 0) cnt[x] = c;
        __syncthreads();
        const int ci = l < ws.groups ? cnt[l] : 0;
        const int inc = wave_inclusive_scan(ci);
        total = __builtin_amdgcn_readlane(inc, kWave - 1);
        const int xu = __builtin_amdgcn_readfirstlane(x);
        pos = (uint32_t)(__builtin_amdgcn_readlane(inc, xu) - __builtin_amdgcn_readlane(ci, xu));
    };
    int nbuf = -1, total = 0;
    if (lmax < (uint32_t)NBIN) {
        if (has) slice(lmax, count);
        place(total);
        if (total >= need && total <= CAP) {
            if (has && c > 0) slice(lmax, put);
            __syncthreads();
            nbuf = total;
        } else {
            __syncthreads(); // every wave has read the counts before they are rewritten
        }
    }
    if (nbuf < 0) {
        const Digit g = hist_threshold<NT>(sm.hist, sm.scratch, ws.hist_fine, ws.hist_coarse,
                                           ws.groups, row, need);
        const uint32_t Tg = g.d >= 0 ? (uint32_t)g.d << 21 : 0u;
        if (!(g.d >= 0 && g.above + g.at <= CAP && Tg > order_key(-INFINITY))) {
            nbuf = prepare_buf(sm, r, need, dst);
        } else {
            const uint32_t G = (uint32_t)g.d;
            const bool from_slice = valid && h.x <= g.d; // wave-uniform
            c = 0;
            if (has) {
                if (from_slice)
                    slice(G, count);
                else
                    scan(G, count);
            }
            place(total);
            nbuf = min(total, CAP);
            if (has && c > 0) {
                if (from_slice)
                    slice(G, put);
                else
                    scan(G, put);
            }
            __syncthreads();
        }
    }
    if (nbuf >= 0) select_from_buf(sm, nbuf, need, dst);
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

int select_slice_groups_max() { return NW; }

hipError_t launch_select_slices(const SelectArgs &a, const uint32_t *hist_fine,
                                const uint32_t *hist_coarse, const int4 *slice_hdr,
                                const uint2 *slice_ent, int groups, hipStream_t stream)
{
    const int64_t rows = (int64_t)a.batch * a.n_q;
    if (rows == 0) return hipSuccess;
    if (a.cand_ids || a.mode != SELECT_SI || groups < 1 || groups > NW) return hipErrorInvalidValue;
    const SliceWs w{hist_fine, hist_coarse, slice_hdr, slice_ent, groups};
    hipLaunchKernelGGL(slice_finish_kernel, dim3((unsigned)rows), dim3(NT), 0, stream, a, w);
    return hipGetLastError();
}

hipError_t launch_select(const SelectArgs &a, void *ws, hipStream_t stream)
{
    return launch_select_hist(a, ws, nullptr, nullptr, 0, stream);
}

hipError_t launch_select_hist(const SelectArgs &a, void *ws, const uint32_t *hist_fine,
                              const uint32_t *hist_coarse, int groups, hipStream_t stream)
{
    const int64_t rows = (int64_t)a.batch * a.n_q;
    if (rows == 0) return hipSuccess;
    if (!use_chunked(a)) {
        if (a.cand_ids)
            hipLaunchKernelGGL(select_kernel_cand, dim3((unsigned)rows), dim3(NT), 0, stream, a);
        else if (a.n_in > CAP && a.n_in <= (int64_t)NT * RI)
            hipLaunchKernelGGL(select_kernel_regs, dim3((unsigned)rows), dim3(NT), 0, stream, a);
        else
            hipLaunchKernelGGL(select_kernel_flat, dim3((unsigned)rows), dim3(NT), 0, stream, a);
        return hipGetLastError();
    }
    const int64_t nc = (a.n_in + CHUNK - 1) / CHUNK;
    auto r256 = [](size_t x) { return (x + 255) / 256 * 256; };
    uint8_t *p = static_cast<uint8_t *>(ws);
    ChunkWs w;
    w.count = reinterpret_cast<int *>(p);
    p += r256(rows * nc * 4);
    w.cval = reinterpret_cast<float *>(p);
    p += r256(rows * nc * CHUNK_CAP * 4);
    w.cid = reinterpret_cast<int32_t *>(p);
    w.n_chunks = (int)nc;
    w.hist_fine = a.cand_ids ? nullptr : hist_fine;
    w.hist_coarse = hist_coarse;
    w.groups = groups;
    if (a.cand_ids)
        hipLaunchKernelGGL(chunk_collect_kernel<true>, dim3((unsigned)nc, (unsigned)rows),
                           dim3(CNT_THREADS), 0, stream, a, w);
    else
        hipLaunchKernelGGL(chunk_collect_kernel<false>, dim3((unsigned)nc, (unsigned)rows),
                           dim3(CNT_THREADS), 0, stream, a, w);
    hipLaunchKernelGGL(chunk_finish_kernel, dim3((unsigned)rows), dim3(NT), 0, stream, a, w);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Library-held scratch for the selection's chunked path, for callers that cannot allocate.
// One fixed array per device (the code object's own copy on each GPU, alive until the process
// ends).  Host code never uses the array's name as an address: the first call on a device asks
// the runtime for that device's address of it and keeps it.
// ------------------------------------------------------------------------------------------
constexpr size_t kSelectScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kSelectScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];
} // namespace

size_t select_scratch_bytes() { return kSelectScratchBytes; }

hipError_t select_scratch(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

} // namespace lsa
