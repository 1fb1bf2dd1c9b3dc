// score.hip -- Lightning-Indexer scoring on gfx950 bf16 MFMA.
//
//   I[t,s] = sum_h w[t,h] * ReLU( q[t,h] . k[s] )       (times scale[s] for e4m3 keys)
//
// (Baidu Cloud article on DeepSeek's Lightning Indexer, "1. Lightweight Scoring Module": ReLU of
// query-key dot products; the indexer weights its heads per query.)
//
// The contraction over d runs on v_mfma_f32_32x32x16_bf16: the M dimension holds indexer rows
// (query, head) pairs, N holds 32 keys, K is d.  The ReLU, the head weights and the head sum are
// fused into the epilogue on the fp32 accumulators, so only one fp32 per (query, key) leaves the
// kernel.  e4m3 keys are widened to bf16 exactly (gfx950 cvt_scalef32_pk_bf16_fp8, unit scale) and
// their per-token scale is applied once after the head sum.
//
// Two kernels:
//  * stream: each wave owns its own 32-key blocks, loads them from HBM in contiguous 16-byte
//    pieces (non-temporal: no reuse between waves, since decode has one query per sequence and
//    the key cache is read exactly once) and passes them through its own LDS slab into the MFMA
//    operand layout.  Also runs the fine stage of Hierarchical Indexing, where
//    the blocks come from each query's recalled pages.
//  * tile: prefill.  A workgroup owns WAVES*NQW queries; key tiles (256 keys at 64 heads of
//    width 128, 128 keys otherwise) are staged once in LDS (bf16, padded rows) and shared by
//    every wave, double-buffered against the next tile's global loads.  With fp8 queries the
//    same kernel runs on the 8-bit MFMA.
//
// Operand layout.  The two lane halves split d: half g = l/32 holds d in [g*D/2, (g+1)*D/2);
// K-step kk feeds d = g*D/2 + 8*kk + [0,8) as the MFMA's K index 8*g + [0,8).  This permutes the
// contraction index identically for q and k, so a lane loads D/2 contiguous elements of a key
// row.  Accumulator register r of M-tile mt in lane half g is indexer row
//   r' = 16*MT*g + 16*mt + r,   (query slot, head) = (r' / H, r' % H)
// so with 16*MT >= H every lane holds whole queries and the head sum stays in the lane; with
// H = 32*MT the two halves each hold half of one query's heads and one cross-half add finishes.
#include <algorithm>
#include <type_traits>

#include "device.hpp"
#include "internal.hpp"

namespace lsa {
namespace {

// Indexer-row geometry of a wave.
template <int H, int MT, bool ONEQ>
struct Geo {
    static constexpr int ROWS = 32 * MT;
    static constexpr int VPL = 16 * MT;                       // accumulator values per lane
    static constexpr bool SPLIT = ONEQ || (H > VPL);          // query spans both lane halves
    static constexpr int NQW = ONEQ ? 1 : (ROWS / H);         // queries per wave
    static constexpr int NQL = SPLIT ? 1 : (VPL / H);         // queries per lane half
    static_assert(ONEQ || ROWS % H == 0, "heads must divide the wave's rows");
    static_assert(ONEQ || H <= VPL || H == ROWS, "unsupported head split");
};

// Indexer row r' of A-operand row rho of M-tile mt.
template <int MT>
__device__ __forceinline__ int a_row_to_rprime(int mt, int rho)
{
    return 16 * MT * ((rho >> 2) & 1) + 16 * mt + 4 * (rho >> 3) + (rho & 3);
}

template <int H, bool ONEQ>
__device__ __forceinline__ void rprime_to_qh(int rp, int &qs, int &h, bool &valid)
{
    if (ONEQ) {
        qs = 0;
        h = rp;
        valid = rp < H;
    } else {
        qs = rp / H;
        h = rp % H;
        valid = true;
    }
}

// Valid key range [lo, hi) of query t of sequence b.
__device__ __forceinline__ void row_range(const ScoreArgs &a, int b, int64_t t, int64_t &lo,
                                          int64_t &hi)
{
    const int64_t V = valid_len(a.seq_len, a.seq_pos0, b, t, a.kv_len, a.q_pos0);
    if (a.mask == MASK_CAUSAL) {
        lo = 0;
        hi = V;
    } else { // MASK_PAGES
        if (V <= a.k) {
            lo = 0;
            hi = 0;
        } else {
            lo = a.sink / a.page;
            hi = (V - a.window - 1) / a.page + 1;
        }
    }
}

template <int D, int H, int MT, bool ONEQ>
__device__ __forceinline__ void load_q(bf16x8_t (&qf)[MT][D / 16], const uint16_t *qbase,
                                       int nq_avail)
{
    const int l = lane_id(), rho = l & 31, gk = l >> 5;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        int qs, h;
        bool valid;
        rprime_to_qh<H, ONEQ>(a_row_to_rprime<MT>(mt, rho), qs, h, valid);
        valid = valid && qs < nq_avail;
        const uint16_t *src = qbase + ((int64_t)qs * H + h) * D + (D / 2) * gk;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            uint4 v = valid ? *reinterpret_cast<const uint4 *>(src + 8 * kk) : make_uint4(0, 0, 0, 0);
            qf[mt][kk] = bitcast<bf16x8_t>(v);
        }
    }
}

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// fp8 query fragments for v_mfma_f32_32x32x64_f8f6f4: lane l supplies A row l%32 (the indexer
// row of load_q) and 32 codes of it; lane half g takes d in [g*D/2, (g+1)*D/2), K-step kk the 32
// codes g*D/2 + 32*kk + [0, 32) -- the same (half, byte) -> d map the key operand uses, so the
// contraction covers every d once.
template <int D, int H, int MT>
__device__ __forceinline__ void load_q8(i32x8_t (&qf)[MT][D / 64], const uint8_t *qbase,
                                        int nq_avail)
{
    const int l = lane_id(), rho = l & 31, gk = l >> 5;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        int qs, h;
        bool valid;
        rprime_to_qh<H, false>(a_row_to_rprime<MT>(mt, rho), qs, h, valid);
        valid = valid && qs < nq_avail;
        const uint8_t *src = qbase + ((int64_t)qs * H + h) * D + (D / 2) * gk;
#pragma unroll
        for (int kk = 0; kk < D / 64; ++kk) {
            const uint4 x = valid ? ld16(src + 32 * kk) : make_uint4(0, 0, 0, 0);
            const uint4 y = valid ? ld16(src + 32 * kk + 16) : make_uint4(0, 0, 0, 0);
            qf[mt][kk] = i32x8_t{(int)x.x, (int)x.y, (int)x.z, (int)x.w,
                                 (int)y.x, (int)y.y, (int)y.z, (int)y.w};
        }
    }
}

// D(32x32, fp32) += A(32x64, e4m3) * B(64x32, e4m3), no block scales: lane l supplies A row
// l%32 and B column l%32 with the same 32 K slots for the same (l/32, byte); D in the layout of
// mfma_32x32x16.
__device__ __forceinline__ f32x16_t mfma_32x32x64_f8(i32x8_t a, i32x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int H, int MT, bool ONEQ>
__device__ __forceinline__ void load_w(float (&wv)[16 * MT], const float *wbase, int nq_avail)
{
    const int g = lane_id() >> 5;
#pragma unroll
    for (int v = 0; v < 16 * MT; ++v) {
        int qs, h;
        bool valid;
        rprime_to_qh<H, ONEQ>(16 * MT * g + v, qs, h, valid);
        wv[v] = (valid && qs < nq_avail) ? wbase[qs * H + h] : 0.0f;
    }
}

// ReLU, head weights and head sum over the lane's accumulators.  part[u] is the partial score of
// lane-half query slot u (all slots complete unless SPLIT, where a cross-half add follows).
// wf(v) is the head weight of accumulator value v of this lane (registers or LDS).
template <int H, int MT, bool ONEQ, typename WF>
__device__ __forceinline__ void epilogue(const f32x16_t (&acc)[MT], WF wf,
                                         float (&part)[Geo<H, MT, ONEQ>::NQL])
{
    using G = Geo<H, MT, ONEQ>;
    // four independent accumulation chains per query slot, combined in a fixed order
    constexpr int NC = H >= 4 ? 4 : H;
    float p[G::NQL][NC];
#pragma unroll
    for (int u = 0; u < G::NQL; ++u)
#pragma unroll
        for (int c = 0; c < NC; ++c) p[u][c] = 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int v = 16 * mt + r;
            const int u = G::SPLIT ? 0 : v / H;
            p[u][r % NC] = fmaf(wf(v), relu(acc[mt][r]), p[u][r % NC]);
        }
    }
#pragma unroll
    for (int u = 0; u < G::NQL; ++u) part[u] = (p[u][0] + p[u][1]) + (p[u][2] + p[u][3]);
    if (G::SPLIT) { // lanes l < 32 receive lane l + 32's partial (gfx950 v_permlane32_swap)
        const float other = bitcast<float>(__builtin_amdgcn_permlane32_swap(
            bitcast<uint32_t>(part[0]), bitcast<uint32_t>(part[0]), false, false)[1]);
        part[0] += other;
    }
}

// ------------------------------------------------------------------------------------------
// stream kernel
// ------------------------------------------------------------------------------------------

// A block of 32 consecutive key rows, loaded with fully contiguous 16-byte pieces (lane l of
// piece i reads bytes 1024*i + 16*l of the block: every load instruction covers 1 KB of HBM
// without gaps), then passed through the wave's LDS slab to reach the MFMA operand layout.
// In the slab, 16-byte chunk c of row n sits at chunk slot c ^ (n & SW): the writes of 8
// consecutive lanes cover one row and the operand reads of 8 consecutive lanes hit 8 rows, and
// both land on distinct banks.
template <bool FP8, int D>
struct KeyBlock {
    static constexpr int ESZ = FP8 ? 1 : 2;
    static constexpr int RB = D * ESZ;                  // bytes per key row
    static constexpr int BB = 32 * RB;                  // bytes per block
    static constexpr int NP = BB / 1024;                // 16-byte pieces per lane
    static constexpr int CPR = RB / 16;                 // chunks per row
    static constexpr int SW = (CPR < 8 ? CPR : 8) - 1;  // swizzle mask
    static_assert(BB % 1024 == 0, "whole pieces");
    uint4 raw[NP];

    __device__ __forceinline__ void load(const uint8_t *keys_b, int64_t row0, int64_t n_keys, int l)
    {
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int f = i * kWave + l;
            int64_t row = row0 + f / CPR;
            if (row >= n_keys) row = n_keys - 1; // tail block: any valid row, masked later
            raw[i] = ld16(keys_b + row * RB + (f % CPR) * 16);
        }
    }
    __device__ __forceinline__ void to_slab(uint8_t *slab, int l) const
    {
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int f = i * kWave + l;
            const int n = f / CPR, c = f % CPR;
            *reinterpret_cast<uint4 *>(slab + n * RB + ((c ^ (n & SW)) * 16)) = raw[i];
        }
    }
    // Operand chunk j (16 bytes) of lane (n = l%32, half g): key bytes [RB/2*g + 16j, +16).
    __device__ static __forceinline__ uint4 chunk(const uint8_t *slab, int l, int j)
    {
        const int n = l & 31, c = (CPR / 2) * (l >> 5) + j;
        return *reinterpret_cast<const uint4 *>(slab + n * RB + ((c ^ (n & SW)) * 16));
    }
};

// LDS stage of a scoring workgroup's scores for the fused selection's slice: block b (32
// positions) of the workgroup's range sits in quarter b / 64 at column b % 64, position j of the
// block in row j of 65 words (the padding keeps both the block's write and the column reads of
// the compaction free of bank conflicts).
constexpr int kStageQ = 32 * 65;
__device__ __forceinline__ int stage_index(int blk, int j) { return (blk >> 6) * kStageQ + j * 65 + (blk & 63); }

// The fused selection's slice of one scoring workgroup (flat decode launch, after its histogram
// and stage are complete).  Every wave finds the highest bin L whose suffix count in the
// workgroup's histogram reaches a.slice_target (one bin higher if that would keep more than
// kSliceCap; 0 = every bin when the workgroup holds fewer), then compacts the scores of its
// quarter of the range in bins >= L: lane l takes block 64 w + l, so lane order is position
// order and a lane's picks are contiguous.  Positions outside the middle region [o_lo, o_hi) are
// skipped.  Wave 0 also leaves the 32 coarse sums of the histogram in `lcoarse`.  A selection
// whose row threshold bin is >= L finds all of this range's candidates in the slice.
template <int WAVES>
__device__ __forceinline__ void slice_compact(const ScoreArgs &a, const uint32_t *lhist,
                                              uint32_t *lcoarse, const float *lsc, int64_t slice,
                                              int64_t o_base, int64_t o_lo, int64_t o_hi)
{
    static_assert(WAVES * 64 * 32 == kSliceSpan, "one quarter of 64 blocks per wave");
    __shared__ int sinfo[WAVES];
    __shared__ uint32_t lcw[WAVES - 1][32]; // the coarse sums of waves 1.. (wave 0: lcoarse)
    const int l = lane_id(), w = wave_id();
    // The 32 coarse sums (64 bins each), read without bank conflicts: lane l sums the 4-bin
    // chunks l + 64 i (i < 8), which lie in group l / 16 + 4 i; a scan over each 16-lane row
    // leaves a group's sum in the row's last lane.  Each wave keeps its own copy in LDS (a wave's
    // LDS accesses complete in order: no barrier).
    uint32_t *cw = w == 0 ? lcoarse : lcw[w - 1];
    {
        const uint4 *h4 = reinterpret_cast<const uint4 *>(lhist);
        uint32_t part[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint4 x = h4[l + 64 * i];
            part[i] = x.x + x.y + x.z + x.w;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            part[i] = row_inclusive_scan(part[i]);
            if ((l & 15) == 15) cw[(l >> 4) + 4 * i] = part[i];
        }
    }
    const uint32_t c = l < 32 ? cw[31 - l] : 0u; // lane i < 32: coarse group 31 - i (top down)
    const int t = a.slice_target;
    const int inc = wave_inclusive_scan((int)c);
    const uint64_t ge = __ballot(l < 32 && inc >= t);
    uint32_t L = 0;
    if (ge) {
        const int g = (int)__builtin_ctzll(ge), grp = 31 - g;
        const int exg = __builtin_amdgcn_readlane(inc, g) - __builtin_amdgcn_readlane((int)c, g);
        const int f = (int)lhist[64 * grp + 63 - l];
        const int inc2 = exg + wave_inclusive_scan(f);
        const int i = (int)__builtin_ctzll(__ballot(inc2 >= t)); // exists: the group reaches t
        L = (uint32_t)(64 * grp + 63 - i);
        if (__builtin_amdgcn_readlane(inc2, i) > kSliceCap) L += 1;
    }
    // Per lane, not per position: a lane's 32 positions are consecutive, so a bit mask and one
    // wave scan of the lane counts order the picks, and the write loop runs over picks only.
    const int q0 = (64 * w + l) * 32; // the lane's first position, relative to o_base
    const int lo = (int)(o_lo - o_base), hi = max(lo, (int)(o_hi - o_base)); // may be empty
    const float *col = lsc + w * kStageQ + l;
    // key(f) >> 21 >= L as one float comparison: f >= the float whose key is L << 21 (every
    // finite f when L << 21 lies below key(-inf), none when L is past the last bin: NaN).
    // Every read is issued before any is used; stage slots outside the middle region hold stale
    // values and are masked out.
    const uint32_t T = L << 21;
    const float tf = L <= 3u      ? -INFINITY
                     : L >= 2048u ? __uint_as_float(0x7fc00000u)
                                  : __uint_as_float((T & 0x80000000u) ? T & 0x7fffffffu : ~T);
    uint32_t mask = 0;
#pragma unroll 8
    for (int j = 0; j < 32; ++j) {
        const uint32_t in = (uint32_t)(q0 + j - lo) < (uint32_t)(hi - lo);
        mask |= (in & (uint32_t)(col[j * 65] >= tf)) << j;
    }
    const int cnt = __popc(mask);
    const int incl = wave_inclusive_scan(cnt);
    if (l == kWave - 1) sinfo[w] = incl;
    __syncthreads();
    int base = 0, total = 0;
    for (int i = 0; i < WAVES; ++i) {
        const int x = sinfo[i];
        base += i < w ? x : 0;
        total += x;
    }
    uint2 *ent = a.slice_ent + slice * kSliceCap;
    uint32_t slot = (uint32_t)(base + incl - cnt);
    const uint32_t p0 = (uint32_t)o_base + (uint32_t)q0;
    // total <= kSliceCap by the choice of L
    for (uint32_t m = mask; m != 0u && slot < (uint32_t)kSliceCap; m &= m - 1u, ++slot) {
        const int j = __builtin_ctz(m);
        ent[slot] = make_uint2(__float_as_uint(col[j * 65]), p0 + (uint32_t)j);
    }
    if (threadIdx.x == 0)
        a.slice_hdr[slice] = make_int4((int)L, total, (int)o_lo, (int)max(o_hi, o_lo));
}

// PD: blocks prefetched ahead of the one being computed (register ring of PD + 1 blocks).
// BPW > 0: each wave takes BPW blocks, the block loop fully unrolled.  BPW == 0: each wave takes
// ceil(blocks / (gridDim.x * WAVES)) blocks in a loop whose body is one turn of the ring, so
// every ring slot is still a compile-time constant while the code stays one ring long.
// HIST (flat decode launch, one query per workgroup): the workgroup also counts its middle-region
// scores [S, V-W) into a 2048-bin LDS histogram of key bits 31..21 while they are in registers,
// and writes it (32 coarse sums of 64 bins, and the fine bins of the non-empty groups) to its
// slice of a.hist_fine / a.hist_coarse, so the selection that follows reads the row's exact
// threshold bin instead of sampling the row.  With a.slice_ent (a workgroup owns at most
// kSliceSpan keys) it also stages those scores in LDS and leaves its slice (slice_compact).
// PAGED: the keys (and scales) are pools of blocks of 2^lbs >= 32 rows under a block table.  A
// 32-key block then lies inside one table block (blocks start at multiples of 32 and the last
// one is not moved back: its rows past the keys are pool rows of the same table block, read and
// masked).  The workgroup's table entries are cached in LDS first, so a lookup waits on LDS
// only, never behind the key loads in flight.
template <bool FP8, int D, int H, int MT, bool ONEQ, bool FINE, int WAVES, int BPW, int PD = 1,
          bool HIST = false, bool PAGED = false>
__global__ __launch_bounds__(WAVES *kWave) void score_stream_kernel(ScoreArgs a)
{
    using G = Geo<H, MT, ONEQ>;
    using KB = KeyBlock<FP8, D>;
    constexpr int KS = D / 16;
    static_assert(PD >= 1 && (BPW == 0 || PD < BPW), "ring shape");
    static_assert(!HIST || (BPW == 0 && !FINE && G::NQW == 1 && G::SPLIT), "histogram launch");
    constexpr int HBINS = 2048;
    // two slabs per wave: block i is transposed in slab i&1 while block i-1 may still be read
    __shared__ __attribute__((aligned(16))) uint8_t slabs[WAVES][2][KB::BB];
    __shared__ __attribute__((aligned(16))) uint32_t lhist[HIST ? HBINS : 4];
    // HIST with slices: the workgroup's middle-region scores, by position within its range
    __shared__ float lsc[HIST ? kSliceSpan / 2048 * kStageQ : 1];
    if constexpr (HIST) {
        for (int i = threadIdx.x; i < HBINS / 4; i += WAVES * kWave)
            reinterpret_cast<uint4 *>(lhist)[i] = make_uint4(0u, 0u, 0u, 0u);
        __syncthreads();
    }
    const int b = blockIdx.z;
    const int64_t t0 = (int64_t)blockIdx.y * G::NQW;
    const int nq_avail = (int)min((int64_t)G::NQW, (int64_t)a.n_q - t0);
    const int l = lane_id(), wv_id = wave_id(), g = l >> 5, n = l & 31;

    bf16x8_t qf[MT][KS];
    load_q<D, H, MT, ONEQ>(qf, a.q + ((int64_t)b * a.n_q + t0) * H * D, nq_avail);
    float wv[G::VPL];
    load_w<H, MT, ONEQ>(wv, a.w + ((int64_t)b * a.n_q + t0) * H, nq_avail);

    // Valid ranges of the lane's query slots, their hull and their intersection.
    int64_t lo[G::NQL], hi[G::NQL];
    int64_t lo_all = INT64_MAX, hi_all = 0;
    int64_t lo_in = 0, hi_in = INT64_MAX;
#pragma unroll
    for (int u = 0; u < G::NQL; ++u) {
        const int qs = G::SPLIT ? 0 : g * G::NQL + u;
        if (qs < nq_avail) {
            row_range(a, b, t0 + qs, lo[u], hi[u]);
        } else {
            lo[u] = 0;
            hi[u] = 0;
        }
    }
    if (FINE) {
        const int64_t V = valid_len(a.seq_len, a.seq_pos0, b, t0, a.kv_len, a.q_pos0);
        lo_all = lo_in = a.sink;
        hi_all = hi_in = V > a.k ? V - a.window : 0;
        lo[0] = lo_all;
        hi[0] = hi_all;
    } else {
        for (int qs = 0; qs < nq_avail; ++qs) {
            int64_t x, y;
            row_range(a, b, t0 + qs, x, y);
            lo_in = max(lo_in, x);
            hi_in = min(hi_in, y);
            if (y > x) {
                lo_all = min(lo_all, x);
                hi_all = max(hi_all, y);
            }
        }
    }
    hi_in = min(hi_in, a.n_keys);
    // middle region of the (single) query row, for the histogram
    int64_t mid_lo = 0, mid_hi = 0;
    if constexpr (HIST) {
        if (hi[0] > a.k) {
            mid_lo = a.sink;
            mid_hi = hi[0] - a.window;
        }
    }

    const uint8_t *keys_b = reinterpret_cast<const uint8_t *>(a.keys) +
                            (PAGED ? 0 : (int64_t)b * a.n_keys * KB::RB); // a pool: pool rows
    const float *scale_b = FP8 ? a.kscale + (PAGED ? 0 : (int64_t)b * a.n_keys) : nullptr;
    const int32_t *pages_row = FINE ? a.pages + ((int64_t)b * a.n_q + t0) * a.m_pages : nullptr;
    const int64_t n_blocks = (a.n_out + 31) / 32;
    // blocks per wave; the workgroup's waves interleave over its contiguous range of blocks
    const int bpw = BPW ? BPW : (int)((n_blocks + (int64_t)gridDim.x * WAVES - 1) /
                                      ((int64_t)gridDim.x * WAVES));
    // the slices need the workgroup's range staged whole in LDS (the host launches them so)
    const bool stage = HIST && a.slice_ent && bpw * WAVES * 32 <= kSliceSpan;
    // PAGED: the table entries of the workgroup's blocks [x * bpw * WAVES, (x + 1) * bpw * WAVES)
    // (the host keeps them within kPagedTab; entries past the table read as outside the pool)
    __shared__ int32_t ptab[PAGED && !FINE ? kPagedTab : 1];
    int64_t pg0 = 0;
    if constexpr (PAGED && !FINE) {
        pg0 = ((int64_t)blockIdx.x * bpw * WAVES * 32) >> a.lbs;
        const int32_t *tab_b = a.btab + (int64_t)b * a.bps;
        for (int i = threadIdx.x; i < kPagedTab; i += WAVES * kWave)
            ptab[i] = pg0 + i < a.bps ? tab_b[pg0 + i] : -1;
        __syncthreads();
    }
    // pool row of key row `row` (a multiple of 32 in the workgroup's range), -1: outside the pool.
    // FINE: the rows of a recalled page, one table block per block of 32 (a wave-uniform load)
    auto pool_row = [&](int64_t row) -> int64_t {
        const int32_t e = FINE ? a.btab[(int64_t)b * a.bps + (row >> a.lbs)]
                               : ptab[(int)((row >> a.lbs) - pg0)];
        return e >= 0 && e < a.n_blocks ? ((int64_t)e << a.lbs) | (row & ((int64_t(1) << a.lbs) - 1))
                                        : int64_t(-1);
    };
    // this lane's byte offsets inside a block (contiguous 1 KB pieces)
    uint32_t lane_off[KB::NP];
#pragma unroll
    for (int i = 0; i < KB::NP; ++i) {
        const int f = i * kWave + l;
        lane_off[i] = (uint32_t)((f / KB::CPR) * KB::RB + (f % KB::CPR) * 16);
    }

    struct Blk {
        int64_t s0, row0; // first output slot and first key row of the block
        int64_t fresh;    // rows below this were already covered by the previous block
        int64_t pool;     // PAGED: pool row of row0 (-1: outside the pool; its scores are -inf)
        bool valid, live;
    };
    // BPW == 0 (flat rows, n_out == n_keys >= 32): every block is loaded in full and without a
    // branch, since a conditional load makes the compiler drain all loads in flight where the
    // branches merge.  The last block is moved back to end at the last key (its rows overlap
    // the previous block's, whose scores it rewrites identically); blocks past the end reload
    // the last one and are not computed.
    constexpr bool FLAT_LOOP = BPW == 0 && !FINE;
    auto locate = [&](int it) {
        Blk k;
        const int64_t blk = ((int64_t)blockIdx.x * bpw + it) * WAVES + wv_id;
        k.valid = blk < n_blocks;
        k.fresh = 0;
        k.pool = 0;
        if constexpr (FLAT_LOOP) {
            k.s0 = k.row0 = PAGED ? blk * 32 : min(blk * 32, a.n_keys - 32);
            k.fresh = blk * 32;
            k.live = k.valid && k.s0 < hi_all && k.s0 + 32 > lo_all;
            if constexpr (PAGED) k.pool = pool_row(k.row0);
            return k;
        }
        k.s0 = blk * 32;
        k.live = false;
        k.row0 = 0;
        if (!k.valid) return k;
        if (FINE) {
            const int64_t pi = k.s0 / a.page;
            const int pid = pages_row[pi];
            k.row0 = (int64_t)pid * a.page + (k.s0 - pi * a.page);
            k.live = pid >= 0 && k.row0 < hi_all && k.row0 + 32 > lo_all;
            if constexpr (PAGED) k.pool = k.live ? pool_row(k.row0) : 0;
        } else {
            k.row0 = k.s0;
            k.live = k.s0 < hi_all && k.s0 + 32 > lo_all;
            if constexpr (PAGED) k.pool = pool_row(k.row0);
        }
        return k;
    };
    const uint8_t *dummy_base =
        (int64_t)a.batch * a.n_q * H * D * 2 >= KB::BB ? reinterpret_cast<const uint8_t *>(a.q)
                                                        : keys_b;
    auto fetch = [&](const Blk &k, KB &kb, float &sc, bool dummy = false) {
        if constexpr (PAGED) { // the whole block from one table block (pool row 0 if outside)
            if (!FLAT_LOOP && !k.live) return;
            const int64_t r0 = k.pool < 0 ? 0 : k.pool;
            const uint8_t *base = FLAT_LOOP && dummy ? dummy_base : keys_b + r0 * KB::RB;
#pragma unroll
            for (int i = 0; i < KB::NP; ++i) kb.raw[i] = ld16_nt(base + lane_off[i]);
            if (FP8) sc = scale_b[r0 + n];
            return;
        }
        if constexpr (FLAT_LOOP) { // keys are read once: non-temporal (about 10% faster)
            // a prefetch past the wave's last block (never used) reads a cached, in-bounds
            // block instead: q when it holds a block's bytes, else the sequence's first keys
            const uint8_t *base = dummy ? dummy_base : keys_b + k.row0 * KB::RB;
#pragma unroll
            for (int i = 0; i < KB::NP; ++i) kb.raw[i] = ld16_nt(base + lane_off[i]);
            if (FP8) sc = scale_b[k.row0 + n];
            return;
        }
        if (!k.live) return;
        if (k.row0 + 32 <= a.n_keys) {
            const uint8_t *base = keys_b + k.row0 * KB::RB;
#pragma unroll
            for (int i = 0; i < KB::NP; ++i) kb.raw[i] = ld16_nt(base + lane_off[i]);
            if (FP8) sc = scale_b[k.row0 + n];
        } else {
            kb.load(keys_b, k.row0, a.n_keys, l);
            if (FP8) sc = scale_b[min(k.row0 + n, a.n_keys - 1)];
        }
    };

    Blk bq[PD + 1];
    KB kq[PD + 1];
    float sq[PD + 1];
    static_for<0, PD>([&](auto I) {
        constexpr int i = decltype(I)::value;
        bq[i] = locate(FLAT_LOOP ? min(i, bpw - 1) : i);
        sq[i] = 1.0f;
        fetch(bq[i], kq[i], sq[i]);
    });
    // block `it` of the wave, held in ring slot CS = it % (PD + 1)
    auto step = [&](auto CS, int it) {
        constexpr int cs = decltype(CS)::value;
        constexpr int ns = (cs + PD) % (PD + 1); // slot that receives block it + PD
        if (it >= bpw) return;
        if constexpr (FLAT_LOOP) { // past the wave's last block: a dummy load (see fetch)
            bq[ns] = locate(min(it + PD, bpw - 1));
            fetch(bq[ns], kq[ns], sq[ns], it + PD >= bpw);
        } else if (it + PD < bpw) {
            bq[ns] = locate(it + PD);
            sq[ns] = 1.0f;
            fetch(bq[ns], kq[ns], sq[ns]);
        }
        const Blk cb = bq[cs];
        if (!cb.valid) return; // later blocks are past the end too

        float part[G::NQL];
        if (cb.live) {
            uint8_t *slab = slabs[wv_id][it & 1];
            f32x16_t acc[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16_t{};
            // through the slab into operand layout (a wave's LDS accesses complete in order)
            kq[cs].to_slab(slab, l);
#pragma unroll
            for (int j = 0; j < KB::CPR / 2; ++j) {
                const uint4 c = KB::chunk(slab, l, j);
                if (FP8) { // one chunk = two K-steps
                    const bf16x8_t b0 = e4m3x8_to_bf16x8(make_uint2(c.x, c.y));
                    const bf16x8_t b1 = e4m3x8_to_bf16x8(make_uint2(c.z, c.w));
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma_32x32x16(qf[mt][2 * j], b0, acc[mt]);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma_32x32x16(qf[mt][2 * j + 1], b1, acc[mt]);
                } else {
                    const bf16x8_t b0 = bitcast<bf16x8_t>(c);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma_32x32x16(qf[mt][j], b0, acc[mt]);
                }
            }
            epilogue<H, MT, ONEQ>(acc, [&](int v) { return wv[v]; }, part);
            if (FP8) {
#pragma unroll
                for (int u = 0; u < G::NQL; ++u) part[u] *= sq[cs];
            }
            if constexpr (PAGED) {
                if (cb.pool < 0) {
#pragma unroll
                    for (int u = 0; u < G::NQL; ++u) part[u] = -INFINITY;
                }
            }
        }

        if (!(G::SPLIT && g != 0)) {
            // a block inside every query's range and inside the output needs no lane masks
            const bool full = cb.live && cb.row0 >= lo_in && cb.row0 + 32 <= hi_in &&
                              cb.s0 + 32 <= a.n_out && nq_avail == G::NQW;
            float *ob = a.out + ((int64_t)b * a.n_q + t0) * a.n_out + cb.s0;
            int32_t *ib = FINE ? a.out_ids + ((int64_t)b * a.n_q + t0) * a.n_out + cb.s0 : nullptr;
            if constexpr (HIST) {
                // each key once (the moved-back last block skips the rows it repeats), middle
                // region only
                const int64_t row = cb.row0 + n;
                if (cb.live && row >= cb.fresh && row >= mid_lo && row < mid_hi) {
                    atomicAdd(&lhist[order_key(part[0]) >> 21], 1u);
                    // block `it` of wave w is block it * WAVES + w of the workgroup's range
                    if (stage) lsc[stage_index(it * WAVES + wv_id, (int)(row - cb.fresh))] = part[0];
                }
            }
            if (full) {
#pragma unroll
                for (int u = 0; u < G::NQL; ++u) {
                    const int qs = G::SPLIT ? 0 : g * G::NQL + u;
                    ob[(int64_t)qs * a.n_out + n] = part[u];
                    if (FINE) ib[(int64_t)qs * a.n_out + n] = (int32_t)(cb.row0 + n);
                }
            } else {
                const int64_t row = cb.row0 + n;
#pragma unroll
                for (int u = 0; u < G::NQL; ++u) {
                    const int qs = G::SPLIT ? 0 : g * G::NQL + u;
                    if (qs >= nq_avail || cb.s0 + n >= a.n_out) continue;
                    const bool ok = cb.live && row >= lo[u] && row < hi[u] && row < a.n_keys;
                    ob[(int64_t)qs * a.n_out + n] = ok ? part[u] : -INFINITY;
                    if (FINE) ib[(int64_t)qs * a.n_out + n] = ok ? (int32_t)row : -1;
                }
            }
        }
    };
    if constexpr (BPW > 0) {
        static_for<0, BPW>([&](auto IT) {
            constexpr int it = decltype(IT)::value;
            step(std::integral_constant<int, it % (PD + 1)>{}, it);
        });
    } else {
        for (int it0 = 0; it0 < bpw; it0 += PD + 1)
            static_for<0, PD + 1>([&](auto J) { step(J, it0 + (int)decltype(J)::value); });
    }
    if constexpr (HIST) {
        // every wave ran the same number of ring turns: all of them reach this barrier
        __syncthreads();
        const int64_t row = (int64_t)b * a.n_q + t0;
        const int64_t slice = row * gridDim.x + blockIdx.x;
        // coarse sums of 64 bins first; only the groups that hold keys (a few of the 32) have
        // their 64 fine bins written -- the reader ignores the fine bins of an empty group
        __shared__ uint32_t lcoarse[32];
        if (stage) {
            // the workgroup's own blocks: positions [x * span, (x + 1) * span) of the row
            const int64_t span = (int64_t)bpw * WAVES * 32, o_base = (int64_t)blockIdx.x * span;
            slice_compact<WAVES>(a, lhist, lcoarse, lsc, slice, o_base, max(o_base, mid_lo),
                                 min(o_base + span, mid_hi));
        } else {
            if (threadIdx.x < 32) {
                const uint4 *h4 = reinterpret_cast<const uint4 *>(lhist + 64 * threadIdx.x);
                uint32_t c = 0;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const uint4 v = h4[i];
                    c += v.x + v.y + v.z + v.w;
                }
                lcoarse[threadIdx.x] = c;
            }
            __syncthreads();
        }
        // the global stores come last: a barrier after a store waits until it completes
        if (threadIdx.x < 32) a.hist_coarse[slice * 32 + threadIdx.x] = lcoarse[threadIdx.x];
        uint4 *hf = reinterpret_cast<uint4 *>(a.hist_fine + slice * HBINS);
        for (int i = threadIdx.x; i < HBINS / 4; i += WAVES * kWave)
            if (lcoarse[i / 16]) hf[i] = reinterpret_cast<const uint4 *>(lhist)[i];
    }
}

// ------------------------------------------------------------------------------------------
// tile kernel (prefill)
// ------------------------------------------------------------------------------------------

// Q8: fp8 queries (a.q8, a.q_scale) against e4m3 keys on v_mfma_f32_32x32x64_f8f6f4; the keys
// are staged in LDS as the codes themselves (a 144-byte padded row at d = 128) and each query
// scale is folded into its head weight.
template <bool FP8, int D, int H, int MT, int WAVES, int KB, bool Q8 = false>
__global__ __launch_bounds__(WAVES *kWave) void score_tile_kernel(ScoreArgs a)
{
    static_assert(!Q8 || FP8, "fp8 queries meet fp8 keys");
    using G = Geo<H, MT, false>;
    constexpr int KS = Q8 ? D / 64 : D / 16;          // MFMA K-steps per key block
    constexpr int QPB = WAVES * G::NQW;
    constexpr int ROWB = Q8 ? D + 16 : D * 2 + 16;    // LDS bytes per staged key (+ pad)
    constexpr int ESZ = FP8 ? 1 : 2;
    constexpr int CPR = D * ESZ / 16;                 // 16-byte source chunks per key row
    constexpr int CHUNKS = KB * CPR;
    constexpr int NT = WAVES * kWave;
    constexpr int CPT = (CHUNKS + NT - 1) / NT;       // chunks per thread per tile
    static_assert(KB % 32 == 0, "tile of whole MFMA blocks");
    static_assert(CHUNKS % NT == 0, "whole chunks per thread");

    __shared__ __attribute__((aligned(16))) uint8_t lds_k[2][KB * ROWB];
    __shared__ float lds_s[2][KB];

    const int b = blockIdx.y;
    const int64_t tq0 = (int64_t)blockIdx.x * QPB;
    const int l = lane_id(), wv_id = wave_id(), g = l >> 5, n = l & 31;
    const int64_t t0 = tq0 + (int64_t)wv_id * G::NQW;
    const int nq_avail = (int)max((int64_t)0, min((int64_t)G::NQW, (int64_t)a.n_q - t0));

    using QF = std::conditional_t<Q8, i32x8_t, bf16x8_t>;
    QF qf[MT][KS];
    float wv[G::VPL];
    if (nq_avail > 0) {
        if constexpr (Q8) {
            load_q8<D, H, MT>(qf, a.q8 + ((int64_t)b * a.n_q + t0) * H * D, nq_avail);
            load_w<H, MT, false>(wv, a.w + ((int64_t)b * a.n_q + t0) * H, nq_avail);
            float qs[G::VPL];
            load_w<H, MT, false>(qs, a.q_scale + ((int64_t)b * a.n_q + t0) * H, nq_avail);
#pragma unroll
            for (int v = 0; v < G::VPL; ++v) wv[v] *= qs[v]; // ReLU(s x) = s ReLU(x), s > 0
        } else {
            load_q<D, H, MT, false>(qf, a.q + ((int64_t)b * a.n_q + t0) * H * D, nq_avail);
            load_w<H, MT, false>(wv, a.w + ((int64_t)b * a.n_q + t0) * H, nq_avail);
        }
    } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) qf[mt][kk] = QF{};
#pragma unroll
        for (int v = 0; v < G::VPL; ++v) wv[v] = 0.0f;
    }
    int64_t lo[G::NQL], hi[G::NQL];
#pragma unroll
    for (int u = 0; u < G::NQL; ++u) {
        const int qs = G::SPLIT ? 0 : g * G::NQL + u;
        if (qs < nq_avail) {
            row_range(a, b, t0 + qs, lo[u], hi[u]);
        } else {
            lo[u] = 0;
            hi[u] = 0;
        }
    }
    // Hull of the block's ranges (ranges are monotone in t, but compute it plainly).
    const int nq_blk = (int)min((int64_t)QPB, (int64_t)a.n_q - tq0);
    int64_t lo_blk = INT64_MAX, hi_blk = 0;
    for (int qs = 0; qs < nq_blk; ++qs) {
        int64_t x, y;
        row_range(a, b, tq0 + qs, x, y);
        if (y > x) {
            lo_blk = min(lo_blk, x);
            hi_blk = max(hi_blk, y);
        }
    }
    int64_t kt_begin = 0, kt_end = 0;
    if (hi_blk > lo_blk) {
        kt_begin = lo_blk / KB;
        kt_end = (hi_blk + KB - 1) / KB;
    }

    const uint8_t *keys_b = reinterpret_cast<const uint8_t *>(a.keys) + (int64_t)b * a.n_keys * D * ESZ;
    const float *scale_b = FP8 ? a.kscale + (int64_t)b * a.n_keys : nullptr;

    uint4 stage[CPT];
    float stage_s = 0.0f;
    // Unconditional loads (rows past the last key re-read the last key; their scores are never
    // stored): a conditional load, or a zero written to a register a load may still be filling,
    // makes the compiler wait for every load and store in flight, including the epilogue's.
    auto fetch = [&](int64_t kt) {
        static_for<0, CPT>([&](auto I) {
            constexpr int i = decltype(I)::value;
            const int c = (int)threadIdx.x + i * NT;
            const int key = c / CPR, col = c % CPR;
            const int64_t row = min(kt * KB + key, a.n_keys - 1);
            stage[i] = reinterpret_cast<const uint4 *>(keys_b + row * D * ESZ)[col];
        });
        if (FP8) {
            const int64_t row = min(kt * KB + (int)(threadIdx.x % KB), a.n_keys - 1);
            stage_s = scale_b[row];
        }
    };
    auto commit = [&](int buf) {
        static_for<0, CPT>([&](auto I) {
            constexpr int i = decltype(I)::value;
            const int c = threadIdx.x + i * NT;
            const int key = c / CPR, col = c % CPR;
            uint8_t *dst = &lds_k[buf][key * ROWB];
            if constexpr (Q8) { // the codes as they are
                *reinterpret_cast<u32x4_t *>(dst + col * 16) = bitcast<u32x4_t>(stage[i]);
            } else if (FP8) {
                const uint2 lo2 = e4m3x4_to_bf16x4(stage[i].x), hi2 = e4m3x4_to_bf16x4(stage[i].y);
                const uint2 lo3 = e4m3x4_to_bf16x4(stage[i].z), hi3 = e4m3x4_to_bf16x4(stage[i].w);
                reinterpret_cast<uint4 *>(dst + col * 32)[0] = make_uint4(lo2.x, lo2.y, hi2.x, hi2.y);
                reinterpret_cast<uint4 *>(dst + col * 32)[1] = make_uint4(lo3.x, lo3.y, hi3.x, hi3.y);
            } else {
                *reinterpret_cast<u32x4_t *>(dst + col * 16) = bitcast<u32x4_t>(stage[i]);
            }
        });
        if (FP8 && threadIdx.x < KB) lds_s[buf][threadIdx.x] = stage_s;
    };

    if (kt_begin < kt_end) {
        fetch(kt_begin);
        commit(0);
    }
    // q and w must be in registers before the loop: without this wait the compiler places the
    // wait for them inside the loop body, where in every iteration it also waits for the next
    // tile's prefetch and so serialises the key loads with the MFMAs.
    __builtin_amdgcn_s_waitcnt(0x0F70); // vmcnt(0)
    __syncthreads();
    for (int64_t kt = kt_begin; kt < kt_end; ++kt) {
        const int buf = (int)((kt - kt_begin) & 1);
        if (kt + 1 < kt_end) fetch(kt + 1);
        if (nq_avail > 0) {
            // Software-pipelined over the tile's 32-key blocks: the MFMAs of block nt+1 are
            // issued before the epilogue of block nt, so the epilogue's VALU work overlaps them.
            f32x16_t acc[2][MT];
            auto mma = [&](int nt, f32x16_t (&ac)[MT]) {
                // lane half g: the key bytes of d in [g*D/2, (g+1)*D/2)
                const uint8_t *src = &lds_k[buf][(nt * 32 + n) * ROWB + (Q8 ? D / 2 : D) * g];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) ac[mt] = f32x16_t{};
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    if constexpr (Q8) {
                        const uint4 x = *reinterpret_cast<const uint4 *>(src + 32 * kk);
                        const uint4 y = *reinterpret_cast<const uint4 *>(src + 32 * kk + 16);
                        const i32x8_t bk = i32x8_t{(int)x.x, (int)x.y, (int)x.z, (int)x.w,
                                                   (int)y.x, (int)y.y, (int)y.z, (int)y.w};
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) ac[mt] = mfma_32x32x64_f8(qf[mt][kk], bk, ac[mt]);
                    } else {
                        const bf16x8_t bk = bitcast<bf16x8_t>(*reinterpret_cast<const uint4 *>(src + 16 * kk));
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) ac[mt] = mfma_32x32x16(qf[mt][kk], bk, ac[mt]);
                    }
                }
            };
            auto epi = [&](int nt, const f32x16_t (&ac)[MT]) {
                const int key = nt * 32 + n;
                float part[G::NQL];
                epilogue<H, MT, false>(ac, [&](int v) { return wv[v]; }, part);
                const int64_t s = kt * KB + key;
                if (FP8) {
                    const float sc = lds_s[buf][key];
#pragma unroll
                    for (int u = 0; u < G::NQL; ++u) part[u] *= sc;
                }
                if (!(G::SPLIT && g != 0)) {
#pragma unroll
                    for (int u = 0; u < G::NQL; ++u) {
                        const int qs = G::SPLIT ? 0 : g * G::NQL + u;
                        if (qs >= nq_avail || s >= a.n_out) continue;
                        const bool ok = s >= lo[u] && s < hi[u];
                        a.out[((int64_t)b * a.n_q + t0 + qs) * a.n_out + s] = ok ? part[u] : -INFINITY;
                    }
                }
            };
            // The next tile is written to the other buffer (read by nobody in this tile) before
            // the epilogue of block CN: its wait for the prefetched keys then covers only the
            // stores of the first CN epilogues, each issued a block of MFMAs earlier, and the
            // keys have had CN + 1 blocks of MFMAs to arrive (measured best: CN = 2).
            constexpr int CN = KB / 32 >= 3 ? 2 : 0;
            mma(0, acc[0]);
            static_for<0, KB / 32>([&](auto NTI) {
                constexpr int nt = decltype(NTI)::value;
                if constexpr (nt + 1 < KB / 32) mma(nt + 1, acc[(nt + 1) & 1]);
                if constexpr (nt == CN)
                    if (kt + 1 < kt_end) commit(buf ^ 1);
                epi(nt, acc[nt & 1]);
            });
        } else if (kt + 1 < kt_end) {
            commit(buf ^ 1);
        }
        __syncthreads();
    }

    // -inf outside the computed tiles, for every query row of the block.
    int64_t c_lo = kt_begin * KB, c_hi = min(kt_end * KB, a.n_out);
    if (kt_begin >= kt_end) c_lo = c_hi = 0;
    for (int qs = 0; qs < nq_blk; ++qs) {
        float *orow = a.out + ((int64_t)b * a.n_q + tq0 + qs) * a.n_out;
        for (int64_t s = threadIdx.x; s < c_lo; s += NT) orow[s] = -INFINITY;
        for (int64_t s = c_hi + threadIdx.x; s < a.n_out; s += NT) orow[s] = -INFINITY;
    }
}

constexpr int STREAM_WAVES = 4, STREAM_BPW_LONG = 32;

// The long flat launch: one round of workgroups (about 512, two per CU), each wave streaming its
// share of the row's 32-key blocks.
bool long_launch(const ScoreArgs &a, int64_t rows)
{
    const int64_t n_blocks = (a.n_out + 31) / 32;
    return n_blocks * rows * a.batch >= (int64_t)512 * STREAM_WAVES * STREAM_BPW_LONG &&
           a.n_keys >= 32 && a.n_out == a.n_keys;
}

int64_t long_groups(const ScoreArgs &a, int64_t rows)
{
    const int64_t n_blocks = (a.n_out + 31) / 32;
    const int64_t units = rows * a.batch;
    const int64_t gx = std::max<int64_t>(1, (512 + units - 1) / units);
    return std::min<int64_t>(gx, (n_blocks + STREAM_WAVES - 1) / STREAM_WAVES);
}

template <bool FP8, int D, int H>
hipError_t launch_flat(const ScoreArgs &a, hipStream_t st)
{
    constexpr int MT = H == 64 ? 2 : 1;
    using G = Geo<H, MT, false>;
    if (a.q8) { // fp8 queries: the tile kernel for every shape (keys e4m3)
        if constexpr (FP8) {
            if (a.hist_fine || a.btab) return hipErrorInvalidValue;
            // 256-key tiles: 2 x 36 KB of LDS at d = 128
            constexpr int WAVES = 8, KB = 256;
            constexpr int QPB = WAVES * G::NQW;
            dim3 grid((unsigned)((a.n_q + QPB - 1) / QPB), (unsigned)a.batch);
            hipLaunchKernelGGL((score_tile_kernel<true, D, H, MT, WAVES, KB, true>), grid,
                               dim3(WAVES * kWave), 0, st, a);
            return hipGetLastError();
        } else {
            return hipErrorInvalidValue;
        }
    }
    if (a.n_q <= 2 * G::NQW) {
        // Long launches (at least 32 blocks = 1024 keys per wave with 512 workgroups): long-lived
        // waves amortise the per-wave load of q and w, and up to 3 blocks in flight per wave
        // (12 KB of keys at 4 KB per block) keep enough bytes outstanding per CU at two waves
        // per SIMD.  Short launches (page keys of Hierarchical Indexing, small batches) need
        // many workgroups more than long waves: two blocks per wave there.
        constexpr int WAVES = STREAM_WAVES, BPW_SHORT = 2;
        constexpr int PD = KeyBlock<FP8, D>::BB <= 4096 ? 3 : 1;
        const int64_t n_blocks = (a.n_out + 31) / 32;
        const int64_t rows = (a.n_q + G::NQW - 1) / G::NQW;
        if (long_launch(a, rows)) {
            // one round of workgroups, two per CU (as many as are resident at once), each wave
            // streaming its share of blocks: no tail round, and the per-wave load of q and w
            // amortised over as many blocks as possible
            dim3 grid((unsigned)long_groups(a, rows), (unsigned)rows, (unsigned)a.batch);
            if constexpr (G::NQW == 1 && G::SPLIT) {
                if (a.hist_fine) {
                    if (a.btab)
                        hipLaunchKernelGGL(
                            (score_stream_kernel<FP8, D, H, MT, false, false, WAVES, 0, PD, true, true>),
                            grid, dim3(WAVES * kWave), 0, st, a);
                    else
                        hipLaunchKernelGGL(
                            (score_stream_kernel<FP8, D, H, MT, false, false, WAVES, 0, PD, true>),
                            grid, dim3(WAVES * kWave), 0, st, a);
                    return hipGetLastError();
                }
            }
            if (a.hist_fine) return hipErrorInvalidValue;
            if (a.btab)
                hipLaunchKernelGGL(
                    (score_stream_kernel<FP8, D, H, MT, false, false, WAVES, 0, PD, false, true>),
                    grid, dim3(WAVES * kWave), 0, st, a);
            else
                hipLaunchKernelGGL((score_stream_kernel<FP8, D, H, MT, false, false, WAVES, 0, PD>),
                                   grid, dim3(WAVES * kWave), 0, st, a);
        } else {
            if (a.hist_fine) return hipErrorInvalidValue;
            dim3 grid((unsigned)((n_blocks + WAVES * BPW_SHORT - 1) / (WAVES * BPW_SHORT)),
                      (unsigned)rows, (unsigned)a.batch);
            if (a.btab)
                hipLaunchKernelGGL(
                    (score_stream_kernel<FP8, D, H, MT, false, false, WAVES, BPW_SHORT, 1, false, true>),
                    grid, dim3(WAVES * kWave), 0, st, a);
            else
                hipLaunchKernelGGL(
                    (score_stream_kernel<FP8, D, H, MT, false, false, WAVES, BPW_SHORT, 1>), grid,
                    dim3(WAVES * kWave), 0, st, a);
        }
    } else {
        if (a.hist_fine || a.btab) return hipErrorInvalidValue;
        // 256-key tiles (139 KB of LDS, one workgroup per CU) where registers already limit
        // the CU to one workgroup (H = 64, d = 128: 252 VGPRs); 128-key tiles elsewhere, so two
        // workgroups can share a CU
        constexpr int WAVES = 8, KB = (H == 64 && D == 128) ? 256 : 128;
        constexpr int QPB = WAVES * G::NQW;
        dim3 grid((unsigned)((a.n_q + QPB - 1) / QPB), (unsigned)a.batch);
        hipLaunchKernelGGL((score_tile_kernel<FP8, D, H, MT, WAVES, KB>), grid,
                           dim3(WAVES * kWave), 0, st, a);
    }
    return hipGetLastError();
}

template <bool FP8, int D, int H>
hipError_t launch_fine(const ScoreArgs &a, hipStream_t st)
{
    constexpr int MT = H > 32 ? 2 : 1;
    // two blocks per wave: both in flight from the start (Hierarchical Indexing's candidate rows
    // are short, so the launch is one round of latency, not a chain of them)
    constexpr int WAVES = 4, BPW = 2;
    const int64_t n_blocks = (a.n_out + 31) / 32;
    dim3 grid((unsigned)((n_blocks + WAVES * BPW - 1) / (WAVES * BPW)), (unsigned)a.n_q,
              (unsigned)a.batch);
    if (a.btab) {
        hipLaunchKernelGGL((score_stream_kernel<FP8, D, H, MT, true, true, WAVES, BPW, 1, false, true>),
                           grid, dim3(WAVES * kWave), 0, st, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((score_stream_kernel<FP8, D, H, MT, true, true, WAVES, BPW>), grid,
                       dim3(WAVES * kWave), 0, st, a);
    return hipGetLastError();
}

template <bool FP8, int D>
hipError_t dispatch_heads(const ScoreArgs &a, hipStream_t st, bool fine)
{
    switch (a.heads) {
    case 4: return fine ? launch_fine<FP8, D, 4>(a, st) : launch_flat<FP8, D, 4>(a, st);
    case 8: return fine ? launch_fine<FP8, D, 8>(a, st) : launch_flat<FP8, D, 8>(a, st);
    case 16: return fine ? launch_fine<FP8, D, 16>(a, st) : launch_flat<FP8, D, 16>(a, st);
    case 32: return fine ? launch_fine<FP8, D, 32>(a, st) : launch_flat<FP8, D, 32>(a, st);
    case 64: return fine ? launch_fine<FP8, D, 64>(a, st) : launch_flat<FP8, D, 64>(a, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t dispatch(const ScoreArgs &a, hipStream_t st, bool fine)
{
    if (a.dim == 128)
        return a.fp8 ? dispatch_heads<true, 128>(a, st, fine) : dispatch_heads<false, 128>(a, st, fine);
    if (a.dim == 64)
        return a.fp8 ? dispatch_heads<true, 64>(a, st, fine) : dispatch_heads<false, 64>(a, st, fine);
    return hipErrorInvalidValue;
}

} // namespace

bool scores_paged_ok(const ScoreArgs &a)
{
    if (a.q8 || a.lbs < 5 || !scores_supported(a.heads, a.dim)) return false;
    // the flat stream path of launch_flat (queries per wave: 32 * MT / H)
    const int nqw = 32 * (a.heads == 64 ? 2 : 1) / a.heads;
    if (a.n_q > 2 * nqw) return false;
    const int64_t rows = (a.n_q + nqw - 1) / nqw;
    int64_t span = 2 * STREAM_WAVES * 32; // a short launch: two blocks per wave
    if (long_launch(a, rows)) {
        const int64_t n_blocks = (a.n_out + 31) / 32, gx = long_groups(a, rows);
        span = (n_blocks + gx * STREAM_WAVES - 1) / (gx * STREAM_WAVES) * STREAM_WAVES * 32;
    }
    return ((span - 1) >> a.lbs) + 2 <= kPagedTab;
}

bool scores_supported(int heads, int dim)
{
    return (dim == 64 || dim == 128) &&
           (heads == 4 || heads == 8 || heads == 16 || heads == 32 || heads == 64);
}

// ------------------------------------------------------------------------------------------
// fp8 query quantisation
// ------------------------------------------------------------------------------------------

namespace {

// binary32 -> e4m3fn code, round to nearest with ties to even, saturating at +-448 (the format:
// bias 7, 3 mantissa bits, subnormals m * 2^-9, no infinities).  Finite inputs.
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float y)
{
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a >= 0x43e00000u) return sign | 0x7eu;             // |y| >= 448
    if (a < 0x3c800000u) {                                   // |y| < 2^-6: subnormal codes
        // m = round_even(|y| * 2^9) in 0..8; 8 is the smallest normal's code (0x08)
        const float m = __builtin_rintf(__uint_as_float(a) * 512.0f); // exact scaling
        return sign | (uint32_t)m;
    }
    // normal: keep 3 mantissa bits of the binary32 with round to nearest even (a carry moves
    // into the exponent), then rebias 127 -> 7
    const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
    const uint32_t code = r - ((127u - 7u) << 3);
    return sign | (code > 0x7eu ? 0x7eu : code);
}

// One wave per row: amax, the binary32 scale, then every element's code.
__global__ __launch_bounds__(256) void quantize_rows_kernel(const uint16_t *x, int64_t rows,
                                                            int d, uint8_t *codes, float *scale)
{
    const int64_t r = (int64_t)blockIdx.x * 4 + wave_id();
    if (r >= rows) return;
    const int l = lane_id();
    const int per = d / kWave; // 1 or 2 elements per lane
    float v[2] = {0.0f, 0.0f};
    if (per == 2) {
        const uint32_t p = *reinterpret_cast<const uint32_t *>(x + r * d + 2 * l);
        v[0] = __uint_as_float(p << 16);
        v[1] = __uint_as_float(p & 0xffff0000u);
    } else {
        v[0] = __uint_as_float((uint32_t)x[r * d + l] << 16);
    }
    const float amax = wave_max(fmaxf(fabsf(v[0]), fabsf(v[1])));
    const float s = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    if (l == 0) scale[r] = s;
    if (per == 2) {
        const uint32_t c0 = f32_to_e4m3_sat(__fdiv_rn(v[0], s));
        const uint32_t c1 = f32_to_e4m3_sat(__fdiv_rn(v[1], s));
        *reinterpret_cast<uint16_t *>(codes + r * d + 2 * l) = (uint16_t)(c0 | (c1 << 8));
    } else {
        codes[r * d + l] = (uint8_t)f32_to_e4m3_sat(__fdiv_rn(v[0], s));
    }
}

} // namespace

hipError_t launch_quantize_rows(const uint16_t *x, int64_t rows, int d, uint8_t *codes,
                                float *scale, hipStream_t stream)
{
    if (rows == 0) return hipSuccess;
    if (d != 64 && d != 128) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                       stream, x, rows, d, codes, scale);
    return hipGetLastError();
}

hipError_t launch_scores(const ScoreArgs &a, hipStream_t stream) { return dispatch(a, stream, false); }

int64_t score_hist_span(const ScoreArgs &a, int groups)
{
    const int64_t n_blocks = (a.n_out + 31) / 32, per = (int64_t)groups * STREAM_WAVES;
    return (n_blocks + per - 1) / per * STREAM_WAVES * 32;
}

int score_hist_groups(const ScoreArgs &a)
{
    // the histogram launch: one query per wave row group (H = 32 or 64, split over the lane
    // halves), few enough queries for the stream kernel, and the long launch
    if (a.mask != MASK_CAUSAL || (a.heads != 32 && a.heads != 64)) return 0;
    if (a.n_q > 2) return 0;
    const int64_t rows = a.n_q;
    if (!long_launch(a, rows)) return 0;
    return (int)long_groups(a, rows);
}

hipError_t launch_fine_scores(const ScoreArgs &a, hipStream_t stream) { return dispatch(a, stream, true); }

} // namespace lsa
