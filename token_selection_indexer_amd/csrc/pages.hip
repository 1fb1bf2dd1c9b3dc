// pages.hip -- page keys for Hierarchical Indexing.
//
// The model card's HI bullet recalls candidate blocks by coarse scores without defining a
// block's coarse key.  This library defines the key of page p (P tokens, P a power of two) as the
// mean of its dequantised indexer keys with a fixed binary32 rounding sequence:
//   v[j]  = fp32(scale[s] * e4m3(kq[s][i]))  (bf16 keys: the value), s = p*P + j; +0 past the
//           sequence's last key (a page wholly past it is the zero key)
//   sum   = pairwise tree sum of v[0..P): halves summed separately, then added, recursively
//   pk    = bf16_rne(sum / n_p), n_p = tokens of the page that exist
// Every multiply, add and divide rounds on its own: contraction into FMA is switched off for
// this file (pragma below, and -ffp-contract=off on its compile line), because HIP's
// __fmul_rn / __fadd_rn are plain operators that the compiler may otherwise fuse.
//
// Layout (pages of at least G tokens, G = 64 / LPR): a wave per page at a time, looping over
// pages with the next page's loads in flight.  A key row is LPR
// 16-byte pieces; lane (g, c) = (lane / LPR, lane % LPR) loads piece c of the TPL = P / G
// consecutive tokens g*TPL .. g*TPL + TPL - 1, so each load instruction reads whole rows and every
// lane's register data is the subtree of TPL adjacent tokens.  Those subtrees are summed in
// registers (a binary counter, fully unrolled), then combined across the G lane groups by xor
// shuffles: group g meets g^1, then pairs meet pairs, ... -- exactly the levels of the pairwise
// tree above the subtrees (binary32 addition is commutative, so which operand is on the left
// does not change the bits).  Smaller pages: D/2 threads per page, each owning two adjacent key
// elements and the whole tree of its page.
#include "device.hpp"
#include "internal.hpp"

#pragma clang fp contract(off)

namespace lsa {
namespace {

template <bool FP8, int P>
__global__ __launch_bounds__(256) void page_summary_kernel(const void *keys, const float *kscale,
                                                           int64_t kv_len, const int32_t *seq_len,
                                                           int D, int64_t page_lo,
                                                           int64_t page_hi, int64_t n_pages,
                                                           uint16_t *pk)
{
    const int tpp = D / 2; // threads per page
    const int b = blockIdx.y;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t p = page_lo + gid / tpp;
    const int pair = (int)(gid % tpp);
    if (p >= page_hi) return;
    const int64_t s0 = p * P;
    const int64_t L = seq_keys(seq_len, b, kv_len); // this sequence's keys
    const int64_t n_p = min((int64_t)P, L - s0);
    if (n_p <= 0) { // a page past the sequence's end: zero key
        *reinterpret_cast<uint32_t *>(pk + ((int64_t)b * n_pages + p) * D + 2 * pair) = 0u;
        return;
    }

    // binary counter over the tokens: before token j the stack holds popcount(j) completed
    // subtrees; token j closes ctz(~j) of them (left + right), all positions known at compile time
    float stk0[10], stk1[10];
    static_for<0, P>([&](auto J) {
        constexpr int j = decltype(J)::value;
        constexpr int depth = __builtin_popcount(j);
        constexpr int merges = __builtin_ctz(~j);
        const int64_t s = s0 + j;
        float x0 = 0.0f, x1 = 0.0f;
        if (j < n_p) {
            if (FP8) {
                const uint8_t *row = reinterpret_cast<const uint8_t *>(keys) + ((int64_t)b * kv_len + s) * D;
                const uint32_t c = *reinterpret_cast<const uint16_t *>(row + 2 * pair);
                const uint2 bf = e4m3x4_to_bf16x4(c);
                const float sc = kscale[(int64_t)b * kv_len + s];
                x0 = __fmul_rn(sc, __uint_as_float(bf.x << 16));
                x1 = __fmul_rn(sc, __uint_as_float(bf.x & 0xffff0000u));
            } else {
                const uint16_t *row = reinterpret_cast<const uint16_t *>(keys) + ((int64_t)b * kv_len + s) * D;
                const uint32_t c = *reinterpret_cast<const uint32_t *>(row + 2 * pair);
                x0 = __uint_as_float(c << 16);
                x1 = __uint_as_float(c & 0xffff0000u);
            }
        }
        static_for<0, merges>([&](auto M) {
            constexpr int m = decltype(M)::value;
            x0 = __fadd_rn(stk0[depth - 1 - m], x0);
            x1 = __fadd_rn(stk1[depth - 1 - m], x1);
        });
        stk0[depth - merges] = x0;
        stk1[depth - merges] = x1;
    });
    const float nf = (float)n_p;
    const float m0 = __fdiv_rn(stk0[0], nf), m1 = __fdiv_rn(stk1[0], nf);
    const uint32_t out = f32_to_bf16_bits(m0) | (f32_to_bf16_bits(m1) << 16);
    *reinterpret_cast<uint32_t *>(pk + ((int64_t)b * n_pages + p) * D + 2 * pair) = out;
}

// Lanes per key row (16-byte pieces) and lane groups per wave.
template <bool FP8, int D>
struct PageGeo {
    static constexpr int EB = FP8 ? 1 : 2;      // bytes per element
    static constexpr int EPL = 16 / EB;         // elements per 16-byte piece
    static constexpr int LPR = D * EB / 16;     // lanes per row
    static constexpr int G = kWave / LPR;       // lane groups
};

// PAGED: the keys (and scales) are pools under pt's block table, a page inside one table block
// (P <= block size); a page whose table entry lies outside the pool gets the zero key.
template <bool FP8, int D, int P, bool PAGED = false>
__global__ __launch_bounds__(256) void page_summary_wave_kernel(const void *keys, const float *kscale,
                                                                int64_t kv_len, const int32_t *seq_len,
                                                                int64_t page_lo,
                                                                int64_t page_hi, int64_t n_pages,
                                                                uint16_t *pk, PagedTab pt)
{
    using Geo = PageGeo<FP8, D>;
    constexpr int EPL = Geo::EPL, LPR = Geo::LPR, G = Geo::G;
    static_assert(P >= G && P % G == 0, "page must cover every lane group");
    constexpr int TPL = P / G;                  // tokens per lane
    constexpr int LEV = __builtin_ctz(TPL) + 1; // binary-counter stack depth
    constexpr int ROW = D * Geo::EB;            // bytes per key row
    const int b = blockIdx.y;
    const int lane = lane_id(), g = lane / LPR, c = lane % LPR;
    const uint8_t *kb = reinterpret_cast<const uint8_t *>(keys) + (PAGED ? 0 : (int64_t)b * kv_len * ROW) + 16 * c;
    const float *sb = FP8 ? kscale + (PAGED ? 0 : (int64_t)b * kv_len) : nullptr;
    const int64_t L = seq_keys(seq_len, b, kv_len); // this sequence's keys (rows past: +0)

    // a lane's raw data for one page: TPL pieces (+ TPL scales); zero past the sequence's end
    uint4 raw[TPL];
    float scl[TPL];
    auto load = [&](int64_t p) {
        const int64_t t0 = p * P + g * TPL;
        int64_t shift = 0; // PAGED: pool row - token position, for the whole page
        bool here = true;  // PAGED: the page's table entry lies inside the pool
        if constexpr (PAGED) {
            const int64_t r0 = p * P;
            const int32_t e = pt.btab[(int64_t)b * pt.bps + (r0 >> pt.lbs)];
            here = e >= 0 && e < pt.n_blocks;
            shift = here ? (((int64_t)e << pt.lbs) | (r0 & ((int64_t(1) << pt.lbs) - 1))) - r0 : 0;
        }
        static_for<0, TPL>([&](auto J) {
            constexpr int j = decltype(J)::value;
            const bool ok = t0 + j < L && here;
            raw[j] = ok ? ld16_nt(kb + (t0 + j + shift) * ROW) : make_uint4(0u, 0u, 0u, 0u); // read once
            if constexpr (FP8) scl[j] = ok ? sb[t0 + j + shift] : 0.0f;
        });
    };

    // grid-stride over pages; the next page's loads are issued before this page's arithmetic
    const int64_t stride = (int64_t)gridDim.x * (blockDim.x / kWave);
    int64_t p = page_lo + (int64_t)blockIdx.x * (blockDim.x / kWave) + wave_id();
    if (p >= page_hi) return; // whole wave
    load(p);
    for (; p < page_hi; p += stride) {
        uint4 cur[TPL];
        float cs[TPL];
        static_for<0, TPL>([&](auto J) {
            constexpr int j = decltype(J)::value;
            cur[j] = raw[j];
            if constexpr (FP8) cs[j] = scl[j];
        });
        if (p + stride < page_hi) load(p + stride);

        float stk[LEV][EPL];
        static_for<0, TPL>([&](auto J) {
            constexpr int j = decltype(J)::value;
            constexpr int depth = __builtin_popcount(j);
            constexpr int merges = __builtin_ctz(~j);
            const uint32_t wd[4] = {cur[j].x, cur[j].y, cur[j].z, cur[j].w};
            float x[EPL];
            if constexpr (FP8) {
                // a zero code times a zero scale is +0: slots past kv_len add +0, as defined
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint2 bf = e4m3x4_to_bf16x4(wd[u]);
                    x[4 * u + 0] = __fmul_rn(cs[j], __uint_as_float(bf.x << 16));
                    x[4 * u + 1] = __fmul_rn(cs[j], __uint_as_float(bf.x & 0xffff0000u));
                    x[4 * u + 2] = __fmul_rn(cs[j], __uint_as_float(bf.y << 16));
                    x[4 * u + 3] = __fmul_rn(cs[j], __uint_as_float(bf.y & 0xffff0000u));
                }
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    x[2 * u + 0] = __uint_as_float(wd[u] << 16);
                    x[2 * u + 1] = __uint_as_float(wd[u] & 0xffff0000u);
                }
            }
            static_for<0, merges>([&](auto M) {
                constexpr int m = decltype(M)::value;
#pragma unroll
                for (int e = 0; e < EPL; ++e) x[e] = __fadd_rn(stk[depth - 1 - m][e], x[e]);
            });
#pragma unroll
            for (int e = 0; e < EPL; ++e) stk[depth - merges][e] = x[e];
        });
        // levels above the per-lane subtrees
#pragma unroll
        for (int m = LPR; m < kWave; m <<= 1)
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                stk[0][e] = __fadd_rn(stk[0][e], __shfl_xor(stk[0][e], m, kWave));
        if (g == 0) {
            const int64_t n_p = min((int64_t)P, L - p * P); // <= 0: past the end, a zero key
            // a full page divides by P = 2^k: multiplying by the exact 2^-k rounds identically
            const bool full = n_p == P;
            const float nf = (float)n_p;
            uint32_t o[EPL / 2];
#pragma unroll
            for (int e = 0; e < EPL / 2; ++e) {
                const float m0 = full ? __fmul_rn(stk[0][2 * e], 1.0f / P) : __fdiv_rn(stk[0][2 * e], nf);
                const float m1 = full ? __fmul_rn(stk[0][2 * e + 1], 1.0f / P) : __fdiv_rn(stk[0][2 * e + 1], nf);
                o[e] = n_p > 0 ? f32_to_bf16_bits(m0) | (f32_to_bf16_bits(m1) << 16) : 0u;
            }
            uint16_t *dst = pk + ((int64_t)b * n_pages + p) * D + c * EPL;
#pragma unroll
            for (int e = 0; e < EPL / 8; ++e)
                *reinterpret_cast<uint4 *>(dst + 8 * e) =
                    make_uint4(o[4 * e], o[4 * e + 1], o[4 * e + 2], o[4 * e + 3]);
        }
    }
}

template <bool FP8, int D, int P>
hipError_t launch_wave(const void *keys, const float *kscale, int batch, int64_t kv_len,
                       const int32_t *seq_len, int64_t page_lo, int64_t page_hi, uint16_t *pk,
                       hipStream_t st, const PagedTab &pt)
{
    const int64_t n_pages = (kv_len + P - 1) / P;
    // about 2048 workgroups in all (8 per CU), each wave looping over its share of the pages
    const int64_t want = batch >= 2048 ? 1 : 2048 / batch;
    const int64_t need = (page_hi - page_lo + 3) / 4;
    const int64_t wg = need < want ? need : want;
    const dim3 grid((unsigned)wg, (unsigned)batch);
    if (pt.btab) {
        if constexpr (P >= 32)
            hipLaunchKernelGGL((page_summary_wave_kernel<FP8, D, P, true>), grid, dim3(256), 0, st,
                               keys, kscale, kv_len, seq_len, page_lo, page_hi, n_pages, pk, pt);
        else
            return hipErrorInvalidValue;
    } else {
        hipLaunchKernelGGL((page_summary_wave_kernel<FP8, D, P>), grid, dim3(256), 0, st, keys,
                           kscale, kv_len, seq_len, page_lo, page_hi, n_pages, pk, pt);
    }
    return hipGetLastError();
}

template <bool FP8, int D>
hipError_t launch_wave_p(const void *keys, const float *kscale, int batch, int64_t kv_len,
                         const int32_t *seq_len, int P, int64_t page_lo, int64_t page_hi,
                         uint16_t *pk, hipStream_t st, bool &done, const PagedTab &pt)
{
    done = true;
    switch (P) {
#define LSA_PW(PP)                                                                                  \
    case PP:                                                                                        \
        if constexpr (PP >= PageGeo<FP8, D>::G)                                                     \
            return launch_wave<FP8, D, PP>(keys, kscale, batch, kv_len, seq_len, page_lo, page_hi, pk, st, pt); \
        break;
        LSA_PW(1) LSA_PW(2) LSA_PW(4) LSA_PW(8) LSA_PW(16) LSA_PW(32) LSA_PW(64) LSA_PW(128) LSA_PW(256)
#undef LSA_PW
    default: break;
    }
    done = false;
    return hipSuccess;
}

template <bool FP8>
hipError_t launch_p(const void *keys, const float *kscale, int batch, int64_t kv_len,
                    const int32_t *seq_len, int D, int P, int64_t page_lo, int64_t page_hi,
                    uint16_t *pk, hipStream_t st, const PagedTab &pt)
{
    // pages of at least one 16-byte piece per lane group take the one-wave-per-page kernel;
    // smaller pages (P <= 8) the per-element one.  Both pointers are 16-byte aligned (checked
    // by the entry point).
    bool done = false;
    hipError_t e = hipSuccess;
    if (D == 128)
        e = launch_wave_p<FP8, 128>(keys, kscale, batch, kv_len, seq_len, P, page_lo, page_hi, pk, st, done, pt);
    else if (D == 64)
        e = launch_wave_p<FP8, 64>(keys, kscale, batch, kv_len, seq_len, P, page_lo, page_hi, pk, st, done, pt);
    if (done) return e;
    if (pt.btab) return hipErrorInvalidValue; // paged pages are at least 32 keys
    const int64_t n_pages = (kv_len + P - 1) / P;
    const int64_t threads = (page_hi - page_lo) * (D / 2);
    const dim3 grid((unsigned)((threads + 255) / 256), (unsigned)batch);
    switch (P) {
#define LSA_PS(PP)                                                                                  \
    case PP:                                                                                        \
        hipLaunchKernelGGL((page_summary_kernel<FP8, PP>), grid, dim3(256), 0, st, keys, kscale,    \
                           kv_len, seq_len, D, page_lo, page_hi, n_pages, pk);                      \
        break;
        LSA_PS(1) LSA_PS(2) LSA_PS(4) LSA_PS(8)
#undef LSA_PS
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace

hipError_t launch_page_summary(const void *keys, int fp8, const float *kscale, int batch,
                               int64_t kv_len, const int32_t *seq_len, int dim, int page,
                               int64_t page_lo, int64_t page_hi, uint16_t *page_keys,
                               hipStream_t stream, const PagedTab &paged)
{
    if (page_hi <= page_lo || batch == 0) return hipSuccess;
    return fp8 ? launch_p<true>(keys, kscale, batch, kv_len, seq_len, dim, page, page_lo, page_hi,
                                page_keys, stream, paged)
               : launch_p<false>(keys, kscale, batch, kv_len, seq_len, dim, page, page_lo, page_hi,
                                 page_keys, stream, paged);
}

} // namespace lsa
