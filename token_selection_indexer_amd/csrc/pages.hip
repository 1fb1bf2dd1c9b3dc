// pages.hip -- page keys for Hierarchical Indexing.
//
// The model card's HI bullet recalls candidate blocks by coarse scores without defining a
// block's coarse key.  This library defines the key of page p (P tokens, P a power of two) as the
// mean of its dequantised indexer keys with a fixed binary32 rounding sequence:
//   v[j]  = fp32(scale[s] * e4m3(kq[s][i]))  (bf16 keys: the value), s = p*P + j; +0 past kv_len
//   sum   = pairwise tree sum of v[0..P): halves summed separately, then added, recursively
//   pk    = bf16_rne(sum / n_p), n_p = tokens of the page that exist
// No FMA contraction anywhere (explicit round-to-nearest multiply / add / divide), so the result
// is reproducible bit for bit.
//
// Layout: D/2 threads per page, each owning two adjacent key elements, so every token of the
// page is one contiguous D-element load across the threads.  The tree is a binary counter over
// the P tokens held in registers (fully unrolled per P).
#include "device.hpp"
#include "internal.hpp"

namespace lsa {
namespace {

template <bool FP8, int P>
__global__ __launch_bounds__(256) void page_summary_kernel(const void *keys, const float *kscale,
                                                           int64_t kv_len, int D, int64_t page_lo,
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
    const int64_t n_p = min((int64_t)P, kv_len - s0);

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

template <bool FP8>
hipError_t launch_p(const void *keys, const float *kscale, int batch, int64_t kv_len, int D,
                    int P, int64_t page_lo, int64_t page_hi, uint16_t *pk, hipStream_t st)
{
    const int64_t n_pages = (kv_len + P - 1) / P;
    const int64_t threads = (page_hi - page_lo) * (D / 2);
    const dim3 grid((unsigned)((threads + 255) / 256), (unsigned)batch);
    switch (P) {
#define LSA_PS(PP)                                                                                  \
    case PP:                                                                                        \
        hipLaunchKernelGGL((page_summary_kernel<FP8, PP>), grid, dim3(256), 0, st, keys, kscale,    \
                           kv_len, D, page_lo, page_hi, n_pages, pk);                               \
        break;
        LSA_PS(1) LSA_PS(2) LSA_PS(4) LSA_PS(8) LSA_PS(16) LSA_PS(32) LSA_PS(64) LSA_PS(128) LSA_PS(256)
#undef LSA_PS
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace

hipError_t launch_page_summary(const void *keys, int fp8, const float *kscale, int batch,
                               int64_t kv_len, int dim, int page, int64_t page_lo,
                               int64_t page_hi, uint16_t *page_keys, hipStream_t stream)
{
    if (page_hi <= page_lo || batch == 0) return hipSuccess;
    return fp8 ? launch_p<true>(keys, kscale, batch, kv_len, dim, page, page_lo, page_hi, page_keys, stream)
               : launch_p<false>(keys, kscale, batch, kv_len, dim, page, page_lo, page_hi, page_keys, stream);
}

} // namespace lsa
