// device.hpp -- device-side building blocks shared by the gfx950 kernels of the LSA library:
// vector types for the bf16 MFMA instructions, number-format conversions, the order-preserving
// float -> uint32 key used by selection, and wave / block scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace lsa {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(16)));
typedef __bf16 bf16x2_t __attribute__((__vector_size__(4)));
typedef float f32x16_t __attribute__((__vector_size__(64)));
typedef float f32x4_t __attribute__((__vector_size__(16)));

constexpr int kWave = 64;

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).  Indices into register
// arrays stay constant expressions, so the arrays never leave registers.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From &f)
{
    static_assert(sizeof(To) == sizeof(From), "size");
    return __builtin_bit_cast(To, f);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load as one native vector value (a struct copy of uint4 becomes a memcpy that keeps
// register arrays of it in scratch memory).
__device__ __forceinline__ uint4 ld16(const void *p)
{
    return bitcast<uint4>(*reinterpret_cast<const u32x4_t *>(p));
}

// The same with the non-temporal hint, for data read once (a key stream, gathered rows): it
// need not stay in the caches, which keeps them for what is read again.
__device__ __forceinline__ uint4 ld16_nt(const void *p)
{
    return bitcast<uint4>(__builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p)));
}

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).  Lane l supplies A row l%32 and B column
// l%32, each with K elements 8*(l/32) .. 8*(l/32)+7; it receives D[8*(r/4) + 4*(l/32) + r%4][l%32]
// in register r.
__device__ __forceinline__ f32x16_t mfma_32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).  Lane l supplies A row l%16 and B column
// l%16, each with K elements 8*(l/16) .. 8*(l/16)+7; it receives D[4*(l/16) + r][l%16] in
// register r.
__device__ __forceinline__ f32x4_t mfma_16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// ReLU as one integer max on the bit pattern: every float with the sign bit set (including -0)
// is a negative int32, every other one a non-negative int32 in the same order.  Exact, and one
// instruction (fmaxf would also quiet NaNs first).
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// binary32 -> bfloat16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Four e4m3fn codes (bytes of `v`, lowest first) -> four bf16 values, exactly (every e4m3fn
// value is a bf16 value).  Uses gfx950's scaled fp8 -> bf16 conversion with a unit scale.
__device__ __forceinline__ uint2 e4m3x4_to_bf16x4(uint32_t v)
{
    bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, false);
    bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, true);
    return make_uint2(bitcast<uint32_t>(lo), bitcast<uint32_t>(hi));
}

// Eight e4m3fn codes -> one MFMA operand of eight bf16.
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16x8(uint2 v)
{
    uint2 a = e4m3x4_to_bf16x4(v.x);
    uint2 b = e4m3x4_to_bf16x4(v.y);
    return bitcast<bf16x8_t>(make_uint4(a.x, a.y, b.x, b.y));
}

// Monotone map of a finite binary32 onto uint32: a > b  <=>  key(a) > key(b); -0 maps like +0.
// Every finite value maps to a key >= 0x00800000 and -inf to 0x007FFFFF, so 0 is free as "no element".
__device__ __forceinline__ uint32_t order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u << 1) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Ragged batches: sequence b holds seq_len[b] valid keys of the kv_len-row (padded) cache, and
// its query i sits at position seq_pos0[b] + i.  Null arrays: every sequence has kv_len keys and
// starts at q_pos0.  Lengths are clamped into [0, kv_len], positions below 0 to 0.
__device__ __forceinline__ int64_t seq_keys(const int32_t *seq_len, int b, int64_t kv_len)
{
    if (!seq_len) return kv_len;
    const int64_t L = seq_len[b];
    return L < 0 ? 0 : (L > kv_len ? kv_len : L);
}

__device__ __forceinline__ int64_t seq_first(const int32_t *seq_pos0, int b, int64_t q_pos0)
{
    if (!seq_pos0) return q_pos0;
    const int64_t p = seq_pos0[b];
    return p < 0 ? 0 : p;
}

// Keys query t of sequence b sees: [0, V).
__device__ __forceinline__ int64_t valid_len(const int32_t *seq_len, const int32_t *seq_pos0,
                                             int b, int64_t t, int64_t kv_len, int64_t q_pos0)
{
    const int64_t L = seq_keys(seq_len, b, kv_len);
    const int64_t V = seq_first(seq_pos0, b, q_pos0) + t + 1;
    return V < L ? V : L;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

// Inclusive prefix sum across the 64 lanes of a wave, in DPP steps (no LDS round trips):
// shifts by 1, 2, 4 and 8 within each row of 16 lanes, then lane 15 of each row added to the
// next row (rows 1 and 3) and lane 31 to the upper half (rows 2 and 3).  Lanes whose source lies
// outside the row, and rows outside the row mask, add 0.
__device__ __forceinline__ int wave_inclusive_scan(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false); // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false); // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false); // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false); // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false); // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false); // row_bcast:31
    return x;
}

// Inclusive prefix sum within each row of 16 lanes (the first four steps above): a row's last
// lane ends with the row's total.
__device__ __forceinline__ uint32_t row_inclusive_scan(uint32_t x)
{
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false); // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false); // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false); // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false); // row_shr:8
    return x;
}

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
    return x;
}

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

// Exclusive prefix sum over the whole block (NWAVES waves) in thread order.  `scratch` holds
// NWAVES + 1 ints of LDS.  Returns the thread's exclusive prefix; *total gets the block sum.
// Contains barriers: every thread of the block must call it.
template <int NWAVES>
__device__ __forceinline__ int block_exclusive_scan(int v, int *scratch, int *total)
{
    const int lane = lane_id(), wid = wave_id();
    int inc = wave_inclusive_scan(v);
    if (lane == kWave - 1) scratch[wid] = inc;
    __syncthreads();
    if (wid == 0) {
        int s = lane < NWAVES ? scratch[lane] : 0;
        int t = wave_inclusive_scan(s);
        if (lane < NWAVES) scratch[lane] = t - s;
        if (lane == NWAVES - 1) scratch[NWAVES] = t;
    }
    __syncthreads();
    int ex = inc - v + scratch[wid];
    *total = scratch[NWAVES];
    __syncthreads();
    return ex;
}

} // namespace lsa
