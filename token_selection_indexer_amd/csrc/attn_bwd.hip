// attn_bwd.hip -- gradients of the attention over the selected tokens (the training path).
//
// (Paper summary page, abstract: LSA trains natively to one million tokens, so the sparse
// attention carries gradients; Baidu Cloud article, "3. Sparse Attention Calculator": the
// forward is ordinary softmax attention over the selected tokens.)  For query t, head h and the
// valid entries j of its index list, with P_j = exp(scale q.K_j - lse) from the forward:
//   dP_j = dO . V_j,   D = dO . O,   dS_j = P_j (dP_j - D)
//   dq  += scale sum_j dS_j K_j,   dK_j += scale dS_j q,   dV_j += P_j dO
// D uses the forward's output O (the softmax-weighted sum of dP equals dO . O).
//
// Latent (MLA) kernel.  A workgroup of 4 waves owns one (sequence, query, group of 16 heads) and
// a chunk of the index list, in rounds of 16 selected rows staged in LDS through registers (as
// in the forward kernel, two workgroups per CU).  Per round:
//   S  [16 rows x 16 heads] = K . Q^T     v_mfma_f32_16x16x32_bf16, waves 0-1 (halves of d_qk)
//   dP [16 rows x 16 heads] = V . dO^T    v_mfma_f32_16x16x32_bf16, waves 2-3 (halves of d_v)
//   P, dS per (row, head) in fp32, then as bf16 pairs hi + lo (hi = bf16(x), lo = bf16(x - hi))
//   so that the products below keep about 16 significant bits of P and dS
//   dQ^T [d_qk x 16 heads] += K^T . (scale dS)     v_mfma_f32_16x16x16_bf16, 9 column tiles per
//                                                  wave, K^T by transposing LDS reads
//   dKV  [16 rows x d_qk]   = (scale dS) . Q + P . dO (first d_v columns), 9 tiles per wave,
//                             added to the cache gradient with fp32 atomics
// At the end every wave adds its dQ columns (fp32 atomics: the chunks of one query add up).
//
// Per-head kernel (any head count, d <= 256, separate K and V): one wave per (query, head),
// lanes own columns; the two dot products per row are wave sums.
#include "device.hpp"
#include "internal.hpp"
#include "si_layout.hpp"

namespace lsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

constexpr int BR = 16;          // selected rows per round
constexpr int MLA_DQK = 576;
constexpr int MLA_DV = 512;
constexpr int MAX_SPLIT = 32;

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4v_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

__device__ __forceinline__ bool row_ok(int32_t id, int64_t n) { return id >= 0 && id < n; }

// gfx950 transposing LDS read: within each group of 16 lanes, lane j receives element j%4 of
// the 8 bytes addressed by lanes j/4 + 4e of the group, e = 0..3.
__device__ __forceinline__ s16x4_t ds_read_tr16(const uint8_t *lds_byte_ptr)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t *)(__attribute__((address_space(3))) uint8_t *)lds_byte_ptr);
}

// D(16x16, fp32) += A(16x16, bf16) * B(16x16, bf16): lane l supplies A row l%16 and B column l%16
// with K elements 4*(l/16) .. +3, and receives D[4*(l/16) + r][l%16] in register r.
__device__ __forceinline__ f32x4v_t mfma_16x16x16(s16x4_t a, s16x4_t b, f32x4v_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// LDS chunk slot of 16-byte chunk c of staged row r: c ^ sigma(r & 7), sigma(x) = 2(x&3) + x/4
// (a bijection on 0..7): the 16-row logit reads (one chunk per row) and the transposing reads
// (4 rows x 2 chunks per 16 lanes) fall on distinct bank groups.
__device__ __forceinline__ int swz(int c, int r)
{
    const int x = r & 7;
    return c ^ ((2 * (x & 3)) | (x >> 2));
}

// bf16 bits of x (round to nearest even) and of the remainder x - bf16(x).
__device__ __forceinline__ void split_bf16(float x, uint16_t &hi, uint16_t &lo)
{
    const uint32_t h = f32_to_bf16_bits(x);
    hi = (uint16_t)h;
    lo = (uint16_t)f32_to_bf16_bits(x - bf16_bits_to_f32(h));
}

// Workgroup barrier that completes only the LDS traffic (the next round's row loads stay in
// flight across it); the compiler-only fences keep memory accesses from moving across it.
__device__ __forceinline__ void ring_barrier()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0); vmcnt and expcnt: no wait
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---- Streaming-Aware entries: which (query, row) pairs the key-major pass takes (si_layout.hpp) ----
using si::SQC;
using si::SRB;
using si::imax;
using si::imin;
using SiPlan = si::Plan;

template <int DQK, int DV>
__global__ __launch_bounds__(256, 2) void mla_attn_bwd_kernel(AttnBwdArgs a)
{
    constexpr int ROWB = DQK * 2;               // LDS bytes per staged row
    constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
    constexpr int NCH = BR * CPR;               // chunks per round
    constexpr int CPT = (NCH + 255) / 256;      // chunks per thread per round (the last partial)
    constexpr int KSH = DQK / 32 / 2;           // logit K-steps per wave (9)
    constexpr int KVH = DV / 32 / 2;            // dP K-steps per wave (8)
    constexpr int NT = DQK / 16 / 4;            // column tiles per wave (9)
    static_assert(KSH >= KVH && (DQK / 16) % 4 == 0 && DV % 64 == 0, "shape");

    __shared__ __attribute__((aligned(16))) uint8_t buf0[BR * ROWB];
    __shared__ __attribute__((aligned(16))) uint8_t buf1[BR * ROWB];
    __shared__ float part[4][BR][17];                      // [wave][row][head] partial products
    __shared__ __attribute__((aligned(16))) uint16_t pA[2][BR][16]; // P hi / lo   [row][head]
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][BR][16]; // dS hi / lo  [row][head]
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][16][BR]; // dS hi / lo  [head][row]
    __shared__ int32_t rid[4][BR];                         // row ids of rounds i .. i+3 (i % 4)
    __shared__ float Dh[16], lse2[16];
    auto slot_buf = [&](auto SLOT) -> uint8_t * {
        if constexpr (decltype(SLOT)::value == 0) return buf0;
        else return buf1;
    };

    const int HG = a.heads / 16;
    const int b = blockIdx.z;
    const int t = blockIdx.y / HG;
    const int hg = blockIdx.y % HG;
    const int split = blockIdx.x;
    const int l = lane_id(), w = wave_id();
    const int g4 = l >> 4, c16 = l & 15;
    const int64_t qrow = (int64_t)b * a.n_q + t;
    const int64_t qh0 = qrow * a.heads + 16 * hg; // (query, head 0 of the group)

    const int chunk = ((a.n_idx + a.n_split - 1) / a.n_split + BR - 1) / BR * BR;
    const int c_begin = split * chunk;
    const int c_end = min(a.n_idx, c_begin + chunk);
    const int n_rounds = c_end > c_begin ? (c_end - c_begin + BR - 1) / BR : 0;
    const int32_t *idx_row = a.idx + qrow * a.n_idx;
    const int64_t seq_rows = seq_keys(a.seq_len, b, a.kv_len);
    // the key-major pass adds this query's Streaming-Aware entries to the cache gradient
    const int64_t v_si = si::valid_len(a, t);
    const bool si_q = a.si && v_si - a.window >= a.sink;
    auto id_load = [&](int round) -> int32_t { // unconditional load of a clamped entry
        const int j = c_begin + round * BR + (int)(threadIdx.x % BR);
        return idx_row[min(j, max(c_end - 1, 0))];
    };
    auto id_mask = [&](int round, int32_t raw) -> int32_t {
        const int j = c_begin + round * BR + (int)(threadIdx.x % BR);
        return (round < n_rounds && j < c_end && row_ok(raw, seq_rows)) ? raw : -1;
    };
    if (threadIdx.x < BR) {
        rid[0][threadIdx.x] = id_mask(0, id_load(0));
        rid[1][threadIdx.x] = id_mask(1, id_load(1));
    }
    // D = dO . O and lse in base 2, per head: 16 threads per head, 32 columns each
    {
        const int h = threadIdx.x >> 4, p = threadIdx.x & 15;
        const uint16_t *dop = a.dout + (qh0 + h) * DV + 32 * p;
        const uint16_t *op = a.out + (qh0 + h) * DV + 32 * p;
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < 32; c += 8) {
            const uint4 x = ld16(dop + c), y = ld16(op + c);
            const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc = fmaf(__uint_as_float(xs[e] << 16), __uint_as_float(ys[e] << 16), acc);
                acc = fmaf(__uint_as_float(xs[e] & 0xffff0000u), __uint_as_float(ys[e] & 0xffff0000u), acc);
            }
        }
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 16);
        if (p == 0) {
            Dh[h] = acc;
            lse2[h] = a.lse[qh0 + h] * kLog2e;
        }
    }
    // Phase-A operands (B side): waves 0-1 Q^T over their half of d_qk, waves 2-3 dO^T over
    // their half of d_v; lane l holds head l%16, K elements 8 (l/16) .. +7 of each 32-step.
    const int role = w >> 1, half = w & 1;
    bf16x8_t af[KSH];
    {
        const uint16_t *src = role == 0 ? a.q + (qh0 + c16) * DQK + 32 * KSH * half
                                        : a.dout + (qh0 + c16) * DV + 32 * KVH * half;
#pragma unroll
        for (int kk = 0; kk < KSH; ++kk)
            af[kk] = (role == 0 || kk < KVH) ? bitcast<bf16x8_t>(ld16(src + 32 * kk + 8 * g4))
                                             : bf16x8_t{};
    }
    // dKV operands (B side): Q[head 4 (l/16) + e][col 16 T + l%16] and the same of dO, for this
    // wave's column tiles T = NT w + tt (dO only on the first DV columns)
    s16x4_t qb[NT], db[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
        const int col = 16 * (NT * w + tt) + c16;
        uint16_t qv[4], dv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qv[e] = a.q[(qh0 + 4 * g4 + e) * DQK + col];
            dv[e] = col < DV ? a.dout[(qh0 + 4 * g4 + e) * DV + col] : (uint16_t)0;
        }
        qb[tt] = s16x4_t{(short)qv[0], (short)qv[1], (short)qv[2], (short)qv[3]};
        db[tt] = s16x4_t{(short)dv[0], (short)dv[1], (short)dv[2], (short)dv[3]};
    }
    f32x4v_t dq[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) dq[tt] = f32x4v_t{};
    const uint8_t *kv_b = reinterpret_cast<const uint8_t *>(a.k) + (int64_t)b * a.kv_len * a.k_stride * 2;
    float *dkv_b = a.dk + (int64_t)b * a.kv_len * DQK;
    const float sl2 = a.scale * kLog2e;
    __syncthreads();

    // A round's rows through registers: thread t loads chunks f = 256 j + t (row f / CPR, chunk
    // f % CPR); the last, partial step re-reads a valid chunk.  Skipped rows read row 0 and
    // are stored as zeros (their weights are zero; zeros keep any non-finite value of row 0 out).
    uint4 stage[CPT];
    auto load_round = [&](const int32_t *ids) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int f = min(j * 256 + (int)threadIdx.x, NCH - 1);
            const int r = f / CPR, c = f % CPR;
            const int32_t id = ids[r];
            stage[j] = ld16(kv_b + (int64_t)(id < 0 ? 0 : id) * a.k_stride * 2 + c * 16);
        }
    };
    auto store_round = [&](uint8_t *dst, const int32_t *ids) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int f = j * 256 + (int)threadIdx.x;
            if (f >= NCH) break;
            const int r = f / CPR, c = f % CPR;
            const uint4 v = ids[r] < 0 ? make_uint4(0, 0, 0, 0) : stage[j];
            *reinterpret_cast<uint4 *>(dst + r * ROWB + swz(c, r) * 16) = v;
        }
    };

    if (n_rounds > 0) {
        load_round(rid[0]);
        store_round(buf0, rid[0]);
    }
    __builtin_amdgcn_s_waitcnt(0);
    for (int i0 = 0; i0 < n_rounds; i0 += 2) static_for<0, 2>([&](auto SLOT) {
        constexpr int S = decltype(SLOT)::value;
        const int i = i0 + S;
        if (i >= n_rounds) return;
        ring_barrier(); // round i is in buf[S]; round i - 1 is fully consumed
        const int32_t *ids = rid[i & 3];
        const int32_t next_raw = id_load(i + 2);
        load_round(rid[(i + 1) & 3]);
        const uint8_t *cb = slot_buf(SLOT);
        // phase A: partial S (waves 0-1) or dP (waves 2-3), lane holds [row 4 g4 + e][head c16]
        {
            f32x4_t acc = f32x4_t{};
            const uint8_t *kr = cb + c16 * ROWB;
            if (role == 0) {
#pragma unroll
                for (int kk = 0; kk < KSH; ++kk) {
                    const int c = 4 * (KSH * half + kk) + g4;
                    acc = mfma_16x16x32(bitcast<bf16x8_t>(ld16(kr + 16 * swz(c, c16))), af[kk], acc);
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < KVH; ++kk) {
                    const int c = 4 * (KVH * half + kk) + g4;
                    acc = mfma_16x16x32(bitcast<bf16x8_t>(ld16(kr + 16 * swz(c, c16))), af[kk], acc);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) part[w][4 * g4 + e][c16] = acc[e];
        }
        ring_barrier();
        // P and scale dS for (row, head) = (thread / 16, thread % 16), as bf16 hi + lo
        {
            const int r = threadIdx.x >> 4, h = threadIdx.x & 15;
            const float s = part[0][r][h] + part[1][r][h];
            const float dp = part[2][r][h] + part[3][r][h];
            const float P = ids[r] >= 0 ? exp2f(s * sl2 - lse2[h]) : 0.0f;
            const float dS = P * (dp - Dh[h]) * a.scale;
            uint16_t ph, pl, sh, sl;
            split_bf16(P, ph, pl);
            split_bf16(dS, sh, sl);
            pA[0][r][h] = ph;
            pA[1][r][h] = pl;
            sA[0][r][h] = sh;
            sA[1][r][h] = sl;
            sB[0][h][r] = sh;
            sB[1][h][r] = sl;
            // ids of round i + 2 into the ring slot rounds i - 2 and earlier used
            if (threadIdx.x < BR) rid[(i + 2) & 3][threadIdx.x] = id_mask(i + 2, next_raw);
        }
        ring_barrier();
        // phase B: dQ^T tiles and the cache-gradient tiles of this wave's columns
        {
            const s16x4_t sbh = *reinterpret_cast<const s16x4_t *>(&sB[0][c16][4 * g4]);
            const s16x4_t sbl = *reinterpret_cast<const s16x4_t *>(&sB[1][c16][4 * g4]);
            const s16x4_t sah = *reinterpret_cast<const s16x4_t *>(&sA[0][c16][4 * g4]);
            const s16x4_t sal = *reinterpret_cast<const s16x4_t *>(&sA[1][c16][4 * g4]);
            const s16x4_t pah = *reinterpret_cast<const s16x4_t *>(&pA[0][c16][4 * g4]);
            const s16x4_t pal = *reinterpret_cast<const s16x4_t *>(&pA[1][c16][4 * g4]);
            int32_t rowid[4]; // -1: no atomic update for this row (skipped, or key-major)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                rowid[e] = ids[4 * g4 + e];
                if (si_q && rowid[e] >= 0 && si::taken(a, v_si, c_begin + i * BR + 4 * g4 + e, rowid[e]))
                    rowid[e] = -1;
            }
            // transposing reads: lane j of group g4 addresses row 4 g4 + j/4, columns
            // 16 T + 4 (j%4) .. +3
            const int vr = 4 * g4 + (c16 >> 2);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const int T = NT * w + tt;
                const int col = 16 * T + 4 * (c16 & 3);
                const s16x4_t kt = ds_read_tr16(cb + vr * ROWB + swz(col >> 3, vr) * 16 + (col & 7) * 2);
                dq[tt] = mfma_16x16x16(kt, sbh, dq[tt]);
                dq[tt] = mfma_16x16x16(kt, sbl, dq[tt]);
                f32x4v_t g = f32x4v_t{};
                g = mfma_16x16x16(sah, qb[tt], g);
                g = mfma_16x16x16(sal, qb[tt], g);
                if (16 * T < DV) {
                    g = mfma_16x16x16(pah, db[tt], g);
                    g = mfma_16x16x16(pal, db[tt], g);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (rowid[e] >= 0) atomicAdd(dkv_b + (int64_t)rowid[e] * DQK + 16 * T + c16, g[e]);
            }
        }
        store_round(slot_buf(std::integral_constant<int, S ^ 1>{}), rid[(i + 1) & 3]);
    });
    // dQ: lane holds dQ[head c16][col 16 T + 4 g4 + e]
    float *dqp = a.dq + (qh0 + c16) * DQK;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) atomicAdd(dqp + 16 * (NT * w + tt) + 4 * g4 + e, dq[tt][e]);
}

// Key-major pass over the Streaming-Aware entries.  Neighbouring queries of a prefill chunk
// share their sink rows and most of their window rows, and the kernel above adds each of those
// rows' gradient once per query through fp32 atomics, whose rate bounds it.  Here a workgroup
// of 8 waves owns SRB consecutive cache rows (a block of the sink, or of the band the windows
// cover) and up to SQC of the queries whose sink or window reach them; it sums their
// contributions in registers and adds each row column once.  Per query (q, dO and out staged
// through registers, the next query's loads in flight during this one's products):
//   S^T  [64 rows x 16 heads] = K . Q^T    v_mfma_f32_16x16x32_bf16, one 16-row tile per wave,
//   dP^T [64 rows x 16 heads] = V . dO^T   waves 0-3 S, waves 4-7 dP
//   P, dS per (row, head) in fp32 (zero where the pair is not this pass's: si_entry), as bf16
//   hi + lo pairs as above
//   dKV [64 rows x d_qk] += (scale dS)^T . Q + P^T . dO   v_mfma_f32_16x16x16_bf16, 2 row tiles
//                                                        x 9 column tiles per wave, Q and dO
//                                                        by transposing LDS reads
template <int DQK, int DV>
__global__ __launch_bounds__(512, 1) void mla_attn_bwd_si_kernel(AttnBwdArgs a, SiPlan p)
{
    constexpr int ROWB = DQK * 2;          // LDS bytes per cache row
    constexpr int CPR = ROWB / 16;         // 16-byte chunks per cache row
    constexpr int QST = DQK * 2 + 16;      // padded LDS bytes per staged q row
    constexpr int OST = DV * 2 + 16;       // padded LDS bytes per staged dO row
    constexpr int QCH = 16 * DQK / 8;      // 16-byte chunks of the 16 heads' q
    constexpr int QPT = (QCH + 511) / 512; // ... per thread (the last step partial)
    constexpr int KS = DQK / 32, VS = DV / 32;
    constexpr int CTW = DQK / 16 / 4;      // column tiles per wave
    static_assert(16 * DV / 8 == 2 * 512 && (DQK / 16) % 4 == 0 && DV % 16 == 0, "shape");

    __shared__ __attribute__((aligned(16))) uint8_t kblk[SRB * ROWB];
    __shared__ __attribute__((aligned(16))) uint8_t qs[16 * QST];
    __shared__ __attribute__((aligned(16))) uint8_t dos[16 * OST];
    __shared__ float part[2][SRB][17];                               // S, dP   [row][head]
    __shared__ __attribute__((aligned(16))) uint16_t pA[2][SRB][16]; // P hi / lo  [row][head]
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][SRB][16]; // dS hi / lo [row][head]
    __shared__ float Dh[16], lse2[16];
    __shared__ int rsel[SRB];                                        // the pair is this pass's

    const int HG = a.heads / 16;
    const int b = blockIdx.z / HG, hg = blockIdx.z % HG;
    // workgroup -> (block, query chunk): the sink blocks' chunks, then the window blocks'
    int blk, chunk;
    si::workgroup(p, (int)blockIdx.x, blk, chunk);
    int64_t r0, r1, t_lo, t_hi;
    si::block(a, p, blk, r0, r1, t_lo, t_hi);
    const int64_t c0 = t_lo + (int64_t)chunk * SQC;
    const int64_t c1 = imin(t_hi, c0 + SQC);
    if (c0 >= c1 || r0 >= r1) return; // the same for every thread
    const bool sink_blk = blk < p.nsb;
    const int tid = threadIdx.x, l = lane_id(), w = wave_id();
    const int g4 = l >> 4, c16 = l & 15;

    // the block's rows, chunks swizzled as in the query-major kernel; rows past r1 are zeros
    const uint8_t *kv_b = reinterpret_cast<const uint8_t *>(a.k) + (int64_t)b * a.kv_len * a.k_stride * 2;
    for (int f = tid; f < SRB * CPR; f += 512) {
        const int r = f / CPR, c = f % CPR;
        const int64_t row = imin(r0 + r, r1 - 1);
        const uint4 v = ld16(kv_b + row * a.k_stride * 2 + c * 16);
        *reinterpret_cast<uint4 *>(kblk + r * ROWB + swz(c, r) * 16) =
            r0 + r < r1 ? v : make_uint4(0, 0, 0, 0);
    }

    // one query's operands through registers: q chunk f = 512 u + tid (head f / (DQK / 8));
    // dO and out: thread tid holds chunks 2 (tid % 32) + {0, 1} of head tid / 32; lse of head
    // tid (tid < 16); the index entry the layout gives row r0 + tid (tid < SRB)
    uint4 qreg[QPT], dreg[2], oreg[2];
    float lreg = 0.0f;
    int32_t ireg = -1;
    auto load_query = [&](int64_t t) {
        const int64_t qrow = (int64_t)b * a.n_q + t;
        const int64_t qh0 = qrow * a.heads + 16 * hg;
        const uint16_t *qp = a.q + qh0 * DQK;
#pragma unroll
        for (int u = 0; u < QPT; ++u) qreg[u] = ld16(qp + 8 * min(512 * u + tid, QCH - 1));
        const int64_t ob = (qh0 + (tid >> 5)) * DV + 16 * (tid & 31);
        dreg[0] = ld16(a.dout + ob);
        dreg[1] = ld16(a.dout + ob + 8);
        oreg[0] = ld16(a.out + ob);
        oreg[1] = ld16(a.out + ob + 8);
        lreg = a.lse[qh0 + (tid & 15)];
        const int64_t V = si::valid_len(a, t), r = r0 + (tid & (SRB - 1));
        const int64_t j = sink_blk ? r : a.sink + r - (V - a.window);
        ireg = a.idx[qrow * a.n_idx + imin(imax(j, 0), a.n_idx - 1)]; // clamped, always valid
    };
    auto stage_query = [&](int64_t t) {
#pragma unroll
        for (int u = 0; u < QPT; ++u) {
            const int f = 512 * u + tid;
            if (f < QCH)
                *reinterpret_cast<uint4 *>(qs + (f / (DQK / 8)) * QST + (f % (DQK / 8)) * 16) = qreg[u];
        }
        const int h = tid >> 5, c = 2 * (tid & 31);
        *reinterpret_cast<uint4 *>(dos + h * OST + c * 16) = dreg[0];
        *reinterpret_cast<uint4 *>(dos + h * OST + (c + 1) * 16) = dreg[1];
        // D = dO . out for head h: 32 threads x 16 columns
        float acc = 0.0f;
        const uint32_t xs[8] = {dreg[0].x, dreg[0].y, dreg[0].z, dreg[0].w,
                                dreg[1].x, dreg[1].y, dreg[1].z, dreg[1].w};
        const uint32_t ys[8] = {oreg[0].x, oreg[0].y, oreg[0].z, oreg[0].w,
                                oreg[1].x, oreg[1].y, oreg[1].z, oreg[1].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc = fmaf(__uint_as_float(xs[e] << 16), __uint_as_float(ys[e] << 16), acc);
            acc = fmaf(__uint_as_float(xs[e] & 0xffff0000u), __uint_as_float(ys[e] & 0xffff0000u), acc);
        }
        // sum over the head's 32 lanes: row sums of 16 lanes, then row 1 (3) adds row 0 (2)
#define LSA_DPP_ADD(CTRL, ROWS) \
    acc += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc), CTRL, ROWS, 0xf, false))
        LSA_DPP_ADD(0x111, 0xf); // row_shr:1
        LSA_DPP_ADD(0x112, 0xf); // row_shr:2
        LSA_DPP_ADD(0x114, 0xf); // row_shr:4
        LSA_DPP_ADD(0x118, 0xf); // row_shr:8
        LSA_DPP_ADD(0x142, 0xa); // row_bcast:15
#undef LSA_DPP_ADD
        if ((tid & 31) == 31) Dh[h] = acc;
        if (tid < 16) lse2[tid] = lreg * kLog2e;
        if (tid < SRB) {
            const int64_t V = si::valid_len(a, t), r = r0 + tid;
            const bool in = r < r1 && (sink_blk || (r >= V - a.window && r < V));
            rsel[tid] = in && (int64_t)ireg == r;
        }
    };

    f32x4_t acc[2][CTW];
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int tt = 0; tt < CTW; ++tt) acc[q2][tt] = f32x4_t{};
    const float sl2 = a.scale * kLog2e;
    const int rt = w & 3, role = w >> 2; // S / dP phase: row tile and operand
    // dKV phase: row tiles rp, rp + 1 and column tiles cg + 4 tt (every wave gets one of the
    // last four tiles, which have no dO part)
    const int rp = 2 * (w >> 2), cg = w & 3;
    load_query(c0);
    for (int64_t t = c0; t < c1; ++t) {
        ring_barrier(); // the previous query's LDS operands are consumed
        stage_query(t);
        if (t + 1 < c1) load_query(t + 1);
        ring_barrier();
        {
            // two accumulator chains (even and odd K-steps), added at the end
            f32x4_t sacc[2] = {f32x4_t{}, f32x4_t{}};
            const int rr = 16 * rt + c16;
            const uint8_t *kr = kblk + rr * ROWB;
            if (role == 0) {
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    const int c = 4 * kk + g4;
                    sacc[kk & 1] = mfma_16x16x32(bitcast<bf16x8_t>(ld16(kr + 16 * swz(c, rr))),
                                                 bitcast<bf16x8_t>(ld16(qs + c16 * QST + c * 16)),
                                                 sacc[kk & 1]);
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < VS; ++kk) {
                    const int c = 4 * kk + g4;
                    sacc[kk & 1] = mfma_16x16x32(bitcast<bf16x8_t>(ld16(kr + 16 * swz(c, rr))),
                                                 bitcast<bf16x8_t>(ld16(dos + c16 * OST + c * 16)),
                                                 sacc[kk & 1]);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) part[role][16 * rt + 4 * g4 + e][c16] = sacc[0][e] + sacc[1][e];
        }
        ring_barrier();
#pragma unroll
        for (int i = 0; i < SRB * 16 / 512; ++i) {
            const int x = tid + 512 * i, r = x >> 4, h = x & 15;
            const float P = rsel[r] ? exp2f(part[0][r][h] * sl2 - lse2[h]) : 0.0f;
            const float dS = P * (part[1][r][h] - Dh[h]) * a.scale;
            uint16_t ph, pl, sh, sl;
            split_bf16(P, ph, pl);
            split_bf16(dS, sh, sl);
            pA[0][r][h] = ph;
            pA[1][r][h] = pl;
            sA[0][r][h] = sh;
            sA[1][r][h] = sl;
        }
        ring_barrier();
        {
            // K index k of the products: hi / lo part k / 16 of head k % 16.  Lane (g4, l%16)
            // supplies A row l%16 with k = 8 g4 .. +7: part g4 / 2, heads 8 (g4 & 1) .. +7
            bf16x8_t sa[2], pa[2];
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
                const int r = 16 * (rp + q2) + c16;
                sa[q2] = bitcast<bf16x8_t>(*reinterpret_cast<const uint4 *>(&sA[g4 >> 1][r][8 * (g4 & 1)]));
                pa[q2] = bitcast<bf16x8_t>(*reinterpret_cast<const uint4 *>(&pA[g4 >> 1][r][8 * (g4 & 1)]));
            }
            // B column l%16 with the same k: heads 8 (g4 & 1) .. +7 of Q (dO), by two transposing
            // reads in which lane j of group g4 addresses head hb + j/4 (hb + 4 + j/4), columns
            // 16 T + 4 (j%4) .. +3; lane l receives [head hb + e][column 16 T + l%16]
            const int hb = 8 * (g4 & 1) + (c16 >> 2);
            auto cat8 = [](s16x4_t lo, s16x4_t hi) {
                const uint2 x = bitcast<uint2>(lo), y = bitcast<uint2>(hi);
                return bitcast<bf16x8_t>(make_uint4(x.x, x.y, y.x, y.y));
            };
#pragma unroll
            for (int tt = 0; tt < CTW; ++tt) {
                const int T = cg + 4 * tt;
                const int col = 16 * T + 4 * (c16 & 3);
                const bf16x8_t qb = cat8(ds_read_tr16(qs + hb * QST + col * 2),
                                         ds_read_tr16(qs + (hb + 4) * QST + col * 2));
#pragma unroll
                for (int q2 = 0; q2 < 2; ++q2) acc[q2][tt] = mfma_16x16x32(sa[q2], qb, acc[q2][tt]);
                if (16 * T < DV) {
                    const bf16x8_t db = cat8(ds_read_tr16(dos + hb * OST + col * 2),
                                             ds_read_tr16(dos + (hb + 4) * OST + col * 2));
#pragma unroll
                    for (int q2 = 0; q2 < 2; ++q2) acc[q2][tt] = mfma_16x16x32(pa[q2], db, acc[q2][tt]);
                }
            }
        }
    }
    // the block's sums into the cache gradient (lane: [row 16 R + 4 g4 + e][column 16 T + l%16])
    float *dkv_b = a.dk + (int64_t)b * a.kv_len * DQK;
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int tt = 0; tt < CTW; ++tt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t row = r0 + 16 * (rp + q2) + 4 * g4 + e;
                const float v = acc[q2][tt][e];
                if (row < r1 && v != 0.0f) atomicAdd(dkv_b + row * DQK + 16 * (cg + 4 * tt) + c16, v);
            }
}

// Per-head kernel: one wave per (query, head); lane l owns columns l, l + 64, ... (d <= 256).
constexpr int MHA_MAXD = 256;

__global__ __launch_bounds__(256) void mha_attn_bwd_kernel(AttnBwdArgs a)
{
    constexpr int CPL = MHA_MAXD / kWave;
    const int l = lane_id(), w = wave_id();
    const int64_t total = (int64_t)a.batch * a.n_q * a.heads;
    const int64_t unit = (int64_t)blockIdx.x * 4 + w; // (b * n_q + t) * heads + h
    if (unit >= total) return;                         // no barriers below
    const int64_t qrow = unit / a.heads;
    const int b = (int)(qrow / a.n_q);
    const int64_t seq_rows = seq_keys(a.seq_len, b, a.kv_len);
    float qv[CPL], gv[CPL], dq[CPL];
    float D = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = l + kWave * i;
        qv[i] = c < a.d_qk ? bf16_bits_to_f32(a.q[unit * a.d_qk + c]) : 0.0f;
        gv[i] = c < a.d_v ? bf16_bits_to_f32(a.dout[unit * a.d_v + c]) : 0.0f;
        const float ov = c < a.d_v ? bf16_bits_to_f32(a.out[unit * a.d_v + c]) : 0.0f;
        D = fmaf(gv[i], ov, D);
        dq[i] = 0.0f;
    }
    D = wave_sum(D);
    const float lse2 = a.lse[unit] * kLog2e;
    const float sl2 = a.scale * kLog2e;
    const uint16_t *kb = a.k + (int64_t)b * a.kv_len * a.k_stride;
    const uint16_t *vb = a.v + (int64_t)b * a.kv_len * a.v_stride;
    float *dkb = a.dk + (int64_t)b * a.kv_len * a.d_qk;
    float *dvb = a.dv + (int64_t)b * a.kv_len * a.d_v;
    const int32_t *idx_row = a.idx + qrow * a.n_idx;
    for (int j = 0; j < a.n_idx; ++j) {
        const int32_t id = idx_row[j];
        if (!row_ok(id, seq_rows)) continue; // wave-uniform
        float kr[CPL], s = 0.0f, dp = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = l + kWave * i;
            kr[i] = c < a.d_qk ? bf16_bits_to_f32(kb[(int64_t)id * a.k_stride + c]) : 0.0f;
            const float vv = c < a.d_v ? bf16_bits_to_f32(vb[(int64_t)id * a.v_stride + c]) : 0.0f;
            s = fmaf(qv[i], kr[i], s);
            dp = fmaf(gv[i], vv, dp);
        }
        s = wave_sum(s);
        dp = wave_sum(dp);
        const float P = exp2f(s * sl2 - lse2);
        const float dS = P * (dp - D) * a.scale;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = l + kWave * i;
            dq[i] = fmaf(dS, kr[i], dq[i]);
            if (c < a.d_qk) atomicAdd(dkb + (int64_t)id * a.d_qk + c, dS * qv[i]);
            if (c < a.d_v) atomicAdd(dvb + (int64_t)id * a.d_v + c, P * gv[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = l + kWave * i;
        if (c < a.d_qk) a.dq[unit * a.d_qk + c] += dq[i]; // this wave is the only writer
    }
}

} // namespace

int attn_bwd_splits(int batch, int n_q, int heads, int n_idx, int latent)
{
    if (!latent) return 1;
    const int64_t units = (int64_t)batch * n_q * (heads / 16);
    const int max_split = (n_idx + 4 * BR - 1) / (4 * BR); // at least 4 rounds per workgroup
    int64_t want = (512 + units - 1) / units;              // two workgroups per CU
    if (want > max_split) want = max_split;
    if (want > MAX_SPLIT) want = MAX_SPLIT;
    return want < 1 ? 1 : (int)want;
}


hipError_t launch_sparse_attn_backward(const AttnBwdArgs &args, hipStream_t st)
{
    const int64_t rows = (int64_t)args.batch * args.n_q;
    if (rows == 0) return hipSuccess;
    AttnBwdArgs a = args;
    if (a.latent) {
        SiPlan p{};
        int nblk = 0, nchunk = 0;
        a.si = a.latent && !a.seq_len &&
                       si::plan(a, p, nblk, nchunk, (int64_t)a.batch * (a.heads / 16))
                   ? 1
                   : 0;
        dim3 grid((unsigned)a.n_split, (unsigned)(a.n_q * (a.heads / 16)), (unsigned)a.batch);
        hipLaunchKernelGGL((mla_attn_bwd_kernel<MLA_DQK, MLA_DV>), grid, dim3(256), 0, st, a);
        if (a.si) {
            dim3 sgrid((unsigned)nchunk, 1u, (unsigned)(a.batch * (a.heads / 16)));
            hipLaunchKernelGGL((mla_attn_bwd_si_kernel<MLA_DQK, MLA_DV>), sgrid, dim3(512), 0, st, a, p);
        }
    } else {
        const int64_t units = rows * a.heads;
        hipLaunchKernelGGL(mha_attn_bwd_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, st, a);
    }
    return hipGetLastError();
}

} // namespace lsa
