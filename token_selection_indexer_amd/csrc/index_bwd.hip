// index_bwd.hip -- gradients of the Lightning-Indexer scores at the selected entries.
//
// (Paper summary page, abstract: LSA trains natively to one million tokens; Baidu Cloud
// article, "1. Lightweight Scoring Module": I[t,s] = sum_h w[t,h] ReLU(q[t,h] . k[s]).)  Given
// the gradient g_j of the score at each selected entry s_j of query t (entries outside [0, V_t)
// carry none), with ReLU'(0) = 0 and G[j,h] = g_j w[t,h] [q[t,h] . k[s_j] > 0]:
//   dw[t,h] += sum_j g_j ReLU(q[t,h] . k[s_j])
//   dq[t,h] += sum_j G[j,h] k[s_j]
//   dk[s_j] += sum_h G[j,h] q[t,h]
//
// One workgroup per (sequence, query, chunk of the index list), one wave per 16 heads (the last
// wave's surplus heads are zero: any head count up to 64), in rounds of 16 selected key rows
// staged in LDS through registers.  Per round and wave:
//   S [16 rows x 16 heads] = K . Q^T                 v_mfma_f32_16x16x32_bf16
//   G from S, g and w in fp32, then as bf16 hi + lo (hi = bf16(G), lo = bf16(G - hi))
//   dQ^T [d x 16 heads] += K^T . G                   v_mfma_f32_16x16x16_bf16, K^T by
//                                                    transposing LDS reads, G in the registers
//                                                    the S tile left it in
//   dK [16 rows x d] = G . Q (this wave's heads)     v_mfma_f32_16x16x16_bf16, G transposed
//                                                    through LDS; the waves' parts are summed
//                                                    in LDS and added to the key gradient with
//                                                    fp32 atomics
// With the Streaming-Aware layout passed (prefill chunks), the sink and window entries' key
// gradient is left to a key-major pass (below) that sums it over the queries sharing each row;
// a round whose entries are all that pass's (or skipped) does no key-gradient work here.
#include "device.hpp"
#include "internal.hpp"
#include "si_layout.hpp"

namespace lsa {
namespace {

constexpr int BR = 16; // selected rows per round
constexpr int MAX_SPLIT = 32;

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4v_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

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

// LDS chunk slot of 16-byte chunk c of staged row r: c ^ sigma(r & 7), sigma(x) = 2(x&3) + x/4.
__device__ __forceinline__ int swz(int c, int r)
{
    const int x = r & 7;
    return c ^ ((2 * (x & 3)) | (x >> 2));
}

__device__ __forceinline__ void ring_barrier()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0); vmcnt and expcnt: no wait
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void index_bwd_kernel(IndexBwdArgs a)
{
    constexpr int ROWB = 2 * D;            // LDS bytes per staged row
    constexpr int CPR = D / 8;             // 16-byte chunks per row
    constexpr int NCH = BR * CPR;          // chunks per round
    constexpr int NTH = NW * 64;
    constexpr int CPT = (NCH + NTH - 1) / NTH;
    constexpr int KS = D / 32;             // K-steps of S
    constexpr int NT = D / 16;             // column tiles of dQ^T and dK
    __shared__ __attribute__((aligned(16))) uint8_t buf0[BR * ROWB];
    __shared__ __attribute__((aligned(16))) uint8_t buf1[BR * ROWB];
    __shared__ __attribute__((aligned(16))) uint16_t gT[NW][2][BR][16]; // G hi / lo [row][head]
    __shared__ float red[NW][BR][D + 4];                                 // waves' dK parts
    __shared__ int32_t rid[4][BR];                                       // ids of rounds i..i+3
    __shared__ int rkey[4];   // the round has key-gradient work here (an entry not skipped and
                              // not the key-major pass's)
    auto slot_buf = [&](auto SLOT) -> uint8_t * {
        if constexpr (decltype(SLOT)::value == 0) return buf0;
        else return buf1;
    };

    const int b = blockIdx.z, t = blockIdx.y, split = blockIdx.x;
    const int l = lane_id(), w = wave_id();
    const int g4 = l >> 4, c16 = l & 15;
    const int H = a.heads;
    const int h = 16 * w + c16; // this lane's head; h >= H is padding
    const int64_t qrow = (int64_t)b * a.n_q + t;
    const int64_t V = valid_len(a.seq_len, a.seq_pos0, b, t, a.kv_len, a.q_pos0);

    const int chunk = ((a.n_idx + a.n_split - 1) / a.n_split + BR - 1) / BR * BR;
    const int c_begin = split * chunk;
    const int c_end = min(a.n_idx, c_begin + chunk);
    const int n_rounds = c_end > c_begin ? (c_end - c_begin + BR - 1) / BR : 0;
    const int32_t *idx_row = a.idx + qrow * a.n_idx;
    const float *g_row = a.dscore + qrow * a.n_idx;
    auto id_load = [&](int round) -> int32_t { // unconditional load of a clamped entry
        const int j = c_begin + round * BR + (int)(threadIdx.x % BR);
        return idx_row[min(j, max(c_end - 1, 0))];
    };
    auto id_mask = [&](int round, int32_t raw) -> int32_t {
        const int j = c_begin + round * BR + (int)(threadIdx.x % BR);
        return (round < n_rounds && j < c_end && raw >= 0 && raw < V) ? raw : -1;
    };
    // ids of round `round` into ring slot `slot`, and whether any entry of it adds its key
    // gradient here (wave 0: threads 0 .. BR-1 hold the round's entries)
    auto put_ids = [&](int slot, int round, int32_t id) {
        if (w != 0) return;
        const int j = c_begin + round * BR + (int)threadIdx.x;
        const bool here = threadIdx.x < BR && id >= 0 && !(a.si && si::taken(a, V, j, id));
        const uint64_t m = __ballot(here);
        if (threadIdx.x < BR) rid[slot][threadIdx.x] = id;
        if (threadIdx.x == 0) rkey[slot] = m != 0u;
    };
    {
        const int32_t id0 = threadIdx.x < BR ? id_mask(0, id_load(0)) : -1;
        const int32_t id1 = threadIdx.x < BR ? id_mask(1, id_load(1)) : -1;
        put_ids(0, 0, id0);
        put_ids(1, 1, id1);
    }
    // operands: head h's q (S, B side), Q[16 w + 4 g4 + e][16 T + c16] (dK, B side), w[h]
    bf16x8_t qf[KS];
    s16x4_t qb[NT];
    {
        const uint16_t *qp = a.q + (qrow * H + min(h, H - 1)) * D + 8 * g4;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
            qf[kk] = h < H ? bitcast<bf16x8_t>(ld16(qp + 32 * kk)) : bf16x8_t{};
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            uint16_t v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int hh = 16 * w + 4 * g4 + e;
                v[e] = hh < H ? a.q[(qrow * H + hh) * D + 16 * tt + c16] : (uint16_t)0;
            }
            qb[tt] = s16x4_t{(short)v[0], (short)v[1], (short)v[2], (short)v[3]};
        }
    }
    const float wh = h < H ? a.w[qrow * H + h] : 0.0f;
    f32x4v_t dq[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) dq[tt] = f32x4v_t{};
    float dw = 0.0f;
    const uint8_t *k_b = reinterpret_cast<const uint8_t *>(a.keys) + (int64_t)b * a.kv_len * ROWB;
    float *dk_b = a.dkeys + (int64_t)b * a.kv_len * D;
    __syncthreads();

    // rows through registers (chunk f = NTH j + thread; the last partial step re-reads a valid
    // chunk); skipped rows read row 0 and are stored as zeros
    uint4 stage[CPT];
    auto load_round = [&](const int32_t *ids) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int f = min(j * NTH + (int)threadIdx.x, NCH - 1);
            const int r = f / CPR, c = f % CPR;
            const int32_t id = ids[r];
            stage[j] = ld16(k_b + (int64_t)(id < 0 ? 0 : id) * ROWB + c * 16);
        }
    };
    auto store_round = [&](uint8_t *dst, const int32_t *ids) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int f = j * NTH + (int)threadIdx.x;
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
        // this round's score gradients, rows 4 g4 + e (0 for skipped entries)
        float gv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * g4 + e;
            gv[e] = ids[r] >= 0 ? g_row[c_begin + i * BR + r] : 0.0f;
        }
        // S tile: lane holds S[row 4 g4 + e][head h]
        f32x4_t s = f32x4_t{};
        {
            const uint8_t *kr = cb + c16 * ROWB;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
                s = mfma_16x16x32(bitcast<bf16x8_t>(ld16(kr + 16 * swz(4 * kk + g4, c16))), qf[kk], s);
        }
        uint16_t gh[4], gl[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float G = s[e] > 0.0f ? gv[e] * wh : 0.0f;
            dw = fmaf(gv[e], fmaxf(s[e], 0.0f), dw);
            gh[e] = (uint16_t)f32_to_bf16_bits(G);
            gl[e] = (uint16_t)f32_to_bf16_bits(G - bf16_bits_to_f32(gh[e]));
            gT[w][0][4 * g4 + e][c16] = gh[e];
            gT[w][1][4 * g4 + e][c16] = gl[e];
        }
        const s16x4_t ghi = s16x4_t{(short)gh[0], (short)gh[1], (short)gh[2], (short)gh[3]};
        const s16x4_t glo = s16x4_t{(short)gl[0], (short)gl[1], (short)gl[2], (short)gl[3]};
        // dQ^T tiles: transposing reads, lane j of group g4 addresses row 4 g4 + j/4, columns
        // 16 tt + 4 (j%4) .. +3
        {
            const int vr = 4 * g4 + (c16 >> 2);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const int col = 16 * tt + 4 * (c16 & 3);
                const s16x4_t kt = ds_read_tr16(cb + vr * ROWB + swz(col >> 3, vr) * 16 + (col & 7) * 2);
                dq[tt] = mfma_16x16x16(kt, ghi, dq[tt]);
                dq[tt] = mfma_16x16x16(kt, glo, dq[tt]);
            }
        }
        // dK part of this wave's heads: A = G [row c16][heads 4 g4 ..], through LDS (skipped
        // for a round whose entries are all skipped or the key-major pass's; uniform)
        const bool key_work = rkey[i & 3] != 0;
        if (key_work) {
            const s16x4_t gah = *reinterpret_cast<const s16x4_t *>(&gT[w][0][c16][4 * g4]);
            const s16x4_t gal = *reinterpret_cast<const s16x4_t *>(&gT[w][1][c16][4 * g4]);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                f32x4v_t p = mfma_16x16x16(gah, qb[tt], f32x4v_t{});
                p = mfma_16x16x16(gal, qb[tt], p);
                // lane holds dK[row 4 g4 + e][col 16 tt + c16]
                if constexpr (NW == 1) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int32_t id = ids[4 * g4 + e];
                        if (id >= 0 && !(a.si && si::taken(a, V, c_begin + i * BR + 4 * g4 + e, id)))
                            atomicAdd(dk_b + (int64_t)id * D + 16 * tt + c16, p[e]);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) red[w][4 * g4 + e][16 * tt + c16] = p[e];
                }
            }
        }
        if (NW > 1 && key_work) {
            ring_barrier(); // every wave's part is in red
            for (int f = threadIdx.x; f < BR * D; f += NTH) {
                const int r = f / D, c = f % D;
                const int32_t id = ids[r];
                float sum = 0.0f;
#pragma unroll
                for (int v = 0; v < NW; ++v) sum += red[v][r][c];
                // the key-major pass adds the Streaming-Aware entries' share
                if (id >= 0 && !(a.si && si::taken(a, V, c_begin + i * BR + r, id)))
                    atomicAdd(dk_b + (int64_t)id * D + c, sum);
            }
        }
        // ids of round i + 2 into the ring slot rounds i - 2 and earlier used
        put_ids((i + 2) & 3, i + 2, threadIdx.x < BR ? id_mask(i + 2, next_raw) : -1);
        store_round(slot_buf(std::integral_constant<int, S ^ 1>{}), rid[(i + 1) & 3]);
    });
    if (h < H) {
        // lane holds dQ[head h][col 16 tt + 4 g4 + e]
        float *dqp = a.dq + (qrow * H + h) * D;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int e = 0; e < 4; ++e) atomicAdd(dqp + 16 * tt + 4 * g4 + e, dq[tt][e]);
    }
    dw += __shfl_xor(dw, 16, kWave);
    dw += __shfl_xor(dw, 32, kWave);
    if (g4 == 0 && h < H) atomicAdd(a.dw + qrow * H + h, dw);
}


// Key-major pass over the Streaming-Aware entries (si_layout.hpp).  A workgroup of 8 waves owns
// SRB = 64 consecutive key rows (a block of the sink, or of the band the windows cover) and up
// to SQC = 128 of the queries whose sink or window reach them, d = 128, all heads (up to 64;
// missing heads are zero).  Per query (its q, w, and the score gradient of every block row the
// list holds where the layout puts it, staged through registers one query ahead):
//   S^T [64 rows x 64 heads] = K . Q^T       v_mfma_f32_16x16x32_bf16, 2 tiles per wave
//   G = g w [S > 0] in fp32 (0 where the row is not this pass's), as bf16 hi + lo
//   dK [64 rows x d] += G . Q                v_mfma_f32_16x16x32_bf16 over 32 heads a step,
//                                            Q by transposing LDS reads, 4 tiles per wave
// and the block's sums are added to the key gradient once, at the end.
constexpr int SI_D = 128, SI_H = 64;

__global__ __launch_bounds__(512, 1) void index_bwd_si_kernel(IndexBwdArgs a, si::Plan p)
{
    constexpr int SRB = si::SRB, SQC = si::SQC, D = SI_D;
    constexpr int ROWB = 2 * D;            // LDS bytes per key row
    constexpr int CPR = D / 8;             // 16-byte chunks per key row
    constexpr int QST = 2 * D + 16;        // padded LDS bytes per staged q row (head)
    constexpr int GST = SI_H + 8;          // padded bf16 per row of G
    constexpr int QCH = SI_H * D / 8;      // 16-byte chunks of one query's q (all heads)
    constexpr int QPT = QCH / 512;         // ... per thread
    constexpr int KS = D / 32;
    static_assert(QCH % 512 == 0 && SRB == 64 && SI_H == 64, "shape");

    __shared__ __attribute__((aligned(16))) uint8_t kblk[SRB * ROWB];
    __shared__ __attribute__((aligned(16))) uint8_t qs[SI_H * QST];
    __shared__ __attribute__((aligned(16))) uint16_t gA[2][SRB][GST]; // G hi / lo [row][head]
    __shared__ float wt[SI_H], gsel[SRB];

    const int b = blockIdx.z;
    int blk, chunk;
    si::workgroup(p, (int)blockIdx.x, blk, chunk);
    int64_t r0, r1, t_lo, t_hi;
    si::block(a, p, blk, r0, r1, t_lo, t_hi);
    const int64_t c0 = t_lo + (int64_t)chunk * SQC;
    const int64_t c1 = si::imin(t_hi, c0 + SQC);
    if (c0 >= c1 || r0 >= r1) return; // the same for every thread
    const bool sink_blk = blk < p.nsb;
    const int tid = threadIdx.x, l = lane_id(), w = wave_id();
    const int g4 = l >> 4, c16 = l & 15;
    const int H = a.heads;

    // the block's key rows, chunks swizzled; rows past r1 are zeros
    const uint8_t *k_b = reinterpret_cast<const uint8_t *>(a.keys) + (int64_t)b * a.kv_len * ROWB;
    for (int f = tid; f < SRB * CPR; f += 512) {
        const int r = f / CPR, c = f % CPR;
        const int64_t row = si::imin(r0 + r, r1 - 1);
        const uint4 v = ld16(k_b + row * ROWB + c * 16);
        *reinterpret_cast<uint4 *>(kblk + r * ROWB + swz(c, r) * 16) =
            r0 + r < r1 ? v : make_uint4(0, 0, 0, 0);
    }

    // one query's operands through registers: q chunk f = 512 u + tid (head f / CPR; heads past
    // H read head H - 1 and are stored as zeros); w of head tid (tid < 64); for block row
    // r0 + tid (tid < 64) the list entry the layout gives it, and that entry's score gradient
    uint4 qreg[QPT];
    float wreg = 0.0f, greg = 0.0f;
    int32_t ireg = -1;
    auto load_query = [&](int64_t t) {
        const int64_t qrow = (int64_t)b * a.n_q + t;
#pragma unroll
        for (int u = 0; u < QPT; ++u) {
            const int f = 512 * u + tid, h = min(f / CPR, H - 1);
            qreg[u] = ld16(a.q + (qrow * H + h) * D + 8 * (f % CPR));
        }
        if (tid < SI_H) wreg = a.w[qrow * H + min(tid, H - 1)];
        if (tid < SRB) {
            const int64_t V = si::valid_len(a, t), r = r0 + tid;
            const int64_t j = si::imin(si::imax(sink_blk ? r : a.sink + r - (V - a.window), 0),
                                       a.n_idx - 1); // clamped, always valid
            ireg = a.idx[qrow * a.n_idx + j];
            greg = a.dscore[qrow * a.n_idx + j];
        }
    };
    auto stage_query = [&](int64_t t) {
#pragma unroll
        for (int u = 0; u < QPT; ++u) {
            const int f = 512 * u + tid, h = f / CPR;
            *reinterpret_cast<uint4 *>(qs + h * QST + (f % CPR) * 16) =
                h < H ? qreg[u] : make_uint4(0, 0, 0, 0);
        }
        if (tid < SI_H) wt[tid] = tid < H ? wreg : 0.0f;
        if (tid < SRB) {
            const int64_t V = si::valid_len(a, t), r = r0 + tid;
            const bool in = r < r1 && (sink_blk || (r >= V - a.window && r < V));
            gsel[tid] = in && (int64_t)ireg == r ? greg : 0.0f;
        }
    };

    // S phase: row tile rt, head tiles 2 hq, 2 hq + 1.  dK phase: row tiles 2 rq, 2 rq + 1 and
    // column tiles cq, cq + 4.
    const int rt = w & 3, hq = w >> 2, rq = w >> 2, cq = w & 3;
    f32x4_t acc[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) acc[x][y] = f32x4_t{};
    load_query(c0);
    for (int64_t t = c0; t < c1; ++t) {
        ring_barrier(); // the previous query's LDS operands are consumed
        stage_query(t);
        if (t + 1 < c1) load_query(t + 1);
        ring_barrier();
        {
            // lane: S[row 16 rt + 4 g4 + e][head 16 (2 hq + x) + c16]
            f32x4_t s[2] = {f32x4_t{}, f32x4_t{}};
            const int rr = 16 * rt + c16;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const int c = 4 * kk + g4;
                const bf16x8_t kf = bitcast<bf16x8_t>(ld16(kblk + rr * ROWB + 16 * swz(c, rr)));
#pragma unroll
                for (int x = 0; x < 2; ++x)
                    s[x] = mfma_16x16x32(kf, bitcast<bf16x8_t>(ld16(qs + (16 * (2 * hq + x) + c16) * QST + c * 16)), s[x]);
            }
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int h = 16 * (2 * hq + x) + c16;
                const float wh = wt[h];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rt + 4 * g4 + e;
                    const float G = s[x][e] > 0.0f ? gsel[r] * wh : 0.0f;
                    const uint32_t hi = f32_to_bf16_bits(G);
                    gA[0][r][h] = (uint16_t)hi;
                    gA[1][r][h] = (uint16_t)f32_to_bf16_bits(G - bf16_bits_to_f32(hi));
                }
            }
        }
        ring_barrier();
        {
            auto cat8 = [](s16x4_t lo, s16x4_t hi) {
                const uint2 x = bitcast<uint2>(lo), y = bitcast<uint2>(hi);
                return bitcast<bf16x8_t>(make_uint4(x.x, x.y, y.x, y.y));
            };
            // K = 32 heads a step: lane (g4, l%16) supplies heads 32 ks + 8 g4 .. +7; Q as B
            // by two transposing reads in which lane j of group g4 addresses head hb + j/4
            // (hb + 4 + j/4), columns 16 T + 4 (j%4) .. +3
#pragma unroll
            for (int ks = 0; ks < SI_H / 32; ++ks) {
                const int hb = 32 * ks + 8 * g4 + (c16 >> 2);
                bf16x8_t ga[2][2];
#pragma unroll
                for (int y = 0; y < 2; ++y) {
                    const int r = 16 * (2 * rq + y) + c16;
#pragma unroll
                    for (int part = 0; part < 2; ++part)
                        ga[y][part] = bitcast<bf16x8_t>(*reinterpret_cast<const uint4 *>(&gA[part][r][32 * ks + 8 * g4]));
                }
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const int col = 16 * (cq + 4 * x) + 4 * (c16 & 3);
                    const bf16x8_t qb = cat8(ds_read_tr16(qs + hb * QST + col * 2),
                                             ds_read_tr16(qs + (hb + 4) * QST + col * 2));
#pragma unroll
                    for (int y = 0; y < 2; ++y) {
                        acc[y][x] = mfma_16x16x32(ga[y][0], qb, acc[y][x]);
                        acc[y][x] = mfma_16x16x32(ga[y][1], qb, acc[y][x]);
                    }
                }
            }
        }
    }
    // the block's sums into the key gradient (lane: [row 16 (2 rq + y) + 4 g4 + e][column
    // 16 (cq + 4 x) + l%16])
    float *dk_b = a.dkeys + (int64_t)b * a.kv_len * D;
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t row = r0 + 16 * (2 * rq + y) + 4 * g4 + e;
                const float v = acc[y][x][e];
                if (row < r1 && v != 0.0f) atomicAdd(dk_b + row * D + 16 * (cq + 4 * x) + c16, v);
            }
}

template <int D>
hipError_t launch_d(const IndexBwdArgs &a, dim3 grid, hipStream_t st)
{
    const int nw = (a.heads + 15) / 16;
    switch (nw) {
    case 1: hipLaunchKernelGGL((index_bwd_kernel<D, 1>), grid, dim3(64), 0, st, a); break;
    case 2: hipLaunchKernelGGL((index_bwd_kernel<D, 2>), grid, dim3(128), 0, st, a); break;
    case 3: hipLaunchKernelGGL((index_bwd_kernel<D, 3>), grid, dim3(192), 0, st, a); break;
    default: hipLaunchKernelGGL((index_bwd_kernel<D, 4>), grid, dim3(256), 0, st, a); break;
    }
    return hipGetLastError();
}

} // namespace

bool index_bwd_supported(int heads, int dim) { return heads >= 1 && heads <= 64 && (dim == 64 || dim == 128); }

int index_bwd_splits(int batch, int n_q, int n_idx)
{
    const int64_t units = (int64_t)batch * n_q;
    const int max_split = (n_idx + 4 * BR - 1) / (4 * BR); // at least 4 rounds per workgroup
    int64_t want = (768 + units - 1) / units;              // about three workgroups per CU
    if (want > max_split) want = max_split;
    if (want > MAX_SPLIT) want = MAX_SPLIT;
    return want < 1 ? 1 : (int)want;
}

hipError_t launch_index_scores_backward(const IndexBwdArgs &args, hipStream_t st)
{
    if ((int64_t)args.batch * args.n_q == 0) return hipSuccess;
    IndexBwdArgs a = args;
    si::Plan p{};
    int nblk = 0, nchunk = 0;
    // the key-major pass: uniform batches, d = 128 (the prefill chunks it pays for)
    a.si = !a.seq_len && !a.seq_pos0 && a.dim == SI_D && a.heads <= SI_H &&
                   si::plan(a, p, nblk, nchunk, a.batch)
               ? 1
               : 0;
    dim3 grid((unsigned)a.n_split, (unsigned)a.n_q, (unsigned)a.batch);
    hipError_t e = a.dim == 64 ? launch_d<64>(a, grid, st) : launch_d<128>(a, grid, st);
    if (e != hipSuccess || !a.si) return e;
    hipLaunchKernelGGL(index_bwd_si_kernel, dim3((unsigned)nchunk, 1u, (unsigned)a.batch),
                       dim3(512), 0, st, a, p);
    return hipGetLastError();
}

} // namespace lsa
