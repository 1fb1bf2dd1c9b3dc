// attn.hip -- attention restricted to the selected tokens.
//
// (Baidu Cloud article, "3. Sparse Attention Calculator": ordinary softmax attention over the
// top-k tokens only; model card: LSA replaces the dense MLA of LongCat-Flash-Lite, so the cache
// is a latent one whose rows serve as both K (all d_qk columns) and V (the first d_v columns),
// shared by every query head.  Paper summary page, strategy (2): the same index list serves
// several consecutive layers.)
//
// Latent (MLA) kernel.  A workgroup of 4 waves owns one (sequence, query, group of 16 heads) and
// a share of the index list: the list's rounds of 32 selected rows (d_qk bf16 each) are dealt
// to the workgroups of that query in turn.  While round i is computed from LDS, every thread
// holds its share of round i+1's rows in registers (16-byte loads; each row is one contiguous
// run in HBM, and the sink / window runs are contiguous across rows) and writes them to the
// other LDS buffer afterwards.  A first round that lies in the sink and window is loaded from
// the Streaming-Aware layout (model card, SI bullet) while the list itself is still arriving,
// then checked against it.  The workgroup uses under half a CU's LDS, so two of them share a CU
// and hide each other's latencies.  Several layers over one index list (Cross-Layer Indexing)
// run in one grid, z = layer * batch + sequence.
//   logits  S[16 x 32] = Q[16 x d_qk] . K^T   v_mfma_f32_16x16x32_bf16; each wave takes one
//                                              16-row tile over half of d_qk
//   softmax online, fp32, base-2 exponent, per head over the rounds
//   output  O[16 x d_v] += P[16 x 32] . V     v_mfma_f32_16x16x32_bf16, d_v/4 columns per wave;
//                                              V operands by transposing LDS reads
// When the list is split over several workgroups, each writes (max, sum, unnormalised O) and a
// combine kernel merges the splits in a fixed order (no atomics: identical inputs give
// identical bits, which also makes reuse across layers reproducible).
//
// Per-head kernel (any head count, d <= 256, separate K and V): one wave per (query, head);
// lanes score one selected row each, then own output columns and stream the V rows.
#include "device.hpp"
#include "internal.hpp"

namespace lsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

constexpr int AR = 32;          // rows per round
constexpr int NBUF = 2;         // row buffers: round i+1 streams in while round i is computed
constexpr int MLA_MAX_DQK = 576;
constexpr int MLA_MAX_DV = 512;

__device__ __forceinline__ bool row_ok(int32_t id, int64_t kv_len) { return id >= 0 && id < kv_len; }

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// LDS chunk slot of 16-byte chunk c of gathered row r: c ^ sigma(r & 7), sigma(x) = 2(x&3) + x/4.
// sigma is a bijection on 0..7, so the logit reads (8 consecutive rows, one chunk) hit 8
// distinct bank groups; and rows x and x+4 land on opposite halves of each pair of slots, so the
// transposing V reads (4 rows x 2 chunks per 16 lanes) hit 8 distinct bank groups too.
__device__ __forceinline__ int swz(int c, int r)
{
    const int x = r & 7;
    return c ^ ((2 * (x & 3)) | (x >> 2));
}

// gfx950 transposing LDS read: within each group of 16 lanes, lane j receives element j%4 of
// the 8 bytes addressed by lanes j/4 + 4e of the group, e = 0..3.
__device__ __forceinline__ uint2 ds_read_tr16(const uint8_t *lds_byte_ptr)
{
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t *)(__attribute__((address_space(3))) uint8_t *)lds_byte_ptr);
    return bitcast<uint2>(v);
}

// Workgroup barrier inside the latent kernel's round loop.  __syncthreads() carries a release
// fence, which on this target waits for every vector-memory operation still outstanding --
// including the next round's row loads, which are meant to stay in flight across the barrier.
// Here only the LDS writes are completed (lgkmcnt(0)) before the barrier, which is all the
// LDS hand-over between waves needs; the compiler-only fences keep memory accesses from being
// moved across it.
__device__ __forceinline__ void ring_barrier()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0); vmcnt and expcnt: no wait
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// MULTI: several layers in one grid (z = layer * batch + b), each layer's pointers taken from the
// argument arrays; the single-layer form reads them from the plain fields, with no lookup that
// depends on the layer before its first loads can issue.
// PAGED: the cache is a pool of blocks (a.btab).  The row arrays then hold pool rows: a round's
// ids are translated through the block table while the round before is computed (the table
// loads in flight with that round's row loads), and round 0's predicted rows through the table
// before anything else.
template <int DQK, int DV, bool MULTI, bool PAGED>
__global__ __launch_bounds__(256, 2) void mla_attn_kernel(AttnArgs a)
{
    constexpr int ROWB = DQK * 2;          // LDS bytes per gathered row
    constexpr int CPR = ROWB / 16;         // 16-byte chunks per row
    constexpr int KS = DQK / 32;           // K-steps of the logit product
    constexpr int KH = KS / 2;             // K-steps per wave (two waves per 16-row tile)
    constexpr int NTW = DV / 4 / 16;       // 16-column output tiles per wave
    constexpr int CPT = AR * CPR / 256;    // 16-byte chunks per thread per round
    static_assert(KS % 2 == 0 && DV % 64 == 0 && CPR % 8 == 0 && AR == 32, "shape");
    static_assert((AR * CPR) % 256 == 0, "whole chunks per thread");

    // Two distinct row buffers (not one indexed array, so every access names its buffer at
    // compile time).  LDS stays under half a CU's 160 KB: two workgroups share a CU, and one
    // computes while the other's rows stream in.  Chunk c of row r sits at chunk slot swz(c, r).
    __shared__ __attribute__((aligned(16))) uint8_t buf0[AR * ROWB];
    __shared__ __attribute__((aligned(16))) uint8_t buf1[AR * ROWB];
    __shared__ float S2[2][16][AR + 1];    // logit halves (two K halves)
    __shared__ __attribute__((aligned(16))) uint16_t Pm[16][AR + 8];
    __shared__ int32_t rid[NBUF][AR];      // rows of the rounds in the buffers, -1 = skip
    __shared__ int32_t rid_p[AR];          // round 0's row ids as the layout predicts them
    __shared__ bool pred_ok;               // ... and they are the list's
    __shared__ float m_run[16], l_run[16], alpha[16];
    auto slot_buf = [&](auto SLOT) -> uint8_t * {
        if constexpr (decltype(SLOT)::value == 0) return buf0;
        else return buf1;
    };

    const int HG = a.heads / 16;
    const int b = MULTI ? (int)(blockIdx.z % (unsigned)a.batch) : (int)blockIdx.z;
    const int layer = MULTI ? (int)(blockIdx.z / (unsigned)a.batch) : 0;
    const uint16_t *q_l = MULTI ? a.lq[layer] : a.q;
    const uint16_t *k_l = MULTI ? a.lk[layer] : a.k;
    uint16_t *out_l = MULTI ? a.lout[layer] : a.out;
    float *lse_l = MULTI ? a.llse[layer] : a.lse;
    float *ws_l = MULTI ? a.ws + layer * a.ws_layer : a.ws;
    const int t = blockIdx.y / HG;
    const int hg = blockIdx.y % HG;
    const int split = blockIdx.x;
    const int l = lane_id(), w = wave_id();
    const int64_t qrow = (int64_t)b * a.n_q + t;

    // The list's rounds of AR entries are dealt to the splits in turn: split s takes rounds
    // s, s + n_split, ...  With the Streaming-Aware layout in front, every split then starts on
    // sink or window entries, whose rows the layout names without reading the list.
    const int rounds_all = (a.n_idx + AR - 1) / AR;
    const int n_rounds = split < rounds_all ? (rounds_all - split + a.n_split - 1) / a.n_split : 0;
    auto entry = [&](int round) { return (split + round * a.n_split) * AR + (int)(threadIdx.x % AR); };

    const int32_t *idx_row = a.idx + qrow * a.n_idx;
    const int64_t seq_rows = seq_keys(a.seq_len, b, a.kv_len); // valid rows of this sequence
    // Row id (threadIdx.x % AR) of a round: an unconditional load of a clamped, always valid
    // entry (a conditional load would make the compiler wait for it at once), masked at use.
    auto id_load = [&](int round) -> int32_t { return idx_row[min(entry(round), a.n_idx - 1)]; };
    auto id_mask = [&](int round, int32_t raw) -> int32_t {
        return (round < n_rounds && entry(round) < a.n_idx && row_ok(raw, seq_rows)) ? raw : -1;
    };
    // The rows round 0 holds if the list has the layout lsa_topk_select writes: with
    // V = min(rows, position + 1), a query with V <= k lists rows 0 .. V-1 then -1; otherwise
    // entries [0, S) are rows 0 .. S-1 and entries [S, S+W) rows V-W .. V-1.  Round 0 is
    // predicted when all its entries lie there; its rows are then loaded together with the
    // list, q and nothing else in the way, and checked against the list once it is in.
    const int64_t V = valid_len(a.seq_len, a.seq_pos0, b, t, a.kv_len, a.q_pos0);
    const int e0 = split * AR;
    const bool predicted = n_rounds > 0 && (V <= a.n_idx || min(e0 + AR, a.n_idx) <= a.sink + a.window);
    // PAGED: the block-table entry of a (masked) id, by an unconditional in-bounds load, and
    // the pool row it gives (-1: skipped, or its block lies outside the pool)
    const int32_t *btab_b = PAGED ? a.btab + (int64_t)b * a.bps : nullptr;
    auto table_entry = [&](int32_t id) -> int32_t { return btab_b[(id < 0 ? 0 : id) >> a.lbs]; };
    auto pool_row = [&](int32_t id, int32_t tab) -> int32_t {
        return id >= 0 && tab >= 0 && tab < a.n_blocks
                   ? (tab << a.lbs) | (id & ((1 << a.lbs) - 1))
                   : -1;
    };
    int32_t raw0 = 0, raw1 = 0, pid = -1;
    if (threadIdx.x < AR) {
        const int e = e0 + (int)threadIdx.x;
        const int64_t p = e >= a.n_idx ? -1
                          : V <= a.n_idx ? (e < V ? e : -1)
                          : e < a.sink ? e
                          : V - a.window + (e - a.sink);
        pid = p >= 0 && p < seq_rows ? (int32_t)p : -1;
        // the predicted rows' table entries first: they wait for nothing issued after them
        const int32_t tab_p = PAGED ? table_entry(pid) : 0;
        raw0 = id_load(0);
        raw1 = id_load(1);
        if constexpr (PAGED) pid = pool_row(pid, tab_p);
        rid_p[threadIdx.x] = pid;
    }
    // Q fragments: wave w computes row tile (w & 1) over K-half (w >> 1); lane l holds head
    // 16*hg + l%16, d = 32*(KH*(w>>1) + kk) + 8*(l/16) + [0,8)
    const int tile = w & 1, kh = w >> 1;
    bf16x8_t qf[KH];
    {
        const uint16_t *qp = q_l + (qrow * a.heads + 16 * hg + (l & 15)) * DQK + 8 * (l >> 4) + 32 * KH * kh;
#pragma unroll
        for (int kk = 0; kk < KH; ++kk) qf[kk] = bitcast<bf16x8_t>(ld16(qp + 32 * kk));
    }
    if (threadIdx.x < 16) {
        m_run[threadIdx.x] = -INFINITY;
        l_run[threadIdx.x] = 0.0f;
    }
    f32x4_t oacc[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) oacc[nt] = f32x4_t{};
    const uint8_t *kv_b = reinterpret_cast<const uint8_t *>(k_l) +
                          (PAGED ? 0 : (int64_t)b * a.kv_len * a.k_stride * 2); // a pool: rows are pool rows
    const float sl2 = a.scale * kLog2e;

    // A round's rows through registers: thread t loads the 16-byte chunks f = 256*j + t of the
    // round (row f / CPR, chunk f % CPR; consecutive threads read consecutive chunks of a row)
    // while the previous round is computed, and stores them after it.  Skipped rows read row 0
    // instead (always valid); their logits are masked, so they never contribute.
    uint4 stage[CPT];
    auto load_round = [&](const int32_t *ids) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int f = j * 256 + (int)threadIdx.x;
            const int r = f / CPR, c = f % CPR;
            const int32_t id = ids[r];
            stage[j] = ld16(kv_b + (int64_t)(id < 0 ? 0 : id) * a.k_stride * 2 + c * 16);
        }
    };
    auto store_round = [&](uint8_t *dst) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int f = j * 256 + (int)threadIdx.x;
            const int r = f / CPR, c = f % CPR;
            *reinterpret_cast<uint4 *>(dst + r * ROWB + swz(c, r) * 16) = stage[j];
        }
    };

    ring_barrier(); // rid_p is visible; the list and q loads stay in flight
    if (predicted) load_round(rid_p);
    if (threadIdx.x < AR) {
        int32_t id0 = n_rounds > 0 ? id_mask(0, raw0) : -1;
        int32_t id1 = n_rounds > 1 ? id_mask(1, raw1) : -1;
        if constexpr (PAGED) {
            const int32_t tab0 = table_entry(id0), tab1 = table_entry(id1);
            id0 = pool_row(id0, tab0);
            id1 = pool_row(id1, tab1);
        }
        rid[0][threadIdx.x] = id0;
        rid[1][threadIdx.x] = id1;
    }
    if (w == 0) { // a prediction that differs from the list in any entry is discarded
        const uint64_t miss = __ballot(threadIdx.x < AR && pid != rid[0][threadIdx.x]);
        if (l == 0) pred_ok = predicted && miss == 0u;
    }
    __syncthreads();
    if (n_rounds > 0) {
        if (!pred_ok) load_round(rid[0]);
        store_round(buf0);
    }
    // Q, the ids and round 0 are in: the loop starts with nothing outstanding, so the waits the
    // compiler places inside it count only the loads the loop itself issues
    __builtin_amdgcn_s_waitcnt(0);
    // rounds in pairs: the ring slot is a compile-time constant in each copy of the body
    for (int i0 = 0; i0 < n_rounds; i0 += NBUF) static_for<0, NBUF>([&](auto SLOT) {
        constexpr int S = decltype(SLOT)::value;
        constexpr int O = S ^ 1; // the other slot
        const int i = i0 + S;
        if (i >= n_rounds) return;
        ring_barrier(); // round i is in buf[S]; round i-1 is fully consumed
        // the rows of round i+1 (into registers) and the ids of round i+2 are loaded while
        // round i is computed.  Unconditionally: after the last round rid[O] is all -1, so the
        // surplus loads read row 0 into a buffer no one reads (a conditional load would make
        // the compiler wait for every load at the merge that follows it).
        const int32_t next_raw = id_load(i + 2); // first: waiting for it then waits for no row
        load_round(rid[O]);
        int32_t next_id = -1, next_tab = 0; // PAGED: round i + 2's ids and table entries
        const uint8_t *cb = slot_buf(SLOT);
        // logits, half of d per wave: S2[kh][h][r] for rows 16*tile .. 16*tile + 15
        {
            f32x4_t acc = f32x4_t{};
            const int r = 16 * tile + (l & 15);
            const uint8_t *kr = cb + r * ROWB;
#pragma unroll
            for (int kk = 0; kk < KH; ++kk) {
                const int c = 4 * (KH * kh + kk) + (l >> 4);
                acc = mfma_16x16x32(qf[kk], bitcast<bf16x8_t>(ld16(kr + 16 * swz(c, r))), acc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) S2[kh][4 * (l >> 4) + e][r] = acc[e];
        }
        ring_barrier();
        // online softmax: 16 threads per head, 2 rows each
        {
            const int h = threadIdx.x >> 4, part = threadIdx.x & 15;
            float sv[2], mx = -INFINITY;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int r = 2 * part + e;
                const float x = (S2[0][h][r] + S2[1][h][r]) * sl2;
                sv[e] = rid[S][r] >= 0 ? x : -INFINITY;
                mx = fmaxf(mx, sv[e]);
            }
#pragma unroll
            for (int off = 8; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 16));
            const float m_old = m_run[h];
            const float m_new = fmaxf(m_old, mx);
            float sum = 0.0f;
            uint32_t pb[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float p = (m_new == -INFINITY || sv[e] == -INFINITY) ? 0.0f : exp2f(sv[e] - m_new);
                pb[e] = f32_to_bf16_bits(p);
                sum += bf16_bits_to_f32(pb[e]); // normalise by what the product actually uses
            }
            *reinterpret_cast<uint32_t *>(&Pm[h][2 * part]) = pb[0] | (pb[1] << 16);
#pragma unroll
            for (int off = 8; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 16);
            ring_barrier(); // every reader of m_run and of rid[S] is done
            if (part == 0) {
                const float al = (m_old == -INFINITY) ? 0.0f : exp2f(m_old - m_new);
                alpha[h] = al;
                l_run[h] = l_run[h] * al + sum;
                m_run[h] = m_new;
            }
            if (threadIdx.x < AR) {
                if constexpr (PAGED) { // translated at the end of the round
                    next_id = id_mask(i + 2, next_raw);
                    next_tab = table_entry(next_id);
                } else {
                    rid[S][threadIdx.x] = id_mask(i + 2, next_raw);
                }
            }
        }
        ring_barrier();
        // O = O * alpha + P . V ; wave w owns columns [w*DV/4, (w+1)*DV/4).  K = the 32 rows:
        // lane group q = l/16 takes rows 8q + [0,8) as two transposing reads of 4 rows.
        {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float al = alpha[4 * (l >> 4) + e];
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) oacc[nt][e] *= al;
            }
            const int q = l >> 4, j = l & 15;   // lane group, lane within group
            const int re = j >> 2, c4 = j & 3;  // source lane role: row e, 4-column segment
            const bf16x8_t pf = bitcast<bf16x8_t>(ld16(reinterpret_cast<const uint8_t *>(&Pm[l & 15][8 * q])));
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                const int col = w * (DV / 4) + 16 * nt + 4 * c4; // this lane's source segment
                uint2 half[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int r = 8 * q + 4 * hh + re;
                    half[hh] = ds_read_tr16(cb + r * ROWB + swz(col >> 3, r) * 16 + (col & 7) * 2);
                }
                const bf16x8_t vf = bitcast<bf16x8_t>(make_uint4(half[0].x, half[0].y, half[1].x, half[1].y));
                oacc[nt] = mfma_16x16x32(pf, vf, oacc[nt]);
            }
        }
        if constexpr (PAGED) // the table entries arrive with the round's rows, awaited below
            if (threadIdx.x < AR) rid[S][threadIdx.x] = pool_row(next_id, next_tab);
        store_round(slot_buf(std::integral_constant<int, O>{}));
    });
    __syncthreads(); // m_run / l_run final

    // epilogue: lane holds O[head 4*(l/16)+e][col w*DV/4 + 16*nt + l%16]
    if (a.n_split == 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int h = 4 * (l >> 4) + e;
            const float lr = l_run[h];
            const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
            uint16_t *op = out_l + (qrow * a.heads + 16 * hg + h) * DV;
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                const int col = w * (DV / 4) + 16 * nt + (l & 15);
                op[col] = (uint16_t)f32_to_bf16_bits(oacc[nt][e] * inv);
            }
        }
        if (lse_l && threadIdx.x < 16) {
            const float lr = l_run[threadIdx.x];
            lse_l[qrow * a.heads + 16 * hg + threadIdx.x] =
                lr > 0.0f ? (m_run[threadIdx.x] + log2f(lr)) * kLn2 : -INFINITY;
        }
    } else {
        // partial block: [DV] O values, then (m, l), per (query, head, split)
        const int64_t stride = DV + 2;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int h = 4 * (l >> 4) + e;
            float *pp = ws_l + ((qrow * a.heads + 16 * hg + h) * a.n_split + split) * stride;
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) pp[w * (DV / 4) + 16 * nt + (l & 15)] = oacc[nt][e];
        }
        if (threadIdx.x < 16) {
            float *pp = ws_l + ((qrow * a.heads + 16 * hg + threadIdx.x) * a.n_split + split) * stride;
            pp[DV] = m_run[threadIdx.x];
            pp[DV + 1] = l_run[threadIdx.x];
        }
    }
}

// Merge the splits of one (query, head): fixed order over splits.
constexpr int MAX_SPLIT = 32;

template <bool MULTI>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a)
{
    __shared__ float wsp[MAX_SPLIT];
    __shared__ float inv_l;
    // the split form only runs for small grids (fewer than 512 units of 16 heads): 32 bits hold
    // every index here
    const unsigned per_layer = (unsigned)a.batch * a.n_q * a.heads;
    const int layer = MULTI ? (int)(blockIdx.x / per_layer) : 0;
    const int64_t qh = MULTI ? blockIdx.x % per_layer : blockIdx.x; // (b * n_q + t) * heads + h
    const int64_t stride = a.d_v + 2;
    const float *base = (MULTI ? a.ws + layer * a.ws_layer : a.ws) + qh * a.n_split * stride;
    float *lse_l = MULTI ? a.llse[layer] : a.lse;
    uint16_t *out_l = MULTI ? a.lout[layer] : a.out;
    if (threadIdx.x < kWave) {
        const int s = threadIdx.x;
        const float m = s < a.n_split ? base[s * stride + a.d_v] : -INFINITY;
        const float lsum = s < a.n_split ? base[s * stride + a.d_v + 1] : 0.0f;
        const float M = wave_max(m);
        const float e = (m == -INFINITY) ? 0.0f : exp2f(m - M);
        const float L = wave_sum(e * lsum);
        if (s < MAX_SPLIT) wsp[s] = e;
        if (s == 0) {
            inv_l = L > 0.0f ? 1.0f / L : 0.0f;
            if (lse_l) lse_l[qh] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
        }
    }
    __syncthreads();
    const float il = inv_l;
    for (int c = threadIdx.x; c < a.d_v; c += blockDim.x) {
        float o = 0.0f;
#pragma unroll 8
        for (int s = 0; s < a.n_split; ++s) o = fmaf(base[s * stride + c], wsp[s], o);
        out_l[qh * a.d_v + c] = (uint16_t)f32_to_bf16_bits(o * il);
    }
}

// Per-head kernel: one wave per (query, head).
constexpr int MHA_CHUNK = 256;
constexpr int MHA_MAXD = 256;

__global__ __launch_bounds__(256) void mha_attn_kernel(AttnArgs a)
{
    __shared__ float qs[4][MHA_MAXD];
    __shared__ float ps[4][MHA_CHUNK];
    __shared__ int32_t ids[4][MHA_CHUNK];
    const int l = lane_id(), w = wave_id();
    const int64_t total = (int64_t)a.batch * a.n_q * a.heads;
    const int64_t unit_raw = (int64_t)blockIdx.x * 4 + w; // (b * n_q + t) * heads + h
    const bool live = unit_raw < total;                   // idle waves still reach the barriers
    const int64_t unit = live ? unit_raw : total - 1;
    const int64_t qrow = unit / a.heads;
    const int b = (int)(qrow / a.n_q);
    const uint16_t *qp = a.q + unit * a.d_qk;
    for (int d = l; d < a.d_qk; d += kWave) qs[w][d] = bf16_bits_to_f32(qp[d]);
    const uint16_t *kb = a.k + (int64_t)b * a.kv_len * a.k_stride;
    const uint16_t *vb = a.v + (int64_t)b * a.kv_len * a.v_stride;
    const int64_t seq_rows = seq_keys(a.seq_len, b, a.kv_len);
    const int32_t *idx_row = a.idx + qrow * a.n_idx;
    const float sl2 = a.scale * kLog2e;
    constexpr int VPL = MHA_MAXD / kWave; // output columns per lane (at most)
    float acc[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) acc[i] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;
    __syncthreads();
    for (int c0 = 0; c0 < a.n_idx; c0 += MHA_CHUNK) {
        const int cn = min(MHA_CHUNK, a.n_idx - c0);
        float cmax = -INFINITY;
        for (int j = l; j < cn; j += kWave) {
            const int32_t id = idx_row[c0 + j];
            float lg = -INFINITY;
            if (row_ok(id, seq_rows)) {
                const uint16_t *kr = kb + (int64_t)id * a.k_stride;
                float dot = 0.0f;
                for (int d = 0; d < a.d_qk; d += 8) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(kr + d);
                    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        dot = fmaf(qs[w][d + 2 * e], __uint_as_float(u[e] << 16), dot);
                        dot = fmaf(qs[w][d + 2 * e + 1], __uint_as_float(u[e] & 0xffff0000u), dot);
                    }
                }
                lg = dot * sl2;
            }
            ps[w][j] = lg;
            ids[w][j] = row_ok(id, seq_rows) ? id : -1;
            cmax = fmaxf(cmax, lg);
        }
        cmax = wave_max(cmax);
        __syncthreads();
        const float m_new = fmaxf(m_run, cmax);
        const float al = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - m_new);
        float csum = 0.0f;
        for (int j = l; j < cn; j += kWave) {
            const float p = (m_new == -INFINITY || ps[w][j] == -INFINITY) ? 0.0f : exp2f(ps[w][j] - m_new);
            ps[w][j] = p;
            csum += p;
        }
        csum = wave_sum(csum);
        __syncthreads();
        l_run = l_run * al + csum;
        m_run = m_new;
#pragma unroll
        for (int i = 0; i < VPL; ++i) acc[i] *= al;
        for (int j = 0; j < cn; ++j) {
            const int32_t id = ids[w][j];
            if (id < 0) continue;
            const float p = ps[w][j];
            const uint16_t *vr = vb + (int64_t)id * a.v_stride;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int c = l + kWave * i;
                if (c < a.d_v) acc[i] = fmaf(p, bf16_bits_to_f32(vr[c]), acc[i]);
            }
        }
        __syncthreads();
    }
    if (!live) return;
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    uint16_t *op = a.out + unit * a.d_v;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int c = l + kWave * i;
        if (c < a.d_v) op[c] = (uint16_t)f32_to_bf16_bits(acc[i] * inv);
    }
    if (a.lse && l == 0) a.lse[unit] = l_run > 0.0f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
}

} // namespace

bool attn_supported(int heads, int d_qk, int d_v, int latent)
{
    if (latent) return heads % 16 == 0 && d_qk == MLA_MAX_DQK && d_v == MLA_MAX_DV;
    return heads >= 1 && d_qk % 8 == 0 && d_v % 8 == 0 && d_qk <= MHA_MAXD && d_v <= MHA_MAXD;
}

int attn_splits(int batch, int n_q, int heads, int n_idx, int latent)
{
    if (!latent) return 1;
    const int64_t units = (int64_t)batch * n_q * (heads / 16);
    const int max_split = (n_idx + AR - 1) / AR;
    int64_t want = (512 + units - 1) / units; // two workgroups per CU
    if (want > max_split) want = max_split;
    if (want > MAX_SPLIT) want = MAX_SPLIT;
    return want < 1 ? 1 : (int)want;
}

size_t attn_workspace_bytes(int batch, int n_q, int heads, int d_v, int n_idx, int latent)
{
    const int s = attn_splits(batch, n_q, heads, n_idx, latent);
    if (s <= 1) return 0;
    return (size_t)batch * n_q * heads * s * (d_v + 2) * sizeof(float);
}

hipError_t launch_sparse_attn(const AttnArgs &a, hipStream_t st)
{
    const int64_t rows = (int64_t)a.batch * a.n_q;
    if (rows == 0) return hipSuccess;
    if (a.layers < 1 || a.layers > kMaxAttnLayers) return hipErrorInvalidValue;
    if (a.latent) {
        // every layer's gathers in one launch, then every layer's splits merged in one launch
        dim3 grid((unsigned)a.n_split, (unsigned)(a.n_q * (a.heads / 16)),
                  (unsigned)(a.batch * a.layers));
        const dim3 cgrid((unsigned)(rows * a.heads * a.layers));
        const bool paged = a.btab != nullptr;
        if (a.layers == 1) {
            if (paged)
                hipLaunchKernelGGL((mla_attn_kernel<MLA_MAX_DQK, MLA_MAX_DV, false, true>), grid, dim3(256), 0, st, a);
            else
                hipLaunchKernelGGL((mla_attn_kernel<MLA_MAX_DQK, MLA_MAX_DV, false, false>), grid, dim3(256), 0, st, a);
            if (a.n_split > 1) hipLaunchKernelGGL(attn_combine_kernel<false>, cgrid, dim3(256), 0, st, a);
        } else {
            if (paged)
                hipLaunchKernelGGL((mla_attn_kernel<MLA_MAX_DQK, MLA_MAX_DV, true, true>), grid, dim3(256), 0, st, a);
            else
                hipLaunchKernelGGL((mla_attn_kernel<MLA_MAX_DQK, MLA_MAX_DV, true, false>), grid, dim3(256), 0, st, a);
            if (a.n_split > 1) hipLaunchKernelGGL(attn_combine_kernel<true>, cgrid, dim3(256), 0, st, a);
        }
    } else {
        if (a.btab) return hipErrorInvalidValue; // the per-head cache is dense
        const int64_t units = rows * a.heads;
        for (int layer = 0; layer < a.layers; ++layer) {
            AttnArgs al = a;
            al.q = a.lq[layer];
            al.k = a.lk[layer];
            al.v = a.lv[layer];
            al.out = a.lout[layer];
            al.lse = a.llse[layer];
            hipLaunchKernelGGL(mha_attn_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, st, al);
        }
    }
    return hipGetLastError();
}

} // namespace lsa
