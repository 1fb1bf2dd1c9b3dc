"""Pins of the CPU oracle to things other than itself (CPU only).

Each test checks the oracle against a library routine on a special case, a closed form, an
invariant of the mathematics or a fixture with a stated derivation, chosen so that a plausible
slip (dropped ReLU or weight, wrong sign, transposed or shifted index, off-by-one causal bound,
wrong tie order, wrong summation order) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import ref
from token_selection_indexer_amd import inputs
from token_selection_indexer_amd.configs import TINY_PREFILL_4K, shrink
from tests.util import bits, u8

GOLD = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    return bits(torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16))


def bf16_vals(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------------------------------ formats
def test_e4m3fn_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    lib_vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    ours = np.array([ref.e4m3fn_to_double(c) for c in codes])
    nan = np.isnan(lib_vals)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(lib_vals[~nan], ours[~nan])
    assert np.array_equal(np.signbit(lib_vals[~nan]), np.signbit(ours[~nan]))


def test_e4m3fn_spec_landmarks():
    for line in open(os.path.join(GOLD, "e4m3fn_landmarks.txt")):
        if line.startswith("#") or not line.strip():
            continue
        code, val = line.split()
        got = ref.e4m3fn_to_double(int(code, 16))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))


def test_bf16_decode_matches_torch():
    b = RNG.integers(0, 1 << 16, size=4000, dtype=np.uint16)
    b = b[(b & 0x7F80) != 0x7F80]  # finite only
    lib_vals = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double().numpy()
    ours = np.array([ref.bf16_to_double(x) for x in b])
    assert np.array_equal(lib_vals, ours)


def test_bf16_rne_matches_torch_including_ties():
    x = RNG.standard_normal(3000).astype(np.float32) * np.float32(100.0)
    u = x.view(np.uint32)
    ties = ((u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)  # exact halfway
    allx = np.concatenate([x, ties, np.float32([0.0, -0.0, 1e-40, -3e38])])
    lib_bits = bits(torch.from_numpy(allx).to(torch.bfloat16))
    ours = np.array([ref.f32_to_bf16_rne(v) for v in allx], np.uint16)
    assert np.array_equal(lib_bits, ours)


# ------------------------------------------------------------------------------ a1 scores
def _rand_q_k(T, H, d, L, seed=0):
    r = np.random.default_rng(seed)
    q = bf16_bits(r.standard_normal((T, H, d)))
    k = bf16_bits(r.standard_normal((L, d)))
    w = r.standard_normal((T, H)).astype(np.float32)
    return q, k, w


def test_scores_single_head_unit_weight_is_relu_matmul():
    T, d, L = 7, 64, 50
    q, k, _ = _rand_q_k(T, 1, d, L)
    w = np.ones((T, 1), np.float32)
    pos = np.full(T, L - 1)
    I, A, E = ref.index_scores(q, w, k, None, pos)
    expect = np.maximum(bf16_vals(q[:, 0]) @ bf16_vals(k).T, 0.0)
    np.testing.assert_allclose(I, expect, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(A, expect, rtol=1e-12, atol=1e-12)  # w > 0: A == I
    assert np.all(E >= A - 1e-12)


def test_scores_causal_bound():
    T, H, d, L = 6, 4, 64, 20
    q, k, w = _rand_q_k(T, H, d, L)
    pos = np.array([0, 3, 10, 18, 19, 40])
    I, _, _ = ref.index_scores(q, w, k, None, pos)
    for t, p in enumerate(pos):
        V = min(L, p + 1)
        assert np.all(np.isfinite(I[t, :V])), t
        assert np.all(np.isneginf(I[t, V:])), t


def test_scores_heads_add_up_and_weights_index_per_query():
    """I(q, w) == sum over heads of single-head scores with w[t,h], each of which is pinned to
    relu(matmul) above; catches a transposed w or a dropped head."""
    T, H, d, L = 5, 4, 32, 40
    q, k, w = _rand_q_k(T, H, d, L, seed=3)
    pos = np.full(T, L)
    I, _, _ = ref.index_scores(q, w, k, None, pos)
    qv, kv = bf16_vals(q), bf16_vals(k)
    total = np.zeros((T, L))
    for h in range(H):
        total += w[:, h:h + 1].astype(np.float64) * np.maximum(qv[:, h] @ kv.T, 0.0)
    np.testing.assert_allclose(I, total, rtol=1e-11, atol=1e-11)


def test_scores_all_positive_dots_reduce_to_gemv():
    """If every q[t,h].k[s] > 0 the ReLU is inactive and I = (sum_h w_h q_h) . k."""
    T, H, d, L = 3, 8, 16, 30
    r = np.random.default_rng(7)
    q = bf16_bits(np.abs(r.standard_normal((T, H, d))) + 0.1)
    k = bf16_bits(np.abs(r.standard_normal((L, d))) + 0.1)
    w = r.standard_normal((T, H)).astype(np.float32)
    I, _, _ = ref.index_scores(q, w, k, None, np.full(T, L))
    qv, kv = bf16_vals(q), bf16_vals(k)
    expect = np.einsum("th,thd->td", w.astype(np.float64), qv) @ kv.T
    np.testing.assert_allclose(I, expect, rtol=1e-11)


def test_scores_one_hot_query_closed_form():
    """q[h] = e_i (one-hot) gives ReLU(k[s][i]) per head."""
    H, d, L = 3, 16, 25
    r = np.random.default_rng(9)
    k = bf16_bits(r.standard_normal((L, d)))
    qf = np.zeros((1, H, d))
    qf[0, 0, 2] = 1.0
    qf[0, 1, 5] = 1.0
    qf[0, 2, 2] = -1.0
    w = np.array([[0.5, -2.0, 1.0]], np.float32)
    I, _, _ = ref.index_scores(bf16_bits(qf), w, k, None, np.array([L]))
    kv = bf16_vals(k)
    expect = 0.5 * np.maximum(kv[:, 2], 0) - 2.0 * np.maximum(kv[:, 5], 0) + np.maximum(-kv[:, 2], 0)
    np.testing.assert_allclose(I[0], expect, rtol=1e-15, atol=0)


def test_scores_fp8_keys_are_scaled_dequantised_keys():
    """e4m3 keys: I(q, scale*kq) must equal the bf16-free computation on torch-dequantised keys
    (library decode) times the scale, i.e. homogeneity in the key scale."""
    T, H, d, L = 4, 4, 64, 33
    r = np.random.default_rng(11)
    q = bf16_bits(r.standard_normal((T, H, d)))
    w = r.standard_normal((T, H)).astype(np.float32)
    kf = torch.from_numpy(r.standard_normal((L, d)).astype(np.float32))
    codes, scale = inputs.quantize_e4m3(kf)
    I, _, _ = ref.index_scores(q, w, u8(codes), scale.numpy(), np.full(T, L))
    deq = codes.view(torch.float8_e4m3fn).double().numpy() * scale.double().numpy()[:, None]
    qv = bf16_vals(q)
    expect = np.zeros((T, L))
    for h in range(H):
        expect += w[:, h:h + 1].astype(np.float64) * np.maximum(qv[:, h] @ deq.T, 0.0)
    np.testing.assert_allclose(I, expect, rtol=1e-11, atol=1e-12)
    # homogeneity: doubling every scale doubles every score exactly
    I2, _, _ = ref.index_scores(q, w, u8(codes), 2 * scale.numpy(), np.full(T, L))
    assert np.array_equal(I2, 2 * I)


def test_scores_weight_homogeneity_and_head_permutation():
    T, H, d, L = 3, 6, 32, 21
    q, k, w = _rand_q_k(T, H, d, L, seed=5)
    pos = np.full(T, L)
    I, _, _ = ref.index_scores(q, w, k, None, pos)
    I3, _, _ = ref.index_scores(q, (w * np.float32(4.0)), k, None, pos)
    np.testing.assert_allclose(I3, 4 * I, rtol=1e-13, atol=1e-13)
    perm = np.random.default_rng(0).permutation(H)
    Ip, _, _ = ref.index_scores(q[:, perm], w[:, perm], k, None, pos)
    np.testing.assert_allclose(Ip, I, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------------------ fp8 queries
def _e4m3_torch(x: np.ndarray) -> np.ndarray:
    """Library routine: torch's binary32 -> float8_e4m3fn conversion (after a clamp to the
    format's range, so the conversion saturates)."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_f32_to_e4m3fn_matches_torch_including_ties_and_saturation():
    codes = np.arange(0x7F, dtype=np.uint8)  # non-negative finite codes
    vals = np.array([ref.e4m3fn_to_double(c) for c in codes])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)  # exact halfway points (ties)
    r = np.random.default_rng(3)
    rand = (r.standard_normal(4000) * 60).astype(np.float32)
    edge = np.float32([0.0, -0.0, 1e-30, -1e-30, 2.0 ** -10, 2.0 ** -9, 447.9, 448.0, 449.0,
                       463.9, 464.0, 1e6, -1e6])
    x = np.concatenate([vals.astype(np.float32), -vals.astype(np.float32), mids, -mids, rand, edge])
    ours = np.array([ref.f32_to_e4m3fn_sat(v) for v in x], np.uint8)
    lib = _e4m3_torch(x)
    # +-0: both give a zero of the input's sign
    assert np.array_equal(ours, lib)


def test_quantize_rows_scale_codes_and_error_bound():
    r = np.random.default_rng(4)
    x = bf16_bits(r.standard_normal((50, 128)) * np.exp(r.uniform(-6, 6, (50, 1))))
    x[7] = 0  # an all-zero row: scale 1, codes 0
    codes, scale = ref.quantize_rows(x)
    xv = bf16_vals(x)
    amax = np.abs(xv).max(axis=1)
    want_scale = np.where(amax > 0, (amax.astype(np.float32) / np.float32(448.0)), 1.0)
    assert np.array_equal(scale, want_scale.astype(np.float32))
    assert not codes[7].any() and scale[7] == 1.0
    # codes are the library conversion of x / scale (binary32 division)
    y = (xv.astype(np.float32) / scale[:, None]).astype(np.float32)
    assert np.array_equal(codes, _e4m3_torch(y))
    # every row's largest magnitude maps to +-448; dequantised values within half a step
    deq = np.array([[ref.e4m3fn_to_double(c) for c in row] for row in codes]) * scale[:, None]
    top = np.abs(np.array([[ref.e4m3fn_to_double(c) for c in row] for row in codes])).max(axis=1)
    assert np.all(top[amax > 0] == 448.0)
    rel = np.abs(deq - xv) / np.maximum(np.abs(xv), 2.0 ** -6 * scale[:, None])
    assert rel.max() <= 2.0 ** -4 + 1e-12


def test_quantize_rows_power_of_two_scaling():
    """Scaling a row by 2^m scales its scale by 2^m and keeps its codes."""
    r = np.random.default_rng(5)
    xv = r.standard_normal((20, 64)).astype(np.float32)
    c1, s1 = ref.quantize_rows(bf16_bits(xv))
    c2, s2 = ref.quantize_rows(bf16_bits(xv * np.float32(2.0 ** 5)))
    assert np.array_equal(c1, c2)
    assert np.array_equal(s2, s1 * np.float32(32.0))


def test_scores_q8_equal_scores_of_the_dequantised_query():
    """With the scales folded into exactly representable values, the quantised-query scores are
    the ordinary scores of the dequantised query: unit scales give the scores of q = e4m3(code)
    (every e4m3 value is a bf16 value); power-of-two scales move into the head weights."""
    r = np.random.default_rng(6)
    T, H, d, L = 3, 4, 64, 200
    q8 = r.integers(0, 0x7F, size=(T, H, d), dtype=np.uint8) | (r.integers(0, 2, (T, H, d)) << 7).astype(np.uint8)
    w = r.standard_normal((T, H)).astype(np.float32)
    keys = bf16_bits(r.standard_normal((L, d)))
    pos = np.array([L - 1, 50, 120])
    qv = np.array([[[ref.e4m3fn_to_double(c) for c in hd] for hd in row] for row in q8])
    qb = bf16_bits(qv)
    assert np.array_equal(bf16_vals(qb), qv)  # exactly representable
    ones = np.ones((T, H), np.float32)
    I8, A8, E8 = ref.index_scores_q8(q8, ones, w, keys, None, pos)
    Ib, Ab, Eb = ref.index_scores(qb, w, keys, None, pos)
    assert np.array_equal(I8, Ib) and np.array_equal(A8, Ab) and np.array_equal(E8, Eb)
    p2 = (2.0 ** r.integers(-8, 8, size=(T, H))).astype(np.float32)
    I8s, _, _ = ref.index_scores_q8(q8, p2, w, keys, None, pos)
    Ibs, _, _ = ref.index_scores(qb, w * p2, keys, None, pos)
    assert np.array_equal(I8s, Ibs)
    # fp8 keys as well (their own per-token scales)
    k8 = r.integers(0, 0x7F, size=(L, d), dtype=np.uint8)
    ks = (r.uniform(0.5, 2, L)).astype(np.float32)
    I8k, _, _ = ref.index_scores_q8(q8, ones, w, k8, ks, pos)
    Ibk, _, _ = ref.index_scores(qb, w, k8, ks, pos)
    assert np.array_equal(I8k, Ibk)


# ------------------------------------------------------------------------------ a2 select
def _lexsort_top(scores_row, ids, need):
    """Library sort: order by (score desc, id asc), keep need, return ascending ids."""
    o = np.lexsort((ids, -scores_row.astype(np.float64)))
    return np.sort(ids[o[:need]])


def test_select_plain_topk_matches_argpartition():
    T, L, k = 6, 300, 40
    s = np.random.default_rng(1).standard_normal((T, L)).astype(np.float32)
    idx = ref.select(s, np.full(T, L), k, 0, 0)
    for t in range(T):
        expect = np.sort(np.argpartition(-s[t], k)[:k])
        assert np.array_equal(idx[t], expect)
    tk = torch.topk(torch.from_numpy(s), k, dim=-1).indices.sort(dim=-1).values.numpy()
    assert np.array_equal(idx, tk)


@pytest.mark.parametrize("ties", ["zeros", "coarse", "const", "none", "inf"])
def test_select_sink_window_dynamic_against_lexsort(ties):
    T, L, k, S, W = 5, 700, 96, 8, 40
    s = inputs.synthetic_scores(T, L, seed=3, ties=ties).numpy()
    V = np.array([700, 500, 97, 96, 20])
    idx = ref.select(s, V, k, S, W)
    for t in range(T):
        Vt = V[t]
        row = idx[t]
        if Vt <= k:
            assert np.array_equal(row[:Vt], np.arange(Vt))
            assert np.all(row[Vt:] == -1)
            continue
        assert np.array_equal(row[:S], np.arange(S))
        assert np.array_equal(row[S:S + W], np.arange(Vt - W, Vt))
        mid = np.arange(S, Vt - W)
        assert np.array_equal(row[S + W:], _lexsort_top(s[t, S:Vt - W], mid, k - S - W))


def test_select_invariants_on_random_rows():
    T, L, k, S, W = 20, 1000, 128, 16, 48
    s = inputs.synthetic_scores(T, L, seed=4, ties="zeros").numpy()
    V = np.random.default_rng(2).integers(1, L + 1, size=T)
    idx = ref.select(s, V, k, S, W)
    for t in range(T):
        sel = idx[t][idx[t] >= 0]
        assert len(sel) == min(k, V[t])
        assert len(set(sel.tolist())) == len(sel)
        assert np.all(sel < V[t])
        if V[t] > k:
            assert set(range(S)) <= set(sel.tolist())
            assert set(range(V[t] - W, V[t])) <= set(sel.tolist())
            dyn = idx[t][S + W:]
            assert np.all(np.diff(dyn) > 0)
            rest = np.setdiff1d(np.arange(S, V[t] - W), dyn)
            assert s[t, rest].max() <= s[t, dyn].min()


def test_select_candidate_mode_equals_flat_when_all_tokens_are_candidates():
    T, L, k, S, W = 4, 600, 64, 8, 24
    s = inputs.synthetic_scores(T, L, seed=6, ties="coarse").numpy()
    V = np.array([600, 300, 64, 65])
    flat = ref.select(s, V, k, S, W)
    ids = np.tile(np.arange(L, dtype=np.int32), (T, 1))
    ids[:, 50:60] = -1  # holes are skipped ...
    s2 = s.copy()
    s2[:, 50:60] = np.float32(1e30)  # ... whatever their score
    ids[:, 50:60] = -1
    cand = ref.select(s2, V, k, S, W, cand_ids=ids)
    # remove the holes from the flat problem too
    s3 = s.copy()
    s3[:, 50:60] = -np.inf
    flat3 = ref.select(s3, V, k, S, W)
    assert np.array_equal(cand, flat3)
    assert flat.shape == cand.shape


def test_select_candidate_mode_fewer_candidates_pads():
    k, S, W = 32, 4, 8
    ids = np.full((1, 10), -1, np.int32)
    ids[0, :5] = [20, 21, 40, 41, 90]
    sc = np.arange(10, dtype=np.float32)[None]
    idx = ref.select(sc, np.array([200]), k, S, W, cand_ids=ids)
    assert np.array_equal(idx[0, :S], np.arange(S))
    assert np.array_equal(idx[0, S:S + W], np.arange(192, 200))
    assert np.array_equal(idx[0, S + W:S + W + 5], [20, 21, 40, 41, 90])
    assert np.all(idx[0, S + W + 5:] == -1)


# ------------------------------------------------------------------------------ a3 pages
def test_page_key_tree_sum_fixtures():
    for line in open(os.path.join(GOLD, "page_tree_sum.txt")):
        if line.startswith("#") or not line.strip():
            continue
        P, n, vals, expect, _ = [x.strip() for x in line.split("|")]
        P, n = int(P), int(n)
        v = np.array([float(x) for x in vals.split()], np.float32)[:, None]
        assert len(v) == n
        kb = bf16_bits(v)
        assert np.array_equal(bf16_vals(kb)[:, 0], v[:, 0])  # fixture values are bf16-exact
        pk = ref.page_keys(kb, None, P)
        assert bf16_vals(pk)[0, 0] == float(expect), line


def test_page_keys_constant_page_and_single_token_pages():
    r = np.random.default_rng(3)
    row = bf16_bits(r.standard_normal((1, 32)))
    pk = ref.page_keys(np.repeat(row, 64, axis=0), None, 64)
    assert np.array_equal(pk[0], row[0])
    k = bf16_bits(r.standard_normal((37, 32)))
    assert np.array_equal(ref.page_keys(k, None, 1), k)


def test_page_keys_near_exact_mean_fp8_and_partial_page():
    L, d, P = 64 * 5 + 17, 128, 64
    kf = torch.from_numpy(np.random.default_rng(8).standard_normal((L, d)).astype(np.float32))
    codes, scale = inputs.quantize_e4m3(kf)
    pk = ref.page_keys(u8(codes), scale.numpy(), P)
    deq = codes.view(torch.float8_e4m3fn).double().numpy() * scale.double().numpy()[:, None]
    n_pages = (L + P - 1) // P
    assert pk.shape == (n_pages, d)
    for p in range(n_pages):
        exact = deq[p * P:(p + 1) * P].mean(axis=0)  # present tokens only
        got = bf16_vals(pk[p])
        # bf16 rounding (2^-9 relative) plus the fp32 sum's rounding
        bound = np.abs(exact) * 2.0 ** -8 + 64 * 2.0 ** -24 * np.abs(deq[p * P:(p + 1) * P]).mean(0)
        assert np.all(np.abs(got - exact) <= bound + 1e-30), p
        expect_rne = bf16_bits(exact.astype(np.float32))
        assert np.mean(expect_rne == pk[p]) > 0.95


# ------------------------------------------------------------------------------ a4/a5 HI
def _hi_problem(L=1024, d=32, H=4, seed=0, fp8=False):
    r = np.random.default_rng(seed)
    q = bf16_bits(r.standard_normal((1, H, d)))
    w = (r.standard_normal((1, H)) * 0.5).astype(np.float32)
    kf = r.standard_normal((L, d)).astype(np.float32)
    if fp8:
        c, sc = inputs.quantize_e4m3(torch.from_numpy(kf))
        return q, w, u8(c), sc.numpy()
    return q, w, bf16_bits(kf), None


@pytest.mark.parametrize("fp8", [False, True])
def test_hi_with_all_pages_recalled_equals_flat(fp8):
    L, P, k, S, W = 1024, 16, 96, 8, 24
    q, w, keys, scale = _hi_problem(L=L, fp8=fp8)
    pos = np.array([L - 1])
    V = np.array([L])
    M = L // P  # M * P >= L
    pk = ref.page_keys(keys, scale, P)
    hi = ref.page_recall(q, w, pk, keys, scale, pos, k, S, W, P, M)
    I, _, _ = ref.index_scores(q, w, keys, scale, pos)
    flat = ref.select(I.astype(np.float32), V, k, S, W)
    got = ref.select(hi["cand_scores"].astype(np.float32), V, k, S, W, cand_ids=hi["cand_ids"])
    assert np.array_equal(got, flat)
    # every page recalled: the candidates are exactly the middle region [S, V-W), in order
    cid = hi["cand_ids"][0]
    assert np.array_equal(cid[cid >= 0], np.arange(S, L - W))
    elig = np.arange(S // P, (L - W - 1) // P + 1)
    assert np.array_equal(hi["page_ids"][0][:len(elig)], elig)
    assert np.all(hi["page_ids"][0][len(elig):] == -1)


def test_hi_single_token_pages_equal_flat_for_any_m_at_least_dynamic_budget():
    """P = 1 with bf16 keys: the page key is the key, coarse == fine, so recalling the top
    M >= k-S-W pages already contains the flat dynamic picks."""
    L, k, S, W = 512, 64, 4, 12
    q, w, keys, _ = _hi_problem(L=L, seed=2)
    pos = np.array([L - 1])
    pk = ref.page_keys(keys, None, 1)
    assert np.array_equal(pk, keys)
    I, _, _ = ref.index_scores(q, w, keys, None, pos)
    flat = ref.select(I.astype(np.float32), np.array([L]), k, S, W)
    for M in (k - S - W, k - S - W + 7, 300):
        hi = ref.page_recall(q, w, pk, keys, None, pos, k, S, W, 1, M)
        got = ref.select(hi["cand_scores"].astype(np.float32), np.array([L]), k, S, W,
                         cand_ids=hi["cand_ids"])
        assert np.array_equal(got, flat), M


def test_hi_structure_cost_and_recall_order():
    L, P, M, k, S, W = 2048, 32, 6, 128, 16, 40
    q, w, keys, scale = _hi_problem(L=L, seed=4, fp8=True)
    pos = np.array([L - 1, 1500, 100])
    pk = ref.page_keys(keys, scale, P)
    hi = ref.page_recall(np.repeat(q, 3, 0), np.repeat(w, 3, 0), pk, keys, scale, pos, k, S, W,
                         P, M)
    for t, p in enumerate(pos):
        V = min(L, p + 1)
        pid = hi["page_ids"][t]
        if V <= k:
            assert np.all(pid == -1) and np.all(hi["cand_ids"][t] == -1)
            assert hi["n_scored"][t] == 0
            continue
        first, last = S // P, (V - W - 1) // P
        n_elig = last - first + 1
        assert np.all(np.diff(pid[pid >= 0]) > 0)
        assert np.all((pid[pid >= 0] >= first) & (pid[pid >= 0] <= last))
        coarse = hi["coarse"][t]
        elig = np.arange(first, last + 1)
        assert np.all(np.isfinite(coarse[elig]))
        assert np.all(np.isneginf(np.delete(coarse, elig)))
        rest = np.setdiff1d(elig, pid)
        assert coarse[rest].max() <= coarse[pid[pid >= 0]].min()
        cid = hi["cand_ids"][t]
        ok = cid >= 0
        assert np.all((cid[ok] >= S) & (cid[ok] < V - W))
        assert np.all(np.diff(cid[ok]) > 0)
        n_fine = ok.sum()
        assert hi["n_scored"][t] == n_elig + n_fine
        assert hi["n_scored"][t] <= L / P + M * P  # O(L/P + MP)
        # fine scores are the flat scores of the same tokens
        I, _, _ = ref.index_scores(q, w, keys, scale, np.array([p]))
        assert np.array_equal(hi["cand_scores"][t][ok], I[0][cid[ok]])


def test_hi_planted_page_is_recalled_first():
    """A page whose keys all point along the weighted query direction ranks first."""
    L, P, M, k, S, W = 1024, 16, 3, 64, 4, 12
    q, w, keys, _ = _hi_problem(L=L, seed=6)
    u = (w[0][:, None].astype(np.float64) * bf16_vals(q[0])).sum(0)
    kv = bf16_vals(keys).copy()
    kv[20 * P:21 * P] = 6.0 * u / np.linalg.norm(u)
    keys = bf16_bits(kv)
    # make sure every head responds positively to the planted direction
    w = np.abs(w)
    pk = ref.page_keys(keys, None, P)
    hi = ref.page_recall(q, w, pk, keys, None, np.array([L - 1]), k, S, W, P, M)
    assert 20 in hi["page_ids"][0]


# ------------------------------------------------------------------------------ a6/a7 attn
def _attn_problem(T=3, Hq=2, d=32, dv=24, L=50, seed=0):
    r = np.random.default_rng(seed)
    q = bf16_bits(r.standard_normal((T, Hq, d)))
    C = bf16_bits(r.standard_normal((L, max(d, dv))))
    return q, C


def test_attn_full_selection_equals_dense_causal_sdpa():
    T, Hq, d, L = 6, 2, 32, 6
    r = np.random.default_rng(1)
    q = bf16_bits(r.standard_normal((T, Hq, d)))
    K = bf16_bits(r.standard_normal((L, d)))
    Vm = bf16_bits(r.standard_normal((L, d)))
    idx = np.full((T, 8), -1, np.int32)
    for t in range(T):
        idx[t, :t + 1] = np.arange(t + 1)
    tau = 1 / math.sqrt(d)
    o, lse = ref.sparse_attn(q, K, Vm, idx, tau)
    qt = torch.from_numpy(bf16_vals(q)).permute(1, 0, 2)  # [H,T,d]
    kt = torch.from_numpy(bf16_vals(K))[None].expand(Hq, L, d)
    vt = torch.from_numpy(bf16_vals(Vm))[None].expand(Hq, L, d)
    dense = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                             scale=tau)
    np.testing.assert_allclose(o, dense.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)
    logits = torch.einsum("htd,hsd->hts", qt, kt) * tau
    logits = logits.masked_fill(torch.triu(torch.ones(T, L, dtype=torch.bool), 1), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(logits, -1).T.numpy(), rtol=1e-12)


def test_attn_latent_cache_matches_sdpa_with_sliced_values():
    T, Hq, dqk, dv, L = 2, 4, 40, 32, 30
    r = np.random.default_rng(2)
    q = bf16_bits(r.standard_normal((T, Hq, dqk)))
    C = bf16_bits(r.standard_normal((L, dqk)))
    idx = np.stack([r.permutation(L)[:12].astype(np.int32) for _ in range(T)])
    tau = 1 / math.sqrt(dqk)
    o, _ = ref.sparse_attn(q, C, C, idx, tau, d_qk=dqk, d_v=dv)
    Cv = bf16_vals(C)
    for t in range(T):
        kt = torch.from_numpy(Cv[idx[t]])
        qt = torch.from_numpy(bf16_vals(q[t]))
        dense = torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None],
                                                                 kt[None, :, :dv], scale=tau)[0]
        np.testing.assert_allclose(o[t], dense.numpy(), rtol=1e-10, atol=1e-12)


def test_attn_single_index_zero_query_and_order_invariance():
    q, C = _attn_problem(T=1, Hq=2, d=16, dv=16, L=40)
    tau = 0.3
    idx = np.full((1, 6), -1, np.int32)
    idx[0, 2] = 17
    o, lse = ref.sparse_attn(q, C, C, idx, tau)
    Cv = bf16_vals(C)
    for h in range(2):
        assert np.array_equal(o[0, h], Cv[17])
        assert lse[0, h] == pytest.approx(tau * bf16_vals(q[0, h]) @ Cv[17], rel=1e-14)
    zq = np.zeros_like(q)
    sel = np.array([[3, 9, 11, 30, -1, -1]], np.int32)
    o0, _ = ref.sparse_attn(zq, C, C, sel, tau)
    np.testing.assert_allclose(o0[0, 0], Cv[[3, 9, 11, 30]].mean(0), rtol=1e-13, atol=1e-15)
    o1, l1 = ref.sparse_attn(q, C, C, sel, tau)
    o2, l2 = ref.sparse_attn(q, C, C, np.array([[-1, 30, 3, -1, 11, 9]], np.int32), tau)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l1, l2, rtol=1e-14)
    oe, le = ref.sparse_attn(q, C, C, np.full((1, 4), -1, np.int32), tau)
    assert np.all(oe == 0) and np.all(np.isneginf(le))


def test_cross_layer_reuse_is_per_layer_attention_with_the_same_indices():
    q1, C1 = _attn_problem(seed=1)
    q2, C2 = _attn_problem(seed=2)
    idx = np.stack([np.random.default_rng(t).permutation(50)[:10].astype(np.int32)
                    for t in range(3)])
    outs = ref.cross_layer_attn([(q1, C1, C1), (q2, C2, C2)], idx, 0.2)
    a1 = ref.sparse_attn(q1, C1, C1, idx, 0.2)
    a2 = ref.sparse_attn(q2, C2, C2, idx, 0.2)
    assert np.array_equal(outs[0][0], a1[0]) and np.array_equal(outs[1][0], a2[0])
    assert not np.allclose(outs[0][0], outs[1][0])


# ------------------------------------------------------------------------------ end to end
def test_tiny_workload_end_to_end_structure():
    """A cut-down tiny-prefill workload through the whole oracle path: SI structure holds and
    the k >= V rows reduce to dense causal attention."""
    w = shrink(TINY_PREFILL_4K, n_q=300, kv_len=300)
    inp = inputs.index_inputs(w)
    q, wt = bits(inp["q"][0]), inp["w"][0].numpy()
    keys = bits(inp["keys"][0])
    pos = ref.positions(0, 300)
    I, A, E = ref.index_scores(q, wt, keys, None, pos)
    V = ref.valid_lengths(300, 0, 300)
    b = w.budget
    idx = ref.select(I.astype(np.float32), V, b.k, b.sink, b.window)
    att = inputs.attn_inputs(w)
    o, lse = ref.sparse_attn(bits(att["q"][0]), bits(att["k"][0]), bits(att["v"][0]), idx,
                             w.attn.scale)
    assert o.shape == (300, 1, 128)
    # rows with V <= k attend to every past token: compare to dense causal SDPA
    qt = torch.from_numpy(bf16_vals(bits(att["q"][0]))[:, 0])[None]
    kt = torch.from_numpy(bf16_vals(bits(att["k"][0])))[None]
    vt = torch.from_numpy(bf16_vals(bits(att["v"][0])))[None]
    dense = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                             scale=w.attn.scale)[0].numpy()
    np.testing.assert_allclose(o[:b.k, 0], dense[:b.k], rtol=1e-9, atol=1e-12)
