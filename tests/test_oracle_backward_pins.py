"""Pins of the oracle's backward functions (CPU only).

The backward functions are checked against central finite differences of the oracle's own
forward definitions (so a wrong sign, a dropped softmax term, a transposed operand or a
gradient routed to the wrong row fails), against torch's autograd of dense attention where the
selection covers every token, and against closed forms (one selected entry, all-positive
indexer dot products) and invariants (the softmax Jacobian's zero row sums).
"""
import math

import numpy as np
import pytest
import torch

from oracle import ref
from tests.util import bits


def bf16_bits(x):
    return bits(torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16))


def central_diff(f, x, eps):
    """d f / d x by central differences, element by element (x float64, modified in place and
    restored)."""
    g = np.zeros_like(x)
    for i in np.ndindex(x.shape):
        v = x[i]
        x[i] = v + eps
        fp = f()
        x[i] = v - eps
        fm = f()
        x[i] = v
        g[i] = (fp - fm) / (2 * eps)
    return g


# ------------------------------------------------------------------------------ attention
def _attn_case(seed=0, T=3, Hq=2, dqk=8, dv=6, L=10):
    r = np.random.default_rng(seed)
    q = r.standard_normal((T, Hq, dqk))
    K = r.standard_normal((L, dqk))
    V = r.standard_normal((L, dv))
    # a skipped entry, an entry past the cache, a row selected twice by one query
    idx = np.array([[0, 3, 5, -1, 9], [2, 2, 7, 1, 4], [6, 8, 0, 3, L + 5]], np.int32)[:T]
    g = r.standard_normal((T, Hq, dv))
    return q, K, V, idx, g


def test_attn_f64_forward_equals_the_bf16_forward_on_bf16_values():
    r = np.random.default_rng(3)
    T, Hq, d, dv, L = 4, 3, 24, 16, 40
    qb = bf16_bits(r.standard_normal((T, Hq, d)))
    Cb = bf16_bits(r.standard_normal((L, d)))
    idx = np.stack([r.permutation(L)[:9].astype(np.int32) for _ in range(T)])
    idx[1, 4] = -1
    o, lse = ref.sparse_attn(qb, Cb, Cb, idx, 0.2, d_qk=d, d_v=dv)
    o2, lse2 = ref.sparse_attn_f64(ref.bf16_bits_to_f64(qb), ref.bf16_bits_to_f64(Cb), None, idx,
                                   0.2, d_qk=d, d_v=dv)
    np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse2, lse, rtol=1e-14)


def test_attn_backward_matches_central_differences():
    q, K, V, idx, g = _attn_case()
    tau = 0.3
    dq, dK, dV = ref.sparse_attn_backward(q, K, V, idx, tau, g)

    def loss():
        return float((ref.sparse_attn_f64(q, K, V, idx, tau)[0] * g).sum())

    for name, x, an in (("q", q, dq), ("K", K, dK), ("V", V, dV)):
        fd = central_diff(loss, x, 1e-6)
        np.testing.assert_allclose(an, fd, rtol=1e-6, atol=1e-8, err_msg=name)
    # rows nobody selected have no gradient
    assert np.all(dK[[x for x in range(10) if x not in idx]] == 0)


def test_attn_backward_latent_cache_gradient_is_dk_plus_dv():
    """One matrix C serves as K (all columns) and V (the first dv columns)."""
    r = np.random.default_rng(5)
    T, Hq, dqk, dv, L = 2, 3, 10, 6, 9
    q = r.standard_normal((T, Hq, dqk))
    C = r.standard_normal((L, dqk))
    idx = np.array([[1, 4, 7, 0], [4, 8, 2, -1]], np.int32)
    g = r.standard_normal((T, Hq, dv))
    dq, dK, dV = ref.sparse_attn_backward(q, C, C, idx, 0.4, g, d_qk=dqk, d_v=dv)

    def loss():
        return float((ref.sparse_attn_f64(q, C, C, idx, 0.4, d_qk=dqk, d_v=dv)[0] * g).sum())

    fd = central_diff(loss, C, 1e-6)
    comb = dK.copy()
    comb[:, :dv] += dV
    np.testing.assert_allclose(comb, fd, rtol=1e-6, atol=1e-8)


def test_attn_backward_equals_autograd_of_dense_causal_attention():
    """Full selection (every past token) is dense causal attention: torch's SDPA backward in
    float64 gives the same gradients."""
    T, Hq, d, L = 7, 2, 16, 7
    r = np.random.default_rng(7)
    q = r.standard_normal((T, Hq, d))
    K = r.standard_normal((L, d))
    V = r.standard_normal((L, d))
    g = r.standard_normal((T, Hq, d))
    idx = np.full((T, 8), -1, np.int32)
    for t in range(T):
        idx[t, :t + 1] = np.arange(t + 1)[::-1]
    tau = 1 / math.sqrt(d)
    dq, dK, dV = ref.sparse_attn_backward(q, K, V, idx, tau, g)
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(K, requires_grad=True)
    vt = torch.tensor(V, requires_grad=True)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt.permute(1, 0, 2), kt[None].expand(Hq, L, d), vt[None].expand(Hq, L, d),
        is_causal=True, scale=tau)
    (o.permute(1, 0, 2) * torch.tensor(g)).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dK, kt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dV, vt.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_attn_backward_closed_forms_and_invariants():
    r = np.random.default_rng(9)
    T, Hq, d, dv, L = 3, 4, 12, 8, 30
    q = r.standard_normal((T, Hq, d))
    K = r.standard_normal((L, d))
    V = r.standard_normal((L, dv))
    g = r.standard_normal((T, Hq, dv))
    # one valid entry per row: softmax is constant 1, so dq = 0, dK = 0, dV[r] = sum of g
    one = np.array([[5, -1, -1], [-1, 11, -1], [-1, -1, 29]], np.int32)
    dq, dK, dV = ref.sparse_attn_backward(q, K, V, one, 0.5, g)
    assert np.all(dq == 0) and np.abs(dK).max() < 1e-14
    for t, rr in enumerate((5, 11, 29)):
        np.testing.assert_allclose(dV[rr], g[t].sum(0), rtol=1e-14)
    # softmax rows sum to one and the Jacobian's rows to zero: sum_r dV[r] = sum of all g,
    # sum_r dK[r] = 0
    idx = np.stack([r.permutation(L)[:10].astype(np.int32) for _ in range(T)])
    dq, dK, dV = ref.sparse_attn_backward(q, K, V, idx, 0.5, g)
    np.testing.assert_allclose(dV.sum(0), g.sum((0, 1)), rtol=1e-12, atol=1e-12)
    assert np.abs(dK.sum(0)).max() < 1e-12
    # entry order and -1 padding change nothing
    perm = np.concatenate([idx[:, ::-1], np.full((T, 3), -1, np.int32)], 1)
    dq2, dK2, dV2 = ref.sparse_attn_backward(q, K, V, perm, 0.5, g)
    np.testing.assert_allclose(dq2, dq, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dK2, dK, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dV2, dV, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------------------ indexer
def _index_case(seed=1, T=3, H=4, d=8, L=12):
    r = np.random.default_rng(seed)
    q = r.standard_normal((T, H, d))
    w = r.standard_normal((T, H))
    K = r.standard_normal((L, d))
    # skipped, future (past V_t) and repeated entries
    idx = np.array([[0, 3, 5, -1, 9], [2, 2, 7, 1, 4], [6, 8, 0, 3, 11]], np.int32)[:T]
    pos = np.array([7, 11, 10], np.int64)[:T]
    gI = r.standard_normal((T, idx.shape[1]))
    return q, w, K, idx, pos, gI


def test_index_sel_f64_equals_the_scores_at_the_selected_entries():
    r = np.random.default_rng(4)
    T, H, d, L = 5, 4, 16, 50
    qb = bf16_bits(r.standard_normal((T, H, d)))
    kb = bf16_bits(r.standard_normal((L, d)))
    w = r.standard_normal((T, H)).astype(np.float32)
    pos = np.array([10, 49, 30, 5, 49], np.int64)
    I, _, _ = ref.index_scores(qb, w, kb, None, pos)
    idx = np.stack([r.permutation(L)[:12].astype(np.int32) for _ in range(T)])
    idx[0, 0] = -1
    Is = ref.index_scores_sel_f64(ref.bf16_bits_to_f64(qb), w.astype(np.float64),
                                  ref.bf16_bits_to_f64(kb), idx, pos)
    for t in range(T):
        for j in range(12):
            s = idx[t, j]
            want = I[t, s] if 0 <= s <= pos[t] else 0.0
            assert Is[t, j] == pytest.approx(want, rel=1e-14, abs=1e-14)


def test_index_backward_matches_central_differences():
    q, w, K, idx, pos, gI = _index_case()
    # no dot product near the ReLU kink, so the differences stay on one linear piece
    dots = np.einsum("thd,sd->ths", q, K)
    assert np.abs(dots).min() > 1e-3
    dq, dw, dk = ref.index_scores_backward(q, w, K, idx, pos, gI)

    def loss():
        return float((ref.index_scores_sel_f64(q, w, K, idx, pos) * gI).sum())

    for name, x, an in (("q", q, dq), ("w", w, dw), ("k", K, dk)):
        fd = central_diff(loss, x, 1e-7)
        np.testing.assert_allclose(an, fd, rtol=1e-6, atol=1e-7, err_msg=name)


def test_index_backward_gemv_closed_form():
    """H = 1, w = 1 and every dot product positive: the score is the plain dot product, so
    dq = sum_j g_j k_j, dk[s] = sum over the entries at s of g q, dw = sum_j g_j q.k_j."""
    r = np.random.default_rng(11)
    T, d, L, k = 4, 6, 20, 7
    q = np.abs(r.standard_normal((T, 1, d))) + 0.1
    K = np.abs(r.standard_normal((L, d))) + 0.1
    w = np.ones((T, 1))
    idx = np.stack([r.permutation(L)[:k].astype(np.int32) for _ in range(T)])
    pos = np.full(T, L, np.int64)
    gI = r.standard_normal((T, k))
    dq, dw, dk = ref.index_scores_backward(q, w, K, idx, pos, gI)
    want_dk = np.zeros_like(K)
    for t in range(T):
        np.testing.assert_allclose(dq[t, 0], gI[t] @ K[idx[t]], rtol=1e-13)
        assert dw[t, 0] == pytest.approx(float(gI[t] @ (K[idx[t]] @ q[t, 0])), rel=1e-13)
        for j in range(k):
            want_dk[idx[t, j]] += gI[t, j] * q[t, 0]
    np.testing.assert_allclose(dk, want_dk, rtol=1e-13, atol=1e-15)


def test_index_backward_ignores_skipped_and_future_entries():
    q, w, K, idx, pos, gI = _index_case(seed=2)
    dq, dw, dk = ref.index_scores_backward(q, w, K, idx, pos, gI)
    clean = idx.copy()
    for t in range(idx.shape[0]):
        clean[t][(idx[t] < 0) | (idx[t] > pos[t])] = -1
    assert not np.array_equal(clean, idx)
    dq2, dw2, dk2 = ref.index_scores_backward(q, w, K, clean, pos, gI)
    assert np.array_equal(dq, dq2) and np.array_equal(dw, dw2) and np.array_equal(dk, dk2)
    # key 11 is only selected by row 2, whose V is 11: never in range
    assert np.all(dk[11] == 0)
