"""The training path on the GPU: lsa_sparse_attn_backward and lsa_index_scores_backward against
the oracle's fp64 backward (oracle/lsa_ref.c) on the same bf16 inputs, element by element.

Tolerances, per element, against magnitude sums computed alongside (M = the sum of the absolute
values of the terms the gradient element adds up):
  attention  |gpu - ref| <= 4e-3 M + 2 M_D + 1e-6.  4e-3 covers the probabilities' relative
             error: the forward's lse sums bf16-rounded probabilities (2^-9) and the logits are fp32
             sums of 576 exact products; P and dS enter the products as bf16 hi + lo pairs
             (2^-17).  M_D bounds the effect of D = dO . out taken from the forward's bf16 output
             (|out - exact| <= 2^-8 sum_j P_j |V_j|).
  indexer    |gpu - ref| <= 1e-4 M + A + 1e-6, where A holds the full contribution of every
             (query, head, entry) whose dot product lies within fp32 accumulation error of zero
             (|q.k| <= 1e-5 sum |q_i k_i|): there the GPU's fp32 sign test may legitimately
             differ from the oracle's fp64 one.  1e-4 covers the fp32 accumulation and the
             bf16 hi + lo products (2^-17).
The cache and key gradients are fp32 atomic sums (order varies between runs); every tolerance
above already holds for any summation order.
"""
import math

import numpy as np
import pytest
import torch

from oracle import ref
from token_selection_indexer_amd import lsa
from tests.gpu_checks import say
from tests.util import bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lsa.lib()
    yield
    torch.cuda.synchronize()


def _gen(seed):
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def _f64(t):
    return ref.bf16_bits_to_f64(bits(t.cpu()))


# ------------------------------------------------------------------------------ attention
def _attn_mag(q, K, V, idx, tau, g, n_rows):
    """Magnitude sums for the attention gradients of one sequence (float64 numpy): M and M_D for
    dq [T,H,dqk], the K rows [n_rows,dqk] and the V rows [n_rows,dv]."""
    T, H, dqk = q.shape
    dv = V.shape[1]
    Mq, MDq = np.zeros_like(q), np.zeros_like(q)
    MK, MDK, MV = np.zeros((n_rows, dqk)), np.zeros((n_rows, dqk)), np.zeros((n_rows, dv))
    for t in range(T):
        sel = idx[t]
        s = sel[(sel >= 0) & (sel < n_rows)]
        if s.size == 0:
            continue
        Ks, Vs = K[s], V[s]
        lg = tau * q[t] @ Ks.T
        P = np.exp(lg - lg.max(1, keepdims=True))
        P /= P.sum(1, keepdims=True)
        dP = g[t] @ Vs.T
        D = (P * dP).sum(1, keepdims=True)
        eD = 2.0 ** -8 * (P * (np.abs(g[t]) @ np.abs(Vs).T)).sum(1, keepdims=True)
        w = tau * P * (np.abs(dP) + np.abs(D))
        wD = tau * P * eD
        Mq[t] = w @ np.abs(Ks)
        MDq[t] = wD @ np.abs(Ks)
        np.add.at(MK, s, w.T @ np.abs(q[t]))
        np.add.at(MDK, s, wD.T @ np.abs(q[t]))
        np.add.at(MV, s, P.T @ np.abs(g[t]))
    return Mq, MDq, MK, MDK, MV


def _check(label, gpu, want, M, MD, rel):
    tol = rel * M + 2.0 * MD + 1e-6
    err = np.abs(gpu - want)
    ratio = float((err / tol).max()) if err.size else 0.0
    say(f"[bwd] {label}: max|err| {err.max() if err.size else 0:.3g}, max err/tol {ratio:.3g}")
    bad = np.argwhere(err > tol)
    assert bad.size == 0, (f"{label}: {len(bad)} elements out of tolerance, first {bad[:3]}, "
                           f"gpu {gpu[tuple(bad[0])]}, ref {want[tuple(bad[0])]}, tol {tol[tuple(bad[0])]}")


def _attn_case(B, T, H, L, k, latent, dqk=576, dv=512, seed=0, seq_lens=None, pad=0.0,
               lists=None, si=None):
    """Random bf16 q / cache / output gradient, index lists with skipped (-1), out-of-range and
    repeated entries (or the given lists); forward and backward on the GPU; oracle backward per
    sequence.  si = (sink, window, q_pos0): the lists' Streaming-Aware layout, passed on to the
    backward call."""
    g = _gen(seed)
    q = torch.randn((B, T, H, dqk), generator=g).to(torch.bfloat16)
    if latent:
        kv = torch.randn((B, L, dqk), generator=g).to(torch.bfloat16)
        v = None
    else:
        kv = torch.randn((B, L, dqk), generator=g).to(torch.bfloat16)
        v = torch.randn((B, L, dv), generator=g).to(torch.bfloat16)
    dout = torch.randn((B, T, H, dv), generator=g).to(torch.bfloat16)
    idx = torch.stack([torch.stack([torch.randperm(L, generator=g)[:k] for _ in range(T)])
                       for _ in range(B)]).to(torch.int32)
    m = torch.rand((B, T, k), generator=g)
    idx = torch.where(m < pad, torch.full_like(idx, -1), idx)
    if k > 8:
        idx[:, :, 3] = idx[:, :, 5]          # a row selected twice by one query
        idx[:, 0, 7] = L + 3                 # past the cache: skipped
    if lists is not None:
        idx = torch.from_numpy(lists)
    tau = 1.0 / math.sqrt(dqk)
    qd, kvd, dod, idd = q.to(DEV), kv.to(DEV), dout.to(DEV), idx.to(DEV)
    vd = None if latent else v.to(DEV)
    lens = None if seq_lens is None else torch.tensor(seq_lens, dtype=torch.int32, device=DEV)
    out, lse = lsa.sparse_attn(qd, kvd, vd, idd, tau, d_v=dv, seq_lens=lens)
    sink, window, q_pos0 = si if si is not None else (0, 0, 0)
    d_q, d_k, d_v = lsa.sparse_attn_backward(qd, kvd, vd, idd, out, lse, dod, tau, d_v=dv,
                                             seq_lens=lens, sink=sink, window=window,
                                             q_pos0=q_pos0)
    torch.cuda.synchronize()
    gq, gk, gv = (x.cpu().numpy().astype(np.float64) for x in (d_q, d_k, d_v))
    for b in range(B):
        n_rows = L if seq_lens is None else seq_lens[b]
        qb = _f64(q[b])
        Kb = _f64(kv[b])[:n_rows]
        Vb = Kb[:, :dv] if latent else _f64(v[b])[:n_rows]
        gb = _f64(dout[b])
        ib = idx[b].numpy()
        if n_rows == 0:
            rq = np.zeros_like(qb)
            rK, rV = np.zeros((0, dqk)), np.zeros((0, dv))
            Mq = MDq = rq
            MK = MDK = rK
            MV = rV
        else:
            rq, rK, rV = ref.sparse_attn_backward(qb, Kb, Vb, ib, tau, gb, d_qk=dqk, d_v=dv)
            Mq, MDq, MK, MDK, MV = _attn_mag(qb, Kb, Vb, ib, tau, gb, n_rows)
        _check(f"dq b={b}", gq[b], rq, Mq, MDq, 4e-3)
        if latent:
            want = rK.copy()
            want[:, :dv] += rV
            M = MK.copy()
            M[:, :dv] += MV
            _check(f"dkv b={b}", gk[b, :n_rows], want, M, MDK, 4e-3)
        else:
            _check(f"dk b={b}", gk[b, :n_rows], rK, MK, MDK, 4e-3)
            _check(f"dv b={b}", gv[b, :n_rows], rV, MV, np.zeros_like(MV), 4e-3)
        # rows past a sequence's length get nothing
        assert np.all(gk[b, n_rows:] == 0)


def test_mla_backward_small_with_splits():
    """16 and 32 heads (one and two head groups), 200 entries per query in three chunks."""
    assert lsa.lsa_workspace_bytes  # binding loaded
    _attn_case(B=2, T=3, H=16, L=600, k=200, latent=True, seed=1, pad=0.05)
    _attn_case(B=1, T=2, H=32, L=300, k=130, latent=True, seed=2)


def test_mla_backward_decode_shape():
    """Decode at k = 2048: the index list in 32 chunks whose dQ parts add up atomically."""
    _attn_case(B=2, T=1, H=16, L=8192, k=2048, latent=True, seed=3)


def test_mla_backward_prefill_rows_shared_by_many_queries():
    """128 queries over a 2048-row cache with 512 entries each: every cache row collects the
    gradients of about 32 queries x 16 heads through atomics."""
    _attn_case(B=1, T=128, H=16, L=2048, k=512, latent=True, seed=4)


def test_mla_backward_ragged():
    _attn_case(B=3, T=2, H=16, L=700, k=96, latent=True, seed=5, seq_lens=[700, 250, 0])


def _si_lists(B, T, L, q_pos0, k, S, W, seed):
    """Index lists in the layout lsa_topk_select writes: with V = min(L, q_pos0 + t + 1), a
    query with V <= k takes rows 0 .. V-1; else sink rows 0 .. S-1, window rows V-W .. V-1, then
    distinct rows from [S, V - W) and -1 padding."""
    rng = np.random.default_rng(seed)
    idx = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        for t in range(T):
            V = min(L, q_pos0 + t + 1)
            if V <= k:
                idx[b, t, :V] = np.arange(V)
                continue
            idx[b, t, :S] = np.arange(S)
            idx[b, t, S:S + W] = np.arange(V - W, V)
            pool = np.arange(S, V - W)
            dyn = rng.choice(pool, size=min(k - S - W, pool.size), replace=False)
            idx[b, t, S + W:S + W + dyn.size] = dyn
    return idx


@pytest.mark.parametrize("H", [16, 32])
def test_mla_backward_streaming_aware_lists(H):
    """Prefill-shaped lists in the Streaming-Aware layout, with the layout passed to the
    backward call: the sink and window entries' cache gradient is summed row by row over the
    queries (the key-major pass), the rest per query.  Entries that break the layout are left
    to the per-query path: a window entry holding another row, a sink entry holding another
    row, a skipped (-1) sink entry, and a window row selected a second time among the dynamic
    picks (added once by each path).  Queries past the cache end (V = L for the last ones)."""
    B, T, L, q0, k, S, W = 2, 300, 1480, 1200, 256, 16, 112
    idx = _si_lists(B, T, L, q0, k, S, W, seed=21)
    idx[:, 5, S + 3] = 40
    idx[:, 7, 2] = 500
    idx[:, 9, 1] = -1
    idx[:, 11, S + W] = idx[:, 11, S + W - 1]
    if H == 32:
        B, T = 1, 120
        idx = idx[:1, :T]
    _attn_case(B=B, T=T, H=H, L=L, k=k, latent=True, seed=22, lists=idx, si=(S, W, q0))


def test_mla_backward_streaming_aware_early_queries():
    """A chunk from the start of a sequence: the first queries see fewer than k rows and take
    all of them, so their sink entries match the layout and their window entries mostly do not;
    the earliest have a window reaching into the sink (no entry of theirs is key-major).  64
    sink rows (one whole block) and a 64-row window."""
    B, T, L, q0, k, S, W = 1, 400, 400, 0, 200, 64, 64
    idx = _si_lists(B, T, L, q0, k, S, W, seed=23)
    _attn_case(B=B, T=T, H=16, L=L, k=k, latent=True, seed=24, lists=idx, si=(S, W, q0))


def test_mha_backward():
    _attn_case(B=2, T=5, H=3, L=300, k=40, latent=False, dqk=64, dv=48, seed=6, pad=0.1)
    _attn_case(B=1, T=3, H=1, L=500, k=64, latent=False, dqk=128, dv=128, seed=7)


def test_backward_accumulates_into_given_gradients():
    """Two calls into the same arrays give twice one call (the gradients are added into)."""
    g = _gen(8)
    B, T, H, L, k = 1, 2, 16, 400, 64
    q = torch.randn((B, T, H, 576), generator=g).to(torch.bfloat16).to(DEV)
    kv = torch.randn((B, L, 576), generator=g).to(torch.bfloat16).to(DEV)
    dout = torch.randn((B, T, H, 512), generator=g).to(torch.bfloat16).to(DEV)
    idx = torch.stack([torch.randperm(L, generator=g)[:k] for _ in range(T)])[None].to(torch.int32).to(DEV)
    out, lse = lsa.sparse_attn(q, kv, None, idx, 0.05, d_v=512)
    d1q, d1k, _ = lsa.sparse_attn_backward(q, kv, None, idx, out, lse, dout, 0.05, d_v=512)
    d2q, d2k, _ = lsa.sparse_attn_backward(q, kv, None, idx, out, lse, dout, 0.05, d_v=512)
    lsa.sparse_attn_backward(q, kv, None, idx, out, lse, dout, 0.05, d_v=512, d_q=d2q, d_k=d2k)
    torch.cuda.synchronize()
    torch.testing.assert_close(d2q, 2 * d1q, rtol=1e-5, atol=1e-6)
    torch.testing.assert_close(d2k, 2 * d1k, rtol=1e-5, atol=1e-6)


# ------------------------------------------------------------------------------ indexer
def _index_mag(q, w, K, idx, pos, gI, n_rows):
    """Magnitude sums M and ambiguous-sign contributions A for dq, dw and the key rows."""
    T, H, d = q.shape
    Mq, Aq = np.zeros_like(q), np.zeros_like(q)
    Mw, Aw = np.zeros((T, H)), np.zeros((T, H))
    MK, AK = np.zeros((n_rows, d)), np.zeros((n_rows, d))
    for t in range(T):
        V = min(n_rows, pos[t] + 1)
        sel = idx[t]
        ok = (sel >= 0) & (sel < V)
        s = sel[ok]
        if s.size == 0:
            continue
        Ks = K[s]
        dots = q[t] @ Ks.T
        amb = np.abs(dots) <= 1e-5 * (np.abs(q[t]) @ np.abs(Ks).T)
        G = np.abs(gI[t, ok])[None, :] * np.abs(w[t])[:, None]
        on = (dots > 0) | amb
        Mq[t] = (G * on) @ np.abs(Ks)
        Aq[t] = (G * amb) @ np.abs(Ks)
        Mw[t] = (np.abs(gI[t, ok])[None, :] * np.abs(dots) * on).sum(1)
        Aw[t] = (np.abs(gI[t, ok])[None, :] * np.abs(dots) * amb).sum(1)
        np.add.at(MK, s, (G * on).T @ np.abs(q[t]))
        np.add.at(AK, s, (G * amb).T @ np.abs(q[t]))
    return (Mq, Aq), (Mw, Aw), (MK, AK)


def _index_case(B, T, H, d, L, k, seed, q_pos0=None, seq_lens=None, seq_pos0=None, lists=None,
                si=(0, 0)):
    """Random bf16 q / keys, head weights and score gradients over random lists with skipped and
    repeated entries (or the given lists); the GPU backward against the oracle per sequence.
    si = (sink, window): the lists' Streaming-Aware layout, passed on to the backward call."""
    g = _gen(seed)
    q = torch.randn((B, T, H, d), generator=g).to(torch.bfloat16)
    w = (torch.randn((B, T, H), generator=g) / 2).to(torch.float32)
    keys = torch.randn((B, L, d), generator=g).to(torch.bfloat16)
    idx = torch.stack([torch.stack([torch.randperm(L, generator=g)[:k] for _ in range(T)])
                       for _ in range(B)]).to(torch.int32)
    idx[:, :, 1] = -1
    if k > 6:
        idx[:, :, 4] = idx[:, :, 6]
    if lists is not None:
        idx = torch.from_numpy(lists)
    gI = torch.randn((B, T, k), generator=g).to(torch.float32)
    pos0 = L - T if q_pos0 is None else q_pos0
    lens = None if seq_lens is None else torch.tensor(seq_lens, dtype=torch.int32, device=DEV)
    p0 = None if seq_pos0 is None else torch.tensor(seq_pos0, dtype=torch.int32, device=DEV)
    d_q, d_w, d_k = lsa.index_scores_backward(q.to(DEV), w.to(DEV), keys.to(DEV), idx.to(DEV),
                                              gI.to(DEV), q_pos0=pos0, seq_lens=lens, seq_pos0=p0,
                                              sink=si[0], window=si[1])
    torch.cuda.synchronize()
    gq, gw, gk = (x.cpu().numpy().astype(np.float64) for x in (d_q, d_w, d_k))
    for b in range(B):
        n_rows = L if seq_lens is None else seq_lens[b]
        first = pos0 if seq_pos0 is None else seq_pos0[b]
        pos = first + np.arange(T, dtype=np.int64)
        qb, Kb = _f64(q[b]), _f64(keys[b])[:max(n_rows, 1)]
        wb = w[b].numpy().astype(np.float64)
        ib, gb = idx[b].numpy(), gI[b].numpy().astype(np.float64)
        if n_rows == 0:
            assert np.all(gq[b] == 0) and np.all(gw[b] == 0) and np.all(gk[b] == 0)
            continue
        rq, rw, rk = ref.index_scores_backward(qb, wb, Kb, ib, pos, gb)
        (Mq, Aq), (Mw, Aw), (MK, AK) = _index_mag(qb, wb, Kb, ib, pos, gb, n_rows)
        for name, gpu, want, M, A in (("dq", gq[b], rq, Mq, Aq), ("dw", gw[b], rw, Mw, Aw),
                                      ("dk", gk[b, :n_rows], rk, MK, AK)):
            tol = 1e-4 * M + A + 1e-6
            err = np.abs(gpu - want)
            say(f"[bwd] index {name} b={b}: max|err| {err.max():.3g}, max err/tol "
                f"{float((err / tol).max()):.3g}, ambiguous terms {int((A > 0).sum())}")
            bad = np.argwhere(err > tol)
            assert bad.size == 0, (f"index {name} b={b}: {len(bad)} out of tolerance, first "
                                   f"{bad[:3]}")
        assert np.all(gk[b, n_rows:] == 0)


@pytest.mark.parametrize("H,d", [(64, 128), (4, 64), (20, 128), (48, 64)])
def test_index_backward_heads_and_widths(H, d):
    """One to four waves per workgroup (16 heads each, the last one padded)."""
    _index_case(B=2, T=4, H=H, d=d, L=500, k=128, seed=11 + H)


@pytest.mark.parametrize("H", [64, 20])
def test_index_backward_streaming_aware_lists(H):
    """Prefill-shaped lists in the Streaming-Aware layout with the layout passed on: the sink and
    window entries' key gradient is summed row by row over the queries (the key-major pass), the
    rest per query.  Entries that break the layout stay with the per-query path: a window entry
    holding another row, a sink entry holding another row, a skipped sink entry, and a window
    row selected again among the dynamic picks.  Queries past the cache end (V = L for the
    last ones); 20 heads leave the pass's missing heads zero."""
    B, T, L, q0, k, S, W = 2, 300, 1480, 1200, 256, 16, 112
    idx = _si_lists(B, T, L, q0, k, S, W, seed=31)
    idx[:, 5, S + 3] = 40
    idx[:, 7, 2] = 500
    idx[:, 9, 1] = -1
    idx[:, 11, S + W] = idx[:, 11, S + W - 1]
    _index_case(B=B, T=T, H=H, d=128, L=L, k=k, seed=32 + H, q_pos0=q0, lists=idx, si=(S, W))


def test_index_backward_streaming_aware_early_queries():
    """A chunk from the start of a sequence: the first queries see fewer than k rows and take
    all of them; the earliest have a window reaching into the sink (none of their entries is
    key-major).  64 sink rows (one whole block) and a 64-row window."""
    B, T, L, q0, k, S, W = 1, 400, 400, 0, 200, 64, 64
    idx = _si_lists(B, T, L, q0, k, S, W, seed=33)
    _index_case(B=B, T=T, H=64, d=128, L=L, k=k, seed=34, q_pos0=q0, lists=idx, si=(S, W))


def test_index_backward_causal_prefill_and_splits():
    """Queries at positions 300..363 of a 700-key cache: entries past each query's position are
    skipped; 256 entries per query in several chunks."""
    _index_case(B=1, T=64, H=64, d=128, L=700, k=256, seed=21, q_pos0=300)


def test_index_backward_decode_shape():
    _index_case(B=2, T=1, H=64, d=128, L=16384, k=2048, seed=22)


def test_index_backward_ragged():
    _index_case(B=3, T=2, H=64, d=128, L=900, k=128, seed=23, seq_lens=[900, 300, 0],
                seq_pos0=[898, 298, 0])


# ------------------------------------------------------------------------------ full shape
def _sample_rows(kv_f64, ids):
    """The selected rows of one query, re-indexed 0..k-1 (-1 kept): the oracle then needs only
    those rows (a query's own gradient depends on its own rows alone)."""
    ok = ids >= 0
    rows = kv_f64[np.where(ok, ids, 0)]
    return rows, np.where(ok, np.arange(ids.size), -1).astype(np.int32)[None]


def test_backward_prefill_8k_128k_full_shape():
    """The training path at the chunked-prefill shape (8192 queries, 128K keys, k = 2048), on
    the GPU's own selection, whose Streaming-Aware layout is passed on (the sink and window
    entries' cache gradient goes through the key-major pass, about half of all entries): sampled
    queries' dq (all heads) and dw against the oracle, and over
    the whole launch the identities the gradients obey exactly:
      attention  sum_r dV_r = sum_(t,h) dO_(t,h)            (softmax rows sum to one)
                 <dKV, KV> - <dq, q> = sum_(t,h) dO . out    (the logits are bilinear in q and K;
                                                             <dV, V> = sum dO . O)
      indexer    <dq, q> = <dk, K> = <dw, w>                 (the score has degree 1 in each)
    The identities pair every row's gradient with its own row, so misrouted or dropped updates
    break them.  Tolerances: 2^-8 of the magnitude for terms carrying the forward's bf16 output
    and lse (reading in the header), plus 1e-6 of the magnitude of the inner products (sum of
    the absolute products) for the fp32 gradients' rounding.  That last term is statistical, not
    a worst case: the atomic sums' rounding errors have random signs, so their effect on an
    inner product of N terms scales like 2^-24 sqrt(n) / sqrt(N) of the magnitude, over 100
    times below 1e-6 here; and 1e-6 of the magnitude stays well below each identity's own value,
    so a dropped or misrouted share of the gradient fails."""
    from token_selection_indexer_amd import configs, inputs
    w = configs.PREFILL_8K_AT_128K
    s, b, a = w.index, w.budget, w.attn
    inp = inputs.index_inputs(w, DEV)
    att = inputs.attn_inputs(w, 0, DEV)
    scores = lsa.index_scores(inp["q"], inp["w"], inp["keys"], None, q_pos0=s.q_pos0)
    idx = lsa.topk_select(scores, b.k, b.sink, b.window, kv_len=s.kv_len, q_pos0=s.q_pos0)
    del scores
    out, lse = lsa.sparse_attn(att["q"], att["kv"], None, idx, a.scale, b.sink, b.window, d_v=a.d_v)
    g = torch.Generator(device=DEV)
    g.manual_seed(17)
    dout = torch.randn(out.shape, generator=g, device=DEV).to(torch.bfloat16)
    dsc = torch.randn(idx.shape, generator=g, device=DEV)
    d_q, d_kv, _ = lsa.sparse_attn_backward(att["q"], att["kv"], None, idx, out, lse, dout,
                                            a.scale, d_v=a.d_v, sink=b.sink, window=b.window,
                                            q_pos0=s.q_pos0)
    di_q, di_w, di_k = lsa.index_scores_backward(inp["q"], inp["w"], inp["keys"], idx, dsc,
                                                 q_pos0=s.q_pos0, sink=b.sink, window=b.window)
    torch.cuda.synchronize()
    dv = a.d_v
    # attention identities
    dO = dout.double()
    lhs = d_kv[0, :, :dv].double().sum(0)
    rhs = dO.sum((0, 1, 2))
    tol = 2.0 ** -8 * dO.abs().sum((0, 1, 2)) + 1e-3
    assert bool(((lhs - rhs).abs() <= tol).all()), float(((lhs - rhs).abs() / tol).max())
    kvd, qd = att["kv"].double(), att["q"].double()
    e_kv, e_q = (d_kv.double() * kvd), (d_q.double() * qd)
    euler = float(e_kv.sum() - e_q.sum())
    want = float((dO * out.double()).sum())
    tol = (2.0 ** -8 * float((dO.abs() * out.double().abs()).sum())
           + 1e-6 * float(e_kv.abs().sum() + e_q.abs().sum()))
    say(f"[bwd] attention full shape: sum dV vs sum dO ok; <dKV,KV> - <dq,q> = {euler:.6g}, "
        f"sum dO.out = {want:.6g}, tol {tol:.3g}")
    assert abs(euler - want) <= tol
    # indexer identity
    iq = float((di_q.double() * inp["q"].double()).sum())
    ik = float((di_k.double() * inp["keys"].double()).sum())
    iw = float((di_w.double() * inp["w"].double()).sum())
    mag = float((di_q.double() * inp["q"].double()).abs().sum() +
                (di_k.double() * inp["keys"].double()).abs().sum() +
                (di_w.double() * inp["w"].double()).abs().sum())
    say(f"[bwd] indexer full shape: <dq,q> {iq:.6g}, <dk,K> {ik:.6g}, <dw,w> {iw:.6g}, mag {mag:.3g}")
    assert abs(iq - ik) <= 1e-6 * mag and abs(iq - iw) <= 1e-6 * mag
    # sampled queries against the oracle
    kv_f = _f64(att["kv"][0])
    keys_f = _f64(inp["keys"][0])
    tau = a.scale
    for t in (0, 1, 4095, 4096, 8191):
        ids = idx[0, t].cpu().numpy()
        rows, ir = _sample_rows(kv_f, ids)
        qt = _f64(att["q"][0, t:t + 1])
        gt = _f64(dout[0, t:t + 1])
        rq, _, _ = ref.sparse_attn_backward(qt, rows, rows, ir, tau, gt, d_qk=a.d_qk, d_v=dv)
        Mq, MDq, _, _, _ = _attn_mag(qt, rows, rows[:, :dv], ir, tau, gt, rows.shape[0])
        _check(f"full-shape dq t={t}", d_q[0, t:t + 1].cpu().numpy().astype(np.float64), rq, Mq,
               MDq, 4e-3)
        krows, kir = _sample_rows(keys_f, ids)
        qi = _f64(inp["q"][0, t:t + 1])
        wi = inp["w"][0, t:t + 1].cpu().numpy().astype(np.float64)
        gi = dsc[0, t:t + 1].cpu().numpy().astype(np.float64)
        pos = np.array([ids.size], np.int64)  # every re-indexed row is in the past
        rq2, rw2, _ = ref.index_scores_backward(qi, wi, krows, kir, pos, gi)
        (Mq2, Aq2), (Mw2, Aw2), _ = _index_mag(qi, wi, krows, kir, pos, gi, krows.shape[0])
        for name, gpu, want2, M, A in (("dq", di_q[0, t:t + 1], rq2, Mq2, Aq2),
                                       ("dw", di_w[0, t:t + 1], rw2, Mw2, Aw2)):
            err = np.abs(gpu.cpu().numpy().astype(np.float64) - want2)
            assert (err <= 1e-4 * M + A + 1e-6).all(), (name, t, float(err.max()))
    say("[bwd] full-shape sampled queries ok")
