"""Comparisons of GPU outputs with the CPU oracle, shared by the GPU test modules.

Bars (the same everywhere): indexer scores within 1e-3 of the error scale max(A, E/100)
(tests/util.py: score_tol); index lists bit-exact when both sides select from the same fp32
scores, else equal up to near-ties with recall >= 99.9% over all rows checked; page keys
bit-exact; attention within 2e-2 max-abs of the fp64 oracle on the GPU's own index lists.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import ref
from tests.util import NearTie, bits, check_si_layout, f32, keys_np, score_tol


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def assert_scores(gpu_row, I, A, E, label=""):
    g = np.asarray(gpu_row, np.float64)
    neg = np.isneginf(I)
    assert np.array_equal(np.isneginf(g), neg), f"{label}: -inf pattern differs"
    tol = score_tol(A, E)
    err = np.abs(g[~neg] - I[~neg])
    bad = err > tol[~neg]
    assert not bad.any(), f"{label}: {bad.sum()} scores out of tolerance, worst {err.max()}"


def oracle_scores(inp, b, rows, q_pos0):
    """Oracle scores of sequence b for query rows `rows` (absolute positions q_pos0 + row)."""
    keys, scale = keys_np(inp, b)
    q = bits(inp["q"][b])[rows]
    w = f32(inp["w"][b])[rows]
    return ref.index_scores(q, w, keys, scale, q_pos0 + np.asarray(rows, np.int64))


def kth_of(ridx_row, I_row, S, W):
    """The oracle's k-th (weakest) dynamic pick of a row and its score."""
    dyn = ridx_row[S + W:]
    dyn = dyn[dyn >= 0]
    kth = dyn[np.argmin(I_row[dyn])]
    return kth, I_row[kth]


def selection_vs_oracle_scores(nt: NearTie, gpu_row, I, A, E, V, k, S, W, cand_ids=None):
    """One GPU-selected row against the oracle's selection from its own fp64 scores (rounded to
    fp32, the precision both sides decide in): the dynamic picks must agree up to near-ties.
    I, A, E are over the row's scored elements (tokens, or candidate slots with cand_ids)."""
    scores32 = I.astype(np.float32)[None]
    cid = None if cand_ids is None else np.asarray(cand_ids)[None]
    ridx = ref.select(scores32, np.array([V]), k, S, W, cand_ids=cid)[0]
    if V <= k:
        assert np.array_equal(gpu_row, ridx)
        return 0
    # map token ids to positions in I (flat: the id itself; candidate mode: its slot)
    if cand_ids is None:
        pos_of = lambda ids: ids
    else:
        c = np.asarray(cand_ids)
        slot = {int(t): i for i, t in enumerate(c) if t >= 0}
        pos_of = lambda ids: np.array([slot[int(t)] for t in ids], np.int64)
    g_dyn = np.asarray(gpu_row[S + W:])
    r_dyn = ridx[S + W:]
    g_dyn, r_dyn = g_dyn[g_dyn >= 0], r_dyn[r_dyn >= 0]
    if np.array_equal(np.sort(g_dyn), np.sort(r_dyn)):
        nt.add(g_dyn, r_dyn, {}, 0.0, 0.0)
        return 0
    pg, pr = pos_of(g_dyn), pos_of(r_dyn)
    kpos = pr[np.argmin(I[pr])]
    ref_score = {int(t): I[int(p)] for t, p in zip(np.concatenate([g_dyn, r_dyn]),
                                                     np.concatenate([pg, pr]))}
    return nt.add(g_dyn, r_dyn, ref_score, I[kpos], score_tol(A[kpos], E[kpos]))


def check_rows_exact(gpu_idx, scores32, V, k, S, W, cand_ids=None):
    """GPU selection of whole rows vs ref.select on the same fp32 scores: bit-exact, plus the
    sink | window | dynamic layout of every row."""
    want = ref.select(scores32, V, k, S, W, cand_ids=cand_ids)
    assert np.array_equal(gpu_idx, want)
    for r in range(gpu_idx.shape[0]):
        check_si_layout(gpu_idx[r], int(V[r]), k, S, W,
                        None if cand_ids is None else cand_ids[r])


def hi_case(w, b, inp, pk, res, nt_pages: NearTie, check_cands=True, t=0):
    """GPU page recall of query t of sequence b against the oracle: recalled pages equal up to
    near-ties in the coarse scores; candidate ids follow the GPU's own recalled pages exactly;
    candidate scores within the score tolerance.  Returns the oracle's result."""
    s, bud, hi = w.index, w.budget, w.hi
    keys, scale = keys_np(inp, b)
    q = bits(inp["q"][b, t:t + 1])
    wt = f32(inp["w"][b, t:t + 1])
    pkn = bits(pk[b])
    pos = s.q_pos0 + t
    r = ref.page_recall(q, wt, pkn, keys, scale, np.array([pos]), bud.k, bud.sink,
                        bud.window, hi.page, hi.m_pages)
    gp = res[0][b, t].cpu().numpy()
    rp = r["page_ids"][0]
    coarse = r["coarse"][0]
    # recalled ids ascending, -1 padded, unique
    n = int((gp >= 0).sum())
    assert np.all(gp[n:] == -1) and np.all(np.diff(gp[:n]) > 0)
    if np.array_equal(gp, rp):
        nt_pages.add(gp, rp, {}, 0.0, 0.0)
    else:
        sel = rp[rp >= 0]
        kth = sel[np.argmin(coarse[sel])]
        # coarse error scale: fp32 accumulation over H*d products of page keys
        _, Ac, Ec = ref.index_scores(q, wt, pkn, None, np.array([len(pkn)]))
        nt_pages.add(gp, rp, coarse, coarse[kth], score_tol(Ac[0][kth], Ec[0][kth]))
    if check_cands:
        gi = res[2][b, t].cpu().numpy()
        gs = res[1][b, t].cpu().numpy()
        ok = gi >= 0
        P = hi.page
        V = min(s.kv_len, pos + 1)
        for i, p in enumerate(gp):
            seg = gi[i * P:(i + 1) * P]
            if p < 0:
                assert np.all(seg == -1)
                continue
            tok = p * P + np.arange(P)
            inmid = (tok >= bud.sink) & (tok < V - bud.window)
            assert np.array_equal(seg, np.where(inmid, tok, -1))
        if ok.any():
            tok = gi[ok]
            sub_scale = None if scale is None else scale[tok]
            I, A, E = ref.index_scores(q, wt, keys[tok], sub_scale, np.array([len(tok) - 1]))
            assert_scores(gs[ok], I[0], A[0], E[0], "fine")
        assert np.all(np.isneginf(gs[~ok]))
    return r


def attn_check(q, kv, v, idx, scale, out, lse, latent, d_v, rows=None, seqs=None, tol=2e-2):
    """GPU attention outputs of the given (sequence, query) rows against the fp64 oracle over
    the same index lists.  Only the rows the list names are copied to the host (kept in their
    order, the list remapped onto them): the kernel itself read them in place in HBM."""
    idn = idx.cpu().numpy()
    o = bits(out)
    B, T = q.shape[0], q.shape[1]
    L = kv.shape[1]
    worst = 0.0
    for b in (range(B) if seqs is None else seqs):
        for t in (range(T) if rows is None else rows):
            ids = idn[b, t]
            ok = (ids >= 0) & (ids < L)
            uniq = np.unique(ids[ok])
            local = np.full_like(ids, -1)
            local[ok] = np.searchsorted(uniq, ids[ok])
            sel = torch.from_numpy(uniq.astype(np.int64)).to(kv.device)
            kn = bits(kv[b].index_select(0, sel)) if len(uniq) else np.zeros((1, kv.shape[2]),
                                                                              np.uint16)
            vn = kn if latent else (bits(v[b].index_select(0, sel)) if len(uniq)
                                    else np.zeros((1, v.shape[2]), np.uint16))
            ro, rl = ref.sparse_attn(bits(q[b, t])[None], kn, vn, local[None], scale,
                                     d_qk=q.shape[3], d_v=d_v)
            go = (o[b, t].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            err = np.abs(go - ro[0]).max()
            worst = max(worst, err)
            assert err <= tol, (b, t, err)
            if lse is not None:
                gl = lse[b, t].cpu().numpy().astype(np.float64)
                fin = np.isfinite(rl[0])
                assert np.array_equal(fin, np.isfinite(gl))
                if fin.any():
                    assert np.abs(gl[fin] - rl[0][fin]).max() <= 1e-3 * max(1.0, np.abs(rl[0][fin]).max())
    return worst
