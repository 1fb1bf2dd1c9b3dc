"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Bars: index lists and page keys bit-exact; scores within 1e-3 relative (error scale
max(A, E/100), tests/util.py); attention within 2e-2 max-abs of the fp64 oracle (bf16 output).
Where fp32 score rounding can flip a near-tie, selections are compared with the near-tie rule.
Small cases span several tiles with ragged tails; the full-size workloads are checked on sampled
rows, in the same launch configuration the bench uses (same shapes, same entry points).
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import ref
from token_selection_indexer_amd import inputs, lsa
from token_selection_indexer_amd.configs import (DECODE_128K, DECODE_1M_HI, DECODE_256K_HI_CLI,
                                                 PREFILL_8K_AT_128K, TINY_PREFILL_4K, Budget,
                                                 HiParams, IndexShape, Workload, shrink)
from tests.util import bits, check_near_tie_sets, f32, keys_np, score_tol, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lsa.lib()  # fail loudly if the HIP library is missing
    yield
    torch.cuda.synchronize()


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


# ------------------------------------------------------------------------------ scores
def test_fp8_decode_all_codes_exact():
    """Every finite e4m3fn code through the scoring kernel: with q[h0] = e_0, q[h1] = -e_0 and
    w = (1, -1, 0, ...) the score is exactly the key's element 0, i.e. the decoded code."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    L, d, H = len(codes), 64, 4
    keys = np.zeros((1, L, d), np.uint8)
    keys[0, :, 0] = codes
    keys[0, :, 1:] = 0x38  # 1.0 elsewhere (ignored by the one-hot query)
    qf = np.zeros((1, 1, H, d), np.float32)
    qf[0, 0, 0, 0], qf[0, 0, 1, 0] = 1.0, -1.0
    q = torch.from_numpy(qf).to(torch.bfloat16).to(DEV)
    w = torch.tensor([[[1.0, -1.0, 0.0, 0.0]]], device=DEV)
    kt = torch.from_numpy(keys).to(DEV)
    scale = torch.ones((1, L), device=DEV)
    s = lsa.index_scores(q, w, kt, scale, q_pos0=L - 1).cpu().numpy()[0, 0]
    expect = np.array([ref.e4m3fn_to_double(c) for c in codes])
    assert np.array_equal(s.astype(np.float64), expect)


@pytest.mark.parametrize("H,d,kd", [(64, 128, "fp8"), (64, 128, "bf16"), (4, 64, "bf16"),
                                    (8, 64, "fp8"), (16, 128, "bf16"), (32, 64, "bf16")])
@pytest.mark.parametrize("n_q", [1, 3, 37])
def test_scores_small_ragged(H, d, kd, n_q):
    L = 1000  # not a multiple of the 32-key block or the 64-key tile
    w = Workload(name="t", index=IndexShape(
        batch=2, n_q=n_q, kv_len=L, q_pos0=L - n_q - 5, heads=H, head_dim=d, key_dtype=kd),
        budget=TINY_PREFILL_4K.budget, attn=TINY_PREFILL_4K.attn, seed=11)
    inp = inputs.index_inputs(w, DEV)
    s = lsa.index_scores(inp["q"], inp["w"], inp["keys"], inp["scale"], q_pos0=w.index.q_pos0)
    s = s.cpu().numpy()
    for b in range(2):
        I, A, E = oracle_scores(inp, b, np.arange(n_q), w.index.q_pos0)
        assert_scores(s[b], I, A, E, f"b={b}")


def test_scores_tiny_prefill_full():
    w = TINY_PREFILL_4K
    inp = inputs.index_inputs(w, DEV)
    s = lsa.index_scores(inp["q"], inp["w"], inp["keys"], None, q_pos0=0).cpu().numpy()
    I, A, E = oracle_scores(inp, 0, np.arange(4096), 0)
    assert_scores(s[0], I, A, E, "tiny prefill")


def test_scores_decode_128k_sampled():
    """Full decode workload (32 x 128K fp8 keys); the oracle checks whole rows of 3 sequences."""
    w = DECODE_128K
    inp = inputs.index_inputs(w, DEV)
    s = lsa.index_scores(inp["q"], inp["w"], inp["keys"], inp["scale"], q_pos0=w.index.q_pos0)
    torch.cuda.synchronize()
    for b in (0, 17, 31):
        I, A, E = oracle_scores(inp, b, [0], w.index.q_pos0)
        assert_scores(s[b, 0].cpu().numpy(), I[0], A[0], E[0], f"seq {b}")
        say(f"decode_128k seq {b} ok")


@pytest.mark.parametrize("back", [1, 1000])
def test_scores_long_launch_ragged(back):
    """A long decode launch (one round of workgroups, each wave looping over ~64 blocks) whose key
    count is not a multiple of the 32-key block: the last block is moved back to end at the last
    key and rewrites its overlap with the previous block.  Whole rows of three sequences against
    the oracle; back = 1000 also cuts the causal range short of the end."""
    L = 131072 - 5
    w = shrink(DECODE_128K, batch=17, kv_len=L, q_pos0=L - back)
    inp = inputs.index_inputs(w, DEV)
    s = lsa.index_scores(inp["q"], inp["w"], inp["keys"], inp["scale"], q_pos0=w.index.q_pos0)
    torch.cuda.synchronize()
    for b in (0, 8, 16):
        I, A, E = oracle_scores(inp, b, [0], w.index.q_pos0)
        assert_scores(s[b, 0].cpu().numpy(), I[0], A[0], E[0], f"seq {b}")
        say(f"long ragged launch (back {back}) seq {b} ok")


def test_scores_prefill_8k_sampled():
    """Full chunked-prefill workload (8192 queries x 128K bf16 keys, 4.3 GB of scores); the
    oracle checks whole rows at the first, a middle and the last query."""
    w = PREFILL_8K_AT_128K
    inp = inputs.index_inputs(w, DEV)
    s = lsa.index_scores(inp["q"], inp["w"], inp["keys"], None, q_pos0=w.index.q_pos0)
    torch.cuda.synchronize()
    rows = [0, 4097, 8191]
    I, A, E = oracle_scores(inp, 0, rows, w.index.q_pos0)
    for i, t in enumerate(rows):
        assert_scores(s[0, t].cpu().numpy(), I[i], A[i], E[i], f"row {t}")
    del s
    torch.cuda.empty_cache()


# ------------------------------------------------------------------------------ selection
@pytest.mark.parametrize("ties", ["none", "zeros", "coarse", "const", "inf"])
def test_select_flat_exact(ties):
    rows, L = 40, 3001
    k, S, W = 96, 8, 40
    sc = inputs.synthetic_scores(rows, L, seed=5, ties=ties, device=DEV).reshape(4, 10, L)
    for pos0 in (0, 90, L - 10):  # rows with V <= k, rows just past k, full rows
        idx = lsa.topk_select(sc, k, S, W, kv_len=L, q_pos0=pos0).cpu().numpy()
        V = ref.valid_lengths(L, pos0, 10)
        for b in range(4):
            expect = ref.select(sc[b].cpu().numpy(), V, k, S, W)
            assert np.array_equal(idx[b], expect), (ties, pos0, b)


def test_select_candidate_mode_exact():
    rows, n = 12, 2048
    k, S, W = 256, 16, 112
    sc = inputs.synthetic_scores(rows, n, seed=6, ties="coarse", device=DEV).reshape(3, 4, n)
    g = torch.Generator().manual_seed(0)
    ids = torch.stack([torch.randperm(20000, generator=g)[:n] for _ in range(rows)])
    ids = torch.sort(ids.reshape(3, 4, n), -1).values.to(torch.int32)
    ids[:, :, ::7] = -1  # holes
    ids[0, 0, 100:] = -1  # a row with fewer candidates than the dynamic budget
    idx = lsa.topk_select(sc, k, S, W, kv_len=30000, q_pos0=30000 - 4,
                          cand_ids=ids.to(DEV)).cpu().numpy()
    V = ref.valid_lengths(30000, 30000 - 4, 4)
    for b in range(3):
        expect = ref.select(sc[b].cpu().numpy(), V, k, S, W, cand_ids=ids[b].numpy())
        assert np.array_equal(idx[b], expect), b


@pytest.mark.parametrize("k,S,W", [(64, 0, 0), (64, 32, 32), (2048, 64, 960), (5000, 100, 100)])
def test_select_budget_edges(k, S, W):
    L = 4500
    sc = inputs.synthetic_scores(3, L, seed=7, ties="zeros", device=DEV).reshape(1, 3, L)
    idx = lsa.topk_select(sc, k, S, W, kv_len=L, q_pos0=L - 3).cpu().numpy()
    expect = ref.select(sc[0].cpu().numpy(), ref.valid_lengths(L, L - 3, 3), k, S, W)
    assert np.array_equal(idx[0], expect)


def test_select_decode_128k_full_exact():
    """Selection at the decode workload's full shape (32 rows x 131072) on synthetic scores with
    exact zeros; every row checked."""
    w = DECODE_128K
    L, b = w.index.kv_len, w.budget
    sc = inputs.synthetic_scores(32, L, seed=8, ties="zeros", device=DEV).reshape(32, 1, L)
    idx = lsa.topk_select(sc, b.k, b.sink, b.window, kv_len=L, q_pos0=L - 1).cpu().numpy()
    scn = sc.cpu().numpy()
    for r in range(32):
        expect = ref.select(scn[r], np.array([L]), b.k, b.sink, b.window)
        assert np.array_equal(idx[r], expect), r


@pytest.mark.parametrize("ties", ["none", "zeros", "coarse", "const", "ramp", "inf"])
def test_select_sampled_rows_exact(ties):
    """Rows longer than the LDS buffer on the one-workgroup path: the sampled threshold and its
    fallbacks (heavy ties: too many elements reach the threshold; "ramp": every pick in the last
    wave's segment, whose list overflows, so an ordered pass collects them)."""
    B, T, L = 3, 4, 20000
    k, S, W = 2048, 64, 960
    sc = inputs.synthetic_scores(B * T, L, seed=13, ties=ties, device=DEV).reshape(B, T, L)
    for pos0 in (L - T, 9000):
        idx = lsa.topk_select(sc, k, S, W, kv_len=L, q_pos0=pos0).cpu().numpy()
        V = ref.valid_lengths(L, pos0, T)
        for b in range(B):
            expect = ref.select(sc[b].cpu().numpy(), V, k, S, W)
            assert np.array_equal(idx[b], expect), (ties, pos0, b)


@pytest.mark.parametrize("ties", ["none", "zeros", "coarse", "const", "ramp", "inf"])
def test_select_chunked_rows_exact(ties):
    """Few long rows (the chunked path), every tie pattern: heavy ties overflow the per-chunk
    slices and fall back to one workgroup per row; rows with V <= k take everything."""
    B, T, L = 2, 3, 40000
    k, S, W = 2048, 64, 960
    sc = inputs.synthetic_scores(B * T, L, seed=10, ties=ties, device=DEV).reshape(B, T, L)
    for pos0 in (L - T, 2046, 0):
        idx = lsa.topk_select(sc, k, S, W, kv_len=L, q_pos0=pos0).cpu().numpy()
        V = ref.valid_lengths(L, pos0, T)
        for b in range(B):
            expect = ref.select(sc[b].cpu().numpy(), V, k, S, W)
            assert np.array_equal(idx[b], expect), (ties, pos0, b)


def test_select_chunked_candidate_mode_exact():
    B, n = 4, 16384
    k, S, W = 2048, 128, 896
    sc = inputs.synthetic_scores(B, n, seed=11, ties="coarse", device=DEV).reshape(B, 1, n)
    g = torch.Generator().manual_seed(1)
    ids = torch.stack([torch.sort(torch.randperm(1 << 20, generator=g)[:n]).values for _ in range(B)])
    ids = ids.to(torch.int32).reshape(B, 1, n)
    ids[:, :, 3::5] = -1
    ids[1, 0, 900:] = -1  # fewer candidates than the dynamic budget
    idx = lsa.topk_select(sc, k, S, W, kv_len=1 << 20, q_pos0=(1 << 20) - 1,
                          cand_ids=ids.to(DEV)).cpu().numpy()
    for b in range(B):
        expect = ref.select(sc[b].cpu().numpy(), np.array([1 << 20]), k, S, W,
                            cand_ids=ids[b].numpy())
        assert np.array_equal(idx[b], expect), b


def test_select_prefill_rows_sampled():
    """Selection rows at the chunked-prefill shape (8192 rows x 131072); sampled rows checked."""
    w = PREFILL_8K_AT_128K
    L, b, T = w.index.kv_len, w.budget, 1024  # 1024 of the 8192 rows, same row length
    sc = inputs.synthetic_scores(T, L, seed=9, device=DEV).reshape(1, T, L)
    pos0 = w.index.q_pos0 + 8192 - T
    idx = lsa.topk_select(sc, b.k, b.sink, b.window, kv_len=L, q_pos0=pos0).cpu().numpy()
    rows = [0, 511, 1023]
    V = ref.valid_lengths(L, pos0, T)[rows]
    expect = ref.select(sc[0, rows].cpu().numpy(), V, b.k, b.sink, b.window)
    assert np.array_equal(idx[0, rows], expect)


def test_tiny_prefill_end_to_end_selection():
    """GPU scores -> GPU selection vs oracle scores (fp64, decided in fp32) -> oracle selection:
    equal up to near-ties."""
    w = TINY_PREFILL_4K
    b = w.budget
    inp = inputs.index_inputs(w, DEV)
    s = lsa.index_scores(inp["q"], inp["w"], inp["keys"], None, q_pos0=0)
    idx = lsa.topk_select(s, b.k, b.sink, b.window, kv_len=4096, q_pos0=0).cpu().numpy()[0]
    I, A, E = oracle_scores(inp, 0, np.arange(4096), 0)
    V = ref.valid_lengths(4096, 0, 4096)
    ridx = ref.select(I.astype(np.float32), V, b.k, b.sink, b.window)
    mism = 0
    for t in range(4096):
        if np.array_equal(idx[t], ridx[t]):
            continue
        dyn = ridx[t][b.sink + b.window:]
        kth = dyn[np.argmin(I[t][dyn])]
        _, nd = check_near_tie_sets(idx[t], ridx[t], I[t], I[t][kth],
                                    score_tol(A[t][kth], E[t][kth]), min_recall=0.99)
        mism += nd
    total = 4096 * b.dynamic
    assert mism / total < 1e-3


# ------------------------------------------------------------------------------ page keys
@pytest.mark.parametrize("kd,P,L,d", [
    ("fp8", 64, 5000, 128), ("bf16", 64, 4096, 128), ("fp8", 32, 999, 128), ("bf16", 256, 1300, 128),
    ("fp8", 1, 77, 128), ("fp8", 8, 1000, 128), ("bf16", 4, 333, 128), ("bf16", 2, 301, 128),
    ("fp8", 256, 3000, 128), ("fp8", 16, 1000, 64), ("bf16", 8, 700, 64), ("fp8", 128, 2000, 64),
    ("fp8", 4, 500, 64)])
def test_page_summary_bit_exact(kd, P, L, d):
    """Pages of at least one 16-byte piece per lane group take the one-wave-per-page kernel,
    smaller pages the per-element one; both must give the oracle's bits, partial last page
    included."""
    w = Workload(name="p", index=IndexShape(
        batch=2, n_q=1, kv_len=L, q_pos0=L - 1, heads=64, head_dim=d, key_dtype=kd),
        budget=TINY_PREFILL_4K.budget, attn=TINY_PREFILL_4K.attn, seed=12)
    inp = inputs.index_inputs(w, DEV)
    pk = lsa.page_summary(inp["keys"], inp["scale"], P)
    got = bits(pk)
    for b in range(2):
        keys, scale = keys_np(inp, b)
        assert np.array_equal(got[b], ref.page_keys(keys, scale, P)), b
    # a sub-range is rewritten alone
    n_pages = (L + P - 1) // P
    pk2 = torch.zeros_like(pk)
    lo, hi = n_pages // 3, n_pages // 3 + max(1, n_pages // 4)
    lsa.page_summary(inp["keys"], inp["scale"], P, lo, hi, out=pk2)
    g2 = bits(pk2)
    assert np.array_equal(g2[:, lo:hi], got[:, lo:hi])
    assert not g2[:, :lo].any() and not g2[:, hi:].any()


# ------------------------------------------------------------------------------ HI recall
def _hi_case(w: Workload, b: int, inp, pk, res, check_cands=True, t=0):
    """Compare GPU page recall of query t of sequence b with the oracle."""
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
    if not np.array_equal(gp, rp):
        # near-ties in the coarse scores only
        sel = rp[rp >= 0]
        kth = sel[np.argmin(coarse[sel])]
        # coarse error scale: fp32 accumulation over H*d products of page keys
        Ic, Ac, Ec = ref.index_scores(q, wt, pkn, None, np.array([len(pkn)]))
        check_near_tie_sets(gp, rp, coarse, coarse[kth], score_tol(Ac[0][kth], Ec[0][kth]),
                            min_recall=0.99)
    if check_cands:
        # candidates: ids follow the GPU's own recalled pages; scores checked against the oracle
        gi = res[2][b, t].cpu().numpy()
        gs = res[1][b, t].cpu().numpy()
        ok = gi >= 0
        P = hi.page
        for i, p in enumerate(gp):
            seg = gi[i * P:(i + 1) * P]
            if p < 0:
                assert np.all(seg == -1)
                continue
            tok = p * P + np.arange(P)
            V = min(s.kv_len, pos + 1)
            inmid = (tok >= bud.sink) & (tok < V - bud.window)
            assert np.array_equal(seg, np.where(inmid, tok, -1))
        if ok.any():
            tok = gi[ok]
            sub_scale = None if scale is None else scale[tok]
            I, A, E = ref.index_scores(q, wt, keys[tok], sub_scale, np.array([len(tok) - 1]))
            assert_scores(gs[ok], I[0], A[0], E[0], "fine")
        assert np.all(np.isneginf(gs[~ok]))
    return r


def test_page_recall_small():
    w = Workload(name="hi", index=IndexShape(
        batch=3, n_q=1, kv_len=9000, q_pos0=8999, heads=64, head_dim=128, key_dtype="fp8"),
        budget=Budget(k=512, sink=32, window=224), attn=DECODE_1M_HI.attn, seed=13,
        hi=HiParams(page=64, m_pages=16), planted_frac=0.05)
    inp = inputs.index_inputs(w, DEV)
    pk = lsa.page_summary(inp["keys"], inp["scale"], 64)
    res = lsa.page_recall(inp["q"], inp["w"], pk, inp["keys"], inp["scale"], 512, 32, 224, 64, 16,
                          q_pos0=8999)
    for b in range(3):
        _hi_case(w, b, inp, pk, res)


def test_page_recall_causal_prefill():
    """Hierarchical Indexing for a causal chunk of queries: every query has its own valid length,
    so its own eligible pages and candidates.  The first rows have V <= k (nothing recalled);
    the window covers at least one page (W >= P - 1).  Recall and candidates of sampled rows are
    checked against the oracle, and the candidate-mode selection of every row against the
    oracle's selection over the GPU's own candidate list."""
    L, T, P, M, k, S, W = 5000, 300, 32, 8, 512, 32, 96
    pos0 = 400  # the last row sees 700 keys: 19 eligible pages, 8 recalled
    w = Workload(name="hi_prefill", index=IndexShape(
        batch=2, n_q=T, kv_len=L, q_pos0=pos0, heads=64, head_dim=128, key_dtype="fp8"),
        budget=Budget(k=k, sink=S, window=W), attn=DECODE_1M_HI.attn, seed=21,
        hi=HiParams(page=P, m_pages=M), planted_frac=0.05)
    inp = inputs.index_inputs(w, DEV)
    pk = lsa.page_summary(inp["keys"], inp["scale"], P)
    res = lsa.page_recall(inp["q"], inp["w"], pk, inp["keys"], inp["scale"], k, S, W, P, M,
                          q_pos0=pos0)
    idx = lsa.topk_select(res[1], k, S, W, kv_len=L, q_pos0=pos0, cand_ids=res[2])
    torch.cuda.synchronize()
    n_small = k - pos0  # rows with V <= k
    assert 0 < n_small < T
    pid = res[0].cpu().numpy()
    assert np.all(pid[:, :n_small] == -1)
    assert np.all(res[2][:, :n_small].cpu().numpy() == -1)
    for b in range(2):
        for t in (n_small, n_small + 1, 201, T - 1):
            _hi_case(w, b, inp, pk, res, t=t)
    cs, ci, gi = res[1].cpu().numpy(), res[2].cpu().numpy(), idx.cpu().numpy()
    V = ref.valid_lengths(L, pos0, T)
    for b in range(2):
        want = ref.select(cs[b], V, k, S, W, cand_ids=ci[b])
        assert np.array_equal(gi[b], want), b


def test_hi_all_pages_equals_flat_on_gpu():
    """M * P >= L: Hierarchical Indexing selects exactly what flat selection does (GPU vs GPU
    and vs the oracle's flat selection up to near-ties)."""
    L, P, k, S, W = 6000, 64, 512, 32, 224
    M = (L + P - 1) // P
    w = Workload(name="hi2", index=IndexShape(
        batch=2, n_q=1, kv_len=L, q_pos0=L - 1, heads=64, head_dim=128, key_dtype="fp8"),
        budget=Budget(k=k, sink=S, window=W), attn=DECODE_1M_HI.attn, seed=14)
    inp = inputs.index_inputs(w, DEV)
    pk = lsa.page_summary(inp["keys"], inp["scale"], P)
    pid, cs, ci = lsa.page_recall(inp["q"], inp["w"], pk, inp["keys"], inp["scale"], k, S, W, P, M,
                                  q_pos0=L - 1)
    hi_idx = lsa.topk_select(cs, k, S, W, kv_len=L, q_pos0=L - 1, cand_ids=ci)
    s = lsa.index_scores(inp["q"], inp["w"], inp["keys"], inp["scale"], q_pos0=L - 1)
    flat_idx = lsa.topk_select(s, k, S, W, kv_len=L, q_pos0=L - 1)
    assert torch.equal(hi_idx, flat_idx)


def test_page_recall_decode_1m_sampled():
    """Full long-context workload: 4 x 1M fp8 keys, P=64, M=256; page keys, recall and
    candidates of two sequences checked; planted pages reported."""
    w = DECODE_1M_HI
    s, bud, hi = w.index, w.budget, w.hi
    inp = inputs.index_inputs(w, DEV)
    pk = lsa.page_summary(inp["keys"], inp["scale"], hi.page)
    res = lsa.page_recall(inp["q"], inp["w"], pk, inp["keys"], inp["scale"], bud.k, bud.sink,
                          bud.window, hi.page, hi.m_pages, q_pos0=s.q_pos0)
    torch.cuda.synchronize()
    for b in (0, 3):
        keys, scale = keys_np(inp, b)
        assert np.array_equal(bits(pk[b]), ref.page_keys(keys, scale, hi.page)), b
        _hi_case(w, b, inp, pk, res)
        planted = inputs.planted_pages(w, b, DEV).cpu().numpy()
        got = res[0][b, 0].cpu().numpy()
        say(f"decode_1m seq {b}: planted pages recalled {np.isin(planted, got).sum()}/{len(planted)}")


# ------------------------------------------------------------------------------ attention
def _attn_check(q, kv, v, idx, scale, out, lse, latent, d_v, rows=None, tol=2e-2):
    qn, kvn = bits(q), bits(kv)
    vn = kvn if latent else bits(v)
    idn = idx.cpu().numpy()
    o = bits(out).view(np.uint16)
    B, T = q.shape[0], q.shape[1]
    for b in range(B):
        rs = range(T) if rows is None else rows
        for t in rs:
            ro, rl = ref.sparse_attn(qn[b, t][None], kvn[b], vn[b], idn[b, t][None], scale,
                                     d_qk=q.shape[3], d_v=d_v)
            go = (o[b, t].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            assert np.abs(go - ro[0]).max() <= tol, (b, t, np.abs(go - ro[0]).max())
            if lse is not None:
                gl = lse[b, t].cpu().numpy().astype(np.float64)
                fin = np.isfinite(rl[0])
                assert np.array_equal(fin, np.isfinite(gl))
                assert np.abs(gl[fin] - rl[0][fin]).max() <= 1e-3 * max(1.0, np.abs(rl[0][fin]).max())


@pytest.mark.parametrize("B,T,k,L", [(2, 3, 2048, 9000), (1, 40, 300, 5000), (3, 1, 77, 500)])
def test_mla_attn_small(B, T, k, L):
    w = Workload(name="a", index=IndexShape(
        batch=B, n_q=T, kv_len=L, q_pos0=L - T, heads=64, head_dim=128, key_dtype="fp8"),
        budget=DECODE_128K.budget, attn=DECODE_128K.attn, seed=15)
    att = inputs.attn_inputs(w, 0, DEV)
    S, W = min(64, k // 4), min(200, k // 4)
    V = ref.valid_lengths(L, L - T, T)
    idx = torch.stack([inputs.synthetic_index_lists(T, k, S, W, V, seed=20 + b)
                       for b in range(B)]).to(DEV)
    if T > 1:
        idx[0, 0, 5:9] = -1  # holes inside a row
    out, lse = lsa.sparse_attn(att["q"], att["kv"], None, idx, w.attn.scale, S, W, d_v=512)
    _attn_check(att["q"], att["kv"], None, idx, w.attn.scale, out, lse, True, 512)


def test_mla_attn_empty_and_single_rows():
    L, k = 1000, 128
    w = shrink(DECODE_128K, batch=1, n_q=3, kv_len=L, q_pos0=L - 3)
    att = inputs.attn_inputs(w, 0, DEV)
    idx = torch.full((1, 3, k), -1, dtype=torch.int32)
    idx[0, 1, 77] = 432
    idx[0, 2, :] = torch.arange(k, dtype=torch.int32) * 7
    idx[0, 2, 3] = L + 5  # out of range: skipped like -1
    idx = idx.to(DEV)
    out, lse = lsa.sparse_attn(att["q"], att["kv"], None, idx, w.attn.scale, d_v=512)
    o = out.float().cpu()
    assert torch.all(o[0, 0] == 0) and torch.all(torch.isneginf(lse[0, 0].cpu()))
    row = att["kv"][0, 432, :512].float().cpu()
    assert torch.equal(o[0, 1], row.expand(16, 512))
    idx2 = idx.clone()
    idx2[0, 2, 3] = -1
    out2, _ = lsa.sparse_attn(att["q"], att["kv"], None, idx2, w.attn.scale, d_v=512)
    assert torch.equal(out2[0, 2], out[0, 2])


def test_mha_attn_tiny_prefill_with_oracle_indices():
    """Single-head d=128 attention of the tiny prefill workload over the oracle's own index
    lists (sampled rows, including rows with V <= k)."""
    w = TINY_PREFILL_4K
    b = w.budget
    inp = inputs.index_inputs(w, "cpu")
    I, _, _ = ref.index_scores(bits(inp["q"][0]), f32(inp["w"][0]), bits(inp["keys"][0]), None,
                               np.arange(4096))
    ridx = ref.select(I.astype(np.float32), ref.valid_lengths(4096, 0, 4096), b.k, b.sink,
                      b.window)
    att = inputs.attn_inputs(w, 0, DEV)
    idx = torch.from_numpy(ridx)[None].to(DEV)
    out, lse = lsa.sparse_attn(att["q"], att["k"], att["v"], idx, w.attn.scale, b.sink, b.window)
    rows = list(range(0, 4096, 97)) + [4095]
    _attn_check(att["q"], att["k"], att["v"], idx, w.attn.scale, out, lse, False, 128, rows=rows)


def test_mla_attn_decode_128k_sampled():
    w = DECODE_128K
    b = w.budget
    att = inputs.attn_inputs(w, 0, DEV)
    V = [w.index.kv_len] * w.index.n_q
    idx = torch.stack([inputs.synthetic_index_lists(1, b.k, b.sink, b.window, V, seed=30 + i)
                       for i in range(w.index.batch)]).to(DEV)
    out, lse = lsa.sparse_attn(att["q"], att["kv"], None, idx, w.attn.scale, b.sink, b.window,
                               d_v=512)
    torch.cuda.synchronize()
    for s in (0, 31):
        _attn_check(att["q"][s:s + 1], att["kv"][s:s + 1], None, idx[s:s + 1], w.attn.scale,
                    out[s:s + 1], lse[s:s + 1], True, 512)


@pytest.mark.parametrize("L", [1, 2, 5, 31, 33, 100])
def test_degenerate_lengths_end_to_end(L):
    """Caches shorter than one 32-key block, than the budget, or than sink plus window: scores,
    selection and MLA attention of a short causal chunk against the oracle."""
    T = min(3, L)
    k, S, W = 16, 2, 4
    w = Workload(name="deg", index=IndexShape(
        batch=2, n_q=T, kv_len=L, q_pos0=L - T, heads=64, head_dim=128, key_dtype="fp8"),
        budget=Budget(k=k, sink=S, window=W), attn=DECODE_128K.attn, seed=30 + L)
    inp = inputs.index_inputs(w, DEV)
    sc = lsa.index_scores(inp["q"], inp["w"], inp["keys"], inp["scale"], q_pos0=L - T)
    idx = lsa.topk_select(sc, k, S, W, kv_len=L, q_pos0=L - T)
    sn, gi = sc.cpu().numpy(), idx.cpu().numpy()
    V = ref.valid_lengths(L, L - T, T)
    for b in range(2):
        I, A, E = oracle_scores(inp, b, np.arange(T), L - T)
        assert_scores(sn[b], I, A, E, f"b={b}")
        assert np.array_equal(gi[b], ref.select(sn[b], V, k, S, W)), b
    att = inputs.attn_inputs(w, 0, DEV)
    out, lse = lsa.sparse_attn(att["q"], att["kv"], None, idx, w.attn.scale, S, W, d_v=512)
    _attn_check(att["q"], att["kv"], None, idx, w.attn.scale, out, lse, True, 512)


def test_cross_layer_reuse_bitwise_and_oracle():
    """One index list, four layers: each layer's output equals that layer's single call
    bitwise, and matches the oracle."""
    w = shrink(DECODE_256K_HI_CLI, batch=2, kv_len=20000, q_pos0=19999)
    b = w.budget
    idx = torch.stack([inputs.synthetic_index_lists(1, b.k, b.sink, b.window, [20000], seed=40 + i)
                       for i in range(2)]).to(DEV)
    outs = []
    for layer in range(w.layers):
        att = inputs.attn_inputs(w, layer, DEV)
        o1, l1 = lsa.sparse_attn(att["q"], att["kv"], None, idx, w.attn.scale, b.sink, b.window,
                                 d_v=512)
        o2, l2 = lsa.sparse_attn(att["q"], att["kv"], None, idx, w.attn.scale, b.sink, b.window,
                                 d_v=512)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        _attn_check(att["q"], att["kv"], None, idx, w.attn.scale, o1, l1, True, 512)
        outs.append(o1)
    assert not torch.equal(outs[0], outs[1])


# ------------------------------------------------------------------------------ determinism
def test_determinism_decode_path():
    w = shrink(DECODE_128K, batch=4, kv_len=20000, q_pos0=19999)
    b = w.budget
    inp = inputs.index_inputs(w, DEV)
    r1 = lsa.index_scores(inp["q"], inp["w"], inp["keys"], inp["scale"], q_pos0=19999)
    r2 = lsa.index_scores(inp["q"], inp["w"], inp["keys"], inp["scale"], q_pos0=19999)
    assert torch.equal(r1, r2)
    i1 = lsa.topk_select(r1, b.k, b.sink, b.window, kv_len=20000, q_pos0=19999)
    i2 = lsa.topk_select(r2, b.k, b.sink, b.window, kv_len=20000, q_pos0=19999)
    assert torch.equal(i1, i2)


def test_graph_replay_of_decode_step_matches_eager():
    """The decode step (scores -> chunked selection -> split MLA attention) captured in a HIP
    graph and replayed several times, with eager work and synchronisations in between: every
    replay's outputs equal the eager step's bit for bit."""
    w = shrink(DECODE_128K, batch=4, kv_len=40000)
    s, bud, a = w.index, w.budget, w.attn
    inp = inputs.index_inputs(w, DEV)
    att = inputs.attn_inputs(w, 0, DEV)
    B, L = s.batch, s.kv_len
    ws_sel, ws_att = lsa.Workspace(), lsa.Workspace()

    def run(scores, idx, out):
        lsa.index_scores(inp["q"], inp["w"], inp["keys"], inp["scale"], q_pos0=s.q_pos0, out=scores)
        lsa.topk_select(scores, bud.k, bud.sink, bud.window, kv_len=L, q_pos0=s.q_pos0, out=idx,
                        ws=ws_sel)
        lsa.sparse_attn(att["q"], att["kv"], None, idx, a.scale, bud.sink, bud.window, d_v=a.d_v,
                        ws=ws_att, out=out)

    def bufs():
        return (torch.empty((B, 1, L), dtype=torch.float32, device=DEV),
                torch.empty((B, 1, bud.k), dtype=torch.int32, device=DEV),
                torch.empty((B, 1, a.heads, a.d_v), dtype=torch.bfloat16, device=DEV))

    ref_b = bufs()
    run(*ref_b)
    torch.cuda.synchronize()
    g_b = bufs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(*g_b)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(*g_b)
    other = bufs()
    for rep in range(3):
        for t in g_b:
            t.zero_()
        graph.replay()
        run(*other)  # eager work between replays
        torch.cuda.synchronize()
        for got, ref_t in zip(g_b, ref_b):
            assert torch.equal(got.view(torch.int32) if got.dtype != torch.bfloat16 else got,
                               ref_t.view(torch.int32) if ref_t.dtype != torch.bfloat16 else ref_t), rep
        say(f"graph replay {rep} ok")
