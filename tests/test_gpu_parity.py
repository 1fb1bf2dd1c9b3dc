"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Bars: index lists and page keys bit-exact; scores within 1e-3 relative (error scale
max(A, E/100), tests/util.py); attention within 2e-2 max-abs of the fp64 oracle (bf16 output).
Where fp32 score rounding can flip a near-tie (a selection from the oracle's fp64 scores, or a
page recall), sets are compared with the near-tie rule: every mismatch's oracle score lies
within the score tolerance of the k-th, and recall over all rows checked is >= 99.9%.  Every
selected row is also checked for its layout (size, sink | window | ascending dynamic, -1 tail,
no duplicates).  Small cases span several tiles with ragged tails; tests/test_gpu_workloads.py
checks the five workloads at their own full shapes.
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
from tests.gpu_checks import (assert_scores, attn_check, hi_case, oracle_scores, say,
                              selection_vs_oracle_scores)
from tests.util import NearTie, bits, check_si_layout, f32, keys_np, score_tol, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lsa.lib()  # fail loudly if the HIP library is missing
    yield
    torch.cuda.synchronize()


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
def test_select_register_rows_exact(ties):
    """Flat rows past the LDS buffer but within 16 elements per thread of the one-workgroup path
    are read once into registers and histogrammed whole (heavy ties fall back to the streaming
    path).  Lengths around both limits; 12001 lacks 16-byte rows and 17500 is past the limit
    (the streaming paths); rows with V <= k and just past it."""
    B, T = 2, 3
    k, S, W = 2048, 64, 960
    for L in (9000, 12000, 12001, 16384, 17400, 17500):
        sc = inputs.synthetic_scores(B * T, L, seed=17, ties=ties, device=DEV).reshape(B, T, L)
        for pos0 in (L - T, 2046, 9000 - T):
            idx = lsa.topk_select(sc, k, S, W, kv_len=L, q_pos0=pos0).cpu().numpy()
            V = ref.valid_lengths(L, pos0, T)
            for b in range(B):
                expect = ref.select(sc[b].cpu().numpy(), V, k, S, W)
                assert np.array_equal(idx[b], expect), (ties, L, pos0, b)


@pytest.mark.parametrize("ties", ["coarse", "none", "const", "ramp", "inf"])
def test_select_hi_candidate_rows_exact(ties):
    """Candidate rows of Hierarchical Indexing's size (16384 candidates: past the LDS buffer,
    sampled on the one-workgroup path): holes, a row with fewer candidates than the dynamic
    budget, and every tie pattern's scores."""
    B, n = 3, 16384
    k, S, W = 2048, 64, 960
    sc = inputs.synthetic_scores(B, n, seed=19, ties=ties, device=DEV).reshape(B, 1, n)
    g = torch.Generator().manual_seed(2)
    ids = torch.stack([torch.sort(torch.randperm(1 << 20, generator=g)[:n]).values for _ in range(B)])
    ids = ids.to(torch.int32).reshape(B, 1, n)
    ids[:, :, 5::9] = -1
    ids[2, 0, 700:] = -1  # fewer candidates than the dynamic budget
    idx = lsa.topk_select(sc, k, S, W, kv_len=1 << 20, q_pos0=(1 << 20) - 1,
                          cand_ids=ids.to(DEV)).cpu().numpy()
    for b in range(B):
        expect = ref.select(sc[b].cpu().numpy(), np.array([1 << 20]), k, S, W,
                            cand_ids=ids[b].numpy())
        assert np.array_equal(idx[b], expect), b
        check_si_layout(idx[b, 0], 1 << 20, k, S, W, cand_ids=ids[b, 0].numpy())


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
    """Candidate rows long enough for the chunked path (few rows, at least 32768 candidates):
    holes, and a row with fewer candidates than the dynamic budget."""
    B, n = 4, 40000
    k, S, W = 2048, 128, 896
    sc = inputs.synthetic_scores(B, n, seed=11, ties="coarse", device=DEV).reshape(B, 1, n)
    g = torch.Generator().manual_seed(1)
    ids = torch.stack([torch.sort(torch.randperm(1 << 20, generator=g)[:n]).values for _ in range(B)])
    ids = ids.to(torch.int32).reshape(B, 1, n)
    ids[:, :, 3::5] = -1
    ids[1, 0, 900:] = -1  # fewer candidates than the dynamic budget
    idx = lsa.topk_select(sc, k, S, W, kv_len=1 << 20, q_pos0=(1 << 20) - 1,
                          cand_ids=ids.to(DEV)).cpu().numpy()
    assert lsa.lsa_workspace_bytes(lsa.OP_TOPK_SELECT, lsa.IndexShape(B, 1, 64, 128, 1 << 20, 0),
                                   lsa.Budget(k, S, W), n_cand=n) > 0  # the chunked path
    for b in range(B):
        expect = ref.select(sc[b].cpu().numpy(), np.array([1 << 20]), k, S, W,
                            cand_ids=ids[b].numpy())
        assert np.array_equal(idx[b], expect), b
        check_si_layout(idx[b, 0], 1 << 20, k, S, W, cand_ids=ids[b, 0].numpy())


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
    """GPU scores -> GPU selection of all 4096 rows vs the oracle's selection from its own fp64
    scores (decided in fp32): equal up to near-ties, recall >= 99.9% over all rows; and vs
    ref.select on the GPU's own fp32 scores: bit-exact, with the layout of every row."""
    w = TINY_PREFILL_4K
    b = w.budget
    inp = inputs.index_inputs(w, DEV)
    s = lsa.index_scores(inp["q"], inp["w"], inp["keys"], None, q_pos0=0)
    idx = lsa.topk_select(s, b.k, b.sink, b.window, kv_len=4096, q_pos0=0).cpu().numpy()[0]
    V = ref.valid_lengths(4096, 0, 4096)
    from tests.gpu_checks import check_rows_exact
    check_rows_exact(idx, s[0].cpu().numpy(), V, b.k, b.sink, b.window)
    I, A, E = oracle_scores(inp, 0, np.arange(4096), 0)
    nt = NearTie()
    for t in range(4096):
        selection_vs_oracle_scores(nt, idx[t], I[t], A[t], E[t], int(V[t]), b.k, b.sink,
                                   b.window)
    say(f"tiny prefill: recall {nt.recall:.6f}, {nt.mismatches} near-tie mismatches")
    nt.check(0.999)


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
def test_page_recall_small():
    w = Workload(name="hi", index=IndexShape(
        batch=3, n_q=1, kv_len=9000, q_pos0=8999, heads=64, head_dim=128, key_dtype="fp8"),
        budget=Budget(k=512, sink=32, window=224), attn=DECODE_1M_HI.attn, seed=13,
        hi=HiParams(page=64, m_pages=16), planted_frac=0.05)
    inp = inputs.index_inputs(w, DEV)
    pk = lsa.page_summary(inp["keys"], inp["scale"], 64)
    res = lsa.page_recall(inp["q"], inp["w"], pk, inp["keys"], inp["scale"], 512, 32, 224, 64, 16,
                          q_pos0=8999)
    nt = NearTie()
    for b in range(3):
        hi_case(w, b, inp, pk, res, nt)
    nt.check(0.999)


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
    nt = NearTie()
    for b in range(2):
        for t in (n_small, n_small + 1, 201, T - 1):
            hi_case(w, b, inp, pk, res, nt, t=t)
    nt.check(0.999)
    cs, ci, gi = res[1].cpu().numpy(), res[2].cpu().numpy(), idx.cpu().numpy()
    V = ref.valid_lengths(L, pos0, T)
    for b in range(2):
        want = ref.select(cs[b], V, k, S, W, cand_ids=ci[b])
        assert np.array_equal(gi[b], want), b
        for t in range(T):
            check_si_layout(gi[b, t], int(V[t]), k, S, W, cand_ids=ci[b, t])


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
    nt = NearTie()
    for b in (0, 3):
        keys, scale = keys_np(inp, b)
        assert np.array_equal(bits(pk[b]), ref.page_keys(keys, scale, hi.page)), b
        hi_case(w, b, inp, pk, res, nt)
        planted = inputs.planted_pages(w, b, DEV).cpu().numpy()
        got = res[0][b, 0].cpu().numpy()
        say(f"decode_1m seq {b}: planted pages recalled {np.isin(planted, got).sum()}/{len(planted)}")
    nt.check(0.999)


# ------------------------------------------------------------------------------ attention
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
    attn_check(att["q"], att["kv"], None, idx, w.attn.scale, out, lse, True, 512)


def _layout_case(B, T, L, k, S, W, seed, perturb=None, hint_pos0=None, seq_lens=None):
    """Attention over Streaming-Aware lists with the layout passed as a hint, and again with no
    hint: the kernel loads each split's first rows from the layout before the list arrives and
    falls back to the listed rows where they differ, so the two calls agree bit for bit; the
    hinted call also matches the oracle."""
    w = Workload(name="a", index=IndexShape(
        batch=B, n_q=T, kv_len=L, q_pos0=L - T, heads=64, head_dim=128, key_dtype="fp8"),
        budget=DECODE_128K.budget, attn=DECODE_128K.attn, seed=seed)
    att = inputs.attn_inputs(w, 0, DEV)
    lens = [L] * B if seq_lens is None else seq_lens
    idx = torch.stack([inputs.synthetic_index_lists(T, k, S, W, ref.valid_lengths(lens[b], L - T, T),
                                                    seed=seed + b) for b in range(B)])
    if perturb is not None:
        perturb(idx)
    idx = idx.to(DEV)
    sl = None if seq_lens is None else torch.tensor(seq_lens, dtype=torch.int32, device=DEV)
    pos0 = L - T if hint_pos0 is None else hint_pos0
    out, lse = lsa.sparse_attn(att["q"], att["kv"], None, idx, w.attn.scale, S, W, d_v=512,
                               q_pos0=pos0, seq_lens=sl)
    out0, lse0 = lsa.sparse_attn(att["q"], att["kv"], None, idx, w.attn.scale, 0, 0, d_v=512,
                                 q_pos0=0, seq_lens=sl)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out0.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse0.view(torch.int32))
    kv = att["kv"]
    if seq_lens is not None:  # rows past a sequence's length are skipped: the oracle's view
        ids = idx.clone()
        for b in range(B):
            ids[b][ids[b] >= seq_lens[b]] = -1
        idx = ids
    attn_check(att["q"], kv, None, idx, w.attn.scale, out, lse, True, 512)


def _hole_sink(idx):
    idx[0, 0, 3] = -1


def _move_window(idx):
    idx[1, 0, 20] = 7


def _past_cache(idx):
    idx[2, 0, 0] = 1 << 20


def _swap_first_round(idx):
    idx[3, 0, [0, 31]] = idx[3, 0, [31, 0]]


@pytest.mark.parametrize("perturb", [None, _hole_sink, _move_window, _past_cache, _swap_first_round])
def test_mla_attn_layout_hint_decode(perturb):
    """Decode shape, 8 splits of 32-entry rounds dealt in turn: splits 0-3 start on sink and
    window rounds (predicted), 4-7 on dynamic ones; with one list per case made to differ from
    the layout inside a predicted round (a skipped sink entry, a window entry naming another
    row, an entry past the cache, two entries swapped)."""
    _layout_case(B=4, T=1, L=5000, k=256, S=16, W=112, seed=41, perturb=perturb)


def test_mla_attn_layout_hint_short_rows_and_wrong_positions():
    """Rows with V <= k (the list is rows 0 .. V-1, then -1) are predicted whole; a hint with
    wrong query positions predicts the window wrongly and every such round falls back."""
    _layout_case(B=2, T=3, L=150, k=256, S=16, W=112, seed=43)
    _layout_case(B=2, T=1, L=5000, k=256, S=16, W=112, seed=45, hint_pos0=100)
    _layout_case(B=1, T=40, L=3000, k=300, S=64, W=100, seed=47)


def test_mla_attn_layout_hint_ragged():
    """Per-sequence lengths: the layout's window ends at each sequence's own length."""
    _layout_case(B=3, T=1, L=4000, k=256, S=16, W=112, seed=49, seq_lens=[4000, 1200, 200])


@pytest.mark.parametrize("shift", [0, 7])
def test_mla_attn_layout_hint_per_sequence_positions(shift):
    """Per-sequence query positions (seq_pos0) with per-sequence lengths: two queries per
    sequence at its last two positions, so V differs per sequence and per query.  shift = 7
    hands the kernel positions 7 short of the lists' own: the window rounds fall back."""
    B, T, L, k, S, W = 3, 2, 4000, 256, 16, 112
    lens, pos = [4000, 1500, 300], [3998, 1498, 298]
    w = Workload(name="a", index=IndexShape(
        batch=B, n_q=T, kv_len=L, q_pos0=L - T, heads=64, head_dim=128, key_dtype="fp8"),
        budget=DECODE_128K.budget, attn=DECODE_128K.attn, seed=53)
    att = inputs.attn_inputs(w, 0, DEV)
    idx = torch.stack([inputs.synthetic_index_lists(T, k, S, W, ref.valid_lengths(lens[b], pos[b], T),
                                                    seed=55 + b) for b in range(B)]).to(DEV)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    sp = torch.tensor([p - shift for p in pos], dtype=torch.int32, device=DEV)
    out, lse = lsa.sparse_attn(att["q"], att["kv"], None, idx, w.attn.scale, S, W, d_v=512,
                               seq_lens=sl, seq_pos0=sp)
    out0, lse0 = lsa.sparse_attn(att["q"], att["kv"], None, idx, w.attn.scale, 0, 0, d_v=512,
                                 seq_lens=sl)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out0.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse0.view(torch.int32))
    attn_check(att["q"], att["kv"], None, idx, w.attn.scale, out, lse, True, 512)


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
    attn_check(att["q"], att["k"], att["v"], idx, w.attn.scale, out, lse, False, 128, rows=rows)


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
        attn_check(att["q"][s:s + 1], att["kv"][s:s + 1], None, idx[s:s + 1], w.attn.scale,
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
    attn_check(att["q"], att["kv"], None, idx, w.attn.scale, out, lse, True, 512)


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
        attn_check(att["q"], att["kv"], None, idx, w.attn.scale, o1, l1, True, 512)
        outs.append(o1)
    assert not torch.equal(outs[0], outs[1])


def _layers_case(B, T, L, k, S, W, n, seed, exact, seq_lens=None, want_lse=True, rows=None):
    """n latent layers over one index list in one lsa_sparse_attn_layers call: every layer
    against the oracle, a second identical call bit for bit, and each layer against its own
    lsa_sparse_attn call -- bit for bit where the two cut the list into the same number of
    parts (`exact`), else within the oracle tolerance of it."""
    w = Workload(name="a", index=IndexShape(
        batch=B, n_q=T, kv_len=L, q_pos0=L - T, heads=64, head_dim=128, key_dtype="fp8"),
        budget=DECODE_128K.budget, attn=DECODE_128K.attn, seed=seed)
    lens = [L] * B if seq_lens is None else seq_lens
    idx = torch.stack([inputs.synthetic_index_lists(T, k, S, W, ref.valid_lengths(lens[b], L - T, T),
                                                    seed=seed + b) for b in range(B)]).to(DEV)
    sl = None if seq_lens is None else torch.tensor(seq_lens, dtype=torch.int32, device=DEV)
    atts = [inputs.attn_inputs(w, layer, DEV) for layer in range(n)]
    qs, kvs = [a["q"] for a in atts], [a["kv"] for a in atts]
    outs, lses = lsa.sparse_attn_layers(qs, kvs, idx, w.attn.scale, S, W, d_v=512, seq_lens=sl,
                                        want_lse=want_lse)
    outs2, _ = lsa.sparse_attn_layers(qs, kvs, idx, w.attn.scale, S, W, d_v=512, seq_lens=sl,
                                      want_lse=want_lse)
    assert lses is None or len(lses) == n
    oidx = idx.clone()
    if seq_lens is not None:  # rows past a sequence's length are skipped: the oracle's view
        for b in range(B):
            oidx[b][oidx[b] >= seq_lens[b]] = -1
    for layer, a in enumerate(atts):
        assert torch.equal(outs[layer].view(torch.int16), outs2[layer].view(torch.int16)), layer
        o, l1 = lsa.sparse_attn(a["q"], a["kv"], None, idx, w.attn.scale, S, W, d_v=512, seq_lens=sl)
        if exact:
            assert torch.equal(outs[layer].view(torch.int16), o.view(torch.int16)), layer
            if want_lse:
                assert torch.equal(lses[layer].view(torch.int32), l1.view(torch.int32)), layer
        else:
            assert (outs[layer].float() - o.float()).abs().max().item() <= 2e-2, layer
        attn_check(a["q"], a["kv"], None, oidx, w.attn.scale, outs[layer],
                   None if lses is None else lses[layer], True, 512, rows=rows)


# (the split counts follow from 512 workgroups wanted per launch: a single call with B x T query
# rows and a call of n layers plan like B x T and n x B x T rows, capped by the list's rounds)
@pytest.mark.parametrize("B,T,L,k,n,exact,rows", [
    (8, 1, 6000, 256, 4, True, None),      # 8 splits either way (8 rounds of 32 entries)
    (2, 3, 3000, 2048, 3, False, None),    # 32 splits alone, 29 over the 3 layers
    (1, 600, 3000, 256, 2, True, [0, 1, 299, 599]),  # one part either way (the prefill form)
    (3, 1, 700, 128, 8, True, None),       # 4 splits either way; the 8-layer limit
    (4, 1, 6000, 256, 1, True, None),      # one layer: the single-layer launch itself
])
def test_attn_layers_against_single_calls_and_oracle(B, T, L, k, n, exact, rows):
    _layers_case(B, T, L, k, min(64, k // 4), min(200, k // 4), n, seed=51 + n, exact=exact,
                 rows=rows)


def test_attn_layers_ragged_and_no_lse():
    _layers_case(3, 1, 4000, 256, 16, 112, 3, seed=61, exact=True, seq_lens=[4000, 900, 0])
    _layers_case(2, 1, 4000, 256, 16, 112, 2, seed=63, exact=True, want_lse=False)


def _to_pool(kvs, bs, spare, seed, bad=()):
    """Dense latent caches [B, L, row] (one per layer) as pools of bs-row blocks under one block
    table [B, ceil(L / bs)]: the blocks in a random order among `spare` unused ones, which hold
    noise.  bad: (b, j, entry) table entries to overwrite (outside the pool: skipped tokens)."""
    B, L, row = kvs[0].shape
    bps = -(-L // bs)
    n = B * bps + spare
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(n, generator=g)[:B * bps].view(B, bps)
    pools = []
    for kv in kvs:
        pool = torch.randn((n, bs, row), generator=g).to(torch.bfloat16).to(kv.device)
        pad = torch.zeros((B, bps * bs, row), dtype=kv.dtype, device=kv.device)
        pad[:, :L] = kv
        pool[perm.view(-1).to(kv.device)] = pad.view(B * bps, bs, row)
        pools.append(pool)
    tab = perm.to(torch.int32)
    for b, j, e in bad:
        tab[b, j] = e
    return pools, tab.to(kvs[0].device)


def _paged_case(B, T, L, k, S, W, bs, seed, n=1, seq_lens=None, spare=5, bad=()):
    """The attention over a paged copy of the caches equals the attention over the dense caches
    bit for bit (the same rows in the same order: only their addresses differ), for one layer and
    for n layers in one call; table entries outside the pool equal the dense call with those
    blocks' ids replaced by -1."""
    w = Workload(name="a", index=IndexShape(
        batch=B, n_q=T, kv_len=L, q_pos0=L - T, heads=64, head_dim=128, key_dtype="fp8"),
        budget=DECODE_128K.budget, attn=DECODE_128K.attn, seed=seed)
    lens = [L] * B if seq_lens is None else seq_lens
    idx = torch.stack([inputs.synthetic_index_lists(T, k, S, W, ref.valid_lengths(lens[b], L - T, T),
                                                    seed=seed + b) for b in range(B)]).to(DEV)
    sl = None if seq_lens is None else torch.tensor(seq_lens, dtype=torch.int32, device=DEV)
    atts = [inputs.attn_inputs(w, layer, DEV) for layer in range(n)]
    qs, kvs = [a["q"] for a in atts], [a["kv"] for a in atts]
    pools, tab = _to_pool(kvs, bs, spare, seed + 100, bad)
    didx = idx.clone()
    for b, j, _ in bad:
        blk = (didx[b] >= j * bs) & (didx[b] < (j + 1) * bs)
        didx[b][blk] = -1
    say(f"paged B={B} T={T} L={L} k={k} bs={bs} layers={n} bad={len(bad)}")
    scale = w.attn.scale
    for layer in range(n):
        o_d, l_d = lsa.sparse_attn(qs[layer], kvs[layer], None, didx, scale, S, W, d_v=512,
                                   seq_lens=sl)
        o_p, l_p = lsa.sparse_attn(qs[layer], pools[layer], None, idx, scale, S, W, d_v=512,
                                   seq_lens=sl, block_table=tab, kv_len=L)
        assert torch.equal(o_p.view(torch.int16), o_d.view(torch.int16)), layer
        assert torch.equal(l_p.view(torch.int32), l_d.view(torch.int32)), layer
    if n > 1:
        outs_d, lses_d = lsa.sparse_attn_layers(qs, kvs, didx, scale, S, W, d_v=512, seq_lens=sl)
        outs_p, lses_p = lsa.sparse_attn_layers(qs, pools, idx, scale, S, W, d_v=512, seq_lens=sl,
                                                block_table=tab, kv_len=L)
        for layer in range(n):
            assert torch.equal(outs_p[layer].view(torch.int16), outs_d[layer].view(torch.int16))
            assert torch.equal(lses_p[layer].view(torch.int32), lses_d[layer].view(torch.int32))
    if not bad:  # and the dense call against the oracle, so the paged one is pinned too
        oidx = idx.clone()
        if seq_lens is not None:
            for b in range(B):
                oidx[b][oidx[b] >= seq_lens[b]] = -1
        o_p, l_p = lsa.sparse_attn(qs[0], pools[0], None, idx, scale, S, W, d_v=512, seq_lens=sl,
                                   block_table=tab, kv_len=L)
        attn_check(qs[0], kvs[0], None, oidx, scale, o_p, l_p, True, 512,
                   rows=None if B * T <= 8 else [0, B * T - 1])


@pytest.mark.parametrize("B,T,L,k,S,W,bs", [
    (4, 1, 6000, 256, 16, 112, 64),     # decode, the layout hint taken through the table
    (2, 3, 3000, 2048, 64, 960, 16),    # every row listed: split-K over the whole cache
    (3, 1, 700, 128, 16, 48, 1),        # one-row blocks
    (2, 1, 900, 128, 8, 24, 4096),      # one block per sequence, larger than the cache
    (1, 300, 2000, 256, 16, 112, 128),  # a prefill chunk (one split per query)
])
def test_attn_paged_equals_dense(B, T, L, k, S, W, bs):
    _paged_case(B, T, L, k, S, W, bs, seed=81 + bs)


def test_attn_paged_layers_and_ragged():
    _paged_case(3, 1, 4000, 256, 16, 112, 64, seed=91, n=3)
    _paged_case(3, 1, 4000, 256, 16, 112, 32, seed=93, seq_lens=[4000, 900, 0])


def test_attn_paged_entries_outside_the_pool():
    """Table entries of -1 or >= n_blocks (one in the sink's block, one in the window's, one in
    the middle) skip those blocks' tokens, exactly as -1 ids would."""
    L, bs = 6000, 64
    last = (L - 1) // bs
    _paged_case(2, 1, L, 256, 16, 112, bs, seed=97,
                bad=[(0, 0, -1), (0, last, 1 << 30), (1, 40, 2 * ((L + bs - 1) // bs) + 5)])


def _key_pool(keys, scale, bs, spare, seed, bad=()):
    """Dense indexer keys [B, L, d] (and fp8 scales [B, L]) as pools of bs-row blocks under one
    block table [B, ceil(L / bs)], in a random order among `spare` unused blocks.  Pool rows past
    a sequence's keys and the unused blocks hold other valid keys (finite codes, positive
    scales).  bad: (b, j, entry) table entries to overwrite."""
    B, L, d = keys.shape
    bps = -(-L // bs)
    n = B * bps + spare
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(n, generator=g)[:B * bps].view(B, bps)
    filler = keys.reshape(-1, d)[torch.randint(0, B * L, (n * bs,), generator=g).to(keys.device)]
    pool = filler.view(n, bs, d).clone()
    pad = pool[perm.view(-1).to(keys.device)].view(B, bps * bs, d)
    pad[:, :L] = keys
    pool[perm.view(-1).to(keys.device)] = pad.view(B * bps, bs, d)
    spool = None
    if scale is not None:
        spool = (torch.rand((n, bs), generator=g) + 0.5).to(scale.device)
        spad = spool[perm.view(-1).to(scale.device)].view(B, bps * bs)
        spad[:, :L] = scale
        spool[perm.view(-1).to(scale.device)] = spad.view(B * bps, bs)
    tab = perm.to(torch.int32)
    for b, j, e in bad:
        tab[b, j] = e
    return pool, spool, tab.to(keys.device)


def _paged_scores_case(B, T, L, H, kd, bs, seed, fused=None, seq_lens=None, bad=(), d=128):
    """Scores (and, with fused = (k, S, W), the fused selection) over a paged copy of the keys
    equal those over the dense keys bit for bit; blocks whose table entry lies outside the pool
    score -inf, and the selection is the one from those scores."""
    w = Workload(name="p", index=IndexShape(batch=B, n_q=T, kv_len=L, q_pos0=L - T, heads=H,
                                            head_dim=d, key_dtype=kd),
                 budget=DECODE_128K.budget, attn=DECODE_128K.attn, seed=seed)
    inp = inputs.index_inputs(w, DEV)
    pool, spool, tab = _key_pool(inp["keys"], inp["scale"], bs, 3, seed + 7, bad)
    sl = None if seq_lens is None else torch.tensor(seq_lens, dtype=torch.int32, device=DEV)
    say(f"paged scores B={B} T={T} L={L} H={H} {kd} bs={bs} fused={fused} bad={len(bad)}")
    dense = lsa.index_scores(inp["q"], inp["w"], inp["keys"], inp["scale"], seq_lens=sl)
    for b, j, _ in bad:
        dense[b, :, j * bs:(j + 1) * bs] = -math.inf
    paged = lsa.index_scores(inp["q"], inp["w"], pool, spool, seq_lens=sl, block_table=tab,
                             kv_len=L)
    assert torch.equal(paged.view(torch.int32), dense.view(torch.int32))
    if fused is not None:
        k, S, W = fused
        sc, idx = lsa.index_select(inp["q"], inp["w"], pool, spool, k, S, W, seq_lens=sl,
                                   block_table=tab, kv_len=L)
        assert torch.equal(sc.view(torch.int32), dense.view(torch.int32))
        expect = lsa.topk_select(dense, k, S, W, kv_len=L, q_pos0=L - T, seq_lens=sl)
        assert torch.equal(idx, expect)


@pytest.mark.parametrize("B,T,L,H,kd,bs", [
    (2, 1, 5000, 64, "fp8", 64),      # a short launch (two blocks per wave), ragged tail
    (3, 2, 3001, 64, "bf16", 32),     # bf16 keys, two queries, the smallest blocks
    (2, 4, 2000, 16, "fp8", 4096),    # four queries per sequence, one block larger than the keys
    (4, 1, 524365, 64, "fp8", 128),   # a long launch (one round of workgroups), ragged tail
])
def test_scores_paged_equals_dense(B, T, L, H, kd, bs):
    _paged_scores_case(B, T, L, H, kd, bs, seed=101 + bs)


@pytest.mark.parametrize("kd,H,T", [("fp8", 64, 1), ("bf16", 8, 8)])
def test_scores_paged_head_dim_64(kd, H, T):
    _paged_scores_case(2, T, 3000, H, kd, 64, seed=131, d=64)


def test_index_select_paged_fused_decode():
    """The fused decode path (histograms and slices in the scoring launch) over paged keys."""
    _paged_scores_case(16, 1, 131072, 64, "fp8", 64, seed=111, fused=(2048, 64, 960))
    _paged_scores_case(16, 1, 131072, 64, "fp8", 256, seed=113, fused=(2048, 64, 960),
                       seq_lens=[131072 - 977 * i for i in range(16)])


def test_scores_paged_entries_outside_the_pool():
    L, bs = 131072, 64
    _paged_scores_case(16, 1, L, 64, "fp8", bs, seed=117, fused=(2048, 64, 960),
                       bad=[(0, 0, -1), (3, 700, 1 << 30), (5, L // bs - 1, -7)])
    _paged_scores_case(2, 1, 5000, 64, "fp8", bs, seed=119, bad=[(1, 10, -1)])


@pytest.mark.parametrize("kd,P,bs", [("fp8", 64, 64), ("fp8", 64, 256), ("bf16", 32, 128)])
def test_hi_paged_equals_dense(kd, P, bs):
    """Page keys and page recall over paged keys equal those over the dense keys bit for bit;
    a table entry outside the pool gives its pages the zero key and its tokens the fine score
    -inf."""
    B, L = 3, 40017
    w = Workload(name="h", index=IndexShape(batch=B, n_q=1, kv_len=L, q_pos0=L - 1, heads=64,
                                            head_dim=128, key_dtype=kd),
                 budget=DECODE_128K.budget, attn=DECODE_128K.attn, seed=141 + P + bs)
    inp = inputs.index_inputs(w, DEV)
    k, S, W, M = 1024, 64, 448, 64
    for bad in ((), ((1, 5, -1),)):
        say(f"paged HI {kd} P={P} bs={bs} bad={bad}")
        pool, spool, tab = _key_pool(inp["keys"], inp["scale"], bs, 3, 143, bad)
        pk = lsa.page_summary(inp["keys"], inp["scale"], P)
        pk_p = lsa.page_summary(pool, spool, P, block_table=tab, kv_len=L)
        for b, j, _ in bad:
            pk[b, j * bs // P:(j + 1) * bs // P] = 0
        assert torch.equal(pk_p.view(torch.int16), pk.view(torch.int16))
        ids, cs, ci = lsa.page_recall(inp["q"], inp["w"], pk, inp["keys"], inp["scale"], k, S, W,
                                      P, M)
        ids_p, cs_p, ci_p = lsa.page_recall(inp["q"], inp["w"], pk, pool, spool, k, S, W, P, M,
                                            block_table=tab, kv_len=L)
        for b, j, _ in bad:
            cs[b][(ci[b] >= j * bs) & (ci[b] < (j + 1) * bs)] = -math.inf
        assert torch.equal(ids_p, ids) and torch.equal(ci_p, ci)
        assert torch.equal(cs_p.view(torch.int32), cs.view(torch.int32))


def test_attn_layers_per_head_cache():
    """A per-head (non-latent) cache: the layers run one after another, each equal to its own
    call."""
    B, T, H, L, k, d = 2, 3, 2, 400, 64, 64
    g = torch.Generator().manual_seed(71)
    qs = [torch.randn((B, T, H, d), generator=g).to(torch.bfloat16).to(DEV) for _ in range(2)]
    ks = [torch.randn((B, L, d), generator=g).to(torch.bfloat16).to(DEV) for _ in range(2)]
    vs = [torch.randn((B, L, d), generator=g).to(torch.bfloat16).to(DEV) for _ in range(2)]
    idx = torch.randint(-1, L, (B, T, k), generator=g, dtype=torch.int32).to(DEV)
    outs, lses = lsa.sparse_attn_layers(qs, ks, idx, 0.125, vs=vs, latent=False)
    for layer in range(2):
        o, l1 = lsa.sparse_attn(qs[layer], ks[layer], vs[layer], idx, 0.125, latent=False)
        assert torch.equal(outs[layer].view(torch.int16), o.view(torch.int16))
        assert torch.equal(lses[layer].view(torch.int32), l1.view(torch.int32))
    attn_check(qs[1], ks[1], vs[1], idx, 0.125, outs[1], lses[1], False, d)


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
