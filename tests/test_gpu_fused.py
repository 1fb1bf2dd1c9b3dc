"""Decode scoring with the selection's histogram fused in (lsa_index_select) on the GPU.

Its outputs must be bitwise those of lsa_index_scores followed by lsa_topk_select (which the
other GPU tests tie to the oracle), and its selection bit-exact against the oracle's selection
on the same fp32 scores.  Cases: the decode workload at full size, fp8 and bf16 keys, 32 and 64
heads, a key count off the 32-key block (the moved-back last block must not be counted twice in
the histogram), a causal cut short of the cache end, a second query per sequence, rows with
V <= k, a row where every score ties (the histogram's threshold bin overflows the buffer: the
exact fallback), rows whose best keys crowd into one scoring workgroup's range (its slice does
not reach the row's threshold bin: that range is read from the score row), and an unfused shape
(the two ordinary launches).
"""
import numpy as np
import pytest
import torch

from oracle import ref
from token_selection_indexer_amd import inputs, lsa
from token_selection_indexer_amd.configs import DECODE_128K, Budget, IndexShape, Workload, shrink
from tests.gpu_checks import check_rows_exact, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lsa.lib()
    yield
    torch.cuda.synchronize()


def _fused(q, w, keys, scale, b, q_pos0):
    return lsa.index_select(q, w, keys, scale, b.k, b.sink, b.window, q_pos0=q_pos0)


def _separate(q, w, keys, scale, b, q_pos0):
    sc = lsa.index_scores(q, w, keys, scale, q_pos0=q_pos0)
    idx = lsa.topk_select(sc, b.k, b.sink, b.window, kv_len=keys.shape[1], q_pos0=q_pos0)
    return sc, idx


def _is_fused(wl):
    s, b = wl.index, wl.budget
    shape = lsa.IndexShape(s.batch, s.n_q, s.heads, s.head_dim, s.kv_len, s.q_pos0)
    fused = lsa.lsa_workspace_bytes(lsa.OP_INDEX_SELECT, shape, lsa.Budget(b.k, b.sink, b.window))
    plain = lsa.lsa_workspace_bytes(lsa.OP_TOPK_SELECT, shape, lsa.Budget(b.k, b.sink, b.window))
    return fused != plain


def _case(wl, check_rows=None):
    s, b = wl.index, wl.budget
    inp = inputs.index_inputs(wl, DEV)
    sc1, i1 = _fused(inp["q"], inp["w"], inp["keys"], inp["scale"], b, s.q_pos0)
    sc2, i2 = _separate(inp["q"], inp["w"], inp["keys"], inp["scale"], b, s.q_pos0)
    torch.cuda.synchronize()
    assert torch.equal(sc1.view(torch.int32), sc2.view(torch.int32))
    assert torch.equal(i1, i2)
    scn, gi = sc1.cpu().numpy(), i1.cpu().numpy()
    V = ref.valid_lengths(s.kv_len, s.q_pos0, s.n_q)
    for r in (range(s.batch) if check_rows is None else check_rows):
        check_rows_exact(gi[r], scn[r], V, b.k, b.sink, b.window)
    return inp, sc1, i1


def test_fused_decode_128k_full():
    wl = DECODE_128K
    assert _is_fused(wl)
    _case(wl)
    say("fused decode 32 x 128K: bitwise equal to the separate calls")


# batch x blocks of 32 keys reach the long scoring launch (at least 65536 blocks), which is the
# one that emits the histograms.  32 query rows or more with at most 8192 keys per scoring
# workgroup take the slices (32 x 70000, the two 16 x 2-query cases, 64 x 65536 with 8 scoring
# workgroups per row); the others read the rows through the histograms.
@pytest.mark.parametrize("kd,H,L,back,nq,B", [("fp8", 64, 131072 - 5, 0, 1, 16),
                                              ("bf16", 64, 70000, 3000, 1, 32),
                                              ("fp8", 32, 100003, 0, 2, 11),
                                              ("bf16", 32, 90000, 17, 1, 24),
                                              ("fp8", 64, 131072 - 77, 5, 2, 16),
                                              ("bf16", 32, 120001, 0, 2, 16),
                                              ("fp8", 64, 65536, 0, 1, 64)])
def test_fused_shapes(kd, H, L, back, nq, B):
    wl = Workload(name="f", index=IndexShape(batch=B, n_q=nq, kv_len=L, q_pos0=L - nq - back,
                                             heads=H, head_dim=128, key_dtype=kd),
                  budget=Budget(k=2048, sink=64, window=960), attn=DECODE_128K.attn, seed=61 + H)
    assert _is_fused(wl)
    _case(wl)


def test_fused_rows_within_budget_and_ties():
    """Sequences whose query sees at most k keys take everything; a sequence whose keys are all
    equal has one score for every key: its threshold bin holds the whole middle, which cannot
    fit the buffer, so the exact one-workgroup path selects (lowest ids win the ties)."""
    L, B = 131072, 16
    wl = Workload(name="ft", index=IndexShape(batch=B, n_q=1, kv_len=L, q_pos0=L - 1, heads=64,
                                              head_dim=128, key_dtype="fp8"),
                  budget=Budget(k=2048, sink=64, window=960), attn=DECODE_128K.attn, seed=71)
    inp = inputs.index_inputs(wl, DEV)
    keys, scale = inp["keys"].clone(), inp["scale"].clone()
    keys[1] = keys[1, 5]       # every key of sequence 1 equal
    scale[1] = scale[1, 5]
    b = wl.budget
    assert _is_fused(wl)
    for pos0 in (L - 1, 1000):  # decode, then a query that sees 1001 <= k keys
        sc1, i1 = _fused(inp["q"], inp["w"], keys, scale, b, pos0)
        sc2, i2 = _separate(inp["q"], inp["w"], keys, scale, b, pos0)
        torch.cuda.synchronize()
        assert torch.equal(sc1.view(torch.int32), sc2.view(torch.int32)), pos0
        assert torch.equal(i1, i2), pos0
        V = ref.valid_lengths(L, pos0, 1)
        scn, gi = sc1.cpu().numpy(), i1.cpu().numpy()
        for r in range(B):
            check_rows_exact(gi[r], scn[r], V, b.k, b.sink, b.window)
    sc1, i1 = _fused(inp["q"], inp["w"], keys, scale, b, L - 1)
    gi = i1.cpu().numpy()
    dyn = gi[1, 0, b.sink + b.window:]
    assert np.array_equal(dyn, np.arange(b.sink, b.sink + b.k - b.sink - b.window))


@pytest.mark.parametrize("B", [16, 32])
def test_fused_clustered_best_keys(B):
    """With 32 sequences each scoring workgroup keeps only its own best few (about twice its
    share of the row's picks) in a slice; with 16 the selection reads the rows through the
    histograms.  Here one sequence's best keys crowd into one stretch (copies of its best key
    with rising scales, so distinct and far above the rest), another's into tied copies: the
    slices of the stretch's workgroups lack keys at the row's threshold bin, so the selection
    reads those ranges from the score row.  Results stay bitwise those of the separate calls."""
    L = 131072
    wl = Workload(name="fc", index=IndexShape(batch=B, n_q=1, kv_len=L, q_pos0=L - 1, heads=64,
                                              head_dim=128, key_dtype="fp8"),
                  budget=Budget(k=2048, sink=64, window=960), attn=DECODE_128K.attn, seed=73)
    b = wl.budget
    inp = inputs.index_inputs(wl, DEV)
    keys, scale = inp["keys"].clone(), inp["scale"].clone()
    sc0, _ = _separate(inp["q"], inp["w"], keys, scale, b, L - 1)
    top = sc0[:, 0, b.sink:L - b.window].argmax(dim=1) + b.sink
    lo, n = 7000, 2000  # straddles a workgroup boundary (every 4096 or 8192 keys here)
    a1, a2 = int(top[1]), int(top[2])
    keys[1, lo:lo + n] = keys[1, a1]
    scale[1, lo:lo + n] = scale[1, a1] * torch.linspace(1.0, 3.0, n, device=DEV)
    keys[2, lo:lo + n] = keys[2, a2]
    scale[2, lo:lo + n] = scale[2, a2]
    assert _is_fused(wl)
    sc1, i1 = _fused(inp["q"], inp["w"], keys, scale, b, L - 1)
    sc2, i2 = _separate(inp["q"], inp["w"], keys, scale, b, L - 1)
    torch.cuda.synchronize()
    assert torch.equal(sc1.view(torch.int32), sc2.view(torch.int32))
    assert torch.equal(i1, i2)
    V = ref.valid_lengths(L, L - 1, 1)
    scn, gi = sc1.cpu().numpy(), i1.cpu().numpy()
    for r in range(B):
        check_rows_exact(gi[r], scn[r], V, b.k, b.sink, b.window)
    need = b.k - b.sink - b.window
    # sequence 2: the tied copies outrank everything but the original, lowest ids first
    dyn2 = gi[2, 0, b.sink + b.window:]
    expect = np.concatenate([[a2], np.arange(lo, lo + need - 1)]) if a2 < lo else np.arange(lo, lo + need)
    assert np.array_equal(dyn2, expect)
    # sequence 1: the copies with the largest scales (factors 2 .. 3, above every other key)
    assert np.array_equal(gi[1, 0, b.sink + b.window:], np.arange(lo + n - need, lo + n))


def test_unfused_shape_matches():
    """A prefill chunk is not fused; lsa_index_select runs the two ordinary launches."""
    wl = shrink(DECODE_128K, batch=1, n_q=40, kv_len=5000, q_pos0=4960)
    assert not _is_fused(wl)
    _case(wl)


def test_fused_slices_workspace_across_shapes():
    """One workspace through sliced calls of different shapes (32 x 128K, then 32 x 70000 and 16
    x 2 queries): every slice header and entry the selection reads is written by the scoring
    launch of the same call, whatever the previous call left."""
    ws = lsa.Workspace()
    shapes = [(131072, 1, 32, 81), (70000, 1, 32, 82), (120001, 2, 16, 83), (131072, 1, 32, 84)]
    for L, nq, B, seed in shapes:
        wl = Workload(name="fw", index=IndexShape(batch=B, n_q=nq, kv_len=L, q_pos0=L - nq,
                                                  heads=64, head_dim=128, key_dtype="fp8"),
                      budget=Budget(k=2048, sink=64, window=960), attn=DECODE_128K.attn, seed=seed)
        s, b = wl.index, wl.budget
        assert _is_fused(wl)
        inp = inputs.index_inputs(wl, DEV)
        sc1, i1 = lsa.index_select(inp["q"], inp["w"], inp["keys"], inp["scale"], b.k, b.sink,
                                   b.window, q_pos0=s.q_pos0, ws=ws)
        sc2, i2 = _separate(inp["q"], inp["w"], inp["keys"], inp["scale"], b, s.q_pos0)
        torch.cuda.synchronize()
        assert torch.equal(sc1.view(torch.int32), sc2.view(torch.int32)), (L, nq, B)
        assert torch.equal(i1, i2), (L, nq, B)
        del inp, sc1, sc2, i1, i2
        torch.cuda.empty_cache()


def test_fused_repeated_calls_reuse_workspace():
    """The workspace is reused across calls with stale contents from the previous call (the
    fine bins of groups that were empty are never read): identical results every time."""
    wl = shrink(DECODE_128K, batch=32, kv_len=65536, q_pos0=65535)
    s, b = wl.index, wl.budget
    assert _is_fused(wl)
    inp = inputs.index_inputs(wl, DEV)
    ws = lsa.Workspace()
    first = None
    for rep in range(4):
        sc, idx = lsa.index_select(inp["q"], inp["w"], inp["keys"], inp["scale"], b.k, b.sink,
                                   b.window, q_pos0=s.q_pos0, ws=ws)
        torch.cuda.synchronize()
        if first is None:
            first = (sc.clone(), idx.clone())
        assert torch.equal(idx, first[1]) and torch.equal(sc, first[0]), rep
    _, i2 = _separate(inp["q"], inp["w"], inp["keys"], inp["scale"], b, s.q_pos0)
    assert torch.equal(first[1], i2)
