"""The five workloads at their own full shapes, end to end on the GPU, against the CPU oracle.

Each test runs the path the way the bench runs it (same shapes, same entry points, same launch
configurations) and checks, stage by stage on the GPU's own inputs to that stage:
  scores      whole rows of sampled queries within the score tolerance;
  selection   every row bit-exact against ref.select on the GPU's own fp32 scores, with its
              sink | window | dynamic layout; sampled rows against the oracle's selection from
              its own fp64 scores, up to near-ties, recall >= 99.9% over the rows checked;
  HI          page keys bit-exact; recalled pages up to near-ties in the coarse scores
              (recall >= 99.9% over the rows checked); candidate ids exact on the GPU's pages,
              candidate scores within tolerance; the final set against the oracle's selection
              from its fp64 scores of the GPU's candidates;
  attention   sampled (sequence, query) rows, all heads, against the fp64 oracle over the GPU's
              own index lists, within 2e-2; cross-layer reuse bitwise reproducible.
Quality figures the pages motivate (planted-page recall at 1M, overlap of the HI and flat
selections) are printed, not gated.
"""
import numpy as np
import pytest
import torch

from oracle import ref
from token_selection_indexer_amd import inputs, lsa
from token_selection_indexer_amd.configs import (DECODE_128K, DECODE_1M_HI, DECODE_256K_HI_CLI,
                                                 PREFILL_8K_AT_128K, TINY_PREFILL_4K)
from tests.gpu_checks import (assert_scores, attn_check, check_rows_exact, hi_case,
                              oracle_scores, say, selection_vs_oracle_scores)
from tests.util import NearTie, bits, check_si_layout, f32, keys_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lsa.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _attn_ws_bytes(w, n_q_rows):
    s, b, a = w.index, w.budget, w.attn
    return lsa.lsa_workspace_bytes(
        lsa.OP_SPARSE_ATTN, lsa.IndexShape(s.batch, n_q_rows, 64, 128, s.kv_len, 0),
        lsa.Budget(b.k, b.sink, b.window),
        attn=lsa.AttnShape(a.heads, a.d_qk, a.d_v, 1, a.d_qk, a.d_qk, a.scale))


def test_tiny_prefill_4k_attention_on_gpu_selection():
    """Tiny prefill: GPU scores -> GPU selection -> per-head attention (1 head, d = 128), the
    attention checked on the GPU's own index lists at sampled rows (V <= k rows included)."""
    w = TINY_PREFILL_4K
    b, a = w.budget, w.attn
    inp = inputs.index_inputs(w, DEV)
    sc = lsa.index_scores(inp["q"], inp["w"], inp["keys"], None, q_pos0=0)
    idx = lsa.topk_select(sc, b.k, b.sink, b.window, kv_len=4096, q_pos0=0)
    att = inputs.attn_inputs(w, 0, DEV)
    out, lse = lsa.sparse_attn(att["q"], att["k"], att["v"], idx, a.scale, b.sink, b.window)
    rows = [0, 1, 100, 255, 256, 257, 2048, 4095] + list(range(3, 4096, 211))
    worst = attn_check(att["q"], att["k"], att["v"], idx, a.scale, out, lse, False, a.d_v,
                       rows=rows)
    say(f"tiny prefill attention: worst |err| {worst:.2e}")


def test_decode_b32_128k_end_to_end():
    """Decode, 32 x 131072 fp8 keys, k = 2048 (64 | 960 | 1024), 16-head MLA."""
    w = DECODE_128K
    s, b, a = w.index, w.budget, w.attn
    inp = inputs.index_inputs(w, DEV)
    sc = lsa.index_scores(inp["q"], inp["w"], inp["keys"], inp["scale"], q_pos0=s.q_pos0)
    idx = lsa.topk_select(sc, b.k, b.sink, b.window, kv_len=s.kv_len, q_pos0=s.q_pos0)
    torch.cuda.synchronize()
    scn, gi = sc.cpu().numpy(), idx.cpu().numpy()
    V = np.array([s.kv_len])
    for r in range(s.batch):
        check_rows_exact(gi[r], scn[r], V, b.k, b.sink, b.window)
    nt = NearTie()
    for r in (0, 9, 20, 31):
        I, A, E = oracle_scores(inp, r, [0], s.q_pos0)
        assert_scores(scn[r, 0], I[0], A[0], E[0], f"seq {r}")
        selection_vs_oracle_scores(nt, gi[r, 0], I[0], A[0], E[0], s.kv_len, b.k, b.sink,
                                   b.window)
    say(f"decode 128K: selection recall vs fp64 oracle {nt.recall:.6f} ({nt.mismatches} near ties)")
    nt.check(0.999)
    del sc
    att = inputs.attn_inputs(w, 0, DEV)
    out, lse = lsa.sparse_attn(att["q"], att["kv"], None, idx, a.scale, b.sink, b.window,
                               d_v=a.d_v)
    worst = attn_check(att["q"], att["kv"], None, idx, a.scale, out, lse, True, a.d_v,
                       seqs=(0, 13, 31))
    say(f"decode 128K attention: worst |err| {worst:.2e}")


def test_prefill_chunk8k_128k_end_to_end():
    """Chunked prefill: 8192 queries at positions 122880.. over 131072 bf16 keys, k = 2048
    (128 | 896 | 1024), MLA attention in the bench's launch (one workgroup per (query, head
    group), no split: 64 rounds of 32 rows each)."""
    w = PREFILL_8K_AT_128K
    s, b, a = w.index, w.budget, w.attn
    inp = inputs.index_inputs(w, DEV)
    sc = lsa.index_scores(inp["q"], inp["w"], inp["keys"], None, q_pos0=s.q_pos0)
    idx = lsa.topk_select(sc, b.k, b.sink, b.window, kv_len=s.kv_len, q_pos0=s.q_pos0)
    torch.cuda.synchronize()
    rows = [0, 1, 2, 1000, 4095, 4096, 6000, 8190, 8191]
    gi = idx[0].cpu().numpy()
    V = ref.valid_lengths(s.kv_len, s.q_pos0, s.n_q)
    for t in range(s.n_q):  # layout of every row
        check_si_layout(gi[t], int(V[t]), b.k, b.sink, b.window)
    scr = sc[0, rows].cpu().numpy()
    check_rows_exact(gi[rows], scr, V[rows], b.k, b.sink, b.window)
    I, A, E = oracle_scores(inp, 0, rows, s.q_pos0)
    nt = NearTie()
    for i, t in enumerate(rows):
        assert_scores(scr[i], I[i], A[i], E[i], f"row {t}")
        selection_vs_oracle_scores(nt, gi[t], I[i], A[i], E[i], int(V[t]), b.k, b.sink, b.window)
    say(f"prefill 8K: selection recall vs fp64 oracle {nt.recall:.6f} ({nt.mismatches} near ties)")
    nt.check(0.999)
    del sc
    torch.cuda.empty_cache()
    assert _attn_ws_bytes(w, s.n_q) == 0  # the unsplit launch the bench times
    att = inputs.attn_inputs(w, 0, DEV)
    out, lse = lsa.sparse_attn(att["q"], att["kv"], None, idx, a.scale, b.sink, b.window,
                               d_v=a.d_v)
    worst = attn_check(att["q"], att["kv"], None, idx, a.scale, out, lse, True, a.d_v,
                       rows=[0, 1, 4095, 4096, 8191])
    say(f"prefill 8K attention: worst |err| {worst:.2e}")


def _hi_end_to_end(w, check_seqs, attn_seqs, flat_overlap_seqs):
    """Page keys -> recall -> candidate selection -> attention (every layer), as the bench runs
    them; returns the per-sequence planted-page recall and HI/flat overlap for the report."""
    s, b, a, hi = w.index, w.budget, w.attn, w.hi
    inp = inputs.index_inputs(w, DEV)
    pk = lsa.page_summary(inp["keys"], inp["scale"], hi.page)
    res = lsa.page_recall(inp["q"], inp["w"], pk, inp["keys"], inp["scale"], b.k, b.sink,
                          b.window, hi.page, hi.m_pages, q_pos0=s.q_pos0)
    idx = lsa.topk_select(res[1], b.k, b.sink, b.window, kv_len=s.kv_len, q_pos0=s.q_pos0,
                          cand_ids=res[2])
    torch.cuda.synchronize()
    cs, ci, gi = res[1].cpu().numpy(), res[2].cpu().numpy(), idx.cpu().numpy()
    V = np.array([s.kv_len])
    for r in range(s.batch):  # candidate-mode selection, every sequence
        check_rows_exact(gi[r], cs[r], V, b.k, b.sink, b.window, cand_ids=ci[r])
    nt_pages, nt_final = NearTie(), NearTie()
    for r in check_seqs:
        keys, scale = keys_np(inp, r)
        assert np.array_equal(bits(pk[r]), ref.page_keys(keys, scale, hi.page)), r
        hi_case(w, r, inp, pk, res, nt_pages)
        # final set: the oracle's selection from its fp64 scores of the GPU's candidates
        ok = ci[r, 0] >= 0
        I = np.full(ci.shape[2], -np.inf)
        A = np.zeros(ci.shape[2])
        E = np.zeros(ci.shape[2])
        tok = ci[r, 0][ok]
        Ii, Ai, Ei = ref.index_scores(bits(inp["q"][r, 0:1]), f32(inp["w"][r, 0:1]), keys[tok],
                                      None if scale is None else scale[tok],
                                      np.array([len(tok) - 1]))
        I[ok], A[ok], E[ok] = Ii[0], Ai[0], Ei[0]
        selection_vs_oracle_scores(nt_final, gi[r, 0], I, A, E, s.kv_len, b.k, b.sink, b.window,
                                   cand_ids=ci[r, 0])
    say(f"{w.name}: page recall vs oracle {nt_pages.recall:.6f}, final set {nt_final.recall:.6f}")
    nt_pages.check(0.999)
    nt_final.check(0.999)
    report = {}
    if w.planted_frac > 0:
        for r in range(s.batch):
            planted = inputs.planted_pages(w, r, DEV).cpu().numpy()
            report[f"planted_recall_seq{r}"] = float(np.isin(planted, res[0][r, 0].cpu().numpy()).mean())
    # overlap of the HI selection with flat selection over every token (dynamic picks only)
    sc = lsa.index_scores(inp["q"], inp["w"], inp["keys"], inp["scale"], q_pos0=s.q_pos0)
    flat = lsa.topk_select(sc, b.k, b.sink, b.window, kv_len=s.kv_len, q_pos0=s.q_pos0)
    fl = flat.cpu().numpy()
    for r in flat_overlap_seqs:
        d = b.sink + b.window
        report[f"hi_flat_overlap_seq{r}"] = float(np.isin(gi[r, 0, d:], fl[r, 0, d:]).mean())
    del sc, flat, res
    torch.cuda.empty_cache()
    # attention of every layer over the one HI index list: one call per layer, then (several
    # layers) the same layers in one lsa_sparse_attn_layers call
    atts = [inputs.attn_inputs(w, layer, DEV) for layer in range(w.layers)]
    singles = []
    for layer, att in enumerate(atts):
        o1, l1 = lsa.sparse_attn(att["q"], att["kv"], None, idx, a.scale, b.sink, b.window,
                                 d_v=a.d_v)
        if layer == 0:
            o2, l2 = lsa.sparse_attn(att["q"], att["kv"], None, idx, a.scale, b.sink, b.window,
                                     d_v=a.d_v)
            assert torch.equal(o1, o2) and torch.equal(l1, l2)
        worst = attn_check(att["q"], att["kv"], None, idx, a.scale, o1, l1, True, a.d_v,
                           seqs=attn_seqs)
        say(f"{w.name}: layer {layer} attention worst |err| {worst:.2e}")
        singles.append(o1)
    if w.layers > 1:
        outs, lses = lsa.sparse_attn_layers([x["q"] for x in atts], [x["kv"] for x in atts], idx,
                                            a.scale, b.sink, b.window, d_v=a.d_v)
        for layer, att in enumerate(atts):
            assert (outs[layer].float() - singles[layer].float()).abs().max().item() <= 2e-2
            worst = attn_check(att["q"], att["kv"], None, idx, a.scale, outs[layer], lses[layer],
                               True, a.d_v, seqs=attn_seqs)
            say(f"{w.name}: layer {layer} of one multi-layer call, worst |err| {worst:.2e}")
        del outs, lses
    del atts, singles
    torch.cuda.empty_cache()
    say(f"{w.name}: {report}")
    return report


def test_decode_b4_1m_hi_end_to_end():
    """Long context: 4 x 1M fp8 keys with planted pages, HI with P = 64, M = 256, k = 2048,
    MLA attention over the 1M-row latent cache (sequence 3's rows sit 3.6 GB into it)."""
    rep = _hi_end_to_end(DECODE_1M_HI, check_seqs=(0, 1, 2, 3), attn_seqs=(0, 3),
                         flat_overlap_seqs=(0, 1, 2, 3))
    assert min(v for k, v in rep.items() if k.startswith("planted")) > 0.5


def test_decode_b8_256k_hi_cli4_end_to_end():
    """8 x 256K fp8 keys, HI with P = 64, M = 128, one index list reused by 4 MLA layers with
    independent caches, per layer and in one multi-layer call."""
    _hi_end_to_end(DECODE_256K_HI_CLI, check_seqs=(0, 7), attn_seqs=(0, 7),
                   flat_overlap_seqs=(0, 7))
