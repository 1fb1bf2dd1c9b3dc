"""fp8 queries (lsa_quantize_queries + lsa_index_scores_q8) on the GPU against the oracle.

Quantised queries and their scales must equal the oracle's bit for bit (the quantisation is a
definition both sides follow in binary32).  Scores of the quantised queries must match the
oracle's scores of the same quantised queries within the usual score tolerance.  How far the
quantised-query selection moves from the bf16-query selection is printed (a quality figure of
the approximation, not a parity bar).
"""
import numpy as np
import pytest
import torch

from oracle import ref
from token_selection_indexer_amd import inputs, lsa
from token_selection_indexer_amd.configs import (PREFILL_8K_AT_128K, TINY_PREFILL_4K, IndexShape,
                                                 Workload)
from tests.gpu_checks import assert_scores, say
from tests.util import bits, f32, keys_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lsa.lib()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("d", [64, 128])
def test_quantize_queries_bit_exact(d):
    g = torch.Generator(device=DEV).manual_seed(9)
    B, T, H = 3, 7, 16
    x = torch.randn((B, T, H, d), generator=g, device=DEV)
    x = x * torch.exp(torch.randn((B, T, H, 1), generator=g, device=DEV) * 4)  # wide magnitudes
    q = x.to(torch.bfloat16)
    q[0, 0, 3] = 0                       # all-zero row
    q[1, 2, 5] = 0
    q[1, 2, 5, 7] = 1e-30                # a lone subnormal-sized value
    q8, qs = lsa.quantize_queries(q)
    rc, rs = ref.quantize_rows(bits(q))
    assert np.array_equal(q8.cpu().numpy(), rc)
    assert np.array_equal(qs.cpu().numpy().view(np.uint32), rs.view(np.uint32))


def _q8_case(w, rows=None):
    s = w.index
    inp = inputs.index_inputs(w, DEV)
    q8, qs = lsa.quantize_queries(inp["q"])
    sc = lsa.index_scores_q8(q8, qs, inp["w"], inp["keys"], inp["scale"], q_pos0=s.q_pos0)
    torch.cuda.synchronize()
    return inp, q8, qs, sc


@pytest.mark.parametrize("H,d", [(64, 128), (4, 64), (16, 128), (32, 64)])
@pytest.mark.parametrize("n_q", [1, 3, 37])
def test_q8_scores_small_ragged(H, d, n_q):
    L = 1000  # not a multiple of the 256-key tile
    w = Workload(name="q8", index=IndexShape(batch=2, n_q=n_q, kv_len=L, q_pos0=L - n_q - 5,
                                             heads=H, head_dim=d, key_dtype="fp8"),
                 budget=TINY_PREFILL_4K.budget, attn=TINY_PREFILL_4K.attn, seed=91)
    inp, q8, qs, sc = _q8_case(w)
    q8n, qsn, scn = q8.cpu().numpy(), qs.cpu().numpy(), sc.cpu().numpy()
    for b in range(2):
        keys, scale = keys_np(inp, b)
        I, A, E = ref.index_scores_q8(q8n[b], qsn[b], f32(inp["w"][b]), keys, scale,
                                      w.index.q_pos0 + np.arange(n_q))
        assert_scores(scn[b], I, A, E, f"b={b}")


def test_q8_prefill_8k_at_128k_sampled_and_quality():
    """The chunked-prefill shape (8192 queries x 131072 keys) with fp8 keys: whole rows of three
    queries against the oracle; then the overlap of the quantised-query and bf16-query
    selections is reported."""
    from dataclasses import replace
    w = replace(PREFILL_8K_AT_128K, index=replace(PREFILL_8K_AT_128K.index, key_dtype="fp8"))
    s, b = w.index, w.budget
    inp, q8, qs, sc = _q8_case(w)
    rows = [0, 4097, 8191]
    keys, scale = keys_np(inp, 0)
    I, A, E = ref.index_scores_q8(q8[0].cpu().numpy()[rows], qs[0].cpu().numpy()[rows],
                                  f32(inp["w"][0])[rows], keys, scale, s.q_pos0 + np.array(rows))
    for i, t in enumerate(rows):
        assert_scores(sc[0, t].cpu().numpy(), I[i], A[i], E[i], f"row {t}")
    idx8 = lsa.topk_select(sc, b.k, b.sink, b.window, kv_len=s.kv_len, q_pos0=s.q_pos0)
    del sc
    torch.cuda.empty_cache()
    sc16 = lsa.index_scores(inp["q"], inp["w"], inp["keys"], inp["scale"], q_pos0=s.q_pos0)
    idx16 = lsa.topk_select(sc16, b.k, b.sink, b.window, kv_len=s.kv_len, q_pos0=s.q_pos0)
    torch.cuda.synchronize()
    d0 = b.sink + b.window
    a8, a16 = idx8[0, :, d0:].cpu().numpy(), idx16[0, :, d0:].cpu().numpy()
    ov = np.mean([np.isin(a8[t], a16[t]).mean() for t in range(0, s.n_q, 64)])
    say(f"fp8-query vs bf16-query dynamic selection overlap (128 sampled rows): {ov:.4f}")
    assert ov > 0.5
