"""The no-allocation selection entry point (lsa_topk_select_noalloc) against lsa_topk_select.

Two calls in a row through the C ABI, the second with a smaller input, each compared bit for bit
with lsa_topk_select on the same scores (which tests/test_gpu_parity.py ties to the oracle):
  1. the decode workload's shape, 32 rows x 131072 flat scores (the chunked path: scratch used);
  2. 4 candidate rows of 40000 (chunked, fewer chunks) with holes and a short row.
Then a call that needs no scratch (many short rows) and a third chunked call, to check that what
the scratch held from earlier calls does not leak into a later one."""
import numpy as np
import pytest
import torch

from oracle import ref
from token_selection_indexer_amd import inputs, lsa
from tests.util import check_si_layout

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(shape, bud, sc, n, cand):
    B, T = shape.batch, shape.n_q
    want = torch.empty((B, T, bud.k), dtype=torch.int32, device=DEV)
    nb = lsa.lsa_workspace_bytes(lsa.OP_TOPK_SELECT, shape, bud, n_cand=n)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=DEV)
    lsa.lsa_topk_select(shape, bud, sc, n, cand, want, ws if nb else None, nb)
    got = torch.full((B, T, bud.k), -7, dtype=torch.int32, device=DEV)
    lsa.lsa_topk_select_noalloc(shape, bud, sc, n, cand, got)
    torch.cuda.synchronize()
    return nb, got.cpu().numpy(), want.cpu().numpy()


def test_noalloc_matches_workspace_entry_point():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lsa.lib()
    # 1. decode shape, flat
    L, bud = 131072, lsa.Budget(2048, 64, 960)
    sc = inputs.synthetic_scores(32, L, seed=51, ties="zeros", device=DEV).reshape(32, 1, L)
    sh = lsa.IndexShape(32, 1, 64, 128, L, L - 1)
    nb, got, want = _both(sh, bud, sc, L, None)
    assert nb > 0  # the chunked path, through the scratch
    assert np.array_equal(got, want)
    scn = sc.cpu().numpy()
    for r in (0, 31):
        assert np.array_equal(got[r], ref.select(scn[r], np.array([L]), 2048, 64, 960))
    # 2. smaller: candidate rows
    n, bud2 = 40000, lsa.Budget(2048, 128, 896)
    sc2 = inputs.synthetic_scores(4, n, seed=52, ties="coarse", device=DEV).reshape(4, 1, n)
    g = torch.Generator().manual_seed(3)
    ids = torch.stack([torch.sort(torch.randperm(1 << 20, generator=g)[:n]).values
                       for _ in range(4)]).to(torch.int32).reshape(4, 1, n)
    ids[:, :, 5::9] = -1
    ids[2, 0, 700:] = -1
    ids = ids.to(DEV)
    sh2 = lsa.IndexShape(4, 1, 64, 128, 1 << 20, (1 << 20) - 1)
    nb2, got2, want2 = _both(sh2, bud2, sc2, n, ids)
    assert 0 < nb2 < nb
    assert np.array_equal(got2, want2)
    for r in range(4):
        check_si_layout(got2[r, 0], 1 << 20, 2048, 128, 896, cand_ids=ids[r, 0].cpu().numpy())
    # 3. no scratch needed (one workgroup per row), then chunked again at another shape
    sc3 = inputs.synthetic_scores(64, 5000, seed=53, device=DEV).reshape(8, 8, 5000)
    nb3, got3, want3 = _both(lsa.IndexShape(8, 8, 64, 128, 5000, 4992), lsa.Budget(256, 16, 112),
                             sc3, 5000, None)
    assert nb3 == 0 and np.array_equal(got3, want3)
    sc4 = inputs.synthetic_scores(3, 70000, seed=54, ties="inf", device=DEV).reshape(3, 1, 70000)
    nb4, got4, want4 = _both(lsa.IndexShape(3, 1, 64, 128, 70000, 69999), lsa.Budget(1024, 32, 480),
                             sc4, 70000, None)
    assert nb4 > 0 and np.array_equal(got4, want4)
