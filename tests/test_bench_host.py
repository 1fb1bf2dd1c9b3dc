"""bench.py on the host (no GPU): it refuses more than one GPU before touching one, and its
algorithmic byte counts are the per-unit figures the roofline is stated in (written out here
from the shapes, not from bench.py's own helpers)."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, env=e, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2 and "one GPU" in r.stderr
    r = _run([], env={"WORLD_SIZE": "8"})
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_algorithmic_bytes_of_the_decode_workload():
    b = _bench()
    # scores: 32 queries x 131072 fp8 keys, each pair reading a 128-byte key row and its fp32
    # scale and writing one fp32 score; each query reads 64 x 128 bf16 q and 64 fp32 w
    n_q, L, H, d = 32, 131072, 64, 128
    assert b.score_bytes(n_q * L, d, True, H, n_q) == n_q * L * (128 + 4 + 4) + n_q * H * (256 + 4)
    assert b.score_bytes(n_q * L, d, True, H, n_q) == 570_957_824
    # attention: 2048 latent rows of 576 bf16 per query, plus 16 heads of q (576) and out (512)
    # in bf16 and the 2048-entry int32 list
    assert b.attn_bytes(n_q * 2048, 1152, n_q, 16, 576, 512, 2048) == 76_873_728
    # page recall at 4 x 1M, P = 64, M = 256: every eligible page key (bf16 128 + fp32 coarse
    # score), then 256 pages x 64 candidate rows (fp8 row + scale, score + id written)
    n_pages = (1 << 20) // 64
    assert b.recall_bytes(4, n_pages, 128, 256, 64, True) == 4 * (n_pages * 260 + 16384 * 140)


def test_warm_queueing_only_for_short_stages():
    b = _bench()
    assert 0.0 < b.SHORT_STAGE_MS < 0.1  # the decode index stage (about 0.12 ms) is not queued


def test_paged_copy_places_every_block_by_its_table_entry():
    import torch
    b = _bench()
    kv = torch.arange(3 * 256 * 8, dtype=torch.float32).view(3, 256, 8)
    pool, tab = b.paged_copy(torch, kv, 64)
    assert pool.shape == (12, 64, 8) and tab.shape == (3, 4) and tab.dtype == torch.int32
    assert sorted(tab.view(-1).tolist()) == list(range(12))
    for s in range(3):
        for j in range(4):
            assert torch.equal(pool[tab[s, j]], kv[s, 64 * j:64 * (j + 1)])
