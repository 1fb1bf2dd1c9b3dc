#!/usr/bin/env python3
"""Benchmark of the LSA token-selection path on one MI355X.

Headline step: one decode step of the 32-sequence x 128K-token workload (fp8 indexer keys,
64 x 128 indexer, k = 2048 with a 64-token sink and a 960-token window, 16-head MLA attention
over a 576-wide latent cache), all of it on the GPU:
    lsa_index_scores -> lsa_topk_select -> lsa_sparse_attn
`value` = queries completed per second through that whole step (inputs resident in HBM).
Per-stage HIP-event times give the indexed queries/s (score + top-k) and the sparse-attention
TB/s.  Extra sections (not the headline): chunked prefill 8K @ 128K, Hierarchical Indexing at
1M tokens (with flat indexing at 1M for comparison), and Cross-Layer Indexing over 4 layers at
256K.  The CPU oracle is timed on a bounded sample of the headline workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexed queries/s (score+top-k) and sparse-attn TB/s at 128K and 1M ctx, 1 GPU"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- byte / flop counts
def score_bytes(n_queries_keys: int, d: int, fp8: bool, H: int, n_queries: int) -> float:
    """Algorithmic bytes of scoring: keys (+ per-token scale) once per (query, key) pair for
    decode, q and w per query, one fp32 score written per pair."""
    kb = d * (1 if fp8 else 2) + (4 if fp8 else 0)
    return n_queries_keys * (kb + 4) + n_queries * H * (2 * d + 4)


def attn_bytes(n_sel: int, row_bytes: int, n_queries: int, Hq: int, d_qk: int, d_v: int,
               k: int) -> float:
    return n_sel * row_bytes + n_queries * (Hq * d_qk * 2 + Hq * d_v * 2 + k * 4)


# ----------------------------------------------------------------------------- profile lookup
def source_digest(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profile_traffic(name: str, kernel_sources) -> tuple:
    """HBM bytes per launch recorded in profiles/<name>.txt by the PMC runs, if the kernel's
    sources are unchanged since (else None)."""
    path = os.path.join(ROOT, "profiles", name + ".txt")
    if not os.path.exists(path):
        return None, None
    txt = open(path).read()
    m_src = re.search(r"source_digest:\s*(\w+)", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_src or not m_b:
        return None, None
    if m_src.group(1) != source_digest(kernel_sources):
        return None, "stale"
    return float(m_b.group(1)), path


# ----------------------------------------------------------------------------- timing helper
class StageTimer:
    """HIP events recorded on the current stream around each stage of each step."""

    def __init__(self, torch, names):
        self.torch = torch
        self.names = names
        self.events = []

    def step(self):
        evs = [self.torch.cuda.Event(enable_timing=True) for _ in range(len(self.names) + 1)]
        self.events.append(evs)
        return evs

    def mean_ms(self):
        out = {n: 0.0 for n in self.names}
        for evs in self.events:
            for i, n in enumerate(self.names):
                out[n] += evs[i].elapsed_time(evs[i + 1])
        return {n: v / max(1, len(self.events)) for n, v in out.items()}


def run_timed(torch, fn, names, steps, warmup):
    for _ in range(warmup):
        fn(None)
    torch.cuda.synchronize()
    timer = StageTimer(torch, names)
    t0 = time.perf_counter()
    for _ in range(steps):
        fn(timer.step())
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    return wall, timer.mean_ms()


# ----------------------------------------------------------------------------- sections
def headline(torch, lsa, inputs, cfg, steps, warmup):
    w = cfg.DECODE_128K
    s, b, a = w.index, w.budget, w.attn
    dev = "cuda"
    log(f"[bench] generating {w.name} inputs")
    inp = inputs.index_inputs(w, dev)
    att = inputs.attn_inputs(w, 0, dev)
    B, L = s.batch, s.kv_len
    scores = torch.empty((B, 1, L), dtype=torch.float32, device=dev)
    idx = torch.empty((B, 1, b.k), dtype=torch.int32, device=dev)
    out = torch.empty((B, 1, a.heads, a.d_v), dtype=torch.bfloat16, device=dev)
    ws, ws_sel = lsa.Workspace(), lsa.Workspace()

    def step(ev):
        if ev: ev[0].record()
        lsa.index_scores(inp["q"], inp["w"], inp["keys"], inp["scale"], q_pos0=s.q_pos0, out=scores)
        if ev: ev[1].record()
        lsa.topk_select(scores, b.k, b.sink, b.window, kv_len=L, q_pos0=s.q_pos0, out=idx, ws=ws_sel)
        if ev: ev[2].record()
        lsa.sparse_attn(att["q"], att["kv"], None, idx, a.scale, b.sink, b.window, d_v=a.d_v,
                        ws=ws, out=out, want_lse=True)
        if ev: ev[3].record()

    log("[bench] headline: timing")
    # wall time of the bare step; per-stage times from a second run with events between stages
    wall, _ = run_timed(torch, lambda _ev: step(None), [], steps, warmup)
    _, st = run_timed(torch, step, ["score", "topk", "attn"], steps, warmup)
    n_q = B * s.n_q
    sb = score_bytes(n_q * L, s.head_dim, True, s.heads, n_q)
    ab = attn_bytes(n_q * b.k, a.d_qk * 2, n_q, a.heads, a.d_qk, a.d_v, b.k)
    res = {
        "wall_ms_per_step": wall,
        "stage_ms": st,
        "indexed_qps": n_q / ((st["score"] + st["topk"]) * 1e-3),
        "score_GBps": sb / (st["score"] * 1e-3) / 1e9,
        "score_hbm_frac": sb / (st["score"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "score_algorithmic_bytes": sb,
        "topk_GBps": n_q * (L - b.sink - b.window) * 4 / (st["topk"] * 1e-3) / 1e9,
        "sparse_attn_TBps": ab / (st["attn"] * 1e-3) / 1e12,
        "attn_algorithmic_bytes": ab,
    }
    del inp, att, scores, idx, out
    torch.cuda.empty_cache()
    return w, res


def extra_prefill(torch, lsa, inputs, cfg, iters=3):
    w = cfg.PREFILL_8K_AT_128K
    s, b, a = w.index, w.budget, w.attn
    dev = "cuda"
    inp = inputs.index_inputs(w, dev)
    att = inputs.attn_inputs(w, 0, dev)
    scores = torch.empty((1, s.n_q, s.kv_len), dtype=torch.float32, device=dev)
    idx = torch.empty((1, s.n_q, b.k), dtype=torch.int32, device=dev)
    out = torch.empty((1, s.n_q, a.heads, a.d_v), dtype=torch.bfloat16, device=dev)
    ws = lsa.Workspace()

    def step(ev):
        if ev: ev[0].record()
        lsa.index_scores(inp["q"], inp["w"], inp["keys"], None, q_pos0=s.q_pos0, out=scores)
        if ev: ev[1].record()
        lsa.topk_select(scores, b.k, b.sink, b.window, kv_len=s.kv_len, q_pos0=s.q_pos0, out=idx,
                        ws=ws)
        if ev: ev[2].record()
        lsa.sparse_attn(att["q"], att["kv"], None, idx, a.scale, b.sink, b.window, d_v=a.d_v,
                        ws=ws, out=out, want_lse=False)
        if ev: ev[3].record()

    wall, st = run_timed(torch, step, ["score", "topk", "attn"], iters, 1)
    V = [min(s.kv_len, s.q_pos0 + t + 1) for t in range(s.n_q)]
    pairs = sum(V)
    flops = 2.0 * pairs * s.heads * s.head_dim
    mid = sum(max(0, v - b.sink - b.window) for v in V)
    n_sel = s.n_q * b.k
    res = {
        "workload": w.name, "stage_ms": st, "wall_ms_per_step": wall,
        "score_TFLOPs": flops / (st["score"] * 1e-3) / 1e12,
        "score_mfma_frac": flops / (st["score"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS,
        "topk_GBps": mid * 4 / (st["topk"] * 1e-3) / 1e9,
        "topk_hbm_frac": mid * 4 / (st["topk"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "sparse_attn_effective_TBps": attn_bytes(n_sel, a.d_qk * 2, s.n_q, a.heads, a.d_qk, a.d_v, b.k)
        / (st["attn"] * 1e-3) / 1e12,
        "indexed_qps": s.n_q / ((st["score"] + st["topk"]) * 1e-3),
    }
    del inp, att, scores, idx, out
    torch.cuda.empty_cache()
    return res


def extra_hi(torch, lsa, inputs, w, iters=10, layers=1):
    s, b, a, hi = w.index, w.budget, w.attn, w.hi
    dev = "cuda"
    inp = inputs.index_inputs(w, dev)
    B, L = s.batch, s.kv_len
    pk = torch.empty((B, (L + hi.page - 1) // hi.page, s.head_dim), dtype=torch.bfloat16, device=dev)
    ws, ws_sel = lsa.Workspace(), lsa.Workspace()
    # page keys: built once per completed page in a decode loop; timed as a full rebuild
    wall_pk, st_pk = run_timed(
        torch, lambda ev: (ev and ev[0].record(), lsa.page_summary(inp["keys"], inp["scale"],
                                                                   hi.page, out=pk),
                           ev and ev[1].record()), ["summary"], 3, 1)
    idx = torch.empty((B, 1, b.k), dtype=torch.int32, device=dev)

    def hi_step(ev):
        if ev: ev[0].record()
        pid, cs, ci = lsa.page_recall(inp["q"], inp["w"], pk, inp["keys"], inp["scale"], b.k,
                                      b.sink, b.window, hi.page, hi.m_pages, q_pos0=s.q_pos0, ws=ws)
        if ev: ev[1].record()
        lsa.topk_select(cs, b.k, b.sink, b.window, kv_len=L, q_pos0=s.q_pos0, cand_ids=ci, out=idx,
                        ws=ws_sel)
        if ev: ev[2].record()

    _, st_hi = run_timed(torch, hi_step, ["recall", "topk"], iters, 2)
    scores = torch.empty((B, 1, L), dtype=torch.float32, device=dev)
    idx_f = torch.empty_like(idx)

    def flat_step(ev):
        if ev: ev[0].record()
        lsa.index_scores(inp["q"], inp["w"], inp["keys"], inp["scale"], q_pos0=s.q_pos0, out=scores)
        if ev: ev[1].record()
        lsa.topk_select(scores, b.k, b.sink, b.window, kv_len=L, q_pos0=s.q_pos0, out=idx_f,
                        ws=ws_sel)
        if ev: ev[2].record()

    _, st_flat = run_timed(torch, flat_step, ["score", "topk"], iters, 2)
    del scores, idx_f
    # attention layers sharing the HI index list
    atts = [inputs.attn_inputs(w, l, dev) for l in range(layers)]
    outs = [torch.empty((B, 1, a.heads, a.d_v), dtype=torch.bfloat16, device=dev) for _ in atts]

    def attn_step(ev):
        if ev: ev[0].record()
        for at, o in zip(atts, outs):
            lsa.sparse_attn(at["q"], at["kv"], None, idx, a.scale, b.sink, b.window, d_v=a.d_v,
                            ws=ws, out=o, want_lse=False)
        if ev: ev[1].record()

    _, st_attn = run_timed(torch, attn_step, ["attn"], iters, 2)
    n_q = B * s.n_q
    t_hi = st_hi["recall"] + st_hi["topk"]
    t_flat = st_flat["score"] + st_flat["topk"]
    ab = attn_bytes(n_q * b.k, a.d_qk * 2, n_q, a.heads, a.d_qk, a.d_v, b.k) * layers
    res = {
        "workload": w.name,
        "page_summary_ms": st_pk["summary"],
        "page_summary_GBps": B * L * (s.head_dim + 4) / (st_pk["summary"] * 1e-3) / 1e9,
        "hi_stage_ms": st_hi, "flat_stage_ms": st_flat,
        "hi_indexed_qps": n_q / (t_hi * 1e-3),
        "flat_indexed_qps": n_q / (t_flat * 1e-3),
        "hi_speedup_vs_flat": t_flat / t_hi,
        "attn_layers": layers,
        "attn_ms_all_layers": st_attn["attn"],
        "sparse_attn_TBps": ab / (st_attn["attn"] * 1e-3) / 1e12,
    }
    del inp, atts, outs, pk, idx
    torch.cuda.empty_cache()
    return res


def cpu_baseline(inputs, cfg, budget_s=15.0):
    """The oracle, as it stands, on a bounded sample of the headline workload: whole decode
    steps (scores, selection, attention) of as many sequences as fit in ~budget_s seconds."""
    import numpy as np
    import torch

    from oracle import ref
    w = cfg.DECODE_128K
    s, b, a = w.index, w.budget, w.attn
    n_max = 16
    inp = inputs.index_inputs(cfg.shrink(w, batch=n_max), "cpu")
    att = inputs.attn_inputs(cfg.shrink(w, batch=n_max), 0, "cpu")

    def np16(t):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)

    done, t0 = 0, time.perf_counter()
    while done < n_max:
        q, wt = np16(inp["q"][done]), inp["w"][done].numpy()
        keys, scale = inp["keys"][done].numpy().view(np.uint8), inp["scale"][done].numpy()
        I, _, _ = ref.index_scores(q, wt, keys, scale, np.array([s.q_pos0]))
        idx = ref.select(I.astype(np.float32), np.array([s.kv_len]), b.k, b.sink, b.window)
        ref.sparse_attn(np16(att["q"][done]), np16(att["kv"][done]), None, idx, a.scale,
                        d_qk=a.d_qk, d_v=a.d_v)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "queries/s", "cores": ref.num_threads(), "kind": "oracle",
            "sample": f"{done} of the 32 decode queries (whole step: scores over 131072 fp8 keys, "
                      f"selection, 16-head MLA attention), {dt:.1f} s"}


def only_stage(torch, lsa, inputs, cfg, stage, steps):
    """One stage of the headline decode step (or of the chunked prefill), `steps` times, for
    counter runs.  `copy` is the calibration kernel: out = src + 0 over 256 MiB of fp32 (reads
    and writes 256 MiB)."""
    dev = "cuda"
    if stage.startswith("prefill_"):
        w = cfg.PREFILL_8K_AT_128K
        s, b = w.index, w.budget
        inp = inputs.index_inputs(w, dev)
        scores = lsa.index_scores(inp["q"], inp["w"], inp["keys"], None, q_pos0=s.q_pos0)
        ws = lsa.Workspace()
        idx = lsa.topk_select(scores, b.k, b.sink, b.window, kv_len=s.kv_len, q_pos0=s.q_pos0, ws=ws)
        torch.cuda.synchronize()
        for _ in range(steps):
            if stage == "prefill_score":
                lsa.index_scores(inp["q"], inp["w"], inp["keys"], None, q_pos0=s.q_pos0, out=scores)
            else:
                lsa.topk_select(scores, b.k, b.sink, b.window, kv_len=s.kv_len, q_pos0=s.q_pos0,
                                out=idx, ws=ws)
        torch.cuda.synchronize()
        log(f"[bench] {stage} x{steps} done")
        return
    if stage == "copy":
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(steps):
            torch.add(src, 0.0, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] copy x{steps}: {src.numel() * 4} bytes read and written per launch")
        return
    w = cfg.DECODE_128K
    s, b, a = w.index, w.budget, w.attn
    inp = inputs.index_inputs(w, dev)
    L = s.kv_len
    scores = lsa.index_scores(inp["q"], inp["w"], inp["keys"], inp["scale"], q_pos0=s.q_pos0)
    ws = lsa.Workspace()
    idx = lsa.topk_select(scores, b.k, b.sink, b.window, kv_len=L, q_pos0=s.q_pos0, ws=ws)
    att = inputs.attn_inputs(w, 0, dev) if stage == "attn" else None
    torch.cuda.synchronize()
    for _ in range(steps):
        if stage == "score":
            lsa.index_scores(inp["q"], inp["w"], inp["keys"], inp["scale"], q_pos0=s.q_pos0,
                             out=scores)
        elif stage == "topk":
            lsa.topk_select(scores, b.k, b.sink, b.window, kv_len=L, q_pos0=s.q_pos0, out=idx,
                            ws=ws)
        else:
            lsa.sparse_attn(att["q"], att["kv"], None, idx, a.scale, b.sink, b.window,
                            d_v=a.d_v, ws=ws)
    torch.cuda.synchronize()
    log(f"[bench] {stage} x{steps} done")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--extras", action=argparse.BooleanOptionalAction, default=True)
    ap.add_argument("--cpu-baseline", action=argparse.BooleanOptionalAction, default=True)
    ap.add_argument("--only", choices=["score", "topk", "attn", "copy", "prefill_score", "prefill_topk"],
                    help="run one stage of the headline step (or a plain 256 MiB device copy) "
                         "--steps times and exit; for hardware-counter runs under rocprofv3")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}): the LSA path "
              f"is built and measured on a single MI355X (decode would shard the batch across "
              f"GPUs, longer contexts the key length; that exchange is not built).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from token_selection_indexer_amd import configs as cfg
    from token_selection_indexer_amd import inputs, lsa
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    lsa.lib()
    torch.cuda.set_device(0)
    if args.only:
        only_stage(torch, lsa, inputs, cfg, args.only, args.steps)
        return

    w, head = headline(torch, lsa, inputs, cfg, args.steps, args.warmup)
    s, b = w.index, w.budget
    n_q = s.batch * s.n_q
    value = n_q / (head["wall_ms_per_step"] * 1e-3)

    score_src = ["token_selection_indexer_amd/csrc/score.hip",
                 "token_selection_indexer_amd/csrc/device.hpp"]
    traffic, _ = profile_traffic("score_stream_decode_b32_128k_pmc", score_src)
    t_score = head["stage_ms"]["score"] * 1e-3
    roof = {"kernel": "score_stream_kernel (lsa_index_scores, fp8 keys, decode)",
            "bound": "hbm", "achieved": head["score_algorithmic_bytes"] / t_score / 1e9,
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": head["score_algorithmic_bytes"] / t_score / 1e9 / HBM_PEAK_GBS,
            "traffic": traffic}

    extras = {}
    if args.extras:
        log("[bench] extra: chunked prefill 8K @ 128K")
        extras["prefill_8k_128k"] = extra_prefill(torch, lsa, inputs, cfg)
        log("[bench] extra: HI at 1M")
        extras["decode_1m_hi"] = extra_hi(torch, lsa, inputs, cfg.DECODE_1M_HI)
        log("[bench] extra: HI + cross-layer x4 at 256K")
        extras["decode_256k_hi_cli4"] = extra_hi(torch, lsa, inputs, cfg.DECODE_256K_HI_CLI,
                                                 layers=cfg.DECODE_256K_HI_CLI.layers)
    cpu = None
    if args.cpu_baseline:
        log("[bench] CPU oracle baseline")
        cpu = cpu_baseline(inputs, cfg)

    line = {
        "metric": METRIC, "value": value, "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["wall_ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": s.batch, "kv_len": s.kv_len,
                   "indexer": f"{s.heads}x{s.head_dim} fp8-e4m3 keys", "k": b.k,
                   "sink": b.sink, "window": b.window, "attn": "MLA 16 heads, 576/512 latent"},
        "indexed_qps": head["indexed_qps"],
        "sparse_attn_TBps": head["sparse_attn_TBps"],
        "stage_ms": head["stage_ms"],
        "roofline": roof,
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
