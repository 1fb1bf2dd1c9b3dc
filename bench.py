#!/usr/bin/env python3
"""Benchmark of the LSA token-selection path on one MI355X.

Headline workload: decode, 32 sequences x 131072 tokens (fp8 indexer keys, 64 x 128 indexer,
k = 2048 with a 64-token sink and a 960-token window, 16-head MLA attention over a 576-wide
latent cache).  One step is the whole path on the GPU, inputs resident in HBM:
    lsa_index_select (scores + selection, fused) -> lsa_sparse_attn
`value` is the metric's indexed queries/s: queries / (score + top-k time), from HIP events
recorded around each stage of the K timed steps; `ms_per_step` is the wall time of a whole step
(attention included).  The unfused stages (lsa_index_scores, lsa_topk_select) are timed too.  Every stage is also timed on its own, >= 50 runs (or >= 200 ms), warm
(back to back) and cold (L2 and the 256 MB MALL flushed by reading 1 GiB before each run), as
median / p10 / p90 / mean.  Extra sections: chunked prefill 8K @ 128K, Hierarchical Indexing at
1M tokens and at 256K (flat indexing timed beside it, planted-page recall and HI/flat overlap
reported), cross-layer reuse over 4 layers.  The CPU oracle is timed on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu-baseline]
    python bench.py --only STAGE [--cold] --steps N     (one stage N times, for rocprofv3)
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
MFMA_FP8_PEAK_TFS = 5000.0
FLUSH_BYTES = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- byte / flop counts
def score_bytes(n_pairs: int, d: int, fp8: bool, H: int, n_queries: int) -> float:
    """Algorithmic bytes of decode scoring: every valid (query, key) pair reads the key row (+ its
    fp32 scale) and writes one fp32 score; every query reads its q and w."""
    kb = d * (1 if fp8 else 2) + (4 if fp8 else 0)
    return n_pairs * (kb + 4) + n_queries * H * (2 * d + 4)


def attn_bytes(n_sel: int, row_bytes: int, n_queries: int, Hq: int, d_qk: int, d_v: int,
               k: int) -> float:
    """Selected rows gathered once each, plus q, out and the index list per query."""
    return n_sel * row_bytes + n_queries * (Hq * d_qk * 2 + Hq * d_v * 2 + k * 4)


def recall_bytes(n_q: int, n_elig: int, d: int, M: int, P: int, fp8: bool) -> float:
    """Page recall per query: eligible page keys (bf16) + coarse score written, then the recalled
    pages' key rows (+ scales) with one fp32 score and one id written per candidate."""
    kb = d * (1 if fp8 else 2) + (4 if fp8 else 0)
    return n_q * (n_elig * (2 * d + 4) + M * P * (kb + 8))


# ----------------------------------------------------------------------------- profile lookup
def source_digest(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profile_traffic(name: str, kernel_sources):
    """HBM bytes per launch recorded in profiles/<name>.txt by the PMC runs, if the kernel's
    sources are unchanged since (else None)."""
    path = os.path.join(ROOT, "profiles", name + ".txt")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_src = re.search(r"source_digest:\s*(\w+)", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_src or not m_b or m_src.group(1) != source_digest(kernel_sources):
        return None
    return float(m_b.group(1))


# ----------------------------------------------------------------------------- timing
SHORT_STAGE_MS = 0.06  # warm runs of stages up to this long are queued behind a GPU wait


class Timing:
    """HIP events on the current stream (the stream the binding hands the library), and a 1 GiB
    buffer streamed through to flush L2 and the MALL before cold runs."""

    def __init__(self, torch):
        self.torch = torch
        self._flush = None

    def flush(self):
        """Read 1 GiB (a sum into one preallocated scalar): every line of L2 and the MALL is
        replaced by a clean one.  A read-only stream on purpose: a flush that wrote its buffer
        would leave dirty lines whose write-back lands in the timed run that follows."""
        if self._flush is None:
            self._flush = self.torch.ones(FLUSH_BYTES // 4, dtype=self.torch.float32,
                                          device="cuda")
            self._acc = self.torch.zeros((), dtype=self.torch.float32, device="cuda")
        self.torch.sum(self._flush, dim=0, out=self._acc)

    def queue_ahead(self, runs: int):
        """Warm runs of short stages: hold the GPU in a timed-out wait (about 0.3 ms per run, at
        most 40 ms) while the host enqueues every run, so that each run's events bracket its
        kernels and not the host's time to launch them (a stage shorter than its Python call
        would otherwise time the host).  The wait itself is outside every event pair.  Long
        stages keep the GPU ahead of the host by themselves, and after such a wait the chip
        runs them slower (its clocks drop while it idles), so they are not queued; cold runs
        need none either: the flush before each keeps the GPU busy while the host catches up."""
        try:
            self.torch.cuda._sleep(int(2.4e9 * min(0.04, 3e-4 * runs)))
        except (AttributeError, RuntimeError):
            pass

    def stats(self, fn, est_ms: float, cold: bool, runs=None, queue=None):
        """>= 50 runs (>= 200 ms for long stages) of fn, each between two events; returns
        mean / median / p10 / p90 / min in ms."""
        torch = self.torch
        if runs is None:
            runs = 50 if est_ms * 50 <= 1000 else max(15, math.ceil(200.0 / est_ms))
        fn()
        torch.cuda.synchronize()
        if not cold and (est_ms <= SHORT_STAGE_MS if queue is None else queue):
            self.queue_ahead(runs)
        evs = []
        for _ in range(runs):
            if cold:
                self.flush()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) for a, b in evs)

        def pct(p):
            x = (len(t) - 1) * p
            lo, hi = int(math.floor(x)), int(math.ceil(x))
            return t[lo] + (t[hi] - t[lo]) * (x - lo)
        return {"n": runs, "mean": sum(t) / len(t), "median": pct(0.5), "p10": pct(0.1),
                "p90": pct(0.9), "min": t[0]}

    def both(self, fn, est_ms, cold_too=True, queue=None):
        """queue: force (True) or forbid (False) queueing the warm runs; None decides by est_ms."""
        out = {"warm": self.stats(fn, est_ms, cold=False, queue=queue)}
        if cold_too:
            out["cold"] = self.stats(fn, est_ms, cold=True)
        return out


PAGE_BLOCK = 64  # rows per block of the paged cache timed beside the dense one
HI_PAGE_BLOCK = 256  # ... and for Hierarchical Indexing (a table block holds whole pages)


def paged_copy(torch, kv, bs):
    """A dense cache [B, L, row] as a pool of bs-row blocks in a random order, and its block
    table [B, L / bs] (L a multiple of bs)."""
    B, L, row = kv.shape
    n = B * (L // bs)
    g = torch.Generator(device=kv.device).manual_seed(7)
    perm = torch.randperm(n, device=kv.device, generator=g)
    pool = torch.empty((n, bs, row), dtype=kv.dtype, device=kv.device)
    pool[perm] = kv.reshape(n, bs, row)
    return pool, perm.view(B, L // bs).to(torch.int32)


def rnd(x, nd=4):
    if isinstance(x, dict):
        return {k: rnd(v, nd) for k, v in x.items()}
    if isinstance(x, float):
        return float(f"{x:.{nd}g}")
    return x


# ----------------------------------------------------------------------------- headline
def headline(torch, lsa, inputs, cfg, tm: Timing, steps, warmup):
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
    ws, ws_sel, ws_idx = lsa.Workspace(), lsa.Workspace(), lsa.Workspace()

    def f_index():  # scores + selection, fused
        lsa.index_select(inp["q"], inp["w"], inp["keys"], inp["scale"], b.k, b.sink, b.window,
                         q_pos0=s.q_pos0, scores=scores, idx=idx, ws=ws_idx)

    def f_score():
        lsa.index_scores(inp["q"], inp["w"], inp["keys"], inp["scale"], q_pos0=s.q_pos0, out=scores)

    def f_topk():
        lsa.topk_select(scores, b.k, b.sink, b.window, kv_len=L, q_pos0=s.q_pos0, out=idx,
                        ws=ws_sel)

    def f_attn():
        lsa.sparse_attn(att["q"], att["kv"], None, idx, a.scale, b.sink, b.window, d_v=a.d_v,
                        ws=ws, out=out, want_lse=True)

    for _ in range(warmup):
        f_index(), f_attn()
    torch.cuda.synchronize()
    log(f"[bench] headline: {steps} timed steps")
    evs = []
    t0 = time.perf_counter()
    for _ in range(steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        f_index()
        e[1].record()
        f_attn()
        e[2].record()
        evs.append(e)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) / steps * 1e3
    st = {n: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / steps
          for i, n in enumerate(("index", "attn"))}
    log("[bench] headline: per-stage distributions (warm and cold)")
    dist = {"index": tm.both(f_index, st["index"]), "score": tm.both(f_score, 0.1),
            "topk": tm.both(f_topk, 0.02), "attn": tm.both(f_attn, st["attn"])}
    # the same attention over a paged copy of the cache: 64-row blocks in a shuffled pool
    pool, tab = paged_copy(torch, att["kv"], PAGE_BLOCK)

    def f_attn_paged():
        lsa.sparse_attn(att["q"], pool, None, idx, a.scale, b.sink, b.window, d_v=a.d_v, ws=ws,
                        out=out, want_lse=True, block_table=tab, kv_len=L)
    f_attn_paged()
    dist["attn_paged"] = tm.both(f_attn_paged, st["attn"])
    del pool, tab
    # and the fused scores + selection over paged indexer keys (64-row blocks, shuffled)
    kpool, ktab = paged_copy(torch, inp["keys"], PAGE_BLOCK)
    spool, stab = paged_copy(torch, inp["scale"].unsqueeze(-1), PAGE_BLOCK)
    spool = spool.squeeze(-1)
    assert torch.equal(stab, ktab)  # one seeded order for both pools

    def f_index_paged():
        lsa.index_select(inp["q"], inp["w"], kpool, spool, b.k, b.sink, b.window,
                         q_pos0=s.q_pos0, scores=scores, idx=idx, ws=ws_idx, block_table=ktab,
                         kv_len=L)
    f_index_paged()
    dist["index_paged"] = tm.both(f_index_paged, st["index"])
    del kpool, spool, ktab
    f_index()
    n_q = B * s.n_q
    sb = score_bytes(n_q * L, s.head_dim, True, s.heads, n_q)
    ab = attn_bytes(n_q * b.k, a.d_qk * 2, n_q, a.heads, a.d_qk, a.d_v, b.k)
    tb = n_q * (L - b.sink - b.window) * 4 + n_q * b.k * 4
    res = {
        "wall_ms_per_step": wall_ms, "stage_ms": st, "dist": dist,
        "indexed_qps": n_q / (st["index"] * 1e-3),
        "indexed_qps_unfused": n_q / ((dist["score"]["warm"]["mean"] + dist["topk"]["warm"]["mean"]) * 1e-3),
        "step_qps": n_q / (wall_ms * 1e-3),
        "score_algorithmic_bytes": sb, "attn_algorithmic_bytes": ab, "topk_algorithmic_bytes": tb,
        "sparse_attn_TBps": ab / (st["attn"] * 1e-3) / 1e12,
        "hbm_frac_cold_mean": {
            "index_fused": (sb + tb) / (dist["index"]["cold"]["mean"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "score": sb / (dist["score"]["cold"]["mean"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "topk": tb / (dist["topk"]["cold"]["mean"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "attn": ab / (dist["attn"]["cold"]["mean"] * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "hbm_frac_warm_mean": {
            "index_fused": (sb + tb) / (dist["index"]["warm"]["mean"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "score": sb / (dist["score"]["warm"]["mean"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "topk": tb / (dist["topk"]["warm"]["mean"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "attn": ab / (dist["attn"]["warm"]["mean"] * 1e-3) / 1e9 / HBM_PEAK_GBS},
    }
    del inp, att, scores, idx, out
    torch.cuda.empty_cache()
    return w, res


# ----------------------------------------------------------------------------- extras
def extra_prefill(torch, lsa, inputs, cfg, tm: Timing):
    w = cfg.PREFILL_8K_AT_128K
    s, b, a = w.index, w.budget, w.attn
    dev = "cuda"
    inp = inputs.index_inputs(w, dev)
    att = inputs.attn_inputs(w, 0, dev)
    scores = torch.empty((1, s.n_q, s.kv_len), dtype=torch.float32, device=dev)
    idx = torch.empty((1, s.n_q, b.k), dtype=torch.int32, device=dev)
    out = torch.empty((1, s.n_q, a.heads, a.d_v), dtype=torch.bfloat16, device=dev)
    ws = lsa.Workspace()

    def f_score():
        lsa.index_scores(inp["q"], inp["w"], inp["keys"], None, q_pos0=s.q_pos0, out=scores)

    def f_topk():
        lsa.topk_select(scores, b.k, b.sink, b.window, kv_len=s.kv_len, q_pos0=s.q_pos0, out=idx,
                        ws=ws)

    def f_attn():
        lsa.sparse_attn(att["q"], att["kv"], None, idx, a.scale, b.sink, b.window, d_v=a.d_v,
                        ws=ws, out=out, want_lse=False)

    f_score(), f_topk(), f_attn()
    d = {"score": tm.both(f_score, 14.0),               # keys + q: 170 MB, cold matters
         "topk": tm.both(f_topk, 0.85, cold_too=False),  # reads 4.2 GB: never cache-resident
         "attn": tm.both(f_attn, 2.1)}
    V = [min(s.kv_len, s.q_pos0 + t + 1) for t in range(s.n_q)]
    flops = 2.0 * sum(V) * s.heads * s.head_dim
    mid = sum(max(0, v - b.sink - b.window) for v in V)
    t_s, t_k, t_a = (d["score"]["warm"]["mean"], d["topk"]["warm"]["mean"],
                     d["attn"]["warm"]["mean"])
    res = {
        "workload": w.name, "dist": d,
        "score_TFLOPs": flops / (t_s * 1e-3) / 1e12,
        "score_mfma_frac": flops / (t_s * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS,
        "score_mfma_frac_cold": flops / (d["score"]["cold"]["mean"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS,
        "score_flops": flops,
        "topk_GBps": (mid + s.n_q * b.k) * 4 / (t_k * 1e-3) / 1e9,
        "topk_hbm_frac": (mid + s.n_q * b.k) * 4 / (t_k * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "sparse_attn_effective_TBps": attn_bytes(s.n_q * b.k, a.d_qk * 2, s.n_q, a.heads, a.d_qk,
                                                 a.d_v, b.k) / (t_a * 1e-3) / 1e12,
        "indexed_qps": s.n_q / ((t_s + t_k) * 1e-3),
    }
    del inp, att, scores, idx, out
    torch.cuda.empty_cache()
    return res


def extra_prefill_q8(torch, lsa, inputs, cfg, tm: Timing):
    """The chunked-prefill shape with fp8 keys, scored with fp8 queries on the 8-bit MFMA
    (quantisation timed apart) and, beside it, with bf16 queries against the same fp8 keys."""
    from dataclasses import replace
    base = cfg.PREFILL_8K_AT_128K
    w = replace(base, name=base.name + "_fp8keys", index=replace(base.index, key_dtype="fp8"))
    s, b = w.index, w.budget
    dev = "cuda"
    inp = inputs.index_inputs(w, dev)
    scores = torch.empty((1, s.n_q, s.kv_len), dtype=torch.float32, device=dev)
    q8, qs = lsa.quantize_queries(inp["q"])

    def f_quant():
        lsa.quantize_queries(inp["q"], q8=q8, q_scale=qs)

    def f_q8():
        lsa.index_scores_q8(q8, qs, inp["w"], inp["keys"], inp["scale"], q_pos0=s.q_pos0, out=scores)

    def f_bf16q():
        lsa.index_scores(inp["q"], inp["w"], inp["keys"], inp["scale"], q_pos0=s.q_pos0, out=scores)

    f_quant(), f_q8(), f_bf16q()
    d = {"quantize": tm.both(f_quant, 0.05, cold_too=False), "score_q8": tm.both(f_q8, 8.0),
         "score_bf16q": tm.both(f_bf16q, 14.0)}
    V = [min(s.kv_len, s.q_pos0 + t + 1) for t in range(s.n_q)]
    flops = 2.0 * sum(V) * s.heads * s.head_dim
    t8, t16 = d["score_q8"]["warm"]["mean"], d["score_bf16q"]["warm"]["mean"]
    res = {"workload": w.name, "dist": d, "score_flops": flops,
           "score_q8_TFLOPs": flops / (t8 * 1e-3) / 1e12,
           "score_q8_mfma_frac_fp8_peak": flops / (t8 * 1e-3) / 1e12 / MFMA_FP8_PEAK_TFS,
           "score_bf16q_TFLOPs": flops / (t16 * 1e-3) / 1e12,
           "speedup_q8_vs_bf16q": t16 / t8,
           "indexed_qps_q8": s.n_q / ((t8 + d["quantize"]["warm"]["mean"]) * 1e-3)}
    del inp, scores, q8, qs
    torch.cuda.empty_cache()
    return res


def _bwd_setup(torch, lsa, inputs, cfg):
    """The chunked-prefill shape's training step: its selection, the forward attention (out,
    lse) and random output / score gradients, for the two backward calls."""
    w = cfg.PREFILL_8K_AT_128K
    s, b, a = w.index, w.budget, w.attn
    dev = "cuda"
    inp = inputs.index_inputs(w, dev)
    att = inputs.attn_inputs(w, 0, dev)
    scores = lsa.index_scores(inp["q"], inp["w"], inp["keys"], None, q_pos0=s.q_pos0)
    idx = lsa.topk_select(scores, b.k, b.sink, b.window, kv_len=s.kv_len, q_pos0=s.q_pos0)
    del scores
    out, lse = lsa.sparse_attn(att["q"], att["kv"], None, idx, a.scale, b.sink, b.window, d_v=a.d_v)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed + 100)
    d_out = torch.randn(out.shape, generator=g, device=dev).to(torch.bfloat16)
    d_sc = torch.randn(idx.shape, generator=g, device=dev)
    grads = {"d_q": torch.zeros((1, s.n_q, a.heads, a.d_qk), dtype=torch.float32, device=dev),
             "d_kv": torch.zeros((1, s.kv_len, a.d_qk), dtype=torch.float32, device=dev),
             "di_q": torch.zeros((1, s.n_q, s.heads, s.head_dim), dtype=torch.float32, device=dev),
             "di_w": torch.zeros((1, s.n_q, s.heads), dtype=torch.float32, device=dev),
             "di_k": torch.zeros((1, s.kv_len, s.head_dim), dtype=torch.float32, device=dev)}

    def f_attn_bwd():
        lsa.sparse_attn_backward(att["q"], att["kv"], None, idx, out, lse, d_out, a.scale,
                                 d_v=a.d_v, d_q=grads["d_q"], d_k=grads["d_kv"], sink=b.sink,
                                 window=b.window, q_pos0=s.q_pos0)

    def f_index_bwd():
        lsa.index_scores_backward(inp["q"], inp["w"], inp["keys"], idx, d_sc, q_pos0=s.q_pos0,
                                  d_q=grads["di_q"], d_w=grads["di_w"], d_keys=grads["di_k"],
                                  sink=b.sink, window=b.window)
    return w, f_attn_bwd, f_index_bwd


def extra_backward(torch, lsa, inputs, cfg, tm: Timing):
    """The training path at the chunked-prefill shape (8192 queries over 128K keys, k = 2048):
    the sparse-attention backward (MLA 16 x 576/512) and the indexer backward (64 x 128, bf16
    keys) over the GPU's own selection.  Gradients are added into fp32 arrays, so repeated calls
    accumulate; the timed region is the call alone."""
    w, f_attn_bwd, f_index_bwd = _bwd_setup(torch, lsa, inputs, cfg)
    s, b, a = w.index, w.budget, w.attn
    f_attn_bwd(), f_index_bwd()
    d = {"attn_bwd": tm.both(f_attn_bwd, 60.0, cold_too=False),
         "index_bwd": tm.both(f_index_bwd, 30.0, cold_too=False)}
    n_sel = s.n_q * b.k
    # entries whose cache (key) gradient the key-major passes sum over queries before adding it
    # (the sink and window entries of every query whose sink and window are disjoint); the
    # query-major kernels add the rest, one fp32 atomic per row column
    t_si = max(0, b.sink + b.window - s.q_pos0 - 1)
    n_si = max(0, s.n_q - t_si) * (b.sink + b.window)
    attn_flops = 2.0 * n_sel * a.heads * (3 * a.d_qk + 2 * a.d_v)
    idx_flops = 2.0 * 3 * n_sel * s.heads * s.head_dim
    ta, ti = d["attn_bwd"]["warm"]["mean"], d["index_bwd"]["warm"]["mean"]
    res = {"workload": w.name + "_backward", "dist": d,
           "attn_bwd_flops": attn_flops, "attn_bwd_TFLOPs": attn_flops / (ta * 1e-3) / 1e12,
           "attn_bwd_mfma_frac": attn_flops / (ta * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS,
           "attn_bwd_entries": n_sel, "attn_bwd_entries_key_major": n_si,
           "attn_bwd_G_entries_per_s": n_sel / (ta * 1e-3) / 1e9,
           "attn_bwd_atomic_updates_query_major": (n_sel - n_si) * a.d_qk,
           "index_bwd_flops": idx_flops, "index_bwd_TFLOPs": idx_flops / (ti * 1e-3) / 1e12,
           "index_bwd_mfma_frac": idx_flops / (ti * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS,
           "index_bwd_entries": n_sel, "index_bwd_entries_key_major": n_si,
           "index_bwd_G_entries_per_s": n_sel / (ti * 1e-3) / 1e9,
           "index_bwd_atomic_updates_query_major": (n_sel - n_si) * s.head_dim}
    torch.cuda.empty_cache()
    return res


def extra_hi(torch, lsa, inputs, w, tm: Timing):
    import numpy as np
    s, b, a, hi = w.index, w.budget, w.attn, w.hi
    dev = "cuda"
    inp = inputs.index_inputs(w, dev)
    B, L = s.batch, s.kv_len
    n_pages = (L + hi.page - 1) // hi.page
    pk = torch.empty((B, n_pages, s.head_dim), dtype=torch.bfloat16, device=dev)
    ws, ws_sel = lsa.Workspace(), lsa.Workspace()
    n_q = B * s.n_q

    def f_summary():  # built once per completed page in a decode loop; timed as a full rebuild
        lsa.page_summary(inp["keys"], inp["scale"], hi.page, out=pk)

    f_summary()
    res_hold = {}

    def f_recall():
        res_hold["r"] = lsa.page_recall(inp["q"], inp["w"], pk, inp["keys"], inp["scale"], b.k,
                                        b.sink, b.window, hi.page, hi.m_pages, q_pos0=s.q_pos0,
                                        ws=ws)

    f_recall()
    idx = torch.empty((B, 1, b.k), dtype=torch.int32, device=dev)

    def f_hi_topk():
        _, cs, ci = res_hold["r"]
        lsa.topk_select(cs, b.k, b.sink, b.window, kv_len=L, q_pos0=s.q_pos0, cand_ids=ci,
                        out=idx, ws=ws_sel)

    scores = torch.empty((B, 1, L), dtype=torch.float32, device=dev)
    idx_f = torch.empty_like(idx)

    def f_flat_score():
        lsa.index_scores(inp["q"], inp["w"], inp["keys"], inp["scale"], q_pos0=s.q_pos0, out=scores)

    def f_flat_topk():
        lsa.topk_select(scores, b.k, b.sink, b.window, kv_len=L, q_pos0=s.q_pos0, out=idx_f,
                        ws=ws_sel)

    ws_idx = lsa.Workspace()

    def f_flat_index():  # flat scores + selection, fused (the faster flat path)
        lsa.index_select(inp["q"], inp["w"], inp["keys"], inp["scale"], b.k, b.sink, b.window,
                         q_pos0=s.q_pos0, scores=scores, idx=idx_f, ws=ws_idx)

    f_hi_topk(), f_flat_score(), f_flat_topk(), f_flat_index()
    d = {"page_summary": tm.both(f_summary, 0.12), "recall": tm.both(f_recall, 0.04),
         "hi_topk": tm.both(f_hi_topk, 0.02), "flat_score": tm.both(f_flat_score, 0.1),
         "flat_topk": tm.both(f_flat_topk, 0.03), "flat_index_fused": tm.both(f_flat_index, 0.12)}
    # page keys and recall over paged keys: 256-row blocks (4 pages each) in shuffled pools
    if L % HI_PAGE_BLOCK == 0 and HI_PAGE_BLOCK >= hi.page:
        kpool, ktab = paged_copy(torch, inp["keys"], HI_PAGE_BLOCK)
        spool, stab = paged_copy(torch, inp["scale"].unsqueeze(-1), HI_PAGE_BLOCK)
        spool = spool.squeeze(-1)
        assert torch.equal(stab, ktab)
        pk_p = torch.empty_like(pk)

        def f_summary_paged():
            lsa.page_summary(kpool, spool, hi.page, out=pk_p, block_table=ktab, kv_len=L)

        def f_recall_paged():
            lsa.page_recall(inp["q"], inp["w"], pk, kpool, spool, b.k, b.sink, b.window, hi.page,
                            hi.m_pages, q_pos0=s.q_pos0, ws=ws, block_table=ktab, kv_len=L)
        f_summary_paged(), f_recall_paged()
        torch.cuda.synchronize()
        assert torch.equal(pk_p.view(torch.int16), pk.view(torch.int16))
        d["page_summary_paged"] = tm.both(f_summary_paged, 0.12)
        d["recall_paged"] = tm.both(f_recall_paged, 0.04)
        del kpool, spool, ktab, pk_p
    f_recall(), f_hi_topk(), f_flat_index()
    torch.cuda.synchronize()
    # quality: planted pages recalled, overlap of the HI and flat dynamic picks
    gi, fl = idx.cpu().numpy(), idx_f.cpu().numpy()
    dd = b.sink + b.window
    overlap = float(np.mean([np.isin(gi[r, 0, dd:], fl[r, 0, dd:]).mean() for r in range(B)]))
    quality = {"hi_flat_dynamic_overlap": overlap}
    if w.planted_frac > 0:
        pid = res_hold["r"][0].cpu().numpy()
        rec = [float(np.isin(inputs.planted_pages(w, r, dev).cpu().numpy(), pid[r, 0]).mean())
               for r in range(B)]
        quality["planted_pages_per_seq"] = int(round(w.planted_frac * n_pages))
        quality["planted_recall_mean"] = float(np.mean(rec))
        quality["planted_recall_min"] = float(np.min(rec))
    del scores, idx_f, res_hold
    torch.cuda.empty_cache()
    # attention layers sharing the HI index list
    atts = [inputs.attn_inputs(w, l, dev) for l in range(w.layers)]
    outs = [torch.empty((B, 1, a.heads, a.d_v), dtype=torch.bfloat16, device=dev) for _ in atts]

    def f_attn():
        for at, o in zip(atts, outs):
            lsa.sparse_attn(at["q"], at["kv"], None, idx, a.scale, b.sink, b.window, d_v=a.d_v,
                            ws=ws, out=o, want_lse=False)

    # several Python calls (or one with per-layer checks) cost the host more than the GPU time:
    # both forms are queued
    d["attn_all_layers"] = tm.both(f_attn, 0.02 * w.layers, queue=True)
    ws_layers = lsa.Workspace()

    def f_attn_layers():  # the same layers in one call: one gather launch, one combine launch
        lsa.sparse_attn_layers([at["q"] for at in atts], [at["kv"] for at in atts], idx, a.scale,
                               b.sink, b.window, d_v=a.d_v, ws=ws_layers, outs=outs,
                               want_lse=False)

    if w.layers > 1:
        d["attn_layers_one_call"] = tm.both(f_attn_layers, 0.02 * w.layers, queue=True)
    t = {k: v["warm"]["mean"] for k, v in d.items()}
    tc = {k: v["cold"]["mean"] for k, v in d.items()}
    t_hi, t_flat = t["recall"] + t["hi_topk"], t["flat_index_fused"]
    ab = attn_bytes(n_q * b.k, a.d_qk * 2, n_q, a.heads, a.d_qk, a.d_v, b.k) * w.layers
    n_elig = (L - b.window - 1) // hi.page - b.sink // hi.page + 1
    rb = recall_bytes(n_q, n_elig, s.head_dim, hi.m_pages, hi.page, s.key_dtype == "fp8")
    res = {
        "workload": w.name, "dist": d, "quality": quality,
        "page_summary_GBps": B * L * (s.head_dim + 4) / (t["page_summary"] * 1e-3) / 1e9,
        "page_summary_hbm_frac_cold": B * L * (s.head_dim + 4 + 2 * s.head_dim / hi.page)
        / (tc["page_summary"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "recall_algorithmic_bytes": rb,
        "hi_indexed_qps": n_q / (t_hi * 1e-3), "flat_indexed_qps": n_q / (t_flat * 1e-3),
        "hi_speedup_vs_flat": t_flat / t_hi,
        "hi_speedup_vs_flat_cold": tc["flat_index_fused"] / (tc["recall"] + tc["hi_topk"]),
        "hi_speedup_vs_flat_unfused": (t["flat_score"] + t["flat_topk"]) / t_hi,
        "attn_layers": w.layers,
        "sparse_attn_TBps": ab / (t["attn_all_layers"] * 1e-3) / 1e12,
    }
    if "recall_paged" in t:  # time ratios, paged over dense keys
        res["paged_vs_dense"] = {
            st: {"warm": t[st + "_paged"] / t[st], "cold": tc[st + "_paged"] / tc[st]}
            for st in ("page_summary", "recall")}
    if w.layers > 1:
        res["sparse_attn_TBps_one_call"] = ab / (t["attn_layers_one_call"] * 1e-3) / 1e12
        res["attn_layers_one_call_speedup"] = t["attn_all_layers"] / t["attn_layers_one_call"]
        res["attn_layers_one_call_speedup_cold"] = (tc["attn_all_layers"]
                                                    / tc["attn_layers_one_call"])
    del inp, atts, outs, pk, idx
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- CPU baseline
def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inputs, cfg, budget_s=12.0, budget_1t_s=8.0):
    """The oracle, as it stands, on a bounded sample of the headline workload: whole decode
    queries (scores over 131072 fp8 keys, selection, 16-head MLA attention), each stage timed,
    on all the threads it is given and on one.  The value is indexed queries/s (score +
    selection), the metric's own quantity."""
    import numpy as np
    import torch

    from oracle import ref
    w = cfg.DECODE_128K
    s, b, a = w.index, w.budget, w.attn
    n_max = 8
    small = cfg.shrink(w, batch=n_max)
    inp = inputs.index_inputs(small, "cpu")
    att = inputs.attn_inputs(small, 0, "cpu")

    def np16(t):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)

    def run(limit_s, threads):
        ref.set_num_threads(threads)
        tot = {"score": 0.0, "select": 0.0, "attn": 0.0}
        done, t_start = 0, time.perf_counter()
        while done < n_max:
            q, wt = np16(inp["q"][done]), inp["w"][done].numpy()
            keys, scale = inp["keys"][done].numpy().view(np.uint8), inp["scale"][done].numpy()
            t0 = time.perf_counter()
            I, _, _ = ref.index_scores(q, wt, keys, scale, np.array([s.q_pos0]))
            t1 = time.perf_counter()
            idx = ref.select(I.astype(np.float32), np.array([s.kv_len]), b.k, b.sink, b.window)
            t2 = time.perf_counter()
            ref.sparse_attn(np16(att["q"][done]), np16(att["kv"][done]), None, idx, a.scale,
                            d_qk=a.d_qk, d_v=a.d_v)
            t3 = time.perf_counter()
            tot["score"] += t1 - t0
            tot["select"] += t2 - t1
            tot["attn"] += t3 - t2
            done += 1
            if time.perf_counter() - t_start > limit_s:
                break
        per_q = {k: v / done for k, v in tot.items()}
        return done, per_q

    nthreads = ref.num_threads()
    done, per_q = run(budget_s, nthreads)
    done1, per_q1 = run(budget_1t_s, 1)
    ref.set_num_threads(nthreads)
    return {"value": 1.0 / (per_q["score"] + per_q["select"]), "unit": "queries/s",
            "cores": nthreads, "kind": "oracle",
            "sample": f"{done} of the 32 decode queries of the 32 x 131072 workload (fp64 scores "
                      f"over 131072 fp8 keys + selection; attention timed beside), {nthreads} "
                      f"OpenMP threads",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "stage_s_per_query": per_q,
            "value_1thread": 1.0 / (per_q1["score"] + per_q1["select"]),
            "stage_s_per_query_1thread": per_q1,
            "sample_1thread": f"{done1} decode queries on 1 thread"}


# ----------------------------------------------------------------------------- single stages
def only_stage(torch, lsa, inputs, cfg, stage, steps, cold):
    """One stage, `steps` times (cold: L2 + MALL flushed before each), for counter and trace
    runs.  `copy` is the calibration kernel: out = src + 0 over 256 MiB of fp32."""
    dev = "cuda"
    tm = Timing(torch)
    if stage == "copy":
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(steps):
            torch.add(src, 0.0, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] copy x{steps}: {src.numel() * 4} bytes read and written per launch")
        return
    if stage == "prefill_q8":
        from dataclasses import replace
        base = cfg.PREFILL_8K_AT_128K
        w = replace(base, index=replace(base.index, key_dtype="fp8"))
        s = w.index
        inp = inputs.index_inputs(w, dev)
        q8, qs = lsa.quantize_queries(inp["q"])
        scores = lsa.index_scores_q8(q8, qs, inp["w"], inp["keys"], inp["scale"], q_pos0=s.q_pos0)
        fns = {"prefill_q8": lambda: lsa.index_scores_q8(q8, qs, inp["w"], inp["keys"],
                                                         inp["scale"], q_pos0=s.q_pos0,
                                                         out=scores)}
    elif stage.startswith("bwd_"):
        _, f_attn_bwd, f_index_bwd = _bwd_setup(torch, lsa, inputs, cfg)
        fns = {"bwd_attn": f_attn_bwd, "bwd_index": f_index_bwd}
    elif stage.startswith("prefill_"):
        w = cfg.PREFILL_8K_AT_128K
        s, b, a = w.index, w.budget, w.attn
        inp = inputs.index_inputs(w, dev)
        scores = lsa.index_scores(inp["q"], inp["w"], inp["keys"], None, q_pos0=s.q_pos0)
        ws = lsa.Workspace()
        idx = lsa.topk_select(scores, b.k, b.sink, b.window, kv_len=s.kv_len, q_pos0=s.q_pos0, ws=ws)
        att = inputs.attn_inputs(w, 0, dev) if stage == "prefill_attn" else None
        fns = {"prefill_score": lambda: lsa.index_scores(inp["q"], inp["w"], inp["keys"], None,
                                                          q_pos0=s.q_pos0, out=scores),
               "prefill_topk": lambda: lsa.topk_select(scores, b.k, b.sink, b.window,
                                                        kv_len=s.kv_len, q_pos0=s.q_pos0,
                                                        out=idx, ws=ws),
               "prefill_attn": lambda: lsa.sparse_attn(att["q"], att["kv"], None, idx, a.scale,
                                                        b.sink, b.window, d_v=a.d_v, ws=ws,
                                                        want_lse=False)}
    elif stage.startswith("hi1m_"):
        w = cfg.DECODE_1M_HI
        s, b, hi = w.index, w.budget, w.hi
        inp = inputs.index_inputs(w, dev)
        pk = lsa.page_summary(inp["keys"], inp["scale"], hi.page)
        ws, ws_sel = lsa.Workspace(), lsa.Workspace()
        r = lsa.page_recall(inp["q"], inp["w"], pk, inp["keys"], inp["scale"], b.k, b.sink,
                            b.window, hi.page, hi.m_pages, q_pos0=s.q_pos0, ws=ws)
        fns = {"hi1m_summary": lambda: lsa.page_summary(inp["keys"], inp["scale"], hi.page, out=pk),
               "hi1m_recall": lambda: lsa.page_recall(inp["q"], inp["w"], pk, inp["keys"],
                                                      inp["scale"], b.k, b.sink, b.window,
                                                      hi.page, hi.m_pages, q_pos0=s.q_pos0, ws=ws),
               "hi1m_topk": lambda: lsa.topk_select(r[1], b.k, b.sink, b.window, kv_len=s.kv_len,
                                                    q_pos0=s.q_pos0, cand_ids=r[2], ws=ws_sel)}
    elif stage.startswith("cli4_"):
        # 4 attention layers on one Hierarchical-Indexing list (8 x 256K decode): per-layer calls
        # or one multi-layer call
        w = cfg.DECODE_256K_HI_CLI
        s, b, a, hi = w.index, w.budget, w.attn, w.hi
        inp = inputs.index_inputs(w, dev)
        pk = lsa.page_summary(inp["keys"], inp["scale"], hi.page)
        _, cs, ci = lsa.page_recall(inp["q"], inp["w"], pk, inp["keys"], inp["scale"], b.k, b.sink,
                                    b.window, hi.page, hi.m_pages, q_pos0=s.q_pos0)
        idx = lsa.topk_select(cs, b.k, b.sink, b.window, kv_len=s.kv_len, q_pos0=s.q_pos0,
                              cand_ids=ci)
        del inp, pk, cs, ci
        atts = [inputs.attn_inputs(w, l, dev) for l in range(w.layers)]
        ws = lsa.Workspace()

        def per_layer():
            for at in atts:
                lsa.sparse_attn(at["q"], at["kv"], None, idx, a.scale, b.sink, b.window, d_v=a.d_v,
                                ws=ws, want_lse=False)
        fns = {"cli4_attn": per_layer,
               "cli4_attn_layers": lambda: lsa.sparse_attn_layers(
                   [at["q"] for at in atts], [at["kv"] for at in atts], idx, a.scale, b.sink,
                   b.window, d_v=a.d_v, ws=ws, want_lse=False)}
    else:
        w = cfg.DECODE_128K
        s, b, a = w.index, w.budget, w.attn
        inp = inputs.index_inputs(w, dev)
        L = s.kv_len
        scores = lsa.index_scores(inp["q"], inp["w"], inp["keys"], inp["scale"], q_pos0=s.q_pos0)
        ws, ws_idx = lsa.Workspace(), lsa.Workspace()
        idx = lsa.topk_select(scores, b.k, b.sink, b.window, kv_len=L, q_pos0=s.q_pos0, ws=ws)
        att = inputs.attn_inputs(w, 0, dev) if stage == "attn" else None
        fns = {"score": lambda: lsa.index_scores(inp["q"], inp["w"], inp["keys"], inp["scale"],
                                                 q_pos0=s.q_pos0, out=scores),
               "topk": lambda: lsa.topk_select(scores, b.k, b.sink, b.window, kv_len=L,
                                               q_pos0=s.q_pos0, out=idx, ws=ws),
               "index": lambda: lsa.index_select(inp["q"], inp["w"], inp["keys"], inp["scale"],
                                                 b.k, b.sink, b.window, q_pos0=s.q_pos0,
                                                 scores=scores, idx=idx, ws=ws_idx),
               "attn": lambda: lsa.sparse_attn(att["q"], att["kv"], None, idx, a.scale, b.sink,
                                               b.window, d_v=a.d_v, ws=ws)}
        if stage == "index_paged":
            kpool, ktab = paged_copy(torch, inp["keys"], PAGE_BLOCK)
            spool = paged_copy(torch, inp["scale"].unsqueeze(-1), PAGE_BLOCK)[0].squeeze(-1)
            fns[stage] = lambda: lsa.index_select(inp["q"], inp["w"], kpool, spool, b.k, b.sink,
                                                  b.window, q_pos0=s.q_pos0, scores=scores,
                                                  idx=idx, ws=ws_idx, block_table=ktab, kv_len=L)
        if stage == "attn_paged":
            att = inputs.attn_inputs(w, 0, dev)
            pool, tab = paged_copy(torch, att["kv"], PAGE_BLOCK)
            fns[stage] = lambda: lsa.sparse_attn(att["q"], pool, None, idx, a.scale, b.sink,
                                                 b.window, d_v=a.d_v, ws=ws, block_table=tab,
                                                 kv_len=L)
    fn = fns[stage]
    fn()
    torch.cuda.synchronize()
    for _ in range(steps):
        if cold:
            tm.flush()
        fn()
    torch.cuda.synchronize()
    log(f"[bench] {stage} x{steps} ({'cold' if cold else 'warm'}) done")


STAGES = ["score", "topk", "index", "attn", "copy", "prefill_score", "prefill_topk", "prefill_attn",
          "prefill_q8", "bwd_attn", "bwd_index",
          "hi1m_summary", "hi1m_recall", "hi1m_topk", "cli4_attn", "cli4_attn_layers", "attn_paged", "index_paged"]


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--extras", action=argparse.BooleanOptionalAction, default=True)
    ap.add_argument("--cpu-baseline", action=argparse.BooleanOptionalAction, default=True)
    ap.add_argument("--only", choices=STAGES,
                    help="run one stage --steps times and exit (for rocprofv3 runs); copy is a "
                         "plain 256 MiB device copy used to calibrate the traffic counters")
    ap.add_argument("--cold", action="store_true", help="with --only: flush L2 and MALL first")
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
        only_stage(torch, lsa, inputs, cfg, args.only, args.steps, args.cold)
        return

    tm = Timing(torch)
    w, head = headline(torch, lsa, inputs, cfg, tm, args.steps, args.warmup)
    s, b = w.index, w.budget
    n_q = s.batch * s.n_q

    score_src = ["token_selection_indexer_amd/csrc/score.hip",
                 "token_selection_indexer_amd/csrc/device.hpp"]
    t_cold = head["dist"]["score"]["cold"]["mean"] * 1e-3
    t_warm = head["dist"]["score"]["warm"]["mean"] * 1e-3
    sb = head["score_algorithmic_bytes"]
    roof = {"kernel": "score_stream_kernel (lsa_index_scores, fp8 keys, decode 32 x 131072)",
            "bound": "hbm", "achieved": sb / t_cold / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": sb / t_cold / 1e9 / HBM_PEAK_GBS,
            "traffic": profile_traffic("score_stream_decode_b32_128k_pmc", score_src),
            "algorithmic_bytes_per_launch": sb,
            "timing": "mean of 50 cold runs (L2 + MALL flushed by a 1 GiB read before each), "
                      "HIP events on the library's stream",
            "frac_warm": sb / t_warm / 1e9 / HBM_PEAK_GBS}

    extras = {}
    if args.extras:
        log("[bench] extra: chunked prefill 8K @ 128K")
        extras["prefill_8k_128k"] = extra_prefill(torch, lsa, inputs, cfg, tm)
        log("[bench] extra: chunked prefill with fp8 queries")
        extras["prefill_8k_128k_fp8q"] = extra_prefill_q8(torch, lsa, inputs, cfg, tm)
        log("[bench] extra: backward at the chunked-prefill shape")
        extras["prefill_8k_128k_backward"] = extra_backward(torch, lsa, inputs, cfg, tm)
        log("[bench] extra: HI at 1M")
        extras["decode_1m_hi"] = extra_hi(torch, lsa, inputs, cfg.DECODE_1M_HI, tm)
        log("[bench] extra: HI + cross-layer x4 at 256K")
        extras["decode_256k_hi_cli4"] = extra_hi(torch, lsa, inputs, cfg.DECODE_256K_HI_CLI, tm)
    cpu = None
    if args.cpu_baseline:
        log("[bench] CPU oracle baseline")
        cpu = cpu_baseline(inputs, cfg)

    line = {
        "metric": METRIC, "value": head["indexed_qps"], "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["wall_ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": s.batch, "kv_len": s.kv_len,
                   "indexer": f"{s.heads}x{s.head_dim} fp8-e4m3 keys", "k": b.k,
                   "sink": b.sink, "window": b.window, "attn": "MLA 16 heads, 576/512 latent"},
        "value_def": "queries / (score + top-k time): HIP events around lsa_index_select "
                     "(fused scores + selection) in each timed step; ms_per_step is the whole "
                     "step (scores + selection + attention)",
        "indexed_qps_unfused": head["indexed_qps_unfused"],
        "step_qps": head["step_qps"],
        "sparse_attn_TBps": head["sparse_attn_TBps"],
        "paged_vs_dense": {  # time ratios with 64-row blocks in shuffled pools
            st: {m: head["dist"][st + "_paged"][m]["mean"] / head["dist"][st][m]["mean"]
                 for m in ("warm", "cold")} for st in ("index", "attn")},
        "stage_ms": head["stage_ms"],
        "stage_dist_ms": rnd(head["dist"]),
        "hbm_frac_cold_mean": head["hbm_frac_cold_mean"],
        "hbm_frac_warm_mean": head["hbm_frac_warm_mean"],
        "roofline": roof,
        "cpu_baseline": cpu,
        "extras": rnd(extras, 5),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
