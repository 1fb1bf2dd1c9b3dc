"""Small conversions and tolerance checks shared by the tests (no method arithmetic)."""
from __future__ import annotations

import numpy as np
import torch


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().view(np.uint8)


def f32(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().cpu().float().numpy()
    return np.asarray(t, np.float32)


def keys_np(inp, b):
    """Host copy of sequence b's keys (+ scale) in the oracle's formats."""
    k = inp["keys"][b]
    if k.dtype == torch.bfloat16:
        return bits(k), None
    return u8(k), f32(inp["scale"][b])


def score_tol(A: np.ndarray, E: np.ndarray, rel: float = 1e-3) -> np.ndarray:
    """Tolerance on an indexer score: rel * max(A, E/100).  A = sum_h |w| ReLU(q.k) is the size
    of the terms summed; E = sum_h |w| sum_i |q_i k_i| bounds the fp32 rounding of the dot
    products (<= d * 2^-24 * E), which dominates A only after heavy cancellation."""
    return rel * np.maximum(A, E / 100.0)


def check_si_layout(row: np.ndarray, V: int, k: int, S: int, W: int, cand_ids=None):
    """Structure of one selected row: sink | window | dynamic, each ascending, then -1.
    V <= k: exactly 0..V-1 then -1.  V > k: [0,S), [V-W,V), then at most k-S-W distinct middle
    tokens in [S, V-W), strictly ascending (exactly k-S-W in flat mode, where the middle always
    holds more); ids taken from cand_ids if given.  Also: no duplicates anywhere."""
    row = np.asarray(row, np.int64)
    assert row.shape == (k,)
    if V <= k:
        assert np.array_equal(row[:V], np.arange(V)), "V <= k: the row must be 0..V-1"
        assert np.all(row[V:] == -1)
        return
    assert np.array_equal(row[:S], np.arange(S)), "sink"
    assert np.array_equal(row[S:S + W], np.arange(V - W, V)), "window"
    dyn = row[S + W:]
    n = int((dyn >= 0).sum())
    assert np.all(dyn[:n] >= 0) and np.all(dyn[n:] == -1), "-1 only at the tail"
    d = dyn[:n]
    assert np.all(np.diff(d) > 0), "dynamic picks strictly ascending"
    assert n == 0 or (d[0] >= S and d[-1] < V - W), "dynamic picks inside the middle"
    if cand_ids is None:
        assert n == k - S - W, "flat mode fills the dynamic budget"
    else:
        c = np.asarray(cand_ids)
        assert np.all(np.isin(d, c[c >= 0])), "picks come from the candidates"
    assert len(np.unique(row[row >= 0])) == int((row >= 0).sum()), "duplicates"


class NearTie:
    """Near-tie comparison of selected sets, aggregated over rows.  For each row, every element
    in one set only must have a reference score within tol of the reference k-th score; the
    recall |A and B| / |B| summed over all rows must reach min_recall (the bar is 99.9%)."""

    def __init__(self):
        self.common = 0
        self.total = 0
        self.mismatches = 0
        self.rows = 0

    def add(self, sel_a, sel_b, ref_score, kth_score: float, tol_kth: float):
        a = set(int(x) for x in sel_a if x >= 0)
        b = set(int(x) for x in sel_b if x >= 0)
        diff = a ^ b
        for x in diff:
            assert abs(ref_score[x] - kth_score) <= tol_kth, (x, ref_score[x], kth_score, tol_kth)
        self.common += len(a & b)
        self.total += len(b)
        self.mismatches += len(diff)
        self.rows += 1
        return len(diff)

    @property
    def recall(self) -> float:
        return self.common / max(1, self.total)

    def check(self, min_recall: float = 0.999):
        assert self.recall >= min_recall, (self.recall, self.mismatches, self.rows)
        return self.recall
