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


def check_near_tie_sets(sel_a: np.ndarray, sel_b: np.ndarray, ref_score: np.ndarray,
                        kth_score: float, tol_kth: float, min_recall: float = 0.999):
    """Two index sets (ints, -1 ignored) selected from the same scores must agree except at near
    ties: every element in one set only must have a reference score within tol of the k-th
    score.  Returns (recall, number of mismatches)."""
    a = set(int(x) for x in sel_a if x >= 0)
    b = set(int(x) for x in sel_b if x >= 0)
    diff = a ^ b
    for x in diff:
        assert abs(ref_score[x] - kth_score) <= tol_kth, (x, ref_score[x], kth_score, tol_kth)
    recall = len(a & b) / max(1, len(b))
    assert recall >= min_recall, recall
    return recall, len(diff)
