"""numpy front end of the CPU oracle (oracle/lsa_ref.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the CPU-baseline leg of
the bench, never by the product path.  It shares nothing with the HIP library.

bf16 tensors travel as uint16 bit patterns, e4m3fn keys as uint8 codes.  Every function works on
one sequence; the *_batch helpers loop over the batch.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblsa_ref.so")
KEY_BF16, KEY_E4M3 = 1, 2

_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"oracle library missing: build it with python oracle/build.py "
                               f"({LIB_PATH})")
        L = ctypes.CDLL(LIB_PATH)
        L.lsa_ref_num_threads.restype = ctypes.c_int
        L.lsa_ref_set_num_threads.argtypes = [ctypes.c_int]
        L.lsa_ref_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.lsa_ref_bf16_to_double.restype = ctypes.c_double
        L.lsa_ref_e4m3fn_to_double.argtypes = [ctypes.c_uint8]
        L.lsa_ref_e4m3fn_to_double.restype = ctypes.c_double
        L.lsa_ref_f32_to_bf16_rne.argtypes = [ctypes.c_float]
        L.lsa_ref_f32_to_bf16_rne.restype = ctypes.c_uint16
        L.lsa_ref_index_scores.argtypes = [_I64, _I32, _I32, _I64, _P, _P, _P, _P, _I32, _P,
                                           _P, _P, _P]
        L.lsa_ref_select.argtypes = [_I64, _I64, _P, _P, _P, _I32, _I32, _I32, _P]
        L.lsa_ref_f32_to_e4m3fn_sat.argtypes = [ctypes.c_float]
        L.lsa_ref_f32_to_e4m3fn_sat.restype = ctypes.c_uint8
        L.lsa_ref_quantize_rows.argtypes = [_I64, _I32, _P, _P, _P]
        L.lsa_ref_index_scores_q8.argtypes = [_I64, _I32, _I32, _I64, _P, _P, _P, _P, _P, _I32,
                                              _P, _P, _P, _P]
        L.lsa_ref_page_keys.argtypes = [_I64, _I32, _I32, _P, _I32, _P, _P]
        L.lsa_ref_page_recall.argtypes = [_I64, _I32, _I32, _I64, _P, _P, _P, _P, _P, _I32, _P,
                                          _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P]
        L.lsa_ref_sparse_attn.argtypes = [_I64, _I32, _I32, _I32, _I32, _P, _P, _I64, _P, _I64,
                                          _P, ctypes.c_double, _P, _P]
        L.lsa_ref_sparse_attn_f64.argtypes = [_I64, _I32, _I32, _I32, _I32, _P, _P, _I64, _P,
                                              _I64, _P, _I64, ctypes.c_double, _P, _P]
        L.lsa_ref_sparse_attn_backward.argtypes = [_I64, _I32, _I32, _I32, _I32, _P, _P, _I64, _P,
                                                   _I64, _P, _I64, ctypes.c_double, _P, _P, _P,
                                                   _P]
        L.lsa_ref_index_scores_sel_f64.argtypes = [_I64, _I32, _I32, _I32, _P, _P, _P, _P, _P,
                                                   _I64, _P]
        L.lsa_ref_index_scores_backward.argtypes = [_I64, _I32, _I32, _I32, _P, _P, _P, _P, _P,
                                                    _I64, _P, _P, _P, _P]
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _key_args(keys, scale):
    keys = np.ascontiguousarray(keys)
    if keys.dtype == np.uint16:
        return keys, KEY_BF16, None
    assert keys.dtype == np.uint8 and scale is not None
    return keys, KEY_E4M3, _c(scale, np.float32)


def num_threads() -> int:
    return lib().lsa_ref_num_threads()


def set_num_threads(n: int) -> None:
    lib().lsa_ref_set_num_threads(int(n))


# --------------------------------------------------------------------------------- formats
def bf16_to_double(bits: int) -> float:
    return lib().lsa_ref_bf16_to_double(int(bits))


def e4m3fn_to_double(code: int) -> float:
    return lib().lsa_ref_e4m3fn_to_double(int(code))


def f32_to_bf16_rne(x: float) -> int:
    return lib().lsa_ref_f32_to_bf16_rne(float(x))


# --------------------------------------------------------------------------------- a1 scores
def index_scores(q, w, keys, scale, pos):
    """q uint16 [T,H,d], w f32 [T,H], keys [L,d] (uint16 bf16 bits or uint8 e4m3 codes),
    scale f32 [L] or None, pos int64 [T] -> (I, A, E) fp64 [T,L]."""
    q = _c(q, np.uint16)
    T, H, d = q.shape
    keys, kd, scale = _key_args(keys, scale)
    L = keys.shape[0]
    w = _c(w, np.float32)
    pos = _c(pos, np.int64)
    I = np.empty((T, L), np.float64)
    A = np.empty((T, L), np.float64)
    E = np.empty((T, L), np.float64)
    lib().lsa_ref_index_scores(T, H, d, L, _ptr(pos), _ptr(q), _ptr(w), _ptr(keys), kd,
                               _ptr(scale), _ptr(I), _ptr(A), _ptr(E))
    return I, A, E


# --------------------------------------------------------------------------------- fp8 queries
def f32_to_e4m3fn_sat(x: float) -> int:
    return lib().lsa_ref_f32_to_e4m3fn_sat(float(x))


def quantize_rows(x):
    """x uint16 (bf16 bits) [..., d] -> (codes uint8 [..., d], scale f32 [...]): per-row e4m3
    quantisation (scale = amax / 448)."""
    x = _c(x, np.uint16)
    d = x.shape[-1]
    rows = x.size // d
    codes = np.empty(x.shape, np.uint8)
    scale = np.empty(x.shape[:-1], np.float32)
    lib().lsa_ref_quantize_rows(rows, d, _ptr(x), _ptr(codes), _ptr(scale))
    return codes, scale


def index_scores_q8(q8, q_scale, w, keys, scale, pos):
    """q8 uint8 [T,H,d] e4m3 codes, q_scale f32 [T,H], w f32 [T,H], keys / scale as for
    index_scores -> (I, A, E) fp64 [T,L]."""
    q8 = _c(q8, np.uint8)
    T, H, d = q8.shape
    keys, kd, scale = _key_args(keys, scale)
    L = keys.shape[0]
    qs = _c(q_scale, np.float32)
    w = _c(w, np.float32)
    pos = _c(pos, np.int64)
    I = np.empty((T, L), np.float64)
    A = np.empty((T, L), np.float64)
    E = np.empty((T, L), np.float64)
    lib().lsa_ref_index_scores_q8(T, H, d, L, _ptr(pos), _ptr(q8), _ptr(qs), _ptr(w), _ptr(keys),
                                  kd, _ptr(scale), _ptr(I), _ptr(A), _ptr(E))
    return I, A, E


# --------------------------------------------------------------------------------- a2 select
def select(scores, V, k, S, W, cand_ids=None):
    """scores f32 [T,n] (flat: n == L), V int64 [T] valid lengths, cand_ids int32 [T,n] or None
    -> idx int32 [T,k]."""
    scores = _c(scores, np.float32)
    T, n = scores.shape
    V = _c(V, np.int64)
    cid = None if cand_ids is None else _c(cand_ids, np.int32)
    idx = np.empty((T, k), np.int32)
    lib().lsa_ref_select(T, n, _ptr(scores), _ptr(cid), _ptr(V), k, S, W, _ptr(idx))
    return idx


# --------------------------------------------------------------------------------- a3 pages
def page_keys(keys, scale, P):
    keys, kd, scale = _key_args(keys, scale)
    L, d = keys.shape
    pk = np.empty(((L + P - 1) // P, d), np.uint16)
    lib().lsa_ref_page_keys(L, d, P, _ptr(keys), kd, _ptr(scale), _ptr(pk))
    return pk


# --------------------------------------------------------------------------------- a4/a5 HI
def page_recall(q, w, pk, keys, scale, pos, k, S, W, P, M):
    """-> dict(page_ids [T,M], cand_ids [T,M*P], cand_scores fp64 [T,M*P],
    coarse fp64 [T,n_pages], n_scored [T])."""
    q = _c(q, np.uint16)
    T, H, d = q.shape
    keys, kd, scale = _key_args(keys, scale)
    L = keys.shape[0]
    n_pages = (L + P - 1) // P
    pk = _c(pk, np.uint16)
    assert pk.shape == (n_pages, d)
    w = _c(w, np.float32)
    pos = _c(pos, np.int64)
    out = dict(page_ids=np.empty((T, M), np.int32), cand_ids=np.empty((T, M * P), np.int32),
               cand_scores=np.empty((T, M * P), np.float64),
               coarse=np.empty((T, n_pages), np.float64), n_scored=np.empty(T, np.int64))
    lib().lsa_ref_page_recall(T, H, d, L, _ptr(pos), _ptr(q), _ptr(w), _ptr(pk), _ptr(keys), kd,
                              _ptr(scale), k, S, W, P, M, _ptr(out["page_ids"]),
                              _ptr(out["cand_ids"]), _ptr(out["cand_scores"]),
                              _ptr(out["coarse"]), _ptr(out["n_scored"]))
    return out


# --------------------------------------------------------------------------------- a6/a7 attn
def sparse_attn(q, kmat, vmat, idx, tau, d_qk=None, d_v=None):
    """q uint16 [T,Hq,d_qk]; kmat uint16 [L,ks] (first d_qk columns are K); vmat uint16 [L,vs]
    (first d_v columns are V; may be the same array as kmat for a latent cache);
    idx int32 [T,k] -> (o fp64 [T,Hq,d_v], lse fp64 [T,Hq])."""
    q = _c(q, np.uint16)
    T, Hq, dq = q.shape
    d_qk = dq if d_qk is None else d_qk
    kmat = _c(kmat, np.uint16)
    vmat = kmat if vmat is None else _c(vmat, np.uint16)
    d_v = vmat.shape[1] if d_v is None else d_v
    idx = _c(idx, np.int32)
    k = idx.shape[1]
    o = np.empty((T, Hq, d_v), np.float64)
    lse = np.empty((T, Hq), np.float64)
    lib().lsa_ref_sparse_attn(T, Hq, d_qk, d_v, k, _ptr(q), _ptr(kmat), kmat.shape[1],
                              _ptr(vmat), vmat.shape[1], _ptr(idx), float(tau), _ptr(o),
                              _ptr(lse))
    return o, lse


def cross_layer_attn(layers, idx, tau, d_qk=None, d_v=None):
    """Cross-Layer Indexing: every layer (q, kmat, vmat) attends over the same idx."""
    return [sparse_attn(q, km, vm, idx, tau, d_qk, d_v) for (q, km, vm) in layers]


# --------------------------------------------------------------------------------- f4 backward
def sparse_attn_f64(q, kmat, vmat, idx, tau, d_qk=None, d_v=None):
    """The sparse attention on float64 inputs: q [T,Hq,d_qk]; kmat [L,ks] (first d_qk columns
    are K); vmat [L,vs] (first d_v columns are V, may be kmat); idx int32 [T,k], entries outside
    [0, L) skipped -> (o [T,Hq,d_v], lse [T,Hq])."""
    q = _c(q, np.float64)
    T, Hq, dq = q.shape
    d_qk = dq if d_qk is None else d_qk
    kmat = _c(kmat, np.float64)
    vmat = kmat if vmat is None else _c(vmat, np.float64)
    d_v = vmat.shape[1] if d_v is None else d_v
    idx = _c(idx, np.int32)
    k = idx.shape[1]
    o = np.empty((T, Hq, d_v), np.float64)
    lse = np.empty((T, Hq), np.float64)
    lib().lsa_ref_sparse_attn_f64(T, Hq, d_qk, d_v, k, _ptr(q), _ptr(kmat), kmat.shape[1],
                                  _ptr(vmat), vmat.shape[1], _ptr(idx), kmat.shape[0], float(tau),
                                  _ptr(o), _ptr(lse))
    return o, lse


def sparse_attn_backward(q, kmat, vmat, idx, tau, g, d_qk=None, d_v=None):
    """Gradients of sparse_attn_f64 for the output gradient g [T,Hq,d_v] ->
    (dq [T,Hq,d_qk], dK [L,d_qk], dV [L,d_v]) in float64.  A latent cache (vmat is kmat) has
    the row gradient dK + dV (dV on the first d_v columns)."""
    q = _c(q, np.float64)
    T, Hq, dq_ = q.shape
    d_qk = dq_ if d_qk is None else d_qk
    kmat = _c(kmat, np.float64)
    vmat = kmat if vmat is None else _c(vmat, np.float64)
    d_v = vmat.shape[1] if d_v is None else d_v
    idx = _c(idx, np.int32)
    k = idx.shape[1]
    g = _c(g, np.float64)
    assert g.shape == (T, Hq, d_v)
    L = kmat.shape[0]
    dq = np.empty((T, Hq, d_qk), np.float64)
    dK = np.empty((L, d_qk), np.float64)
    dV = np.empty((L, d_v), np.float64)
    lib().lsa_ref_sparse_attn_backward(T, Hq, d_qk, d_v, k, _ptr(q), _ptr(kmat), kmat.shape[1],
                                       _ptr(vmat), vmat.shape[1], _ptr(idx), L, float(tau), _ptr(g),
                                       _ptr(dq), _ptr(dK), _ptr(dV))
    return dq, dK, dV


def index_scores_sel_f64(q, w, keys, idx, pos):
    """Indexer scores at the selected entries on float64 inputs: q [T,H,d], w [T,H], keys
    [L,d], idx int32 [T,k], pos int64 [T] -> I [T,k] (0 where the entry is not in [0, V_t))."""
    q = _c(q, np.float64)
    T, H, d = q.shape
    w = _c(w, np.float64)
    keys = _c(keys, np.float64)
    idx = _c(idx, np.int32)
    pos = _c(pos, np.int64)
    k = idx.shape[1]
    I = np.empty((T, k), np.float64)
    lib().lsa_ref_index_scores_sel_f64(T, H, d, k, _ptr(pos), _ptr(q), _ptr(w), _ptr(keys),
                                       _ptr(idx), keys.shape[0], _ptr(I))
    return I


def index_scores_backward(q, w, keys, idx, pos, gI):
    """Gradients of index_scores_sel_f64 for gI [T,k] -> (dq [T,H,d], dw [T,H], dk [L,d])."""
    q = _c(q, np.float64)
    T, H, d = q.shape
    w = _c(w, np.float64)
    keys = _c(keys, np.float64)
    idx = _c(idx, np.int32)
    pos = _c(pos, np.int64)
    gI = _c(gI, np.float64)
    k = idx.shape[1]
    L = keys.shape[0]
    dq = np.empty((T, H, d), np.float64)
    dw = np.empty((T, H), np.float64)
    dk = np.empty((L, d), np.float64)
    lib().lsa_ref_index_scores_backward(T, H, d, k, _ptr(pos), _ptr(q), _ptr(w), _ptr(keys),
                                        _ptr(idx), L, _ptr(gI), _ptr(dq), _ptr(dw), _ptr(dk))
    return dq, dw, dk


def bf16_bits_to_f64(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------------- helpers
def valid_lengths(L: int, q_pos0: int, n_q: int) -> np.ndarray:
    """V_t = min(L, q_pos0 + t + 1) for t in [0, n_q)."""
    return np.minimum(L, q_pos0 + np.arange(n_q, dtype=np.int64) + 1)


def positions(q_pos0: int, n_q: int) -> np.ndarray:
    return q_pos0 + np.arange(n_q, dtype=np.int64)
