"""Python binding of liblsa.so (include/lsa.h), by ctypes.

Argument marshalling only: every step of the path runs in the library's HIP kernels.  torch is
used for device memory (tensors in, outputs and workspaces allocated with torch.empty) and for
the current stream.  There is no fallback: if the library is missing or a call fails, this
module raises.

The functions named like the C entry points (lsa_index_scores, ...) take every argument the C
function takes; the short names (index_scores, ...) allocate outputs and workspace and derive
shapes from the tensors.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblsa.so")

KEY_BF16, KEY_FP8_E4M3 = 1, 2
OP_TOPK_SELECT, OP_PAGE_RECALL, OP_SPARSE_ATTN = 1, 2, 3
STATUS = {0: "LSA_OK", 1: "LSA_ERR_NULL_POINTER", 2: "LSA_ERR_BAD_SHAPE", 3: "LSA_ERR_BAD_DTYPE",
          4: "LSA_ERR_UNSUPPORTED", 5: "LSA_ERR_WORKSPACE_TOO_SMALL", 6: "LSA_ERR_DEVICE"}
EXPORTS = ("lsa_index_scores", "lsa_topk_select", "lsa_page_summary", "lsa_page_recall",
           "lsa_sparse_attn", "lsa_workspace_bytes", "lsa_status_string")


class IndexShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("kv_len", ctypes.c_int64),
                ("q_pos0", ctypes.c_int64)]


class Budget(ctypes.Structure):
    _fields_ = [("k", ctypes.c_int32), ("sink", ctypes.c_int32), ("window", ctypes.c_int32)]


class AttnShape(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("latent", ctypes.c_int32), ("k_row_stride", ctypes.c_int64),
                ("v_row_stride", ctypes.c_int64), ("scale", ctypes.c_float)]


class LsaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


_lib = None
_VP, _I64, _I32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t


def lib():
    """Load liblsa.so (built in-tree by token_selection_indexer_amd/build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        ip, bud, ap = ctypes.POINTER(IndexShape), Budget, ctypes.POINTER(AttnShape)
        L.lsa_index_scores.argtypes = [ip, _VP, _VP, _VP, _I32, _VP, _VP, _VP]
        L.lsa_topk_select.argtypes = [ip, bud, _VP, _I64, _VP, _VP, _VP, _SZ, _VP]
        L.lsa_page_summary.argtypes = [ip, _I32, _VP, _I32, _VP, _I64, _I64, _VP, _VP]
        L.lsa_page_recall.argtypes = [ip, bud, _I32, _I32, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _VP,
                                      _VP, _VP, _SZ, _VP]
        L.lsa_sparse_attn.argtypes = [ip, ap, bud, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]
        L.lsa_workspace_bytes.argtypes = [_I32, ip, bud, _I32, _I32, _I64, ap]
        L.lsa_workspace_bytes.restype = _SZ
        L.lsa_status_string.argtypes = [_I32]
        L.lsa_status_string.restype = ctypes.c_char_p
        for f in EXPORTS[:5]:
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _s(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(fn: str, st: int):
    if st != 0:
        raise LsaError(fn, st)


# ------------------------------------------------------------------ same-named C entry points
def lsa_index_scores(shape: IndexShape, q, w, keys, key_dtype: int, key_scale, scores,
                     stream=None):
    _check("lsa_index_scores", lib().lsa_index_scores(
        ctypes.byref(shape), _p(q), _p(w), _p(keys), key_dtype, _p(key_scale), _p(scores),
        _s(stream)))


def lsa_topk_select(shape: IndexShape, budget: Budget, scores, n_cand: int, cand_ids, idx,
                    ws=None, ws_bytes: int = 0, stream=None):
    _check("lsa_topk_select", lib().lsa_topk_select(
        ctypes.byref(shape), budget, _p(scores), n_cand, _p(cand_ids), _p(idx), _p(ws),
        ws_bytes, _s(stream)))


def lsa_page_summary(shape: IndexShape, page_size: int, keys, key_dtype: int, key_scale,
                     page_lo: int, page_hi: int, page_keys, stream=None):
    _check("lsa_page_summary", lib().lsa_page_summary(
        ctypes.byref(shape), page_size, _p(keys), key_dtype, _p(key_scale), page_lo, page_hi,
        _p(page_keys), _s(stream)))


def lsa_page_recall(shape: IndexShape, budget: Budget, page_size: int, m_pages: int, q, w,
                    page_keys, keys, key_dtype: int, key_scale, page_ids, cand_scores, cand_ids,
                    ws, ws_bytes: int, stream=None):
    _check("lsa_page_recall", lib().lsa_page_recall(
        ctypes.byref(shape), budget, page_size, m_pages, _p(q), _p(w), _p(page_keys), _p(keys),
        key_dtype, _p(key_scale), _p(page_ids), _p(cand_scores), _p(cand_ids), _p(ws), ws_bytes,
        _s(stream)))


def lsa_sparse_attn(shape: IndexShape, attn: AttnShape, budget: Budget, q, k, v, idx, out, lse,
                    ws, ws_bytes: int, stream=None):
    _check("lsa_sparse_attn", lib().lsa_sparse_attn(
        ctypes.byref(shape), ctypes.byref(attn), budget, _p(q), _p(k), _p(v), _p(idx), _p(out),
        _p(lse), _p(ws), ws_bytes, _s(stream)))


def lsa_workspace_bytes(op: int, shape: Optional[IndexShape], budget: Budget, page_size: int = 0,
                        m_pages: int = 0, n_cand: int = 0, attn: Optional[AttnShape] = None) -> int:
    n = lib().lsa_workspace_bytes(op, ctypes.byref(shape) if shape is not None else None, budget,
                                  page_size, m_pages, n_cand,
                                  ctypes.byref(attn) if attn is not None else None)
    if n == ctypes.c_size_t(-1).value:
        raise LsaError("lsa_workspace_bytes", 2)
    return n


def lsa_status_string(status: int) -> str:
    return lib().lsa_status_string(status).decode()


# ------------------------------------------------------------------ tensor-level helpers
@dataclass
class Workspace:
    """A reusable device workspace (grown on demand, 256-byte aligned by torch's allocator)."""
    buf: Optional[torch.Tensor] = None

    def get(self, nbytes: int, device) -> Optional[torch.Tensor]:
        if nbytes == 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != torch.device(device):
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        return self.buf


def _need(t: torch.Tensor, name: str, dtype=None, dim=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, got {t.dim()}")


def _key_args(keys: torch.Tensor, key_scale: Optional[torch.Tensor]):
    if keys.dtype == torch.bfloat16:
        return KEY_BF16, None
    if keys.dtype in (torch.uint8, torch.float8_e4m3fn):
        if key_scale is None:
            raise ValueError("fp8 keys need key_scale")
        return KEY_FP8_E4M3, key_scale
    raise ValueError(f"keys must be bf16 or e4m3 codes, got {keys.dtype}")


def index_shape(q: torch.Tensor, keys: torch.Tensor, q_pos0: Optional[int] = None) -> IndexShape:
    B, T, H, d = q.shape
    L = keys.shape[1]
    return IndexShape(B, T, H, d, L, L - T if q_pos0 is None else q_pos0)


def index_scores(q, w, keys, key_scale=None, q_pos0=None, out=None, stream=None):
    """scores [B, n_q, L] fp32 (q_pos0 defaults to L - n_q: the queries are the last tokens)."""
    _need(q, "q", torch.bfloat16, 4)
    _need(w, "w", torch.float32, 3)
    _need(keys, "keys", dim=3)
    kd, ks = _key_args(keys, key_scale)
    shape = index_shape(q, keys, q_pos0)
    if out is None:
        out = torch.empty((shape.batch, shape.n_q, shape.kv_len), dtype=torch.float32,
                          device=q.device)
    lsa_index_scores(shape, q, w, keys, kd, ks, out, stream)
    return out


def topk_select(scores, k, sink, window, kv_len, q_pos0, cand_ids=None, out=None,
                ws: Optional[Workspace] = None, stream=None):
    """idx [B, n_q, k] int32 from flat scores [B, n_q, L] or candidates (scores, cand_ids)."""
    _need(scores, "scores", torch.float32, 3)
    B, T, n = scores.shape
    shape = IndexShape(B, T, 1, 64, kv_len, q_pos0)
    if cand_ids is not None:
        _need(cand_ids, "cand_ids", torch.int32, 3)
    if out is None:
        out = torch.empty((B, T, k), dtype=torch.int32, device=scores.device)
    bud = Budget(k, sink, window)
    nb = lsa_workspace_bytes(OP_TOPK_SELECT, shape, bud, n_cand=n)
    wsb = (ws or Workspace()).get(nb, scores.device)
    lsa_topk_select(shape, bud, scores, n, cand_ids, out, wsb, nb, stream)
    return out


def page_summary(keys, key_scale, page, page_lo=0, page_hi=None, out=None, stream=None):
    """page keys [B, ceil(L/P), d] bf16."""
    _need(keys, "keys", dim=3)
    kd, ks = _key_args(keys, key_scale)
    B, L, d = keys.shape
    n_pages = (L + page - 1) // page
    if out is None:
        out = torch.empty((B, n_pages, d), dtype=torch.bfloat16, device=keys.device)
    shape = IndexShape(B, 1, 64, d, L, L - 1)
    lsa_page_summary(shape, page, keys, kd, ks, page_lo, n_pages if page_hi is None else page_hi,
                     out, stream)
    return out


def page_recall(q, w, page_keys, keys, key_scale, k, sink, window, page, m_pages, q_pos0=None,
                ws: Optional[Workspace] = None, stream=None):
    """(page_ids [B,n_q,M], cand_scores [B,n_q,M*P], cand_ids [B,n_q,M*P])."""
    _need(q, "q", torch.bfloat16, 4)
    _need(w, "w", torch.float32, 3)
    _need(page_keys, "page_keys", torch.bfloat16, 3)
    kd, ks = _key_args(keys, key_scale)
    shape = index_shape(q, keys, q_pos0)
    B, T = shape.batch, shape.n_q
    bud = Budget(k, sink, window)
    dev = q.device
    page_ids = torch.empty((B, T, m_pages), dtype=torch.int32, device=dev)
    cs = torch.empty((B, T, m_pages * page), dtype=torch.float32, device=dev)
    ci = torch.empty((B, T, m_pages * page), dtype=torch.int32, device=dev)
    nb = lsa_workspace_bytes(OP_PAGE_RECALL, shape, bud, page, m_pages)
    wsb = (ws or Workspace()).get(nb, dev)
    lsa_page_recall(shape, bud, page, m_pages, q, w, page_keys, keys, kd, ks, page_ids, cs, ci,
                    wsb, nb, stream)
    return page_ids, cs, ci


def sparse_attn(q, k, v, idx, scale, sink=0, window=0, d_v=None, latent=None, want_lse=True,
                ws: Optional[Workspace] = None, out=None, stream=None):
    """out [B, n_q, Hq, d_v] bf16 and lse [B, n_q, Hq] fp32 (or None).  Latent cache: pass v=None
    (or v is k) and d_v = the value width."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 3)
    _need(idx, "idx", torch.int32, 3)
    if latent is None:
        latent = v is None or v is k
    if v is None:
        v = k
    B, T, Hq, dqk = q.shape
    L = k.shape[1]
    if d_v is None:
        d_v = v.shape[2] if not latent else dqk
    attn = AttnShape(Hq, dqk, d_v, 1 if latent else 0, k.shape[2], v.shape[2], scale)
    shape = IndexShape(B, T, 64, 128, L, 0)
    bud = Budget(idx.shape[2], sink, window)
    dev = q.device
    if out is None:
        out = torch.empty((B, T, Hq, d_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, T, Hq), dtype=torch.float32, device=dev) if want_lse else None
    nb = lsa_workspace_bytes(OP_SPARSE_ATTN, shape, bud, attn=attn)
    wsb = (ws or Workspace()).get(nb, dev)
    lsa_sparse_attn(shape, attn, bud, q, k, v, idx, out, lse, wsb, nb, stream)
    return out, lse
