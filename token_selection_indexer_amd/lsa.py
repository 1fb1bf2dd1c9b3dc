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
OP_TOPK_SELECT, OP_PAGE_RECALL, OP_SPARSE_ATTN, OP_INDEX_SELECT = 1, 2, 3, 4
STATUS = {0: "LSA_OK", 1: "LSA_ERR_NULL_POINTER", 2: "LSA_ERR_BAD_SHAPE", 3: "LSA_ERR_BAD_DTYPE",
          4: "LSA_ERR_UNSUPPORTED", 5: "LSA_ERR_WORKSPACE_TOO_SMALL", 6: "LSA_ERR_DEVICE"}
EXPORTS = ("lsa_index_scores", "lsa_topk_select", "lsa_page_summary", "lsa_page_recall",
           "lsa_sparse_attn", "lsa_workspace_bytes", "lsa_status_string",
           "lsa_topk_select_noalloc", "lsa_index_select", "lsa_quantize_queries",
           "lsa_index_scores_q8", "lsa_sparse_attn_backward", "lsa_index_scores_backward",
           "lsa_sparse_attn_layers")
MAX_ATTN_LAYERS = 8


class IndexShape(ctypes.Structure):
    """lsa_index_shape.  seq_len / seq_pos0: device pointers of per-sequence int32 arrays (ragged
    batches) or None.  block_table / block_size / blocks_per_seq / n_blocks: paged indexer keys
    (the table a device pointer), or None / 0 for dense keys."""
    _fields_ = [("batch", ctypes.c_int32), ("n_q", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("kv_len", ctypes.c_int64),
                ("q_pos0", ctypes.c_int64), ("seq_len", ctypes.c_void_p),
                ("seq_pos0", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("block_size", ctypes.c_int32), ("blocks_per_seq", ctypes.c_int32),
                ("n_blocks", ctypes.c_int64)]


class Budget(ctypes.Structure):
    _fields_ = [("k", ctypes.c_int32), ("sink", ctypes.c_int32), ("window", ctypes.c_int32)]


class AttnShape(ctypes.Structure):
    """lsa_attn_shape.  block_table / block_size / blocks_per_seq / n_blocks: a paged latent
    cache (the table a device pointer), or None / 0 for dense caches."""
    _fields_ = [("n_heads", ctypes.c_int32), ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("latent", ctypes.c_int32), ("k_row_stride", ctypes.c_int64),
                ("v_row_stride", ctypes.c_int64), ("scale", ctypes.c_float),
                ("block_table", ctypes.c_void_p), ("block_size", ctypes.c_int32),
                ("blocks_per_seq", ctypes.c_int32), ("n_blocks", ctypes.c_int64)]


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
        L.lsa_topk_select_noalloc.argtypes = [ip, bud, _VP, _I64, _VP, _VP, _VP]
        L.lsa_index_select.argtypes = [ip, bud, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _VP, _SZ, _VP]
        L.lsa_quantize_queries.argtypes = [ip, _VP, _VP, _VP, _VP]
        L.lsa_index_scores_q8.argtypes = [ip, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _VP]
        L.lsa_page_summary.argtypes = [ip, _I32, _VP, _I32, _VP, _I64, _I64, _VP, _VP]
        L.lsa_page_recall.argtypes = [ip, bud, _I32, _I32, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _VP,
                                      _VP, _VP, _SZ, _VP]
        L.lsa_sparse_attn.argtypes = [ip, ap, bud, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]
        L.lsa_sparse_attn_layers.argtypes = [ip, ap, bud, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                             _SZ, _VP]
        L.lsa_sparse_attn_backward.argtypes = [ip, ap, bud, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                               _VP, _VP, _VP, _VP]
        L.lsa_index_scores_backward.argtypes = [ip, bud, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                                _VP]
        L.lsa_workspace_bytes.argtypes = [_I32, ip, bud, _I32, _I32, _I64, ap]
        L.lsa_workspace_bytes.restype = _SZ
        L.lsa_status_string.argtypes = [_I32]
        L.lsa_status_string.restype = ctypes.c_char_p
        for f in EXPORTS[:5] + EXPORTS[7:]:
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


def lsa_quantize_queries(shape: IndexShape, q, q8, q_scale, stream=None):
    _check("lsa_quantize_queries", lib().lsa_quantize_queries(
        ctypes.byref(shape), _p(q), _p(q8), _p(q_scale), _s(stream)))


def lsa_index_scores_q8(shape: IndexShape, q8, q_scale, w, keys, key_dtype: int, key_scale,
                        scores, stream=None):
    _check("lsa_index_scores_q8", lib().lsa_index_scores_q8(
        ctypes.byref(shape), _p(q8), _p(q_scale), _p(w), _p(keys), key_dtype, _p(key_scale),
        _p(scores), _s(stream)))


def lsa_index_select(shape: IndexShape, budget: Budget, q, w, keys, key_dtype: int, key_scale,
                     scores, idx, ws=None, ws_bytes: int = 0, stream=None):
    _check("lsa_index_select", lib().lsa_index_select(
        ctypes.byref(shape), budget, _p(q), _p(w), _p(keys), key_dtype, _p(key_scale),
        _p(scores), _p(idx), _p(ws), ws_bytes, _s(stream)))


def lsa_topk_select_noalloc(shape: IndexShape, budget: Budget, scores, n_cand: int, cand_ids,
                            idx, stream=None):
    _check("lsa_topk_select_noalloc", lib().lsa_topk_select_noalloc(
        ctypes.byref(shape), budget, _p(scores), n_cand, _p(cand_ids), _p(idx), _s(stream)))


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


def lsa_sparse_attn_backward(shape: IndexShape, attn: AttnShape, budget: Budget, q, k, v, idx,
                             out, lse, d_out, d_q, d_k, d_v, stream=None):
    _check("lsa_sparse_attn_backward", lib().lsa_sparse_attn_backward(
        ctypes.byref(shape), ctypes.byref(attn), budget, _p(q), _p(k), _p(v), _p(idx), _p(out),
        _p(lse), _p(d_out), _p(d_q), _p(d_k), _p(d_v), _s(stream)))


def lsa_index_scores_backward(shape: IndexShape, budget: Budget, q, w, keys, idx, d_scores, d_q,
                              d_w, d_keys, stream=None):
    _check("lsa_index_scores_backward", lib().lsa_index_scores_backward(
        ctypes.byref(shape), budget, _p(q), _p(w), _p(keys), _p(idx), _p(d_scores), _p(d_q),
        _p(d_w), _p(d_keys), _s(stream)))


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


def _on_device(t: torch.Tensor) -> bool:
    return t.is_cuda


def _need(t: torch.Tensor, name: str, dtype=None, dim=None, shape=None, device=None):
    """Refuse what would hand the library a host pointer, a strided view, the wrong element type
    or a buffer of the wrong size."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not _on_device(t):
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, got {t.dim()}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _out(out, name, shape, dtype, device):
    """A caller-supplied output must match exactly; otherwise allocate one."""
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _need(out, name, dtype, shape=shape, device=device)
    return out


def _key_args(keys: torch.Tensor, key_scale: Optional[torch.Tensor]):
    """(key dtype code, scale) after checking that the scale matches the keys [B, L, d]."""
    if keys.dtype == torch.bfloat16:
        if key_scale is not None:
            raise ValueError("bf16 keys take no key_scale")
        return KEY_BF16, None
    if keys.dtype in (torch.uint8, torch.float8_e4m3fn):
        if key_scale is None:
            raise ValueError("fp8 keys need key_scale")
        _need(key_scale, "key_scale", torch.float32, shape=keys.shape[:2], device=keys.device)
        return KEY_FP8_E4M3, key_scale
    raise ValueError(f"keys must be bf16 or e4m3 codes, got {keys.dtype}")


def _check_index_operands(q, w, keys, paged=False):
    """paged: keys is a pool [n_blocks, block_size, d] (and key_scale [n_blocks, block_size])."""
    B, T, H, _ = q.shape
    _need(w, "w", torch.float32, shape=(B, T, H), device=q.device)
    _need(keys, "keys", (torch.bfloat16, torch.uint8, torch.float8_e4m3fn), dim=3, device=q.device)
    if (not paged and keys.shape[0] != B) or keys.shape[2] != q.shape[3]:
        raise ValueError(f"keys {tuple(keys.shape)} do not match q {tuple(q.shape)}")


def _ragged(shape: IndexShape, device, seq_lens=None, seq_pos0=None) -> IndexShape:
    """Attach per-sequence lengths / first-query positions (int32 device tensors [B])."""
    for t, name in ((seq_lens, "seq_lens"), (seq_pos0, "seq_pos0")):
        if t is not None:
            _need(t, name, torch.int32, shape=(shape.batch,), device=device)
    shape.seq_len = None if seq_lens is None else seq_lens.data_ptr()
    shape.seq_pos0 = None if seq_pos0 is None else seq_pos0.data_ptr()
    return shape


def index_shape(q: torch.Tensor, keys: torch.Tensor, q_pos0: Optional[int] = None,
                seq_lens=None, seq_pos0=None, block_table=None, kv_len=None) -> IndexShape:
    """block_table [B, blocks_per_seq] int32: keys is a pool [n_blocks, block_size, d] of paged
    keys (kv_len defaults to blocks_per_seq * block_size)."""
    B, T, H, d = q.shape
    if block_table is None:
        L = keys.shape[1]
    else:
        _need(block_table, "block_table", torch.int32, 2, device=q.device)
        if block_table.shape[0] != B:
            raise ValueError(f"block_table {tuple(block_table.shape)} does not match q {tuple(q.shape)}")
        L = block_table.shape[1] * keys.shape[1] if kv_len is None else kv_len
    sh = IndexShape(B, T, H, d, L, L - T if q_pos0 is None else q_pos0)
    if block_table is not None:
        sh.block_table = block_table.data_ptr()
        sh.block_size = keys.shape[1]
        sh.blocks_per_seq = block_table.shape[1]
        sh.n_blocks = keys.shape[0]
    return _ragged(sh, q.device, seq_lens, seq_pos0)


def index_scores(q, w, keys, key_scale=None, q_pos0=None, out=None, stream=None, seq_lens=None,
                 seq_pos0=None, block_table=None, kv_len=None):
    """scores [B, n_q, L] fp32 (q_pos0 defaults to L - n_q: the queries are the last tokens;
    seq_lens / seq_pos0: per-sequence int32 device tensors for a ragged batch; block_table:
    paged keys, see index_shape)."""
    _need(q, "q", torch.bfloat16, 4)
    _check_index_operands(q, w, keys, block_table is not None)
    kd, ks = _key_args(keys, key_scale)
    shape = index_shape(q, keys, q_pos0, seq_lens, seq_pos0, block_table, kv_len)
    out = _out(out, "out", (shape.batch, shape.n_q, shape.kv_len), torch.float32, q.device)
    lsa_index_scores(shape, q, w, keys, kd, ks, out, stream)
    return out


def quantize_queries(q, q8=None, q_scale=None, stream=None):
    """(q8 [B, n_q, H, d] uint8 e4m3 codes, q_scale [B, n_q, H] fp32) from bf16 q."""
    _need(q, "q", torch.bfloat16, 4)
    B, T, H, d = q.shape
    q8 = _out(q8, "q8", (B, T, H, d), torch.uint8, q.device)
    q_scale = _out(q_scale, "q_scale", (B, T, H), torch.float32, q.device)
    lsa_quantize_queries(IndexShape(B, T, H, d, 1, 0), q, q8, q_scale, stream)
    return q8, q_scale


def index_scores_q8(q8, q_scale, w, keys, key_scale, q_pos0=None, out=None, stream=None,
                    seq_lens=None, seq_pos0=None):
    """scores [B, n_q, L] fp32 of fp8 queries (quantize_queries) against fp8 keys."""
    _need(q8, "q8", torch.uint8, 4)
    B, T, H, d = q8.shape
    _need(q_scale, "q_scale", torch.float32, shape=(B, T, H), device=q8.device)
    _need(w, "w", torch.float32, shape=(B, T, H), device=q8.device)
    _need(keys, "keys", (torch.uint8, torch.float8_e4m3fn), dim=3, device=q8.device)
    if keys.shape[0] != B or keys.shape[2] != d:
        raise ValueError(f"keys {tuple(keys.shape)} do not match q8 {tuple(q8.shape)}")
    kd, ks = _key_args(keys, key_scale)
    L = keys.shape[1]
    shape = _ragged(IndexShape(B, T, H, d, L, L - T if q_pos0 is None else q_pos0), q8.device,
                    seq_lens, seq_pos0)
    out = _out(out, "out", (B, T, L), torch.float32, q8.device)
    lsa_index_scores_q8(shape, q8, q_scale, w, keys, kd, ks, out, stream)
    return out


def index_select(q, w, keys, key_scale, k, sink, window, q_pos0=None, scores=None, idx=None,
                 ws: Optional[Workspace] = None, stream=None, seq_lens=None, seq_pos0=None,
                 block_table=None, kv_len=None):
    """Scores [B, n_q, L] fp32 and the selection idx [B, n_q, k] int32 in one call (fused for
    decode): the outputs of index_scores followed by topk_select (paged keys as there)."""
    _need(q, "q", torch.bfloat16, 4)
    _check_index_operands(q, w, keys, block_table is not None)
    kd, ks = _key_args(keys, key_scale)
    shape = index_shape(q, keys, q_pos0, seq_lens, seq_pos0, block_table, kv_len)
    B, T, L = shape.batch, shape.n_q, shape.kv_len
    scores = _out(scores, "scores", (B, T, L), torch.float32, q.device)
    idx = _out(idx, "idx", (B, T, k), torch.int32, q.device)
    bud = Budget(k, sink, window)
    nb = lsa_workspace_bytes(OP_INDEX_SELECT, shape, bud)
    wsb = (ws or Workspace()).get(nb, q.device)
    lsa_index_select(shape, bud, q, w, keys, kd, ks, scores, idx, wsb, nb, stream)
    return scores, idx


def topk_select(scores, k, sink, window, kv_len, q_pos0, cand_ids=None, out=None,
                ws: Optional[Workspace] = None, stream=None, seq_lens=None, seq_pos0=None):
    """idx [B, n_q, k] int32 from flat scores [B, n_q, L] or candidates (scores, cand_ids)."""
    _need(scores, "scores", torch.float32, 3)
    B, T, n = scores.shape
    shape = _ragged(IndexShape(B, T, 1, 64, kv_len, q_pos0), scores.device, seq_lens, seq_pos0)
    if cand_ids is not None:
        _need(cand_ids, "cand_ids", torch.int32, shape=scores.shape, device=scores.device)
    out = _out(out, "out", (B, T, k), torch.int32, scores.device)
    bud = Budget(k, sink, window)
    nb = lsa_workspace_bytes(OP_TOPK_SELECT, shape, bud, n_cand=n)
    wsb = (ws or Workspace()).get(nb, scores.device)
    lsa_topk_select(shape, bud, scores, n, cand_ids, out, wsb, nb, stream)
    return out


def page_summary(keys, key_scale, page, page_lo=0, page_hi=None, out=None, stream=None,
                 seq_lens=None, block_table=None, kv_len=None):
    """page keys [B, ceil(L/P), d] bf16.  block_table [B, blocks_per_seq] int32: keys (and
    key_scale) are pools [n_blocks, block_size, d] with page <= block_size."""
    _need(keys, "keys", (torch.bfloat16, torch.uint8, torch.float8_e4m3fn), dim=3)
    kd, ks = _key_args(keys, key_scale)
    if block_table is None:
        B, L, d = keys.shape
    else:
        _need(block_table, "block_table", torch.int32, 2, device=keys.device)
        B, d = block_table.shape[0], keys.shape[2]
        L = block_table.shape[1] * keys.shape[1] if kv_len is None else kv_len
    n_pages = (L + page - 1) // page
    out = _out(out, "out", (B, n_pages, d), torch.bfloat16, keys.device)
    shape = _ragged(IndexShape(B, 1, 64, d, L, L - 1), keys.device, seq_lens)
    if block_table is not None:
        shape.block_table = block_table.data_ptr()
        shape.block_size = keys.shape[1]
        shape.blocks_per_seq = block_table.shape[1]
        shape.n_blocks = keys.shape[0]
    lsa_page_summary(shape, page, keys, kd, ks, page_lo, n_pages if page_hi is None else page_hi,
                     out, stream)
    return out


def page_recall(q, w, page_keys, keys, key_scale, k, sink, window, page, m_pages, q_pos0=None,
                ws: Optional[Workspace] = None, stream=None, seq_lens=None, seq_pos0=None,
                block_table=None, kv_len=None):
    """(page_ids [B,n_q,M], cand_scores [B,n_q,M*P], cand_ids [B,n_q,M*P]); paged keys as for
    index_scores, with page <= block_size."""
    _need(q, "q", torch.bfloat16, 4)
    _check_index_operands(q, w, keys, block_table is not None)
    kd, ks = _key_args(keys, key_scale)
    shape = index_shape(q, keys, q_pos0, seq_lens, seq_pos0, block_table, kv_len)
    _need(page_keys, "page_keys", torch.bfloat16, device=q.device,
          shape=(shape.batch, (shape.kv_len + page - 1) // page, shape.head_dim))
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


def _attn_layer(q, k, v, idx, d_v, latent, ref=None, paged=False):
    """Checks one layer's q [B, n_q, Hq, d_qk] / cache / index lists; returns (v, d_v, latent,
    AttnShape args).  ref: the first layer's q and cache, which every later layer must match.
    paged: k is a pool [n_blocks, block_size, row] (latent only)."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 3)
    _need(idx, "idx", torch.int32, 3)
    if latent is None:
        latent = v is None or v is k
    if v is None:
        v = k
    if paged and not latent:
        raise ValueError("a paged cache is a latent cache (v is k)")
    B, T, Hq, dqk = q.shape
    dev = q.device
    _need(k, "k", torch.bfloat16, device=dev)
    if (not paged and k.shape[0] != B) or k.shape[2] < dqk:
        raise ValueError(f"k {tuple(k.shape)} does not match q {tuple(q.shape)}")
    _need(v, "v", torch.bfloat16, 3, device=dev)
    if v.shape[:2] != k.shape[:2]:
        raise ValueError(f"v {tuple(v.shape)} does not match k {tuple(k.shape)}")
    _need(idx, "idx", torch.int32, device=dev)
    if idx.shape[:2] != (B, T):
        raise ValueError(f"idx {tuple(idx.shape)} does not match q {tuple(q.shape)}")
    if d_v is None:
        d_v = v.shape[2] if not latent else dqk
    if d_v > v.shape[2]:
        raise ValueError(f"d_v {d_v} exceeds the value rows ({v.shape[2]})")
    if ref is not None:
        q0, k0, v0 = ref
        if q.shape != q0.shape or k.shape != k0.shape or v.shape != v0.shape or q.device != q0.device:
            raise ValueError("every layer needs the first layer's q and cache shapes")
    return v, d_v, latent, (Hq, dqk, d_v, 1 if latent else 0, k.shape[2], v.shape[2])


def _attn_shape(q, k, idx, sink, window, seq_lens, q_pos0, seq_pos0, block_table=None,
                kv_len=None):
    B, T = q.shape[0], q.shape[1]
    if block_table is None:
        L = k.shape[1]
    else:
        _need(block_table, "block_table", torch.int32, 2, device=q.device)
        if block_table.shape[0] != B:
            raise ValueError(f"block_table {tuple(block_table.shape)} does not match q {tuple(q.shape)}")
        L = block_table.shape[1] * k.shape[1] if kv_len is None else kv_len
    pos0 = max(0, L - T) if q_pos0 is None else q_pos0
    shape = _ragged(IndexShape(B, T, 64, 128, L, pos0), q.device, seq_lens, seq_pos0)
    return shape, Budget(idx.shape[2], sink, window)


def _paged(attn: AttnShape, k, block_table):
    """Fill the paged-cache fields of attn: k is the pool [n_blocks, block_size, row]."""
    if block_table is not None:
        attn.block_table = block_table.data_ptr()
        attn.block_size = k.shape[1]
        attn.blocks_per_seq = block_table.shape[1]
        attn.n_blocks = k.shape[0]
    return attn


def sparse_attn(q, k, v, idx, scale, sink=0, window=0, d_v=None, latent=None, want_lse=True,
                ws: Optional[Workspace] = None, out=None, stream=None, seq_lens=None, q_pos0=None,
                seq_pos0=None, block_table=None, kv_len=None):
    """out [B, n_q, Hq, d_v] bf16 and lse [B, n_q, Hq] fp32 (or None).  Latent cache: pass v=None
    (or v is k) and d_v = the value width.  sink, window and the query positions (q_pos0, default
    L - n_q; seq_pos0 for a ragged batch) describe the lists' Streaming-Aware layout: the kernel
    starts loading the rows that layout names before the lists arrive (the result never depends
    on them).  block_table [B, blocks_per_seq] int32: k is a paged latent cache, a pool
    [n_blocks, block_size, row] (kv_len defaults to blocks_per_seq * block_size)."""
    v, d_v, latent, ashape = _attn_layer(q, k, v, idx, d_v, latent, paged=block_table is not None)
    attn = _paged(AttnShape(*ashape, scale), k, block_table)
    shape, bud = _attn_shape(q, k, idx, sink, window, seq_lens, q_pos0, seq_pos0, block_table,
                             kv_len)
    B, T, Hq = q.shape[:3]
    dev = q.device
    out = _out(out, "out", (B, T, Hq, d_v), torch.bfloat16, dev)
    lse = torch.empty((B, T, Hq), dtype=torch.float32, device=dev) if want_lse else None
    nb = lsa_workspace_bytes(OP_SPARSE_ATTN, shape, bud, attn=attn)
    wsb = (ws or Workspace()).get(nb, dev)
    lsa_sparse_attn(shape, attn, bud, q, k, v, idx, out, lse, wsb, nb, stream)
    return out, lse


def lsa_sparse_attn_layers(shape: IndexShape, attn: AttnShape, budget: Budget, qs, ks, vs, idx,
                           outs, lses, ws, ws_bytes: int, stream=None):
    n = len(qs)
    arr = lambda ts: (ctypes.c_void_p * n)(*[None if t is None else t.data_ptr() for t in ts])
    lse_arr = None if lses is None else arr(lses)
    _check("lsa_sparse_attn_layers", lib().lsa_sparse_attn_layers(
        ctypes.byref(shape), ctypes.byref(attn), budget, n, arr(qs), arr(ks), arr(vs), _p(idx),
        arr(outs), lse_arr, _p(ws), ws_bytes, _s(stream)))


def sparse_attn_layers(qs, ks, idx, scale, sink=0, window=0, d_v=None, vs=None, latent=None,
                       want_lse=True, ws: Optional[Workspace] = None, outs=None, stream=None,
                       seq_lens=None, q_pos0=None, seq_pos0=None, block_table=None, kv_len=None):
    """sparse_attn for a group of layers sharing one index list (Cross-Layer Indexing) in one
    call: lists of per-layer q and cache (vs: per-layer value caches, None for latent caches)
    -> lists of out and lse.  Each layer computes what its own sparse_attn call computes; the
    split merge is planned for the whole launch, so the last bits can differ from that call."""
    n = len(qs)
    if not 1 <= n <= MAX_ATTN_LAYERS or len(ks) != n or (vs is not None and len(vs) != n):
        raise ValueError(f"1..{MAX_ATTN_LAYERS} layers, one q and one cache each")
    vs = [None] * n if vs is None else list(vs)
    paged = block_table is not None
    v0, d_v0, latent0, ashape = _attn_layer(qs[0], ks[0], vs[0], idx, d_v, latent, paged=paged)
    vv = [v0]
    for l in range(1, n):
        v, _, lat, ash = _attn_layer(qs[l], ks[l], vs[l], idx, d_v, latent, (qs[0], ks[0], v0),
                                     paged=paged)
        if lat != latent0 or ash != ashape:
            raise ValueError("every layer needs the first layer's attention shape")
        vv.append(v)
    attn = _paged(AttnShape(*ashape, scale), ks[0], block_table)
    shape, bud = _attn_shape(qs[0], ks[0], idx, sink, window, seq_lens, q_pos0, seq_pos0,
                             block_table, kv_len)
    B, T, Hq = qs[0].shape[:3]
    dev = qs[0].device
    outs = [_out(None if outs is None else outs[l], "out", (B, T, Hq, d_v0), torch.bfloat16, dev)
            for l in range(n)]
    lses = ([torch.empty((B, T, Hq), dtype=torch.float32, device=dev) for _ in range(n)]
            if want_lse else None)
    nb = n * lsa_workspace_bytes(OP_SPARSE_ATTN, shape, bud, attn=attn)
    wsb = (ws or Workspace()).get(nb, dev)
    lsa_sparse_attn_layers(shape, attn, bud, qs, ks, vv, idx, outs, lses, wsb, nb, stream)
    return outs, lses


def sparse_attn_backward(q, k, v, idx, out, lse, d_out, scale, d_v=None, latent=None, d_q=None,
                         d_k=None, d_vg=None, stream=None, seq_lens=None, sink=0, window=0,
                         q_pos0=0):
    """Gradients of sparse_attn, ADDED into fp32 d_q [B,n_q,Hq,d_qk], d_k [B,L,d_qk] and d_vg
    [B,L,d_v] (zeros are allocated for the ones not given).  Latent cache (v None or v is k):
    one cache gradient d_k, whose first d_v columns also take dV; d_vg is then d_k.  sink,
    window and q_pos0 describe the lists' Streaming-Aware layout (as topk_select writes it),
    which lets the library sum the sink and window rows' gradients key by key."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 3, device=q.device)
    _need(idx, "idx", torch.int32, 3, device=q.device)
    if latent is None:
        latent = v is None or v is k
    if v is None:
        v = k
    B, T, Hq, dqk = q.shape
    L = k.shape[1]
    dev = q.device
    if k.shape[0] != B or k.shape[2] < dqk:
        raise ValueError(f"k {tuple(k.shape)} does not match q {tuple(q.shape)}")
    _need(v, "v", torch.bfloat16, 3, device=dev)
    if v.shape[:2] != k.shape[:2]:
        raise ValueError(f"v {tuple(v.shape)} does not match k {tuple(k.shape)}")
    if idx.shape[:2] != (B, T):
        raise ValueError(f"idx {tuple(idx.shape)} does not match q {tuple(q.shape)}")
    if d_v is None:
        d_v = v.shape[2] if not latent else dqk
    if d_v > v.shape[2]:
        raise ValueError(f"d_v {d_v} exceeds the value rows ({v.shape[2]})")
    _need(out, "out", torch.bfloat16, shape=(B, T, Hq, d_v), device=dev)
    _need(lse, "lse", torch.float32, shape=(B, T, Hq), device=dev)
    _need(d_out, "d_out", torch.bfloat16, shape=(B, T, Hq, d_v), device=dev)
    d_q = _zeros_or(d_q, "d_q", (B, T, Hq, dqk), dev)
    d_k = _zeros_or(d_k, "d_k", (B, L, dqk), dev)
    if latent:
        if d_vg is not None and d_vg is not d_k:
            raise ValueError("a latent cache has one gradient: d_vg must be d_k or None")
        d_vg = d_k
    else:
        d_vg = _zeros_or(d_vg, "d_vg", (B, L, d_v), dev)
    attn = AttnShape(Hq, dqk, d_v, 1 if latent else 0, k.shape[2], v.shape[2], scale)
    shape = _ragged(IndexShape(B, T, 64, 128, L, int(q_pos0)), dev, seq_lens)
    lsa_sparse_attn_backward(shape, attn, Budget(idx.shape[2], int(sink), int(window)), q, k, v,
                             idx, out, lse, d_out, d_q, d_k, d_vg, stream)
    return d_q, d_k, d_vg


def index_scores_backward(q, w, keys, idx, d_scores, q_pos0=None, d_q=None, d_w=None,
                          d_keys=None, stream=None, seq_lens=None, seq_pos0=None, sink=0, window=0):
    """Gradients of the indexer scores at the selected entries idx [B,n_q,k] for d_scores
    [B,n_q,k] fp32, ADDED into fp32 d_q [B,n_q,H,d], d_w [B,n_q,H], d_keys [B,L,d] (zeros are
    allocated for the ones not given).  bf16 keys.  sink and window (with q_pos0) describe the
    lists' Streaming-Aware layout, which lets the library sum the sink and window rows' key
    gradients row by row."""
    _need(q, "q", torch.bfloat16, 4)
    _check_index_operands(q, w, keys)
    if keys.dtype != torch.bfloat16:
        raise ValueError("the indexer backward takes bf16 keys")
    B, T, H, d = q.shape
    L = keys.shape[1]
    dev = q.device
    _need(idx, "idx", torch.int32, 3, device=dev)
    if idx.shape[:2] != (B, T):
        raise ValueError(f"idx {tuple(idx.shape)} does not match q {tuple(q.shape)}")
    _need(d_scores, "d_scores", torch.float32, shape=idx.shape, device=dev)
    d_q = _zeros_or(d_q, "d_q", (B, T, H, d), dev)
    d_w = _zeros_or(d_w, "d_w", (B, T, H), dev)
    d_keys = _zeros_or(d_keys, "d_keys", (B, L, d), dev)
    shape = index_shape(q, keys, q_pos0, seq_lens, seq_pos0)
    lsa_index_scores_backward(shape, Budget(idx.shape[2], sink, window), q, w, keys, idx,
                              d_scores, d_q, d_w, d_keys, stream)
    return d_q, d_w, d_keys


def _zeros_or(t, name, shape, device):
    """A caller-supplied gradient accumulator (checked), or a fresh zero one."""
    if t is None:
        return torch.zeros(shape, dtype=torch.float32, device=device)
    _need(t, name, torch.float32, shape=shape, device=device)
    return t
