"""The C ABI on the host (no GPU): the library loads, exports exactly what include/lsa.h
declares, sizes workspaces, and rejects bad arguments before touching the device.

Pointers passed here are fake (aligned integers): every call below fails validation, which runs
before any HIP call, so nothing is ever dereferenced or launched.
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest

from token_selection_indexer_amd import lsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lsa.h")
FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(lsa.LIB_PATH):
        from token_selection_indexer_amd import build
        build.build()
    return lsa.lib()


def declared_symbols():
    src = open(HEADER).read()
    return set(re.findall(r"LSA_API\s+[\w\s\*]+?\b(lsa_\w+)\s*\(", src))


def test_exports_match_header(L):
    decl = declared_symbols()
    assert decl == set(lsa.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", lsa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert exported == decl
    for s in decl:
        assert hasattr(L, s)


def test_status_strings(L):
    for code, name in lsa.STATUS.items():
        assert lsa.lsa_status_string(code) == name
    assert lsa.lsa_status_string(99) == "LSA_ERR_UNKNOWN"


def _shape(B=2, T=1, H=64, d=128, Lk=4096, pos=None):
    return lsa.IndexShape(B, T, H, d, Lk, Lk - 1 if pos is None else pos)


def test_workspace_sizes(L):
    sh = _shape(B=4, T=1, Lk=1 << 20)
    b = lsa.Budget(2048, 128, 896)
    n = lsa.lsa_workspace_bytes(lsa.OP_PAGE_RECALL, sh, b, 64, 256)
    assert n == 4 * 1 * (1 << 14) * 4
    # few long rows are split over workgroups (workspace); many rows use one workgroup each
    assert lsa.lsa_workspace_bytes(lsa.OP_TOPK_SELECT, sh, b) > 0
    assert lsa.lsa_workspace_bytes(lsa.OP_TOPK_SELECT, _shape(B=1, T=8192, Lk=131072), b) == 0
    assert lsa.lsa_workspace_bytes(lsa.OP_TOPK_SELECT, _shape(B=4, Lk=4096), b) == 0
    att = lsa.AttnShape(16, 576, 512, 1, 576, 576, 576 ** -0.5)
    n_att = lsa.lsa_workspace_bytes(lsa.OP_SPARSE_ATTN, _shape(B=32), b, attn=att)
    assert n_att > 0 and n_att % 256 == 0
    # one query per sequence and many sequences: no split, no workspace
    assert lsa.lsa_workspace_bytes(lsa.OP_SPARSE_ATTN, _shape(B=1, T=8192), b, attn=att) == 0
    with pytest.raises(lsa.LsaError):
        lsa.lsa_workspace_bytes(lsa.OP_PAGE_RECALL, sh, b, 48, 256)  # page not a power of two
    with pytest.raises(lsa.LsaError):
        lsa.lsa_workspace_bytes(99, sh, b)


def _scores_call(L, shape, q=FAKE, w=FAKE, keys=FAKE, kd=lsa.KEY_BF16, scale=None, out=FAKE):
    return L.lsa_index_scores(ctypes.byref(shape) if shape is not None else None,
                              ctypes.c_void_p(q) if q else None, ctypes.c_void_p(w) if w else None,
                              ctypes.c_void_p(keys) if keys else None, kd,
                              ctypes.c_void_p(scale) if scale else None,
                              ctypes.c_void_p(out) if out else None, None)


def test_index_scores_rejects(L):
    assert _scores_call(L, None) == 1
    assert _scores_call(L, _shape(), q=0) == 1
    assert _scores_call(L, _shape(), out=0) == 1
    assert _scores_call(L, _shape(H=12)) == 4          # head count not built
    assert _scores_call(L, _shape(d=96)) == 4
    assert _scores_call(L, _shape(Lk=0)) == 2
    assert _scores_call(L, _shape(pos=-1)) == 2
    assert _scores_call(L, _shape(), kd=7) == 3
    assert _scores_call(L, _shape(), kd=lsa.KEY_FP8_E4M3, scale=None) == 3
    assert _scores_call(L, _shape(), kd=lsa.KEY_BF16, scale=FAKE) == 3
    assert _scores_call(L, _shape(), q=FAKE + 2) == 2  # misaligned q


def _topk_call(L, shape, budget, n_cand, cand=None, scores=FAKE, idx=FAKE):
    return L.lsa_topk_select(ctypes.byref(shape), budget, ctypes.c_void_p(scores) if scores else None,
                             n_cand, ctypes.c_void_p(cand) if cand else None,
                             ctypes.c_void_p(idx) if idx else None, None, 0, None)


def test_topk_rejects(L):
    sh = _shape()
    assert _topk_call(L, sh, lsa.Budget(0, 0, 0), sh.kv_len) == 2
    assert _topk_call(L, sh, lsa.Budget(64, 40, 40), sh.kv_len) == 2  # S + W > k
    assert _topk_call(L, sh, lsa.Budget(64, -1, 4), sh.kv_len) == 2
    assert _topk_call(L, sh, lsa.Budget(64, 4, 4), sh.kv_len - 1) == 2  # flat: n_cand != L
    assert _topk_call(L, sh, lsa.Budget(64, 4, 4), 0, cand=FAKE) == 2
    assert _topk_call(L, sh, lsa.Budget(64, 4, 4), sh.kv_len, scores=0) == 1
    assert _topk_call(L, sh, lsa.Budget(64, 4, 4), sh.kv_len, scores=FAKE + 4) == 2
    assert _topk_call(L, sh, lsa.Budget(1 << 20, 0, 0), sh.kv_len) == 4
    big = _shape(B=4, Lk=1 << 20)  # chunked selection: the workspace is required
    assert _topk_call(L, big, lsa.Budget(2048, 128, 896), big.kv_len) == 5


def test_page_summary_rejects(L):
    sh = _shape(Lk=1000)
    f = L.lsa_page_summary
    v = ctypes.c_void_p
    assert f(ctypes.byref(sh), 48, v(FAKE), lsa.KEY_BF16, None, 0, 1, v(FAKE), None) == 2
    assert f(ctypes.byref(sh), 512, v(FAKE), lsa.KEY_BF16, None, 0, 1, v(FAKE), None) == 2
    assert f(ctypes.byref(sh), 64, v(FAKE), lsa.KEY_BF16, None, 0, 17, v(FAKE), None) == 2
    assert f(ctypes.byref(sh), 64, v(FAKE), lsa.KEY_BF16, None, 5, 4, v(FAKE), None) == 2
    assert f(ctypes.byref(sh), 64, v(FAKE), lsa.KEY_FP8_E4M3, None, 0, 1, v(FAKE), None) == 3
    assert f(ctypes.byref(sh), 64, v(FAKE), lsa.KEY_BF16, None, 0, 1, None, None) == 1
    sh96 = _shape(d=96)
    assert f(ctypes.byref(sh96), 64, v(FAKE), lsa.KEY_BF16, None, 0, 1, v(FAKE), None) == 4


def test_page_recall_rejects(L):
    sh = _shape(B=4, Lk=1 << 20)
    b = lsa.Budget(2048, 128, 896)
    v = ctypes.c_void_p

    def call(P=64, M=256, ws=FAKE, nbytes=None, q=FAKE):
        nb = lsa.lsa_workspace_bytes(lsa.OP_PAGE_RECALL, sh, b, 64, 256) if nbytes is None else nbytes
        return L.lsa_page_recall(ctypes.byref(sh), b, P, M, v(q) if q else None, v(FAKE), v(FAKE),
                                 v(FAKE), lsa.KEY_FP8_E4M3, v(FAKE), v(FAKE), v(FAKE), v(FAKE),
                                 v(ws) if ws else None, nb, None)
    assert call(P=16) == 2       # fine stage needs pages of whole 32-key blocks
    assert call(P=96) == 2
    assert call(M=0) == 2
    assert call(q=0) == 1
    assert call(ws=0) == 5
    assert call(nbytes=1024) == 5
    # a causal chunk whose window is shorter than a page could recall a page holding later
    # tokens: refused
    pre = _shape(B=1, T=512, Lk=1 << 20, pos=(1 << 20) - 1024)
    nb = lsa.lsa_workspace_bytes(lsa.OP_PAGE_RECALL, pre, b, 64, 256)
    for W, want in ((32, 4), (63, 5)):  # 63 = P - 1 passes the check (and then lacks a ws)
        assert L.lsa_page_recall(ctypes.byref(pre), lsa.Budget(2048, 128, W), 64, 256, v(FAKE),
                                 v(FAKE), v(FAKE), v(FAKE), lsa.KEY_FP8_E4M3, v(FAKE), v(FAKE),
                                 v(FAKE), v(FAKE), None, nb, None) == want


def test_sparse_attn_rejects(L):
    sh = _shape(B=32)
    b = lsa.Budget(2048, 64, 960)
    v = ctypes.c_void_p

    def call(attn, k=FAKE, vv=FAKE, ws=None, nb=0, idx=FAKE):
        return L.lsa_sparse_attn(ctypes.byref(sh), ctypes.byref(attn), b, v(FAKE), v(k), v(vv),
                                 v(idx) if idx else None, v(FAKE), None, v(ws) if ws else None, nb,
                                 None)
    mla = lsa.AttnShape(16, 576, 512, 1, 576, 576, 0.04)
    assert call(mla, vv=FAKE + 4096) == 2                     # latent: v must be k
    assert call(mla, idx=0) == 1
    assert call(mla) == 5                                       # split-K needs a workspace
    assert call(lsa.AttnShape(8, 576, 512, 1, 576, 576, 0.04)) == 4   # heads % 16
    assert call(lsa.AttnShape(16, 512, 512, 1, 576, 576, 0.04)) == 4  # not the MLA shape
    assert call(lsa.AttnShape(1, 128, 128, 0, 100, 128, 0.1)) == 2   # stride % 8
    assert call(lsa.AttnShape(1, 512, 128, 0, 512, 128, 0.1)) == 4   # per-head d <= 256
    assert call(lsa.AttnShape(1, 128, 128, 0, 64, 128, 0.1)) == 2    # stride < d_qk


def test_sparse_attn_layers_rejects(L):
    sh = _shape(B=32)
    b = lsa.Budget(2048, 64, 960)
    v = ctypes.c_void_p
    mla = lsa.AttnShape(16, 576, 512, 1, 576, 576, 0.04)
    arr = lambda *p: (v * len(p))(*p)

    def call(n, q=None, k=None, out=None, ws=None, nb=0, idx=FAKE):
        q = q or arr(*[FAKE] * max(n, 1))
        k = k or arr(*[FAKE + 4096] * max(n, 1))
        out = out or arr(*[FAKE + 8192] * max(n, 1))
        return L.lsa_sparse_attn_layers(ctypes.byref(sh), ctypes.byref(mla), b, n, q, k, k,
                                        v(idx) if idx else None, out, None, v(ws) if ws else None,
                                        nb, None)
    assert call(0) == 2 and call(9) == 2                         # 1 .. 8 layers
    assert call(2, q=arr(FAKE, None)) == 1                       # a NULL entry
    assert call(2, idx=0) == 1
    assert call(2, k=arr(FAKE + 4096, FAKE + 4100)) == 2         # a misaligned cache
    one = lsa.lsa_workspace_bytes(lsa.OP_SPARSE_ATTN, sh, b, attn=mla)
    assert one > 0
    assert call(3, ws=FAKE, nb=one // 2) == 5                    # too small for 3 layers
    assert call(3, ws=None, nb=0) == 5                           # split-K needs a workspace
    nullarr = ctypes.cast(None, ctypes.POINTER(v))
    assert L.lsa_sparse_attn_layers(ctypes.byref(sh), ctypes.byref(mla), b, 2, nullarr,
                                    arr(FAKE, FAKE), arr(FAKE, FAKE), v(FAKE), arr(FAKE, FAKE),
                                    None, None, 0, None) == 1


def test_no_host_fallback_and_missing_library_fails_loudly(tmp_path):
    """The binding has no CPU path: host tensors are refused, and without the built library every
    call raises instead of computing anything some other way."""
    import torch
    q = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16)
    w = torch.zeros((1, 1, 64), dtype=torch.float32)
    keys = torch.zeros((1, 64, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        lsa.index_scores(q, w, keys)
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from token_selection_indexer_amd import lsa\n"
            "lsa.LIB_PATH = %r\n"
            "try:\n"
            "    lsa.lib()\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n") % (ROOT, str(tmp_path / "liblsa.so"))
    out = subprocess.run([sys.executable, "-c", code], capture_output=True,
                         text=True, timeout=120)
    assert "raised: HIP library not built" in out.stdout, out.stdout + out.stderr


def test_binding_checks_every_tensor(monkeypatch):
    """Every tensor the binding hands to the library is checked (device, dtype, shape,
    contiguity) before the call: a host key_scale, a wrong-shaped out= or a mismatched w is
    refused with ValueError, so no host pointer or undersized buffer reaches a kernel.  Host
    tensors stand in for device ones here (no GPU); the library itself must never be reached."""
    import torch

    def no_lib():
        raise AssertionError("the library was called despite a bad argument")

    monkeypatch.setattr(lsa, "lib", no_lib)
    host_scale = torch.ones((1, 64), dtype=torch.float32)
    monkeypatch.setattr(lsa, "_on_device", lambda t: t is not host_scale)
    q = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16)
    w = torch.zeros((1, 1, 64), dtype=torch.float32)
    keys8 = torch.zeros((1, 64, 128), dtype=torch.uint8)
    with pytest.raises(ValueError, match="key_scale must be a device tensor"):
        lsa.index_scores(q, w, keys8, host_scale)
    with pytest.raises(ValueError, match="key_scale must have shape"):
        lsa.index_scores(q, w, keys8, torch.ones((1, 63), dtype=torch.float32))
    with pytest.raises(ValueError, match="out must have shape"):
        lsa.index_scores(q, w, keys8, torch.ones((1, 64)), out=torch.empty((1, 1, 63)))
    with pytest.raises(ValueError, match="out must be"):
        lsa.index_scores(q, w, keys8, torch.ones((1, 64)), out=torch.empty((1, 1, 64),
                                                                            dtype=torch.float64))
    with pytest.raises(ValueError, match="w must have shape"):
        lsa.index_scores(q, torch.zeros((1, 1, 32)), keys8, torch.ones((1, 64)))
    with pytest.raises(ValueError, match="keys .* do not match"):
        lsa.index_scores(q, w, torch.zeros((2, 64, 128), dtype=torch.uint8), torch.ones((2, 64)))
    with pytest.raises(ValueError, match="bf16 keys take no key_scale"):
        lsa.index_scores(q, w, keys8.to(torch.bfloat16), torch.ones((1, 64)))
    sc = torch.zeros((1, 1, 64), dtype=torch.float32)
    with pytest.raises(ValueError, match="cand_ids must have shape"):
        lsa.topk_select(sc, 16, 2, 4, kv_len=64, q_pos0=63,
                        cand_ids=torch.zeros((1, 1, 32), dtype=torch.int32))
    with pytest.raises(ValueError, match="out must have shape"):
        lsa.topk_select(sc, 16, 2, 4, kv_len=64, q_pos0=63, out=torch.empty((1, 1, 8),
                                                                             dtype=torch.int32))
    aq = torch.zeros((1, 1, 16, 576), dtype=torch.bfloat16)
    kv = torch.zeros((1, 64, 576), dtype=torch.bfloat16)
    idx = torch.zeros((1, 1, 16), dtype=torch.int32)
    with pytest.raises(ValueError, match="out must have shape"):
        lsa.sparse_attn(aq, kv, None, idx, 0.04, d_v=512,
                        out=torch.empty((1, 1, 16, 256), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="idx .* does not match"):
        lsa.sparse_attn(aq, kv, None, torch.zeros((2, 1, 16), dtype=torch.int32), 0.04, d_v=512)
    with pytest.raises(ValueError, match="v .* does not match"):
        lsa.sparse_attn(aq[..., :128].contiguous(), kv[..., :128].contiguous(),
                        torch.zeros((1, 32, 128), dtype=torch.bfloat16), idx, 0.1)
    pool = torch.zeros((4, 64, 576), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="paged cache is a latent cache"):
        lsa.sparse_attn(torch.zeros((1, 1, 1, 128), dtype=torch.bfloat16),
                        pool[..., :128].contiguous(), torch.zeros((4, 64, 128), dtype=torch.bfloat16),
                        torch.zeros((1, 1, 16), dtype=torch.int32), 0.1, latent=False,
                        block_table=torch.zeros((1, 4), dtype=torch.int32))
    with pytest.raises(ValueError, match="block_table .* does not match"):
        lsa.sparse_attn(torch.zeros((2, 1, 16, 576), dtype=torch.bfloat16), pool, None,
                        torch.zeros((2, 1, 16), dtype=torch.int32), 0.04, d_v=512,
                        block_table=torch.zeros((1, 4), dtype=torch.int32))
    with pytest.raises(ValueError, match="page_keys must have shape"):
        lsa.page_recall(q, w, torch.zeros((1, 3, 128), dtype=torch.bfloat16), keys8,
                        torch.ones((1, 64)), 16, 2, 4, 32, 1)


def test_topk_select_noalloc_rejects(L):
    """The no-allocation selection validates like lsa_topk_select and refuses, before any HIP
    call, a chunked selection whose scratch would exceed the library's 16 MiB."""
    sh = _shape()
    v = ctypes.c_void_p

    def call(shape, budget, n_cand, scores=FAKE, cand=None):
        return L.lsa_topk_select_noalloc(ctypes.byref(shape), budget,
                                         v(scores) if scores else None, n_cand,
                                         v(cand) if cand else None, v(FAKE), None)
    assert call(sh, lsa.Budget(0, 0, 0), sh.kv_len) == 2
    assert call(sh, lsa.Budget(64, 4, 4), sh.kv_len - 1) == 2
    assert call(sh, lsa.Budget(64, 4, 4), sh.kv_len, scores=0) == 1
    huge = _shape(B=1000, Lk=1 << 20)  # 1000 long rows: far beyond the scratch
    b = lsa.Budget(2048, 128, 896)
    assert lsa.lsa_workspace_bytes(lsa.OP_TOPK_SELECT, huge, b) > 16 << 20
    assert call(huge, b, huge.kv_len) == 4


def test_paged_keys_rejects(L):
    """Paged indexer keys: a power-of-two block size of at least 32 whose table covers kv_len;
    scoring at decode shapes only, page keys and recall with pages inside one table block; the
    fp8-query scoring and the indexer backward take dense keys only."""
    v = ctypes.c_void_p

    def paged(T=1, bs=64, bps=None, nblk=1 << 12, tab=FAKE, Lk=4096):
        sh = _shape(B=2, T=T, Lk=Lk)
        sh.block_table, sh.block_size, sh.n_blocks = tab, bs, nblk
        sh.blocks_per_seq = -(-Lk // bs) if bps is None else bps
        return sh
    fp8 = dict(kd=lsa.KEY_FP8_E4M3, scale=FAKE)
    assert _scores_call(L, paged(bs=16), **fp8) == 2           # at least 32 rows per block
    assert _scores_call(L, paged(bs=96), **fp8) == 2           # a power of two
    assert _scores_call(L, paged(bps=4096 // 64 - 1), **fp8) == 2  # the table covers kv_len
    assert _scores_call(L, paged(nblk=0), **fp8) == 2
    assert _scores_call(L, paged(nblk=(1 << 31) // 64), **fp8) == 2
    assert _scores_call(L, paged(tab=FAKE + 1), **fp8) == 2
    assert _scores_call(L, paged(T=64), **fp8) == 4             # prefill (the tile kernel)
    sh = paged()
    # pages inside one table block: page_size <= block_size (and pages of at least 32 keys)
    assert L.lsa_page_summary(ctypes.byref(sh), 128, v(FAKE), lsa.KEY_FP8_E4M3, v(FAKE), 0, 1,
                              v(FAKE), None) == 4
    assert L.lsa_page_summary(ctypes.byref(sh), 16, v(FAKE), lsa.KEY_FP8_E4M3, v(FAKE), 0, 1,
                              v(FAKE), None) == 4
    assert L.lsa_page_summary(ctypes.byref(paged(bs=48)), 32, v(FAKE), lsa.KEY_FP8_E4M3, v(FAKE),
                              0, 1, v(FAKE), None) == 2
    assert L.lsa_page_recall(ctypes.byref(sh), lsa.Budget(256, 16, 127), 128, 8, v(FAKE), v(FAKE),
                             v(FAKE), v(FAKE), lsa.KEY_FP8_E4M3, v(FAKE), v(FAKE), v(FAKE),
                             v(FAKE), v(FAKE), 1 << 20, None) == 4
    assert L.lsa_index_scores_q8(ctypes.byref(sh), v(FAKE), v(FAKE), v(FAKE), v(FAKE),
                                 lsa.KEY_FP8_E4M3, v(FAKE), v(FAKE), None) == 4
    assert L.lsa_index_scores_backward(ctypes.byref(sh), lsa.Budget(256, 0, 0), v(FAKE), v(FAKE),
                                       v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE),
                                       None) == 4


def test_q8_entry_points_reject(L):
    """fp8 queries need fp8 keys; quantisation needs d in {64, 128}."""
    v = ctypes.c_void_p
    sh = _shape()
    assert L.lsa_index_scores_q8(ctypes.byref(sh), v(FAKE), v(FAKE), v(FAKE), v(FAKE),
                                 lsa.KEY_BF16, None, v(FAKE), None) == 3
    assert L.lsa_index_scores_q8(ctypes.byref(sh), None, v(FAKE), v(FAKE), v(FAKE),
                                 lsa.KEY_FP8_E4M3, v(FAKE), v(FAKE), None) == 1
    assert L.lsa_index_scores_q8(ctypes.byref(sh), v(FAKE + 4), v(FAKE), v(FAKE), v(FAKE),
                                 lsa.KEY_FP8_E4M3, v(FAKE), v(FAKE), None) == 2
    assert L.lsa_quantize_queries(ctypes.byref(_shape(d=96)), v(FAKE), v(FAKE), v(FAKE), None) == 4
    assert L.lsa_quantize_queries(ctypes.byref(_shape()), None, v(FAKE), v(FAKE), None) == 1


def test_sparse_attn_paged_rejects(L):
    """A paged cache is a latent cache with a power-of-two block size, a table that covers
    kv_len and a pool under 2^31 rows; the backward takes dense caches only."""
    sh = _shape(B=32)
    b = lsa.Budget(2048, 64, 960)
    v = ctypes.c_void_p

    def paged(latent=True, bs=64, bps=None, nblk=4096, tab=FAKE):
        att = (lsa.AttnShape(16, 576, 512, 1, 576, 576, 0.04) if latent
               else lsa.AttnShape(1, 128, 128, 0, 128, 128, 0.1))
        att.block_table, att.block_size, att.n_blocks = tab, bs, nblk
        att.blocks_per_seq = -(-sh.kv_len // bs) if bps is None else bps
        return att

    def call(attn, ws=None, nb=0):
        vv = FAKE if attn.latent else FAKE + 4096
        return L.lsa_sparse_attn(ctypes.byref(sh), ctypes.byref(attn), b, v(FAKE), v(FAKE), v(vv),
                                 v(FAKE), v(FAKE), None, v(ws) if ws else None, nb, None)
    assert call(paged(latent=False)) == 4                 # per-head caches are dense
    assert call(paged(bs=48)) == 2                        # a power of two
    assert call(paged(bs=1 << 21)) == 2                   # at most 2^20
    assert call(paged(bps=sh.kv_len // 64 - 1)) == 2      # the table must cover kv_len
    assert call(paged(nblk=0)) == 2
    assert call(paged(nblk=(1 << 31) // 64)) == 2         # pool rows must fit int32
    assert call(paged(tab=FAKE + 2)) == 2                 # int32 alignment
    assert call(paged()) == 5                             # valid: then the workspace is missing
    assert call(paged(bs=1, nblk=1 << 20)) == 5           # one-row blocks are blocks too
    assert L.lsa_sparse_attn_backward(ctypes.byref(sh), ctypes.byref(paged()), b, v(FAKE),
                                      v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE),
                                      v(FAKE), v(FAKE + 8192), v(FAKE + 8192), None) == 4


def test_backward_entry_points_reject(L):
    """The training-path calls validate like the forward ones: a latent cache has one gradient
    array, a non-latent one two; the indexer backward takes up to 64 heads of width 64 or 128."""
    v = ctypes.c_void_p
    sh = _shape(B=4)
    b = lsa.Budget(2048, 0, 0)
    mla = lsa.AttnShape(16, 576, 512, 1, 576, 576, 0.04)
    mha = lsa.AttnShape(1, 128, 128, 0, 128, 128, 0.1)

    def attn_call(attn, k=FAKE, vv=FAKE, dk=FAKE + 8192, dv=FAKE + 8192, lse=FAKE, dout=FAKE):
        return L.lsa_sparse_attn_backward(ctypes.byref(sh), ctypes.byref(attn), b, v(FAKE), v(k),
                                          v(vv), v(FAKE), v(FAKE), v(lse) if lse else None,
                                          v(dout) if dout else None, v(FAKE), v(dk), v(dv), None)
    assert attn_call(mla, dv=FAKE + 16384) == 2          # latent: one gradient array
    assert attn_call(mla, vv=FAKE + 4096) == 2           # latent: v must be k
    assert attn_call(mha) == 2                           # per-head: separate dK and dV
    assert attn_call(mla, lse=0) == 1                    # the forward's lse is required
    assert attn_call(mla, dout=0) == 1
    assert attn_call(mla, dk=FAKE + 2, dv=FAKE + 2) == 2  # fp32 alignment
    assert attn_call(lsa.AttnShape(8, 576, 512, 1, 576, 576, 0.04)) == 4

    def idx_call(shape, k=2048, q=FAKE, keys=FAKE, dsc=FAKE, sink=0, window=0):
        return L.lsa_index_scores_backward(ctypes.byref(shape), lsa.Budget(k, sink, window),
                                           v(q) if q else None, v(FAKE), v(keys), v(FAKE),
                                           v(dsc) if dsc else None, v(FAKE), v(FAKE), v(FAKE), None)
    assert idx_call(_shape(H=128)) == 4                  # at most 64 heads
    assert idx_call(_shape(d=96)) == 4                   # head_dim 64 or 128
    assert idx_call(_shape(), k=0) == 2
    assert idx_call(_shape(), q=0) == 1
    assert idx_call(_shape(), dsc=0) == 1
    assert idx_call(_shape(), keys=FAKE + 8) == 2        # 16-byte aligned keys
    assert idx_call(_shape(), sink=-1) == 2              # the layout: 0 <= S, W; S + W <= k
    assert idx_call(_shape(), sink=1024, window=1025) == 2
