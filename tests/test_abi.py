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
