"""Seeded synthetic inputs for the LSA token-selection path.

This module is shared by the tests, the bench and the smoke check.  It draws inputs only: it
holds none of the method's arithmetic (no scoring, selection, page keys or attention).

Recipe (every tensor has its own generator, seeded from (workload seed, tensor tag)):
  indexer q      ~ N(0,1), rounded to bf16 (round to nearest even, torch's conversion)
  head weights w ~ N(0,1) * w_std, fp32
  indexer keys   ~ N(0,1); bf16 as above, or fp8: per-token scale = max|k| / 448 (1 for an
                   all-zero row), codes = OCP e4m3fn(k / scale) (clamped to +-448 first)
  planted pages  (long-context HI workload) before quantisation: round(frac * n_pages) pages,
                   chosen uniformly without replacement, get every key shifted by
                   shift * u, u = unit vector along sum_h w[h] q[h] of that sequence's query
  attention q    ~ N(0,1) bf16;  latent cache / K / V rows ~ N(0,1) bf16
Large caches are drawn per (layer, sequence) so any piece can be regenerated alone.
"""
from __future__ import annotations

import hashlib
from typing import Dict, Optional

import torch

from .configs import Workload

_TAGS = ("index_q", "index_w", "index_k", "plant", "attn_q", "attn_kv", "attn_v", "scores",
         "idx")


def _seed(seed: int, tag: str, *sub: int) -> int:
    h = hashlib.sha256(f"{seed}:{tag}:{':'.join(map(str, sub))}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, seed: int, tag: str, *sub: int) -> torch.Generator:
    assert tag in _TAGS, tag
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, tag, *sub))
    return g


def _randn(shape, device, seed, tag, *sub) -> torch.Tensor:
    return torch.randn(shape, generator=_gen(device, seed, tag, *sub), device=device,
                       dtype=torch.float32)


def quantize_e4m3(k: torch.Tensor):
    """Per-token e4m3fn codes (uint8) and fp32 scales for fp32 keys [..., d]."""
    amax = k.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    codes = (k / scale.unsqueeze(-1)).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return codes.view(torch.uint8), scale.to(torch.float32)


def index_inputs(w: Workload, device="cpu") -> Dict[str, Optional[torch.Tensor]]:
    """q [B,n_q,H,d] bf16, w [B,n_q,H] fp32, keys [B,L,d] (bf16, or uint8 e4m3fn codes),
    scale [B,L] fp32 (fp8 keys) or None."""
    s = w.index
    B, T, L, H, d = s.batch, s.n_q, s.kv_len, s.heads, s.head_dim
    q = _randn((B, T, H, d), device, w.seed, "index_q").to(torch.bfloat16)
    wt = _randn((B, T, H), device, w.seed, "index_w") * w.w_std
    keys, scale = [], []
    for b in range(B):
        k = _randn((L, d), device, w.seed, "index_k", b)
        if w.planted_frac > 0 and w.hi is not None:
            P = w.hi.page
            n_pages = (L + P - 1) // P
            n_plant = int(round(w.planted_frac * n_pages))
            u = (wt[b, 0].double().unsqueeze(-1) * q[b, 0].double()).sum(0)
            u = (u / u.norm()).float()
            pages = torch.randperm(n_pages, generator=_gen(device, w.seed, "plant", b),
                                   device=device)[:n_plant]
            tok = (pages.unsqueeze(1) * P + torch.arange(P, device=device)).reshape(-1)
            tok = tok[tok < L]
            k[tok] += w.planted_shift * u
        if s.key_dtype == "bf16":
            keys.append(k.to(torch.bfloat16))
        else:
            c, sc = quantize_e4m3(k)
            keys.append(c)
            scale.append(sc)
        del k
    out = {"q": q, "w": wt, "keys": torch.stack(keys)}
    out["scale"] = torch.stack(scale) if scale else None
    return out


def planted_pages(w: Workload, b: int, device="cpu") -> torch.Tensor:
    """The page ids that index_inputs planted in sequence b (sorted)."""
    P = w.hi.page
    n_pages = (w.index.kv_len + P - 1) // P
    n_plant = int(round(w.planted_frac * n_pages))
    pages = torch.randperm(n_pages, generator=_gen(device, w.seed, "plant", b),
                           device=device)[:n_plant]
    return pages.sort().values


def attn_inputs(w: Workload, layer: int = 0, device="cpu") -> Dict[str, torch.Tensor]:
    """Attention inputs of one layer.  Latent (MLA) workloads: q [B,n_q,Hq,d_qk] and
    kv [B,L,d_qk] (V = first d_v columns).  Otherwise q, k [B,L,d_qk], v [B,L,d_v]."""
    s, a = w.index, w.attn
    B, T, L = s.batch, s.n_q, s.kv_len
    q = _randn((B, T, a.heads, a.d_qk), device, w.seed, "attn_q", layer).to(torch.bfloat16)
    kv = torch.empty((B, L, a.d_qk), dtype=torch.bfloat16, device=device)
    for b in range(B):
        kv[b] = _randn((L, a.d_qk), device, w.seed, "attn_kv", layer, b).to(torch.bfloat16)
    if a.latent:
        return {"q": q, "kv": kv}
    v = torch.empty((B, L, a.d_v), dtype=torch.bfloat16, device=device)
    for b in range(B):
        v[b] = _randn((L, a.d_v), device, w.seed, "attn_v", layer, b).to(torch.bfloat16)
    return {"q": q, "k": kv, "v": v}


def synthetic_scores(rows: int, n: int, seed: int, ties: str = "none", device="cpu"):
    """Score rows for selection tests.  ties: "none" (continuous N(0,1)), "zeros" (a third of the
    entries exactly +0 or -0), "coarse" (values on a grid of 17 levels: heavy exact ties),
    "const" (every entry equal), "ramp" (rising with position plus small noise: the best
    entries all sit at the end of the row), "inf" (1% of the entries +inf, 2% -inf: infinite
    scores still compete, +inf above and -inf below every finite one)."""
    x = _randn((rows, n), device, seed, "scores")
    if ties == "zeros":
        g = _gen(device, seed, "scores", 1)
        m = torch.rand((rows, n), generator=g, device=device)
        x = torch.where(m < 1 / 6, torch.zeros_like(x), x)
        x = torch.where((m >= 1 / 6) & (m < 1 / 3), -torch.zeros_like(x), x)
    elif ties == "coarse":
        x = torch.round(x * 4.0) / 4.0
    elif ties == "const":
        x = torch.full_like(x, 0.75)
    elif ties == "ramp":
        x = torch.linspace(-1.0, 1.0, n, device=device).unsqueeze(0) + 0.01 * x
    elif ties == "inf":
        g = _gen(device, seed, "scores", 2)
        m = torch.rand((rows, n), generator=g, device=device)
        x = torch.where(m < 0.01, torch.full_like(x, float("inf")), x)
        x = torch.where((m >= 0.01) & (m < 0.03), torch.full_like(x, float("-inf")), x)
    return x.contiguous()


def synthetic_index_lists(rows: int, k: int, sink: int, window: int, valid, seed: int,
                          device="cpu") -> torch.Tensor:
    """Index lists with the sink | window | dynamic layout for attention tests: for a row with
    `valid` tokens (an int or a per-row list), sink [0,S), window [V-W,V), then k-S-W distinct
    random middle tokens ascending; V <= k gives [0,V) and -1 padding."""
    g = _gen("cpu", seed, "idx")
    out = torch.full((rows, k), -1, dtype=torch.int32)
    for r in range(rows):
        V = int(valid[r] if hasattr(valid, "__len__") else valid)
        if V <= k:
            out[r, :V] = torch.arange(V, dtype=torch.int32)
            continue
        mid = torch.randperm(V - window - sink, generator=g)[: k - sink - window] + sink
        out[r, :sink] = torch.arange(sink, dtype=torch.int32)
        out[r, sink:sink + window] = torch.arange(V - window, V, dtype=torch.int32)
        out[r, sink + window:] = mid.sort().values.to(torch.int32)
    return out.to(device)
