"""The five seeded synthetic workloads of the LSA token-selection path, and their shapes.

Shapes only: nothing here computes any part of the method.  Each workload has a name that says
what it is; the sizes follow the decode / prefill / long-context settings in which the
LongCat Sparse Attention pages discuss the method (1M-token native context and the >= 256K
break-even of Hierarchical Indexing on the paper summary page; k = 2048 selections per query in
the Baidu Cloud Lightning Indexer article, "Dynamic Token Selector").
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional


@dataclass(frozen=True)
class IndexShape:
    batch: int
    n_q: int          # queries per sequence
    kv_len: int       # L, keys in the cache
    q_pos0: int       # absolute position of query 0; query i sees keys [0, min(L, q_pos0+i+1))
    heads: int        # indexer heads H
    head_dim: int     # indexer dim d
    key_dtype: str    # "bf16" or "fp8" (OCP e4m3fn + per-token fp32 scale)


@dataclass(frozen=True)
class Budget:
    k: int
    sink: int
    window: int

    @property
    def dynamic(self) -> int:
        return self.k - self.sink - self.window


@dataclass(frozen=True)
class AttnShape:
    heads: int        # query heads Hq
    d_qk: int
    d_v: int
    latent: bool      # True: MLA latent cache, V = first d_v columns of the K rows
    scale: float      # softmax temperature tau


@dataclass(frozen=True)
class HiParams:
    page: int         # P tokens per page
    m_pages: int      # M pages recalled per query


@dataclass(frozen=True)
class Workload:
    name: str
    index: IndexShape
    budget: Budget
    attn: AttnShape
    seed: int
    hi: Optional[HiParams] = None
    layers: int = 1               # consecutive attention layers sharing one index list
    planted_frac: float = 0.0     # fraction of pages given a high-score cluster
    planted_shift: float = 0.5
    w_std: float = 0.5            # head weights ~ N(0, w_std^2)


MLA_576 = AttnShape(heads=16, d_qk=576, d_v=512, latent=True, scale=1.0 / math.sqrt(576))

TINY_PREFILL_4K = Workload(
    name="tiny_prefill_4k",
    index=IndexShape(batch=1, n_q=4096, kv_len=4096, q_pos0=0, heads=4, head_dim=64,
                     key_dtype="bf16"),
    budget=Budget(k=256, sink=16, window=112),
    attn=AttnShape(heads=1, d_qk=128, d_v=128, latent=False, scale=1.0 / math.sqrt(128)),
    seed=0,
)

DECODE_128K = Workload(
    name="decode_b32_128k_flat",
    index=IndexShape(batch=32, n_q=1, kv_len=131072, q_pos0=131071, heads=64, head_dim=128,
                     key_dtype="fp8"),
    budget=Budget(k=2048, sink=64, window=960),
    attn=MLA_576,
    seed=1,
)

PREFILL_8K_AT_128K = Workload(
    name="prefill_chunk8k_128k_flat",
    index=IndexShape(batch=1, n_q=8192, kv_len=131072, q_pos0=131072 - 8192, heads=64,
                     head_dim=128, key_dtype="bf16"),
    budget=Budget(k=2048, sink=128, window=896),
    attn=MLA_576,
    seed=2,
)

DECODE_1M_HI = Workload(
    name="decode_b4_1m_hi",
    index=IndexShape(batch=4, n_q=1, kv_len=1 << 20, q_pos0=(1 << 20) - 1, heads=64,
                     head_dim=128, key_dtype="fp8"),
    budget=Budget(k=2048, sink=128, window=896),
    attn=MLA_576,
    seed=3,
    hi=HiParams(page=64, m_pages=256),
    planted_frac=0.01,
)

DECODE_256K_HI_CLI = Workload(
    name="decode_b8_256k_hi_cli4",
    index=IndexShape(batch=8, n_q=1, kv_len=1 << 18, q_pos0=(1 << 18) - 1, heads=64,
                     head_dim=128, key_dtype="fp8"),
    budget=Budget(k=2048, sink=128, window=896),
    attn=MLA_576,
    seed=4,
    hi=HiParams(page=64, m_pages=128),
    layers=4,
)

WORKLOADS = {w.name: w for w in (TINY_PREFILL_4K, DECODE_128K, PREFILL_8K_AT_128K,
                                 DECODE_1M_HI, DECODE_256K_HI_CLI)}


def shrink(w: Workload, **index_changes) -> Workload:
    """The same workload with some index-shape fields changed (for small parity cases)."""
    return replace(w, index=replace(w.index, **index_changes))
