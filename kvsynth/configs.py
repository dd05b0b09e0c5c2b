"""The five workload shapes of the selection-then-decode path.

C0  tiny fp32 layer (GQA 2, d 64, n 512, window 8, budget 64 per KV head)
C1  one Llama-3-8B-shaped bf16 layer (32/8 heads, d 128, n 8192, window 32,
    budget 1024 per KV head), sink + 1 % heavy hitters + recency term
C2  32 such layers, batch 4, n 32768, per-layer bounded budgets (ZigZagKV
    page, Eq. 4 and Eq. 6) with mean 20 % and floor 5 % of the context
C3  FastGen-style head policies (local / special / global in 3:3:2) on a
    RoPE-pair-pruned cache (RAP page: 44 of 64 pairs kept, d 88), batch 8
C4  128K context with ChunkLLM-style chunk top-k (about 48 % of tokens kept)

`dataclasses.replace` makes reduced variants (shorter n, ragged tails) for the
parity tests; every generator seed includes the config id, so a reduced
variant keeps its parent's value laws.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    dtype: str                  # "fp32" or "bf16": storage type of q, K, V
    layers: int
    batch: int
    hq: int
    hkv: int
    d: int                      # stored head dim
    n: int                      # cached tokens per KV head
    w: int                      # window queries (0: no window-score step)
    mode: str                   # "topb" | "policy" | "chunk"
    d_rope: int = 0             # pre-pruning head dim (C3); 0 means d
    hh_frac: float = 0.01       # heavy-hitter fraction (C2 draws per layer)
    hh_frac_range: tuple = ()   # (lo, hi) per-layer uniform draw (C2)
    recency: int = 0            # keys at the tail that get +0.5u
    budget: int = 0             # uniform TOPB budget per KV head (C0, C1)
    avg_budget_frac: float = 0.0    # ZigZag mean budget fraction (C2)
    floor_budget_frac: float = 0.0  # ZigZag floor fraction (C2)
    kept_pairs: int = 0         # C3: RoPE pairs kept of d_rope/2
    local_window: int = 0       # C3: LOCAL heads keep the last tokens
    special_frac: float = 0.0   # C3: special-token fraction
    head_ratio: tuple = ()      # C3: (local, special, global) counts
    chunk_mean: int = 0         # C4: geometric mean chunk length
    chunk_dim: int = 0          # C4: compressed chunk-key dim
    keep_frac: float = 0.0      # C4: fraction of tokens to keep

    @property
    def G(self) -> int:
        return self.hq // self.hkv

    @property
    def d_gen(self) -> int:
        """Head dim the generator draws in (before pair pruning)."""
        return self.d_rope or self.d

    @property
    def scale(self) -> float:
        # Softmax scale 1/sqrt(head dim of the unpruned model): pair pruning
        # folds the expansion into W_q, so logits keep the original scale.
        return 1.0 / math.sqrt(self.d_gen)

    @property
    def es(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    @property
    def avg_budget(self) -> int:
        return int(math.floor(self.avg_budget_frac * self.n))

    @property
    def floor_budget(self) -> int:
        return int(math.ceil(self.floor_budget_frac * self.n))

    @property
    def n_special(self) -> int:
        return int(math.floor(self.special_frac * self.n))

    @property
    def keep_tokens(self) -> int:
        return int(math.ceil(self.keep_frac * self.n - 1e-9))

    def hh_count(self, frac: float) -> int:
        return int(math.floor(frac * self.n + 0.5))


C0 = Config(cid=0, name="c0_tiny_fp32", dtype="fp32", layers=1, batch=1, hq=4, hkv=2,
            d=64, n=512, w=8, mode="topb", budget=64)
C1 = Config(cid=1, name="c1_llama3_layer_8k", dtype="bf16", layers=1, batch=1, hq=32,
            hkv=8, d=128, n=8192, w=32, mode="topb", budget=1024, recency=256)
C2 = Config(cid=2, name="c2_zigzag_32l_32k", dtype="bf16", layers=32, batch=4, hq=32,
            hkv=8, d=128, n=32768, w=32, mode="topb", recency=256,
            hh_frac_range=(0.005, 0.04), avg_budget_frac=0.2, floor_budget_frac=0.05)
C3 = Config(cid=3, name="c3_fastgen_rap_d88_32k", dtype="bf16", layers=1, batch=8,
            hq=32, hkv=8, d=88, d_rope=128, n=32768, w=0, mode="policy", kept_pairs=44,
            local_window=2048, special_frac=0.02, head_ratio=(3, 3, 2))
C4 = Config(cid=4, name="c4_chunk_128k", dtype="bf16", layers=1, batch=1, hq=32, hkv=8,
            d=128, n=131072, w=0, mode="chunk", chunk_mean=32, chunk_dim=64,
            keep_frac=0.48)

CONFIGS = [C0, C1, C2, C3, C4]


def get_config(cid: int, **overrides) -> Config:
    cfg = CONFIGS[cid]
    return replace(cfg, **overrides) if overrides else cfg
