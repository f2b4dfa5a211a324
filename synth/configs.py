"""The five synthetic workloads of the token-sparse attention path.

Shapes follow the models the Jenga pages evaluate (Llama2-7B: 32 heads of 128;
Llama3-8B: 32 query heads sharing 8 KV heads; token blocks of 64), with the
selection rules, heavy-hitter structure and segment counts of each workload.
"""
from __future__ import annotations

import math
from dataclasses import dataclass


@dataclass(frozen=True)
class Config:
    name: str
    index: int              # 1..5, used in the seeds
    batch: int
    seq_len: int
    n_heads_q: int
    n_heads_kv: int
    head_dim: int
    block: int
    dtype: str              # "f32" or "bf16": storage and MFMA operand type of Q, K, V
    select_mode: str        # "topk" or "thresh_rel"
    select_param: float     # keep ratio (topk) or alpha (threshold = alpha * mean score)
    force_first: bool       # block 0 always kept
    unit_scale: bool        # Q, K, V ~ N(0,1) (True) or N(0,1)/sqrt(head_dim) (False)
    hh_frac: float          # fraction of key blocks that receive the heavy-hitter direction
    hh_per_head: bool       # heavy-hitter blocks drawn per KV head (True) or shared (False)
    n_layers: int = 1
    n_segments: int = 1

    @property
    def n_blocks(self) -> int:
        return self.seq_len // self.block

    @property
    def n_hh(self) -> int:
        return int(round(self.hh_frac * self.n_blocks))

    def describe(self) -> str:
        sel = (f"top-k {self.select_param}" if self.select_mode == "topk"
               else f"threshold {self.select_param}x mean")
        return (f"{self.name}: B{self.batch} S{self.seq_len} Hq{self.n_heads_q} Hkv{self.n_heads_kv} "
                f"D{self.head_dim} block{self.block} {self.dtype} {sel}"
                f"{' +block0' if self.force_first else ''} layers{self.n_layers} seg{self.n_segments}")


CONFIGS = [
    Config("c1_tiny_f32", 1, 1, 1024, 8, 8, 64, 64, "f32", "topk", 0.5, False, True, 0.0, False),
    Config("c2_llama2_4k", 2, 1, 4096, 32, 32, 128, 64, "bf16", "topk", 0.5, False, False, 0.10, False),
    Config("c3_llama2_8k_thresh", 3, 1, 8192, 32, 32, 128, 128, "bf16", "thresh_rel", 1.5, False, False,
           0.15, True),
    Config("c4_llama3_16k_gqa", 4, 1, 16384, 32, 8, 128, 64, "bf16", "topk", 0.35, True, False, 0.10, False),
    Config("c5_long_32k_4layer", 5, 1, 32768, 32, 32, 128, 128, "bf16", "topk", 0.5, False, False, 0.08,
           False, n_layers=4, n_segments=8),
]


def config_by_name(name: str) -> Config:
    for c in CONFIGS:
        if c.name == name or c.name.startswith(name + "_") or f"c{c.index}" == name:
            return c
    raise KeyError(name)


def qkv_std(cfg: Config) -> float:
    return 1.0 if cfg.unit_scale else 1.0 / math.sqrt(cfg.head_dim)
