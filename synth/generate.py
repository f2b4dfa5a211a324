"""Seeded synthetic Q/K/V, residual stream and upstream gradient for each workload.

Recipe (per layer l of workload c):
  rng = numpy.random.default_rng(1000*c + l)
  Q [B,S,Hq,D], then K [B,S,Hkv,D], then V [B,S,Hkv,D] ~ N(0,1) float32, times the
  workload's std (1 or 1/sqrt(D));
  u = rng.standard_normal(D) (float64), u /= |u|: one shared unit direction;
  heavy-hitter key blocks: rng.choice(nKB, n_hh, replace=False), once for all KV heads
  or once per KV head (h = 0..Hkv-1 in order); 3*u is added to every K row of those blocks.
  Residual and upstream gradient: rng2 = default_rng(1000*c + 500) draws X0 then dOut,
  both [B,S,Hq,D] ~ N(0,1) float32 (once per workload, shared by all layers).
bf16 workloads round Q, K, V to bfloat16 (round to nearest even); the rounded values are
returned as float32 so that every consumer sees the same stored bits.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np

from .configs import Config, qkv_std


def to_bf16_bits_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); return them as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    out = rounded.view(np.float32).copy()
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.float32("nan")
    return out


def bf16_bits_u16(x_bf16_valued: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are exactly bfloat16-representable."""
    bits = np.ascontiguousarray(x_bf16_valued, dtype=np.float32).view(np.uint32)
    return (bits >> np.uint32(16)).astype(np.uint16)


@dataclass
class LayerInputs:
    q: np.ndarray            # [B,S,Hq,D] float32 (bf16-valued for bf16 workloads)
    k: np.ndarray            # [B,S,Hkv,D]
    v: np.ndarray            # [B,S,Hkv,D]
    hh_blocks: np.ndarray    # [n_hh] shared, or [Hkv, n_hh] per head


@dataclass
class Inputs:
    cfg: Config
    layers: List[LayerInputs]
    x0: np.ndarray           # [B,S,Hq,D] float32 residual stream entering layer 0
    dout: np.ndarray         # [B,S,Hq,D] float32 gradient of the loss w.r.t. the final residual


def make_layer(cfg: Config, layer: int = 0, seq_len: Optional[int] = None,
               round_bf16: bool = True) -> LayerInputs:
    """One layer's Q/K/V.  round_bf16=False leaves bf16 workloads in float32 for a caller that
    rounds to bfloat16 itself (torch's cast rounds to nearest even, giving the same bits)."""
    S = cfg.seq_len if seq_len is None else seq_len
    B, Hq, Hkv, D, blk = cfg.batch, cfg.n_heads_q, cfg.n_heads_kv, cfg.head_dim, cfg.block
    nkb = S // blk
    rng = np.random.default_rng(1000 * cfg.index + layer)
    std = np.float32(qkv_std(cfg))
    q = rng.standard_normal((B, S, Hq, D), dtype=np.float32)
    k = rng.standard_normal((B, S, Hkv, D), dtype=np.float32)
    v = rng.standard_normal((B, S, Hkv, D), dtype=np.float32)
    if std != 1:
        q *= std
        k *= std
        v *= std
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    shift = (3.0 * u).astype(np.float32)
    n_hh = int(round(cfg.hh_frac * nkb))
    if n_hh > 0:
        if cfg.hh_per_head:
            hh = np.stack([rng.choice(nkb, n_hh, replace=False) for _ in range(Hkv)])
            for g in range(Hkv):
                for n in hh[g]:
                    k[:, n * blk:(n + 1) * blk, g, :] += shift
        else:
            hh = rng.choice(nkb, n_hh, replace=False)
            for n in hh:
                k[:, n * blk:(n + 1) * blk, :, :] += shift
    else:
        hh = np.zeros((0,), dtype=np.int64)
    if cfg.dtype == "bf16" and round_bf16:
        q, k, v = to_bf16_bits_f32(q), to_bf16_bits_f32(k), to_bf16_bits_f32(v)
    return LayerInputs(q=q, k=k, v=v, hh_blocks=np.asarray(hh))


def make_resid_dout(cfg: Config, seq_len: Optional[int] = None):
    S = cfg.seq_len if seq_len is None else seq_len
    rng2 = np.random.default_rng(1000 * cfg.index + 500)
    shape = (cfg.batch, S, cfg.n_heads_q, cfg.head_dim)
    x0 = rng2.standard_normal(shape, dtype=np.float32)
    dout = rng2.standard_normal(shape, dtype=np.float32)
    return x0, dout


def make_inputs(cfg: Config, seq_len: Optional[int] = None, n_layers: Optional[int] = None) -> Inputs:
    L = cfg.n_layers if n_layers is None else n_layers
    layers = [make_layer(cfg, l, seq_len) for l in range(L)]
    x0, dout = make_resid_dout(cfg, seq_len)
    return Inputs(cfg=cfg, layers=layers, x0=x0, dout=dout)


def random_kept_blocks(n_blocks: int, n_keep: int, seed: int) -> np.ndarray:
    """A seeded, sorted, scattered kept-block set (exercises index resolution)."""
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(n_blocks, n_keep, replace=False)).astype(np.int32)
