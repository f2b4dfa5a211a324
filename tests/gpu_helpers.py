"""Helpers shared by the GPU parity tests: upload seeded inputs, run the HIP path through
the C ABI binding, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

BF16_TOL = 2e-2
F32_TOL = 1e-4


def say(msg: str) -> None:
    """Name the case before each GPU step (flushed, so a fault still leaves it in the log)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def tol_for(dtype: str) -> float:
    return BF16_TOL if dtype == "bf16" else F32_TOL


def to_device(x: np.ndarray, dtype: str, dev="cuda"):
    """Upload float32 values (bf16-representable for bf16) with the exact stored bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)           # exact: the values already are bfloat16 values
    return t.to(dev)


def kept_tensor(kept_list, nkb: int, dev="cuda"):
    """[B][nkb] int32 (ascending kept blocks, -1 padded) and n_kept [B] on the device."""
    import torch
    B = len(kept_list)
    arr = np.full((B, nkb), -1, dtype=np.int32)
    n = np.zeros((B,), dtype=np.int32)
    for b, kb in enumerate(kept_list):
        arr[b, :len(kb)] = kb
        n[b] = len(kb)
    return torch.from_numpy(arr).to(dev), torch.from_numpy(n).to(dev)


def max_abs(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))


def random_inputs(B, S, Hq, Hkv, D, dtype, seed, std=None):
    """Seeded N(0, std) Q/K/V plus residual and upstream gradient (float32 arrays)."""
    from synth.generate import to_bf16_bits_f32
    rng = np.random.default_rng(seed)
    std = (1.0 if dtype == "f32" else 1.0 / np.sqrt(D)) if std is None else std
    q = (rng.standard_normal((B, S, Hq, D), dtype=np.float32) * std).astype(np.float32)
    k = (rng.standard_normal((B, S, Hkv, D), dtype=np.float32) * std).astype(np.float32)
    v = (rng.standard_normal((B, S, Hkv, D), dtype=np.float32) * std).astype(np.float32)
    if dtype == "bf16":
        q, k, v = to_bf16_bits_f32(q), to_bf16_bits_f32(k), to_bf16_bits_f32(v)
    x0 = rng.standard_normal((B, S, Hq, D), dtype=np.float32)
    dout = rng.standard_normal((B, S, Hq, D), dtype=np.float32)
    return q, k, v, x0, dout
