"""Seeded input generation.

Q, K and V are drawn in that order, in C order, as float32 from numpy's
``Generator(PCG64(seed))`` and then rounded to the storage type with
round-to-nearest-even.  The result is returned as the storage type's bit
patterns (``uint16`` for fp16 and bf16, ``float32`` for fp32), so that the
oracle and the GPU library read exactly the same bits.
"""

import numpy as np

from .configs import Workload


def storage_itemsize(dtype: str) -> int:
    return {"f32": 4, "f16": 2, "bf16": 2}[dtype]


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage type (nearest, ties to even) and
    return its bit patterns.  Inputs must be finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        return u.astype(np.uint16)
    raise ValueError(f"unknown storage type {dtype!r}")


def make_inputs(w: Workload) -> dict:
    """Draw Q, K, V for a workload; returns {"q", "k", "v"} bit arrays of
    shape [B, H, N, D]."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    shape = w.shape
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    if w.qk_sigma != 1.0:
        q *= np.float32(w.qk_sigma)
        k *= np.float32(w.qk_sigma)
    if w.v_dist == "normal":
        v = rng.standard_normal(shape, dtype=np.float32)
    elif w.v_dist == "uniform":
        v = rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)
    else:
        raise ValueError(f"unknown V distribution {w.v_dist!r}")
    q, k, v = (round_to_storage(t, w.dtype) for t in (q, k, v))
    if w.uniform_head and w.N > 0:
        k[0, 0, :, :] = k[0, 0, 0, :]
    return {"q": q, "k": k, "v": v}
