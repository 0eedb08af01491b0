"""Shared helpers of the GPU tests: moving seeded storage bits to the device,
running the library, and the parity tolerances.

Tolerances (max-abs error against the fp64 oracle):
  * fp32 storage: 1e-5.
  * fp16 storage: 2e-3.
  * bf16 storage: 2e-3 plus half a bf16 ulp of the exact value, elementwise.
    Storing O in bf16 alone already costs up to half an ulp (2^-9 relative),
    which exceeds 2e-3 wherever |O| > 1; the bound therefore grants that
    unavoidable output rounding and holds the rest of the arithmetic to
    2e-3.  The literal max-abs error is reported beside it.
"""

import numpy as np
import torch

import tiled_attention_fa_amd as fa
from workloads import make_inputs

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
ABS_TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}


def to_device(bits: np.ndarray, dtype: str, device="cuda:0") -> torch.Tensor:
    a = np.ascontiguousarray(bits)
    t = torch.from_numpy(a if dtype == "f32" else a.view(np.int16))
    return t.view(TORCH_DTYPES[dtype]).to(device)


def to_numpy64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def run(x: dict, dtype: str, scale: float, causal: bool, stream=None) -> np.ndarray:
    q, k, v = (to_device(x[n], dtype) for n in "qkv")
    if stream is not None:
        stream.wait_stream(torch.cuda.current_stream())
    o = fa.forward(q, k, v, scale=scale, causal=causal, stream=stream)
    torch.cuda.synchronize()
    return to_numpy64(o)


def half_ulp(ref: np.ndarray, dtype: str) -> np.ndarray:
    """Half a unit in the last place of the storage type at each |ref|."""
    if dtype == "f32":
        mant = 24
    elif dtype == "f16":
        mant = 11
    else:
        mant = 8
    _, e = np.frexp(np.abs(ref))  # |ref| in [2^(e-1), 2^e)
    h = np.ldexp(1.0, e - 1 - mant)  # ulp/2 = 2^(e-1-(mant-1)) / 2
    return np.where(ref == 0, 0.0, h)


def parity(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> dict:
    """Assert the parity bar; returns the error figures."""
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    max_abs = float(err.max()) if err.size else 0.0
    if dtype == "bf16":
        bound = ABS_TOL[dtype] + half_ulp(ref, dtype)
        worst = float((err - bound).max()) if err.size else -1.0
        assert worst <= 0, (f"{what}: bf16 error exceeds 2e-3 + half ulp by {worst:.3e} "
                            f"(literal max abs {max_abs:.3e})")
        return {"max_abs": max_abs, "bound": "2e-3 + half a bf16 ulp, elementwise",
                "worst_over_bound": worst}
    assert max_abs <= ABS_TOL[dtype], f"{what}: max abs error {max_abs:.3e} > {ABS_TOL[dtype]}"
    return {"max_abs": max_abs, "bound": f"{ABS_TOL[dtype]:g}"}


# ---- strided layouts and grouped key/value heads

def bits_to(t_bits, dtype, layout, device="cuda:0", pad=0):
    """Dense [B, Hx, N, D] storage bits -> a device tensor viewed as
    [B, Hx, N, D] in the given memory layout: "bhnd" dense, "bnhd" with
    heads inside rows, "pad" with each row padded by `pad` elements."""
    a = np.ascontiguousarray(t_bits)
    host = torch.from_numpy(a if dtype == "f32" else a.view(np.int16)).view(TORCH_DTYPES[dtype])
    B, Hx, N, D = host.shape
    if layout == "bhnd":
        return host.to(device)
    if layout == "bnhd":
        return host.permute(0, 2, 1, 3).contiguous().to(device).permute(0, 2, 1, 3)
    if layout == "pad":
        buf = torch.zeros((B, Hx, N, D + pad), dtype=host.dtype)
        buf[..., :D] = host
        return buf.to(device)[..., :D]
    raise ValueError(layout)


def empty_out(B, H, N, D, dtype, layout, pad=0, device="cuda:0"):
    t = TORCH_DTYPES[dtype]
    if layout == "bhnd":
        return torch.empty((B, H, N, D), dtype=t, device=device)
    if layout == "bnhd":
        return torch.empty((B, N, H, D), dtype=t, device=device).permute(0, 2, 1, 3)
    return torch.empty((B, H, N, D + pad), dtype=t, device=device)[..., :D]


def make_gqa_inputs(w, H_kv):
    """Q with H heads, K and V with H_kv heads (the workload recipe drawn at
    H_kv heads for K and V)."""
    xq = make_inputs(w)
    xkv = make_inputs(w.with_(H=H_kv, seed=w.seed + 1))
    return xq["q"], xkv["k"], xkv["v"]


def expand(bits, group):
    return np.ascontiguousarray(np.repeat(bits, group, axis=1))
