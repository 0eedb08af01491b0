"""GPU parity at the largest sizes that run in seconds: one 65,536-token
head (row offsets of millions of elements; causal, non-causal and split
into four key ranges), 16,384-token rows on the two-key-group kernel, a
4,096-head grid (B=32, H=128), and a bf16
D=128 long head in the [B, N, H, D] layout with multi-query K/V.  Sampled
rows, including the first and last rows and rows at block edges, are checked
against the fp64 oracle one by one."""

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_fa_amd as fa
from gpu_helpers import parity, to_device, to_numpy64
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def sample_rows(N, BH, rng, n=40):
    fixed = [0, 1, 127, 128, 255, 256, N // 2, N - 257, N - 256, N - 129, N - 128, N - 2, N - 1]
    rows = sorted({r for r in fixed if 0 <= r < N} | set(rng.integers(0, N, n).tolist()))
    heads = sorted({0, BH - 1, *rng.integers(0, BH, 3).tolist()})
    bh = np.repeat(heads, len(rows))
    ri = np.tile(rows, len(heads))
    return bh, ri


@pytest.mark.parametrize("causal", [False, True])
def test_one_long_head(causal):
    w = Workload("limit_n65536", 1, 1, 65536, 64, "f16", causal, seed=9001)
    _say(f"[limits] {w.name} causal={causal}")
    x = make_inputs(w)
    q, k, v = (to_device(x[n], "f16") for n in "qkv")
    o = fa.forward(q, k, v, causal=causal)
    # 256 query blocks already fill the device (the suggestion is 1): split
    # each block's 1024 key tiles into 4 ranges anyway
    assert fa.fa_splitkv_suggest(1, 1, w.N, w.D, fa.FA_F16, causal) >= 1
    o_split, lse = fa.forward_ex(q, k, v, causal=causal, num_splits=4, lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    bh, ri = sample_rows(w.N, 1, rng)
    ref, ref_lse = oracle.rows(x["q"], x["k"], x["v"], "f16", w.scale, causal, bh, ri, return_lse=True)
    e = parity(to_numpy64(o)[0, 0][ri], ref, "f16", "N=65536")
    parity(to_numpy64(o_split)[0, 0][ri], ref, "f16", "N=65536 split")
    err_lse = float(np.abs(lse.double().cpu().numpy()[0, 0][ri] - ref_lse).max())
    assert err_lse <= 1e-3, err_lse
    _say(f"[limits] N=65536 causal={causal}: max abs err {e['max_abs']:.3e}, lse {err_lse:.3e}")


@pytest.mark.parametrize("dtype,D,H,causal", [("f16", 64, 1, False), ("bf16", 128, 2, True), ("f16", 96, 1, True)])
def test_long_rows_two_key_groups(dtype, D, H, causal):
    """16,384-token rows on grids small enough for key groups (two at D = 64,
    chains of 128 64-key tiles per group; four at D = 96 and 128, chains of
    128 32-key tiles), merged at the end.  Sampled rows against the oracle,
    with fa_forward_ex's log-sum-exp."""
    N = 16384
    want = 2 if D == 64 else 4
    assert fa.fa_key_groups_suggest(1, H, N, D, {"f16": fa.FA_F16, "bf16": fa.FA_BF16}[dtype], causal) == want
    w = Workload(f"limit_kg2_{dtype}_d{D}", 1, H, N, D, dtype, causal, seed=9010 + D)
    _say(f"[limits] {w.name} H={H} causal={causal}")
    x = make_inputs(w)
    q, k, v = (to_device(x[n], dtype) for n in "qkv")
    o, lse = fa.forward_ex(q, k, v, causal=causal, num_splits=1, lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(D)
    bh, ri = sample_rows(N, H, rng)
    ref, ref_lse = oracle.rows(x["q"], x["k"], x["v"], dtype, w.scale, causal, bh, ri, return_lse=True)
    got = to_numpy64(o).reshape(H, N, D)[bh, ri]
    e = parity(got, ref, dtype, w.name)
    err_lse = float(np.abs(lse.double().cpu().numpy().reshape(H, N)[bh, ri] - ref_lse).max())
    assert err_lse <= 1e-3, err_lse
    _say(f"[limits] {w.name}: max abs err {e['max_abs']:.3e}, lse {err_lse:.3e}")


def test_many_heads_grid():
    w = Workload("limit_b32h128", 32, 128, 64, 128, "f16", True, seed=9002)
    _say(f"[limits] {w.name}")
    x = make_inputs(w)
    q, k, v = (to_device(x[n], "f16") for n in "qkv")
    o = fa.forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    BH = w.B * w.H
    heads = sorted({0, 1, 127, 128, BH // 2, BH - 2, BH - 1, *rng.integers(0, BH, 20).tolist()})
    bh = np.repeat(heads, 8)
    ri = np.tile([0, 1, 7, 31, 32, 33, 62, 63], len(heads))
    ref = oracle.rows(x["q"], x["k"], x["v"], "f16", w.scale, True, bh, ri)
    parity(to_numpy64(o).reshape(BH, w.N, w.D)[bh, ri], ref, "f16", "4096 heads")


def test_long_bf16_d128_bnhd_mqa():
    w = Workload("limit_bnhd_mqa", 1, 8, 16384, 128, "bf16", True, seed=9003, qk_sigma=2.0)
    _say(f"[limits] {w.name}")
    xq = make_inputs(w)
    xkv = make_inputs(w.with_(H=1, seed=w.seed + 1))
    dense = lambda bits: to_device(bits, "bf16")
    q = dense(xq["q"]).permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    k = dense(xkv["k"]).permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    v = dense(xkv["v"]).permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    o = torch.empty((1, w.N, w.H, w.D), dtype=torch.bfloat16, device="cuda:0").permute(0, 2, 1, 3)
    fa.fa_forward_strided(q, k, v, o, causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    bh, ri = sample_rows(w.N, w.H, rng, n=20)
    kx = np.ascontiguousarray(np.repeat(xkv["k"], w.H, axis=1))
    vx = np.ascontiguousarray(np.repeat(xkv["v"], w.H, axis=1))
    ref = oracle.rows(xq["q"], kx, vx, "bf16", w.scale, True, bh, ri)
    parity(to_numpy64(o.contiguous()).reshape(w.H, w.N, w.D)[bh, ri], ref, "bf16", "bnhd mqa long")


def test_device_info():
    cus, clk = fa.fa_device_info()
    prop = torch.cuda.get_device_properties(torch.cuda.current_device())
    assert cus == prop.multi_processor_count
    assert 500_000 <= clk <= 5_000_000  # kHz
    assert fa.load_library().fa_device_info(None, None) == 0
