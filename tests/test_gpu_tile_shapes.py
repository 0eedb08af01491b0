"""GPU parity of every workgroup shape of the tile-calibration library
(libfa_tune.so, include/fa_tune.h), the matrix-core kernel's and the fp32
kernel's, against the fp64 oracle: the sweep may only choose among shapes
that compute the same attention.  Ragged lengths (a partial last tile of
every key-tile size, and a 128-key tile whose second half holds no key),
both masks, all head dimensions, fp16, bf16 and fp32, through the C ABI."""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import parity, to_device, to_numpy64
from tiled_attention_fa_amd import tile_sweep
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tune():
    return tile_sweep.load_tune()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_every_shape_matches_oracle(tune, dtype, D, causal):
    code = 1 if dtype == "f16" else 2
    for N, BH in ((200, (1, 2)), (129, (2, 1)), (1, (1, 1)), (383, (1, 1))):
        w = Workload(f"shape_{dtype}_d{D}_n{N}", BH[0], BH[1], N, D, dtype, causal,
                     seed=60_000 + N + D + (1 if causal else 0))
        x = make_inputs(w)
        ref = oracle.forward(x["q"], x["k"], x["v"], dtype, w.scale, causal)
        q, k, v = (to_device(x[n], dtype) for n in "qkv")
        for waves, occ, ks, bn in tile_sweep.shapes(tune, D):
            print(f"[shape] {w.name} causal={causal} waves={waves} occ={occ} key_groups={ks} block_n={bn}",
                  flush=True)
            o = torch.empty_like(q)
            tile_sweep.tune_forward(tune, q, k, v, o, w.scale, causal, code, waves, occ, ks, bn, 0)
            torch.cuda.synchronize()
            parity(to_numpy64(o), ref, dtype, f"{w.name} causal={causal} shape {waves}x{occ}x{ks} bn{bn}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_split_merge_closed_forms(tune, dtype):
    """The split-KV merge kernel on partials with known results: equal
    log-sum-exps average the ranges; a range with lse = -inf has weight 0;
    lse_r = ln 3 and ln 1 weigh the ranges 3:1 and give lse = ln 4; a row that
    no range saw (every lse_r = -inf) is written as 0 with lse = -inf."""
    import math
    rows, D, S = 4, 64, 3
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(17)
    po = torch.from_numpy(rng.uniform(-1, 1, (S, rows, D)).astype(np.float32)).to(dev)
    ninf = float("-inf")
    lse_in = np.array([[0.5, ninf, math.log(3.0), ninf],
                       [0.5, 1.25, 0.0, ninf],
                       [0.5, ninf, ninf, ninf]], dtype=np.float32)
    pl = torch.from_numpy(lse_in).to(dev)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    code = {"f32": 0, "f16": 1, "bf16": 2}[dtype]
    o = torch.full((rows, D), 7.0, dtype=tdt, device=dev)
    lse = torch.full((rows,), 7.0, dtype=torch.float32, device=dev)
    st = tune.fa_tune_split_merge(po.data_ptr(), pl.data_ptr(), o.data_ptr(), lse.data_ptr(), rows, D, S,
                                  code, None)
    assert st == 0
    torch.cuda.synchronize()
    P = po.double().cpu().numpy()
    expect = np.stack([P[:, 0].mean(axis=0), P[1, 1], (3 * P[0, 2] + P[1, 2]) / 4, np.zeros(D)])
    expect_lse = np.array([0.5 + math.log(3.0), 1.25, math.log(4.0), ninf])
    got = o.double().cpu().numpy()
    tol = {"f32": 1e-6, "f16": 2e-3, "bf16": 8e-3}[dtype]
    assert np.abs(got - expect).max() <= tol, np.abs(got - expect).max()
    gl = lse.double().cpu().numpy()
    assert gl[3] == ninf and np.all(got[3] == 0.0)
    assert np.abs(gl[:3] - expect_lse[:3]).max() <= 2e-6


@pytest.mark.parametrize("D", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_every_f32_shape_matches_oracle(tune, D, causal):
    """The fp32 kernel at every shape of the sweep (rows per workgroup, key
    groups): ragged lengths (a partial last 16-key tile, fewer tiles than
    key groups), both masks."""
    for N, BH in ((200, (1, 2)), (129, (2, 1)), (1, (1, 1)), (40, (1, 1))):
        w = Workload(f"shape_f32_d{D}_n{N}", BH[0], BH[1], N, D, "f32", causal,
                     seed=61_000 + N + D + (1 if causal else 0))
        x = make_inputs(w)
        ref = oracle.forward(x["q"], x["k"], x["v"], "f32", w.scale, causal)
        q, k, v = (to_device(x[n], "f32") for n in "qkv")
        for shape in tile_sweep.f32_shapes(tune, D):
            label = tile_sweep.f32_label(shape)
            print(f"[shape] {w.name} causal={causal} fp32 {label}", flush=True)
            o = torch.empty_like(q)
            tile_sweep.tune_forward_f32(tune, q, k, v, o, w.scale, causal, shape, 0)
            torch.cuda.synchronize()
            parity(to_numpy64(o), ref, "f32", f"{w.name} causal={causal} fp32 {label}")
