"""GPU parity of every workgroup shape of the tile-calibration library
(libfa_tune.so, include/fa_tune.h) against the fp64 oracle: the sweep may
only choose among shapes that compute the same attention.  Ragged lengths,
both masks, all head dimensions, fp16 and bf16, through the C ABI."""

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
    for N, BH in ((200, (1, 2)), (129, (2, 1)), (1, (1, 1))):
        w = Workload(f"shape_{dtype}_d{D}_n{N}", BH[0], BH[1], N, D, dtype, causal,
                     seed=60_000 + N + D + (1 if causal else 0))
        x = make_inputs(w)
        ref = oracle.forward(x["q"], x["k"], x["v"], dtype, w.scale, causal)
        q, k, v = (to_device(x[n], dtype) for n in "qkv")
        for waves, occ, ks in tile_sweep.shapes(tune, D):
            print(f"[shape] {w.name} causal={causal} waves={waves} occ={occ} key_groups={ks}", flush=True)
            o = torch.empty_like(q)
            tile_sweep.tune_forward(tune, q, k, v, o, w.scale, causal, code, waves, occ, ks, 0)
            torch.cuda.synchronize()
            parity(to_numpy64(o), ref, dtype, f"{w.name} causal={causal} shape {waves}x{occ}x{ks}")
