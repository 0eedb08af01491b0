"""GPU: the workgroup shape fa_forward launches for causal grids in each
fill band, as fa_workgroup_shape names it, and the results on those grids
against the fp64 oracle.

The sweep of "Flash Attention on Android: tiled SGEMM with RenderScript",
section "The detail that breaks naive ports: tile calibration" (the best
tile differs per device and has to be measured), put causal work on other
one-group shapes than the non-causal table on MI355X, depending on how many
passes the grid makes over the workgroup slots: 2 waves with 32-key tiles
at D = 128 up to one pass, 4 waves with 32-key tiles beyond it (bf16
always, fp16 outside two to three passes and below 8192-key rows), 32-key
tiles at D = 64 beyond a pass and a quarter (fp16 at about two passes: 8
waves with 64-key tiles) and at D = 96 from three passes; one pass
of rows of 4096 keys or more runs two key groups in 8-wave workgroups (four
at D = 96; bf16 at D = 128 excepted).  Each case asserts the shape (the
expected shapes assume a 256-CU MI355X and are skipped on other devices)
and checks sampled rows (first and last rows, block edges, random rows of
the first, last and random heads) against the oracle one by one, to the
elementwise bound of gpu_helpers.parity.
"""

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_fa_amd as fa
from gpu_helpers import parity, to_device, to_numpy64
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

CODES = {"f16": 1, "bf16": 2}

# (B, H, N, D, dtype, (waves, key groups, keys per LDS tile) on 256 CUs)
CASES = [
    (1, 12, 4096, 128, "bf16", (2, 1, 32)),  # the 8-wave grid fills 3/4 of the slots
    (1, 14, 4096, 128, "bf16", (2, 1, 32)),  # up to one pass
    (1, 24, 4096, 128, "bf16", (4, 1, 32)),  # beyond
    (1, 4, 4096, 128, "bf16", (8, 4, 32)),  # at most 1/2: four key groups at D = 128
    (1, 12, 2048, 96, "bf16", (4, 1, 64)),  # 3/4 band at D = 96: one group
    (1, 48, 2048, 96, "bf16", (4, 1, 32)),  # D = 96, three passes: 32-key tiles
    (4, 32, 2048, 64, "bf16", (4, 1, 32)),  # D = 64, four passes: 32-key tiles
    (1, 28, 2048, 64, "bf16", (4, 1, 64)),  # one pass: the table's tiles
    (1, 24, 2048, 64, "bf16", (4, 1, 64)),  # three quarters at D = 64: one group
    (1, 40, 2048, 64, "f16", (4, 1, 64)),  # a pass and a quarter: 64-key tiles
    (1, 48, 2048, 64, "f16", (4, 1, 32)),  # a pass and a half: 32-key tiles
    (1, 12, 4096, 128, "f16", (8, 2, 64)),  # fp16 keeps two groups up to 3/4
    (1, 14, 4096, 128, "f16", (8, 2, 64)),  # above, up to one pass, rows of 4096+: two groups
    (1, 8, 8192, 128, "f16", (8, 2, 64)),
    (1, 8, 8192, 128, "bf16", (2, 1, 32)),  # bf16 at D = 128 keeps one group
    (1, 8, 8192, 64, "f16", (8, 2, 64)),  # D = 64, one pass of long rows: 8 waves, two groups
    (1, 8, 4096, 96, "f16", (8, 4, 32)),  # D = 96: four groups
    (1, 20, 4096, 128, "f16", (4, 1, 32)),  # between one and two passes
    (1, 32, 4096, 128, "f16", (8, 1, 64)),  # two passes: the table's shape
    (1, 12, 8192, 128, "f16", (8, 1, 64)),  # 1.5 passes of 8192-key rows: the table's shape
    (1, 12, 2048, 96, "f16", (8, 2, 64)),
    (1, 48, 2048, 96, "f16", (4, 1, 32)),
    (4, 32, 2048, 64, "f16", (4, 1, 32)),
    (1, 32, 4096, 64, "f16", (8, 1, 64)),  # fp16 D = 64 at two passes: 8 waves, 64-key tiles
    (1, 32, 4096, 64, "bf16", (4, 1, 32)),
]


def _say(msg):
    print(msg, flush=True)


def sample_rows(N, BH, rng, n=48):
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, N // 2, N - 257, N - 129, N - 65, N - 33, N - 2, N - 1]
    rows = sorted({r for r in fixed if 0 <= r < N} | set(rng.integers(0, N, n).tolist()))
    heads = sorted({0, BH - 1, *rng.integers(0, BH, 2).tolist()})
    return np.repeat(heads, len(rows)), np.tile(rows, len(heads))


@pytest.mark.parametrize("B,H,N,D,dtype,shape", CASES)
def test_causal_shape_and_parity(B, H, N, D, dtype, shape):
    got_shape = fa.fa_workgroup_shape(B, H, N, D, CODES[dtype], True)
    assert isinstance(got_shape, tuple), f"fa_workgroup_shape returned {got_shape}"
    assert got_shape[1] == fa.fa_key_groups_suggest(B, H, N, D, CODES[dtype], True)
    cus, _ = fa.fa_device_info()
    w = Workload(f"shape_b{B}h{H}n{N}d{D}_{dtype}", B, H, N, D, dtype, True, seed=81_000 + H + N + D)
    _say(f"[shape] {w.name} causal shape={got_shape} cus={cus}")
    if cus == 256:
        assert got_shape == shape, f"{w.name}: {got_shape} != {shape}"
    x = make_inputs(w)
    q, k, v = (to_device(x[n], dtype) for n in "qkv")
    o = fa.forward(q, k, v, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(H * 7 + D)
    bh, ri = sample_rows(N, B * H, rng)
    ref = oracle.rows(x["q"], x["k"], x["v"], dtype, w.scale, True, bh, ri)
    got = to_numpy64(o).reshape(B * H, N, D)[bh, ri]
    e = parity(got, ref, dtype, w.name)
    _say(f"[shape] {w.name}: {len(ri)} rows, max abs err {e['max_abs']:.3e}")


def test_shape_query_matches_key_groups_noncausal():
    """Non-causal and fp16 grids keep the table's one-group shapes."""
    for B, H, N, D in ((1, 32, 2048, 64), (1, 16, 4096, 128), (2, 8, 1000, 96), (1, 8, 2048, 128)):
        for dtype in ("f16", "bf16"):
            s = fa.fa_workgroup_shape(B, H, N, D, CODES[dtype], False)
            assert isinstance(s, tuple)
            g = fa.fa_key_groups_suggest(B, H, N, D, CODES[dtype], False)
            assert s[1] == g
            if g == 1:
                waves = 4 if D == 96 else 8
                bn = 32 if (D == 128 and dtype == "bf16") else 64
                assert s == (waves, 1, bn), (B, H, N, D, dtype, s)


@pytest.mark.parametrize("B,H,N,D,H_kv", [(1, 12, 4096, 128, 4), (1, 16, 4096, 128, 8), (4, 32, 2048, 64, 8)])
def test_bf16_causal_shapes_strided_grouped(B, H, N, D, H_kv):
    """The bf16 causal shapes above through fa_forward_strided: Q and O as
    [B, N, H, D], K and V with H_kv heads in rows padded by 8 elements.
    Sampled rows against the oracle on the expanded K/V heads."""
    from gpu_helpers import bits_to, empty_out, expand, make_gqa_inputs
    got_shape = fa.fa_workgroup_shape(B, H, N, D, fa.FA_BF16, True)
    w = Workload(f"shape_strided_b{B}h{H}kv{H_kv}n{N}d{D}_bf16", B, H, N, D, "bf16", True, seed=82_000 + H + D)
    _say(f"[shape strided] {w.name} shape={got_shape}")
    q_bits, k_bits, v_bits = make_gqa_inputs(w, H_kv)
    q = bits_to(q_bits, "bf16", "bnhd")
    k = bits_to(k_bits, "bf16", "pad", pad=8)
    v = bits_to(v_bits, "bf16", "pad", pad=8)
    o = empty_out(B, H, N, D, "bf16", "bnhd")
    fa.fa_forward_strided(q, k, v, o, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(H + D)
    bh, ri = sample_rows(N, B * H, rng, n=32)
    group = H // H_kv
    ref = oracle.rows(q_bits, expand(k_bits, group), expand(v_bits, group), "bf16", w.scale, True, bh, ri)
    got = to_numpy64(o.contiguous()).reshape(B * H, N, D)[bh, ri]
    e = parity(got, ref, "bf16", w.name)
    _say(f"[shape strided] {w.name}: {len(ri)} rows, max abs err {e['max_abs']:.3e}")
