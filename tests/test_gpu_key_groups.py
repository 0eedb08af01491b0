"""GPU parity of the key groups of the matrix-core kernel (two, or four at
D = 96 and 128), and of the one group on the same problems, against the fp64
oracle, through the C ABI.

When B*H times the query blocks leave most of the device idle (few heads,
short rows), fa_forward, fa_forward_strided and fa_forward_ex (one key range)
run workgroups whose waves form two or four groups over the same query rows,
taking every second or fourth key tile; each group keeps its own running
maximum, denominator and accumulator, and they are merged in LDS by the
rescaling rule of the online softmax ("Android Transformer Optimization: Attention and Mobile GPU
Bottlenecks", sections "The Essence of FlashAttention: Reordering the
Computation" and "A Complete Tile Loop").  fa_key_groups_suggest names the
choice, so every case here asserts which path it runs:

  * small grids: two groups at D = 64, four at D = 96 and 128 (ragged N,
    both masks, every head dimension, fp16 and bf16; rows whose later groups
    see no key at all);
  * the same heads repeated until the grid fills the device: one group, on
    the same feature matrix (log-sum-exp output, strided layouts, grouped
    key/value heads), so that both kernels keep that coverage;
  * fp32: 16-row workgroups in four groups on small grids, and one grid per
    band of the fp32 shape rule (fa_workgroup_shape names the shape).

Tolerances as for fa_forward (gpu_helpers) and the log-sum-exp bound of the
split-KV tests (1e-3 for 16-bit storage).
"""

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_fa_amd as fa
from gpu_helpers import bits_to, empty_out, expand, make_gqa_inputs, parity, to_device, to_numpy64
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

CODES = {"f16": 1, "bf16": 2}
LSE_TOL = 1e-3
# ragged lengths, and whole tiles in odd counts (3 and 5 tiles: the second
# group's last tile lies past the range, which the loop must not take)
CASES = [(65, (1, 2)), (129, (2, 1)), (200, (1, 3)), (1000, (2, 2)), (192, (1, 2)), (320, (2, 1))]


def _say(msg):
    print(msg, flush=True)


def groups(B, H, N, D, dtype, causal):
    g = fa.fa_key_groups_suggest(B, H, N, D, CODES[dtype], causal)
    assert g in (1, 2, 4), f"fa_key_groups_suggest returned {g}"
    return g


def heads_for_one_group(N, D, dtype, causal):
    """Fewest heads (a power of two) at which B = 1 runs one key group."""
    H = 1
    while groups(1, H, N, D, dtype, causal) != 1:
        H *= 2
    return H


def tile_heads(bits, H):
    """[B, h, N, D] -> [B, H, N, D], head j a copy of head j % h."""
    h = bits.shape[1]
    reps = -(-H // h)
    return np.ascontiguousarray(np.tile(bits, (1, reps, 1, 1))[:, :H])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_two_groups_small_grid(dtype, D, causal):
    for N, (B, H) in CASES:
        want = 2 if D == 64 else 4
        assert groups(B, H, N, D, dtype, causal) == want, f"N={N} B={B} H={H}: expected {want} key groups"
        w = Workload(f"kg2_{dtype}_d{D}_n{N}", B, H, N, D, dtype, causal,
                     seed=70_000 + 17 * N + D + (1 if causal else 0))
        _say(f"[key groups {want}] {w.name} causal={causal} B={B} H={H}")
        x = make_inputs(w)
        ref, ref_lse = oracle.forward(x["q"], x["k"], x["v"], dtype, w.scale, causal, return_lse=True)
        q, k, v = (to_device(x[n], dtype) for n in "qkv")
        o = fa.forward(q, k, v, scale=w.scale, causal=causal)
        torch.cuda.synchronize()
        parity(to_numpy64(o), ref, dtype, f"{w.name} causal={causal} fa_forward")
        o2, lse = fa.forward_ex(q, k, v, scale=w.scale, causal=causal, num_splits=1, lse=True)
        torch.cuda.synchronize()
        parity(to_numpy64(o2), ref, dtype, f"{w.name} causal={causal} fa_forward_ex")
        err = float(np.abs(lse.double().cpu().numpy() - ref_lse).max())
        assert err <= LSE_TOL, f"{w.name} causal={causal}: lse error {err:.3e}"


def test_one_tile_rows_take_one_group():
    """N <= 64: a single key tile, nothing to split."""
    for N in (1, 17, 64):
        assert groups(1, 1, N, 64, "f16", False) == 1
        assert groups(1, 1, N, 128, "bf16", True) == 1
    assert groups(1, 1, 65, 64, "f16", False) == 2


def test_full_grids_take_one_group():
    """The benchmark workloads fill the device: one group."""
    assert groups(1, 32, 2048, 64, "f16", False) == 1
    assert groups(4, 32, 2048, 64, "bf16", True) == 1
    assert groups(1, 16, 8192, 128, "f16", True) == 1
    cus, _ = fa.fa_device_info()
    # the ragged workload: 16 heads x 4 blocks of 256 rows, a quarter of the
    # CUs: four groups at D = 96
    assert groups(2, 8, 1000, 96, "f16", False) == (4 if 4 * 16 * 4 <= cus else 1)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_one_group_same_problems(dtype, D, causal):
    """The small cases with their heads repeated until the grid takes one
    group; every head checked against the oracle of the head it copies."""
    for N, (B, h) in CASES[:3]:
        H = heads_for_one_group(N, D, dtype, causal)
        assert groups(B, H, N, D, dtype, causal) == 1
        w = Workload(f"kg1_{dtype}_d{D}_n{N}", B, h, N, D, dtype, causal,
                     seed=71_000 + 17 * N + D + (1 if causal else 0))
        _say(f"[key groups 1] {w.name} causal={causal} B={B} H={H} (copies of {h} heads)")
        x = make_inputs(w)
        ref, ref_lse = oracle.forward(x["q"], x["k"], x["v"], dtype, w.scale, causal, return_lse=True)
        q, k, v = (to_device(tile_heads(x[n], H), dtype) for n in "qkv")
        o, lse = fa.forward_ex(q, k, v, scale=w.scale, causal=causal, num_splits=1, lse=True)
        torch.cuda.synchronize()
        parity(to_numpy64(o), tile_heads(ref, H), dtype, f"{w.name} causal={causal} one group")
        err = float(np.abs(lse.double().cpu().numpy() - tile_heads(ref_lse[..., None], H)[..., 0]).max())
        assert err <= LSE_TOL, f"{w.name} causal={causal}: lse error {err:.3e}"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 96, 128])
def test_two_groups_causal_partial_grids(dtype, D):
    """Causal grids between half and three quarters of the slots run two
    groups (8-wave workgroups at D = 96 and 128), except bf16 at D = 96 and
    128, which runs one group there (2 waves with 32-key tiles at D = 128);
    non-causal ones of the same size run one.  Three heads of each are
    checked against the oracle."""
    cus, _ = fa.fa_device_info()
    block, per_cu = {64: (128, 2), 96: (128, 1), 128: (256, 1)}[D]
    N = 2048
    blocks = N // block
    slots = cus * per_cu
    H = (5 * slots // 8) // blocks  # ~5/8 of the slots
    assert 2 * H * blocks > slots and 4 * H * blocks <= 3 * slots
    want = 1 if (dtype == "bf16" and D != 64) else 2
    assert groups(1, H, N, D, dtype, True) == want
    assert groups(1, H, N, D, dtype, False) == 1
    w = Workload(f"kgp_{dtype}_d{D}", 1, H, N, D, dtype, True, seed=73_000 + D)
    _say(f"[key groups {want}, partial causal grid] {w.name} H={H}")
    x = make_inputs(w)
    q, k, v = (to_device(x[n], dtype) for n in "qkv")
    o = fa.forward(q, k, v, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    got = to_numpy64(o)
    for h in (0, H // 2, H - 1):
        ref = oracle.forward(x["q"][:, h:h + 1], x["k"][:, h:h + 1], x["v"][:, h:h + 1], dtype, w.scale, True)
        parity(got[:, h:h + 1], ref, dtype, f"{w.name} head {h}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 96, 128])
def test_noncausal_quarter_to_half_grids(dtype, D):
    """Non-causal grids whose 256-row blocks cover between a quarter and half
    of the CUs: two groups in 8-wave workgroups at D = 64 and 128, one group
    at D = 96.  Three heads checked against the oracle."""
    cus, _ = fa.fa_device_info()
    N = 2048
    H = (3 * cus // 8) // (N // 256)  # ~3/8 of the CUs
    assert 4 * H * (N // 256) > cus and 2 * H * (N // 256) <= cus
    want = 1 if D == 96 else 2
    assert groups(1, H, N, D, dtype, False) == want
    w = Workload(f"kgq_{dtype}_d{D}", 1, H, N, D, dtype, False, seed=74_000 + D)
    _say(f"[key groups {want}, quarter-to-half grid] {w.name} H={H}")
    x = make_inputs(w)
    q, k, v = (to_device(x[n], dtype) for n in "qkv")
    o = fa.forward(q, k, v, scale=w.scale, causal=False)
    torch.cuda.synchronize()
    got = to_numpy64(o)
    for h in (0, H // 2, H - 1):
        ref = oracle.forward(x["q"][:, h:h + 1], x["k"][:, h:h + 1], x["v"][:, h:h + 1], dtype, w.scale, False)
        parity(got[:, h:h + 1], ref, dtype, f"{w.name} head {h}")


LAYOUTS = [("bnhd", "bnhd", "bnhd", "bnhd"), ("pad", "bhnd", "pad", "bnhd")]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_strided_gqa_both_paths(dtype, D, causal):
    """Strided layouts with grouped key/value heads: on a small grid (two
    key groups at D = 64, four at D = 128) and with the query heads repeated
    to fill the device (one group; the key/value heads repeated alike keep
    each query head's pairing)."""
    N, H, Hkv = 200, 4, 2
    w = Workload(f"kgs_{dtype}_d{D}", 1, H, N, D, dtype, causal, seed=72_000 + D + (1 if causal else 0))
    q, k, v = make_gqa_inputs(w, Hkv)
    ref = oracle.forward(q, expand(k, H // Hkv), expand(v, H // Hkv), dtype, w.scale, causal)
    H1 = max(heads_for_one_group(N, D, dtype, causal), H)
    for Hq, want in ((H, 2 if D == 64 else 4), (H1, 1)):
        assert groups(1, Hq, N, D, dtype, causal) == want
        rep = Hq // H
        qb, kb, vb = tile_heads(q, Hq), tile_heads(k, Hkv * rep), tile_heads(v, Hkv * rep)
        for layouts in LAYOUTS:
            _say(f"[key groups {want}] {w.name} causal={causal} H={Hq} H_kv={Hkv * rep} {layouts}")
            lq, lk, lv, lo = layouts
            o = empty_out(1, Hq, N, D, dtype, lo, pad=8)
            fa.fa_forward_strided(bits_to(qb, dtype, lq, pad=8), bits_to(kb, dtype, lk, pad=8),
                                  bits_to(vb, dtype, lv, pad=8), o, scale=w.scale, causal=causal)
            torch.cuda.synchronize()
            parity(to_numpy64(o), tile_heads(ref, Hq), dtype, f"{w.name} causal={causal} H={Hq} {layouts}")


def _f32_check(B, H, N, D, causal, label):
    w = Workload(f"kg_f32_b{B}h{H}n{N}d{D}", B, H, N, D, "f32", causal, seed=73_000 + H + N + D)
    x = make_inputs(w)
    ref, ref_lse = oracle.forward(x["q"], x["k"], x["v"], "f32", w.scale, causal, return_lse=True)
    q, k, v = (to_device(x[n], "f32") for n in "qkv")
    _say(f"[fp32 {label}] {w.name} causal={causal}")
    o = fa.forward(q, k, v, scale=w.scale, causal=causal)
    o2, lse = fa.forward_ex(q, k, v, scale=w.scale, causal=causal, num_splits=1, lse=True)
    torch.cuda.synchronize()
    parity(to_numpy64(o), ref, "f32", f"{w.name} causal={causal}")
    parity(to_numpy64(o2), ref, "f32", f"{w.name} causal={causal} (ex)")
    err = float(np.abs(lse.double().cpu().numpy() - ref_lse).max())
    assert err <= LSE_TOL, f"{w.name} causal={causal}: lse error {err:.3e}"


@pytest.mark.parametrize("N", [64, 255, 256, 1000])
@pytest.mark.parametrize("D", [64, 96, 128])
def test_f32_small_grid_and_parity(N, D):
    """fp32 on a grid far smaller than the device (3 heads): 16-row
    workgroups in four key groups (some of whose groups see no key at N =
    64), against the oracle with fa_forward (dense) and fa_forward_ex
    (log-sum-exp), causal and not."""
    cus, _ = fa.fa_device_info()
    if 3 * ((N + 63) // 64) < cus:
        assert fa.fa_key_groups_suggest(1, 3, N, D, fa.FA_F32, False) == 4
        assert fa.fa_workgroup_shape(1, 3, N, D, fa.FA_F32, False) == (4, 4, 32)
    for causal in (False, True):
        _f32_check(1, 3, N, D, causal, "16r x4")


# (H, N, D, causal) -> (waves, key groups) on a 256-CU device: one grid per
# band of the fp32 shape rule
F32_BANDS = [
    (8, 1024, 64, False, (8, 4)),    # half the CUs: a tie, 32 rows in four groups
    (16, 1024, 96, True, (8, 4)),    # causal, one 64-row block per CU
    (16, 2048, 64, True, (4, 2)),    # causal, two per CU, D = 64: 32 rows in two groups
    (32, 1024, 128, True, (8, 2)),   # causal, two per CU, D = 128: 64 rows in two groups
    (16, 1024, 64, False, (8, 2)),   # full grid: 64 rows in two groups
    (32, 1024, 128, False, (4, 1)),  # non-causal D = 128, two per CU: one group
]


@pytest.mark.parametrize("H,N,D,causal,want", F32_BANDS)
def test_f32_shape_bands_and_parity(H, N, D, causal, want):
    """The fp32 shape rule on a 256-CU device (the MI355X), one grid per
    band, and every output element of each against the oracle."""
    cus, _ = fa.fa_device_info()
    if cus == 256:
        waves, groups, bn = fa.fa_workgroup_shape(1, H, N, D, fa.FA_F32, causal)
        assert (waves, groups, bn) == (*want, 32)
        assert fa.fa_key_groups_suggest(1, H, N, D, fa.FA_F32, causal) == want[1]
    _f32_check(1, H, N, D, causal, f"{want[0]} waves x{want[1]}")
