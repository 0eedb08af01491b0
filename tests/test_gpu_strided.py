"""GPU parity of fa_forward_strided: tensors laid out by strides ([B, N, H, D]
as LLM stacks keep them, padded rows, mixed layouts) and grouped key/value
heads (grouped-query and multi-query attention), against the fp64 oracle,
through the C ABI.

The oracle takes dense [B, H, N, D] storage bits with one head count, so the
tests hand it the same values densely: each key/value head repeated for the
H / H_kv query heads that read it (query head h reads key/value head
h // (H / H_kv)), which is the definition of the grouped mapping.
"""

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_fa_amd as fa
import workloads
from gpu_helpers import bits_to, empty_out, expand, make_gqa_inputs, parity, to_numpy64
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def run_strided(q_bits, k_bits, v_bits, dtype, scale, causal, layouts, H, pad=8):
    lq, lk, lv, lo = layouts
    q = bits_to(q_bits, dtype, lq, pad=pad)
    k = bits_to(k_bits, dtype, lk, pad=pad)
    v = bits_to(v_bits, dtype, lv, pad=pad)
    B, _, N, D = q_bits.shape
    o = empty_out(B, H, N, D, dtype, lo, pad=pad)
    fa.fa_forward_strided(q, k, v, o, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return to_numpy64(o)


LAYOUTS = [("bnhd", "bnhd", "bnhd", "bnhd"), ("pad", "pad", "pad", "pad"), ("bhnd", "bnhd", "pad", "bnhd"),
           ("bnhd", "bhnd", "bhnd", "pad")]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("D", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_layouts_and_groups(dtype, D, causal):
    for i, (N, H, Hkv) in enumerate([(1, 2, 1), (65, 4, 2), (200, 4, 4), (129, 6, 3), (300, 8, 1)]):
        layouts = LAYOUTS[i % len(LAYOUTS)]
        w = Workload(f"str_{dtype}_d{D}_n{N}_h{H}_{Hkv}", 2 if i % 2 else 1, H, N, D, dtype, causal,
                     seed=40_000 + 31 * N + D + H + (1 if causal else 0))
        _say(f"[strided] {w.name} causal={causal} layouts={layouts}")
        q, k, v = make_gqa_inputs(w, Hkv)
        got = run_strided(q, k, v, dtype, w.scale, causal, layouts, H)
        ref = oracle.forward(q, expand(k, H // Hkv), expand(v, H // Hkv), dtype, w.scale, causal)
        parity(got, ref, dtype, f"{w.name} causal={causal} {layouts}")


def test_prefill_bnhd_bitwise_equals_dense():
    """The 1B-LLM prefill shape in the [B, N, H, D] layout: the same kernel
    with other strides, so O is bit-identical to fa_forward on dense
    tensors; sampled rows against the oracle."""
    w = workloads.get("prefill_b1h32n2048d64_f16")
    x = make_inputs(w)
    dense = [bits_to(x[n], w.dtype, "bhnd") for n in "qkv"]
    od = fa.forward(*dense, scale=w.scale)
    strided = [bits_to(x[n], w.dtype, "bnhd") for n in "qkv"]
    os_ = empty_out(w.B, w.H, w.N, w.D, w.dtype, "bnhd")
    fa.fa_forward_strided(*strided, os_, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(od, os_), "strided result differs from the dense one"
    rng = np.random.default_rng(5)
    bh = rng.integers(0, w.H, 64)
    ri = rng.integers(0, w.N, 64)
    ref = oracle.rows(x["q"], x["k"], x["v"], w.dtype, w.scale, w.causal, bh, ri)
    parity(to_numpy64(os_)[0][bh, ri], ref, w.dtype, "prefill bnhd sampled")


def test_gqa_full_size_sampled():
    """32 query heads over 8 key/value heads (4 per group) at N = 2048,
    causal bf16, [B, N, H, D] layout: sampled rows against the oracle."""
    w = workloads.get("prefill_causal_b4h32n2048d64_bf16").with_(B=1)
    q, k, v = make_gqa_inputs(w, 8)
    got = run_strided(q, k, v, w.dtype, w.scale, True, ("bnhd",) * 4, w.H)
    rng = np.random.default_rng(6)
    bh = rng.integers(0, w.H, 64)
    ri = rng.integers(0, w.N, 64)
    ref = oracle.rows(q, expand(k, 4), expand(v, 4), w.dtype, w.scale, True, bh, ri)
    parity(got[0][bh, ri], ref, w.dtype, "gqa full size sampled")


def test_output_guard_and_inputs_untouched():
    """O rows inside a padded, sentinel-filled buffer: the padding is
    untouched, the inputs are bit-identical afterwards."""
    w = Workload("str_guard", 2, 4, 130, 128, "f16", True, seed=4242)
    q_b, k_b, v_b = make_gqa_inputs(w, 2)
    q = bits_to(q_b, "f16", "bnhd")
    k = bits_to(k_b, "f16", "pad", pad=24)
    v = bits_to(v_b, "f16", "bnhd")
    before = [t.clone() for t in (q, k, v)]
    buf = torch.full((2, 4, 130, 128 + 40), 3.0, dtype=torch.float16, device="cuda:0")
    o = buf[..., 8:136]
    fa.fa_forward_strided(q, k, v, o, causal=True)
    torch.cuda.synchronize()
    assert torch.all(buf[..., :8] == 3.0) and torch.all(buf[..., 136:] == 3.0)
    for t0, t1 in zip(before, (q, k, v)):
        assert torch.equal(t0, t1)
    ref = oracle.forward(q_b, expand(k_b, 2), expand(v_b, 2), "f16", w.scale, True)
    parity(to_numpy64(o), ref, "f16", "guarded strided output")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 96, 128])
def test_full_grid_ragged_rows_guarded(dtype, D):
    """A full non-causal grid (64 heads, one key group; its waves stage O
    through LDS and store whole rows) with N = 1000, so the last row block
    of every head has rows past N: O sits in a buffer with sentinel columns
    on both sides of each row and a sentinel head after the last one.  The
    guards stay untouched and every element matches the oracle."""
    H, N = 64, 1000
    shape = fa.fa_workgroup_shape(1, H, N, D, {"f16": fa.FA_F16, "bf16": fa.FA_BF16}[dtype], False)
    assert shape[1] == 1, f"expected one key group, got {shape}"
    w = Workload(f"str_full_{dtype}_d{D}", 1, H, N, D, dtype, False, seed=4300 + D)
    x = make_inputs(w)
    q, k, v = (bits_to(x[n], dtype, "bhnd") for n in "qkv")
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    buf = torch.full((1, H + 1, N, D + 16), 3.0, dtype=tdt, device="cuda:0")
    o = buf[:, :H, :, 8:8 + D]
    _say(f"[strided] {w.name} shape={shape}")
    fa.fa_forward_strided(q, k, v, o, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.all(buf[..., :8] == 3.0) and torch.all(buf[..., 8 + D:] == 3.0), "row guards written"
    assert torch.all(buf[:, H] == 3.0), "guard head written"
    ref = oracle.forward(x["q"], x["k"], x["v"], dtype, w.scale, False)
    parity(to_numpy64(o), ref, dtype, f"{w.name} full grid, guarded")


def test_strided_rejected_calls_raise():
    q = torch.zeros((1, 4, 64, 64), dtype=torch.float16, device="cuda:0")
    kv = torch.zeros((1, 3, 64, 64), dtype=torch.float16, device="cuda:0")
    o = torch.empty_like(q)
    with pytest.raises(fa.FAError, match="DIM"):
        fa.fa_forward_strided(q, kv, kv, o)  # 4 % 3 != 0
    big = torch.zeros((1, 4, 64, 72), dtype=torch.float16, device="cuda:0")
    with pytest.raises(fa.FAError, match="ALIGN"):
        fa.fa_forward_strided(big[..., 4:68], q, q, o)  # row start not 16-byte aligned
    over = torch.empty((1, 4, 64, 64), dtype=torch.float16, device="cuda:0")
    with pytest.raises(fa.FAError, match="STRIDE"):
        fa.fa_forward_strided(q, q, q, over.as_strided((1, 4, 64, 64), (0, 0, 64, 1)))
    with pytest.raises(fa.FAError, match="ALIAS"):
        fa.fa_forward_strided(q, q, q, q)
