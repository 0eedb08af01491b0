"""GPU parity of fa_forward_ex: the log-sum-exp side output and split-KV
(key ranges per query block, merged by the online-softmax rescaling rule of
"Android Transformer Optimization: Attention and Mobile GPU Bottlenecks",
sections "The Essence of FlashAttention: Reordering the Computation" and "A
Complete Tile Loop"), against the fp64 oracle, through the C ABI.

Tolerances: O as for fa_forward.  The log-sum-exp: 2e-5 for fp32 storage;
1e-3 for fp16 and bf16.  For fp16 the kernel's denominator is the sum of the
probabilities as rounded to fp16 (so that the weights applied to V sum to
one), which moves ln l by up to the fp16 unit roundoff 2^-11 ~ 4.9e-4; the
fp32 score sums over D <= 128 products add at most a few 1e-5 on these
inputs.
"""

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_fa_amd as fa
import workloads
from gpu_helpers import parity, to_device, to_numpy64
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

LSE_TOL = {"f32": 2e-5, "f16": 1e-3, "bf16": 1e-3}


def _say(msg):
    print(msg, flush=True)


def run_ex(x, dtype, scale, causal, splits, want_lse=True):
    q, k, v = (to_device(x[n], dtype) for n in "qkv")
    res = fa.forward_ex(q, k, v, scale=scale, causal=causal, num_splits=splits, lse=want_lse)
    torch.cuda.synchronize()
    if want_lse:
        o, lse = res
        return to_numpy64(o), lse.double().cpu().numpy()
    return to_numpy64(res), None


def lse_parity(got, ref, dtype, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite lse"
    err = float(np.abs(got - ref).max()) if got.size else 0.0
    assert err <= LSE_TOL[dtype], f"{what}: lse max abs error {err:.3e} > {LSE_TOL[dtype]}"
    return err


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("D", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_lse_and_splits_sweep(dtype, D, causal):
    """Every split count from 1 (LSE only) to more ranges than key tiles
    (empty ranges), on ragged lengths and on whole tiles cut unevenly."""
    for i, (N, S) in enumerate([(1, 1), (65, 1), (200, 2), (129, 3), (300, 5), (65, 16), (1000, 4),
                                (192, 2), (256, 3)]):
        BH = (1, 1) if i % 2 == 0 else (1, 3)
        w = Workload(f"ex_{dtype}_d{D}_n{N}_s{S}", BH[0], BH[1], N, D, dtype, causal,
                     seed=30_000 + 53 * N + D + 7 * S + (1 if causal else 0))
        _say(f"[ex] {w.name} causal={causal} BH={BH} splits={S}")
        x = make_inputs(w)
        o, lse = run_ex(x, dtype, w.scale, causal, S)
        ref_o, ref_lse = oracle.forward(x["q"], x["k"], x["v"], dtype, w.scale, causal, return_lse=True)
        parity(o, ref_o, dtype, f"{w.name} causal={causal} O")
        lse_parity(lse, ref_lse, dtype, f"{w.name} causal={causal}")


def test_ragged_workload_lse_and_two_ranges():
    """The ragged N=1000 D=96 workload with two key ranges: every element
    against the oracle, and the uniform head's log-sum-exp = s + ln N.  (Its
    rows are too short for splitting to pay: the suggestion is 1.)"""
    w = workloads.get("ragged_b2h8n1000d96_f16_uniform_head")
    S = fa.fa_splitkv_suggest(w.B, w.H, w.N, w.D, fa.FA_F16, w.causal)
    _say(f"[ex] {w.name}: suggested splits {S}")
    assert S == 1
    x = make_inputs(w)
    o, lse = run_ex(x, w.dtype, w.scale, w.causal, 2)
    ref_o, ref_lse = oracle.forward(x["q"], x["k"], x["v"], w.dtype, w.scale, w.causal, return_lse=True)
    e = parity(o, ref_o, w.dtype, "ragged split auto O")
    el = lse_parity(lse, ref_lse, w.dtype, "ragged split auto")
    qd = oracle.decode(x["q"][0, 0], "f16")
    kd = oracle.decode(x["k"][0, 0, 0], "f16")
    uni = w.scale * qd @ kd + np.log(w.N)
    assert np.abs(lse[0, 0] - uni).max() <= LSE_TOL["f16"]
    _say(f"[ex] ragged two ranges: O err {e['max_abs']:.3e}, lse err {el:.3e}")


def test_few_heads_long_rows_split_auto():
    """Two heads of the long head-dim-128 causal prefill: 64 workgroups
    without splits; the suggestion splits them, and sampled rows (O, lse)
    match the oracle."""
    w = workloads.get("long_prefill_causal_b1h16n8192d128_f16_sigma3").with_(H=2)
    S = fa.fa_splitkv_suggest(w.B, w.H, w.N, w.D, fa.FA_F16, w.causal)
    _say(f"[ex] {w.name} H=2: suggested splits {S}")
    assert 2 <= S <= 16
    x = make_inputs(w)
    o, lse = run_ex(x, w.dtype, w.scale, w.causal, 0)
    rng = np.random.default_rng(17)
    bh = np.repeat([0, 1], 40)
    ri = np.concatenate([rng.integers(0, w.N, 36), [0, 1, w.N - 2, w.N - 1]] * 2)
    ref_o, ref_lse = oracle.rows(x["q"], x["k"], x["v"], w.dtype, w.scale, w.causal, bh, ri,
                                 return_lse=True)
    parity(o.reshape(2, w.N, w.D)[bh, ri], ref_o, w.dtype, "few heads split auto O")
    lse_parity(lse.reshape(2, w.N)[bh, ri], ref_lse, w.dtype, "few heads split auto")


@pytest.mark.parametrize("N,D,causal,want", [(1024, 128, False, 1), (4096, 64, False, 4),
                                             (2048, 64, True, 4)])
def test_f32_split_suggestion_against_key_groups(N, D, causal, want):
    """fp32, one head: the suggestion keeps one range where the 16-row
    four-group workgroups leave less key-tile work per SIMD than the ranges
    (N = 1024, D = 128), and splits where the two tie (on a 256-CU device);
    either way every element of O and the log-sum-exp match the oracle."""
    cus, _ = fa.fa_device_info()
    S = fa.fa_splitkv_suggest(1, 1, N, D, fa.FA_F32, causal)
    _say(f"[ex] fp32 N={N} D={D} causal={causal}: suggested splits {S}")
    if cus == 256:
        assert S == want
    w = Workload(f"ex_f32_auto_n{N}_d{D}", 1, 1, N, D, "f32", causal, seed=31_000 + N + D)
    x = make_inputs(w)
    o, lse = run_ex(x, "f32", w.scale, causal, 0)
    ref_o, ref_lse = oracle.forward(x["q"], x["k"], x["v"], "f32", w.scale, causal, return_lse=True)
    parity(o, ref_o, "f32", f"{w.name} causal={causal} O")
    lse_parity(lse, ref_lse, "f32", f"{w.name} causal={causal}")


@pytest.mark.parametrize("name,splits", [("prefill_b1h32n2048d64_f16", 2),
                                         ("prefill_causal_b4h32n2048d64_bf16", 3),
                                         ("long_prefill_causal_b1h16n8192d128_f16_sigma3", 4)])
def test_full_size_splits_sampled(name, splits):
    """Full-size workloads split into ranges: sampled rows (O and lse)
    against the oracle, and O against the unsplit fa_forward."""
    w = workloads.get(name)
    if w.N > 4096:
        w = w.with_(H=2)
    _say(f"[ex] {w.name} splits={splits}")
    x = make_inputs(w)
    o, lse = run_ex(x, w.dtype, w.scale, w.causal, splits)
    q, k, v = (to_device(x[n], w.dtype) for n in "qkv")
    plain = to_numpy64(fa.forward(q, k, v, scale=w.scale, causal=w.causal))
    BH = w.B * w.H
    rng = np.random.default_rng(w.seed + 7)
    heads = sorted({0, BH - 1, *rng.integers(0, BH, 2).tolist()})
    fixed = [0, 1, 63, 64, 255, 256, w.N // 2, w.N - 1]
    bh, ri = [], []
    for h in heads:
        rows = sorted(set(fixed) | set(rng.integers(0, w.N, 24).tolist()))
        bh += [h] * len(rows)
        ri += rows
    bh, ri = np.array(bh), np.array(ri)
    ref_o, ref_lse = oracle.rows(x["q"], x["k"], x["v"], w.dtype, w.scale, w.causal, bh, ri,
                                 return_lse=True)
    parity(o.reshape(BH, w.N, w.D)[bh, ri], ref_o, w.dtype, f"{name} split O")
    lse_parity(lse.reshape(BH, w.N)[bh, ri], ref_lse, w.dtype, f"{name} split")
    d = float(np.abs(o - plain).max())
    _say(f"[ex] {w.name}: split vs unsplit max abs diff {d:.3e}")
    assert d <= 2 * 2e-3 + (2.0 ** -8 * np.abs(plain).max() if w.dtype == "bf16" else 0.0)


def test_lse_scale_edge_cases():
    """Zero scale gives ln(visible count); a negative scale matches the
    oracle."""
    w = Workload("ex_scale", 1, 2, 150, 64, "f16", False, seed=808)
    x = make_inputs(w)
    for causal in (False, True):
        for S in (1, 3):
            _, lse = run_ex(x, "f16", 0.0, causal, S)
            cnt = np.arange(1, w.N + 1) if causal else np.full(w.N, w.N)
            assert np.abs(lse - np.log(cnt)[None, None, :]).max() <= 1e-5, (causal, S)
            o, lse = run_ex(x, "f16", -0.2, causal, S)
            ref_o, ref_lse = oracle.forward(x["q"], x["k"], x["v"], "f16", -0.2, causal, return_lse=True)
            parity(o, ref_o, "f16", f"negative scale causal={causal} S={S}")
            lse_parity(lse, ref_lse, "f16", f"negative scale causal={causal} S={S}")


def test_ex_without_lse_and_guard_bands():
    """lse NULL: only O is written; O and lse inside sentinel-filled buffers:
    nothing outside them changes; the workspace can be reused by a smaller
    call."""
    w = Workload("ex_guard", 1, 3, 333, 128, "bf16", True, seed=909)
    x = make_inputs(w)
    q, k, v = (to_device(x[n], "bf16") for n in "qkv")
    ws = fa.splitkv_workspace(q, 4, True)
    pad = 1024
    obuf = torch.full((pad + q.numel() + pad,), 5.0, dtype=q.dtype, device=q.device)
    o = obuf[pad:pad + q.numel()].view(q.shape)
    lbuf = torch.full((pad + 3 * w.N + pad,), 9.0, dtype=torch.float32, device=q.device)
    lse = lbuf[pad:pad + 3 * w.N].view(1, 3, w.N)
    fa.fa_forward_ex(q, k, v, o, lse, scale=w.scale, causal=True, num_splits=4, workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(obuf[:pad] == 5.0) and torch.all(obuf[pad + q.numel():] == 5.0)
    assert torch.all(lbuf[:pad] == 9.0) and torch.all(lbuf[pad + 3 * w.N:] == 9.0)
    ref_o, ref_lse = oracle.forward(x["q"], x["k"], x["v"], "bf16", w.scale, True, return_lse=True)
    parity(to_numpy64(o), ref_o, "bf16", "guard O")
    lse_parity(lse.double().cpu().numpy(), ref_lse, "bf16", "guard")
    # no lse, smaller problem, same workspace
    w2 = Workload("ex_guard2", 1, 1, 90, 64, "bf16", False, seed=910)
    x2 = make_inputs(w2)
    q2, k2, v2 = (to_device(x2[n], "bf16") for n in "qkv")
    o2 = torch.empty_like(q2)
    fa.fa_forward_ex(q2, k2, v2, o2, None, scale=w2.scale, causal=False, num_splits=2, workspace=ws)
    torch.cuda.synchronize()
    parity(to_numpy64(o2), oracle.forward(x2["q"], x2["k"], x2["v"], "bf16", w2.scale, False), "bf16",
           "reused workspace, no lse")


def test_ex_rejected_calls_raise():
    q = torch.zeros((1, 1, 256, 64), dtype=torch.float16, device="cuda:0")
    o = torch.empty_like(q)
    ws = fa.splitkv_workspace(q, 2)
    with pytest.raises(fa.FAError, match="SPLITS"):
        fa.fa_forward_ex(q, q, q, o, None, num_splits=65, workspace=ws)
    with pytest.raises(fa.FAError, match="WORKSPACE"):
        fa.fa_forward_ex(q, q, q, o, None, num_splits=2, workspace=ws[:-256])
    with pytest.raises(fa.FAError, match="WORKSPACE"):
        fa.fa_forward_ex(q, q, q, o, None, num_splits=2, workspace=None)
    lse_bad = torch.empty(256 + 1, dtype=torch.float32, device="cuda:0")[1:].view(1, 1, 256)
    fa.fa_forward_ex(q, q, q, o, lse_bad, num_splits=1)  # 4-byte aligned: accepted
    with pytest.raises(ValueError):
        fa.fa_forward_ex(q, q, q, o, torch.empty((1, 1, 255), dtype=torch.float32, device="cuda:0"))
    torch.cuda.synchronize()
