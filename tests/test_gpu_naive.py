"""GPU parity of the three-pass attention (fa_naive_forward: S to memory,
row softmax to P, then P V) against the fp64 oracle, through the C ABI.

The three-pass path is the comparison the pages measure tiling against
("Android Transformer Optimization: Attention and Mobile GPU Bottlenecks",
section "The Self-Attention Bottleneck Is Memory Traffic, Not Compute";
"Flash Attention on Android: tiled SGEMM with RenderScript", section
"Benchmark results: Snapdragon vs. Dimensity").  It must give the same O as
the tiled pass, to the same tolerance.  The workspace it leaves behind is
checked too: S against the plain definition scale * Q K^T, P against the
softmax invariants (rows sum to one, masked entries exactly zero).
"""

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_fa_amd as fa
import workloads
from gpu_helpers import TORCH_DTYPES, parity, to_device, to_numpy64
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def run_naive(x, dtype, scale, causal, workspace=None):
    q, k, v = (to_device(x[n], dtype) for n in "qkv")
    o = fa.naive_forward(q, k, v, scale=scale, causal=causal, workspace=workspace)
    torch.cuda.synchronize()
    return to_numpy64(o)


def run_fused(x, dtype, scale, causal):
    q, k, v = (to_device(x[n], dtype) for n in "qkv")
    o = fa.forward(q, k, v, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return to_numpy64(o)


NAIVE_N = [1, 2, 31, 63, 64, 65, 129, 200]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_naive_sweep(dtype, D, causal):
    for i, N in enumerate(NAIVE_N):
        BH = (1, 1) if i % 2 == 0 else (1, 3)
        w = Workload(f"naive_{dtype}_d{D}_n{N}", BH[0], BH[1], N, D, dtype, causal,
                     seed=20_000 + 41 * N + D + (1 if causal else 0))
        _say(f"[naive sweep] {w.name} causal={causal} BH={BH}")
        x = make_inputs(w)
        got = run_naive(x, dtype, w.scale, causal)
        ref = oracle.forward(x["q"], x["k"], x["v"], dtype, w.scale, causal)
        parity(got, ref, dtype, f"naive {w.name} causal={causal}")


def test_naive_prefill_matches_oracle_and_fused():
    """The 1B-LLM prefill shape (B=1, H=32, N=2048, D=64, fp16): every
    element against the oracle, and against the tiled pass."""
    w = workloads.get("prefill_b1h32n2048d64_f16")
    _say(f"[naive] {w.name}")
    x = make_inputs(w)
    got = run_naive(x, w.dtype, w.scale, w.causal)
    ref = oracle.forward(x["q"], x["k"], x["v"], w.dtype, w.scale, w.causal)
    e = parity(got, ref, w.dtype, "naive prefill")
    fused = run_fused(x, w.dtype, w.scale, w.causal)
    d = float(np.abs(got - fused).max())
    _say(f"[naive] max abs err vs oracle {e['max_abs']:.3e}, vs tiled pass {d:.3e}")
    assert d <= 4e-3


@pytest.mark.parametrize("name", ["prefill_causal_b4h32n2048d64_bf16",
                                  "long_prefill_causal_b1h16n8192d128_f16_sigma3"])
def test_naive_large_sampled(name):
    """Causal bf16 prefill at full size, and the long head-dim-128 causal
    prefill with large logits (two heads): sampled rows against the oracle."""
    w = workloads.get(name)
    if w.N > 4096:
        w = w.with_(H=2)
    _say(f"[naive] {w.name} shape={w.shape}")
    x = make_inputs(w)
    got = run_naive(x, w.dtype, w.scale, w.causal)
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(w.seed + 1)
    BH = w.B * w.H
    heads = sorted({0, BH - 1, *rng.integers(0, BH, 2).tolist()})
    fixed = [0, 1, 63, 64, 127, 128, w.N // 2, w.N - 65, w.N - 64, w.N - 1]
    bh, ri = [], []
    for h in heads:
        rows = sorted(set(fixed) | set(rng.integers(0, w.N, 30).tolist()))
        bh += [h] * len(rows)
        ri += rows
    bh, ri = np.array(bh), np.array(ri)
    ref = oracle.rows(x["q"], x["k"], x["v"], w.dtype, w.scale, w.causal, bh, ri)
    e = parity(got.reshape(BH, w.N, w.D)[bh, ri], ref, w.dtype, f"naive {name} sampled")
    _say(f"[naive] {w.name}: max abs err {e['max_abs']:.3e}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_naive_workspace_contents(dtype, causal):
    """S equals scale * Q K^T where it is read; P rows sum to one, entries
    past N and (causal) past the diagonal inside the row's 64-key block are
    exactly zero (after undoing the documented key order within groups of
    16)."""
    w = Workload(f"naive_ws_{dtype}", 1, 2, 150, 96, dtype, causal, seed=303)
    x = make_inputs(w)
    q, k, v = (to_device(x[n], dtype) for n in "qkv")
    ws = fa.naive_workspace(q)
    nbytes = fa.fa_naive_workspace_bytes(1, 2, w.N, fa.FA_F16 if dtype == "f16" else fa.FA_BF16)
    assert ws.numel() == nbytes
    fa.naive_forward(q, k, v, scale=w.scale, causal=causal, workspace=ws)
    torch.cuda.synchronize()
    BH, N = 2, w.N
    NP = (N + 63) // 64 * 64
    s_bytes = BH * N * NP * 4
    p_off = (s_bytes + 255) // 256 * 256
    p_bytes = BH * N * NP * 2
    plo_off = (p_off + p_bytes + 255) // 256 * 256
    S = ws[:s_bytes].view(torch.float32).view(BH, N, NP).cpu().numpy().astype(np.float64)[:, :, :N]
    P = ws[p_off:p_off + p_bytes].view(TORCH_DTYPES[dtype]).view(BH, N, NP).float().cpu().numpy()
    P = P.astype(np.float64)
    if dtype == "bf16":
        P = P + ws[plo_off:plo_off + p_bytes].view(torch.bfloat16).view(BH, N, NP).float().cpu().numpy()
    # undo the stored key order: within each 16 keys, groups of 4 keys 1 and 2 trade places
    order = np.arange(NP).reshape(-1, 4, 4)[:, [0, 2, 1, 3], :].reshape(-1)
    P = P[:, :, order]
    qd = oracle.decode(x["q"], dtype).reshape(BH, N, w.D)
    kd = oracle.decode(x["k"], dtype).reshape(BH, N, w.D)
    S_ref = w.scale * np.einsum("hid,hjd->hij", qd, kd)
    vis = np.tril(np.ones((N, N), bool)) if causal else np.ones((N, N), bool)
    err_s = np.abs(S - S_ref)[:, vis].max()
    _say(f"[naive ws] {dtype} causal={causal}: S max abs err {err_s:.3e}")
    assert err_s <= 1e-4
    for i in range(N):
        n_out = min(NP, (i // 64 + 1) * 64) if causal else NP
        n_vis = i + 1 if causal else N
        assert np.all(P[:, i, n_vis:n_out] == 0.0), f"row {i}: masked P not zero"
        assert np.all(P[:, i, :n_vis] >= 0.0)
    sums = np.array([[P[h, i, :(i + 1 if causal else N)].sum() for i in range(N)] for h in range(BH)])
    tol = 1e-3 if dtype == "f16" else 1e-4
    assert np.abs(sums - 1.0).max() <= tol, np.abs(sums - 1.0).max()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_naive_scale_edge_cases(dtype):
    w = Workload(f"naive_scale_{dtype}", 1, 2, 300, 64, dtype, False, seed=78)
    x = make_inputs(w)
    for scale in (0.0, -0.125, 2.0):
        for causal in (False, True):
            _say(f"[naive scale] {dtype} scale={scale} causal={causal}")
            got = run_naive(x, dtype, scale, causal)
            ref = oracle.forward(x["q"], x["k"], x["v"], dtype, scale, causal)
            parity(got, ref, dtype, f"naive scale={scale} causal={causal}")


def test_naive_reused_workspace_and_guard_bands():
    """A workspace reused for a smaller problem, O inside a sentinel-filled
    buffer: only O's bytes change, inputs stay bit-identical."""
    big = Workload("naive_big", 1, 2, 333, 64, "f16", True, seed=404)
    xb = make_inputs(big)
    qb = to_device(xb["q"], "f16")
    ws = fa.naive_workspace(qb)
    parity(run_naive(xb, "f16", big.scale, True, workspace=ws),
           oracle.forward(xb["q"], xb["k"], xb["v"], "f16", big.scale, True), "f16", "naive big")
    w = Workload("naive_small", 1, 1, 70, 128, "f16", False, seed=405)
    x = make_inputs(w)
    q, k, v = (to_device(x[n], "f16") for n in "qkv")
    before = [t.clone() for t in (q, k, v)]
    pad = 2048
    buf = torch.full((pad + q.numel() + pad,), 7.0, dtype=q.dtype, device=q.device)
    o = buf[pad:pad + q.numel()].view(q.shape)
    fa.fa_naive_forward(q, k, v, o, ws, scale=w.scale, causal=False)
    torch.cuda.synchronize()
    assert torch.all(buf[:pad] == 7.0) and torch.all(buf[pad + q.numel():] == 7.0)
    for t0, t1 in zip(before, (q, k, v)):
        assert torch.equal(t0, t1)
    parity(to_numpy64(o), oracle.forward(x["q"], x["k"], x["v"], "f16", w.scale, False), "f16",
           "naive reused workspace")


def test_naive_rejected_calls_raise():
    q = torch.zeros((1, 1, 64, 64), dtype=torch.float16, device="cuda:0")
    o = torch.empty_like(q)
    ws = fa.naive_workspace(q)
    with pytest.raises(fa.FAError, match="WORKSPACE"):
        fa.fa_naive_forward(q, q, q, o, ws[:-256])
    with pytest.raises(fa.FAError, match="WORKSPACE"):
        fa.fa_naive_forward(q, q, q, o, ws[16:])
    both = torch.empty(ws.numel() + q.numel() * 2, dtype=torch.uint8, device="cuda:0")
    o_in_ws = both[:q.numel() * 2].view(torch.float16).view(q.shape)
    with pytest.raises(fa.FAError, match="WORKSPACE"):
        fa.fa_naive_forward(q, q, q, o_in_ws, both)
    q32 = q.float()
    with pytest.raises(fa.FAError, match="DTYPE"):
        fa.fa_naive_forward(q32, q32, q32, torch.empty_like(q32), ws)
    with pytest.raises(fa.FAError, match="ALIAS"):
        fa.fa_naive_forward(q, q, q, q, ws)
