"""GPU: the allocating wrappers of the binding on a stream other than torch's
current one.  The output, log-sum-exp and workspace they allocate are written
by kernels on that stream after the wrapper has returned; the wrapper records
the stream on them, so memory allocated and overwritten on the current stream
meanwhile never lands in those buffers.  Checked against the fp64 oracle."""

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


def _churn(like_bytes, device, rounds=6):
    """Allocate buffers of the sizes just freed and overwrite them, on the
    current stream, while the side stream may still be running."""
    for r in range(rounds):
        for n in like_bytes:
            t = torch.empty(max(int(n), 1), dtype=torch.uint8, device=device)
            t.fill_(0xA5 ^ r)
            del t


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_side_stream_split_and_three_pass(dtype):
    w = Workload(f"side_stream_{dtype}", 1, 4, 4096, 64, dtype, False, seed=4242)
    _say(f"[side stream] {w.name} splits=4 and three-pass")
    x = make_inputs(w)
    q, k, v = (to_device(x[n], dtype) for n in "qkv")
    dev = q.device
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    code = fa.FA_F16 if dtype == "f16" else fa.FA_BF16
    ws_split = fa.fa_forward_ex_workspace_bytes(w.B, w.H, w.N, w.D, code, w.causal, 4)
    ws_naive = fa.fa_naive_workspace_bytes(w.B, w.H, w.N, code)
    # work queued on the side stream ahead of the calls keeps it busy while
    # the current stream churns through memory
    busy = torch.empty_like(q)
    with torch.cuda.stream(side):
        for _ in range(4):
            fa.fa_forward(q, k, v, busy, scale=w.scale, stream=side)
    o, lse = fa.forward_ex(q, k, v, scale=w.scale, causal=w.causal, num_splits=4, lse=True,
                           stream=side)
    o_naive = fa.naive_forward(q, k, v, scale=w.scale, causal=w.causal, stream=side)
    _churn([ws_split, ws_naive, q.numel() * q.element_size(), w.B * w.H * w.N * 4], dev)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.forward(x["q"], x["k"], x["v"], dtype, w.scale, w.causal, return_lse=True)
    parity(to_numpy64(o), ref_o, dtype, "split-KV on a side stream")
    parity(to_numpy64(o_naive), ref_o, dtype, "three-pass on a side stream")
    err = float(np.abs(lse.double().cpu().numpy() - ref_lse).max())
    _say(f"[side stream] lse max abs err {err:.3e}")
    assert err <= 1e-3
