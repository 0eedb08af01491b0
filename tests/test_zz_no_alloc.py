"""GPU: fa_forward_ex_noalloc (split-KV partials in the library's fixed
per-device scratch, no allocation) against fa_forward_ex with a caller
workspace, through the C ABI: two calls in a row, the second smaller, each
bit-identical to fa_forward_ex (the same kernels) and within the parity bar
of the fp64 oracle.  Also: a call whose partials exceed the scratch is
rejected before anything is enqueued, and one split needs no scratch."""

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_fa_amd as fa
from gpu_helpers import parity, to_device, to_numpy64
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

SCRATCH = 64 * 1024 * 1024


def _say(msg):
    print(msg, flush=True)


def _both(w, splits):
    x = make_inputs(w)
    q, k, v = (to_device(x[n], w.dtype) for n in "qkv")
    code = fa.FA_F16 if w.dtype == "f16" else fa.FA_BF16
    need = fa.fa_forward_ex_workspace_bytes(w.B, w.H, w.N, w.D, code, w.causal, splits)
    assert 0 <= need <= SCRATCH
    # reference: the existing entry point with a caller workspace
    o_ref = torch.empty_like(q)
    lse_ref = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q.device)
    ws = fa.splitkv_workspace(q, splits, w.causal)
    fa.fa_forward_ex(q, k, v, o_ref, lse_ref, scale=w.scale, causal=w.causal, num_splits=splits,
                     workspace=ws)
    # the no-allocation entry point, through the C ABI; outputs prefilled
    # with NaN so that an unwritten element shows
    o = torch.full_like(q, float("nan"))
    lse = torch.full((w.B, w.H, w.N), float("nan"), dtype=torch.float32, device=q.device)
    st = fa.fa_forward_ex_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                      lse.data_ptr(), w.B, w.H, w.N, w.D, w.scale, w.causal, code,
                                      splits, torch.cuda.current_stream().cuda_stream)
    assert st == 0, fa.fa_status_string(st)
    torch.cuda.synchronize()
    return x, o, lse, o_ref, lse_ref, need


def test_noalloc_matches_workspace_entry_point_twice():
    cases = [
        (Workload("noalloc_big_f16_causal", 1, 4, 4096, 128, "f16", True, seed=811), 4),
        (Workload("noalloc_small_bf16", 1, 2, 1000, 64, "bf16", False, seed=812), 3),
    ]
    for w, splits in cases:
        _say(f"[noalloc] {w.name} B={w.B} H={w.H} N={w.N} D={w.D} splits={splits}")
        x, o, lse, o_ref, lse_ref, need = _both(w, splits)
        _say(f"[noalloc] {w.name}: partials {need} bytes of {SCRATCH}")
        assert torch.equal(o, o_ref), "O differs from fa_forward_ex with a workspace"
        assert torch.equal(lse, lse_ref), "lse differs from fa_forward_ex with a workspace"
        ref_o, ref_lse = oracle.forward(x["q"], x["k"], x["v"], w.dtype, w.scale, w.causal,
                                        return_lse=True)
        parity(to_numpy64(o), ref_o, w.dtype, w.name)
        assert float(np.abs(lse.double().cpu().numpy() - ref_lse).max()) <= 1e-3


def test_noalloc_rejects_partials_beyond_scratch_and_one_split_needs_none():
    # B*H*N*(D+1)*4 bytes per split: 8 heads x 8192 rows x 129 x 4 x 4 splits
    # = 135 MB > 64 MiB
    B, H, N, D = 1, 8, 8192, 128
    need = fa.fa_forward_ex_workspace_bytes(B, H, N, D, fa.FA_F16, False, 4)
    assert need > SCRATCH
    q = torch.zeros((B, H, N, D), dtype=torch.float16, device="cuda:0")
    k, v = torch.zeros_like(q), torch.zeros_like(q)
    o = torch.full_like(q, 3.0)
    st = fa.fa_forward_ex_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), 0,
                                      B, H, N, D, 0.125, False, fa.FA_F16, 4, 0)
    assert fa.STATUS_NAMES[st] == "FA_ERR_SCRATCH"
    torch.cuda.synchronize()
    assert torch.all(o == 3.0), "a rejected call wrote its output"
    # one split: no partials, the fused kernel writes O directly
    w = Workload("noalloc_one_split", 1, 2, 300, 96, "f16", True, seed=813)
    x, o, lse, o_ref, lse_ref, need = _both(w, 1)
    assert need == 0
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
