"""Benchmark of the attention forward pass on one MI355X.

One step = one fa_forward call over the whole workload (all heads), inputs
resident in HBM.  Prints one JSON line:

  metric / value / unit   attention forward TFLOP/s (algorithmic FLOPs:
                          4*B*H*N^2*D, half that when causal) over the timed
                          region, whole job
  roofline                the forward kernel against MI355X dense fp16/bf16
                          matrix-core peak (2.5 PFLOP/s): achieved = FLOPs per
                          launch / mean launch duration (HIP events around K
                          back-to-back launches); traffic = HBM bytes per launch
                          from rocprofv3 counters when a profile of the
                          current kernel source is committed, else null
  cpu_baseline            the fp64 oracle timed on this host's cores on a
                          bounded sample of the same workload (reported
                          baseline only); the heads it computes double as a
                          parity check of the GPU output
                          (max_abs_err_oracle_heads)
  naive_three_pass        (16-bit storage) the three-pass attention on the
                          same inputs: time per call, the tiled pass's
                          speed-up over it, both byte counts

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

import argparse
import ctypes
import hashlib
import glob
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

METRIC = "attention fwd TFLOP/s + % MFMA fp16 peak, H=32 D=64 N=2048 (1 GPU)"
PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}  # MI355X dense peaks
PEAK_HBM_GBS = 8000.0
PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


KERNEL_SOURCES = {
    # files that define the kernel a workload of each storage type runs
    "f16": ["fa_api.hip", "fa_internal.h", "fa_mfma.h", "fa_mfma_f16.hip"],
    "bf16": ["fa_api.hip", "fa_internal.h", "fa_mfma.h", "fa_mfma_bf16.hip"],
    "f32": ["fa_api.hip", "fa_internal.h", "fa_f32.hip"],
}


# files that define the three kernels of the three-pass comparison path
NAIVE_SOURCES = {dt: ["fa_api.hip", "fa_internal.h", "fa_mfma.h", "fa_naive.hip"] for dt in ("f16", "bf16")}


def kernel_source_hash(dtype: str, sources=None) -> str:
    """Hash of the sources of the kernel that a workload of this storage type
    runs (or of the files listed), with comments and whitespace removed, so
    that a counter profile stays valid across comment-only edits and edits
    of other kernels."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tiled_attention_fa_amd", "csrc")
    for name in (sources if sources is not None else KERNEL_SOURCES[dtype]):
        text = open(os.path.join(csrc, name), encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        text = " ".join(text.split())
        h.update(name.encode())
        h.update(text.encode())
    return h.hexdigest()[:16]


def committed_traffic(name: str, sources=None):
    """HBM bytes per call from a committed counter profile (traffic_<name>.json,
    name = a workload, or "naive_" / "cold_" + a workload) of the current
    kernel source, or None."""
    path = os.path.join(PROFILE_DIR, f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    base = name
    for prefix in ("naive_", "cold_"):
        if base.startswith(prefix):
            base = base[len(prefix):]
    dtype = workloads.get(base).dtype
    if rec.get("kernel_source_hash") != kernel_source_hash(dtype, sources):
        return None
    return rec.get("hbm_bytes_per_launch")


def torch_inputs(w, x, device):
    import torch
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[w.dtype]
    out = []
    for n in "qkv":
        a = np.ascontiguousarray(x[n])
        t = torch.from_numpy(a if w.dtype == "f32" else a.view(np.int16)).view(tdt)
        out.append(t.to(device))
    return out


def cpu_baseline(w, x, o=None, budget_s: float = 20.0):
    """Time the fp64 oracle on a bounded sample of the workload: whole heads,
    as many as fit the budget (estimated from one head).  With o (the GPU
    output as a [B, H, N, D] tensor) also the largest difference between it
    and the oracle on those heads."""
    import oracle
    BH = w.B * w.H
    q = x["q"].reshape(BH, 1, w.N, w.D)
    k = x["k"].reshape(BH, 1, w.N, w.D)
    v = x["v"].reshape(BH, 1, w.N, w.D)
    t0 = time.perf_counter()
    _, _, used = oracle.forward(q[:1], k[:1], v[:1], w.dtype, w.scale, w.causal, return_rowsum=True)
    one = time.perf_counter() - t0
    heads = int(max(1, min(BH, budget_s / max(one, 1e-6))))
    t0 = time.perf_counter()
    ref, _, used = oracle.forward(q[:heads], k[:heads], v[:heads], w.dtype, w.scale, w.causal,
                                  return_rowsum=True)
    dt = time.perf_counter() - t0
    flops = workloads.flops(w) * heads / BH
    rec = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(used), "kind": "oracle",
           "sample": f"{heads} of {BH} heads of {w.name} (fp64, S and P rows materialised), "
                     f"{dt:.2f} s"}
    if o is not None:
        got = o.contiguous().float().cpu().numpy().astype(np.float64).reshape(BH, w.N, w.D)[:heads]
        rec["max_abs_err_vs_gpu"] = float(np.abs(got - ref.reshape(heads, w.N, w.D)).max())
    return rec


def naive_leg(w, q, k, v, o, stream, code, lib, steps, tiled_ms):
    """The three-pass comparison (S and P through HBM) on the same inputs:
    mean time per call over `steps` back-to-back calls, its bytes against
    the tiled pass, and its largest difference from the tiled pass's O."""
    import torch
    import tiled_attention_fa_amd as fa
    ws = fa.naive_workspace(q)
    on = torch.empty_like(o)
    cargs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), on.data_ptr(), w.B, w.H, w.N, w.D,
             float(w.scale), int(w.causal), code, ws.data_ptr(), ws.numel(), stream.cuda_stream)

    def call():
        st = lib.fa_naive_forward(*cargs)
        if st != 0:
            raise fa.FAError(st)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        call()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    # the median of individually bracketed calls, as the pages report theirs
    singles = []
    for _ in range(max(20, min(steps, 50))):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        e1.synchronize()
        singles.append(e0.elapsed_time(e1) * 1e3)
    nb = workloads.naive_bytes(w)
    diff = float((on.float() - o.float()).abs().max().item())
    log(f"three-pass: {ms * 1e3:.2f} us per call ({steps} calls), {nb / (ms * 1e-3) / 1e9:.0f} GB/s "
        f"algorithmic; tiled pass {ms / tiled_ms:.2f}x faster")
    return {
        "ms_per_call": round(ms, 5),
        "calls": steps,
        "median_single_call_us": round(float(np.median(singles)), 3),
        "single_calls": len(singles),
        "tiled_speedup": round(ms / tiled_ms, 3),
        "algorithmic_bytes": nb,
        "achieved_GBs": round(nb / (ms * 1e-3) / 1e9, 1),
        "frac_hbm_peak": round(nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "tiled_min_bytes": workloads.min_bytes(w),
        "bytes_ratio": round(nb / workloads.min_bytes(w), 2),
        "workspace_bytes": ws.numel(),
        "traffic": committed_traffic("naive_" + w.name, sources=NAIVE_SOURCES[w.dtype]),
        "max_abs_diff_vs_tiled": diff,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=workloads.HEADLINE, choices=workloads.ORDER + workloads.PAGE_TABLE)
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="seconds of untimed launches before the warm-up steps, so that the "
                         "GPU clock has left its ramp (it takes tens of ms under this load)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true",
                    help="skip comparing the GPU output with the oracle heads of the CPU baseline")
    ap.add_argument("--layout", choices=("bhnd", "bnhd"), default="bhnd",
                    help="memory layout of q, k, v, o: dense [B, H, N, D] (fa_forward) or "
                         "[B, N, H, D] (fa_forward_strided)")
    ap.add_argument("--kv-heads", type=int, default=0,
                    help="key/value heads (grouped-query attention through fa_forward_strided; "
                         "0: as many as query heads)")
    ap.add_argument("--heads", type=int, default=0,
                    help="run the workload with this many heads instead (same recipe and seed); "
                         "for the few-head cases that split-KV is for")
    ap.add_argument("--splits", type=int, default=1,
                    help="key ranges per query block (fa_forward_ex split-KV; 0: the library's "
                         "suggestion for this device); 1 times fa_forward itself")
    ap.add_argument("--no-naive", action="store_true",
                    help="skip the three-pass comparison leg (16-bit storage only)")
    ap.add_argument("--cold-flush-mib", type=int, default=0,
                    help="cold-cache run: before every launch, write a buffer of this many MiB "
                         "(512 evicts L2 and the 256 MB Infinity Cache); each launch is timed on its own "
                         "and value is from their median")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of attention, time a plain device copy of this many MiB "
                         "(reference kernel for scaling HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the library runs on one GPU; heads are independent, so a caller shards them)", file=sys.stderr)
        sys.exit(2)

    import torch
    import tiled_attention_fa_amd as fa

    dev = torch.device("cuda:0")
    prop = torch.cuda.get_device_properties(dev)
    log(f"device: {prop.name} {getattr(prop, 'gcnArchName', '')} CUs={prop.multi_processor_count}")

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * 2 ** 20 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {args.steps} copies of {args.copy_calibration_mib} MiB")
        return

    w = workloads.get(args.workload)
    if args.heads:
        w = w.with_(H=args.heads)
    x = workloads.make_inputs(w)
    kvh = args.kv_heads or w.H
    if w.H % kvh:
        sys.exit(f"--kv-heads {kvh} must divide the {w.H} query heads")
    if kvh != w.H:  # K and V drawn by the same recipe at kvh heads
        xkv = workloads.make_inputs(w.with_(H=kvh, seed=w.seed + 1))
        x = {"q": x["q"], "k": xkv["k"], "v": xkv["v"]}
    input_sha = {n: hashlib.sha256(np.ascontiguousarray(x[n]).tobytes()).hexdigest()[:16]
                 for n in "qkv"}
    # dense inputs as the oracle takes them: each K/V head repeated for its group
    x_dense = x if kvh == w.H else {"q": x["q"], "k": np.repeat(x["k"], w.H // kvh, axis=1),
                                    "v": np.repeat(x["v"], w.H // kvh, axis=1)}
    q, k, v = torch_inputs(w, x, dev)
    strided = args.layout != "bhnd" or kvh != w.H
    if args.layout == "bnhd":  # stored [B, N, H, D], viewed as [B, H, N, D]
        q, k, v = (t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for t in (q, k, v))
        o = torch.empty((w.B, w.N, w.H, w.D), dtype=q.dtype, device=dev).permute(0, 2, 1, 3)
    else:
        o = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)

    # The binding checks the tensors once; the timed loop then calls the C
    # entry point with the same pointers and sizes (inputs stay resident).
    code = {"f16": fa.FA_F16, "bf16": fa.FA_BF16, "f32": fa.FA_F32}[w.dtype]
    lib = fa.load_library()
    if strided:
        if args.splits != 1:
            sys.exit("--splits applies to the dense layout only")
        fa.fa_forward_strided(q, k, v, o, scale=w.scale, causal=w.causal, stream=stream)
        strides = [(ctypes.c_int64 * 3)(*t.stride()[:3]) for t in (q, k, v, o)]
        sargs = (q.data_ptr(), strides[0], k.data_ptr(), strides[1], v.data_ptr(), strides[2],
                 o.data_ptr(), strides[3], w.B, w.H, kvh, w.N, w.D, float(w.scale), int(w.causal),
                 code, stream.cuda_stream)
    else:
        fa.fa_forward(q, k, v, o, scale=w.scale, causal=w.causal, stream=stream)
    cargs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), w.B, w.H, w.N, w.D,
             float(w.scale), int(w.causal), code, stream.cuda_stream)

    splits = args.splits
    if splits != 1:
        if splits == 0:
            splits = fa.fa_splitkv_suggest(w.B, w.H, w.N, w.D, code, w.causal)
        ws = fa.splitkv_workspace(q, splits, w.causal)
        fa.fa_forward_ex(q, k, v, o, None, scale=w.scale, causal=w.causal, num_splits=splits,
                         workspace=ws, stream=stream)
        xargs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), None, w.B, w.H, w.N, w.D,
                 float(w.scale), int(w.causal), code, splits, ws.data_ptr(), ws.numel(),
                 stream.cuda_stream)

    def launch():
        if strided:
            st = lib.fa_forward_strided(*sargs)
        else:
            st = lib.fa_forward(*cargs) if splits == 1 else lib.fa_forward_ex(*xargs)
        if st != 0:
            raise fa.FAError(st)

    # Cold-cache mode: every launch follows a write of the flush buffer, so
    # no input is left in L2 or the Infinity Cache.
    cold = args.cold_flush_mib > 0
    flush_buf = torch.empty(args.cold_flush_mib * 2 ** 20, dtype=torch.uint8, device=dev) if cold else None
    flushes = [0]

    def step():
        if cold:
            flushes[0] += 1
            flush_buf.fill_(flushes[0] & 0xFF)
        launch()

    # Clock settle, then the W warm-up steps; neither is timed.
    settle_launches = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
        settle_launches += 20
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K back-to-back launches between two events recorded on
    # the stream the kernel runs on.  Cold: K launches, each after a flush
    # and between its own pair of events (the flush is not timed); the
    # median launch stands for the step.
    if cold:
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(args.steps)]
        torch.cuda.synchronize()
        for e0, e1 in pairs:
            flushes[0] += 1
            flush_buf.fill_(flushes[0] & 0xFF)
            e0.record(stream)
            launch()
            e1.record(stream)
        torch.cuda.synchronize()
        cold_us = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in pairs)
        ms_per_step = float(np.median(cold_us)) * 1e-3
    else:
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(args.steps):
            step()
        ev1.record(stream)
        torch.cuda.synchronize()
        total_ms = ev0.elapsed_time(ev1)
        ms_per_step = total_ms / args.steps
    flops = workloads.flops(w)
    value = flops / (ms_per_step * 1e-3) / 1e12
    # Per-launch duration of the forward kernel: the launches are
    # back-to-back on one stream, so the region time over K is the mean
    # kernel duration plus the (small) gap between kernels.  With splits
    # the step is two kernels (the ranges, then the merge) and this is
    # their sum.
    kern_us = ms_per_step * 1e3
    achieved = flops / (kern_us * 1e-6) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    if cold:
        log(f"cold: median launch {kern_us:.2f} us over {args.steps} launches, each after a "
            f"{args.cold_flush_mib} MiB flush")
    else:
        log(f"mean launch {kern_us:.2f} us over {args.steps} back-to-back launches")

    # Median of individually bracketed launches (each with its own event
    # pair, so it includes the event overhead; reported beside the mean).
    singles = cold_us if cold else []
    n_singles = 0 if cold else max(20, min(args.steps, 50))
    for _ in range(n_singles):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        launch()
        e1.record(stream)
        e1.synchronize()
        singles.append(e0.elapsed_time(e1) * 1e3)
    median_single_us = float(np.median(singles))

    naive = None
    if w.dtype != "f32" and not args.no_naive and not strided and not cold:
        naive = naive_leg(w, q, k, v, o, stream, code, lib, max(10, min(args.steps, 50)), ms_per_step)

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "D": w.D,
                   "storage": w.dtype, "causal": w.causal, "parallelism": "none (1 GPU)",
                   "splits": splits, "layout": args.layout, "kv_heads": kvh,
                   "cache": f"cold ({args.cold_flush_mib} MiB written before each launch)" if cold
                   else "warm (back-to-back launches)"},
        "pct_peak": round(100 * value / peak, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            # the committed counter profile is of the dense, unsplit workload
            "traffic": committed_traffic(("cold_" if cold else "") + w.name)
            if (not strided and splits == 1 and not args.heads) else None,
            "kernel_us_mean": round(kern_us, 3),
            "min_bytes": workloads.min_bytes(w) * (w.H + kvh) // (2 * w.H),
        },
        "median_single_launch_us": round(median_single_us, 3),
        # where the timed launches sit among the forward kernel's dispatches
        # (a kernel trace of this run takes its steady-state figure from them)
        "trace_window": {"timed_launches": args.steps, "launches_after_timed": n_singles},
        "untimed_settle": {"seconds": args.settle_s, "launches": settle_launches},
        "device": {"name": prop.name, "arch": getattr(prop, "gcnArchName", ""),
                   "cus": prop.multi_processor_count, "max_clock_mhz": round(fa.fa_device_info()[1] / 1000),
                   "peak_used": f"dense {w.dtype} matrix-core peak {peak} TFLOP/s (published)"},
        "inputs_sha256_16": input_sha,
        "kernel_source_hash": kernel_source_hash(w.dtype),
    }
    if naive is not None:
        rec["naive_three_pass"] = naive
    if not args.no_cpu_baseline:
        # the oracle's heads double as a parity check of the GPU output
        rec["cpu_baseline"] = cpu_baseline(w, x_dense, None if args.no_check else o)
        if not args.no_check:
            rec["max_abs_err_oracle_heads"] = rec["cpu_baseline"]["max_abs_err_vs_gpu"]
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
