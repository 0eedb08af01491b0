"""Tile-size calibration sweep on the current device.

"Flash Attention on Android: tiled SGEMM with RenderScript", section "The
detail that breaks naive ports: tile calibration", found the best tile size
to differ between GPUs and asks for it to be measured on each target;
"Android Transformer Optimization: Attention and Mobile GPU Bottlenecks",
section "Implementation Recommendations", sizes tiles from the on-chip
memory.  On MI355X a wave owns 32 query rows (the 32x32 matrix-core
tile); what is calibrated is the number of keys staged in LDS per tile and
barrier (32, 64 or 128), how many waves share a workgroup (and so its K/V
tiles in LDS), how many workgroups share a CU, and whether the waves split
the key tiles in two or four groups (for grids that leave CUs idle).  This tool times every shape that the calibration
library (libfa_tune.so) instantiates, for each head dimension, storage
type and mask, on synthetic inputs drawn by the workload generator, and
writes a table:

    python -m tiled_attention_fa_amd.tile_sweep --out profiles/tile_sweep_mi355x

It checks every shape's output against libfa.so's fa_forward on the same
inputs (the library's own choice), and reports fa_forward's time beside the
sweep so the table shows whether the shipped choice is the fastest.
`--from-json <out>` rewrites <out>.md from a sweep's saved <out>.json
without a device.
"""

import argparse
import ctypes
import json
import os
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
TUNE_LIB = os.path.join(PKG, "libfa_tune.so")

# (B, H, N, D, causal): per head dimension one non-causal and one causal
# shape at the sizes of the workloads, each in fp16 and bf16, then grids
# that fill a quarter, half and three quarters of the device with the
# one-group shapes (where the key groups may pay), and causal grids from
# half a pass over the workgroup slots to several.
CASES = [
    (1, 32, 2048, 64, False), (4, 32, 2048, 64, True),
    (2, 8, 1000, 96, False), (1, 16, 4096, 96, True),
    (1, 16, 4096, 128, False), (1, 16, 8192, 128, True),
    (1, 8, 2048, 64, False), (1, 16, 2048, 64, False), (1, 24, 2048, 64, False),
    (1, 8, 2048, 64, True), (1, 16, 2048, 64, True),
    (1, 4, 2048, 96, False), (2, 12, 1000, 96, False),
    (1, 8, 2048, 128, False), (1, 4, 4096, 128, True), (1, 12, 4096, 128, True),
    (1, 24, 2048, 64, True), (1, 28, 2048, 64, True), (1, 12, 2048, 96, True), (1, 6, 8192, 128, True),
    (1, 14, 4096, 128, True),
    (1, 20, 2048, 64, True), (1, 32, 2048, 64, True), (1, 40, 2048, 64, True), (2, 32, 2048, 64, True),
    (1, 16, 4096, 128, True), (1, 20, 4096, 128, True), (1, 32, 4096, 128, True), (1, 24, 4096, 96, True),
]
# The causal calibration set: per head dimension, grids that fill the
# one-group kernel's workgroup slots (256 CUs) once, one and a half, two,
# three and four times, at several row lengths.  In a causal launch the
# blocks differ in length, so the best shape depends on the fill as well as
# on D and the storage type.
CAUSAL_CASES = [
    (1, H, N, 64, True) for N, Hs in ((2048, (32, 48, 64, 96, 128)), (4096, (16, 24, 32, 48)), (8192, (8, 16)))
    for H in Hs
] + [
    (1, H, N, 96, True) for N, Hs in ((2048, (16, 24, 32, 48, 64)), (4096, (8, 12, 16, 24, 32)), (8192, (8, 12)))
    for H in Hs
] + [
    (1, H, N, 128, True) for N, Hs in ((2048, (32, 48, 64, 96)), (4096, (16, 20, 24, 32, 48)), (8192, (8, 12, 16, 24)))
    for H in Hs
]
DTYPES = ("f16", "bf16")
# fp32 (matrix-core kernel, five shapes): the single-head workload, grids
# from a few workgroups to several per CU at each D
F32_CASES = [
    (1, 1, 128, 64, False), (1, 1, 512, 64, False), (1, 4, 256, 64, False), (1, 8, 1024, 64, False),
    (1, 16, 1024, 64, False), (1, 16, 2048, 64, False), (1, 2, 2048, 64, True), (1, 8, 2048, 64, True),
    (1, 4, 4096, 64, True), (1, 16, 2048, 64, True), (1, 32, 2048, 64, True), (2, 4, 512, 96, False),
    (2, 8, 1000, 96, False), (1, 16, 1024, 96, True), (2, 16, 1024, 96, True), (1, 2, 512, 128, False),
    (1, 1, 1024, 128, False), (1, 32, 1024, 128, False), (1, 8, 2048, 128, True), (1, 4, 4096, 128, True),
    (1, 16, 1024, 128, True), (1, 32, 1024, 128, True),
]


def load_tune():
    if not os.path.exists(TUNE_LIB):
        raise ImportError(f"{TUNE_LIB} is not built; run tiled_attention_fa_amd/build.py")
    lib = ctypes.CDLL(TUNE_LIB)
    i64, vp, ip = ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(ctypes.c_int)
    lib.fa_tune_shapes.argtypes = [i64, ip, ip, ip, ip, ctypes.c_int]
    lib.fa_tune_shapes.restype = ctypes.c_int
    lib.fa_tune_forward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    lib.fa_tune_forward.restype = ctypes.c_int
    lib.fa_tune_split_merge.argtypes = [vp, vp, vp, vp, i64, i64, ctypes.c_int, ctypes.c_int, vp]
    lib.fa_tune_split_merge.restype = ctypes.c_int
    lib.fa_tune_f32_shapes.argtypes = [i64, ip, ip, ctypes.c_int]
    lib.fa_tune_f32_shapes.restype = ctypes.c_int
    lib.fa_tune_forward_f32.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, vp]
    lib.fa_tune_forward_f32.restype = ctypes.c_int
    return lib


def shapes(lib, D):
    """(waves, waves_per_eu, key_groups, keys per LDS tile) of every shape the
    library has for D."""
    w, o, g, b = ((ctypes.c_int * 16)() for _ in range(4))
    n = lib.fa_tune_shapes(D, w, o, g, b, 16)
    if n < 0:
        raise ValueError(f"no shapes for D={D}")
    return [(w[i], o[i], g[i], b[i]) for i in range(n)]


def f32_shapes(lib, D):
    """(waves of 16 rows per key group, key groups) of every fp32-kernel shape
    the library has for D."""
    r, g = (ctypes.c_int * 8)(), (ctypes.c_int * 8)()
    n = lib.fa_tune_f32_shapes(D, r, g, 8)
    if n < 0:
        raise ValueError(f"no fp32 shapes for D={D}")
    return [(r[i], g[i]) for i in range(n)]


def f32_label(shape):
    """'32r x2' = 32 query rows per workgroup in 2 key groups."""
    rw, kg = shape
    return f"{16 * rw}r x{kg}"


def tune_forward_f32(lib, q, k, v, o, scale, causal, shape, stream):
    B, H, N, D = q.shape
    st = lib.fa_tune_forward_f32(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, H, N, D,
                                 float(scale), int(causal), shape[0], shape[1], stream)
    if st != 0:
        raise RuntimeError(f"fa_tune_forward_f32 status {st}")


def tune_forward(lib, q, k, v, o, scale, causal, code, waves, occ, key_groups, block_n, stream):
    B, H, N, D = q.shape
    st = lib.fa_tune_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, H, N, D,
                             float(scale), int(causal), code, waves, occ, key_groups, block_n, stream)
    if st != 0:
        raise RuntimeError(f"fa_tune_forward status {st}")


def markdown(meta, rows, rows32):
    """The sweep's tables as Markdown, from the records main() prints and
    saves (the JSON file holds the same meta, cases and f32_cases)."""
    lines = [f"# Tile calibration sweep ({meta['arch']}, {meta['cus']} CUs)", "",
             f"Command (repository root): `{meta['command']}`", "",
             f"Mean microseconds per launch over {meta['launches_per_timing']} back-to-back launches (HIP events), "
             f"best of {meta.get('rounds', 3)} interleaved rounds, after 0.25 s of untimed launches per case; "
             "every workgroup shape of libfa_tune.so: `Nw` = N waves per workgroup (32 query rows "
             "each), `occK` = waves_per_eu hint K, `ksG` = the waves in G key groups over 1/G as many "
             "rows, every G-th key tile each, `bnB` = B keys per LDS tile (one barrier each). "
             "`fa_forward` is the shipped library's own choice on the same inputs. The first table "
             "gives the fastest shape per key-tile size, the second every shape.", "",
             "| case | fa_forward | best bn32 | best bn64 | best bn128 | best shape |",
             "|---|---|---|---|---|---|"]

    def label(s):
        return (f"{s['waves']}w occ{s['waves_per_eu']}" + (f" ks{s['key_groups']}" if s["key_groups"] > 1 else "")
                + f" bn{s['block_n']}")

    for r in rows:
        bb = {int(b): us for b, us in r["best_us_by_block_n"].items()}  # JSON keys are strings
        cell = lambda b: str(bb[b]) if b in bb else "-"
        lines.append(f"| {r['case']} | {r['fa_forward_us']} | {cell(32)} | {cell(64)} | {cell(128)} | "
                     f"{label(r['best'])} |")
    nmax = max([len(r["shapes"]) for r in rows] or [0])
    if rows:
        lines += ["", "| case | " + " | ".join(["shape / us"] * nmax) + " |", "|---|" + "---|" * nmax]
    for r in rows:
        cells = [f"{label(s)}: {s['us']}" for s in r["shapes"]]
        cells += [""] * (nmax - len(cells))
        lines.append(f"| {r['case']} | " + " | ".join(cells) + " |")
    worst = max([s["max_abs_diff_vs_fa_forward"] for r in rows for s in r["shapes"]] or [0.0])
    lines += ["", f"Largest difference of any 16-bit shape's O from fa_forward's: {worst:.3e}."]
    if rows32:
        def key32(s):  # records without the pair are the 64-row shapes (4 waves per group)
            return (s.get("row_waves", 4), s.get("key_groups", s["waves"] // 4))
        order = []
        for r in rows32:
            for s in r["shapes"]:
                if key32(s) not in order:
                    order.append(key32(s))
        lines += ["", "fp32 (matrix-core kernel, 16 query rows per wave; `Rr xG` = R query rows per workgroup "
                  "in G key groups taking every G-th 32-key tile, R/16 waves each), microseconds per launch:", "",
                  "| case | fa_forward | " + " | ".join(f32_label(k) for k in order) + " | best |",
                  "|---|---|" + "---|" * len(order) + "---|"]
        for r in rows32:
            by = {key32(s): s["us"] for s in r["shapes"]}
            cells = [str(by[k]) if k in by else "-" for k in order]
            lines.append(f"| {r['case']} | {r['fa_forward_us']} | " + " | ".join(cells) +
                         f" | {f32_label(key32(r['best']))} |")
        w32 = max(s["max_abs_diff_vs_fa_forward"] for r in rows32 for s in r["shapes"])
        lines += ["", f"Largest difference of any fp32 shape's O from fa_forward's: {w32:.3e}."]
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default="", help="write <out>.json and <out>.md")
    ap.add_argument("--launches", type=int, default=40)
    ap.add_argument("--rounds", type=int, default=3,
                    help="interleaved rounds over fa_forward and the shapes; the best round counts")
    ap.add_argument("--only", default="",
                    help="comma-separated substrings: sweep only the cases whose name contains one")
    ap.add_argument("--set", choices=("default", "causal"), default="default",
                    help="default: the mixed case list; causal: the causal calibration grids (no fp32 cases)")
    ap.add_argument("--from-json", default="",
                    help="write <from-json>.md from the saved <from-json>.json and stop (no device)")
    args = ap.parse_args()
    if args.from_json:
        saved = json.load(open(args.from_json + ".json"))
        open(args.from_json + ".md", "w").write(markdown(saved["meta"], saved["cases"], saved.get("f32_cases", [])))
        return
    only = [x for x in args.only.split(",") if x]

    sys.path.insert(0, ROOT)
    import numpy as np
    import torch

    import tiled_attention_fa_amd as fa
    import workloads

    lib = load_tune()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}
    codes = {"f16": fa.FA_F16, "bf16": fa.FA_BF16}

    def timed(fn):
        for _ in range(3):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.launches):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.launches * 1e3

    rows = []
    for B, H, N, D, causal in (CASES if args.set == "default" else CAUSAL_CASES):
        for dt in DTYPES:
            w = workloads.Workload(f"sweep_b{B}h{H}n{N}d{D}_{dt}{'_causal' if causal else ''}", B, H, N, D, dt,
                                   causal, seed=50_000 + N + D)
            if only and not any(o in w.name for o in only):
                continue
            x = workloads.make_inputs(w)
            q, k, v = (torch.from_numpy(np.ascontiguousarray(x[n]).view(np.int16)).view(tdt[dt]).to(dev)
                       for n in "qkv")
            ref = torch.empty_like(q)
            out = torch.empty_like(q)
            # direct C calls with prepared arguments, so that host overhead
            # does not starve the device between launches
            base = (q.data_ptr(), k.data_ptr(), v.data_ptr())
            lib_fa = fa.load_library()
            fwd_args = base + (ref.data_ptr(), B, H, N, D, float(w.scale), int(causal), codes[dt],
                               stream.cuda_stream)

            def call():
                if lib_fa.fa_forward(*fwd_args) != 0:
                    raise RuntimeError("fa_forward failed")

            # the clock drops while the host prepares the inputs: run
            # untimed launches until it is back up
            t0 = time.time()
            while time.time() - t0 < 0.25:
                call()
            torch.cuda.synchronize()
            flops = workloads.flops(w)
            variants = shapes(lib, D)
            best_lib = float("inf")
            best = {sh: float("inf") for sh in variants}
            for _ in range(args.rounds):
                best_lib = min(best_lib, timed(call))
                for sh in variants:
                    targs = base + (out.data_ptr(), B, H, N, D, float(w.scale), int(causal), codes[dt]) + sh + (
                        stream.cuda_stream,)
                    best[sh] = min(best[sh], timed(lambda: lib.fa_tune_forward(*targs)))
            rec = {"case": w.name, "B": B, "H": H, "N": N, "D": D, "dtype": dt, "causal": causal,
                   "fa_forward_us": round(best_lib, 2), "shapes": []}
            for waves, occ, ks, bn in variants:
                tune_forward(lib, q, k, v, out, w.scale, causal, codes[dt], waves, occ, ks, bn,
                             stream.cuda_stream)
                torch.cuda.synchronize()
                diff = float((out.float() - ref.float()).abs().max().item())
                t = best[(waves, occ, ks, bn)]
                rec["shapes"].append({"waves": waves, "rows": 32 * waves // ks, "waves_per_eu": occ,
                                      "key_groups": ks, "block_n": bn, "us": round(t, 2),
                                      "tflops": round(flops / (t * 1e-6) / 1e12, 1),
                                      "max_abs_diff_vs_fa_forward": diff})
            best = min(rec["shapes"], key=lambda s: s["us"])
            rec["best"] = {"waves": best["waves"], "waves_per_eu": best["waves_per_eu"],
                           "key_groups": best["key_groups"], "block_n": best["block_n"], "us": best["us"]}
            by_bn = {}
            for sh in rec["shapes"]:
                by_bn[sh["block_n"]] = min(by_bn.get(sh["block_n"], float("inf")), sh["us"])
            rec["best_us_by_block_n"] = by_bn
            rows.append(rec)
            print(json.dumps(rec), flush=True)
            del q, k, v, ref, out

    rows32 = []
    for B, H, N, D, causal in (F32_CASES if args.set == "default" else []):
        w = workloads.Workload(f"sweep_b{B}h{H}n{N}d{D}_f32{'_causal' if causal else ''}", B, H, N, D, "f32",
                               causal, seed=52_000 + N + D)
        if only and not any(o in w.name for o in only):
            continue
        x = workloads.make_inputs(w)
        q, k, v = (torch.from_numpy(np.ascontiguousarray(x[n]).view(np.float32)).to(dev) for n in "qkv")
        ref = torch.empty_like(q)
        out = torch.empty_like(q)
        lib_fa = fa.load_library()
        base = (q.data_ptr(), k.data_ptr(), v.data_ptr())
        fwd_args = base + (ref.data_ptr(), B, H, N, D, float(w.scale), int(causal), fa.FA_F32, stream.cuda_stream)

        def call32():
            if lib_fa.fa_forward(*fwd_args) != 0:
                raise RuntimeError("fa_forward failed")

        t0 = time.time()
        while time.time() - t0 < 0.25:
            call32()
        torch.cuda.synchronize()
        variants = f32_shapes(lib, D)
        best_lib = float("inf")
        best = {wv: float("inf") for wv in variants}
        for _ in range(args.rounds):
            best_lib = min(best_lib, timed(call32))
            for wv in variants:
                targs = base + (out.data_ptr(), B, H, N, D, float(w.scale), int(causal), wv[0], wv[1],
                                stream.cuda_stream)
                best[wv] = min(best[wv], timed(lambda: lib.fa_tune_forward_f32(*targs)))
        flops = workloads.flops(w)
        rec = {"case": w.name, "B": B, "H": H, "N": N, "D": D, "dtype": "f32", "causal": causal,
               "fa_forward_us": round(best_lib, 2), "shapes": []}
        for wv in variants:
            tune_forward_f32(lib, q, k, v, out, w.scale, causal, wv, stream.cuda_stream)
            torch.cuda.synchronize()
            diff = float((out - ref).abs().max().item())
            rec["shapes"].append({"row_waves": wv[0], "key_groups": wv[1], "waves": wv[0] * wv[1],
                                  "rows": 16 * wv[0], "us": round(best[wv], 2),
                                  "tflops": round(flops / (best[wv] * 1e-6) / 1e12, 3),
                                  "max_abs_diff_vs_fa_forward": diff})
        rec["best"] = min(rec["shapes"], key=lambda s: s["us"])
        rows32.append(rec)
        print(json.dumps(rec), flush=True)
        del q, k, v, ref, out

    if args.out:
        prop = torch.cuda.get_device_properties(dev)
        meta = {"device": prop.name, "arch": getattr(prop, "gcnArchName", ""), "cus": prop.multi_processor_count,
                "launches_per_timing": args.launches, "rounds": args.rounds,
                "command": "python -m tiled_attention_fa_amd.tile_sweep "
                + ("--set causal " if args.set == "causal" else "") + "--out " + args.out}
        json.dump({"meta": meta, "cases": rows, "f32_cases": rows32}, open(args.out + ".json", "w"), indent=1)
        open(args.out + ".md", "w").write(markdown(meta, rows, rows32))


if __name__ == "__main__":
    main()
