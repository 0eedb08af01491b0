"""Summaries of the rocprofv3 runs behind `bench.py`'s roofline figures.

`bench.py` reports `roofline.traffic` from `profiles/traffic_<workload>.json` (and,
with `--cold-flush-mib`, from `traffic_cold_<workload>.json`) when the file's
kernel source hash matches the current sources.  This module writes those files
and the Markdown summaries beside them from the CSV output of the rocprofv3
runs that each summary lists, so every committed figure can be rebuilt:

python -m tiled_attention_fa_amd.profile_report warm --workload W --dir D
python -m tiled_attention_fa_amd.profile_report cold --workload W --dir D

D is the directory the rocprofv3 runs wrote to (their `-d` arguments are
D/prof_FETCH_SIZE_W, D/prof_WRITE_SIZE_W, D/prof_FETCH_SIZE_copy256,
D/prof_WRITE_SIZE_copy256 and D/prof_trace_W, whose bench output is
D/prof_trace_W.log; for "cold", D/prof_FETCH_SIZE_cold_W,
D/prof_WRITE_SIZE_cold_W and the cold bench's output D/cold_bench_W.log).
The counters are scaled by what the same counters read for a plain 256 MiB
device copy, so FETCH_SIZE and WRITE_SIZE become bytes.
"""

import argparse
import collections
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "profiles")  # where the summaries go (--out-dir)


FORWARD = "fa_forward_"  # the forward kernels: fa_forward_kernel (16-bit) and fa_forward_f32_kernel


def is_forward(name, filt=FORWARD):
    if filt != FORWARD:
        return filt in name
    return "fa_forward_kernel" in name or "fa_forward_f32_kernel" in name


def agg(path, filt=FORWARD):
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if is_forward(r["Kernel_Name"], filt):
            per[r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in per.items()}, {k: len(v) for k, v in per.items()}


def steady(trace_csv, rec, filt=FORWARD):
    """Duration of the timed launches alone, from the per-dispatch kernel
    trace: the forward kernel's dispatches in start order, of which the
    bench's timed launches are the `timed_launches` before the last
    `launches_after_timed` (the clock-settle and warm-up launches come
    first).  Returns mean and median in microseconds, or None when the run
    did not record its window."""
    win = rec.get("trace_window")
    if not win or not os.path.exists(trace_csv):
        return None
    every = list(csv.DictReader(open(trace_csv)))
    rows = [r for r in every if is_forward(r["Kernel_Name"], filt)]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    k, after = win["timed_launches"], win["launches_after_timed"]
    timed = rows[len(rows) - after - k:len(rows) - after]
    us = sorted((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in timed)
    if not us:
        return None
    mid = len(us) // 2
    med = us[mid] if len(us) % 2 else 0.5 * (us[mid - 1] + us[mid])
    # time the GPU ran no kernel at all between the first and the last timed
    # launch (kernels of one stream, one after another), per launch
    t0, t1 = int(timed[0]["Start_Timestamp"]), int(timed[-1]["End_Timestamp"])
    busy = sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in every
               if int(r["Start_Timestamp"]) >= t0 and int(r["End_Timestamp"]) <= t1)
    idle = max(0.0, (t1 - t0 - busy) / 1e3 / max(1, len(timed) - 1))
    return {"n": len(us), "mean_us": sum(us) / len(us), "median_us": med, "gap_us": idle,
            "bench_ms_per_step_us": rec["ms_per_step"] * 1e3}


def steady_md(st):
    if st is None:
        return ""
    return (f"\nSteady state: the {st['n']} timed launches alone (from `run_kernel_trace.csv`, the clock-settle, "
            f"warm-up and\nafter-loop launches left out) average {st['mean_us']:.2f} us, median {st['median_us']:.2f} us, "
            f"against the bench's\n{st['bench_ms_per_step_us']:.3f} us per step "
            f"({100 * (st['mean_us'] / st['bench_ms_per_step_us'] - 1):+.2f}%; the events also time any other kernels "
            f"of a step and the gaps between\nlaunches; the GPU ran no kernel for {st.get('gap_us', 0.0):.2f} us per "
            f"launch here).\n"
            + ("\nThose idle gaps are longer than a tenth of the kernel: the next launch had not reached the GPU when "
               "this one\nended, so the bench's events time the launch rate under the tracer, and the kernel durations "
               "above are\nthe kernel's own.\n" if st.get("gap_us", 0.0) > 0.1 * st["mean_us"] else ""))


def warm(W, G):
    import workloads
    import bench
    fk, nk = agg(f'{G}/prof_FETCH_SIZE_{W}/run_counter_collection.csv')
    wk, _ = agg(f'{G}/prof_WRITE_SIZE_{W}/run_counter_collection.csv')
    fc, _ = agg(f'{G}/prof_FETCH_SIZE_copy256/run_counter_collection.csv', 'copyBuffer')
    wc, _ = agg(f'{G}/prof_WRITE_SIZE_copy256/run_counter_collection.csv', 'copyBuffer')
    copy_kib = 256 * 1024
    ffac = fc['FETCH_SIZE'] / copy_kib
    wfac = wc['WRITE_SIZE'] / copy_kib
    fetch_b = fk['FETCH_SIZE'] * 1024 / ffac
    write_b = wk['WRITE_SIZE'] * 1024 / wfac
    log = open(f'{G}/prof_trace_{W}.log').read().splitlines()
    rec = json.loads([l for l in log if l.startswith('{')][-1])
    src_hash = rec['kernel_source_hash']
    w = workloads.get(W)
    minb = workloads.min_bytes(w)
    stats = list(csv.DictReader(open(f'{G}/prof_trace_{W}/run_kernel_stats.csv')))
    kname = [r for r in stats if is_forward(r['Name'])][0]
    out = {
        "workload": W, "kernel": kname['Name'], "kernel_source_hash": src_hash,
        "fetch_size_kib_per_dispatch": round(fk['FETCH_SIZE'], 2), "write_size_kib_per_dispatch": round(wk['WRITE_SIZE'], 2),
        "copy_calibration": {"bytes_read": copy_kib * 1024, "bytes_written": copy_kib * 1024,
                              "fetch_size_kib": round(fc['FETCH_SIZE'], 2), "write_size_kib": round(wc['WRITE_SIZE'], 2),
                              "fetch_factor": round(ffac, 5), "write_factor": round(wfac, 5)},
        "hbm_bytes_per_launch": int(round(fetch_b + write_b)),
        "hbm_read_bytes_per_launch": int(round(fetch_b)), "hbm_write_bytes_per_launch": int(round(write_b)),
        "min_bytes": minb, "ratio_to_min": round((fetch_b + write_b) / minb, 4),
    }
    P = OUT
    os.makedirs(P, exist_ok=True)
    json.dump(out, open(f'{P}/traffic_{W}.json', 'w'), indent=1)
    cmd_pmc = f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {G}/prof_FETCH_SIZE_{W} -o run -- python -u bench.py --workload {W} --steps 20 --warmup 5 --no-cpu-baseline --no-check"
    md = f"""# HBM bytes of the forward kernel: {W}

Kernel `{kname['Name']}` (kernel source hash `{src_hash}` over the source files of the workload's kernel with comments removed, as `bench.py` computes it).

Commands (run from the repository root on one MI355X, each pass its own process):

    {cmd_pmc}
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d {G}/prof_WRITE_SIZE_{W} -o run -- python -u bench.py --workload {W} --steps 20 --warmup 5 --no-cpu-baseline --no-check
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d {G}/prof_FETCH_SIZE_copy256 -o run -- python -u bench.py --copy-calibration-mib 256 --steps 10 --warmup 2
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d {G}/prof_WRITE_SIZE_copy256 -o run -- python -u bench.py --copy-calibration-mib 256 --steps 10 --warmup 2

| quantity | value |
|---|---|
| FETCH_SIZE per dispatch (mean of {nk['FETCH_SIZE']}) | {fk['FETCH_SIZE']:.1f} KiB |
| WRITE_SIZE per dispatch | {wk['WRITE_SIZE']:.1f} KiB |
| plain 256 MiB device copy (`__amd_rocclr_copyBuffer`): FETCH_SIZE | {fc['FETCH_SIZE']:.1f} KiB (factor {ffac:.4f} of the bytes read) |
| same copy: WRITE_SIZE | {wc['WRITE_SIZE']:.1f} KiB (factor {wfac:.4f} of the bytes written) |
| HBM read per launch (FETCH_SIZE / factor) | {fetch_b/1e6:.2f} MB |
| HBM write per launch (WRITE_SIZE / factor) | {write_b/1e6:.2f} MB |
| total | {(fetch_b+write_b)/1e6:.2f} MB |
| minimum Q+K+V+O | {minb/1e6:.2f} MB |
| ratio | {(fetch_b+write_b)/minb:.3f} |

The counters measure L2-to-memory traffic, an upper bound on HBM bytes (reads served by the
Infinity Cache count too).  K and V are read by every query block of a head; the re-reads that the
XCD's L2 serves do not reach these counters, so the ratio shows how much of that re-reading L2 absorbs.
"""
    by = f"\nSummary written by `python -m tiled_attention_fa_amd.profile_report warm --workload {W} --dir {G}`.\n"
    open(f'{P}/fa_forward_{W}_hbm_bytes.md', 'w').write(md + by)
    cmd_tr = f"rocprofv3 --kernel-trace --stats --output-format csv -d {G}/prof_trace_{W} -o run -- python -u bench.py --workload {W} --steps 100 --warmup 20 --no-cpu-baseline"
    rows = '\n'.join(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs'])/1e3:.2f} | {float(r['MinNs'])/1e3:.2f} | {float(r['MaxNs'])/1e3:.2f} | {r['Percentage']} |" for r in stats)
    md2 = f"""# Kernel trace of the benchmark: {W}

Command (repository root, one MI355X):

    {cmd_tr}

`run_kernel_stats.csv` (durations in microseconds; the calls include the clock-settle and warm-up launches and the
one launch the binding makes before the timed loop):

| kernel | calls | average | min | max | % time |
|---|---|---|---|---|---|
{rows}

The JSON line `bench.py` printed in the same run: value {rec['value']} TFLOP/s, mean launch
{rec['roofline']['kernel_us_mean']} us (HIP events around {rec['steps']} back-to-back launches),
against the trace's average of {float(kname['AverageNs'])/1e3:.2f} us for the forward kernel.
{steady_md(steady(f'{G}/prof_trace_{W}/run_kernel_trace.csv', rec))}"""
    open(f'{P}/fa_forward_{W}_kernel_trace.md', 'w').write(md2 + by)
    print(json.dumps(out, indent=1))

    # ---- three-pass comparison path: sum of its three kernels per call
    if w.dtype != 'f32':
        names = ['naive13scores_kernel', 'naive14softmax_kernel', 'naive9pv_kernel', 'naive19softmax_long_kernel']
        def agg_sum(path, counter):
            per = collections.defaultdict(list)
            for r in csv.DictReader(open(path)):
                kn = r['Kernel_Name']
                if 'naive' in kn and r['Counter_Name'] == counter:
                    per[kn].append(float(r['Counter_Value']))
            return {k: (sum(v) / len(v), len(v)) for k, v in per.items()}
        nf = agg_sum(f'{G}/prof_FETCH_SIZE_{W}/run_counter_collection.csv', 'FETCH_SIZE')
        nw = agg_sum(f'{G}/prof_WRITE_SIZE_{W}/run_counter_collection.csv', 'WRITE_SIZE')
        if nf:
            kinds = sorted(nf)
            f_b = sum(nf[k][0] for k in kinds) * 1024 / ffac
            w_b = sum(nw[k][0] for k in kinds) * 1024 / wfac
            nb = workloads.naive_bytes(w)
            nhash = bench.kernel_source_hash(w.dtype, bench.NAIVE_SOURCES[w.dtype])
            nout = {"workload": W, "path": "three-pass (fa_naive_forward)", "kernels": kinds,
                    "kernel_source_hash": nhash,
                    "per_kernel_kib": {k: {"fetch": round(nf[k][0], 1), "write": round(nw[k][0], 1), "dispatches": nf[k][1]} for k in kinds},
                    "hbm_bytes_per_launch": int(round(f_b + w_b)),
                    "hbm_read_bytes_per_launch": int(round(f_b)), "hbm_write_bytes_per_launch": int(round(w_b)),
                    "algorithmic_bytes": nb, "ratio_to_algorithmic": round((f_b + w_b) / nb, 4),
                    "ratio_to_tiled_measured": round((f_b + w_b) / (fetch_b + write_b), 2)}
            json.dump(nout, open(f'{P}/traffic_naive_{W}.json', 'w'), indent=1)
            krows = '\n'.join(f"| `{k[:80]}` | {nf[k][0]:.1f} | {nw[k][0]:.1f} | {nf[k][0]*1024/ffac/1e6:.1f} | {nw[k][0]*1024/wfac/1e6:.1f} |" for k in kinds)
            md3 = f"""# HBM bytes of the three-pass path: {W}

The three kernels of `fa_naive_forward` (scores, softmax, P V), per call, from the same two counter runs as
`fa_forward_{W}_hbm_bytes.md` (the bench runs the three-pass path after the tiled one) and the same copy calibration.
Kernel source hash `{nhash}` over the three-pass sources with comments removed, as `bench.py` computes it.

Commands (repository root, one MI355X, each pass its own process):

    {cmd_pmc}
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d {G}/prof_WRITE_SIZE_{W} -o run -- python -u bench.py --workload {W} --steps 20 --warmup 5 --no-cpu-baseline --no-check

| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB | written MB |
|---|---|---|---|---|
{krows}

| quantity | value |
|---|---|
| HBM bytes per call (read + written) | {(f_b+w_b)/1e6:.1f} MB |
| algorithmic bytes (`workloads.naive_bytes`) | {nb/1e6:.1f} MB |
| ratio | {(f_b+w_b)/nb:.3f} |
| tiled pass, measured | {(fetch_b+write_b)/1e6:.2f} MB |
| three-pass / tiled, measured | {(f_b+w_b)/(fetch_b+write_b):.1f} |
"""
            open(f'{P}/fa_naive_{W}_hbm_bytes.md', 'w').write(md3 + by)
            print(json.dumps(nout, indent=1))



def cold(W, G):
    import bench
    import workloads
    f, nf = agg(f'{G}/prof_FETCH_SIZE_cold_{W}/run_counter_collection.csv')
    wr, nw = agg(f'{G}/prof_WRITE_SIZE_cold_{W}/run_counter_collection.csv')
    P = OUT
    warm = json.load(open(f'{P}/traffic_{W}.json'))
    cal = warm['copy_calibration']
    fb = f['FETCH_SIZE'] * 1024 / cal['fetch_factor']
    wb = wr['WRITE_SIZE'] * 1024 / cal['write_factor']
    w = workloads.get(W)
    rec = json.loads([l for l in open(f'{G}/cold_bench_{W}.log') if l.startswith('{')][-1])
    warm_rec = json.loads([l for l in open(f'{G}/prof_trace_{W}.log') if l.startswith('{')][-1])
    warm_us = warm_rec['ms_per_step'] * 1e3
    longer = 100 * (rec['ms_per_step'] * 1e3 / warm_us - 1)
    out = {"workload": W, "cache": "cold: 512 MiB written before every launch (L2 and the 256 MB Infinity Cache evicted)",
           "kernel": warm['kernel'], "kernel_source_hash": bench.kernel_source_hash(w.dtype),
           "fetch_size_kib_per_dispatch": round(f['FETCH_SIZE'], 2), "write_size_kib_per_dispatch": round(wr['WRITE_SIZE'], 2),
           "dispatches": {"fetch": nf['FETCH_SIZE'], "write": nw['WRITE_SIZE']},
           "copy_calibration": cal, "hbm_bytes_per_launch": int(round(fb + wb)),
           "hbm_read_bytes_per_launch": int(round(fb)), "hbm_write_bytes_per_launch": int(round(wb)),
           "min_bytes": workloads.min_bytes(w), "ratio_to_min": round((fb + wb) / workloads.min_bytes(w), 4),
           "cold_median_launch_us": round(rec['ms_per_step'] * 1e3, 3), "cold_tflops": rec['value']}
    json.dump(out, open(f'{P}/traffic_cold_{W}.json', 'w'), indent=1)
    B = f"python -u bench.py --workload {W} --cold-flush-mib 512 --steps 20 --warmup 5 --settle-s 0.05 --no-cpu-baseline --no-check"
    md = f"""# HBM bytes of the forward kernel with cold caches: {W}

Kernel `{warm['kernel']}` (kernel source hash `{out['kernel_source_hash']}`).  In cold mode `bench.py` writes a
512 MiB buffer before every launch of the forward kernel (settle, warm-up and timed launches alike), which evicts L2
and the 256 MB Infinity Cache, and times each launch between its own pair of events.

Commands (repository root, one MI355X, each pass its own process):

    python -u bench.py --workload {W} --cold-flush-mib 512 --steps 100 --warmup 10 --no-cpu-baseline
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d {G}/prof_FETCH_SIZE_cold_{W} -o run -- {B}
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d {G}/prof_WRITE_SIZE_cold_{W} -o run -- {B}

| | cold | warm (back-to-back launches) |
|---|---|---|
| `FETCH_SIZE` per dispatch (KiB) | {f['FETCH_SIZE']:,.1f} (over {nf['FETCH_SIZE']} dispatches) | {warm['fetch_size_kib_per_dispatch']:,.1f} |
| `WRITE_SIZE` per dispatch (KiB) | {wr['WRITE_SIZE']:,.1f} | {warm['write_size_kib_per_dispatch']:,.1f} |
| HBM bytes per launch (copy-calibrated: fetch x {1 / cal['fetch_factor']:.3f}, write x {1 / cal['write_factor']:.3f}) | {fb + wb:,.0f} | {warm['hbm_bytes_per_launch']:,} |
| ratio to the Q+K+V+O minimum ({workloads.min_bytes(w):,} B) | {(fb + wb) / workloads.min_bytes(w):.4f} | {warm['ratio_to_min']} |
| launch time | {rec['ms_per_step'] * 1e3:.2f} us (median of 100) | {warm_us:.2f} us (mean of back-to-back launches, `prof_trace_{W}`) |

The counters measure L2 egress (requests to the Infinity Fabric, whether the Infinity Cache or DRAM serves them), and
they read the same with cold and warm caches: the 24 MiB of inputs do not survive in L2 from one launch to the next
even when warm.  The difference is where the misses are served: with cold caches every byte comes from DRAM, and the
launch takes {longer:.0f}% longer.
"""
    by = f"\nSummary written by `python -m tiled_attention_fa_amd.profile_report cold --workload {W} --dir {G}`.\n"
    open(f'{P}/fa_forward_{W}_hbm_bytes_cold.md', 'w').write(md + by)
    print(md)



def trace(W, G, run, suffix, out="", note="", title="", bench_args=""):
    """Kernel-trace summary of one `bench.py --workload W` run under
    `rocprofv3 --kernel-trace --stats -d G/run`, its output in G/run.log."""
    stats = list(csv.DictReader(open(f"{G}/{run}/run_kernel_stats.csv")))
    rec = json.loads([l for l in open(f"{G}/{run}.log") if l.startswith("{")][-1])
    fwd = [r for r in stats if is_forward(r["Name"])][0]
    args = bench_args or f"--workload {W} --steps {rec['steps']} --warmup {rec['warmup']} --no-cpu-baseline"
    cmd = f"rocprofv3 --kernel-trace --stats --output-format csv -d {G}/{run} -o run -- python -u bench.py {args}"
    rows = "\n".join(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.4g} |"
                     for r in stats[:6])
    head = f"# {title}" if title else f"# Kernel trace of the benchmark: {W}"
    note_md = f"\n{note}\n" if note else ""
    md = f"""{head}
{note_md}
Command (repository root, one MI355X):

    {cmd}

`run_kernel_stats.csv` (durations in microseconds; the calls include the clock-settle and warm-up launches). The
forward kernel's template arguments end with the waves per workgroup, the waves_per_eu hint and the key groups.

| kernel | calls | average | min | max | % time |
|---|---|---|---|---|---|
{rows}

The JSON line `bench.py` printed in the same run: value {rec['value']} TFLOP/s, mean launch
{rec['ms_per_step'] * 1e3:.3f} us (HIP events around {rec['steps']} back-to-back launches), against the trace's average of
{float(fwd['AverageNs']) / 1e3:.2f} us for the forward kernel.
{steady_md(steady(f"{G}/{run}/run_kernel_trace.csv", rec))}
Summary written by `python -m tiled_attention_fa_amd.profile_report trace --workload {W} --dir {G} --run {run}` with
the title, note and file name given.
"""
    name = out or f"fa_forward_{W}{suffix}_kernel_trace.md"
    open(os.path.join(OUT, name), "w").write(md)


def sq(W, G, pre):
    """SQ counters of the forward kernel from the four counter passes
    G/<pre>_A .. G/<pre>_D (each its own rocprofv3 --pmc run of the bench)."""
    import glob
    vals = collections.defaultdict(list)
    kname = ""
    for f in sorted(glob.glob(f"{G}/{pre}_*/run_counter_collection.csv")):
        for r in csv.DictReader(open(f)):
            if is_forward(r["Kernel_Name"]):
                vals[r["Counter_Name"]].append(float(r["Counter_Value"]))
                kname = r["Kernel_Name"]
    m = {k: sum(v) / len(v) for k, v in vals.items()}
    B = f"python -u bench.py --workload {W} --steps 20 --warmup 5 --no-cpu-baseline --no-check --no-naive"
    passes = {
        "A": "SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS "
             "SQ_WAIT_INST_LDS SQ_WAIT_ANY",
        "B": "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_VALU_TRANS_F32 "
             "SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_SALU",
        "C": "GRBM_GUI_ACTIVE SQ_CYCLES SQ_INST_LEVEL_LDS SQ_ACTIVE_INST_ANY SQ_THREAD_CYCLES_VALU SQ_LDS_DATA_FIFO_FULL "
             "SQ_WAIT_INST_ANY SQ_ACTIVE_INST_MISC",
        "D": "SQ_ACTIVE_INST_SCA SQ_LDS_ADDR_CONFLICT SQ_LDS_UNALIGNED_STALL SQ_LDS_CMD_FIFO_FULL SQ_INST_CYCLES_SALU "
             "SQ_ACTIVE_INST_FLAT SQ_INSTS_BRANCH SQ_ACTIVE_INST_VMEM",
    }
    import workloads
    w = workloads.get(W)
    waves = m["SQ_WAVES"]
    simds = 1024
    # 64-key tiles per wave, averaged over the waves of the workload's grid:
    # N / 64 without the mask; with it, a wave of rows q0 .. q0 + 31 sees the
    # tiles up to its diagonal
    if w.causal:
        per_head = [-(-(q0 + 32) // 64) for q0 in range(0, w.N, 32)]
        tiles = sum(per_head) / len(per_head)
    else:
        tiles = -(-w.N // 64)
    life = m["SQ_WAVE_CYCLES"] * 4 / waves
    mfma = m["SQ_VALU_MFMA_BUSY_CYCLES"] / simds
    valu = m["SQ_ACTIVE_INST_VALU"] * 4 / simds
    coex = m["SQ_VALU_MFMA_COEXEC_CYCLES"] / simds
    span = m["GRBM_GUI_ACTIVE"] / 8

    def per_wave_tile(k):
        return m[k] / waves / tiles

    lines = [f"# SQ counters of the forward kernel: {W}", "",
             f"Kernel `{kname}` ({waves:,.0f} waves of 32 query rows, {tiles:.1f} key tiles of 64 per wave on "
             "average).  Four counter",
             "passes, each its own process (repository root, one MI355X):", ""]
    for k, c in passes.items():
        lines.append(f"    rocprofv3 --pmc {c} --output-format csv -d {G}/{pre}_{k} -o run -- {B}")
    lines += ["", "Mean per dispatch over the ~2000 dispatches of each pass:", "", "| counter | value |", "|---|---|"]
    for k in sorted(m):
        lines.append(f"| `{k}` | {m[k]:,.0f} |")
    lines += ["", "Derived (MI355X: 256 CUs x 4 SIMDs = 1024 SIMDs; SQ cycle counters in units of 4 "
              "cycles; one", "MFMA 32x32x16 counts 32 busy cycles):", "", "| quantity | value |", "|---|---|",
              f"| wave lifetime (SQ_WAVE_CYCLES x 4 / waves) | {life:,.0f} cycles (~{life / 2.0e3:.1f} us at 2.0 GHz) |",
              f"| dispatch span per XCD (GRBM_GUI_ACTIVE / 8 XCDs) | {span:,.0f} cycles |",
              f"| waves resident per SIMD, averaged over the span (SQ_WAVE_CYCLES x 4 / 1024 / span) | "
              f"{m['SQ_WAVE_CYCLES'] * 4 / simds / span:.2f} |",
              f"| matrix-core busy per SIMD (SQ_VALU_MFMA_BUSY_CYCLES / 1024), against the span | "
              f"{mfma:,.0f} cycles = {100 * mfma / span:.0f}% |",
              f"| VALU issue per SIMD, MFMA included (SQ_ACTIVE_INST_VALU x 4 / 1024), against the span | "
              f"{valu:,.0f} cycles = {100 * valu / span:.0f}% |",
              f"| VALU and MFMA together (SQ_VALU_MFMA_COEXEC_CYCLES / 1024) | {coex:,.0f} cycles = "
              f"{100 * coex / mfma:.0f}% of the MFMA-busy time |",
              f"| VALU instructions per wave per 64-key tile (MFMA included) | {per_wave_tile('SQ_INSTS_VALU'):.0f} "
              f"(transcendental: {per_wave_tile('SQ_INSTS_VALU_TRANS_F32'):.1f}) |",
              f"| MFMA instructions per wave per tile | {per_wave_tile('SQ_INSTS_MFMA'):.0f} |",
              f"| LDS instructions per wave per tile | {per_wave_tile('SQ_INSTS_LDS'):.1f} |",
              f"| scalar instructions per wave per tile | {per_wave_tile('SQ_INSTS_SALU'):.1f} |",
              f"| LDS bank conflicts | {m['SQ_LDS_BANK_CONFLICT']:.0f} cycles |", ""]
    lines += ["Under counter collection the dispatches are serialised, but each wave's lifetime is that of the "
              "timed kernel,", "so the per-wave figures describe the kernel as it runs.  SQ_ACTIVE_INST_VALU counts "
              "each MFMA for its busy", "cycles.  Matrix-core busy against the dispatch span is the figure the "
              "roofline fraction follows.", "",
              f"Summary written by `python -m tiled_attention_fa_amd.profile_report sq --workload {W} --dir {G} "
              f"--run {pre}`.", ""]
    open(os.path.join(OUT, f"fa_forward_{W}_sq_counters.md"), "w").write("\n".join(lines))


def requests(G, names):
    """HBM request counts by size (TCC_EA0_RDREQ / _32B, TCC_BUBBLE; TCC_EA0_WRREQ / _64B; the DRAM-bound
    ones) for the forward kernel of each workload and for the 256 MiB copy, from three counter passes each
    (G/req1_<name> .. G/req3_<name>), written to profiles/hbm_request_sizes_mi355x.md."""
    import workloads
    passes = ["TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_32B_sum TCC_BUBBLE_sum", "TCC_EA0_WRREQ_sum TCC_EA0_WRREQ_64B_sum",
              "TCC_EA0_RDREQ_DRAM_sum TCC_EA0_WRREQ_DRAM_sum"]
    rows = []
    for name in names + ["copy256"]:
        vals = collections.defaultdict(list)
        for i in (1, 2, 3):
            for r in csv.DictReader(open(f"{G}/req{i}_{name}/run_counter_collection.csv")):
                kn = r["Kernel_Name"]
                if (name == "copy256" and "copyBuffer" in kn) or (name != "copy256" and is_forward(kn)):
                    vals[r["Counter_Name"]].append(float(r["Counter_Value"]))
        # the copy: its largest dispatch is the 256 MiB copy itself
        m = {k: (max(v) if name == "copy256" else sum(v) / len(v)) for k, v in vals.items()}
        if name == "copy256":
            rmin, wmin = 256 << 20, 256 << 20
        else:
            w = workloads.get(name)
            wmin = w.B * w.H * w.N * w.D * workloads.storage_itemsize(w.dtype)
            rmin = 3 * wmin
        rows.append((name, m, rmin, wmin))
    lines = ["# HBM requests by size on MI355X", "",
             "`FETCH_SIZE` on this ROCm is (TCC_BUBBLE x 128 + (TCC_EA0_RDREQ - TCC_BUBBLE - TCC_EA0_RDREQ_32B) x 64 +",
             "TCC_EA0_RDREQ_32B x 32) / 1024 and `WRITE_SIZE` ((TCC_EA0_WRREQ - TCC_EA0_WRREQ_64B) x 32 + TCC_EA0_WRREQ_64B x 64)",
             "/ 1024 (`rocprofv3 --list-avail`).  The request counters themselves, per dispatch (the workloads: mean over",
             "the dispatches of their forward kernel; the copy: its 256 MiB dispatch), three passes each, each its own process:",
             ""]
    for i, P in enumerate(passes, 1):
        lines.append(f"    rocprofv3 --pmc {P} --output-format csv -d {G}/req{i}_<name> -o run -- <bench command>")
    lines += ["", "with `<bench command>` = `python -u bench.py --workload <name> --steps 20 --warmup 5 --no-cpu-baseline "
              "--no-check --no-naive`, or `python -u bench.py --copy-calibration-mib 256 --steps 10 --warmup 2` for the copy.",
              "", "| dispatch | RDREQ | RDREQ_32B | BUBBLE (128 B) | RDREQ x 128 B | reads, minimum | WRREQ | WRREQ_64B | "
              "WRREQ_64B x 64 B | writes, minimum | RDREQ_DRAM / RDREQ |", "|---|---|---|---|---|---|---|---|---|---|---|"]
    for name, m, rmin, wmin in rows:
        rd, r32, bub = m["TCC_EA0_RDREQ_sum"], m["TCC_EA0_RDREQ_32B_sum"], m["TCC_BUBBLE_sum"]
        wr, w64, rdd = m["TCC_EA0_WRREQ_sum"], m["TCC_EA0_WRREQ_64B_sum"], m["TCC_EA0_RDREQ_DRAM_sum"]
        lines.append(f"| `{name}` | {rd:,.0f} | {r32:,.0f} | {bub:,.0f} | {rd * 128:,.0f} ({rd * 128 / rmin:.4f}x) | "
                     f"{rmin:,} | {wr:,.0f} | {w64:,.0f} | {w64 * 64:,.0f} ({w64 * 64 / wmin:.4f}x) | {wmin:,} | "
                     f"{rdd / rd:.4f} |")
    lines += ["", "Every read request is 128 bytes: no 32-byte requests, and the copy's read requests times 128 B are its",
              "256 MiB exactly, while TCC_BUBBLE, which the expression relies on to count the 128-byte requests, reads 0.",
              "So `FETCH_SIZE` counts each 128-byte request as 64 bytes, and the factor 2 that the copy calibration applies to",
              "it is that request size.  Every write request is 64 bytes and `WRITE_SIZE` needs no factor.  The DRAM-bound",
              "counter equals the total on every kernel, so it does not separate Infinity Cache hits from DRAM reads.", "",
              f"Summary written by `python -m tiled_attention_fa_amd.profile_report requests --dir {G} --workload "
              f"{','.join(names)}`.", ""]
    open(os.path.join(OUT, "hbm_request_sizes_mi355x.md"), "w").write("\n".join(lines))
    print("\n".join(lines))


def pages(G):
    """The second page's comparison table ("Flash Attention on Android: tiled
    SGEMM with RenderScript", section "Benchmark results: Snapdragon vs.
    Dimensity": 32 heads, D = 128, N = 512 and 1024, peak memory bandwidth of a
    naive pass against the tiled one) on MI355X, from the kernel-trace bench
    runs of the page-table workloads (G/prof_trace_W.log) and their committed
    traffic files."""
    import workloads
    rows = []
    for W in workloads.PAGE_TABLE:
        rec = json.loads([l for l in open(f"{G}/prof_trace_{W}.log") if l.startswith("{")][-1])
        n = rec["naive_three_pass"]
        t = json.load(open(os.path.join(OUT, f"traffic_{W}.json")))
        tn = json.load(open(os.path.join(OUT, f"traffic_naive_{W}.json")))
        w = workloads.get(W)
        t_us, n_us = rec["ms_per_step"] * 1e3, n["ms_per_call"] * 1e3
        tb, nb = t["hbm_bytes_per_launch"], tn["hbm_bytes_per_launch"]
        rows.append((w, t_us, rec["median_single_launch_us"], n_us, n["median_single_call_us"], tb, nb))
    lines = ["# Tiled against three-pass attention at the second page's shapes (MI355X)", "",
             "The page's table compares the peak memory bandwidth of a naive FP32 attention with its tiled pass on two",
             "phones, 32 heads, head dimension 128, sequence lengths 512 and 1024 (\"Flash Attention on Android: tiled",
             "SGEMM with RenderScript\", section \"Benchmark results: Snapdragon vs. Dimensity\"; the median of 20",
             "sustained runs, read and write bytes from the vendors' profiler counters).  Here the same shapes run at fp16",
             "storage (the three-pass path takes 16-bit storage; its S is fp32 either way and its P takes 2 bytes where",
             "FP32 would take 4, so these three-pass bytes understate an FP32 baseline's).  Bytes per call are the",
             "copy-calibrated FETCH_SIZE + WRITE_SIZE counters of each path's kernels; time is the mean of back-to-back",
             "calls (sustained) and, beside it, the median of individually timed calls (each after a synchronisation,",
             "so it includes launch latency and a clock that has dropped while idle).", "",
             "| N | path | bytes per call | of which the n x n matrices | us per call (sustained) | median single call (us) | "
             "achieved GB/s (sustained) |",
             "|---|---|---|---|---|---|---|"]
    for w, t_us, t_med, n_us, n_med, tb, nb in rows:
        extra = nb - workloads.min_bytes(w)
        lines.append(f"| {w.N} | tiled (`fa_forward`) | {tb / 1e6:.1f} MB | 0 | {t_us:.2f} | {t_med:.2f} | "
                     f"{tb / (t_us * 1e-6) / 1e9:,.0f} |")
        lines.append(f"| {w.N} | three-pass (`fa_naive_forward`) | {nb / 1e6:.1f} MB | {extra / 1e6:.1f} MB | "
                     f"{n_us:.2f} | {n_med:.2f} | {nb / (n_us * 1e-6) / 1e9:,.0f} |")
    lines += ["", "| N | bytes: three-pass / tiled | time: three-pass / tiled | bandwidth the tiled pass draws, "
              "against the three-pass one | the page's reduction (phones) |", "|---|---|---|---|---|"]
    page = {512: "38.4 -> 23.1 GB/s (-40%), 35.1 -> 21.4 GB/s (-39%)",
            1024: "61.7 -> 29.6 GB/s (-52%), 57.8 -> 26.0 GB/s (-55%)"}
    for w, t_us, t_med, n_us, n_med, tb, nb in rows:
        bw_t, bw_n = tb / (t_us * 1e-6), nb / (n_us * 1e-6)
        lines.append(f"| {w.N} | {nb / tb:.1f}x | {n_us / t_us:.2f}x | {100 * (1 - bw_t / bw_n):.0f}% lower | "
                     f"{page.get(w.N, '-')} |")
    lines += ["", "On the phones the two passes take similar times and the page reports the drop in bandwidth.  Here the",
              "tiled pass also finishes several times sooner, so its bandwidth drop understates what it saves: the",
              "bytes fall by the ratio in the second column.  The per-path summaries and counters are in",
              "`fa_forward_<workload>_hbm_bytes.md` and `fa_naive_<workload>_hbm_bytes.md`.", "",
              f"Written by `python -m tiled_attention_fa_amd.profile_report pages --dir {G}` from the runs those "
              "summaries list.", ""]
    open(os.path.join(OUT, "page_table_comparison_mi355x.md"), "w").write("\n".join(lines))
    print("\n".join(lines))


def main():
    global OUT
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("kind", choices=["warm", "cold", "trace", "sq", "pages", "requests"])
    ap.add_argument("--workload", default="prefill_b1h32n2048d64_f16")
    ap.add_argument("--dir", required=True, help="the directory the rocprofv3 runs wrote to")
    ap.add_argument("--run", default="", help="trace: the run's rocprofv3 -d name under --dir")
    ap.add_argument("--suffix", default="", help="trace: text appended to the workload in the file name")
    ap.add_argument("--out", default="", help="trace: file name under profiles/ (instead of the suffix rule)")
    ap.add_argument("--title", default="", help="trace: heading")
    ap.add_argument("--note", default="", help="trace: paragraph under the heading")
    ap.add_argument("--bench-args", default="", help="trace: the bench.py arguments of the traced run")
    ap.add_argument("--out-dir", default=OUT, help="where the JSON and Markdown files go (default: profiles/)")
    args = ap.parse_args()
    OUT = args.out_dir
    sys.path.insert(0, ROOT)
    G = args.dir.rstrip("/")
    if args.kind == "pages":
        pages(G)
    elif args.kind == "trace":
        trace(args.workload, G, args.run or f"prof_trace_{args.workload}", args.suffix, args.out, args.note, args.title,
              args.bench_args)
    elif args.kind == "sq":
        sq(args.workload, G, args.run or "pmc")
    elif args.kind == "requests":
        requests(G, args.workload.split(","))
    else:
        (warm if args.kind == "warm" else cold)(args.workload, G)


if __name__ == "__main__":
    main()
