#!/usr/bin/env python
"""Benchmark of the NVFP4 linear-layer path on one MI355X.

One step = one linear-layer pass over the three layer workloads, all inputs
resident in HBM before timing starts:
  fprop  Y  = X W^T  : quantize X [4096x5120] and W [5120x5120] (RNE, axis 1),
                       NVFP4 GEMM -> bf16 [4096x5120]
  dgrad  dX = dY W   : quantize dY [8192x20480] (Philox SR, axis 1) and
                       W [20480x5120] (RNE, axis 0), GEMM -> f32 [8192x5120]
  wgrad  dW = X^T dY : RHT-quantize X [8192x5120] (RNE, axis 0) and
                       dY [8192x20480] (SR, axis 0), GEMM -> f32 [5120x20480]
dY's two quantizations run as one dual-layout call (one amax read for both);
W's axis-0 and X's axis-0 RHT quantizations (the backward operands of
forward-time tensors) run on a second stream beside the fprop GEMM.
value = GEMM FLOP of the step / step time (quantization included), TFLOP/s,
timed over K steps that record events only at each step's start and around
the wgrad launch; the per-op breakdown comes from K more steps with an event
after every op.
Also reported: quantizer GB/s per operand and on the 32768x8192 sweep tensor
(RNE/SR x RHT off/on) and its dequantize to bf16 and f32, the fprop operands'
quantization warm and after a 512 MiB cache flush, per-GEMM TFLOP/s, the
roofline of the dominant kernel
(the f32-output GEMM that serves dgrad and wgrad), the same products in bf16
and the same step in MXFP4 as context, and the CPU oracle timed on a bounded
sample of the same step.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "NVFP4 quantize GB/s + block-scaled GEMM TFLOPS (fprop/dgrad/wgrad) at 1 GPU"
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, published
PEAK_F16_TFLOPS = 2500.0        # MI355X dense fp16/bf16 MFMA, published
PEAK_FP4_TFLOPS = 10100.0       # MI355X dense fp4 MFMA, published (context)
# The pages' chip-level matmul figures for NVIDIA GB300 (the Thinking Machines
# article, section on the three formats of one training run): context only,
# another machine's numbers, dense or sparse not stated.
PAGES_CONTEXT = {"platform": "NVIDIA GB300", "nvfp4_PFLOP/s": 15.0, "mxfp8_PFLOP/s": 5.0, "bf16_PFLOP/s": 2.5,
                 "nvfp4_over_bf16": 6.0, "note": "chip-level figures quoted by the pages; not targets"}


def qbytes(n_elem: int, in_bytes: int) -> int:
    """Algorithmic HBM bytes of one quantization: the input is read twice
    (amax pass, encode pass), codes (0.5 B) and scales (1/16 B) written."""
    return n_elem * (2 * in_bytes) + n_elem // 2 + n_elem // 16


def qbytes_dual(n_elem: int, in_bytes: int) -> int:
    """Algorithmic HBM bytes of a dual-layout quantization: the input is read
    twice (the amax pass, then one encode pass that writes both layouts), two
    sets of codes and scales written."""
    return n_elem * (2 * in_bytes) + 2 * (n_elem // 2 + n_elem // 16)


def gemm_bytes(g) -> int:
    """Algorithmic HBM bytes of one NVFP4 GEMM: both operands' codes (1/2 B)
    and block scales (1/16 B) read once, the output written once."""
    m, n, k = g.mnk
    return (m + n) * k * 9 // 16 + m * n * (4 if g.out == "f32" else 2)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# HBM traffic of the dominant kernel comes from two rocprofv3 counter runs of
# this script (FETCH_SIZE, then WRITE_SIZE), reduced by `--traffic` into the
# JSON below.  Each counter is scaled by what it reads for a plain device copy
# of known size that every run performs (CALIB_BYTES, outside the timed
# region).  The profile records a hash of the kernel sources; when they have
# changed since, the traffic is reported as null.
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemm_wgrad_5120x20480x8192_traffic.json")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_wgrad_5120x20480x8192_traffic.md")
GEMM_SOURCES = [os.path.join(ROOT, "gemm_amax_reduce_amd", "csrc", f) for f in ("gemm.hip", "gemm_common.h", "nvfp4_device.h")]
CALIB_BYTES = 256 << 20
MI355X_CUS = 256


def gemm_launch(g, cus: int = MI355X_CUS):
    """(kernel name, work-items) of the one launch nvfp4_gemm_ws makes for the
    layer GEMM g: the stream-K kernel (grids of at least one round of 256 x
    256 tiles, not a whole number of rounds, at least 16 K groups per tile),
    all whole rounds but the last data-parallel plus one round of stream-K
    workgroups, 256 threads each.  dgrad and wgrad share the f32-output
    kernel and differ in grid size."""
    m, n, k = g.mnk
    tiles = -(-m // 256) * -(-n // 256)
    ng = -(-k // 256)
    p_sk = min(cus, 256) // 8 * 8
    assert tiles >= p_sk and tiles % p_sk and ng >= 16 and k % 64 == 0, g.name
    n_dp = (tiles // p_sk - 1) * p_sk
    return "k_gemm_nvfp4_sk<%s, true>" % ("true" if g.out == "bf16" else "false"), (n_dp + p_sk) * 256


def gemm_kinds():
    import workloads
    return [(name, gemm_launch(g)) for name, g in (("fprop", workloads.FPROP), ("dgrad", workloads.DGRAD),
                                                   ("wgrad", workloads.WGRAD))]


def dominant_launch():
    """The dominant kernel: the one with the most time per step, wgrad's."""
    return dict(gemm_kinds())["wgrad"]


def gemm_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def load_traffic():
    """Measured HBM bytes per launch of the dominant kernel, or None."""
    try:
        with open(TRAFFIC_PROFILE) as f:
            prof = json.load(f)
    except (OSError, ValueError):
        return None
    if prof.get("source_sha256") != gemm_source_hash():
        return None
    return prof.get("bytes_per_launch")


def reduce_traffic(fetch_dir: str, write_dir: str) -> dict:
    """Average per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the dominant
    kernel and of the calibration copy from two rocprofv3 --pmc runs; the
    copy's known size gives the scale factor of each counter."""
    import csv
    import glob

    dom_name, dom_grid = dominant_launch()

    def per_kernel(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        out = {}
        for fn in files:
            for r in csv.DictReader(open(fn)):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"]
                dom = dom_name in name and int(r["Grid_Size"]) == dom_grid
                key = "dominant" if dom else "copy" if "copyBuffer" in name else None
                if key:
                    out.setdefault(key, []).append(float(r["Counter_Value"]))
        return out

    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")
    for name, got in (("FETCH_SIZE", fetch), ("WRITE_SIZE", write)):
        if set(got) != {"dominant", "copy"}:
            raise SystemExit(f"--traffic: {name} run lacks {sorted({'dominant', 'copy'} - set(got))} dispatches")
    f_dom = sum(fetch["dominant"]) / len(fetch["dominant"])
    w_dom = sum(write["dominant"]) / len(write["dominant"])
    f_copy = max(fetch["copy"])      # the calibration copy is the largest copy
    w_copy = max(write["copy"])
    f_scale = CALIB_BYTES / (f_copy * 1024.0)
    w_scale = CALIB_BYTES / (w_copy * 1024.0)
    fetch_b = f_dom * 1024.0 * f_scale
    write_b = w_dom * 1024.0 * w_scale
    return {"kernel": dom_name, "grid_work_items": dom_grid, "source_sha256": gemm_source_hash(),
            "fetch_kib_per_dispatch": f_dom, "write_kib_per_dispatch": w_dom,
            "calibration_copy_bytes": CALIB_BYTES, "copy_fetch_kib": f_copy, "copy_write_kib": w_copy,
            "fetch_scale": f_scale, "write_scale": w_scale,
            "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
            "bytes_per_launch": fetch_b + write_b, "dispatches": [len(fetch["dominant"]), len(write["dominant"])]}


QUANT_PROFILE = os.path.join(ROOT, "profiles", "quantizer_sweep_32768x8192_counters.md")
SWEEP_VARIANTS = [(axis, rnd, rht) for axis in (1, 0) for rnd in ("rne", "sr") for rht in (False, True)]
SWEEP_CALLS = 12          # 2 warm-up + 10 timed calls per variant


def _dispatches(d):
    """Per-dispatch rows of a rocprofv3 --pmc run: [(name, grid, start, end, {counter: value})] in order."""
    import csv
    import glob
    disp = {}
    for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(fn)):
            k = int(r["Dispatch_Id"])
            e = disp.setdefault(k, [r["Kernel_Name"], int(r["Grid_Size"]), int(r["Start_Timestamp"]),
                                    int(r["End_Timestamp"]), {}])
            e[4][r["Counter_Name"]] = float(r["Counter_Value"])
    return [disp[k] for k in sorted(disp)]


TRACE_PROFILE = os.path.join(ROOT, "profiles", "linear_layer_step_and_sweep_kernel_trace.md")
def _trace_rows(d):
    """Kernel dispatches of a rocprofv3 --kernel-trace run in start order:
    [(name, work-items, start_ns, end_ns)]."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *kernel_trace.csv under {d}")
    out = []
    for fn in files:
        for r in csv.DictReader(open(fn)):
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            out.append((r["Kernel_Name"], grid, int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    out.sort(key=lambda e: e[2])
    return out


def _sweep_sequence(ds, what):
    """The quantizer sweep's dispatches (meta init, amax, encode per call,
    SWEEP_CALLS calls per variant in SWEEP_VARIANTS order), checked.  The
    spin kernels queued ahead of each variant's timed calls are left out."""
    n = 32768 * 8192
    ds = [e for e in ds if "spin_kernel" not in e[0]]
    first = next(i for i, e in enumerate(ds) if "k_quant_rows<unsigned short, false, false>" in e[0] and e[1] == n // 16)
    seq = ds[first - 2: first - 2 + 3 * SWEEP_CALLS * len(SWEEP_VARIANTS)]
    for v, (axis, rnd, rht) in enumerate(SWEEP_VARIANTS):
        amax = "k_amax_rht_" + ("rows" if axis else "cols") if rht else "k_amax_flat"
        enc = "k_quant_%s<unsigned short, %s, %s>" % ("rows" if axis else "cols", str(rnd == "sr").lower(),
                                                      str(rht).lower())
        for c in range(SWEEP_CALLS):
            trio = seq[3 * (v * SWEEP_CALLS + c): 3 * (v * SWEEP_CALLS + c) + 3]
            if len(trio) < 3 or not ("k_meta_init" in trio[0][0] and amax in trio[1][0] and enc in trio[2][0]):
                raise SystemExit(f"{what}: unexpected dispatch order at variant {v} call {c}")
    return seq


def _short(name: str) -> str:
    import re
    m = re.search(r"(k_\w+(<[^()]*>)?)", name)
    if m and "nvfp4" in name:
        return m.group(1)
    if "Cijk" in name or "gemm" in name.lower() and "nvfp4" not in name:
        return "library GEMM (" + name.split("(")[0][:48] + ")"
    return name.split("(")[0].replace("void ", "")[:70]


def reduce_trace(trace_dir: str, bench_json: str) -> str:
    """The kernel-trace profile of one bench run: per-kernel statistics, the
    GEMM launches of the timed steps against the bench line's own event
    timing, and the quantizer sweep's passes."""
    import csv
    import glob
    with open(bench_json) as f:
        line = [l for l in f.read().splitlines() if l.strip().startswith("{")][-1]
    b = json.loads(line)
    ds = _trace_rows(trace_dir)
    steps, warmup = b["steps"], b["warmup"]
    out = ["# Kernel trace: linear-layer step + 32768x8192 quantizer sweep", "",
           "Commands (repository root, one MI355X): the bench run under the tracer, its JSON line kept, then "
           "the reduction:", "", "```",
           f"rocprofv3 --kernel-trace --stats -d {trace_dir} -o bench --output-format csv -- python3 bench.py "
           f"--steps {steps} --warmup {warmup} --no-cpu-baseline > {bench_json}",
           f"python3 bench.py --trace {trace_dir} {bench_json}", "```", "",
           f"Bench line of this run: value {b['value']} {b['unit']}, {b['ms_per_step']} ms per step "
           f"({steps} timed steps after {warmup} warm-up; the tracer slows the step).", ""]
    # GEMM launches
    out += ["## GEMM launches", "",
            "Each layer GEMM is one `nvfp4_gemm_ws` launch, identified by kernel and grid size. The bench runs "
            f"{warmup} warm-up steps, {steps} timed steps (events only at the step start and around the wgrad "
            f"launch) and {steps} breakdown steps (an event after every op); the columns below average the "
            "timed steps' launches and, separately, the breakdown steps'.", "",
            "| GEMM | kernel | work-items | launches | trace avg of timed ms | min | max | "
            "trace avg of breakdown ms | bench events ms | TFLOP/s (trace, timed) | of 2.5 PF/s |",
            "|---|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    import workloads
    gemms = {"fprop": workloads.FPROP, "dgrad": workloads.DGRAD, "wgrad": workloads.WGRAD}
    bd = b.get("breakdown", {})
    rf = b.get("roofline", {})
    dom = None
    for name, (kern, grid) in gemm_kinds():
        launches = [(e[3] - e[2]) / 1e6 for e in ds if kern in e[0] and e[1] == grid]
        if len(launches) != warmup + 2 * steps:
            raise SystemExit(f"--trace: {len(launches)} launches of {kern} ({grid}), expected "
                             f"{warmup} + 2 x {steps}")
        t = launches[warmup:warmup + steps]
        t_bd = launches[warmup + steps:]
        avg = sum(t) / len(t)
        tf = gemms[name].flops / (avg * 1e-3) / 1e12
        # the timed pass has events around wgrad only; the others' come from the breakdown pass
        ev = rf.get("avg_launch_ms") if name == "wgrad" else bd.get("gemm " + name, {}).get("ms")
        out.append(f"| {name} | `{kern}` | {grid} | {len(launches)} | {avg:.4f} | {min(t):.4f} | {max(t):.4f} | "
                   f"{sum(t_bd) / len(t_bd):.4f} | {ev} | {tf:.1f} | {tf / PEAK_F16_TFLOPS:.4f} |")
        if name == "wgrad":
            dom = (avg, tf)
    out += ["", "bench events: wgrad's from the timed steps' events around it, fprop's and dgrad's from the "
            "breakdown steps.", "",
            f"Dominant kernel (wgrad's launch): the bench line reports `avg_launch_ms` {rf.get('avg_launch_ms')} "
            f"and `frac` {rf.get('frac')} from its HIP events; the trace average of the same {steps} launches is "
            f"{dom[0]:.4f} ms, i.e. frac {dom[1] / PEAK_F16_TFLOPS:.4f}.", ""]
    # quantizer sweep
    if b.get("quantize_sweep_32768x8192_bf16"):
        seq = _sweep_sequence(ds, "--trace")
        sw = b["quantize_sweep_32768x8192_bf16"]
        n = 32768 * 8192
        alg = 2 * n * 2 + n // 2 + n // 16
        out += ["## Quantizer sweep (32768x8192 bf16)", "",
                f"Per call: meta init, amax pass, encode pass. Trace averages over calls 3-{SWEEP_CALLS} of each "
                "variant (the bench times the same ten calls with one pair of events around them).", "",
                "| variant | amax kernel us | encode kernel us | sum of the 3 kernels us | bench call us | "
                "GB/s (alg. 4.5625 B/elem, trace sum) |", "|---|---:|---:|---:|---:|---:|"]
        for v, (axis, rnd, rht) in enumerate(SWEEP_VARIANTS):
            calls = [seq[3 * (v * SWEEP_CALLS + c): 3 * (v * SWEEP_CALLS + c) + 3] for c in range(2, SWEEP_CALLS)]
            am = sum((c[1][3] - c[1][2]) for c in calls) / len(calls) / 1e3
            en = sum((c[2][3] - c[2][2]) for c in calls) / len(calls) / 1e3
            tot = sum(sum(e[3] - e[2] for e in c) for c in calls) / len(calls) / 1e3
            key = f"axis{axis} {rnd}{'+rht' if rht else ''}"
            bms = sw.get(key, {}).get("ms")
            out.append(f"| {key} | {am:.1f} | {en:.1f} | {tot:.1f} | {bms * 1e3 if bms else float('nan'):.1f} | "
                       f"{alg / (tot * 1e-6) / 1e9:.0f} |")
        out.append("")
    # per-kernel statistics
    stats = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if stats:
        rows = list(csv.DictReader(open(stats[0])))
        rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
        out += ["## Per-kernel statistics (the whole run, warm-up and context sections included)", "",
                "| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---:|---:|---:|---:|---:|"]
        for r in rows[:30]:
            out.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                       f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                       f"{float(r['Percentage']):.2f} |")
    return "\n".join(out) + "\n"


def reduce_quant_counters(fetch_dir: str, write_dir: str, valu_dir: str, trace_dir: str) -> str:
    """Per-pass HBM bytes (FETCH_SIZE / WRITE_SIZE scaled by the calibration
    copy), VALU busy and clock of the quantizer sweep's calls from three
    rocprofv3 --pmc runs of this script, and their times from a kernel-trace
    run (counter collection serialises dispatches, and the chip clocks
    differently between them); returns the markdown summary."""
    n = 32768 * 8192
    runs = {}
    for tag, d in (("fetch", fetch_dir), ("write", write_dir), ("valu", valu_dir)):
        ds = _dispatches(d)
        runs[tag] = (ds, _sweep_sequence(ds, f"--quant-counters ({d})"))
    trace_seq = _sweep_sequence(_trace_rows(trace_dir), f"--quant-counters ({trace_dir})")
    copies = [e for e in runs["fetch"][0] if "copyBuffer" in e[0]]
    f_scale = CALIB_BYTES / (max(e[4]["FETCH_SIZE"] for e in copies) * 1024.0)
    copies = [e for e in runs["write"][0] if "copyBuffer" in e[0]]
    w_scale = CALIB_BYTES / (max(e[4]["WRITE_SIZE"] for e in copies) * 1024.0)
    alg_read, alg_write = 2 * n, n // 2 + n // 16
    rows = []
    for v, (axis, rnd, rht) in enumerate(SWEEP_VARIANTS):
        for p, pname in ((1, "amax"), (2, "encode")):
            idx = [3 * (v * SWEEP_CALLS + c) + p for c in range(SWEEP_CALLS)]
            fe = [runs["fetch"][1][i] for i in idx]
            we = [runs["write"][1][i] for i in idx]
            va = [runs["valu"][1][i] for i in idx]
            te = [trace_seq[i] for i in idx]
            us = sum((e[3] - e[2]) / 1e3 for e in te) / len(te)               # kernel trace
            us_pmc = sum((e[3] - e[2]) / 1e3 for e in va) / len(va)          # counter run
            rd = sum(e[4]["FETCH_SIZE"] for e in fe) / len(fe) * 1024.0 * f_scale
            wr = sum(e[4]["WRITE_SIZE"] for e in we) / len(we) * 1024.0 * w_scale
            busy = sum(e[4]["SQ_INSTS_VALU"] * 4 / (e[4]["GRBM_GUI_ACTIVE"] / 8 * 1024) for e in va) / len(va)
            ghz = sum(e[4]["GRBM_GUI_ACTIVE"] / 8 / (e[3] - e[2]) for e in va) / len(va)
            rows.append((f"axis{axis} {rnd}{'+rht' if rht else ''}", pname, fe[0][0].split("::")[-1].split("(")[0],
                         us, rd, alg_read, wr, alg_write if p == 2 else 0, (rd + wr) / (us * 1e-6) / 1e9, busy,
                         us_pmc, ghz))
    run = "--output-format csv -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline"
    lines = ["# Quantizer counters on the 32768x8192 bf16 sweep tensor", "",
             "Commands (repository root, one MI355X), one counter set per run, then the reduction:", "", "```",
             f"rocprofv3 --pmc FETCH_SIZE --kernel-trace -d {fetch_dir} -o run {run}",
             f"rocprofv3 --pmc WRITE_SIZE --kernel-trace -d {write_dir} -o run {run}",
             f"rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR "
             f"--kernel-trace -d {valu_dir} -o run {run}",
             f"rocprofv3 --kernel-trace --stats -d {trace_dir} -o run {run}",
             f"python3 bench.py --quant-counters {fetch_dir} {write_dir} {valu_dir} {trace_dir}", "```", "",
             f"FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what they read for the 256 MiB "
             f"calibration copy of the same run ({f_scale:.2f} and {w_scale:.2f}). The tensor (512 MiB) exceeds the "
             "256 MB MALL. Algorithmic bytes per call: the amax pass reads 537 MB; the encode pass reads 537 MB and "
             "writes 151 MB of codes and scales. VALU busy = SQ_INSTS_VALU x 4 cycles / (GRBM_GUI_ACTIVE/8 x 1024 "
             "SIMDs), the share of SIMD issue cycles spent on VALU instructions at one pass each (quarter-rate "
             "instructions such as the 64-bit multiplies of Philox take more, so SR is undercounted). Times (and "
             "GB/s) from the kernel-trace run; the counter run's own dispatch time and clock (GRBM_GUI_ACTIVE/8 "
             "over that time) beside them: counter collection serialises the dispatches, and the chip runs them "
             f"at another clock. Averages over the {SWEEP_CALLS} calls of each variant.", "",
             "| variant | pass | kernel | us (trace) | HBM read MB (alg.) | HBM write MB (alg.) | achieved GB/s | "
             "VALU busy | us (counter run) | clock GHz (counter run) |",
             "|---|---|---|---:|---:|---:|---:|---:|---:|---:|"]
    for (var, pname, kern, us, rd, ard, wr, awr, gbs, busy, us_pmc, ghz) in rows:
        lines.append(f"| {var} | {pname} | {kern} | {us:.1f} | {rd / 1e6:.0f} ({ard / 1e6:.0f}) | "
                     f"{wr / 1e6:.0f} ({awr / 1e6:.0f}) | {gbs:.0f} | {busy:.2f} | {us_pmc:.1f} | {ghz:.2f} |")
    return "\n".join(lines) + "\n"


def traffic_summary(prof: dict) -> str:
    """Markdown summary of the traffic profile of the dominant kernel."""
    import workloads
    g = workloads.WGRAD
    m, n, k = g.mnk
    alg_r = (m + n) * k * 9 // 16
    alg_w = m * n * 4
    fb, wb = prof["fetch_bytes_per_launch"], prof["write_bytes_per_launch"]
    return "\n".join([
        f"# HBM-side traffic of `{prof['kernel']}` ({prof['grid_work_items']} work-items: the wgrad GEMM "
        f"{m}x{n}x{k})", "",
        "Commands (repository root, one MI355X), each counter in a run of its own, then the reduction:", "",
        "```", *prof["command"].split(" && "), "```", "",
        f"Calibration: every bench run copies a 256 MiB f32 tensor once (`__amd_rocclr_copyBuffer`, outside the "
        f"timed region); that copy read {prof['copy_fetch_kib']:.0f} KiB by FETCH_SIZE and wrote "
        f"{prof['copy_write_kib']:.0f} KiB by WRITE_SIZE for 262144 KiB moved each way, so FETCH_SIZE is scaled by "
        f"{prof['fetch_scale']:.2f} and WRITE_SIZE by {prof['write_scale']:.2f}. Dispatches averaged: "
        f"{prof['dispatches'][0]} (FETCH_SIZE run), {prof['dispatches'][1]} (WRITE_SIZE run). The profile holds the "
        "SHA-256 of the GEMM sources it was taken on; the bench reports `traffic` only while they match.", "",
        "| per launch | counter (KiB) | scaled bytes | algorithmic bytes |", "|---|---:|---:|---:|",
        f"| read | {prof['fetch_kib_per_dispatch']:.0f} | {fb / 1e6:.0f} MB | {alg_r / 1e6:.0f} MB (codes + scales of A "
        "and B once) |",
        f"| write | {prof['write_kib_per_dispatch']:.0f} | {wb / 1e6:.0f} MB | {alg_w / 1e6:.0f} MB (f32 C once) |",
        f"| total | | **{(fb + wb) / 1e6:.0f} MB** | **{(alg_r + alg_w) / 1e6:.0f} MB** |", ""])


BUSY_PROFILE = os.path.join(ROOT, "profiles", "gemm_fprop_dgrad_wgrad_mfma_busy.md")
BUSY_COUNTERS = ("GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_INSTS_MFMA "
                 "SQ_INSTS_VALU SQ_WAIT_INST_ANY SQ_LDS_BANK_CONFLICT")


def reduce_busy(busy_dir: str) -> str:
    """MFMA busy fraction, clock and issue counters of the GEMM kernels from
    one rocprofv3 --pmc run of this script; returns the markdown summary."""
    ds = _dispatches(busy_dir)
    kinds = gemm_kinds()
    lines = ["# MFMA busy fraction and clock of the GEMM kernels (linear-layer step)", "",
             "Command (repository root, one MI355X; one counter pass, 7 SQ + 1 GRBM counters), then the reduction:",
             "", "```",
             f"rocprofv3 --pmc {BUSY_COUNTERS} --kernel-trace -d {busy_dir} -o run --output-format csv -- "
             "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-sweep",
             f"python3 bench.py --busy {busy_dir}", "```", "",
             "Per dispatch, with G = GRBM_GUI_ACTIVE / 8 XCDs (GPU cycles of the kernel): clock = G / kernel "
             "duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (G x 1024 SIMDs); VALU instructions per MFMA = "
             "SQ_INSTS_VALU / SQ_INSTS_MFMA (SQ_INSTS_VALU counts the MFMAs too); VALU active = "
             "4 x SQ_ACTIVE_INST_VALU / (G x 1024) and issue wait = 4 x SQ_WAIT_INST_ANY / (G x 1024), per-wave "
             "fractions of the cycles (the SQ counts these in units of 4 cycles; one wave per SIMD); LDS "
             "bank-conflict cycles per CU = SQ_LDS_BANK_CONFLICT / (G x 256). Averages over the dispatches of "
             "the run (warm-up included).", "",
             "| kernel | dispatches | ms | clock GHz | MFMA busy | VALU instr / MFMA | VALU active | issue wait "
             "| LDS conflict cycles |", "|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for label, (key, grid) in kinds:
        sel = [e for e in ds if key in e[0] and e[1] == grid]
        if not sel:
            raise SystemExit(f"--busy: no {key} dispatches of {grid} work-items in {busy_dir}")
        acc = {"ms": 0.0, "ghz": 0.0, "busy": 0.0, "ipm": 0.0, "va": 0.0, "wait": 0.0, "lds": 0.0}
        for e in sel:
            c, dur = e[4], (e[3] - e[2]) * 1e-9
            g = c["GRBM_GUI_ACTIVE"] / 8
            acc["ms"] += dur * 1e3
            acc["ghz"] += g / dur / 1e9
            acc["busy"] += c["SQ_VALU_MFMA_BUSY_CYCLES"] / (g * 1024)
            acc["ipm"] += c["SQ_INSTS_VALU"] / c["SQ_INSTS_MFMA"]
            acc["va"] += 4 * c["SQ_ACTIVE_INST_VALU"] / (g * 1024)
            acc["wait"] += 4 * c["SQ_WAIT_INST_ANY"] / (g * 1024)
            acc["lds"] += c["SQ_LDS_BANK_CONFLICT"] / (g * 256)
        a = {k: v / len(sel) for k, v in acc.items()}
        lines.append(f"| {key} ({label}) | {len(sel)} | {a['ms']:.3f} | {a['ghz']:.2f} | {a['busy']:.3f} | "
                     f"{a['ipm']:.2f} | {a['va']:.3f} | {a['wait']:.3f} | {a['lds']:.3f} |")
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="reduce two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this script into "
                         "the traffic profile and exit (no GPU needed)")
    ap.add_argument("--quant-counters", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "VALU_DIR", "TRACE_DIR"),
                    help="reduce three rocprofv3 --pmc runs of this script (FETCH_SIZE, WRITE_SIZE, VALU counters) "
                         "and one kernel-trace run into the quantizer counter profile and exit (no GPU needed)")
    ap.add_argument("--trace", nargs=2, metavar=("TRACE_DIR", "BENCH_JSON"),
                    help="reduce a rocprofv3 --kernel-trace --stats run of this script (and the JSON line it "
                         "printed) into the kernel-trace profile and exit (no GPU needed)")
    ap.add_argument("--busy", metavar="BUSY_DIR",
                    help="reduce a rocprofv3 --pmc run of this script with the MFMA-busy counters into the GEMM "
                         "busy profile and exit (no GPU needed)")
    args = ap.parse_args()
    if args.busy:
        md = reduce_busy(args.busy)
        with open(BUSY_PROFILE, "w") as f:
            f.write(md)
        print(md)
        return
    if args.trace:
        md = reduce_trace(*args.trace)
        with open(TRACE_PROFILE, "w") as f:
            f.write(md)
        print(md)
        return
    if args.quant_counters:
        md = reduce_quant_counters(*args.quant_counters)
        with open(QUANT_PROFILE, "w") as f:
            f.write(md)
        print(md)
        return
    if args.traffic:
        prof = reduce_traffic(*args.traffic)
        run = "--output-format csv -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-sweep"
        prof["command"] = (f"rocprofv3 --pmc FETCH_SIZE -d {args.traffic[0]} -o run {run} && "
                           f"rocprofv3 --pmc WRITE_SIZE -d {args.traffic[1]} -o run {run} && "
                           f"python3 bench.py --traffic {args.traffic[0]} {args.traffic[1]}")
        with open(TRAFFIC_PROFILE, "w") as f:
            json.dump(prof, f, indent=1)
        md = traffic_summary(prof)
        with open(TRAFFIC_SUMMARY, "w") as f:
            f.write(md)
        print(md)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU (the path has no multi-GPU code); --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import gemm_amax_reduce_amd as nv
    import workloads

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    nv.lib()
    dev = torch.device("cuda", 0)

    spin = getattr(torch.cuda, "_sleep", None)

    def hold_gpu():
        # Event-timed regions that start on an idle GPU: a spin kernel of
        # about 0.2 ms (500k core clocks) queued ahead of the start event, so
        # the host's launch of the first timed call happens while the GPU is
        # still busy and its latency stays out of the measured interval.
        if spin is not None:
            spin(500_000)
    mask = workloads.rht_sign_mask()
    seed = workloads.SR_SEED

    # ---------------------------------------------------------- inputs ----
    t0 = time.time()
    F, D, Wg = workloads.FPROP, workloads.DGRAD, workloads.WGRAD
    X1 = F.a.generate().to(dev)
    W1 = F.b.generate().to(dev)
    dY = D.a.generate().to(dev)          # shared by dgrad (axis 1) and wgrad (axis 0)
    W2 = D.b.generate().to(dev)
    X2 = Wg.a.generate().to(dev)
    T_host = None if args.no_sweep else workloads.SWEEP.generate()
    T = None if args.no_sweep else T_host.to(dev)
    log(f"[bench] inputs generated and resident in HBM in {time.time() - t0:.1f}s")
    # calibration copy of known size for the HBM traffic counters
    calib_src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    torch.cuda.synchronize()
    # measured ceilings beside the published peaks: the same device copy
    # (read + write), and the MFMA form of the GEMM on its operand values
    copy_ms = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        hold_gpu()
        e0.record()
        calib_dst.copy_(calib_src)
        e1.record()
        torch.cuda.synchronize()
        copy_ms.append(e0.elapsed_time(e1))
    measured_peaks = {"hbm_copy_GB/s": round(2 * CALIB_BYTES / (sorted(copy_ms)[2] * 1e-3) / 1e9, 1),
                      "mfma_f16_probe_TFLOP/s": round(max(nv.nvfp4_probe_mfma(2000) for _ in range(3)), 1)}
    del calib_src, calib_dst

    # ------------------------------------------------ quantizer sweep ----
    # The sweep follows the MFMA probe with no idle gap (its input is
    # generated and uploaded with the others): after an idle second the chip
    # needs 10-20 ms of load before the VALU-heavy encodes run at full clock
    # (SR axis 1 on one MI355X: 229 us right after idle, 206 after the probe),
    # and the step's warm-up follows the sweep the same way.
    sweep = None
    dequant = None
    if not args.no_sweep:
        qT = nv.NVFP4Tensor.empty(32768, 8192)
        qTt = nv.NVFP4Tensor.empty(8192, 32768)
        b = qbytes(T.numel(), 2)
        sweep = {}
        for axis in (1, 0):
            out = qT if axis == 1 else qTt
            for rnd in ("rne", "sr"):
                for rht in (False, True):
                    def call():
                        if rht:
                            nv.nvfp4_rht_quantize(T, mask, axis=axis, rounding=rnd, seed=seed, out=out)
                        else:
                            nv.nvfp4_quantize(T, axis=axis, rounding=rnd, seed=seed, out=out)
                    for _ in range(2):
                        call()
                    n_it = 10
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    torch.cuda.synchronize()
                    hold_gpu()
                    e0.record()
                    for _ in range(n_it):
                        call()
                    e1.record()
                    torch.cuda.synchronize()
                    ms = e0.elapsed_time(e1) / n_it
                    gbs = b / (ms * 1e-3) / 1e9
                    sweep[f"axis{axis} {rnd}{'+rht' if rht else ''}"] = {
                        "ms": round(ms, 4), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBPS, 4),
                        "frac_of_measured_copy": round(gbs / measured_peaks["hbm_copy_GB/s"], 4)}
        # each pass alone (the encode pass with the amax supplied, so it reads
        # the tensor cold, without the MALL reuse the whole call has), and the
        # stochastic-rounding random bits alone (Philox4x32-10 for the
        # tensor's n/8 counters, no memory traffic): the floor the RNG
        # contract puts under an SR encode of this tensor
        amax_buf = torch.empty(1, dtype=torch.float32, device=dev)
        def _t(fn, it=10):
            for _ in range(2):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(it):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / it
        passes = {"philox_floor_ms": round(sorted(nv.nvfp4_probe_philox(T.numel() // 8) for _ in range(5))[2], 4)}
        for axis in (1, 0):
            out = qT if axis == 1 else qTt
            for rnd in ("rne", "sr"):
                for rht in (False, True):
                    a_ms = _t(lambda: nv.nvfp4_amax(T, axis=axis, rht=rht, sign_mask=mask, out=amax_buf))
                    e_ms = _t(lambda: nv.nvfp4_quantize_amax(T, amax_buf, axis=axis, rounding=rnd, seed=seed,
                                                             rht=rht, sign_mask=mask, out=out))
                    passes[f"axis{axis} {rnd}{'+rht' if rht else ''}"] = {"amax_pass_ms": round(a_ms, 4),
                                                                          "encode_pass_ms": round(e_ms, 4)}
        sweep["passes"] = passes
        # dequantize of the same tensor (the last axis-1 result): codes and
        # scales read once (0.5625 B/element), values written once
        dequant = {}
        for name, dt, eb in (("bf16", torch.bfloat16, 2), ("f32", torch.float32, 4)):
            yq = torch.empty((32768, 8192), dtype=dt, device=dev)
            for _ in range(2):
                nv.nvfp4_dequantize(qT, dt, out=yq)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            hold_gpu()
            e0.record()
            for _ in range(10):
                nv.nvfp4_dequantize(qT, dt, out=yq)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 10
            db = T.numel() * 9 // 16 + T.numel() * eb
            dequant[name] = {"ms": round(ms, 4), "GB/s": round(db / (ms * 1e-3) / 1e9, 1),
                             "frac_hbm": round(db / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
            del yq
        del T, qT, qTt

    # outputs preallocated: the timed loop allocates nothing
    qX1 = nv.NVFP4Tensor.empty(4096, 5120)
    qW1 = nv.NVFP4Tensor.empty(5120, 5120)
    qdY = nv.NVFP4Tensor.empty(8192, 20480)
    qW2 = nv.NVFP4Tensor.empty(5120, 20480)
    qX2 = nv.NVFP4Tensor.empty(5120, 8192)
    qdYt = nv.NVFP4Tensor.empty(20480, 8192)
    Y = torch.empty((4096, 5120), dtype=torch.bfloat16, device=dev)
    # the GEMMs run through nvfp4_gemm_ws: with its workspace the last one to
    # two rounds of 256 x 256 tiles run as a stream-K tail (the fprop, dgrad
    # and wgrad layers are 1.25, 2.5 and 6.25 rounds), where nvfp4_gemm runs
    # its mixed-width grid
    ws = nv.gemm_workspace(dev)
    dX = torch.empty((8192, 5120), dtype=torch.float32, device=dev)
    dW = torch.empty((5120, 20480), dtype=torch.float32, device=dev)

    ops = [
        ("q fprop X", lambda: nv.nvfp4_quantize(X1, axis=1, out=qX1), ("q", X1)),
        ("q fprop W", lambda: nv.nvfp4_quantize(W1, axis=1, out=qW1), ("q", W1)),
        ("gemm fprop", lambda: nv.nvfp4_gemm_ws(qX1, qW1, torch.bfloat16, out=Y, workspace=ws), ("g", F.flops)),
        # dY in both layouts from one amax read: axis 1 SR (dgrad, offset 0)
        # and axis 0 RHT SR (wgrad, offset 1)
        ("q dY dual (axis1 SR + axis0 RHT SR)",
         lambda: nv.nvfp4_quantize_dual(dY, rounding1="sr", seed1=seed, offset1=0, rht0=True, sign_mask0=mask,
                                        rounding0="sr", seed0=seed, offset0=1, out1=qdY, out0=qdYt), ("q2", dY)),
        ("q dgrad W (axis0)", lambda: nv.nvfp4_quantize(W2, axis=0, out=qW2), ("q", W2)),
        ("gemm dgrad", lambda: nv.nvfp4_gemm_ws(qdY, qW2, torch.float32, out=dX, workspace=ws), ("g", D.flops)),
        ("q wgrad X (RHT, axis0)", lambda: nv.nvfp4_rht_quantize(X2, mask, axis=0, out=qX2), ("q", X2)),
        ("gemm wgrad", lambda: nv.nvfp4_gemm_ws(qX2, qdYt, torch.float32, out=dW, workspace=ws), ("g", Wg.flops)),
    ]
    step_flops = F.flops + D.flops + Wg.flops
    # The backward operands that come from forward-time tensors (W on axis 0
    # for dgrad, X on axis 0 with the transform for wgrad) are quantized on a
    # second stream (default priority), released once the forward
    # quantizations are issued, so they run beside the fprop GEMM; the dgrad
    # GEMM waits for them.  Same-GPU A/B of the step: 3.199 ms on one stream,
    # 3.147 with the second stream released at the step start, 3.122 released
    # after the forward quantizations; outputs bit-identical.
    SIDE = ("q dgrad W (axis0)", "q wgrad X (RHT, axis0)")
    main_stream = torch.cuda.current_stream(dev)
    side_stream = torch.cuda.Stream(device=dev)
    side_ix = [i for i, (n, _, _) in enumerate(ops) if n in SIDE]
    main_ix = [i for i, (n, _, _) in enumerate(ops) if n not in SIDE]
    release_after = next(i for i, (n, _, _) in enumerate(ops) if n == "q fprop W")
    first_wait = next(i for i, (n, _, _) in enumerate(ops) if n == "gemm dgrad")

    def step(start_ev, release_ev, side_done, events=None, wgrad_evs=None):
        """One step.  `events`: an event after every op (the breakdown pass);
        `wgrad_evs`: a pair of events around the wgrad launch only (the timed
        pass, which records nothing else)."""
        if start_ev is not None:
            start_ev.record(main_stream)
        for i in main_ix:
            if i == first_wait:
                main_stream.wait_event(side_done)
            if wgrad_evs is not None and i == wgrad_ix:
                wgrad_evs[0].record(main_stream)
            ops[i][1]()
            if events is not None:
                events[i].record(main_stream)
            if i == release_after:
                release_ev.record(main_stream)
                side_stream.wait_event(release_ev)
                with torch.cuda.stream(side_stream):
                    for j in side_ix:
                        ops[j][1]()
                        if events is not None:
                            events[j].record(side_stream)
                side_done.record(side_stream)
        if wgrad_evs is not None:
            wgrad_evs[1].record(main_stream)

    wgrad_ix = next(i for i, (n, _, _) in enumerate(ops) if n == "gemm wgrad")
    assert wgrad_ix == main_ix[-1]
    K = args.steps
    nev = max(K, args.warmup)
    start = [torch.cuda.Event(enable_timing=True) for _ in range(nev)]
    release = [torch.cuda.Event() for _ in range(nev)]
    side_done = [torch.cuda.Event() for _ in range(nev)]
    for w in range(args.warmup):
        step(None, release[w], side_done[w])
    torch.cuda.synchronize()

    # ---------------------------------------------------- timed region ----
    # Inside it only three events per step: the step start and the two
    # around the wgrad launch (an event after every op costs about 1 % of
    # the step).
    wg_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for s in range(K):
        step(start[s], release[s], side_done[s], wgrad_evs=wg_evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    wgrad_ms = np.array([a.elapsed_time(b) for a, b in wg_evs])
    step_ms = np.array([start[s].elapsed_time(wg_evs[s][1]) for s in range(K)])

    # ------------------------------------------------ breakdown pass ----
    # K more steps with an event after every op, for the per-op times (not
    # the headline: the events themselves slow the step)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in ops] for _ in range(K)]
    rel_t = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    t_bd = time.perf_counter()
    for s in range(K):
        step(start[s], rel_t[s], side_done[s], evs[s])
    torch.cuda.synchronize()
    bd_ms_per_step = (time.perf_counter() - t_bd) * 1e3 / K
    per_op = np.zeros((K, len(ops)))
    for s in range(K):
        # each stream's ops timed back to back: the main stream's from the
        # step start, the second stream's from its release
        for ix, t0 in ((main_ix, start[s]), (side_ix, rel_t[s])):
            prev = t0
            for i in ix:
                per_op[s, i] = prev.elapsed_time(evs[s][i])
                prev = evs[s][i]
    ms_per_step = wall * 1e3 / K
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    breakdown = {}
    for i, (name, _, kind) in enumerate(ops):
        ms = float(np.mean(per_op[:, i]))
        if kind[0] in ("q", "q2"):
            x = kind[1]
            b = qbytes(x.numel(), x.element_size()) if kind[0] == "q" else qbytes_dual(x.numel(), x.element_size())
            breakdown[name] = {"ms": round(ms, 4), "GB/s": round(b / (ms * 1e-3) / 1e9, 1)}
            if name in SIDE:
                breakdown[name]["stream"] = "second, released after the forward quantizations, beside the fprop GEMM"
        else:
            breakdown[name] = {"ms": round(ms, 4), "TFLOP/s": round(kind[1] / (ms * 1e-3) / 1e12, 1)}

    for i in main_ix:
        if release_after < i < first_wait:
            breakdown[ops[i][0]]["stream"] = "main, overlapped with the second stream's quantizations"

    # dominant kernel: the one kernel launch with the most time per step,
    # wgrad's (2*5120*20480*8192 flop; f32-output stream-K kernel, as dgrad's
    # but on a larger grid; fprop's is the bf16 one); one GEMM call is one
    # kernel launch on torch's current stream, which the two events of the
    # timed region around it are recorded on
    g_ms = float(np.mean(wgrad_ms))
    g_flop = Wg.flops
    achieved = g_flop / (g_ms * 1e-3) / 1e12
    traffic = load_traffic()
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_F16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_F16_TFLOPS, 4),
                "traffic": round(traffic) if traffic else None,
                "kernel": "%s, %d work-items: the wgrad launch of each step" % dominant_launch(),
                "avg_launch_ms": round(g_ms, 4), "flop_per_launch": g_flop,
                "algorithmic_bytes_per_launch": gemm_bytes(Wg),
                "frac_of_fp4_peak": round(achieved / PEAK_FP4_TFLOPS, 4),
                "frac_of_measured_mfma_probe": round(achieved / measured_peaks["mfma_f16_probe_TFLOP/s"], 4),
                "gemm_kernels": {name: "%s, %d work-items (stream-K tail)" % launch for name, launch in gemm_kinds()}}

    # ------------------------------- fprop operands, warm and cold ----
    # The fprop operands (40-50 MB) fit the 256 MB MALL, so in the step the
    # encode pass re-reads them partly from cache.  Each is timed again
    # right after a 512 MiB write that evicts them (the write itself outside
    # the timed region).
    fprop_cache = None
    if not args.no_sweep:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        fprop_cache = {}
        for name, x, out in (("X 4096x5120 bf16", X1, qX1), ("W 5120x5120 bf16", W1, qW1)):
            b = qbytes(x.numel(), x.element_size())
            warm, cold = [], []
            for _ in range(7):
                for label, prep in (("warm", lambda: nv.nvfp4_quantize(x, axis=1, out=out)),
                                    ("cold", lambda: flush.fill_(1))):
                    prep()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    hold_gpu()
                    e0.record()
                    nv.nvfp4_quantize(x, axis=1, out=out)
                    e1.record()
                    torch.cuda.synchronize()
                    (warm if label == "warm" else cold).append(e0.elapsed_time(e1))
            w, c = sorted(warm)[3], sorted(cold)[3]
            fprop_cache[name] = {"warm_ms": round(w, 4), "warm_GB/s": round(b / (w * 1e-3) / 1e9, 1),
                                 "after_flush_ms": round(c, 4), "after_flush_GB/s": round(b / (c * 1e-3) / 1e9, 1)}
        del flush

    # ------------------------------------------- BF16 GEMM context ----
    # The same three products in bf16 through torch.matmul (hipBLASLt), to
    # state the 4-bit path's speed against a 16-bit one as a measured ratio.
    # Context only: it is not the NVFP4 path and does not enter `value`.
    bf16_ctx = None
    if not args.no_sweep:
        W1t = W1.t().contiguous()
        X2t = X2.t().contiguous()
        prods = {"fprop": (lambda: torch.matmul(X1, W1t), F.flops),
                 "dgrad": (lambda: torch.matmul(dY, W2), D.flops),
                 "wgrad": (lambda: torch.matmul(X2t, dY), Wg.flops)}
        bf16_ctx = {}
        tot_bf16 = 0.0
        for name, (fn, fl) in prods.items():
            for _ in range(2):
                fn()
            times = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                hold_gpu()
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            ms = sorted(times)[2]
            tot_bf16 += ms
            bf16_ctx[name] = {"ms": round(ms, 4), "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 1)}
        nv_gemm_ms = sum(float(np.mean(per_op[:, i])) for i, (n, _, _) in enumerate(ops) if n.startswith("gemm"))
        bf16_ctx["gemm_time_ratio_bf16_over_nvfp4"] = round(tot_bf16 / nv_gemm_ms, 3)
        del W1t, X2t

    # ------------------------------------------------ MXFP4 context ----
    # The same linear-layer step in MXFP4 (32-element blocks, power-of-two
    # scales) on the block-scaled FP4 MFMA: the format the pages set NVFP4
    # against, measured on the same operands.  Context only.
    mx_ctx = None
    if not args.no_sweep:
        mX1 = nv.MXFP4Tensor.empty(4096, 5120)
        mW1 = nv.MXFP4Tensor.empty(5120, 5120)
        mdY = nv.MXFP4Tensor.empty(8192, 20480)
        mW2 = nv.MXFP4Tensor.empty(5120, 20480)
        mX2 = nv.MXFP4Tensor.empty(5120, 8192)
        mdYt = nv.MXFP4Tensor.empty(20480, 8192)
        mx_ops = [
            ("q fprop X", lambda: nv.mxfp4_quantize(X1, axis=1, out=mX1)),
            ("q fprop W", lambda: nv.mxfp4_quantize(W1, axis=1, out=mW1)),
            ("gemm fprop", lambda: nv.mxfp4_gemm(mX1, mW1, torch.bfloat16, out=Y)),
            ("q dgrad dY", lambda: nv.mxfp4_quantize(dY, axis=1, out=mdY)),
            ("q dgrad W (axis0)", lambda: nv.mxfp4_quantize(W2, axis=0, out=mW2)),
            ("gemm dgrad", lambda: nv.mxfp4_gemm(mdY, mW2, torch.float32, out=dX)),
            ("q wgrad X (axis0)", lambda: nv.mxfp4_quantize(X2, axis=0, out=mX2)),
            ("q wgrad dY (axis0)", lambda: nv.mxfp4_quantize(dY, axis=0, out=mdYt)),
            ("gemm wgrad", lambda: nv.mxfp4_gemm(mX2, mdYt, torch.float32, out=dW)),
        ]
        for _ in range(2):
            for _, fn in mx_ops:
                fn()
        n_mx = 10
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(mx_ops) + 1)] for _ in range(n_mx)]
        torch.cuda.synchronize()
        for it in range(n_mx):
            ev[it][0].record()
            for i, (_, fn) in enumerate(mx_ops):
                fn()
                ev[it][i + 1].record()
        torch.cuda.synchronize()
        per = np.array([[ev[it][i].elapsed_time(ev[it][i + 1]) for i in range(len(mx_ops))] for it in range(n_mx)])
        step_mx = float(np.median(per.sum(axis=1)))
        mx_ctx = {"ms_per_step": round(step_mx, 4), "TFLOP/s": round(step_flops / (step_mx * 1e-3) / 1e12, 1),
                  "breakdown": {}}
        flops_of = {"gemm fprop": F.flops, "gemm dgrad": D.flops, "gemm wgrad": Wg.flops}
        for i, (name, _) in enumerate(mx_ops):
            ms = float(np.median(per[:, i]))
            ent = {"ms": round(ms, 4)}
            if name in flops_of:
                ent["TFLOP/s"] = round(flops_of[name] / (ms * 1e-3) / 1e12, 1)
                ent["frac_of_fp4_peak"] = round(flops_of[name] / (ms * 1e-3) / 1e12 / PEAK_FP4_TFLOPS, 4)
            mx_ctx["breakdown"][name] = ent
        del mX1, mW1, mdY, mW2, mX2, mdYt

    # ------------------------------------------------ MXFP8 context ----
    # The same step in MXFP8 (E4M3 elements, a power-of-two scale per 32) on
    # the block-scaled FP8 MFMA: the 8-bit format of the pages' three-format
    # training run.  Context only.
    mx8_ctx = None
    if not args.no_sweep:
        PEAK_FP8_TFLOPS = 5000.0
        eX1 = nv.MXFP8Tensor.empty(4096, 5120)
        eW1 = nv.MXFP8Tensor.empty(5120, 5120)
        edY = nv.MXFP8Tensor.empty(8192, 20480)
        eW2 = nv.MXFP8Tensor.empty(5120, 20480)
        eX2 = nv.MXFP8Tensor.empty(5120, 8192)
        edYt = nv.MXFP8Tensor.empty(20480, 8192)
        mx8_ops = [
            ("q fprop X", lambda: nv.mxfp8_quantize(X1, axis=1, out=eX1)),
            ("q fprop W", lambda: nv.mxfp8_quantize(W1, axis=1, out=eW1)),
            ("gemm fprop", lambda: nv.mxfp8_gemm(eX1, eW1, torch.bfloat16, out=Y)),
            ("q dgrad dY", lambda: nv.mxfp8_quantize(dY, axis=1, out=edY)),
            ("q dgrad W (axis0)", lambda: nv.mxfp8_quantize(W2, axis=0, out=eW2)),
            ("gemm dgrad", lambda: nv.mxfp8_gemm(edY, eW2, torch.float32, out=dX)),
            ("q wgrad X (axis0)", lambda: nv.mxfp8_quantize(X2, axis=0, out=eX2)),
            ("q wgrad dY (axis0)", lambda: nv.mxfp8_quantize(dY, axis=0, out=edYt)),
            ("gemm wgrad", lambda: nv.mxfp8_gemm(eX2, edYt, torch.float32, out=dW)),
        ]
        for _ in range(2):
            for _, fn in mx8_ops:
                fn()
        n_mx = 10
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(mx8_ops) + 1)] for _ in range(n_mx)]
        torch.cuda.synchronize()
        for it in range(n_mx):
            ev[it][0].record()
            for i, (_, fn) in enumerate(mx8_ops):
                fn()
                ev[it][i + 1].record()
        torch.cuda.synchronize()
        per = np.array([[ev[it][i].elapsed_time(ev[it][i + 1]) for i in range(len(mx8_ops))] for it in range(n_mx)])
        step_mx8 = float(np.median(per.sum(axis=1)))
        mx8_ctx = {"ms_per_step": round(step_mx8, 4), "TFLOP/s": round(step_flops / (step_mx8 * 1e-3) / 1e12, 1),
                   "breakdown": {}}
        flops_of = {"gemm fprop": F.flops, "gemm dgrad": D.flops, "gemm wgrad": Wg.flops}
        for i, (name, _) in enumerate(mx8_ops):
            ms = float(np.median(per[:, i]))
            ent = {"ms": round(ms, 4)}
            if name in flops_of:
                ent["TFLOP/s"] = round(flops_of[name] / (ms * 1e-3) / 1e12, 1)
                ent["frac_of_fp8_peak"] = round(flops_of[name] / (ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4)
            mx8_ctx["breakdown"][name] = ent
        del eX1, eW1, edY, eW2, eX2, edYt

    # ------------------------------------------------- CPU baseline ----
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(F, D, Wg, mask, seed, step_flops, T_host)

    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "linear-layer step: fprop 4096x5120x5120 (bf16 out), dgrad 8192x5120x20480 "
                               "(dY SR), wgrad 5120x20480x8192 (RHT, dY SR); quantization of all six "
                               "operands included",
                   "gemm_flop_per_step": step_flops, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "measured_peaks": measured_peaks,
        "breakdown": breakdown,
        "quantize_sweep_32768x8192_bf16": sweep,
        "dequantize_32768x8192": dequant,
        "fprop_quantize_warm_vs_flushed": fprop_cache,
        "bf16_gemm_context": bf16_ctx,
        "mxfp4_step_context": mx_ctx,
        "mxfp8_step_context": mx8_ctx,
        "pages_context": PAGES_CONTEXT,
        "device": torch.cuda.get_device_name(0),
        "step_ms_event_median": round(float(np.median(step_ms)), 4),
        "breakdown_pass_ms_per_step": round(bd_ms_per_step, 4),
    }
    print(json.dumps(rec), flush=True)


def cpu_model() -> str:
    """The host CPU's model name (first entry of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads():
    """Threads of the BLAS numpy's float64 matmul runs on (the GEMM oracle)."""
    try:
        import threadpoolctl
        info = [d for d in threadpoolctl.threadpool_info() if d.get("user_api") == "blas"]
        return int(info[0]["num_threads"]) if info else None
    except Exception:
        return None


def cpu_baseline(F, D, Wg, mask, seed, step_flops, sweep_host=None):
    """The oracle (plain C with OpenMP + numpy float64) on the host cores:

    * quantizer: all eight variants ({RNE, SR} x {no RHT, RHT} x {axis 1,
      axis 0}) on the full 32768 x 8192 sweep tensor, as GB/s with the same
      4.5625 B/element formula as the GPU;
    * GEMM: the full fprop oracle (4096 x 5120 x 5120, value and bound);
      dgrad and wgrad on 512-row slices, extrapolated to the full M
      (labelled so);
    * the step: its six quantizations in full plus the three GEMMs, as
      TFLOP/s of GEMM work (the same unit as the GPU value)."""
    import numpy as np

    import oracle
    import workloads

    # quantizer sweep, full tensor
    T = sweep_host if sweep_host is not None else workloads.SWEEP.generate()
    b = qbytes(T.numel(), 2)
    qsweep = {}
    for axis in (1, 0):
        for rnd in ("rne", "sr"):
            for rht in (False, True):
                t = time.perf_counter()
                oracle.quantize(T, axis=axis, rounding=oracle.SR if rnd == "sr" else oracle.RNE, seed=seed,
                                rht=rht, sign_mask=mask)
                dt = time.perf_counter() - t
                qsweep[f"axis{axis} {rnd}{'+rht' if rht else ''}"] = {"s": round(dt, 3),
                                                                      "GB/s": round(b / dt / 1e9, 3)}
    del T
    # the step's quantizations in full, its GEMMs (fprop full, dgrad and
    # wgrad on 512 output rows)
    t_q = 0.0
    gemms = {}
    rows_sample = 512
    for name, g in (("fprop", F), ("dgrad", D), ("wgrad", Wg)):
        refs = []
        for op in (g.a, g.b):
            x = op.generate()
            r = oracle.SR if op.rounding == "sr" else oracle.RNE
            t = time.perf_counter()
            refs.append(oracle.quantize(x, axis=op.axis, rounding=r, seed=seed, offset=op.sr_offset,
                                        rht=op.rht, sign_mask=mask))
            t_q += time.perf_counter() - t
            del x
        m, n, k = g.mnk
        full = name == "fprop"
        rows = None if full else np.arange(rows_sample)
        t = time.perf_counter()
        oracle.gemm(refs[0], refs[1], rows=rows)
        dt = time.perf_counter() - t
        est = dt if full else dt * m / rows_sample
        gemms[name] = {"s": round(est, 3), "TFLOP/s": round(g.flops / est / 1e12, 4),
                       "measured": "full GEMM" if full else f"{rows_sample} of {m} output rows, extrapolated"}
    t_g = sum(v["s"] for v in gemms.values())
    t_step = t_q + t_g
    return {"value": round(step_flops / t_step / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "blas_threads": blas_threads(), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"step: all six operand quantizations in full ({t_q:.1f}s) + the fprop oracle GEMM in full "
                      f"and 512-row slices of dgrad and wgrad extrapolated to the full M ({t_g:.1f}s est.); "
                      f"quantizer: all eight variants on the full 32768x8192 sweep tensor",
            "ms_per_step_est": round(t_step * 1e3, 1),
            "gemm": gemms,
            "quantize_sweep_32768x8192_bf16": qsweep}


if __name__ == "__main__":
    main()
