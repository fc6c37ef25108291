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
value = GEMM FLOP of the step / step time (quantization included), TFLOP/s.
Also reported: quantizer GB/s per operand and on the 32768x8192 sweep tensor
(RNE/SR x RHT off/on), per-GEMM TFLOP/s, the roofline of the dominant kernel
(the f32-output GEMM that serves dgrad and wgrad), and the CPU oracle timed
on a bounded sample of the same step.

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


def qbytes(n_elem: int, in_bytes: int) -> int:
    """Algorithmic HBM bytes of one quantization: the input is read twice
    (amax pass, encode pass), codes (0.5 B) and scales (1/16 B) written."""
    return n_elem * (2 * in_bytes) + n_elem // 2 + n_elem // 16


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
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
    log(f"[bench] inputs generated and resident in HBM in {time.time() - t0:.1f}s")

    # outputs preallocated: the timed loop allocates nothing
    qX1 = nv.NVFP4Tensor.empty(4096, 5120)
    qW1 = nv.NVFP4Tensor.empty(5120, 5120)
    qdY = nv.NVFP4Tensor.empty(8192, 20480)
    qW2 = nv.NVFP4Tensor.empty(5120, 20480)
    qX2 = nv.NVFP4Tensor.empty(5120, 8192)
    qdYt = nv.NVFP4Tensor.empty(20480, 8192)
    Y = torch.empty((4096, 5120), dtype=torch.bfloat16, device=dev)
    dX = torch.empty((8192, 5120), dtype=torch.float32, device=dev)
    dW = torch.empty((5120, 20480), dtype=torch.float32, device=dev)

    ops = [
        ("q fprop X", lambda: nv.nvfp4_quantize(X1, axis=1, out=qX1), ("q", X1)),
        ("q fprop W", lambda: nv.nvfp4_quantize(W1, axis=1, out=qW1), ("q", W1)),
        ("gemm fprop", lambda: nv.nvfp4_gemm(qX1, qW1, torch.bfloat16, out=Y), ("g", F.flops)),
        ("q dgrad dY (SR)", lambda: nv.nvfp4_quantize(dY, axis=1, rounding="sr", seed=seed, offset=0, out=qdY), ("q", dY)),
        ("q dgrad W (axis0)", lambda: nv.nvfp4_quantize(W2, axis=0, out=qW2), ("q", W2)),
        ("gemm dgrad", lambda: nv.nvfp4_gemm(qdY, qW2, torch.float32, out=dX), ("g", D.flops)),
        ("q wgrad X (RHT, axis0)", lambda: nv.nvfp4_rht_quantize(X2, mask, axis=0, out=qX2), ("q", X2)),
        ("q wgrad dY (RHT, SR, axis0)", lambda: nv.nvfp4_rht_quantize(dY, mask, axis=0, rounding="sr", seed=seed,
                                                                      offset=1, out=qdYt), ("q", dY)),
        ("gemm wgrad", lambda: nv.nvfp4_gemm(qX2, qdYt, torch.float32, out=dW), ("g", Wg.flops)),
    ]
    step_flops = F.flops + D.flops + Wg.flops

    def step(events=None):
        for i, (_, fn, _) in enumerate(ops):
            fn()
            if events is not None:
                events[i].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---------------------------------------------------- timed region ----
    K = args.steps
    start = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    evs = [[torch.cuda.Event(enable_timing=True) for _ in ops] for _ in range(K)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for s in range(K):
        start[s].record()
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    per_op = np.zeros((K, len(ops)))
    step_ms = np.zeros(K)
    for s in range(K):
        prev = start[s]
        for i in range(len(ops)):
            per_op[s, i] = prev.elapsed_time(evs[s][i])
            prev = evs[s][i]
        step_ms[s] = start[s].elapsed_time(evs[s][-1])
    ms_per_step = wall * 1e3 / K
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    breakdown = {}
    for i, (name, _, kind) in enumerate(ops):
        ms = float(np.mean(per_op[:, i]))
        if kind[0] == "q":
            x = kind[1]
            b = qbytes(x.numel(), x.element_size())
            breakdown[name] = {"ms": round(ms, 4), "GB/s": round(b / (ms * 1e-3) / 1e9, 1)}
        else:
            breakdown[name] = {"ms": round(ms, 4), "TFLOP/s": round(kind[1] / (ms * 1e-3) / 1e12, 1)}

    # dominant kernel: the f32-output GEMM (dgrad and wgrad launches, each
    # 2*8192*5120*20480 flop); one nvfp4_gemm call is one kernel launch
    gi = [i for i, (n, _, _) in enumerate(ops) if n in ("gemm dgrad", "gemm wgrad")]
    g_ms = float(np.mean(per_op[:, gi]))
    g_flop = D.flops
    achieved = g_flop / (g_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_F16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_F16_TFLOPS, 4), "traffic": None,
                "kernel": "k_gemm_nvfp4<false> (f32 out), avg of dgrad+wgrad launches",
                "avg_launch_ms": round(g_ms, 4), "flop_per_launch": g_flop,
                "frac_of_fp4_peak": round(achieved / PEAK_FP4_TFLOPS, 4)}

    # ------------------------------------------------ quantizer sweep ----
    sweep = None
    if not args.no_sweep:
        T = workloads.SWEEP.generate().to(dev)
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
                    e0.record()
                    for _ in range(n_it):
                        call()
                    e1.record()
                    torch.cuda.synchronize()
                    ms = e0.elapsed_time(e1) / n_it
                    gbs = b / (ms * 1e-3) / 1e9
                    sweep[f"axis{axis} {rnd}{'+rht' if rht else ''}"] = {
                        "ms": round(ms, 4), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBPS, 4)}
        del T, qT, qTt

    # ------------------------------------------------- CPU baseline ----
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(F, D, Wg, mask, seed, step_flops)

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
        "breakdown": breakdown,
        "quantize_sweep_32768x8192_bf16": sweep,
        "device": torch.cuda.get_device_name(0),
        "step_ms_event_median": round(float(np.median(step_ms)), 4),
    }
    print(json.dumps(rec), flush=True)


def cpu_baseline(F, D, Wg, mask, seed, step_flops):
    """The oracle (plain C + numpy float64) on a bounded sample of the step:
    all six quantizations in full, and for each GEMM the full oracle on a
    slice of 64 output rows; the step time is extrapolated as
    t(quantize) + sum_g t(slice_g) * M_g / 64."""
    import numpy as np

    import oracle
    import workloads

    t_q = 0.0
    t_g = 0.0
    rows_sample = 64
    for g in (F, D, Wg):
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
        rows = np.arange(rows_sample)
        t = time.perf_counter()
        oracle.gemm(refs[0], refs[1], rows=rows)
        t_g += (time.perf_counter() - t) * m / rows_sample
    t_step = t_q + t_g
    return {"value": round(step_flops / t_step / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"all six operand quantizations in full ({t_q:.1f}s) + oracle GEMM on {rows_sample} output "
                      f"rows of each GEMM, extrapolated to the full M ({t_g:.1f}s est.); step {t_step:.1f}s",
            "ms_per_step_est": round(t_step * 1e3, 1)}


if __name__ == "__main__":
    main()
