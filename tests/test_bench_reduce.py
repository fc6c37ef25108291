"""Host logic of the benchmark's counter reductions (no GPU): the traffic
profile of the dominant GEMM and the quantizer sweep's counter table, fed
with synthetic rocprofv3 counter_collection.csv files."""
import csv
import os

import pytest

import bench

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
N_SWEEP = 32768 * 8192
COPY = "__amd_rocclr_copyBuffer"


def write_run(d, dispatches):
    """dispatches: [(name, grid, duration_ns, {counter: value})]"""
    os.makedirs(d, exist_ok=True)
    t = 1000
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, grid, dur, counters) in enumerate(dispatches, start=1):
            for cn, cv in counters.items():
                w.writerow({**{k: 0 for k in FIELDS}, "Dispatch_Id": i, "Grid_Size": grid, "Kernel_Name": name,
                            "Counter_Name": cn, "Counter_Value": cv, "Start_Timestamp": t,
                            "End_Timestamp": t + dur})
            t += dur + 10


TRACE_FIELDS = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id", "Kernel_Name",
                "Correlation_Id", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
                "Accum_VGPR_Count", "SGPR_Count", "Workgroup_Size_X", "Workgroup_Size_Y", "Workgroup_Size_Z",
                "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]


def write_trace(d, dispatches, stats=None):
    """dispatches: [(name, work_items, duration_ns)] in order; stats: kernel_stats rows."""
    os.makedirs(d, exist_ok=True)
    t = 1000
    with open(os.path.join(d, "run_kernel_trace.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=TRACE_FIELDS)
        w.writeheader()
        for i, (name, grid, dur) in enumerate(dispatches, start=1):
            w.writerow({**{k: 1 for k in TRACE_FIELDS}, "Dispatch_Id": i, "Kernel_Name": name, "Start_Timestamp": t,
                        "End_Timestamp": t + dur, "Grid_Size_X": grid, "Grid_Size_Y": 1, "Grid_Size_Z": 1})
            t += dur + 10
    if stats:
        with open(os.path.join(d, "run_kernel_stats.csv"), "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                                              "MaxNs", "StdDev"])
            w.writeheader()
            for r in stats:
                w.writerow(r)


def sweep_dispatches(counters_of):
    out = []
    for axis, rnd, rht in bench.SWEEP_VARIANTS:
        amax = ("k_amax_rht_" + ("rows" if axis else "cols")) if rht else "k_amax_flat"
        enc = "k_quant_%s<unsigned short, %s, %s>" % ("rows" if axis else "cols", str(rnd == "sr").lower(),
                                                      str(rht).lower())
        for c in range(bench.SWEEP_CALLS):
            if c == 2:       # the spin kernel queued ahead of the timed calls
                out.append(("at::cuda::(anonymous namespace)::spin_kernel(long)", 1, 200000, counters_of("spin")))
            out.append(("nvfp4::k_meta_init(float*)", 64, 2000, counters_of("meta")))
            out.append((f"void nvfp4::{amax}<unsigned short>(...)", 262144, 90000, counters_of("amax")))
            out.append((f"void nvfp4::{enc}(...)", N_SWEEP // 16, 110000, counters_of("enc")))
    return out


def test_quant_counter_table(tmp_path):
    # the copy reads 2x and writes 1x its size in KiB, so the scales are 0.5 and 1
    kib = bench.CALIB_BYTES / 1024
    step = [("void nvfp4::k_quant_rows<unsigned short, false, false>(...)", 4096 * 5120 // 16, 30000, {})]
    fetch = {"meta": 0.0, "spin": 0.0, "amax": 2 * 2 * N_SWEEP / 1024, "enc": 2 * 2 * N_SWEEP / 1024}
    write = {"meta": 0.0, "spin": 0.0, "amax": 0.0, "enc": (N_SWEEP // 2 + N_SWEEP // 16) / 1024}
    for tag, cname, per, copyv in (("fetch", "FETCH_SIZE", fetch, 2 * kib), ("write", "WRITE_SIZE", write, kib)):
        disp = [(COPY, 1, 100000, {cname: copyv})]
        disp += [(n, g, dur, {cname: 1.0}) for n, g, dur, _ in step]
        disp += sweep_dispatches(lambda kind: {cname: per[kind]})
        write_run(str(tmp_path / tag), disp)
    # VALU run: 2e5 GPU cycles per dispatch (GRBM_GUI_ACTIVE counts 8 XCDs), half the SIMD cycles on VALU
    g = 2.0e5
    valu = [(COPY, 1, 100000, {"GRBM_GUI_ACTIVE": 8.0, "SQ_INSTS_VALU": 0.0})]
    valu += sweep_dispatches(lambda kind: {"GRBM_GUI_ACTIVE": 8.0 * g, "SQ_INSTS_VALU": 0.5 * g * 1024 / 4})
    write_run(str(tmp_path / "valu"), valu)
    # kernel-trace run: the encodes take 120 us there (110 us in the counter runs)
    trace = [(n, g_, 120000 if "k_quant" in n else dur) for n, g_, dur, _ in sweep_dispatches(lambda kind: {})]
    write_trace(str(tmp_path / "trace"), [("void nvfp4::k_quant_rows<unsigned short, false, false>(...)",
                                           4096 * 5120 // 16, 30000)] + trace)
    md = bench.reduce_quant_counters(str(tmp_path / "fetch"), str(tmp_path / "write"), str(tmp_path / "valu"),
                                     str(tmp_path / "trace"))
    rows = [l for l in md.splitlines() if l.startswith("| axis")]
    assert len(rows) == 2 * len(bench.SWEEP_VARIANTS)
    first_enc = [c.strip() for c in rows[1].split("|")]
    assert first_enc[2] == "encode" and "k_quant_rows<unsigned short, false, false>" in first_enc[3]
    assert first_enc[4] == "120.0"                                  # us from the kernel trace
    assert first_enc[5] == "537 (537)"                               # 2 B/element read, scaled by 0.5
    assert first_enc[6] == "151 (151)"
    n = N_SWEEP
    assert first_enc[7] == f"{(2 * n + n // 2 + n // 16) / 120e-6 / 1e9:.0f}"   # trace time
    assert first_enc[8] == "0.50"                                    # VALU busy
    assert first_enc[9] == "110.0"                                   # the counter run's own time
    assert first_enc[10] == "1.82"                                   # 2e5 cycles in 110 us
    assert "(2.00 and 1.00)" not in md and "(0.50 and 1.00)" in md


def test_quant_counter_order_is_checked(tmp_path):
    kib = bench.CALIB_BYTES / 1024
    for tag, cname in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE"), ("valu", "SQ_INSTS_VALU")):
        disp = [(COPY, 1, 100000, {cname: kib, "GRBM_GUI_ACTIVE": 8.0})]
        sw = sweep_dispatches(lambda kind: {cname: 1.0, "GRBM_GUI_ACTIVE": 8.0})
        sw[40], sw[41] = sw[41], sw[40]          # a dispatch out of the expected order
        write_run(str(tmp_path / tag), disp + sw)
    with pytest.raises(SystemExit, match="unexpected dispatch order"):
        bench.reduce_quant_counters(str(tmp_path / "fetch"), str(tmp_path / "write"), str(tmp_path / "valu"),
                                    str(tmp_path / "valu"))


def test_gemm_launches():
    """The layer GEMMs' stream-K grids on 256 CUs: 320, 640 and 1600 tiles
    leave 0, 256 and 1280 data-parallel tiles plus one round."""
    kinds = dict(bench.gemm_kinds())
    assert kinds["fprop"] == ("k_gemm_nvfp4_sk<true, true>", 256 * 256)
    assert kinds["dgrad"] == ("k_gemm_nvfp4_sk<false, true>", 512 * 256)
    assert kinds["wgrad"] == ("k_gemm_nvfp4_sk<false, true>", 1536 * 256)
    assert bench.dominant_launch() == kinds["wgrad"]


def test_traffic_reduction(tmp_path):
    kib = bench.CALIB_BYTES / 1024
    name, grid = bench.dominant_launch()
    dom = f"void nvfp4::{name}(...)"
    # dgrad's launch of the same kernel (smaller grid) is not counted
    write_run(str(tmp_path / "f"), [(COPY, 1, 100, {"FETCH_SIZE": 2 * kib}), (dom, grid, 100, {"FETCH_SIZE": 1000.0}),
                                    (dom, 512 * 256, 100, {"FETCH_SIZE": 7.0}),
                                    (dom, grid, 100, {"FETCH_SIZE": 3000.0})])
    write_run(str(tmp_path / "w"), [(COPY, 1, 100, {"WRITE_SIZE": kib}), (dom, grid, 100, {"WRITE_SIZE": 500.0})])
    prof = bench.reduce_traffic(str(tmp_path / "f"), str(tmp_path / "w"))
    assert prof["fetch_scale"] == pytest.approx(0.5) and prof["write_scale"] == pytest.approx(1.0)
    assert prof["fetch_bytes_per_launch"] == pytest.approx(2000 * 1024 * 0.5)
    assert prof["write_bytes_per_launch"] == pytest.approx(500 * 1024)
    assert prof["dispatches"] == [2, 1]


def test_busy_reduction(tmp_path):
    g = 2.0e6                                    # GPU cycles of the kernel (GRBM_GUI_ACTIVE / 8)
    counters = {"GRBM_GUI_ACTIVE": 8 * g, "SQ_VALU_MFMA_BUSY_CYCLES": g * 1024 * 0.5, "SQ_BUSY_CYCLES": 1.0,
                "SQ_ACTIVE_INST_VALU": g * 1024 / 8, "SQ_INSTS_MFMA": 10.0, "SQ_INSTS_VALU": 60.0,
                "SQ_WAIT_INST_ANY": g * 1024 / 16, "SQ_LDS_BANK_CONFLICT": g * 256 * 0.1}
    f32 = "void nvfp4::k_gemm_nvfp4_sk<false, true>(...)"
    write_run(str(tmp_path / "b"), [("void nvfp4::k_gemm_nvfp4_sk<true, true>(...)", 256 * 256, 1_000_000, counters),
                                    (f32, 512 * 256, 1_000_000, counters),
                                    (f32, 1536 * 256, 1_000_000, counters),
                                    (f32, 1536 * 256, 1_000_000, counters)])
    md = bench.reduce_busy(str(tmp_path / "b"))
    rows = [line for line in md.splitlines() if line.startswith("| k_gemm")]
    assert [r.split("|")[1].strip() for r in rows] == [
        "k_gemm_nvfp4_sk<true, true> (fprop)", "k_gemm_nvfp4_sk<false, true> (dgrad)",
        "k_gemm_nvfp4_sk<false, true> (wgrad)"]
    row = [c.strip() for c in md.splitlines()[-1].split("|")]
    # dispatches, ms, GHz, MFMA busy, VALU/MFMA, VALU active, issue wait, LDS conflict
    assert row[2:10] == ["2", "1.000", "2.00", "0.500", "6.00", "0.500", "0.250", "0.100"]


def test_trace_reduction(tmp_path):
    """GEMM launches classified by kernel and grid, the timed steps' average
    set against the bench line's events, and the sweep's passes summed."""
    steps, warmup = 3, 1
    kinds = dict(bench.gemm_kinds())
    disp = []
    for k in range(warmup + 2 * steps):      # warm-up, timed and breakdown steps
        for name, us in (("fprop", 200), ("dgrad", 1200), ("wgrad", 1250 + 10 * k)):
            kern, grid = kinds[name]
            disp.append((f"void nvfp4::(anonymous namespace)::{kern}(...)", grid, us * 1000))
    disp += [(n, g, dur) for n, g, dur, _ in sweep_dispatches(lambda kind: {})]
    stats = [{"Name": "void nvfp4::(anonymous namespace)::k_gemm_nvfp4_sk<false, true>(...)", "Calls": 8,
              "TotalDurationNs": 8e6, "AverageNs": 1e6, "Percentage": 50.0, "MinNs": 9e5, "MaxNs": 1.1e6,
              "StdDev": 1.0}]
    write_trace(str(tmp_path / "t"), disp, stats)
    sweep = {f"axis{a} {r}{'+rht' if h else ''}": {"ms": 0.21} for a, r, h in bench.SWEEP_VARIANTS}
    line = {"value": 1000.0, "unit": "TFLOP/s", "ms_per_step": 3.2, "steps": steps, "warmup": warmup,
            "roofline": {"avg_launch_ms": 1.3, "frac": 0.53}, "breakdown": {"gemm fprop": {"ms": 0.21}},
            "quantize_sweep_32768x8192_bf16": sweep}
    bj = tmp_path / "bench.json"
    bj.write_text("log line\n" + __import__("json").dumps(line) + "\n")
    md = bench.reduce_trace(str(tmp_path / "t"), str(bj))
    wg = [l for l in md.splitlines() if l.startswith("| wgrad")][0].split("|")
    assert wg[4].strip() == str(warmup + 2 * steps)
    assert [c.strip() for c in wg[5:8]] == ["1.2700", "1.2600", "1.2800"]   # the timed steps' launches
    assert wg[8].strip() == "1.3000"                                         # the breakdown steps'
    assert wg[9].strip() == "1.3"                                            # the timed pass's events
    assert f"{1.27:.4f} ms, i.e. frac {2 * 5120 * 20480 * 8192 / 1.27e-3 / 1e12 / 2500:.4f}" in md
    fp = [l for l in md.splitlines() if l.startswith("| fprop")][0].split("|")
    assert fp[5].strip() == "0.2000"
    assert fp[9].strip() == "0.21"                                            # the breakdown pass's events
    sw = [l for l in md.splitlines() if l.startswith("| axis1 rne |")][0].split("|")
    assert [c.strip() for c in sw[2:6]] == ["90.0", "110.0", "202.0", "210.0"]
    assert "`k_gemm_nvfp4_sk<false, true>`" in md
