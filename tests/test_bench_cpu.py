"""Host-only checks of the benchmark driver: it measures one GPU and says so
when asked for more, and its trace summariser labels every workload."""

import json
import os
import subprocess

import numpy as np
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_trace_summary_labels_each_workload(tmp_path):
    """A synthetic kernel trace: launches of one kernel on one grid, run as two
    workloads one after another, are split at the pause between them."""
    import csv
    trace = tmp_path / "t_kernel_trace.csv"
    fields = ["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "LDS_Block_Size", "VGPR_Count", "Accum_VGPR_Count",
              "Start_Timestamp", "End_Timestamp"]
    rows, t = [], 0
    for dur, gap_after in [(100_000, 1_000)] * 8 + [(100_000, 5_000_000)] + [(700_000, 1_000)] * 8:
        rows.append({"Kernel_Name": "void w4a16::(anonymous namespace)::gemm_kernel<128, false, true>(int)",
                     "Grid_Size_X": 131072, "Workgroup_Size_X": 512, "LDS_Block_Size": 0, "VGPR_Count": 92,
                     "Accum_VGPR_Count": 0, "Start_Timestamp": t, "End_Timestamp": t + dur})
        t += dur + gap_after
    with open(trace, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)
    sys.path.insert(0, ROOT)
    import bench
    out_dir = tmp_path / "profiles"
    out_dir.mkdir()
    old_root = bench.ROOT
    try:
        bench.ROOT = str(tmp_path)
        bench.trace_summary(str(trace), "cmd")
    finally:
        bench.ROOT = old_root
    text = (out_dir / "gemm_prefill_27b_ffn.kernel_trace.md").read_text()
    lines = [ln for ln in text.splitlines() if ln.startswith("| gemm_kernel")]
    assert len(lines) == 2
    assert "| M=512 |" in lines[0] and "| 9 | 100.00 |" in lines[0]
    assert "| M=4096 |" in lines[1] and "| 8 | 700.00 |" in lines[1]


# ---- counter tables (rocprofv3 --pmc counter_collection.csv) ----
COUNTER_FIELDS = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "LDS_Block_Size", "Counter_Name", "Counter_Value",
                  "Start_Timestamp", "End_Timestamp"]


def _write_counters(path, dispatches):
    """dispatches: (kernel name, grid, start ns, duration ns, {counter: value}) in order."""
    import csv
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COUNTER_FIELDS)
        w.writeheader()
        for i, (name, grid, start, dur, counters) in enumerate(dispatches):
            for c, v in counters.items():
                w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Grid_Size": grid, "LDS_Block_Size": 0,
                            "Counter_Name": c, "Counter_Value": v, "Start_Timestamp": start,
                            "End_Timestamp": start + dur})


def _bench():
    sys.path.insert(0, ROOT)
    import bench
    return bench


def test_counter_dispatches_labelled_by_grid_and_time(tmp_path):
    """The grouped GEMM family: the smallest grid is the one-GPU shard, the middle grid
    holds four workloads run one after another (split at the pauses), the largest the
    MoE FFN's down projection; the M = 1 GEMV's three workloads share one grid."""
    bench = _bench()
    grouped = "void w4a16::(anonymous namespace)::grouped_gemm_kernel<32, true, false>(int)"
    gemv = "void w4a16::(anonymous namespace)::gemv_kernel<1, false>(int)"
    d, t = [], 0
    for grid, runs in ((393216, 4), (1572864, 1), (49152, 1)):
        for r in range(runs):
            for _ in range(5):
                d.append((grouped, grid, t, 1000, {"FETCH_SIZE": float(grid + r)}))
                t += 2000
            t += 10_000_000
    for r in range(3):
        for _ in range(6):
            d.append((gemv, 131072, t, 1000, {"FETCH_SIZE": float(r)}))
            t += 2000
        t += 10_000_000
    path = tmp_path / "p_counter_collection.csv"
    _write_counters(path, d)
    got = bench._labelled_dispatches(str(path))
    lab = bench.TRACE_LABELS["grouped_gemm_kernel<32, true, false>"]["by_grid"]
    fam = "grouped_gemm_kernel<32, true, false>"
    assert {x["FETCH_SIZE"] for x in got[(fam, lab[0][0])]} == {49152.0}
    for r, name in enumerate(lab[1]):
        assert {x["FETCH_SIZE"] for x in got[(fam, name)]} == {393216.0 + r}, name
    assert {x["FETCH_SIZE"] for x in got[(fam, lab[2][0])]} == {1572864.0}
    for r, name in enumerate(bench.TRACE_LABELS["gemv_kernel<1, false>"]):
        assert {x["FETCH_SIZE"] for x in got[("gemv_kernel<1, false>", name)]} == {float(r)}, name


def test_traffic_table_scales_by_the_copy_calibration(tmp_path):
    bench = _bench()
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "gemv.traffic.json").write_text(json.dumps({"fetch_scale": 2.0, "write_scale": 1.0}))
    # the two workloads run kernels of one family with different ring depths
    np4 = ["void w4a16::(anonymous namespace)::gemv_mfma_kernel<4, 128, false, 3>(int)",
           "void w4a16::(anonymous namespace)::gemv_mfma_kernel<4, 128, false, 4>(int)"]
    fetch, write, t = [], [], 0
    for r, (kib_read, kib_write) in enumerate(((6000.0, 40.0), (20000.0, 136.0))):
        for _ in range(3):
            fetch.append((np4[r], 131072, t, 1000, {"FETCH_SIZE": kib_read}))
            write.append((np4[r], 131072, t, 1000, {"WRITE_SIZE": kib_write}))
            t += 2000
        t += 10_000_000
    _write_counters(tmp_path / "f.csv", fetch)
    _write_counters(tmp_path / "w.csv", write)
    old = bench.ROOT
    try:
        bench.ROOT = str(tmp_path)
        bench.traffic_table(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "t.md"), "cmd")
    finally:
        bench.ROOT = old
    rows = {ln.split("|")[2].strip(): ln for ln in (tmp_path / "t.md").read_text().splitlines()
            if ln.startswith("| gemv_mfma")}
    # N = 5120 ran first: 6000 KiB x 1024 x 2 = 12.29 MB read, 40 KiB = 0.041 MB written
    assert "| 12.29 | 0.041 | 13.56 | 0.041 |" in rows["N=5120"]
    assert "| 40.96 | 0.139 | 46.00 | 0.139 |" in rows["N=17408"]


def test_stream_counter_table_per_wave_and_fractions(tmp_path):
    bench = _bench()
    m1 = "void w4a16::(anonymous namespace)::gemv_kernel<1, true>(int)"
    p1 = [(m1, 131072, 0, 20_000, {"SQ_WAVES": 2048.0, "SQ_WAVE_CYCLES": 1000.0, "SQ_INSTS_VALU": 4096.0,
                                   "SQ_ACTIVE_INST_ANY": 500.0, "SQ_WAIT_ANY": 250.0})]
    p2 = [(m1, 131072, 0, 20_000, {"TCP_TCC_READ_REQ": 10.0, "TCP_TCC_READ_REQ_LATENCY": 7000.0})]
    _write_counters(tmp_path / "a.csv", p1)
    _write_counters(tmp_path / "b.csv", p2)
    bench.stream_counter_table([str(tmp_path / "a.csv"), str(tmp_path / "b.csv")], str(tmp_path / "s.md"), "cmd")
    row = [ln for ln in (tmp_path / "s.md").read_text().splitlines() if ln.startswith("| gemv_kernel<1, true>")][0]
    cells = [c.strip() for c in row.split("|")[1:-1]]
    # kernel, workload, dispatches, mean us, VALU/wave, SALU, LDS, MFMA, VMEM, active, VALU busy, wait, stall, latency
    assert cells[2:5] == ["1", "20.00", "2"]
    assert cells[9] == "0.500" and cells[11] == "0.250" and cells[13] == "700"


def test_gemm_counter_summary_ratios(tmp_path):
    bench = _bench()
    g = "void w4a16::(anonymous namespace)::gemm_kernel<128, false, true>(int)"
    cycles = 1_000_000.0
    d, t = [], 0
    for r, busy in enumerate((0.4, 0.6)):
        for _ in range(3):
            d.append((g, 131072, t, 500_000, {"GRBM_GUI_ACTIVE": cycles * bench.XCDS,
                                              "SQ_VALU_MFMA_BUSY_CYCLES": busy * 1024 * cycles,
                                              "SQ_INSTS_LDS_LOAD_BANDWIDTH": 64.0 * 256 * cycles / 64,
                                              "SQ_INSTS_VALU": 600.0, "SQ_INSTS_MFMA": 100.0}))
            t += 600_000
        t += 10_000_000
    d.append(("Cijk_Ailk_Bljk_HHS_BH_Bias_HA_S_SAV_UserArgs_MT256x256x64_MI16x16x1_SN_xyz", 65536, t, 500_000,
              {"GRBM_GUI_ACTIVE": cycles * bench.XCDS, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * 1024 * cycles}))
    _write_counters(tmp_path / "g.csv", d)
    bench.counter_summary([str(tmp_path / "g.csv")], str(tmp_path / "g.md"), "cmd")
    text = (tmp_path / "g.md").read_text()
    rows = [ln for ln in text.splitlines() if ln.startswith("| gemm_kernel") or ln.startswith("| vendor")]
    by = {ln.split("|")[2].strip(): [c.strip() for c in ln.split("|")[1:-1]] for ln in rows}
    # 1e6 cycles in 500 us: 2.00 GHz; LDS 64 B/clk/CU; 6 VALU per MFMA
    assert by["M=512"][4:7] == ["2.00", "0.400", ""] and by["M=512"][8:10] == ["64.0", "6.00"]
    assert by["M=4096"][5] == "0.600"
    vendor = [v for k, v in by.items() if k.startswith("Cijk_")]
    assert len(vendor) == 1 and vendor[0][5] == "0.500"


def test_wave_timeline_stats_and_table(tmp_path):
    """Synthetic stamps (10 ns ticks): workgroups start 0.1 us apart by index modulo 4,
    stage at +1 us, finish their first unit at +1.5 us, their loop at +6 us (+7 us for
    wave 7) and end 0.5 us later; unrecorded slots are zero."""
    bench = _bench()
    launches = 3
    a = np.zeros((launches, 256, 8, bench.STAMP_SLOTS), np.uint64)
    base = 1_000_000
    for r in range(launches):
        for b in range(256):
            for w in range(8):
                t = base + r * 100_000 + (b % 4) * 10
                loop_end = t + (700 if w == 7 else 600)
                a[r, b, w, :6] = [t, t + 100, t + 150, loop_end, loop_end + 20, loop_end + 50]
    st = bench.timeline_stats(a)
    assert st["start"]["max"] == 300.0 and abs(st["start"]["mean"] - 150.0) < 1e-9
    assert st["first unit"]["max"] == 1800.0
    assert abs(st["loop"] - 4625.0) < 1e-9          # mean loop end 6275 (one wave in eight at +7 us) - 1650
    assert st["loop end"]["max"] == 7300.0 and st["span"] == 7800.0
    probe = np.zeros_like(a)
    probe[:, :, :, 0] = a[:, :, :, 0]
    probe[:, :, :, 2] = a[:, :, :, 0] + 120
    probe[:, :, :, 3] = a[:, :, :, 0] + 580
    probe[:, :, :, 5] = a[:, :, :, 0] + 600
    sp = bench.timeline_stats(probe)
    assert "staged" not in sp and sp["span"] == 6300.0
    out = tmp_path / "t.md"
    bench.timeline_table({"probe": (sp, 8.8, None), "gemv": (st, 10.5, "probe")}, "cmd", str(out))
    row = [ln for ln in out.read_text().splitlines() if ln.startswith("| gemv")][0]
    cells = [c.strip() for c in row.split("|")[1:-1]]
    assert cells[1] == "10.50" and cells[11] == "1.50"      # span 7.8 us against the probe's 6.3 us
