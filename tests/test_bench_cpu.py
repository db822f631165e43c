"""Host-only checks of the benchmark driver: it measures one GPU and says so
when asked for more, and its trace summariser labels every workload."""

import json
import os
import subprocess
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
