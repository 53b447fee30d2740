"""The profile summarizer of bench.py (host logic, no GPU): from rocprofv3-shaped CSVs it must
calibrate the PMC byte counters on the probe copy, find the roofline kernel by its instantiation
name, and write the traffic record the benchmark reads."""
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

CAL = "void (anonymous namespace)::k_stream_mix<true, true>(uint4 const*, uint4*, long, int, int)"
GEMM = "void pmn::k_nvfp4_grouped_gemm<2, false>(pmn::FwdArgs)"
QUANT = "void pmn::k_nvfp4_rows<2, true>(unsigned short const*, long, long)"


def _write(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_summary_calibrates_counters_and_finds_the_roofline_kernel(tmp_path):
    d = tmp_path / "prof"
    cal_grid = str(bench.CALIB_GRID * 256)
    gemm_grid = "1245184"
    # trace: two launches of the GEMM, 3.0 and 3.2 ms
    _write(str(d / "kt" / "x_kernel_stats.csv"),
           [dict(Name=GEMM, Calls=2, AverageNs=3.1e6, MinNs=3.0e6, MaxNs=3.2e6, Percentage=90.0)])
    _write(str(d / "kt" / "x_kernel_trace.csv"),
           [dict(Kernel_Name=GEMM, Grid_Size_X=gemm_grid, Grid_Size_Y=1, Start_Timestamp=0, End_Timestamp=3000000),
            dict(Kernel_Name=GEMM, Grid_Size_X=gemm_grid, Grid_Size_Y=1, Start_Timestamp=5000000,
                 End_Timestamp=8200000)])
    # FETCH_SIZE reads half of the copy's 1 GiB (factor 2), WRITE_SIZE all of it (factor 1)
    for sub, cal_kib, gemm_kib in (("fetch", 524288.0, 1000000.0), ("write", 1048576.0, 400000.0)):
        _write(str(d / sub / "x_counter_collection.csv"),
               [dict(Kernel_Name=CAL, Grid_Size=cal_grid, Counter_Value=cal_kib),
                dict(Kernel_Name=GEMM, Grid_Size=gemm_grid, Counter_Value=gemm_kib),
                dict(Kernel_Name=QUANT, Grid_Size="4194304", Counter_Value=10.0)])
    rows = []
    for name, grid, dur, counters in ((GEMM, gemm_grid, 3.0e6, dict(GRBM_GUI_ACTIVE=8 * 1.9e9 * 3.0e-3,
                                                                    SQ_VALU_MFMA_BUSY_CYCLES=1024 * 1.9e9 * 3.0e-3 * 0.6,
                                                                    SQ_ACTIVE_INST_VALU=0.0)),):
        for cn, cv in counters.items():
            rows.append(dict(Dispatch_Id=1, Kernel_Name=name, Grid_Size=grid, Counter_Name=cn, Counter_Value=cv,
                             Start_Timestamp=0, End_Timestamp=int(dur)))
    _write(str(d / "clock" / "x_counter_collection.csv"), rows)
    bench_line = dict(ms_per_step=16.4, value=1055.0,
                      roofline=dict(ms_per_launch=3.1, achieved=1241.0, frac=0.4966, peak=2500.0,
                                    flops_per_launch=3.848e12))
    (d / "bench.json").write_text(json.dumps(bench_line) + "\n")
    out = tmp_path / "out"
    out.mkdir()
    bench.summarize_profiles(str(d), out_dir=str(out))
    rec = json.loads((out / "traffic_gemm_fwd.json").read_text())
    assert abs(rec["fetch_bytes_per_launch"] - 1000000.0 * 2 * 1024) < 1
    assert abs(rec["write_bytes_per_launch"] - 400000.0 * 1 * 1024) < 1
    assert rec["kernel"].endswith("4864 workgroups)")
    stats = (out / "ep48_layer_step_kernel_stats.md").read_text()
    assert "averages 3.100 ms per launch" in stats          # the mean of the two traced launches
    assert "FETCH_SIZE x 2.000" in (out / "ep48_layer_step_hbm_traffic.md").read_text()
    clock = (out / "ep48_layer_step_clock_mfma.md").read_text()
    assert "| 1.90 | 0.60 |" in clock                       # clock and MFMA busy at that clock
