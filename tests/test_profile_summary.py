"""Host logic of block_copy_amd/profile_summary.py on small synthetic
rocprofv3 CSV files: the per-kernel trace table, the attribution of decode
steps to copy bursts, and the calibrated byte counters."""
import csv
import json
import os
import types

from block_copy_amd import profile_summary as PS

TRACE_COLS = ["Kind", "Queue_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp",
              "LDS_Block_Size", "Scratch_Size", "VGPR_Count", "Workgroup_Size_X", "Grid_Size_X"]
H2D = "kvc::(anonymous namespace)::kvcopy_h2d_kernel(kvc::ChunkRec const*, unsigned int)"
D2H = "kvc::(anonymous namespace)::kvcopy_d2h_sc1_kernel(kvc::ChunkRec const*, unsigned int)"
GEMV = "(anonymous namespace)::gemv_bf16_kernel(unsigned short const*, int, int)"


def _write(path, cols, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _k(name, t0, t1, q="1", grid=32768, wg=256):
    return {"Kind": "KERNEL_DISPATCH", "Queue_Id": q, "Kernel_Name": name,
            "Start_Timestamp": t0, "End_Timestamp": t1, "LDS_Block_Size": 0,
            "Scratch_Size": 0, "VGPR_Count": 48, "Workgroup_Size_X": wg, "Grid_Size_X": grid}


def test_trace_table(tmp_path, capsys):
    d = tmp_path / "kt"
    _write(str(d / "kt_kernel_trace.csv"), TRACE_COLS,
           [_k(H2D, 0, 1000_000), _k(H2D, 2000_000, 4000_000), _k(D2H, 0, 1500_000)])
    PS.trace(types.SimpleNamespace(dir=str(d), name="t", command="cmd", workload=""))
    out = capsys.readouterr().out
    row = next(ln for ln in out.splitlines() if ln.startswith("| kvcopy_h2d_kernel "))
    cells = [c.strip() for c in row.strip("|").split("|")]
    # kernel, grid, workgroup, calls, average, median, min, max (us)
    assert cells[:8] == ["kvcopy_h2d_kernel", "32768", "256", "2", "1500.0", "1500.0", "1000.0",
                         "2000.0"]
    assert "| kvcopy_d2h_sc1_kernel | 32768 | 256 | 1 | 1500.0 |" in out


def test_bursts_attribute_steps(tmp_path, capsys):
    """Steps of 2 decode kernels, 10 us each; one burst (an H2D and a D2H
    kernel that overlap) covers the second step only."""
    d = tmp_path / "kt"
    rows = []
    t = 0
    for step in range(4):
        for k in range(2):
            rows.append(_k(GEMV, t, t + 10_000, q="4", grid=1024))
            t += 10_000
        t += 5_000
    s2 = 25_000   # the second step runs from 25 us to 45 us
    rows += [_k(H2D, s2 + 1_000, s2 + 15_000, grid=1024), _k(D2H, s2 + 5_000, s2 + 18_000, q="2",
                                                            grid=1024)]
    _write(str(d / "kt_kernel_trace.csv"), TRACE_COLS, rows)
    PS.bursts(types.SimpleNamespace(dir=str(d), name="b", command="cmd", workload="",
                                    decode="gemv_bf16_kernel", per_step=2))
    out = capsys.readouterr().out
    assert "8 decode kernels (4 steps of 2)" in out and "2 copy kernels in 1 bursts" in out
    outside = next(ln for ln in out.splitlines() if ln.startswith("| outside every burst"))
    assert [c.strip() for c in outside.strip("|").split("|")][3] == "3"      # steps outside
    burst = next(ln for ln in out.splitlines() if ln.startswith("| bursts of"))
    cells = [c.strip() for c in burst.strip("|").split("|")]
    assert "kvcopy_h2d_kernel x4 WGs (queue 1)" in cells[0] and "kvcopy_d2h_sc1_kernel" in cells[0]
    assert cells[1] == "1" and cells[2] == "17"          # one burst of 17 us
    assert cells[3] == "1" and cells[4] == "20.0"        # one 20 us step overlaps it
    assert cells[7] == "2"                               # both of its decode kernels


def test_counters_scale_by_the_calibration_kernel(tmp_path):
    cols = ["Counter_Name", "Kernel_Name", "Grid_Size_X", "Counter_Value"]
    neg = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>"
    fdir, wdir = tmp_path / "f", tmp_path / "w"
    # the calibration kernel moves 64 MiB each way and reads FETCH_SIZE = half of it
    _write(str(fdir / "pmc_counter_collection.csv"), cols,
           [{"Counter_Name": "FETCH_SIZE", "Kernel_Name": neg, "Grid_Size_X": 1,
             "Counter_Value": 32768}] * 3 +
           [{"Counter_Name": "FETCH_SIZE", "Kernel_Name": H2D, "Grid_Size_X": 16384,
             "Counter_Value": 32000}] * 5)
    _write(str(wdir / "pmc_counter_collection.csv"), cols,
           [{"Counter_Name": "WRITE_SIZE", "Kernel_Name": neg, "Grid_Size_X": 1,
             "Counter_Value": 65536}] * 3 +
           [{"Counter_Name": "WRITE_SIZE", "Kernel_Name": H2D, "Grid_Size_X": 16384,
             "Counter_Value": 64000}] * 5)
    out = tmp_path / "out"
    out.mkdir()
    PS.counters(types.SimpleNamespace(fetch=str(fdir), write=str(wdir), name="x",
                                      fetch_command="f", write_command="w", out_dir=str(out)))
    j = json.load(open(out / "counters_x.json"))
    k = j["kernels"]["kvcopy_h2d_kernel"]
    assert k["dispatches"] == 5 and k["grid_work_items"] == 16384
    assert k["fetch_bytes_per_dispatch_scaled"] == 32000 * 1024 * 2
    assert k["write_bytes_per_dispatch_scaled"] == 64000 * 1024
    assert (out / "counters_x.md").exists()
