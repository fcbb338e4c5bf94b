"""Host-side logic of bench.py (CPU): the one-GPU guard and the rocprofv3
summaries that profiles/ is made from, on hand-made CSV files."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def write_csv(path, rows):
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        w.writeheader()
        w.writerows(rows)


def trace_row(name, grid, wg, start, us):
    return {"Kernel_Name": name, "Grid_Size_X": grid, "Workgroup_Size_X": wg,
            "Start_Timestamp": start, "End_Timestamp": start + int(us * 1000)}


def test_trace_summary_groups_by_kernel_and_grid(tmp_path):
    k = "void ec::(anonymous namespace)::gemm_tiled_bf16_kernel<256, 192>(ec::GP)"
    rows = [trace_row(k, 256 * 512, 512, 0, 100.0), trace_row(k, 256 * 512, 512, 10 ** 6, 110.0),
            trace_row(k, 256 * 512, 512, 2 * 10 ** 6, 4.0),          # a gated launch that exited
            trace_row(k, 128 * 512, 512, 3 * 10 ** 6, 50.0),         # same kernel, other grid
            trace_row("void ec::(anonymous namespace)::select_rows_kernel(int)", 64, 64, 4 * 10 ** 6, 5.0)]
    write_csv(tmp_path / "run" / "t_kernel_trace.csv", rows)
    table = bench.summarize_trace(str(tmp_path), 6.0).splitlines()
    body = {r.split("|")[1].strip() + " " + r.split("|")[2].strip(): [c.strip() for c in r.split("|")[3:-1]]
            for r in table[2:]}
    assert body["`gemm_tiled_bf16_kernel<256, 192>` 256"] == ["3", "2", "105.0", "110.0", "0.21"]
    assert body["`gemm_tiled_bf16_kernel<256, 192>` 128"] == ["1", "1", "50.0", "50.0", "0.05"]
    assert body["`select_rows_kernel` 1"] == ["1", "0", "-", "5.0", "0.01"]
    assert table[2].startswith("| `gemm_tiled_bf16_kernel<256, 192>` | 256 |")   # largest total first


def counter_rows(dispatch, name, grid, us, counters):
    return [{"Dispatch_Id": dispatch, "Kernel_Name": name, "Grid_Size": grid, "Workgroup_Size": 256,
             "Start_Timestamp": 0, "End_Timestamp": int(us * 1000), "Counter_Name": c,
             "Counter_Value": v} for c, v in counters.items()]


def test_counter_summary_scales_flops_and_leaves_out_exited_dispatches(tmp_path):
    k = "void ec::(anonymous namespace)::attn_bf16_kernel<128>(ec::BP)"
    # run A: two working dispatches and one that exited (no MFMA work)
    a = (counter_rows(1, k, 256 * 256, 100.0, {"SQ_INSTS_VALU_MFMA_MOPS_BF16": 2e6,
                                                "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * 100 * 2400 * 1024,
                                                "GRBM_GUI_ACTIVE": 0.0})
         + counter_rows(2, k, 256 * 256, 300.0, {"SQ_INSTS_VALU_MFMA_MOPS_BF16": 2e6,
                                                  "SQ_VALU_MFMA_BUSY_CYCLES": 0.25 * 300 * 2400 * 1024,
                                                  "GRBM_GUI_ACTIVE": 8 * 300 * 1000 * 2.0})
         + counter_rows(3, k, 256 * 256, 3.0, {"SQ_INSTS_VALU_MFMA_MOPS_BF16": 0.0,
                                                "SQ_VALU_MFMA_BUSY_CYCLES": 0.0, "GRBM_GUI_ACTIVE": 0.0}))
    lm = "void ec::(anonymous namespace)::lmhead_packed_kernel<3>(ec::(anonymous namespace)::GP)"
    a += counter_rows(4, lm, 659 * 256, 190.0, {"SQ_INSTS_VALU_MFMA_MOPS_BF16": 6.5e7,
                                               "SQ_VALU_MFMA_BUSY_CYCLES": 0.07 * 190 * 2400 * 1024,
                                               "GRBM_GUI_ACTIVE": 8 * 190 * 1000 * 2.4})
    a += counter_rows(5, "void at::native::fill_kernel(int)", 64, 2.0, {"SQ_INSTS_VALU_MFMA_MOPS_BF16": 0.0})
    write_csv(tmp_path / "a" / "x_counter_collection.csv", a)
    table = bench.summarize_counters([str(tmp_path / "a")]).splitlines()
    assert len(table) == 4                                       # torch's own kernels are left out
    lm_cells = [c.strip() for c in table[2].split("|")[1:-1]]   # most flops first
    assert lm_cells[0] == "`lmhead_packed_kernel<3>`" and lm_cells[1] == "659" and lm_cells[2] == "1 / 1"
    table = [table[0], table[1], table[3]]
    cells = [c.strip() for c in table[2].split("|")[1:-1]]
    assert cells[0] == "`attn_bf16_kernel<128>`" and cells[1] == "256"
    assert cells[2] == "2 / 3"                                   # dispatches with work / all
    assert cells[3] == "200.0"                                   # median time of the working ones
    assert cells[4] == "1.02"                                    # 2e6 MFMA ops x 512 flops
    assert float(cells[7]) == pytest.approx(0.375, abs=1e-3)     # median of 0.5 and 0.25
    assert cells[8] == "2.00"                                    # clock from the dispatch over 200 us
