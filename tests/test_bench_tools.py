"""Host-side measurement tooling of bench.py, on the CPU: the refusal of more than one GPU, and the
rocprofv3 counter summaries (--pmc-summary, --pmc-table) on hand-made counter files whose expected
figures follow from the copy calibration by hand."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size", "Kernel_Id",
        "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count",
        "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
UNMASKED = ("void qfa::(anonymous namespace)::attn_fwd_kernel<128, 1, 4, false, false, false, false, false, false, "
            "false>(qfa::AttnArgs, int, int)")


def _write(path, counter, rows):
    """rows: (kernel name, grid, [value per XCD row, ...]) per dispatch, values in KiB."""
    os.makedirs(path)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COLS)
        w.writeheader()
        for i, (name, grid, vals) in enumerate(rows):
            for v in vals:   # one row per XCD, summed per dispatch by the summaries
                w.writerow({c: 0 for c in COLS} | {"Dispatch_Id": i + 1, "Kernel_Name": name, "Grid_Size": grid,
                                                   "Counter_Name": counter, "Counter_Value": v,
                                                   "Start_Timestamp": 1000, "End_Timestamp": 1000 + 1000 * (i + 1)})


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_pmc_summary_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    kib = 1024.0
    copy = bench.COPY_BYTES / kib   # KiB the calibration copy moves
    # FETCH_SIZE counts half of what a copy reads, WRITE_SIZE all of it; a small torch copy (same
    # kernel) must not enter the calibration
    fetch = [("__amd_rocclr_copyBuffer", 512, [1.5]), ("__amd_rocclr_copyBuffer", 131072, [copy / 4] * 2),
             (UNMASKED, 458752, [1000.0] * 8), (UNMASKED, 458752, [1000.0] * 8),
             ("void qfa::kmean_partial_kernel<1, 128>(qfa::QuantArgs, int, long)", 1024, [300.0]),
             ("void qfa::kmean_finalize_kernel(qfa::QuantArgs, int)", 64, [10.0]),
             ("void qfa::quantize_kernel<1, 128>(qfa::QuantArgs, long, int, int)", 4096, [400.0]),
             ("void qfa::lse_merge_kernel<128>(qfa::MergeArgs)", 2048, [200.0])]
    write = [("__amd_rocclr_copyBuffer", 512, [1.5]), ("__amd_rocclr_copyBuffer", 131072, [copy / 2] * 2),
             (UNMASKED, 458752, [500.0] * 8), (UNMASKED, 458752, [500.0] * 8),
             ("void qfa::kmean_partial_kernel<1, 128>(qfa::QuantArgs, int, long)", 1024, [7.0]),
             ("void qfa::kmean_finalize_kernel(qfa::QuantArgs, int)", 64, [1.0]),
             ("void qfa::quantize_kernel<1, 128>(qfa::QuantArgs, long, int, int)", 4096, [250.0]),
             ("void qfa::lse_merge_kernel<128>(qfa::MergeArgs)", 2048, [60.0])]
    fd, wd = str(tmp_path / "fetch"), str(tmp_path / "write")
    _write(fd, "FETCH_SIZE", fetch)
    _write(wd, "WRITE_SIZE", write)
    out = tmp_path / "pmc.json"
    monkeypatch.setattr(bench, "PMC_FILE", str(out))
    assert bench.pmc_summary(fd, wd) == 0
    d = json.loads(out.read_text())
    assert d["copy_calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert d["copy_calibration"]["write_scale"] == pytest.approx(1.0)
    un = d["launches"]["unmasked"]
    assert un["fetch_bytes"] == round(8000 * kib * 2) and un["write_bytes"] == round(4000 * kib)
    per = d["bandwidth_kernels"]["per_dispatch"]
    assert per["quantize"]["fetch_bytes"] == round(400 * kib * 2) and per["quantize"]["write_bytes"] == round(250 * kib)
    q = d["bandwidth_kernels"]["quantize_call"]
    assert q["hbm_bytes"] == round((300 + 10 + 400) * kib * 2) + round(7 * kib) + round(kib) + round(250 * kib)
    assert q["algorithmic_bytes"] == 820004864


def test_pmc_summary_needs_the_calibration_copy(tmp_path, monkeypatch):
    fd, wd = str(tmp_path / "fetch"), str(tmp_path / "write")
    _write(fd, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 512, [1.5]), (UNMASKED, 458752, [1.0])])
    _write(wd, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 512, [1.5]), (UNMASKED, 458752, [1.0])])
    monkeypatch.setattr(bench, "PMC_FILE", str(tmp_path / "pmc.json"))
    with pytest.raises(SystemExit, match="calibration copy"):
        bench.pmc_summary(fd, wd)


def test_pmc_table_groups_by_kernel_and_grid(tmp_path, capsys):
    d1, d2 = str(tmp_path / "p1"), str(tmp_path / "p2")
    name = "void qfa::kmean_partial_kernel<1, 128>(qfa::QuantArgs, int, long)"
    _write(d1, "SQ_WAVES", [(name, 1024, [3.0, 5.0]), (name, 1024, [4.0, 6.0]), (name, 2048, [1.0])])
    _write(d2, "SQ_INSTS_SALU", [(name, 1024, [10.0]), (name, 1024, [30.0]), (name, 2048, [7.0])])
    assert bench.pmc_table([d1, d2], "kmean") == 0
    lines = capsys.readouterr().out.splitlines()
    assert lines[0] == "| kernel | grid | dispatches | median us | SQ_INSTS_SALU | SQ_WAVES |"
    rows = {tuple(c.strip() for c in l.split("|")[1:3]): [c.strip() for c in l.split("|")[3:-1]] for l in lines[2:]}
    # grid 1024: 4 dispatches (two per pass); per dispatch the XCD rows add up (8, 10), medians taken
    # over the dispatches that report each counter
    assert rows[("`kmean_partial_kernel<1, 128>`", "1024")][0] == "4"
    assert rows[("`kmean_partial_kernel<1, 128>`", "1024")][2:] == ["20", "9"]
    assert rows[("`kmean_partial_kernel<1, 128>`", "2048")][2:] == ["7", "1"]
