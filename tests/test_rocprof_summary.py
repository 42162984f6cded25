"""The rocprofv3 summariser on small hand-made CSV files: segments split at
the spin kernels, per-call division, byte formulas of the counter summary."""
from __future__ import annotations

import csv
import json
import os

from displaced_patch_diffusion_amd import rocprof_summary as rs

TRACE_COLS = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "VGPR_Count",
              "LDS_Block_Size", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]


def _write(path, cols, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _log(path, labels, reps, flush=False):
    with open(path, "w") as f:
        f.write("noise\nPROFILE_OPS " + json.dumps({"workload": "w", "reps": reps, "labels": labels, "flush": flush,
                                                     "qkv": "fused", "gn_sums": "conv",
                                                     "splice_bytes": 4000}) + "\n")


def _seq(reps):
    """spin, 2x(a,a2), spin, 2x b, spin, 2x copy, spin -- with a stray spin
    and a set-up kernel before the run."""
    seq = [("spin_kernel(long)", 1), ("setup", 5)]
    seq += [("spin_kernel(long)", 1)] + [k for _ in range(reps) for k in (("void ka<1>(int)", 10), ("kb2", 3))]
    seq += [("spin_kernel(long)", 1)] + [("kc", 7)] * reps
    seq += [("spin_kernel(long)", 1)] + [("copy", 4)] * reps
    seq += [("spin_kernel(long)", 1)]
    return seq


def test_ops_trace_segments(tmp_path):
    reps = 2
    rows, t = [], 0
    for i, (name, us) in enumerate(_seq(reps)):
        rows.append({"Kind": "KERNEL_DISPATCH", "Dispatch_Id": i + 1, "Kernel_Name": name, "Start_Timestamp": t,
                     "End_Timestamp": t + us * 1000, "VGPR_Count": 8, "LDS_Block_Size": 0, "Grid_Size_X": 64,
                     "Grid_Size_Y": 1, "Grid_Size_Z": 1})
        t += us * 1000 + 500
    rows.reverse()  # the summariser orders by dispatch id
    _write(str(tmp_path / "d" / "x_kernel_trace.csv"), TRACE_COLS, rows)
    _log(str(tmp_path / "log"), ["a", "b", "copy"], reps)
    text = rs.ops_trace(str(tmp_path / "d"), str(tmp_path / "log"), "cmd")
    res = json.loads(text.splitlines()[-1][len("RESULT "):])
    assert res["ops"]["a"] == {"kernels_per_call": 2, "us_per_call": 13.0, "min_us": 13.0}
    assert res["ops"]["b"]["us_per_call"] == 7.0
    assert res["ops"]["copy"]["kernels_per_call"] == 1


def test_ops_counters_bytes_and_busy(tmp_path):
    reps = 2
    seq = _seq(reps)
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    rows_rd, rows_sq = [], []
    for i, (name, _) in enumerate(seq):
        copy = name == "copy"
        # copy: 10 x 32B + 5 x 64B + 10 x 128B = 1920 bytes read per call, every request classified
        vals = {"TCC_EA0_RDREQ_32B_sum": 10 if copy else 1, "TCC_EA0_RDREQ_64B_sum": 5 if copy else 0,
                "TCC_EA0_RDREQ_128B_sum": 10 if copy else 0, "TCC_EA0_RDREQ_sum": 25 if copy else 1,
                "GRBM_GUI_ACTIVE": 8 * 1000}  # the clock in both passes: averaged, not added
        rows_rd += [{"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": k, "Counter_Value": v}
                    for k, v in vals.items()]
        sq = {"GRBM_GUI_ACTIVE": 8 * 1000, "SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 250 if name == "kc" else 0,
              "SQ_WAVE_CYCLES": 400, "SQ_WAIT_ANY": 100, "SQ_INSTS_VALU_MFMA_MOPS_BF16": 3}
        rows_sq += [{"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": k, "Counter_Value": v}
                    for k, v in sq.items()]
    _write(str(tmp_path / "rd" / "p_counter_collection.csv"), cols, rows_rd)
    _write(str(tmp_path / "sq" / "p_counter_collection.csv"), cols, rows_sq)
    _log(str(tmp_path / "log"), ["a", "b", "splice_copy"], reps)
    text = rs.ops_counters([str(tmp_path / "rd"), str(tmp_path / "sq")], str(tmp_path / "log"), ["c1", "c2"])
    res = json.loads(text.splitlines()[-1][len("RESULT "):])
    cp = res["ops"]["splice_copy"]
    assert cp["read_bytes"] == 32 * 10 + 64 * 5 + 128 * 10
    assert cp["read_req_unclassified"] == 0
    a = res["ops"]["a"]  # two dispatches per call, each one 32-byte request
    assert a["read_bytes"] == 64
    b = res["ops"]["b"]  # kc: a quarter of every SIMD's 1000 clock cycles busy
    assert b["gui_cycles"] == 1000 and b["mfma_busy_pct"] == 25.0
    assert b["any_wait_pct_of_wave"] == 25.0 and b["mfma_bf16_flop"] == 3 * 512
    assert "calibration" in text and "c1" in text and "c2" in text
