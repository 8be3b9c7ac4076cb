"""Host logic of bench.py (CPU only): the counter summary's kernel
classification and copy calibration, and the MFMA summary's arithmetic, from
synthetic rocprofv3 counter CSVs."""

import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write(path, rows, dur_ns=0):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, ctr, val) in enumerate(rows):
            r = {k: 0 for k in FIELDS}
            r.update(Dispatch_Id=i + 1, Kernel_Name=name, Counter_Name=ctr, Counter_Value=val,
                     Start_Timestamp=1000 * i, End_Timestamp=1000 * i + dur_ns)
            w.writerow(r)


def test_summarize_counters_classifies_kernels(tmp_path, monkeypatch):
    names = {
        "void gla::state_kernel<128, 64, false, false>(gla::KernelParams)": "segment",
        "void gla::state_kernel<128, 64, false, true>(gla::KernelParams)": "bwd_segment",
        "gla::scan_kernel(float*, float const*, float const*, long, int, int, int)": "scan",
        "void gla::chunk_kernel<gla::BF16, 128, 64, 0, false>(gla::KernelParams)": "output",
        "void gla::chunk_kernel<gla::BF16, 128, 64, 4, false>(gla::KernelParams)": "states",
        "void gla::bwd_kernel<gla::BF16, 128, 64, 1>(gla::BwdParams)": "bwd",
    }
    rows = []
    for k, (name, _) in enumerate(names.items()):
        rows.append((name, "FETCH_SIZE", 1000.0 * (k + 1)))
    # the calibration copy comes after the last chunk kernel: 1 GiB read counted as 512 MiB
    rows.append(("__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288.0))
    d = tmp_path / "fetch"
    d.mkdir()
    _write(d / "x_counter_collection.csv", rows)
    w = tmp_path / "write"
    w.mkdir()
    _write(w / "x_counter_collection.csv",
           [(n, "WRITE_SIZE", 10.0) for n in names] + [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576.0)])
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    bench.summarize_counters(str(tmp_path), "unit_test")
    out = json.loads((prof / "counters_unit_test.json").read_text())
    med = out["median_per_dispatch_KiB"]
    for k, (_, kind) in enumerate(names.items()):
        assert med[f"{kind}:FETCH_SIZE"] == 1000.0 * (k + 1)
        assert med[f"{kind}:WRITE_SIZE"] == 10.0
    assert abs(out["fetch_factor"] - 2.0) < 1e-12
    assert abs(out["write_factor"] - 1.0) < 1e-12
    assert out["source_digest"] == bench.source_digest()


def test_summarize_mfma_arithmetic(tmp_path):
    out_pass = "void gla::chunk_kernel<gla::BF16, 128, 64, 0, false>(gla::KernelParams)"
    # 1e6 bf16 16x16x32 MFMAs (16384 flops = 32 MOPS units each) in 100 us on
    # a GPU active for 240000 cycles per XCD, 16 busy cycles per instruction
    a = tmp_path / "busy"
    a.mkdir()
    _write(a / "a_counter_collection.csv",
           [(out_pass, "SQ_INSTS_MFMA", 1e6), (out_pass, "SQ_VALU_MFMA_BUSY_CYCLES", 16e6),
            (out_pass, "GRBM_GUI_ACTIVE", 8 * 240000.0),
            ("__amd_rocclr_copyBuffer", "SQ_INSTS_MFMA", 0.0)], dur_ns=100000)
    b = tmp_path / "ops"
    b.mkdir()
    _write(b / "b_counter_collection.csv",
           [(out_pass, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 32e6), (out_pass, "SQ_INSTS_VALU_MFMA_MOPS_F32", 0.0)],
           dur_ns=100000)
    res = bench.summarize_mfma([str(a), str(b)])
    assert set(res) == {"output"}
    r = res["output"]
    assert abs(r["dispatch_us"] - 100.0) < 1e-9
    assert abs(r["util"] - 16e6 / (1024 * 240000.0)) < 1e-12
    assert abs(r["bf16"] - 1e6 * 16384 / 100e-6 / 1e12) < 1e-9   # 163.84 TFLOP/s
    assert r["fp32"] == 0.0


def test_gpu_label():
    # the product from the arch, CU count and peak engine clock, marked as inferred
    assert bench.gpu_label("gfx950:sramecc+:xnack-", 256, 2400, "AMD Radeon Graphics").startswith(
        "AMD Instinct MI355X (inferred")
    assert bench.gpu_label("gfx950", 256, 2200, None).startswith("AMD Instinct MI350X (inferred")
    # anything else keeps the board name the runtime gave
    assert bench.gpu_label("gfx942", 304, 2100, "AMD Instinct MI300X") == "AMD Instinct MI300X"
    assert bench.gpu_label("gfx950", 256, None, "board") == "board"
    # no GPU agent here: the in-process query answers (None, None) or a pair, never raises
    info = bench.hsa_gpu_info()
    assert isinstance(info, tuple) and len(info) == 2
