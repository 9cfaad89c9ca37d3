"""Host-side logic of bench.py (no GPU): the one-GPU contract, the counter ingestion
arithmetic (copy calibration, medians, MFMA-busy formula) and the source hashes that
tie stored counters to the kernels they were taken on."""
import csv
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("extra", [[], ["--requant", "local_share_A"], ["--dgrad", "dgrad_local_share"]])
def test_more_than_one_gpu_exits_with_a_message(extra):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"] + extra,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_ingest_counters_scales_by_the_calibration_copy(tmp_path):
    b = bench()
    gib_kib = b.COPY_BYTES / 1024
    # the copy's FETCH reads half its bytes (the counter's unit), WRITE reads all;
    # three kernel dispatches, the median is taken
    fetch = [dict(Dispatch_Id=1, Kernel_Name="__amd_rocclr_copyBuffer", Counter_Name="FETCH_SIZE",
                  Counter_Value=gib_kib / 2, Start_Timestamp=0, End_Timestamp=10)]
    write = [dict(Dispatch_Id=1, Kernel_Name="__amd_rocclr_copyBuffer", Counter_Name="WRITE_SIZE",
                  Counter_Value=gib_kib, Start_Timestamp=0, End_Timestamp=10)]
    for d, (fv, wv) in enumerate([(100.0, 40.0), (300.0, 60.0), (200.0, 50.0)], start=2):
        fetch.append(dict(Dispatch_Id=d, Kernel_Name="void kg::kg_wgrad_kernel<0>(kg::Params)",
                          Counter_Name="FETCH_SIZE", Counter_Value=fv, Start_Timestamp=0,
                          End_Timestamp=5))
        write.append(dict(Dispatch_Id=d, Kernel_Name="void kg::kg_wgrad_kernel<0>(kg::Params)",
                          Counter_Name="WRITE_SIZE", Counter_Value=wv, Start_Timestamp=0,
                          End_Timestamp=5))
    fp, wp = tmp_path / "f.csv", tmp_path / "w.csv"
    write_csv(fp, fetch)
    write_csv(wp, write)
    b.ingest_counters(str(fp), str(wp), "unit_test", out_dir=str(tmp_path))
    rec = json.load(open(tmp_path / "kg_wgrad_unit_test_traffic.json"))
    assert rec["counters"]["FETCH_SIZE"]["scale"] == pytest.approx(2.0)
    assert rec["counters"]["WRITE_SIZE"]["scale"] == pytest.approx(1.0)
    assert rec["traffic_bytes"] == int(200.0 * 2.0 * 1024 + 50.0 * 1024)
    assert rec["kernel_source"] == b.kernel_source_hash("kg_wgrad")


def test_ingest_mfma_busy_fraction(tmp_path):
    b = bench()
    vals = {"SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 500.0, "SQ_INSTS_VALU_MFMA_MOPS_BF16": 1000.0,
            "SQ_INSTS_VALU_MFMA_MOPS_F8": 0.0, "SQ_ACTIVE_INST_VALU": 1.0,
            "SQ_LDS_BANK_CONFLICT": 10.0, "SQ_LDS_IDX_ACTIVE": 40.0, "SQ_WAVE_CYCLES": 1.0,
            "GRBM_GUI_ACTIVE": 8 * 1000.0, "GRBM_COUNT": 8 * 1000.0}
    rows = [dict(Dispatch_Id=7, Kernel_Name="void kg::kg_requant_kernel<0, 0, 128>(kg::QParams)",
                 Counter_Name=k, Counter_Value=v, Start_Timestamp=0, End_Timestamp=500)
            for k, v in vals.items()]
    p = tmp_path / "m.csv"
    write_csv(p, rows)
    b.ingest_mfma(str(p), "requant:unit_test", "cmd", out_dir=str(tmp_path))
    rec = json.load(open(tmp_path / "kg_requant_unit_test_mfma.json"))
    # busy cycles over (GUI-active cycles of one XCD) x 1024 SIMDs
    assert rec["mfma_busy_frac"] == pytest.approx(0.5)
    assert rec["lds_bank_conflict_per_active"] == pytest.approx(0.25)
    assert rec["mfma_flops_counted"] == 1000.0 * 512
    assert rec["shader_clock_ghz"] == pytest.approx(2.0)  # 1000 cycles in 500 ns
    assert rec["kernel_source"] == b.kernel_source_hash("kg_requant")


def test_source_hashes_per_kernel():
    b = bench()
    h = {k: b.kernel_source_hash(k) for k in b.KERNEL_SOURCES}
    assert len(set(h.values())) == len(h)
    assert all(len(v) == 16 and int(v, 16) >= 0 for v in h.values())
    assert h == {k: b.kernel_source_hash(k) for k in b.KERNEL_SOURCES}
