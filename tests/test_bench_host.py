"""Host-side logic of bench.py (no GPU): the one-GPU guard and the conversion of
rocprofv3 FETCH_SIZE / WRITE_SIZE counters into HBM bytes per launch."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _write_counters(folder, counter, rows):
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


FWD = "void mi355attn::attn_fwd_kernel<0, 128, true, false, false>(unsigned short const*)"
DEC = "void mi355attn::attn_decode_split_kernel<0, 128, false, false, false>(unsigned short const*)"
PAG = "void mi355attn::attn_decode_split_kernel<0, 128, true, false, false>(unsigned short const*)"
DQ = "void mi355attn::attn_bwd_dq_kernel<0, 128, true>(unsigned short const*)"
DKDV = "void mi355attn::attn_bwd_dkdv_kernel<0, 128, true, false>(unsigned short const*)"
DELTA = "void mi355attn::attn_bwd_delta_kernel<0, 128>(unsigned short const*)"
DKDV_DS = "void mi355attn::attn_bwd_dkdv_kernel<0, 128, true, true>(unsigned short const*)"
DQ_DS = "void mi355attn::attn_bwd_dq_ds_kernel<0, 128, true>(unsigned short const*)"
CAL = "void at::native::vectorized_elementwise_kernel<neg_kernel>(int)"


def test_record_traffic_scales_by_the_calibration_kernel(tmp_path, monkeypatch):
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    kib = bench.COPY_CAL_BYTES / 1024.0
    # FETCH_SIZE reads half a KiB per KiB the calibration kernel moves, WRITE_SIZE one;
    # two dispatches per kernel, whose mean is taken.
    _write_counters(tmp_path / "f", "FETCH_SIZE",
                    [(CAL, 0.5 * kib), (CAL, 0.5 * kib), (FWD, 1000.0), (FWD, 3000.0),
                     (DEC, 4096.0), (DEC, 4096.0), (PAG, 5000.0)])
    _write_counters(tmp_path / "w", "WRITE_SIZE",
                    [(CAL, kib), (FWD, 64.0), (DEC, 16.0), (PAG, 32.0)])
    bench.record_traffic(str(tmp_path / "f"), str(tmp_path / "w"), "step")
    rec = json.loads(out.read_text())
    assert rec["_calibration"]["step"]["fetch_counter_bytes_per_byte"] == 0.5
    assert rec["_calibration"]["step"]["write_counter_bytes_per_byte"] == 1.0
    fwd = rec["attn_fwd_kernel/llm_prefill"]
    assert fwd["fetch_bytes"] == 2000 * 1024 * 2 and fwd["write_bytes"] == 64 * 1024
    assert fwd["bytes_per_launch"] == fwd["fetch_bytes"] + fwd["write_bytes"]
    assert rec["attn_decode_split_kernel/decode"]["fetch_bytes"] == 4096 * 1024 * 2
    assert rec["attn_decode_split_kernel/decode_paged"]["write_bytes"] == 32 * 1024
    # bench reports the figure only while the kernel sources are the recorded ones
    assert bench.load_traffic("attn_fwd_kernel/llm_prefill") == fwd["bytes_per_launch"]
    rec["attn_fwd_kernel/llm_prefill"]["source_hash"] = "0" * 16
    out.write_text(json.dumps(rec))
    assert bench.load_traffic("attn_fwd_kernel/llm_prefill") is None
    assert bench.load_traffic("no such kernel") is None
    # a second run (the backward) adds its entries and keeps the others
    _write_counters(tmp_path / "f2", "FETCH_SIZE", [(CAL, kib), (DQ, 10.0), (DKDV, 20.0)])
    _write_counters(tmp_path / "w2", "WRITE_SIZE", [(CAL, kib), (DQ, 1.0), (DKDV, 2.0)])
    bench.record_traffic(str(tmp_path / "f2"), str(tmp_path / "w2"), "bwd")
    rec = json.loads(out.read_text())
    assert rec["attn_bwd_dq_kernel/llm_prefill"]["bytes_per_launch"] == 10 * 1024 + 1024
    assert "attn_decode_split_kernel/decode" in rec and "bwd" in rec["_calibration"]
    assert bench._bwd_traffic() == 10 * 1024 + 1024 + 20 * 1024 + 2 * 1024
    # the stored-dS backward: three kernels, the dK/dV one told apart by its template
    assert bench._bwd_traffic(stored_ds=True) is None
    _write_counters(tmp_path / "f3", "FETCH_SIZE",
                    [(CAL, kib), (DELTA, 3.0), (DKDV_DS, 30.0), (DQ_DS, 40.0)])
    _write_counters(tmp_path / "w3", "WRITE_SIZE",
                    [(CAL, kib), (DELTA, 0.5), (DKDV_DS, 50.0), (DQ_DS, 4.0)])
    bench.record_traffic(str(tmp_path / "f3"), str(tmp_path / "w3"), "bwd_ds")
    assert bench._bwd_traffic(stored_ds=True) == (3 + 30 + 40) * 1024 + (0.5 + 50 + 4) * 1024
    assert bench._bwd_traffic() == 10 * 1024 + 1024 + 20 * 1024 + 2 * 1024


def test_record_traffic_needs_exactly_one_match(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    kib = bench.COPY_CAL_BYTES / 1024.0
    _write_counters(tmp_path / "f", "FETCH_SIZE", [(CAL, kib), (FWD, 1.0), (PAG, 1.0)])
    _write_counters(tmp_path / "w", "WRITE_SIZE", [(CAL, kib), (FWD, 1.0), (PAG, 1.0)])
    with pytest.raises(SystemExit):
        bench.record_traffic(str(tmp_path / "f"), str(tmp_path / "w"), "step")
    with pytest.raises(SystemExit):
        bench.record_traffic(str(tmp_path / "f"), str(tmp_path / "w"), "no such run")
    assert not (tmp_path / "traffic.json").exists()
