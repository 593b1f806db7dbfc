"""Host-side parts of bench.py that need no GPU: the one-GPU guard and the
conversion of two rocprofv3 counter tables into HBM bytes per launch."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

CHUNK = "void comba::chunk_fwd_bf16_kernel<128, 128, 64, unsigned short, false, false>(args)"
FUSED = "void comba::chunk_fwd_bf16_kernel<128, 128, 64, unsigned short, true, false>(args)"
DECODE = "void comba::recurrent_kernel<128, 128, 32, unsigned short, unsigned short>(args)"
COPY = "void at::native::elementwise_copy(args)"
OTHER = "void at::native::some_other_kernel(args)"


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=60)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def write_table(d, counter, rows):
    os.makedirs(d)
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows, start=1):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_record_traffic_scales_by_the_copy(tmp_path, monkeypatch):
    chunk_json, decode_json = tmp_path / "chunk.json", tmp_path / "decode.json"
    monkeypatch.setattr(bench, "COUNTERS_JSON", str(chunk_json))
    monkeypatch.setattr(bench, "DECODE_COUNTERS_JSON", str(decode_json))
    kib = bench.COPY_CAL_BYTES / 1024
    # FETCH counts half the copy's bytes (scale 2), WRITE all of them (scale 1);
    # kernels dispatched after the last counted one but not three times are ignored
    fetch = [(CHUNK, 1000.0), (FUSED, 7.0), (CHUNK, 1002.0), (DECODE, 300.0), (DECODE, 302.0),
             (OTHER, 5.0), (COPY, kib / 2), (COPY, kib / 2), (COPY, kib / 2), (OTHER, 6.0)]
    write = [(CHUNK, 500.0), (FUSED, 7.0), (CHUNK, 500.0), (DECODE, 600.0), (DECODE, 600.0),
             (OTHER, 5.0), (COPY, kib), (COPY, kib), (COPY, kib), (OTHER, 6.0)]
    write_table(tmp_path / "f", "FETCH_SIZE", fetch)
    write_table(tmp_path / "w", "WRITE_SIZE", write)
    bench.record_traffic(str(tmp_path / "f"), str(tmp_path / "w"))
    c, d = json.loads(chunk_json.read_text()), json.loads(decode_json.read_text())
    assert c["kernel_dispatches"] == [2, 2] and d["kernel_dispatches"] == [2, 2]
    assert c["fetch_scale"] == pytest.approx(2.0) and c["write_scale"] == pytest.approx(1.0)
    assert c["hbm_read_bytes_per_launch"] == pytest.approx(1001.0 * 1024 * 2)
    assert c["hbm_write_bytes_per_launch"] == pytest.approx(500.0 * 1024)
    assert d["hbm_bytes_per_launch"] == pytest.approx(301.0 * 1024 * 2 + 600.0 * 1024)
    assert c["kernel_source_hash"] == bench.kernel_source_hash()
    assert d["kernel_source_hash"] == bench.kernel_source_hash(bench.DECODE_SOURCES)
    # the bench line reports traffic only for a matching source hash
    assert bench.measured_traffic(c["kernel_source_hash"]) == pytest.approx(c["hbm_bytes_per_launch"])
    assert bench.measured_traffic("0" * 16) is None


def test_calibration_copy_must_be_identifiable(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "COUNTERS_JSON", str(tmp_path / "chunk.json"))
    monkeypatch.setattr(bench, "DECODE_COUNTERS_JSON", str(tmp_path / "decode.json"))
    rows = [(CHUNK, 1.0), (COPY, 2.0), (COPY, 2.0)]   # two copies: not the calibration's three
    write_table(tmp_path / "f", "FETCH_SIZE", rows)
    write_table(tmp_path / "w", "WRITE_SIZE", rows)
    with pytest.raises(SystemExit):
        bench.record_traffic(str(tmp_path / "f"), str(tmp_path / "w"))
