"""bench.py's host-side logic (no GPU): the one-GPU refusal, the source hash
that decides whether the stored HBM-traffic summary still describes the
GEMV, and the counter calibration that turns FETCH_SIZE / WRITE_SIZE into
bytes per launch."""
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
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_source_hash_ignores_comments_only(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("int f(int x) {  // add one\n  return x + 1; /* done */\n}\n")
    b = tmp_path / "b.hip"
    b.write_text("// header\nint f(int x) {\n  return x + 1;\n}\n")
    c = tmp_path / "c.hip"
    c.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.source_hash(str(a)) == bench.source_hash(str(b))
    assert bench.source_hash(str(a)) != bench.source_hash(str(c))


def _write_counters(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for did, name, value in rows:
            w.writerow({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


def test_counter_calibration(tmp_path, monkeypatch):
    """A copy of COPY_BYTES whose FETCH_SIZE reads half its bytes calibrates
    FETCH at 2x; the GEMV's bytes are its counters times the two scales."""
    kib = bench.COPY_BYTES / 1024.0
    gemv = "void qmat::gemv_rows_kernel<qmat::FmtQ4_0, 1, 1, false>(...)"
    copy = "__amd_rocclr_copyBuffer"
    fetch = [(1, copy, kib / 2), (2, gemv, 12000.0), (3, gemv, 12400.0), (4, copy, 10.0)]
    write = [(1, copy, kib), (2, gemv, 16.0), (3, gemv, 16.0), (4, copy, 5.0)]
    _write_counters(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _write_counters(tmp_path / "w.csv", "WRITE_SIZE", write)
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    t = json.loads(out.read_text())
    assert t["copy_dispatches"] == 1            # the small copy is not a calibration copy
    assert t["fetch_scale"] == pytest.approx(2.0)
    assert t["write_scale"] == pytest.approx(1.0)
    assert t["traffic_bytes_per_launch"] == pytest.approx((12200.0 * 2 + 16.0) * 1024.0)
    assert t["gemv_src_sha256_16"] == bench.source_hash(bench.GEMV_SRC)
    # the stored summary is reported while the GEMV source is unchanged
    assert bench.traffic_for_current_kernel() == pytest.approx(t["traffic_bytes_per_launch"])
    t["gemv_src_sha256_16"] = "0" * 16
    out.write_text(json.dumps(t))
    assert bench.traffic_for_current_kernel() is None


@pytest.mark.parametrize("slice_bytes", [16, 4095, 4096, 25422848, 25804817, 1 << 30, 2 << 30])
def test_read_slices_stay_in_the_buffer(slice_bytes):
    """Every launch of the same-bytes read starts 4 KiB-aligned, reads a
    multiple of 16 bytes, and ends inside the 2 GiB buffer; distinct
    launches read disjoint parts of it."""
    buf = 2 << 30
    n16, stride, slots, launches = bench.read_slices(buf, slice_bytes)
    assert n16 % 16 == 0 and 0 <= slice_bytes - n16 < 16 and stride % 4096 == 0
    assert stride >= n16 and 1 <= launches <= min(64, slots)
    for i in range(launches):
        assert i * stride + n16 <= buf
    if slice_bytes == 25422848:
        assert launches == 64 and launches * n16 > 256 << 20   # beyond the Infinity Cache


def test_read_slices_refuse_what_does_not_fit():
    with pytest.raises(ValueError):
        bench.read_slices(1 << 20, (1 << 20) + 16)
    with pytest.raises(ValueError):
        bench.read_slices(1 << 20, 15)
