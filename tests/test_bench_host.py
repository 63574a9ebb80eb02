"""Host-side logic of bench.py that runs without a GPU: the one-GPU refusal and
the counter-record lookup that gates roofline.traffic on the kernel's sources."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def _record(tmp_path, sha, up=123, down=456):
    p = tmp_path / "traffic.txt"
    p.write_text(f"# a comment: with a colon\nsource_sha256: {sha}\nup_bytes: {up}\ndown_bytes: {down}\n")
    return str(p)


def test_traffic_record_is_used_only_for_the_sources_it_was_taken_on(tmp_path):
    src = tmp_path / "kernel.hip"
    src.write_text("kernel source\n")
    hdr = tmp_path / "header.hpp"
    hdr.write_text("header\n")
    files = [str(src), str(hdr)]
    path = _record(tmp_path, bench.source_sha256(files))
    assert bench.measured_traffic((path, files)) == [123, 456]
    hdr.write_text("header, edited\n")  # any change to either file invalidates the record
    assert bench.measured_traffic((path, files)) is None


def test_missing_or_malformed_traffic_record_reads_as_none(tmp_path):
    src = tmp_path / "kernel.hip"
    src.write_text("x\n")
    files = [str(src)]
    assert bench.measured_traffic((str(tmp_path / "absent.txt"), files)) is None
    bad = tmp_path / "bad.txt"
    bad.write_text(f"source_sha256: {bench.source_sha256(files)}\nup_bytes: many\ndown_bytes: 1\n")
    assert bench.measured_traffic((str(bad), files)) is None
    partial = tmp_path / "partial.txt"
    partial.write_text(f"source_sha256: {bench.source_sha256(files)}\nup_bytes: 1\n")
    assert bench.measured_traffic((str(partial), files)) is None
