"""Host logic of bench.py that runs without a GPU: the HBM-traffic records and
the one-GPU guard."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (bench imports torch only inside its GPU paths)


def _record(workload, kernel, sha, read=1000, write=24):
    return "traffic_record " + json.dumps({
        "workload": workload, "kernel": kernel, "kernel_name": "k",
        "read_bytes": read, "write_bytes": write, "sources_sha256": sha})


def test_traffic_record_matches_current_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.md"
    cur = bench.sources_sha256("grouped_gemm")
    f.write_text("\n".join(["# header", _record("w", "grouped_gemm", cur, 4096, 512)]) + "\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("w", "grouped_gemm") == 4608
    # another workload or kernel has no record
    assert bench.measured_traffic("other", "grouped_gemm") is None
    assert bench.measured_traffic("w", "stream_ffn") is None


def test_traffic_record_of_changed_sources_is_stale(tmp_path, monkeypatch):
    f = tmp_path / "traffic.md"
    f.write_text(_record("w", "stream_ffn", "0" * 64) + "\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("w", "stream_ffn") is None


def test_traffic_without_records_file(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.measured_traffic("w", "grouped_gemm") is None


def test_source_hash_covers_the_kernel_sources():
    # each kernel's hash is over its own source list, in order
    a = bench.sources_sha256("grouped_gemm")
    b = bench.sources_sha256("stream_ffn")
    assert len(a) == 64 and len(b) == 64 and a != b


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""
