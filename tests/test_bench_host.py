"""Host logic of bench.py (no GPU): the HBM-traffic record is used only while
the GEMM kernel's sources are the ones it was measured on, and more than one
GPU is refused with a message."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_traffic_record_used_only_for_its_sources():
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    t = bench.traffic_bytes()
    if rec["gemm_src_sha256_16"] == bench._src_hash(bench.GEMM_SRC):
        assert t == rec["bytes_per_launch"]
    else:                                     # sources edited since the counters were taken
        assert t is None
    # the HBM-side bytes can only exceed the algorithmic ones (each operand
    # read once, the output written once)
    assert rec["bytes_per_launch"] >= rec["algorithmic_bytes_per_launch"]


def test_traffic_record_dropped_when_a_source_changes(tmp_path, monkeypatch):
    copies = []
    for i, src in enumerate(bench.GEMM_SRC):
        dst = tmp_path / f"src{i}"
        data = open(src, "rb").read()
        if i == len(bench.GEMM_SRC) - 1:
            data += b"\n// changed\n"           # a header the kernel compiles in
        dst.write_bytes(data)
        copies.append(str(dst))
    monkeypatch.setattr(bench, "GEMM_SRC", copies)
    assert bench.traffic_bytes() is None


def test_hash_covers_every_source_in_order(tmp_path):
    a, b = tmp_path / "a", tmp_path / "b"
    a.write_bytes(b"x")
    b.write_bytes(b"y")
    assert bench._src_hash([str(a), str(b)]) != bench._src_hash([str(b), str(a)])
    assert bench._src_hash([str(a)]) != bench._src_hash([str(a), str(b)])


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert p.returncode == 2
    line = json.loads(p.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]
