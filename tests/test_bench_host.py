"""Host-side logic of bench.py (no GPU): the single-GPU guard and the stored traffic record."""
import hashlib
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout


def _write_profile(root, src_files, digest, nbytes):
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    with open(os.path.join(root, "profiles", "k.traffic.md"), "w") as f:
        f.write("# k\n\n```\n")
        f.write(f"source_files: {' '.join(src_files)}\n")
        f.write(f"source_sha256: {digest}\n")
        f.write(f"bytes_per_launch: {nbytes}\n```\n")


def test_traffic_record_follows_sources(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_bytes(b"kernel v1")
    digest = hashlib.sha256(b"kernel v1").hexdigest()
    _write_profile(str(tmp_path), ["k.hip"], digest, 12345)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_for(["k.hip"], "k") == 12345
    src.write_bytes(b"kernel v2")  # the kernel changed since it was profiled
    assert bench.traffic_for(["k.hip"], "k") is None
    assert bench.traffic_for(["k.hip"], "missing") is None


def test_committed_traffic_record_parses():
    path = os.path.join(ROOT, "profiles", "fwd_tiles_kernel.traffic.md")
    if not os.path.exists(path):
        pytest.skip("no traffic profile committed")
    keys = {}
    for line in open(path):
        k, sep, v = line.partition(":")
        if sep:
            keys[k.strip()] = v.strip()
    assert int(keys["bytes_per_launch"]) > 0
    assert len(keys["source_sha256"]) == 64
