"""Host logic of bench.py, on the CPU: the source hashes that decide whether a
counter-measured traffic record still describes a kernel, and the one-GPU
guard of the command line."""
import json
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.fixture
def csrc_copy(tmp_path, monkeypatch):
    dst = tmp_path / "csrc"
    shutil.copytree(bench.CSRC, dst)
    monkeypatch.setattr(bench, "CSRC", str(dst))
    return dst


def _hashes():
    return {k: bench.kernel_sources_sha256(k) for k in bench.KERNEL_SOURCE}


def _touch(path):
    with open(path, "a") as f:
        f.write("\n// edited\n")


def test_hash_follows_only_the_kernels_own_sources(csrc_copy):
    h0 = _hashes()
    # a file no measured kernel includes: every record stays valid
    _touch(csrc_copy / "gate_proj.hip")
    assert _hashes() == h0
    # the forward prep kernel's own file: only its record goes stale
    _touch(csrc_copy / "fwd.hip")
    h1 = _hashes()
    assert h1["fwd_prep"] != h0["fwd_prep"]
    assert all(h1[k] == h0[k] for k in h0 if k != "fwd_prep")
    # a header every kernel includes (directly or through another header)
    _touch(csrc_copy / "device_common.h")
    h2 = _hashes()
    assert all(h2[k] != h1[k] for k in h1)


def test_scans_share_one_source(csrc_copy):
    h = _hashes()
    assert h["fwd_scan"] == h["bwd_scan"]
    _touch(csrc_copy / "scan.hip")
    h1 = _hashes()
    assert h1["fwd_scan"] != h["fwd_scan"] and h1["bwd_chunk"] == h["bwd_chunk"]


def test_stale_traffic_record_reads_as_none(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "HERE", str(tmp_path))
    rec = {"kernel": "bwd_chunk", "workload": "w", "fetch_bytes_per_launch": 3.0, "write_bytes_per_launch": 4.0,
           "sources_sha256": bench.kernel_sources_sha256("bwd_chunk")}
    (prof / "traffic_bwd_chunk_w.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("bwd_chunk", "w") == 7.0
    rec["sources_sha256"] = "0" * 64
    (prof / "traffic_bwd_chunk_w.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("bwd_chunk", "w") is None
    assert bench.measured_traffic("bwd_chunk", "missing") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
