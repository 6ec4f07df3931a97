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


def test_algorithmic_bytes_per_token_head():
    """The byte model counts only the operator's own inputs and outputs.  At
    d = 128, C = 64: forward 7 inputs + o + a saved state per chunk; backward
    7 inputs + dO + the saved state + 7 gradients.  With fp32 states and
    gradients that is 3,072 + 6,656 = 9,728 B; as written here (bf16 saved
    states, fp32 gradients) 2,560 + 6,144 = 8,704 B; with bf16 gradients
    6,912 B.  The chunk-gradient kernel alone moves the whole backward's."""
    f, b = bench.step_bytes(128, 64, e=2, es=4, eg=4)
    assert (f, b) == (3072, 6656)
    f, b = bench.step_bytes(128, 64)
    assert (f, b) == (2560, 6144)
    assert sum(bench.step_bytes(128, 64, eg=2)) == 6912
    kb = bench.kernel_bytes(128, 64)
    assert kb["bwd_chunk"] == b
    assert kb["fwd_prep"] + kb["fwd_scan"] == f
    # larger chunks save fewer states
    assert sum(bench.step_bytes(128, 256)) < sum(bench.step_bytes(128, 128)) < sum(bench.step_bytes(128, 64))


def test_roofline_report_arithmetic():
    kern = {"fwd_prep": 0.5, "fwd_scan": 0.25, "bwd_scan": 0.2, "bwd_chunk": 1.0}  # ms
    nth = 8 * 4096 * 16
    kernels, roof, sm = bench.roofline_report(kern, 2.0, 128, 64, nth, "no_such_workload", eg=4)
    assert roof["kernel"] == "bwd_chunk" and roof["traffic"] is None
    assert abs(roof["achieved"] - 6144 * nth / 1e-3 / 1e9) < 1e-6
    assert abs(roof["frac"] - roof["achieved"] / 8000.0) < 1e-12
    assert abs(sm["alg_bytes"] - 8704 * nth) < 1e-3
    assert abs(sm["frac"] - sm["hbm_floor_us"] / 2000.0) < 1e-12  # HBM-bound: bytes floor over step time


def test_per_head_error_catches_a_small_head():
    """The per-(batch, head) error sees an error that the whole-tensor ratio
    hides behind another head's larger scale."""
    import numpy as np
    sys.path.insert(0, HERE)
    from gpu_util import err2, rel_err, rel_err_heads
    y = np.ones((1, 8, 2, 4))
    y[:, :, 1] *= 1e-3            # head 1 is 1000x smaller
    x = y.copy()
    x[0, 3, 1, 2] += 1e-4         # a 10% error inside head 1
    assert rel_err(x, y) < 2e-4
    assert abs(rel_err_heads(x, y, (0, 2)) - 0.1) < 1e-9
    assert err2(x, y, (0, 2)) == rel_err_heads(x, y, (0, 2))
    # an all-zero head contributes its absolute error
    y[:, :, 1] = 0
    x = y.copy()
    x[0, 0, 1, 0] = 3e-3
    assert abs(rel_err_heads(x, y, (0, 2)) - 3e-3) < 1e-12


def test_untile_states_follows_the_documented_tile_layout():
    """The tests' untile helper inverts the saved-state layout of the header:
    element (r, j) at ((r/16)(dv/16) + j/16) 256 + (r%16) 16 + j%16."""
    import torch
    sys.path.insert(0, HERE)
    from gpu_util import untile_states
    dk, dv = 64, 128
    flat = torch.arange(2 * dk * dv, dtype=torch.float64).reshape(2, dk, dv)
    plain = untile_states(flat)
    for r, j in ((0, 0), (5, 17), (16, 0), (63, 127), (31, 100)):
        want = ((r // 16) * (dv // 16) + j // 16) * 256 + (r % 16) * 16 + j % 16
        assert plain[0, r, j] == want and plain[1, r, j] == dk * dv + want
    assert sorted(plain.flatten().tolist()) == flat.flatten().tolist()
