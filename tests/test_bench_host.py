"""Host-side parts of bench.py that need no GPU: the one-GPU contract, the
kernel-source hash, and the rule that measured HBM traffic is reported only
while the kernels are the ones the counters were taken on."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_kernel_source_hash_is_stable_hex():
    h1, h2 = bench.kernel_source_hash(), bench.kernel_source_hash()
    assert h1 == h2 and len(h1) == 16
    int(h1, 16)


def test_traffic_only_for_the_profiled_kernels(tmp_path, monkeypatch):
    t = {"source_sha": bench.kernel_source_hash(),
         "kernels": {"gemm_fprop": {"bytes_per_launch": 123456}}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(t))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("gemm_fprop") == 123456
    assert bench.measured_traffic("not_an_op") is None
    t["source_sha"] = "0" * 16  # kernels changed since the counters were taken
    f.write_text(json.dumps(t))
    assert bench.measured_traffic("gemm_fprop") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("gemm_fprop") is None


@pytest.mark.parametrize("name", ["quant_weight W_moe", "grouped_gemm", "gemm_fprop"])
def test_committed_traffic_covers_the_step(name):
    """The committed counter summary has an entry for every op of the step."""
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        t = json.load(f)
    assert t["kernels"][name]["bytes_per_launch"] > 0
    assert t["copy_calibration"]["fetch_factor"] > 0 and t["copy_calibration"]["write_factor"] > 0
