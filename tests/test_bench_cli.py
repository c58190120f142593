"""bench.py's command-line contract on the CPU: it refuses more than one GPU
with a message, never prints a number without a GPU, and uses committed HBM
counters only for the kernel identity they were recorded with."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def run(*args):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_no_gpu_no_number():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = run("--steps", "1", "--warmup", "0")
    assert r.returncode != 0
    assert r.stdout.strip() == ""


def test_traffic_only_for_the_recorded_kernel(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    from workloads import WORKLOADS
    w = WORKLOADS["b8h32n2048d128_bf16"]
    rec = {w.name: {"kernel_identity": "not-this-kernel", "hbm_bytes_per_launch": 123},
           "bwd:" + w.name: {"kernel_identity": "not-this-kernel", "hbm_bytes_per_call": 456}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic_bwd(w) is None
    rec["bwd:" + w.name]["kernel_identity"] = bench.bwd_identity(w)
    path.write_text(json.dumps(rec))
    assert bench.measured_traffic_bwd(w) == 456
    assert bench.measured_traffic_bwd(w, variant=3) is None
