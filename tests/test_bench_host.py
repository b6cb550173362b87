"""bench.py's host-side contract (CPU only): the one-GPU refusal and the
committed counter records its roofline entry reads."""
import json
import os
import subprocess
import sys

import pytest

import moe_inputs as MI

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


@pytest.mark.parametrize("wl", sorted(k for k in MI.WORKLOADS if k != "tiny_mxfp4_fp8"))
def test_traffic_record(wl):
    """Each measured workload has a counter record whose HBM bytes are its
    FETCH_SIZE and WRITE_SIZE (KiB per launch) scaled by the calibration
    copy, and a kernel-trace summary beside it."""
    path = os.path.join(ROOT, "profiles", f"gemm1_{wl}.traffic.json")
    rec = json.load(open(path))
    assert rec["workload"] == wl and len(rec["gemm_source_sha256"]) == 64
    f = rec["fetch_kib_per_launch"] * 1024 * (rec["copy_bytes"] / 1024 / rec["copy_fetch_kib"])
    w = rec["write_kib_per_launch"] * 1024 * (rec["copy_bytes"] / 1024 / rec["copy_write_kib"])
    assert abs(f + w - rec["traffic_bytes_per_launch"]) <= 1e-6 * rec["traffic_bytes_per_launch"]
    assert os.path.exists(os.path.join(ROOT, "profiles", f"gemm1_{wl}.md"))
