"""Host-side pieces of bench.py that need no GPU: the one-GPU contract, the
algorithmic byte count of a verify call, and the gate that reports counter
traffic only for the kernel sources it was taken on."""

import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_verify_bytes_counts_each_used_row_once():
    # request b reads target rows 0..K_b and draft rows 0..K_b-1: (2 K_b + 1) rows of V
    k = np.array([7] * 64)
    assert bench.verify_bytes(k, 151936) == 291_717_120
    assert bench.verify_bytes([0, 1, 3], 10, elem=4) == (1 + 3 + 7) * 10 * 4


def test_traffic_is_reported_only_for_the_sources_it_was_taken_on():
    h = bench.kernel_source_hash()
    assert h == bench.kernel_source_hash() and len(h) == 16
    traffic = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    taken_on = traffic["kernel_source_hash"]
    assert bench.load_traffic(taken_on)["loss_bytes_per_launch"] > 0
    assert bench.load_traffic("0" * 16 if taken_on != "0" * 16 else "1" * 16) is None
