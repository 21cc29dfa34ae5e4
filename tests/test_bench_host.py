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


def _fake_counter_csv(path, counter, dispatches):
    import csv
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for i, (name, kib) in enumerate(dispatches):
            # two rows per dispatch, as a counter split over dimensions
            for half in (0.25, 0.75):
                w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter,
                            "Counter_Value": kib * half})


def test_traffic_from_counters_scales_by_the_copy_calibration(tmp_path):
    gib_kib = float(1 << 20)
    rows = "void lvtv::vr::(anonymous namespace)::verify_rows_bf16<true, false>(Args)"
    fin = "void lvtv::vr::(anonymous namespace)::verify_finalize<1>(Args)"
    loss = "void lvtv::lf::(anonymous namespace)::loss_halves<true, false, false, false, 1>(Args)"
    finish = "void lvtv::lf::(anonymous namespace)::loss_finish<true, false, false, false>(Args)"
    clear = "lvtv::lf::(anonymous namespace)::clear_words(u32x4*, unsigned long)"
    # the counter reads half of the true fetch bytes (scale 2) and all written bytes
    fetch = [("fill", 10.0)] + [("__amd_rocclr_copyBuffer", gib_kib / 2)] * 3 + [
        (rows, 1000.0), (fin, 10.0), (rows, 2000.0), (fin, 20.0), (rows, 3000.0), (fin, 30.0),
        (clear, 0.0), (loss, 40000.0), (finish, 4.0), (rows, 99.0)]
    write = [("fill", gib_kib)] + [("__amd_rocclr_copyBuffer", gib_kib)] * 3 + [
        (rows, 1.0), (fin, 2.0), (rows, 3.0), (fin, 4.0), (rows, 5.0), (fin, 6.0),
        (clear, 7.0), (loss, 8.0), (finish, 9.0), (rows, 99.0)]
    fp, wp = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _fake_counter_csv(fp, "FETCH_SIZE", fetch)
    _fake_counter_csv(wp, "WRITE_SIZE", write)
    t = bench.traffic_from_counters(str(fp), str(wp))
    assert t["fetch_scale"] == 2.0 and t["write_scale"] == 1.0
    assert t["kernel_source_hash"] == bench.kernel_source_hash()
    assert t["verify_T0.6_rows_fetch"] == 2000.0 * 1024 * 2
    assert t["verify_T1.0_finalize_write"] == 6.0 * 1024
    assert t["loss_bytes_per_launch"] == (40000.0 * 2 + 8.0) * 1024
    assert t["verify_T0.0_bytes_per_launch"] == (1000.0 * 2 + 1.0 + 10.0 * 2 + 2.0) * 1024
    assert t["loss_logits_T1.0_fetch_bytes"] is None
