"""Host-side checks of the benchmark driver (CPU only)."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_committed_counter_summary_is_well_formed():
    sys.path.insert(0, ROOT)
    import bench
    from ring_attention_chunk_amd import workloads as wl

    w = wl.config(1)
    path = os.path.join(ROOT, "profiles", f"{bench.dominant_kernel(w)}_{w.name}_hbm_traffic.json")
    with open(path) as f:
        t = json.load(f)
    for key in ("source_sha256_16", "bytes_per_launch", "algorithmic_bytes_per_launch", "copy_calibration",
                "commands"):
        assert key in t, key
    # measured traffic is at least the algorithmic bytes (inputs read once, output written once)
    assert t["bytes_per_launch"] >= t["algorithmic_bytes_per_launch"]
    # the benchmark reports it only while the kernel source is the one the counters were taken on
    got = bench.traffic_for(w)
    assert got is None or got == t["bytes_per_launch"]
