"""Host-side checks of the benchmark's contract that need no GPU."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_table_is_keyed_by_the_kernel_sources():
    sys.path.insert(0, ROOT)
    import bench
    tab = json.load(open(os.path.join(ROOT, "profiles",
                                      "traffic_dense_rl_N16384_H4096_V131072.json")))
    wl = tab["workload"]
    # a stale table (sources changed since the counters were taken) gives None,
    # a current one gives the per-launch bytes of each GEMM kernel
    if tab["source_sha256"] == bench.kernel_source_hash():
        assert "fwd_tiles" in tab["kernels"] and "dz_tiles" in tab["kernels"]
        for k in tab["kernels"]:
            assert bench.measured_traffic(k, wl) == tab["kernels"][k]["hbm_bytes_per_launch"]
    else:
        assert bench.measured_traffic("dz_tiles", wl) is None
    assert bench.measured_traffic("dz_tiles", "another workload") is None
