"""Host-side contract of bench.py: the multi-GPU request is refused, and the
measured HBM traffic is reported only for the workload and kernel source it
was taken on."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_only_for_its_workload_and_kernel_source():
    with open(bench.TRAFFIC_FILE) as f:
        data = json.load(f)
    t = bench.measured_traffic("c2", 1)
    if data["source_sha256"] == bench.source_sha(bench.GEMM_SRC):
        assert t == data["bytes_per_launch"]
        # counters scaled by the copy calibration, per launch
        fetch = data["fetch"]["gateup_kib_avg"] * 1024 * data["fetch"]["factor"]
        write = data["write"]["gateup_kib_avg"] * 1024 * data["write"]["factor"]
        assert abs(t - (fetch + write)) <= 1e-6 * t
    else:
        assert t is None
    assert bench.measured_traffic("c3", 1) is None
    assert bench.measured_traffic("c2", 2) is None


def test_layer_flops_of_the_gate_up_gemm():
    # the fused gate/up GEMM of a cached c2 layer: 4096 rows x 4096 in x (2 x 16384) out
    fl = bench.layer_flops(4096, 4352, 4096, 16384, 32, 128)
    assert fl["gemm_gateup"] == 2 * 4096 * 4096 * 32768
    # attention: every target row against all 4352 keys, QK^T and PV
    assert fl["attention"] == 2 * 2 * 4096 * 4352 * 128 * 32
