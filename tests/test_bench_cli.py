"""bench.py on the CPU: it imports, refuses more than one GPU with a message,
and the helpers its GPU path calls exist (a missing one would otherwise surface
only on a GPU)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_bench_helpers_exist():
    sys.path.insert(0, ROOT)
    import bench

    for name in ("environment", "host_cpu_model", "gpu_clock", "measured_peaks", "one_gemm",
                 "calibrate_copy", "cpu_baseline", "recorded_traffic", "gemm_source_hash"):
        assert callable(getattr(bench, name)), name
    assert isinstance(bench.host_cpu_model(), str)
