"""bench.py on the host: every mode it offers is defined, and it refuses several GPUs."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_every_mode_has_its_function():
    for name in ("bench_train", "bench_decode", "bench_variants", "cpu_baseline",
                 "bench_workloads", "bench_copy", "measured_traffic", "kernel_source_hash"):
        assert callable(getattr(bench, name, None)), name


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]
