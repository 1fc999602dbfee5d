"""The bench's command-line contract on the CPU: more than one GPU is refused with a message,
a machine without a GPU gets an error rather than a fallback, and the committed HBM-counter
summaries still match the kernel sources they were taken on (the bench reports their
traffic only while the sources hash to the recorded value)."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_no_gpu_is_an_error_not_a_fallback():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible here")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0
    assert "no GPU" in r.stderr
    assert '"metric"' not in r.stdout


@pytest.mark.parametrize("workload", ["llama_gqa4", "wide_gqa6", "skewed_gqa8"])
def test_counter_summaries_match_the_sources(workload):
    bench = _bench_module()
    assert os.path.exists(bench.traffic_profile_path(workload))
    traffic = bench.profiled_traffic(workload)
    assert traffic is not None, f"{workload}: kernel sources changed since the counters were taken"
    assert traffic > 0
