"""The benchmark script's contract, checked without a GPU: it refuses more than
one GPU with a message, and the committed counter summaries under profiles/
belong to the sources that decide what the benchmarked calls run (a summary
taken before a kernel or the configuration choice changed would make the
benchmark report no traffic figure)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "one GPU" in r.stdout


@pytest.mark.parametrize("workload,op", [("sgemm_4096", "sgemm"), ("hgemm_ffn", "hgemm_bias_gelu"),
                                         ("bgemm_ffn", "bgemm_bias_gelu")])
def test_profiles_belong_to_the_current_sources(workload, op):
    traffic = bench.profiled_traffic(workload, op)
    assert traffic is not None, "profiles/%s_counters.md is missing or stale" % workload
    assert traffic > 0
