"""bench.py's command line on a machine without a GPU: the one-GPU rule and
the row-count override are checked before anything touches a device."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused_with_a_message(n):
    r = run_bench("--gpus", n)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


@pytest.mark.parametrize("args", [["--workload", "gemm_8192", "--rows", "512"],
                                  ["--workload", "qwen3_8b_rebatch_fwd", "--rows", "512"],
                                  ["--rows", "0"]])
def test_row_override_only_for_linear_logp_workloads(args):
    r = run_bench(*args)
    assert r.returncode == 2
    assert "--rows" in r.stderr
