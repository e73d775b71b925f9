"""The benchmark's command-line contract on the CPU: more than one GPU is refused with a message, and
without a GPU the benchmark stops instead of measuring anything on the host."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    r = _bench("--gpus", n)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and f"--gpus {n}" in r.stderr
    assert r.stdout == ""   # no JSON line


@pytest.mark.skipif(torch.cuda.is_available(), reason="only meaningful on a host without a GPU")
def test_no_gpu_stops_without_a_result():
    r = _bench("--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "needs a GPU" in r.stderr
    assert r.stdout == ""
