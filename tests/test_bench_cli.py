"""bench.py's command-line contract, checked on the CPU: one GPU only, and a
clear error instead of a number where no GPU is present."""

import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU path")
def test_no_gpu_is_an_error_not_a_number():
    r = _run("--steps", "1", "--warmup", "0", "--no-cpu-baseline")
    assert r.returncode == 2
    assert "needs a GPU" in r.stderr
    assert r.stdout.strip() == ""
