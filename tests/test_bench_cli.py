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


def test_traffic_figure_follows_the_decode_machine_code(tmp_path, monkeypatch):
    """roofline.traffic comes from the committed counters only while the
    library's decode kernel has the machine code they were taken on: the hash
    is read from the built library's gfx950 code object (16 hex digits, stable
    across reads), and a record for other machine code yields None."""
    sys.path.insert(0, ROOT)
    import json
    import bench
    from mla_latent_kv_19_amd import api
    lib = api.library_path()
    if not os.path.exists(lib):
        pytest.skip("libmla.so not built")
    h = bench.kernel_code_hash(lib)
    assert h is not None and len(h) == 16 and int(h, 16) >= 0
    assert bench.kernel_code_hash(lib) == h
    assert bench.kernel_code_hash(lib, r"combine_kernel") not in (None, h)
    rec = {"kernel_code_sha": h, "hbm_bytes_per_launch": 123.0}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic(lib) == 123.0
    rec["kernel_code_sha"] = "0" * 16 if h != "0" * 16 else "1" * 16
    f.write_text(json.dumps(rec))
    assert bench.measured_traffic(lib) is None
