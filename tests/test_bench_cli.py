"""bench.py's command-line contract, checked on the CPU: one GPU only (--gpus
N > 1 exits with a message, before anything touches a GPU), a calibration
copy of at most 2 GiB (one dispatch), and a clear error where no GPU is
present."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=600)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""          # no JSON line


def test_calibration_copy_above_2gib_is_refused():
    r = run_bench("--calib-bytes", str(2 ** 32))
    assert r.returncode == 2
    assert "2 GiB" in r.stderr


def test_no_gpu_is_a_clear_error():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = run_bench("--steps", "1", "--warmup", "0")
    assert r.returncode == 1
    assert "needs a GPU" in r.stderr
