"""bench.py's command line on a host without a GPU: a multi-GPU request is refused with a
message (the path is timed on one GPU), and a run without a GPU fails loudly instead of
falling back to the CPU."""
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent


def _run(*args):
    return subprocess.run([sys.executable, str(ROOT / "bench.py"), *args], capture_output=True, text=True,
                          timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "measures one GPU" in r.stderr and "--gpus 2 is not supported" in r.stderr
    assert r.stdout == ""


def test_no_gpu_fails_loudly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode == 2 and "needs a GPU" in r.stderr
    assert r.stdout == ""
