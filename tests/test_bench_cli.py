"""bench.py's command line on the CPU: a request for more than one GPU is
refused with a message and exit status 2, before torch or the library is
touched (the measured path is one GPU's share of the step)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                         capture_output=True, text=True, timeout=60, cwd=ROOT)
    assert out.returncode == 2
    assert "one GPU only" in out.stderr
    assert out.stdout == ""          # no JSON line for a run that did not happen
