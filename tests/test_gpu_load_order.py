"""The binding binds the library to torch's HIP runtime whatever the import
order: a process that loads the library before it first imports torch must
still run the hot path on torch's buffers and streams (with two runtimes in
one process, the library's would see no device)."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CODE = """
from layer_wise_top_amd import lags
lay = lags.Layout([0, 50000, 60000], [50, 10])    # the library is loaded here
import torch
ws = lags.workspace(lay, 1)
g = torch.randn(60000, device="cuda")
r = torch.zeros_like(g)
mi = torch.empty(60, dtype=torch.int32, device="cuda")
mv = torch.empty(60, device="cuda")
lags.lags_sparsify_layers(lay, g, r, mi, mv, ws)
torch.cuda.synchronize()
assert int((r == 0).sum()) == 60, "sent entries have a zero residual"
print("load order ok", flush=True)
"""


def test_library_loaded_before_torch():
    out = subprocess.run([sys.executable, "-c", CODE], cwd=ROOT, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "load order ok" in out.stdout
