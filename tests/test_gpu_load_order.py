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
import os, sys
import numpy as np
from layer_wise_top_amd import lags
lay = lags.Layout([0, 50000, 60000], [50, 10])    # the library is loaded here
import torch
import oracle
seed = int.from_bytes(os.urandom(4), "little")
print("seed", seed, flush=True)
ws = lags.workspace(lay, 1)
gen = torch.Generator(device="cuda")
gen.manual_seed(seed)
g = torch.randn(60000, device="cuda", generator=gen)
r = torch.zeros_like(g)
mi = torch.empty(60, dtype=torch.int32, device="cuda")
mv = torch.empty(60, device="cuda")
lags.lags_sparsify_layers(lay, g, r, mi, mv, ws)
torch.cuda.synchronize()
gn, rg = g.cpu().numpy(), r.cpu().numpy()
mi_o, mv_o, r_o = oracle.default().sparsify(np.array([0, 50000, 60000]), np.array([50, 10]), gn,
                                            np.zeros(60000, np.float32))
ok_m = np.array_equal(mi.cpu().numpy().view(np.uint32), mi_o)
diff = np.flatnonzero(rg.view(np.uint32) != r_o.view(np.uint32))
if not ok_m or diff.size:
    print("zeros", int((rg == 0).sum()), "messages equal", ok_m, "residual mismatches", diff[:20],
          "report", lags.lags_workspace_report(lay, ws), flush=True)
    sys.exit(1)
print("load order ok", flush=True)
"""


def test_library_loaded_before_torch():
    out = subprocess.run([sys.executable, "-c", CODE], cwd=ROOT, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "load order ok" in out.stdout
