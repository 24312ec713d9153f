"""The allocation-free sparsify (lags_sparsify_layers_static) through the C ABI:
bit for bit the same messages and residual as lags_sparsify_layers with a
workspace, on consecutive calls whose layouts shrink (the static buffer keeps
the previous call's contents) and then return to the first layout (its
tables are copied in again)."""
import ctypes

import numpy as np
import pytest

from gpu_helpers import assert_bits_equal, to_dev, to_np_f32, to_np_u32
from layer_wise_top_amd import lags, workloads as W

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _case(name, seed):
    wl = W.get(name)
    off = wl.offsets()
    num, den = wl.ratios()
    k = lags.k_table(off, num, den)
    lay = lags.Layout(off, k)
    rng = np.random.default_rng(seed)
    g = W.gen_grad(wl, 0)
    r0 = (0.5 * rng.standard_normal(wl.n) * np.abs(g)).astype(np.float32)   # a carried residual
    return lay, g, r0


def _compare(lay, g, r0, flags, tag):
    import torch
    g_d = to_dev(g)
    ws = lags.workspace(lay, 1)
    outs = []
    for static in (False, True):
        r = to_dev(r0)
        mi = torch.full((lay.K,), -1, dtype=torch.int32, device="cuda")
        mv = torch.full((lay.K,), float("nan"), dtype=torch.float32, device="cuda")
        if static:
            lags.lags_sparsify_layers_static(lay, g_d, r, mi, mv, flags)
        else:
            lags.lags_sparsify_layers(lay, g_d, r, mi, mv, ws, flags)
        torch.cuda.synchronize()
        outs.append((to_np_u32(mi), to_np_f32(mv), to_np_f32(r)))
    (ai, av, ar), (bi, bv, br) = outs
    assert_bits_equal(f"{tag} msg_idx", bi, ai)
    assert_bits_equal(f"{tag} msg_val", bv, av)
    assert_bits_equal(f"{tag} residual", br, ar)


def test_static_sparsify_matches_the_workspace_call():
    cases = [("vgg16", 0, 1), ("resnet20", 0, 2), ("resnet20", 1, 3), ("vgg16", 0, 4)]
    layouts = {}
    for name, flags, seed in cases:
        _say(f"[static] {name} flags={flags}")
        if name not in layouts:
            layouts[name] = _case(name, seed)
        lay, g, r0 = layouts[name]
        _compare(lay, g, r0, flags, f"{name}/{flags}/{seed}")


def test_static_sparsify_rejects_a_layout_beyond_its_buffer():
    """The 1.3B-entry layout needs ~480 MiB of tables and scratch: refused
    before anything is launched."""
    wl = W.get("tfm1p3b")
    off = wl.offsets()
    num, den = wl.ratios()
    lay = lags.Layout(off, lags.k_table(off, num, den))
    base = 1 << 40                         # never dereferenced
    rc = lags.lib().lags_sparsify_layers_static(lay.handle, base, base + (8 << 30), base + (16 << 30),
                                                base + (17 << 30), 0, None)
    assert rc == lags.LAGS_ESTATIC
    assert "static" in lags.strerror(rc)
