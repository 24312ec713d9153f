"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
its host-side validation rejects bad arguments before any device call."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import pins
from layer_wise_top_amd import lags

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lags.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lags_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 16
    L = lags.lib()
    for name in names:
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", lags.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (lags_\w+)", out))
    assert set(names) <= exported
    assert set(names) == set(lags.EXPORTED)


def test_strerror():
    for code in range(0, -7, -1):
        assert lags.strerror(code)
    assert lags.strerror(-99) == "unknown status"


def test_k_for_ratio_golden():
    for n, a, b, k in pins.golden()["k_for_ratio"]["cases"]:
        assert lags.lags_k_for_ratio(n, a, b) == k
    assert lags.lags_k_for_ratio(0, 1, 10) == 0
    assert lags.lags_k_for_ratio(-1, 1, 10) == -1
    assert lags.lags_k_for_ratio(10, 0, 10) == -1
    assert lags.lags_k_for_ratio(10, 11, 10) == -1


def test_k_tables_match_oracle(oracle):
    from layer_wise_top_amd import workloads as W
    for name in W.ORDER:
        wl = W.get(name)
        num, den = wl.ratios()
        off = wl.offsets()
        assert np.array_equal(lags.k_table(off, num, den),
                              oracle.k_for_ratio(np.diff(off), num, den))


def _create(off, k):
    off = np.ascontiguousarray(off, np.int64)
    k = np.ascontiguousarray(k, np.int64)
    h = ctypes.c_void_p()
    rc = lags.lib().lags_layout_create(int(k.size), off.ctypes.data, k.ctypes.data, ctypes.byref(h))
    if rc == 0:
        lags.lib().lags_layout_destroy(h)
    return rc


def test_layout_validation():
    assert _create([0, 10, 20], [1, 10]) == 0
    assert _create([1, 10, 20], [1, 1]) == -1      # does not start at 0
    assert _create([0, 10, 10], [1, 1]) == -1      # empty layer
    assert _create([0, 10, 5], [1, 1]) == -1       # decreasing
    assert _create([0, 10, 20], [0, 1]) == -1      # k = 0
    assert _create([0, 10, 20], [11, 1]) == -1     # k > n
    assert _create([0, 2**32], [1]) == -2          # n >= 2^32
    assert _create([0, 2**32 - 1], [1]) == -2      # 0xffffffff stays free as a marker
    assert _create([0, 2**32 - 2], [1]) == 0       # the largest accepted size
    assert lags.lib().lags_layout_create(0, None, None, ctypes.byref(ctypes.c_void_p())) == -1
    off = np.array([0, 1], np.int64)
    k = np.array([1], np.int64)
    assert lags.lib().lags_layout_create(0, off.ctypes.data, k.ctypes.data,
                                         ctypes.byref(ctypes.c_void_p())) == -2


def test_layout_queries_and_workspace():
    from layer_wise_top_amd import workloads as W
    wl = W.get("resnet50")
    off = wl.offsets()
    num, den = wl.ratios()
    k = lags.k_table(off, num, den)
    lay = lags.Layout(off, k)
    assert lay.n == wl.n and lay.K == int(k.sum()) and lay.L == wl.L
    assert lay.msg_offset(0) == 0 and lay.msg_offset(wl.L) == lay.K
    assert lay.msg_offset(5) == int(k[:5].sum())
    assert lay.msg_offset(-1) == -1 and lay.msg_offset(wl.L + 1) == -1
    b1, b16 = lay.workspace_bytes(1), lay.workspace_bytes(16)
    assert 0 < b1 < b16
    assert lay.workspace_bytes(0) == 0 and lay.workspace_bytes(1025) == 0
    lay.close()


def test_calls_reject_bad_arguments_without_a_device():
    """Every rejected call returns before any HIP call, so this runs on the CPU."""
    L = lags.lib()
    lay = lags.Layout([0, 5000, 9000], [5, 4])
    h = lay.handle
    ws_need = lay.workspace_bytes(1)
    base = 1 << 40                              # never dereferenced
    g, r = base, base + (1 << 20)
    mi, mv = base + (2 << 20), base + (3 << 20)
    ws = base + (4 << 20)
    sp = L.lags_sparsify_layers
    assert sp(None, g, r, mi, mv, ws, ws_need, 0, None) == -1
    assert sp(h, None, r, mi, mv, ws, ws_need, 0, None) == -1
    assert sp(h, g + 4, r, mi, mv, ws, ws_need, 0, None) == -1        # misaligned
    assert sp(h, g, r, mi, mv, ws, ws_need, 2, None) == -1            # unknown flag
    assert sp(h, g, r, mi, mv, ws, 16, 0, None) == -3                 # small workspace
    assert sp(h, g, r, mi, mv, None, ws_need, 0, None) == -3
    assert sp(h, g, g + 16, mi, mv, ws, ws_need, 0, None) == -1       # grad / residual overlap
    assert sp(h, g, r, mi, mi + 8, ws, ws_need, 0, None) == -1        # message overlap
    ag = L.lags_aggregate_apply
    wsP = lay.workspace_bytes(4)
    assert ag(h, g, mi, mv, 0, ctypes.c_float(0.1), ws, wsP, None) == -2
    assert ag(h, g, mi, mv, 1025, ctypes.c_float(0.1), ws, wsP, None) == -2
    assert ag(h, g, mi, mv, 4, ctypes.c_float(0.1), ws, wsP, None) == -7      # not initialised
    assert ag(h, g + 8, mi, mv, 4, ctypes.c_float(0.1), ws, wsP, None) == -1
    assert ag(h, g, mi, mi + 16, 4, ctypes.c_float(0.1), ws, wsP, None) == -1  # idx/val overlap
    # layer ranges: bad ranges are rejected, an empty range launches nothing
    spr, agr = L.lags_sparsify_range, L.lags_aggregate_range
    for l0, l1 in ((-1, 1), (0, 3), (2, 1)):
        assert spr(h, l0, l1, g, r, mi, mv, ws, ws_need, 0, None) == -2
        assert agr(h, l0, l1, g, mi, mv, 4, ctypes.c_float(0.1), ws, wsP, None) == -2
    # an empty range still needs an initialised workspace
    assert spr(h, 1, 1, g, r, mi, mv, ws, ws_need, 0, None) == -7
    assert agr(h, 2, 2, g, mi, mv, 4, ctypes.c_float(0.1), ws, wsP, None) == -7
    assert spr(h, 0, 1, g, r, mi, mv, ws, 16, 0, None) == -3
    assert agr(h, 0, 1, g, mi, mi + 16, 4, ctypes.c_float(0.1), ws, wsP, None) == -1
    assert L.lags_trace_enable(None, 1) == -1
    lay.close()


def test_calls_before_workspace_init_fail():
    """The sparsify and aggregate calls accept only a workspace that
    lags_workspace_init prepared for the layout; the check is on the host, so
    it returns before any HIP call."""
    L = lags.lib()
    lay = lags.Layout([0, 5000, 9000], [5, 4])
    h = lay.handle
    base = 1 << 40                              # never dereferenced
    g, r, mi, mv, ws = (base + (i << 20) for i in range(5))
    for P in (1, 4):
        need = lay.workspace_bytes(P)
        assert L.lags_sparsify_layers(h, g, r, mi, mv, ws, need, 0, None) == lags.LAGS_ENOTINIT
        assert L.lags_sparsify_range(h, 0, 2, g, r, mi, mv, ws, need, 0, None) == lags.LAGS_ENOTINIT
        assert L.lags_aggregate_apply(h, g, mi, mv, P, ctypes.c_float(0.1), ws, need,
                                      None) == lags.LAGS_ENOTINIT
        assert L.lags_aggregate_range(h, 1, 2, g, mi, mv, P, ctypes.c_float(0.1), ws, need,
                                      None) == lags.LAGS_ENOTINIT
    assert "lags_workspace_init" in lags.strerror(lags.LAGS_ENOTINIT)


def test_workspace_init_validation():
    """lags_workspace_init rejects a bad layout, worker count or workspace
    before any HIP call."""
    L = lags.lib()
    lay = lags.Layout([0, 5000, 9000], [5, 4])
    h = lay.handle
    ws = 1 << 40
    need = lay.workspace_bytes(4)
    assert L.lags_workspace_init(None, ws, need, 4, None) == -1
    assert L.lags_workspace_init(h, ws, need, 0, None) == -2
    assert L.lags_workspace_init(h, ws, need, 1025, None) == -2
    assert L.lags_workspace_init(h, None, need, 4, None) == -3
    assert L.lags_workspace_init(h, ws + 8, need, 4, None) == -3     # misaligned
    assert L.lags_workspace_init(h, ws, need - 1, 4, None) == -3     # one byte short
    # the workspace grows with the worker count (chunk-start table, chunk tables)
    sizes = [lay.workspace_bytes(P) for P in (1, 4, 64, 1024)]
    assert sizes == sorted(sizes) and sizes[0] < sizes[-1]


def test_no_device_allocation_in_the_library():
    """The library allocates no device memory: its sources call neither
    hipMalloc nor hipFree (the caller's workspace holds every table)."""
    import glob
    srcs = glob.glob(os.path.join(ROOT, "layer_wise_top_amd", "csrc", "*"))
    assert srcs
    for p in srcs:
        text = open(p).read()
        for name in ("hipMalloc", "hipFree", "hipExtMalloc", "hipHostMalloc"):
            assert name not in text, (p, name)


def test_static_sparsify_size_limit_without_a_device():
    """lags_sparsify_layers_static refuses a layout whose tables and scratch
    exceed its static buffer before any HIP call."""
    from layer_wise_top_amd import workloads as W
    wl = W.get("tfm1p3b")
    off = wl.offsets()
    num, den = wl.ratios()
    lay = lags.Layout(off, lags.k_table(off, num, den))
    base = 1 << 40                              # never dereferenced
    rc = lags.lib().lags_sparsify_layers_static(lay.handle, base, base + (8 << 30), base + (16 << 30),
                                                base + (17 << 30), 0, None)
    assert rc == lags.LAGS_ESTATIC
    assert lags.lib().lags_sparsify_layers_static(None, base, base, base, base, 0, None) == -1
