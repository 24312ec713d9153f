"""The library's adaptive per-layer message sizes (lags_adaptive_k; host
code, no GPU) against the reference in oracle/ratio_oracle.py."""
import ctypes
import json
import os
import random

import numpy as np
import pytest

from layer_wise_top_amd import lags
from layer_wise_top_amd import workloads as W
from oracle import ratio_oracle as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "adaptive_ratio_example.json")


def _off(sizes):
    off = np.zeros(len(sizes) + 1, np.int64)
    off[1:] = np.cumsum(sizes)
    return off


def test_golden_cases():
    with open(GOLDEN) as f:
        for case in json.load(f)["cases"]:
            k = lags.lags_adaptive_k(_off(case["sizes"]), case["c"], case["P"], case["alpha"],
                                     case["beta"], tuple(case["rmin"]))
            assert k.tolist() == case["k"], case["name"]


def test_random_against_reference():
    rnd = random.Random(3)
    for _ in range(300):
        L = rnd.randint(1, 40)
        sizes = [rnd.randint(1, 200000) for _ in range(L)]
        c = [rnd.random() * rnd.choice([1e-6, 1e-3, 1.0]) for _ in range(L)]
        P = rnd.randint(1, 64)
        alpha = rnd.random() * rnd.choice([0.0, 1e-6, 1e-4])
        beta = rnd.choice([0.0, 1e-11, 1e-10, 3.3e-9])
        rmin = rnd.choice([(1, 1000), (1, 100), (1, 1), (7, 9)])
        want = R.adaptive_k(sizes, c, P, alpha, beta, *rmin)
        got = lags.lags_adaptive_k(_off(sizes), c, P, alpha, beta, rmin)
        assert got.tolist() == want


@pytest.mark.parametrize("name", ["resnet50", "tfm1p3b"])
def test_workload_tables_and_layouts(name):
    """Backward time proportional to tensor size (synthetic); the sizes match
    the reference and form a valid layout."""
    wl = W.get(name)
    off = wl.offsets()
    c = (np.diff(off) * 66e-12).tolist()
    k = lags.lags_adaptive_k(off, c, wl.P, 20e-6, 1.0 / 50e9, (1, 1000))
    assert k.tolist() == R.adaptive_k(np.diff(off).tolist(), c, wl.P, 20e-6, 1.0 / 50e9, 1, 1000)
    lay = lags.Layout(off, k)
    assert lay.K == int(k.sum())
    lay.close()


def test_rejects_bad_inputs():
    Lb = lags.lib()
    off = np.array([0, 10, 30], np.int64)
    bt = np.ones(2)
    k = np.empty(2, np.int64)

    def call(L=2, off=off, bt=bt, P=4, alpha=0.0, beta=1.0, num=1, den=100):
        return Lb.lags_adaptive_k(L, off.ctypes.data, bt.ctypes.data, P, alpha, beta, num, den,
                                  k.ctypes.data)
    assert call() == 0
    assert call(L=0) == -2
    assert call(P=0) == -2 and call(P=1025) == -2
    assert call(alpha=-1.0) == -1 and call(beta=float("inf")) == -1
    assert call(num=0) == -1 and call(num=3, den=2) == -1
    assert call(off=np.array([1, 10, 30], np.int64)) == -1
    assert call(off=np.array([0, 10, 10], np.int64)) == -1
    assert call(bt=np.array([1.0, -1.0])) == -1
    assert call(off=np.array([0, 10, 1 << 41], np.int64)) == -2
    assert Lb.lags_adaptive_k(2, off.ctypes.data, None, 4, 0.0, 1.0, 1, 100, k.ctypes.data) == -1
