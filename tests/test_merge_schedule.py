"""The library's merged-gradient schedule (lags_merge_schedule,
lags_schedule_finish; host code, no GPU) against the enumeration reference."""
import ctypes
import json
import os
import random

import numpy as np
import pytest

from layer_wise_top_amd import lags
from layer_wise_top_amd import workloads as W
from oracle import merge_oracle as M

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "merge_schedule_example.json")


def _instance(seed, L):
    rnd = random.Random(seed)
    kind = seed % 3
    if kind == 0:                   # integer times and dyadic costs: many ties
        c = [float(rnd.randint(0, 6)) for _ in range(L)]
        alpha, beta = float(rnd.randint(0, 5)), rnd.choice([0.0, 0.125, 0.25, 1.0])
    elif kind == 1:                 # arbitrary doubles
        c = [rnd.random() * 2.0 for _ in range(L)]
        alpha, beta = rnd.random() * 3.0, rnd.random() * 1e-3
    else:                           # a few slow layers among many fast ones
        c = [rnd.choice([0.01, 0.02, 5.0]) for _ in range(L)]
        alpha, beta = rnd.choice([0.1, 1.0, 10.0]), 1e-3
    b = [rnd.choice([8, 64, 512, 8 * rnd.randint(1, 5000)]) for _ in range(L)]
    return c, b, alpha, beta


def test_golden_cases():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        runs, fin = lags.lags_merge_schedule(case["c"], case["bytes"], case["alpha"], case["beta"])
        assert fin == case["best"], case["name"]
        assert M.finish_time(case["c"], case["bytes"], case["alpha"], case["beta"], runs) == fin
        for runs_s, want in case["finish"].items():
            rr = [tuple(r) for r in json.loads(runs_s)]
            assert lags.lags_schedule_finish(case["c"], case["bytes"], case["alpha"],
                                             case["beta"], rr) == want


@pytest.mark.parametrize("L", list(range(1, 13)))
def test_optimum_matches_enumeration(L):
    for seed in range(12):
        c, b, alpha, beta = _instance(1000 * L + seed, L)
        runs, fin = lags.lags_merge_schedule(c, b, alpha, beta)
        best, arg = M.best_finish(c, b, alpha, beta)
        assert fin == best, (L, seed, fin, best)
        assert runs in arg, (L, seed, runs)


def test_sixteen_layers_against_enumeration():
    c, b, alpha, beta = _instance(77, 16)
    runs, fin = lags.lags_merge_schedule(c, b, alpha, beta)
    best, arg = M.best_finish(c, b, alpha, beta)
    assert fin == best and runs in arg


def test_finish_of_given_schedules_matches_reference():
    rnd = random.Random(5)
    for seed in range(50):
        L = 1 + seed % 20
        c, b, alpha, beta = _instance(seed, L)
        cuts = sorted(rnd.sample(range(1, L), rnd.randint(0, L - 1))) if L > 1 else []
        edges = [L] + cuts[::-1] + [0]
        runs = [(edges[j + 1], edges[j]) for j in range(len(edges) - 1)]
        assert lags.lags_schedule_finish(c, b, alpha, beta, runs) == \
            M.finish_time(c, b, alpha, beta, runs)


@pytest.mark.parametrize("name", ["resnet50", "tfm1p3b"])
def test_workload_schedules(name):
    """Whole models: backward time of a tensor taken proportional to its size
    (synthetic), bytes = one worker's message 8 * k[l]; a start-up cost of
    100 us and 25 GB/s.  The schedule is no slower than one message per layer
    or one message for the model, and its reported finish is its own."""
    wl = W.get(name)
    off = wl.offsets()
    num, den = wl.ratios()
    k = lags.k_table(off, num, den)
    n = np.diff(off).astype(np.float64)
    c = (n * 1e-9).tolist()                         # 1 ns per parameter
    b = (8 * k).tolist()
    alpha, beta = 100e-6, 1.0 / 25e9
    runs, fin = lags.lags_merge_schedule(c, b, alpha, beta)
    L = wl.L
    assert runs[0][1] == L and runs[-1][0] == 0
    assert M.finish_time(c, b, alpha, beta, runs) == fin
    assert fin <= M.finish_time(c, b, alpha, beta, M.per_layer(L))
    assert fin <= M.finish_time(c, b, alpha, beta, M.single_message(L))
    assert 1 <= len(runs) < L


def test_closed_forms_through_the_library():
    L = 9
    c, b, _, _ = _instance(3, L)
    # no start-up cost: as fast as one message per layer
    _, fin = lags.lags_merge_schedule(c, b, 0.0, 0.125)
    assert fin == M.finish_time(c, b, 0.0, 0.125, M.per_layer(L))
    # all ready at once: a single message
    runs, fin = lags.lags_merge_schedule([0.0] * L, b, 2.0, 0.5)
    assert runs == [(0, L)] and fin == 2.0 + 0.5 * sum(b)


def test_rejects_bad_inputs():
    Lb = lags.lib()
    bt = np.ones(3)
    nb = np.full(3, 8, np.int64)
    bounds = np.empty(4, np.int32)
    nr, fin = ctypes.c_int32(), ctypes.c_double()

    def call(L=3, bt=bt, nb=nb, alpha=1.0, beta=1.0):
        return Lb.lags_merge_schedule(L, bt.ctypes.data if bt is not None else None,
                                      nb.ctypes.data, alpha, beta, bounds.ctypes.data,
                                      ctypes.byref(nr), ctypes.byref(fin))
    assert call() == 0
    assert call(L=0) == -2
    assert call(L=lags.LAGS_MAX_LAYERS + 1) == -2
    assert call(bt=None) == -1
    assert call(alpha=-1.0) == -1
    assert call(beta=float("nan")) == -1
    assert call(bt=np.array([1.0, -1.0, 1.0])) == -1
    assert call(bt=np.array([1.0, float("inf"), 1.0])) == -1
    assert call(nb=np.array([8, -8, 8], np.int64)) == -1
    assert call(nb=np.array([2 ** 52, 2 ** 52, 8], np.int64)) == -2
    with pytest.raises(ValueError):
        lags.lags_schedule_finish(bt, nb, 1.0, 1.0, [(0, 2), (2, 3)])   # wrong order
    good = np.array([3, 1, 0], np.int32)
    bad = np.array([3, 1, 1], np.int32)
    assert Lb.lags_schedule_finish(3, bt.ctypes.data, nb.ctypes.data, 1.0, 1.0,
                                   good.ctypes.data, 2, ctypes.byref(fin)) == 0
    assert Lb.lags_schedule_finish(3, bt.ctypes.data, nb.ctypes.data, 1.0, 1.0,
                                   bad.ctypes.data, 2, ctypes.byref(fin)) == -1
    assert Lb.lags_schedule_finish(3, bt.ctypes.data, nb.ctypes.data, 1.0, 1.0,
                                   good.ctypes.data, 0, ctypes.byref(fin)) == -1
