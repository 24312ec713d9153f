"""Pins of the merged-gradient schedule reference (oracle/merge_oracle.py)
against values that do not come from it: a hand-worked example, closed forms
and facts of the cost model."""
import json
import os
import random

import pytest

from oracle import merge_oracle as M

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "merge_schedule_example.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_hand_worked_schedules(case):
    for runs_s, want in case["finish"].items():
        runs = [tuple(r) for r in json.loads(runs_s)]
        assert M.finish_time(case["c"], case["bytes"], case["alpha"], case["beta"], runs) == want
    best, arg = M.best_finish(case["c"], case["bytes"], case["alpha"], case["beta"])
    assert best == case["best"]
    assert {json.dumps([list(r) for r in a]).replace(" ", "") for a in arg} == \
        {k for k, v in case["finish"].items() if v == case["best"]}


def test_enumeration_counts_every_cut():
    for L in range(1, 9):
        scheds = list(M.all_schedules(L))
        assert len(scheds) == 2 ** (L - 1)
        assert len({tuple(s) for s in scheds}) == len(scheds)


def _rand(seed, L, integer=True):
    rnd = random.Random(seed)
    c = [float(rnd.randint(0, 20)) for _ in range(L)] if integer else \
        [rnd.random() * 3 for _ in range(L)]
    b = [rnd.randint(1, 4096) for _ in range(L)]
    return c, b


def test_all_ready_at_once_sends_one_message():
    # every gradient exists at time 0: m messages cost m*alpha + beta*sum(B)
    for seed in range(20):
        L = 1 + seed % 8
        _, b = _rand(seed, L)
        c = [0.0] * L
        alpha, beta = 3.0, 0.25
        best, arg = M.best_finish(c, b, alpha, beta)
        assert best == alpha + beta * sum(b)
        assert arg == [[(0, L)]]


def test_no_startup_cost_per_layer_is_optimal():
    # alpha = 0: splitting a message never delays its parts
    for seed in range(20):
        L = 1 + seed % 8
        c, b = _rand(seed, L)
        best, _ = M.best_finish(c, b, 0.0, 0.0625)
        assert best == M.finish_time(c, b, 0.0, 0.0625, M.per_layer(L))


def test_free_bandwidth_closed_form():
    # beta = 0 and equal layer times: the last gradient is ready at L*c and
    # something must be sent after it, so the best is L*c + alpha
    for L in range(1, 9):
        best, arg = M.best_finish([2.0] * L, [100] * L, 5.0, 0.0)
        assert best == 2.0 * L + 5.0
        assert [(0, L)] in arg


def test_best_bounds_and_lower_bound():
    for seed in range(30):
        L = 1 + seed % 9
        c, b = _rand(seed, L, integer=(seed % 2 == 0))
        alpha, beta = 0.5 + seed % 4, 1.0 / (1 + seed % 5)
        best, arg = M.best_finish(c, b, alpha, beta)
        assert best <= M.finish_time(c, b, alpha, beta, M.per_layer(L))
        assert best <= M.finish_time(c, b, alpha, beta, M.single_message(L))
        # the message with layer 0 starts after the backward pass
        assert best >= sum(c[::-1]) * (1 - 1e-12) + alpha
        for runs in arg:
            assert M.finish_time(c, b, alpha, beta, runs) == best


def test_rejects_bad_runs():
    with pytest.raises(ValueError):
        M.finish_time([1, 1], [8, 8], 1, 1, [(0, 1), (1, 2)])     # wrong order
    with pytest.raises(ValueError):
        M.finish_time([1, 1], [8, 8], 1, 1, [(1, 2)])             # layer 0 missing
