"""Pins of the adaptive per-layer message size reference
(oracle/ratio_oracle.py): a hand-worked example, exact-rational checks of
the fit, bounds and monotonicity."""
import json
import os
import random
from fractions import Fraction

import pytest

from oracle import ratio_oracle as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "adaptive_ratio_example.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_hand_worked(case):
    got = R.adaptive_k(case["sizes"], case["c"], case["P"], case["alpha"], case["beta"],
                       case["rmin"][0], case["rmin"][1])
    assert got == case["k"]


def test_lower_bound_is_exact_ceiling():
    for n in (1, 7, 999, 1000, 1001, 123457):
        for num, den in ((1, 1000), (1, 100), (3, 10), (1, 1)):
            k = R.lower_bound(n, num, den)
            assert Fraction(k - 1) < Fraction(n * num, den) <= Fraction(k)


def _random_case(seed):
    rnd = random.Random(seed)
    L = rnd.randint(1, 12)
    sizes = [rnd.randint(1, 5000) for _ in range(L)]
    # dyadic inputs: every double operation below is exact
    c = [rnd.randint(0, 4096) / 64.0 for _ in range(L)]
    P = rnd.randint(1, 9)
    alpha = rnd.randint(0, 64) / 16.0
    beta = rnd.choice([0.0, 1 / 1024, 1 / 256, 1 / 64])
    return sizes, c, P, alpha, beta


def test_chosen_size_fits_the_window_exactly():
    for seed in range(200):
        sizes, c, P, alpha, beta = _random_case(seed)
        ks = R.adaptive_k(sizes, c, P, alpha, beta, 1, 100)
        for l, (n, k) in enumerate(zip(sizes, ks)):
            lo = R.lower_bound(n, 1, 100)
            assert lo <= k <= n
            if P == 1 or beta == 0.0:
                assert k == n
                continue
            if l == 0:
                assert k == lo
                continue
            cost = lambda m: Fraction(alpha) + Fraction(beta) * 8 * (P - 1) * m
            if lo < k < n:
                assert cost(k) <= Fraction(c[l - 1]) < cost(k + 1)
            elif k == lo and lo < n:
                assert Fraction(c[l - 1]) < cost(lo + 1)
            elif k == n and n > lo:
                assert cost(n) <= Fraction(c[l - 1])


def test_more_backward_time_never_shrinks_a_message():
    for seed in range(50):
        sizes, c, P, alpha, beta = _random_case(seed)
        a = R.adaptive_k(sizes, c, P, alpha, beta, 1, 1000)
        b = R.adaptive_k(sizes, [x * 2 for x in c], P, alpha, beta, 1, 1000)
        assert all(y >= x for x, y in zip(a, b))
