"""Property tests (hypothesis) of the CPU oracle over random layouts and value
mixes, and of the library's host-side k table.

The layouts are random tensor tables (1-6 layers of 1-400 entries, random k
per layer); the values mix continuous draws, heavy ties, zeros of both signs,
subnormals and infinities.  Each drawn case is checked against what the
definition fixes independently of the oracle's code: the exact invariants of
a per-layer top-k with residual (sizes, value and residual bits, order, the
tie prefix), a second route to the selected set (numpy's stable argsort of
the negated keys), brute force over all subsets for tiny layers, exact
rational arithmetic for the aggregate on dyadic values, and exact rational
ceilings for k.  derandomize=True: every run draws the same cases.
"""
from fractions import Fraction

import numpy as np
from hypothesis import given, settings, strategies as st

import pins

SETTINGS = dict(max_examples=120, deadline=None, derandomize=True)

# fp32 values the selection must order by magnitude bits: a few fixed
# specials (signed zeros, the smallest subnormals, infinities, values that tie
# in magnitude with opposite signs) and arbitrary finite fp32 draws
_SPECIAL = [0.0, -0.0, 1.0, -1.0, 2.0 ** -149, -(2.0 ** -149), 2.0 ** -126, 3.0, -3.0,
            float("inf"), float("-inf"), 0.5, -0.5]
_finite32 = st.floats(width=32, allow_nan=False, allow_infinity=False)
_value = st.one_of(st.sampled_from(_SPECIAL), _finite32)
_tie = st.sampled_from([0.0, -0.0, 0.25, -0.25, 7.0, -7.0])


@st.composite
def layouts(draw, max_layers=6, max_n=400):
    sizes = draw(st.lists(st.integers(1, max_n), min_size=1, max_size=max_layers))
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    k = np.array([draw(st.integers(1, s)) for s in sizes], np.int64)
    return off, k


@st.composite
def step_inputs(draw):
    off, k = draw(layouts())
    n = int(off[-1])
    mix = draw(st.sampled_from(["any", "ties", "mixed"]))
    elem = {"any": _value, "ties": _tie, "mixed": st.one_of(_value, _tie)}[mix]
    g = np.array(draw(st.lists(elem, min_size=n, max_size=n)), np.float32)
    # the residual stays finite so that acc = g + r never meets inf - inf
    rel = {"any": _finite32, "ties": _tie, "mixed": st.one_of(_finite32, _tie)}[mix]
    r = np.array(draw(st.lists(rel, min_size=n, max_size=n)), np.float32)
    return off, k, g, r


@settings(**SETTINGS)
@given(step_inputs())
def test_selection_invariants_random_layouts(oracle, case):
    """Per layer: exactly k entries, values bit for bit, residual +0.0 at the
    sent entries and acc elsewhere, ascending indices inside the layer, every
    sent key >= every unsent key, ties taken as an index prefix; and the same
    set as numpy's stable argsort of the negated keys."""
    off, k, g, r = case
    mi, mv, r2 = oracle.sparsify(off, k, g, r)
    acc = (g + r).astype(np.float32)
    pins.check_invariants(off, k, acc, mi, mv, r2)
    assert np.array_equal(mi, pins.selection_by_argsort(acc, off, k))


@settings(**SETTINGS)
@given(st.lists(st.one_of(_value, _tie), min_size=1, max_size=7))
def test_tiny_layer_equals_brute_force(oracle, vals):
    """For every k, the selected set is the unique k-subset that precedes
    every other entry in (key descending, index ascending) order, found by
    enumerating all subsets."""
    g = np.array(vals, np.float32)
    n = g.size
    keys = [pins.key_py(float(x)) for x in g]
    want = pins.brute_select(keys)
    z = np.zeros(n, np.float32)
    for kk in range(1, n + 1):
        mi, mv, r2 = oracle.sparsify([0, n], [kk], g, z)
        assert mi.tolist() == want[kk]


@st.composite
def dyadic_messages(draw):
    """P workers' messages over n weights: distinct ascending indices per
    worker, values m * 2^-6 with |m| < 2^10, so every partial sum of up to 8
    workers and the scaled update are exact in fp32."""
    n = draw(st.integers(1, 120))
    P = draw(st.integers(1, 8))
    K = draw(st.integers(1, n))
    idx, val = [], []
    for _ in range(P):
        ids = sorted(draw(st.sets(st.integers(0, n - 1), min_size=K, max_size=K)))
        vs = [draw(st.integers(-1023, 1023)) / 64.0 for _ in range(K)]
        idx.append(ids)
        val.append(vs)
    w = [draw(st.integers(-4096, 4096)) / 64.0 for _ in range(n)]
    lr_exp = draw(st.integers(-4, 0))      # lr = 2^e, P a power of two: s = lr / P exact
    P2 = 1 << (P.bit_length() - 1)
    return (np.array(idx[:P2], np.uint32), np.array(val[:P2], np.float32),
            np.array(w, np.float32), 2.0 ** lr_exp)


@settings(**SETTINGS)
@given(dyadic_messages())
def test_aggregate_exact_on_dyadic_values(oracle, case):
    """With dyadic values every rounding is exact, so the aggregate must equal
    the rational result w - (lr / P) * sum of the workers' values at every
    touched index, and leave untouched weights alone."""
    idx, val, w, lr = case
    P = idx.shape[0]
    got = oracle.aggregate(idx, val, w, lr)
    u = {}
    for p in range(P):
        for i, v in zip(idx[p].tolist(), val[p].tolist()):
            u[i] = u.get(i, Fraction(0)) + Fraction(v)
    s = Fraction(lr) / P
    want = [Fraction(float(x)) for x in w]
    for i, ui in u.items():
        want[i] -= s * ui
    assert all(Fraction(float(got[i])) == want[i] for i in range(w.size))


@settings(**SETTINGS)
@given(st.integers(1, 2 ** 32 - 1), st.integers(1, 1000), st.integers(1, 1000))
def test_k_for_ratio_is_the_exact_ceiling(oracle, n, a, b):
    """k = ceil(n * a / b) by exact rationals, clamped to [1, n], from the
    oracle and from the library's host routine alike."""
    from layer_wise_top_amd import lags
    num, den = min(a, b), max(a, b)           # ratios in (0, 1]
    exact = Fraction(n * num, den)
    k_o = int(oracle.k_for_ratio(n, num, den))
    k_l = int(lags.lags_k_for_ratio(n, num, den))
    assert k_o == k_l
    assert 1 <= k_o <= n
    assert k_o - 1 < exact <= k_o
