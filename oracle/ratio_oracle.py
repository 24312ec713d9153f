"""Per-layer message sizes from the communication-to-computation ratio:
plain reference.

TEST INFRASTRUCTURE ONLY: the test suite is the only caller.  The library's
own routine shares nothing with this file.

What it follows (LAGS review, "proposed method", bullets 2 and 3): each
layer's sparsification ratio adapts to that layer's communication-to-
computation ratio so that, with layer-wise pipelining, a layer's
communication hides behind the back-propagation that follows it.  The pages
give no formula, so the plainest reading is taken:

  * back-propagation produces layers L-1 .. 0; while layer l's message is
    exchanged, the backward pass computes layer l-1, which takes c[l-1];
  * exchanging k entries of one layer costs alpha + beta * B with
    B = 8 * (P - 1) * k bytes (an all-gather of P messages of k (index,
    value) pairs of 8 bytes: each worker receives P - 1 of them);
  * k[l] is the largest count whose exchange fits that window,
    floor((c[l-1] - alpha) / (beta * 8 * (P - 1))), kept within
    [ceil(n_l * rmin_num / rmin_den), n_l]; layer 0 has no window and takes
    the lower bound; with P == 1 or beta == 0 nothing is exchanged and every
    layer is sent whole.

All arithmetic is in the order written: budget = c[l-1] - alpha and
per_entry = beta * (8 * (P - 1)) in IEEE double, then floor(budget /
per_entry); the lower bound in exact integers.
Parity status: pinned by the hand-worked example in tests/golden and by
closed forms (tests/test_ratio_oracle.py).
"""
from __future__ import annotations

import math


def lower_bound(n: int, rmin_num: int, rmin_den: int) -> int:
    """ceil(n * rmin_num / rmin_den), exactly."""
    return -((-n * rmin_num) // rmin_den)


def adaptive_k(sizes, backward_time, P: int, alpha: float, beta: float,
               rmin_num: int, rmin_den: int):
    L = len(sizes)
    per_entry = float(beta) * float(8 * (P - 1))
    out = []
    for l in range(L):
        n = int(sizes[l])
        lo = lower_bound(n, rmin_num, rmin_den)
        if per_entry == 0.0:
            out.append(n)
            continue
        if l == 0:
            out.append(lo)
            continue
        budget = float(backward_time[l - 1]) - float(alpha)
        if budget <= 0.0:
            out.append(lo)
            continue
        q = budget / per_entry
        fit = n if q >= n else int(math.floor(q))
        out.append(min(n, max(lo, fit)))
    return out
