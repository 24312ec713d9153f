"""Merged-gradient communication schedule: plain reference by enumeration.

TEST INFRASTRUCTURE ONLY: the test suite is the only caller.  The library's
own schedule routine shares nothing with this file.

What it follows (MG-WFBP review, "proposed method", bullets 1-3 and 5): the
layers' gradients become ready one after another during back-propagation;
each message pays a start-up cost, so several consecutive layers may be
merged into one message; a schedule is chosen once, before training, to
minimise the iteration time; communication starts as soon as a message's
gradients exist (wait-free back-propagation).  The pages print no cost model,
so the plainest one is taken:

  * layers are numbered in table (forward) order 0..L-1 and back-propagation
    produces them in reverse, L-1 first; layer l takes c[l] time units, so its
    gradient is ready at r[l] = c[L-1] + c[L-2] + ... + c[l], summed in that
    order starting from 0.0;
  * a message of B bytes occupies the link for alpha + beta * B, and the link
    carries one message at a time;
  * a schedule cuts the layers into runs of consecutive layers; a run is one
    message, ready when its last-produced layer (its lowest index) is ready,
    and sent when it is ready and the previous message has finished;
  * the objective is the time the last message (the one holding layer 0)
    finishes; the backward pass and the forward pass are fixed costs.

All arithmetic is IEEE double, one operation at a time, in the order written.
Parity status: pinned by the hand-worked example in tests/golden, by closed
forms and by exhaustive enumeration (tests/test_merge_oracle.py).
"""
from __future__ import annotations

import itertools


def ready_times(c):
    """r[l]: when layer l's gradient exists (back-propagation runs L-1 .. 0)."""
    L = len(c)
    r = [0.0] * L
    t = 0.0
    for l in range(L - 1, -1, -1):
        t = t + float(c[l])
        r[l] = t
    return r


def finish_time(c, nbytes, alpha, beta, runs):
    """Finish of the last message for `runs`, a list of (l0, l1) layer ranges
    [l0, l1) in the order they are sent (back-propagation order: the first
    run holds layer L-1).  The runs must cut [0, L) into consecutive pieces."""
    L = len(c)
    expect_hi = L
    for l0, l1 in runs:
        if l1 != expect_hi or not (0 <= l0 < l1):
            raise ValueError(f"runs do not cut [0, {L}) in back-propagation order: {runs}")
        expect_hi = l0
    if expect_hi != 0:
        raise ValueError(f"runs do not reach layer 0: {runs}")
    r = ready_times(c)
    link_free = 0.0
    for l0, l1 in runs:
        b = 0
        for l in range(l0, l1):
            b += int(nbytes[l])
        start = max(link_free, r[l0])
        link_free = start + (float(alpha) + float(beta) * float(b))
    return link_free


def all_schedules(L):
    """Every cut of [0, L) into runs, each as a list of runs in sending order."""
    for mask in itertools.product((False, True), repeat=L - 1):
        # mask[i] True: a cut between layer i and layer i+1
        runs = []
        hi = L
        for l in range(L - 1, 0, -1):
            if mask[l - 1]:
                runs.append((l, hi))
                hi = l
        runs.append((0, hi))
        yield runs


def best_finish(c, nbytes, alpha, beta):
    """(minimum finish over every schedule, list of the schedules reaching it)."""
    best, arg = None, []
    for runs in all_schedules(len(c)):
        t = finish_time(c, nbytes, alpha, beta, runs)
        if best is None or t < best:
            best, arg = t, [runs]
        elif t == best:
            arg.append(runs)
    return best, arg


def per_layer(L):
    """Wait-free back-propagation without merging: one message per layer."""
    return [(l, l + 1) for l in range(L - 1, -1, -1)]


def single_message(L):
    """Everything in one message after the whole backward pass."""
    return [(0, L)]
