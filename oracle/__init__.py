"""Python access to the LAGS-SGD CPU oracle (plain C, lags_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark are the only callers.  The GPU library never loads it.

Every function copies its inputs; nothing is modified in place.  See
lags_oracle.c for the definition each routine follows and the passages of the
LAGS review it cites.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "lags_oracle.c")
LIB = os.path.join(_HERE, "liblags_oracle.so")
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(src: str = SRC, out: str = LIB, defines=()) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    cmd = ["gcc", *CFLAGS, *[f"-D{d}" for d in defines], src, "-o", out + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_lib_cache = {}


def load(path: str = LIB):
    """Load (building first if nothing is built) the oracle library."""
    if path in _lib_cache:
        return _lib_cache[path]
    if path == LIB and not os.path.exists(LIB):
        build()
    lib = ctypes.CDLL(path)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.oracle_k_for_ratio.restype = i64
    lib.oracle_k_for_ratio.argtypes = [i64, i64, i64]
    lib.oracle_sparsify.restype = ctypes.c_int
    lib.oracle_sparsify.argtypes = [i32, vp, vp, vp, vp, vp, vp]
    lib.oracle_aggregate.restype = ctypes.c_int
    lib.oracle_aggregate.argtypes = [i32, i64, vp, vp, vp, ctypes.c_float, i64, i64]
    _lib_cache[path] = lib
    return lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """Thin wrapper around one build of the oracle library."""

    def __init__(self, path: str = LIB):
        self.lib = load(path)

    def k_for_ratio(self, n, num, den) -> np.ndarray:
        n, num, den = (np.broadcast_to(np.asarray(x, dtype=np.int64), np.shape(n))
                       for x in (n, num, den))
        out = np.array([self.lib.oracle_k_for_ratio(int(a), int(b), int(c))
                        for a, b, c in zip(np.ravel(n), np.ravel(num), np.ravel(den))],
                       dtype=np.int64)
        return out.reshape(np.shape(n))

    def sparsify(self, off, k, grad, residual):
        """Returns (msg_idx uint32 [K], msg_val float32 [K], residual' float32 [n])."""
        off = np.ascontiguousarray(off, dtype=np.int64)
        k = np.ascontiguousarray(k, dtype=np.int64)
        L = off.size - 1
        g = np.ascontiguousarray(grad, dtype=np.float32)
        r = np.array(residual, dtype=np.float32, copy=True)
        K = int(k.sum())
        mi = np.empty(K, dtype=np.uint32)
        mv = np.empty(K, dtype=np.float32)
        rc = self.lib.oracle_sparsify(L, _p(off), _p(k), _p(g), _p(r), _p(mi), _p(mv))
        if rc != 0:
            raise ValueError(f"oracle_sparsify failed ({rc})")
        return mi, mv, r

    def aggregate(self, msg_idx, msg_val, w, lr, lo: int = 0, hi: int | None = None):
        """Apply the P-worker aggregate to w (a copy).  msg_* are [P, K].
        If lo/hi are given, `w` holds only the slice [lo, hi)."""
        mi = np.ascontiguousarray(msg_idx, dtype=np.uint32)
        mv = np.ascontiguousarray(msg_val, dtype=np.float32)
        if mi.ndim == 1:
            mi, mv = mi[None], mv[None]
        P, K = mi.shape
        w2 = np.array(w, dtype=np.float32, copy=True)
        if hi is None:
            hi = lo + w2.size
        if w2.size != hi - lo:
            raise ValueError("w must hold exactly the slice [lo, hi)")
        rc = self.lib.oracle_aggregate(P, K, _p(mi), _p(mv), _p(w2),
                                       float(np.float32(lr)), int(lo), int(hi))
        if rc != 0:
            raise ValueError(f"oracle_aggregate failed ({rc})")
        return w2

    def step(self, off, k, grad, residual, other_idx, other_val, w, lr):
        """One full data-parallel step for worker 0: sparsify, then aggregate
        worker 0's message with the other workers' messages ([P-1, K])."""
        mi, mv, r = self.sparsify(off, k, grad, residual)
        if other_idx is None or np.size(other_idx) == 0:
            ai, av = mi[None], mv[None]
        else:
            ai = np.concatenate([mi[None], np.asarray(other_idx, np.uint32)], axis=0)
            av = np.concatenate([mv[None], np.asarray(other_val, np.float32)], axis=0)
        w2 = self.aggregate(ai, av, w, lr)
        return mi, mv, r, w2


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
