"""Synthetic gradient workloads and seeded input generators.

This module describes the five gradient layouts the library is exercised on
(tensor tables, value distributions, per-layer compression ratios, worker
counts, step counts) and draws their inputs from seeded numpy generators.  It
holds none of the sparsification or aggregation arithmetic: the number of
entries a layer sends is computed by whoever consumes the ratio table (the
oracle on one side, the library's own integer routine on the other), and the
message generator takes that per-layer count as an argument.

Stand-ins.  The LAGS-SGD review ("Layer-wise Adaptive Gradient Sparsification
for Distributed Deep Learning with Convergence Guarantees", main findings)
trains ResNet-20, VGG-16 and ResNet-50 on image data and an LSTM on PTB.  No
dataset or trained model is used here: each workload is the flat fp32 gradient
buffer of that architecture, filled with seeded draws whose scale follows the
tensor's fan-in.  The fifth workload (a 1.3B-parameter transformer) is not on
the pages; it is the largest layout and sets the bandwidth-bound regime.

Seeds.  Every array is drawn per tensor from
``Generator(PCG64(SeedSequence([cfg_id, step, worker, stream, layer])))`` with
stream 0 = gradient, 1 = message indices, 2 = message values, 3 = initial
weights; tensors above 2^24 entries (single-scale ones) are drawn in chunks of
2^24 with the chunk index appended to the seed.  Draws are float64, rounded to
fp32 (the LSTM workload then rounds to bf16 and widens back to fp32, which
creates heavy exact ties).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

STREAM_GRAD, STREAM_MSG_IDX, STREAM_MSG_VAL, STREAM_W0 = 0, 1, 2, 3


@dataclass(frozen=True)
class Tensor:
    name: str
    n: int
    # value scale pieces: list of (count, fan_in).  Most tensors have one
    # piece; the packed ResNet-20 batch-norm tensor has one piece per BN layer.
    pieces: tuple


@dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    description: str
    tensors: tuple
    dist: str            # "normal_fanin" | "laplace_fanin" | "student_t3_bf16" | "normal_const"
    rho_rule: str        # "uniform" | "adaptive"
    rho_uniform: tuple   # (num, den) used when rho_rule == "uniform"
    P: int
    steps: int
    lr: float = 0.1
    const_std: float = 0.02
    extra: dict = field(default_factory=dict)

    @property
    def L(self) -> int:
        return len(self.tensors)

    @property
    def n(self) -> int:
        return int(sum(t.n for t in self.tensors))

    def offsets(self) -> np.ndarray:
        off = np.zeros(self.L + 1, dtype=np.int64)
        off[1:] = np.cumsum([t.n for t in self.tensors])
        return off

    def ratios(self):
        """Per-layer compression ratio rho_l as exact integer pairs (num, den).

        The adaptive rule stands in for the comm/comp-driven ratio of the
        LAGS review (proposed method, second bullet), which gives no formula:
        rho = 1/1000 for tensors of at least 1M entries, 1/100 from 10K up to
        (not including) 1M, and 1 (dense) below 10K.
        """
        num = np.empty(self.L, dtype=np.int64)
        den = np.empty(self.L, dtype=np.int64)
        for i, t in enumerate(self.tensors):
            if self.rho_rule == "uniform":
                a, b = self.rho_uniform
            elif t.n >= 1_000_000:
                a, b = 1, 1000
            elif t.n >= 10_000:
                a, b = 1, 100
            else:
                a, b = 1, 1
            num[i], den[i] = a, b
        return num, den


def _T(name, n, fan_in):
    return Tensor(name, int(n), ((int(n), int(fan_in)),))


# --------------------------------------------------------------------------
# Tensor tables, in parameter-list (forward) order.
# --------------------------------------------------------------------------

def _resnet20_tensors():
    ts = [_T("conv1.w", 16 * 3 * 9, 3 * 9)]
    bn_pieces = [(2 * 16, 3 * 9)]          # bn1 (gamma, beta) owned by conv1
    cin = 16
    for stage, cout in enumerate((16, 32, 64)):
        for blk in range(3):
            for c in range(2):
                ci = cin if c == 0 else cout
                ts.append(_T(f"s{stage}.b{blk}.conv{c}.w", cout * ci * 9, ci * 9))
                bn_pieces.append((2 * cout, ci * 9))
            cin = cout
    ts.append(_T("fc.w", 10 * 64, 64))
    ts.append(_T("fc.b", 10, 64))
    nbn = sum(c for c, _ in bn_pieces)
    ts.append(Tensor("bn.packed", nbn, tuple(bn_pieces)))
    return tuple(ts)


def _vgg16_tensors():
    ts = []
    cin = 3
    for i, cout in enumerate((64, 64, 128, 128, 256, 256, 256,
                              512, 512, 512, 512, 512, 512)):
        ts.append(_T(f"conv{i}.w", cout * cin * 9, cin * 9))
        ts.append(_T(f"conv{i}.b", cout, cin * 9))
        cin = cout
    ts.append(_T("fc0.w", 512 * 512, 512))
    ts.append(_T("fc1.w", 512 * 512, 512))
    ts.append(_T("fc2.w", 10 * 512, 512))
    return tuple(ts)


def _resnet50_tensors():
    ts = []

    def conv_bn(name, cout, cin, kh):
        fan = cin * kh * kh
        ts.append(_T(name + ".w", cout * fan, fan))
        ts.append(_T(name + ".bn.g", cout, fan))
        ts.append(_T(name + ".bn.b", cout, fan))

    conv_bn("conv1", 64, 3, 7)
    cin = 64
    for stage, (width, nblk) in enumerate(((64, 3), (128, 4), (256, 6), (512, 3))):
        for b in range(nblk):
            conv_bn(f"l{stage}.{b}.c1", width, cin, 1)
            conv_bn(f"l{stage}.{b}.c2", width, width, 3)
            conv_bn(f"l{stage}.{b}.c3", 4 * width, width, 1)
            if b == 0:
                conv_bn(f"l{stage}.{b}.down", 4 * width, cin, 1)
            cin = 4 * width
    ts.append(_T("fc.w", 1000 * 2048, 2048))
    ts.append(_T("fc.b", 1000, 2048))
    return tuple(ts)


def _lstm_tensors():
    h, v = 1500, 10000
    return (
        _T("emb.w", v * h, h),
        _T("l0.w", 4 * h * 2 * h, 2 * h),
        _T("l0.b", 4 * h, 2 * h),
        _T("l1.w", 4 * h * 2 * h, 2 * h),
        _T("l1.b", 4 * h, 2 * h),
        _T("dec.w", v * h, h),
        _T("dec.b", v, h),
    )


def _tfm1p3b_tensors():
    d, vocab = 2048, 50304
    ts = [_T("emb.w", vocab * d, d)]
    for b in range(24):
        ts += [
            _T(f"h{b}.ln1.g", d, d), _T(f"h{b}.ln1.b", d, d),
            _T(f"h{b}.qkv.w", 3 * d * d, d),
            _T(f"h{b}.out.w", d * d, d),
            _T(f"h{b}.ln2.g", d, d), _T(f"h{b}.ln2.b", d, d),
            _T(f"h{b}.fc1.w", 4 * d * d, d),
            _T(f"h{b}.fc2.w", d * 4 * d, 4 * d),
        ]
    return tuple(ts)


WORKLOADS = {
    "resnet20": Workload(
        1, "resnet20",
        "ResNet-20-shaped gradient, 269,722 fp32 in 22 tensors (19 convs, fc.w, "
        "fc.b, one packed batch-norm tensor); N(0, 1/fan_in); rho = 1/100; P = 4; "
        "2 steps (a prior step, then the measured one)",
        _resnet20_tensors(), "normal_fanin", "uniform", (1, 100), P=4, steps=2),
    "vgg16": Workload(
        2, "vgg16",
        "VGG-16 (32x32 input) gradient, 15,244,096 fp32 in 29 tensors; "
        "Laplace(0, 1/fan_in); adaptive rho; P = 8; 1 step",
        _vgg16_tensors(), "laplace_fanin", "adaptive", (1, 1), P=8, steps=1),
    "resnet50": Workload(
        3, "resnet50",
        "ResNet-50 gradient, 25,557,032 fp32 in 161 tensors; N(0, 1/fan_in); "
        "adaptive rho; P = 16; 10 steps carrying the residual",
        _resnet50_tensors(), "normal_fanin", "adaptive", (1, 1), P=16, steps=10),
    "lstm": Workload(
        4, "lstm",
        "2-layer LSTM language-model gradient, 66,022,000 fp32 in 7 tensors; "
        "Student-t(3) rounded to bf16 values; rho = 1/1000; P = 16; 1 step",
        _lstm_tensors(), "student_t3_bf16", "uniform", (1, 1000), P=16, steps=1),
    "tfm1p3b": Workload(
        5, "tfm1p3b",
        "1.3B-parameter transformer gradient, 1,311,178,752 fp32 in 193 tensors "
        "(embedding 50304x2048 + 24 blocks of d=2048); N(0, 0.02^2); "
        "rho = 1/1000; P = 16; 1 step",
        _tfm1p3b_tensors(), "normal_const", "uniform", (1, 1000), P=16, steps=1),
    "slgs1p3b": Workload(
        6, "slgs1p3b",
        "the 1.3B transformer gradient selected as one layer (whole-model top-k, "
        "the single-layer SLGS-SGD comparison point of the LAGS review): "
        "1,311,178,752 fp32 in 1 tensor; N(0, 0.02^2); rho = 1/1000; P = 16; 1 step",
        (_T("all", 1_311_178_752, 2048),), "normal_const", "uniform", (1, 1000), P=16, steps=1),
}

ORDER = ("resnet20", "vgg16", "resnet50", "lstm", "tfm1p3b")
EXTRA = ("slgs1p3b",)


def get(name: str) -> Workload:
    return WORKLOADS[name]


# --------------------------------------------------------------------------
# Generators
# --------------------------------------------------------------------------

def rng_for(cfg_id: int, step: int, worker: int, stream: int, layer: int):
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([cfg_id, step, worker, stream, layer])))


def _to_bf16_values(x64: np.ndarray) -> np.ndarray:
    """float64 -> fp32 (round to nearest even) -> bf16 (round to nearest even)
    -> widened back to fp32."""
    f = x64.astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def draw_values(wl: Workload, t: Tensor, rng, count: int | None = None,
                piece_of=None) -> np.ndarray:
    """Draw `count` values (default t.n) from the workload's distribution for
    tensor t.  `piece_of` optionally gives, for each drawn value, the index of
    the scale piece it belongs to (used for message values at chosen
    positions of a multi-piece tensor)."""
    if count is None:
        count = t.n
    if wl.dist == "normal_const":
        return (rng.standard_normal(count) * wl.const_std).astype(np.float32)
    if wl.dist == "student_t3_bf16":
        return _to_bf16_values(rng.standard_t(3, count))
    # per-piece scale from the fan-in
    if piece_of is None:
        scale = np.concatenate([np.full(c, float(f)) for c, f in t.pieces]) \
            if len(t.pieces) > 1 else None
        fan = float(t.pieces[0][1])
    else:
        fans = np.array([float(f) for _, f in t.pieces])
        scale = fans[piece_of]
        fan = None
    if wl.dist == "normal_fanin":
        x = rng.standard_normal(count)
        x = x / np.sqrt(scale) if scale is not None else x / math.sqrt(fan)
    elif wl.dist == "laplace_fanin":
        x = rng.laplace(0.0, 1.0, count)
        x = x / scale if scale is not None else x / fan
    else:
        raise ValueError(wl.dist)
    return x.astype(np.float32)


def _piece_index(t: Tensor, local_idx: np.ndarray) -> np.ndarray:
    bounds = np.cumsum([c for c, _ in t.pieces])
    return np.searchsorted(bounds, local_idx, side="right")


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _fill(n: int, jobs):
    out = np.empty(n, dtype=np.float32)
    def run(j):
        lo, fn = j
        v = fn()
        out[lo:lo + v.size] = v
    if len(jobs) > 1:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(run, jobs))
    else:
        for j in jobs:
            run(j)
    return out


CHUNK = 1 << 24   # tensors above this size are drawn in chunks with their own seeds


def gen_grad_layer(wl: Workload, step: int, worker: int, layer: int) -> np.ndarray:
    t = wl.tensors[layer]
    if t.n <= CHUNK or len(t.pieces) > 1:
        return draw_values(wl, t, rng_for(wl.cfg_id, step, worker, STREAM_GRAD, layer))
    out = np.empty(t.n, dtype=np.float32)

    def run(c):
        lo = c * CHUNK
        cnt = min(CHUNK, t.n - lo)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(
            [wl.cfg_id, step, worker, STREAM_GRAD, layer, c])))
        out[lo:lo + cnt] = draw_values(wl, t, rng, count=cnt)
    nch = (t.n + CHUNK - 1) // CHUNK
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(run, range(nch)))
    return out


def gen_grad(wl: Workload, step: int, worker: int = 0) -> np.ndarray:
    """Gradient of `worker` at `step`: fp32 [n], flat in tensor-table order."""
    off = wl.offsets()
    jobs = [(int(off[l]), (lambda l=l: gen_grad_layer(wl, step, worker, l)))
            for l in range(wl.L)]
    return _fill(wl.n, jobs)


def gen_weights_layer(wl: Workload, layer: int) -> np.ndarray:
    t = wl.tensors[layer]
    if wl.dist == "normal_const" and t.n > CHUNK:
        out = np.empty(t.n, dtype=np.float32)

        def run(c):
            lo = c * CHUNK
            cnt = min(CHUNK, t.n - lo)
            rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(
                [wl.cfg_id, 0, 0, STREAM_W0, layer, c])))
            out[lo:lo + cnt] = (rng.standard_normal(cnt) * wl.const_std).astype(np.float32)
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(run, range((t.n + CHUNK - 1) // CHUNK)))
        return out
    rng = rng_for(wl.cfg_id, 0, 0, STREAM_W0, layer)
    if wl.dist == "normal_const":
        return (rng.standard_normal(t.n) * wl.const_std).astype(np.float32)
    fans = np.concatenate([np.full(c, float(f)) for c, f in t.pieces])
    return (rng.standard_normal(t.n) / np.sqrt(fans)).astype(np.float32)


def gen_weights(wl: Workload) -> np.ndarray:
    """Initial weights w0 ~ N(0, 1/fan_in) (N(0, 0.02^2) for the transformer)."""
    off = wl.offsets()
    jobs = [(int(off[l]), (lambda l=l: gen_weights_layer(wl, l))) for l in range(wl.L)]
    return _fill(wl.n, jobs)


def gen_message_layer(wl: Workload, step: int, worker: int, layer: int, k_l: int):
    """One remote worker's message for one layer: k_l distinct positions drawn
    uniformly from the layer, ascending, as global uint32 indices, with values
    from the workload's distribution."""
    t = wl.tensors[layer]
    off = int(wl.offsets()[layer])
    ri = rng_for(wl.cfg_id, step, worker, STREAM_MSG_IDX, layer)
    rv = rng_for(wl.cfg_id, step, worker, STREAM_MSG_VAL, layer)
    loc = np.sort(ri.choice(t.n, size=int(k_l), replace=False))
    piece = _piece_index(t, loc) if len(t.pieces) > 1 else None
    val = draw_values(wl, t, rv, count=int(k_l), piece_of=piece)
    return (loc + off).astype(np.uint32), val


def gen_messages(wl: Workload, step: int, k, workers=None):
    """Messages of workers 1..P-1 (or the given list) at `step`.

    `k` is the per-layer count of sent entries (length L).  Returns
    (idx uint32 [W, K], val float32 [W, K]) with K = sum(k), laid out per
    worker as the layers in table order, each ascending in index."""
    k = np.asarray(k, dtype=np.int64)
    if workers is None:
        workers = list(range(1, wl.P))
    K = int(k.sum())
    moff = np.zeros(wl.L + 1, dtype=np.int64)
    moff[1:] = np.cumsum(k)
    idx = np.empty((len(workers), K), dtype=np.uint32)
    val = np.empty((len(workers), K), dtype=np.float32)

    def run(job):
        r, p, l = job
        i, v = gen_message_layer(wl, step, p, l, int(k[l]))
        idx[r, moff[l]:moff[l + 1]] = i
        val[r, moff[l]:moff[l + 1]] = v

    jobs = [(r, p, l) for r, p in enumerate(workers) for l in range(wl.L)]
    if len(jobs) > 64:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(run, jobs))
    else:
        for j in jobs:
            run(j)
    return idx, val


# --------------------------------------------------------------------------
# Small synthetic layouts for tests (random tables, adversarial values)
# --------------------------------------------------------------------------

def random_layout(seed: int, L: int, n_max: int, n_min: int = 1):
    """Random layer sizes (int64 offsets, L+1)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([99, seed])))
    sizes = rng.integers(n_min, n_max + 1, size=L)
    off = np.zeros(L + 1, dtype=np.int64)
    off[1:] = np.cumsum(sizes)
    return off


def adversarial_values(seed: int, n: int, kind: str) -> np.ndarray:
    """Value generators with ties, zeros, signed zeros, subnormals and
    infinities, for edge-case tests."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([98, seed])))
    if kind == "normal":
        return rng.standard_normal(n).astype(np.float32)
    if kind == "ties":          # few distinct magnitudes, both signs
        mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0], dtype=np.float32)
        v = mags[rng.integers(0, mags.size, n)]
        return np.where(rng.random(n) < 0.5, -v, v).astype(np.float32)
    if kind == "equal":
        return np.full(n, 0.25, dtype=np.float32)
    if kind == "zeros":         # +0.0 and -0.0 only
        return np.where(rng.random(n) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
    if kind == "special":       # subnormals, infinities, max finite, zeros
        pool = np.array([0.0, -0.0, 1e-45, -1e-45, 1e-40, -3e-39, 1.0, -1.0,
                         np.inf, -np.inf, 3.4028235e38, -3.4028235e38],
                        dtype=np.float32)
        return pool[rng.integers(0, pool.size, n)]
    if kind == "bf16":
        return _to_bf16_values(rng.standard_t(3, n))
    if kind == "int":           # small integers: every fp32 sum stays exact
        return rng.integers(-8, 9, n).astype(np.float32)
    raise ValueError(kind)
