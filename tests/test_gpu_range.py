"""GPU parity of the layer-range calls (lags_sparsify_range,
lags_aggregate_range) through the C ABI.

Layer-wise pipelining produces and applies messages layer range by layer
range, last layers first (the order back-propagation releases them).  Cutting
[0, L) into ranges and calling them in that order must give the oracle's
results bit for bit, as must two disjoint halves launched on two streams with
one shared workspace.
"""
import numpy as np
import pytest

from gpu_helpers import GpuRunner, assert_bits_equal, to_dev, to_np_f32
from layer_wise_top_amd import workloads as W
from oracle import ratio_oracle

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _cuts(rng, L, nranges):
    inner = np.sort(rng.choice(np.arange(1, L), size=min(nranges - 1, L - 1), replace=False))
    return [0] + [int(x) for x in inner] + [L]


def _random_others(rng, off, k, P, K):
    oi = np.empty((P - 1, K), np.uint32)
    ov = np.empty((P - 1, K), np.float32)
    moff = np.concatenate([[0], np.cumsum(k)])
    for p in range(P - 1):
        for l in range(len(k)):
            n_l = int(off[l + 1] - off[l])
            loc = np.sort(rng.choice(n_l, int(k[l]), replace=False))
            oi[p, moff[l]:moff[l + 1]] = loc + off[l]
        ov[p] = rng.standard_normal(K).astype(np.float32)
    return oi, ov


def _expect(oracle, off, k, g, r, w, oi, ov, lr):
    mi_o, mv_o, r_o = oracle.sparsify(off, k, g, r)
    ai = np.concatenate([mi_o[None], oi], 0)
    av = np.concatenate([mv_o[None], ov], 0)
    return mi_o, mv_o, r_o, oracle.aggregate(ai, av, w, lr)


def _compare(tag, run, r_d, w_d, want):
    mi_g, mv_g = run.message()
    assert_bits_equal(f"{tag} msg_idx", mi_g, want[0])
    assert_bits_equal(f"{tag} msg_val", mv_g, want[1])
    assert_bits_equal(f"{tag} residual", to_np_f32(r_d), want[2])
    assert_bits_equal(f"{tag} weights", to_np_f32(w_d), want[3])


def test_ranges_backward_order_resnet50(oracle):
    """ResNet-50's 161 tensors cut into 12 random ranges, each sparsified and
    then aggregated, last range first; two steps so the residual carries."""
    import torch
    from layer_wise_top_amd import lags
    wl = W.get("resnet50")
    off = wl.offsets()
    num, den = wl.ratios()
    k = oracle.k_for_ratio(np.diff(off), num, den)
    P = wl.P
    run = GpuRunner(off, k, P)
    lay = run.layout
    rng = np.random.default_rng(2024)
    r = np.zeros(wl.n, np.float32)
    w = W.gen_weights(wl)
    r_d, w_d = to_dev(r), to_dev(w)
    for step in range(2):
        cuts = _cuts(rng, wl.L, 12)
        _say(f"[resnet50 ranges] step {step}: {len(cuts) - 1} ranges")
        g = W.gen_grad(wl, step)
        oi, ov = W.gen_messages(wl, step, k)
        run.set_others(oi, ov)
        g_d = to_dev(g)
        for i in reversed(range(len(cuts) - 1)):
            l0, l1 = cuts[i], cuts[i + 1]
            lags.lags_sparsify_range(lay, l0, l1, g_d, r_d, run.msg_idx[0], run.msg_val[0], run.ws)
            lags.lags_aggregate_range(lay, l0, l1, w_d, run.msg_idx, run.msg_val, P, wl.lr, run.ws)
        torch.cuda.synchronize()
        want = _expect(oracle, off, k, g, r, w, oi, ov, wl.lr)
        _compare(f"resnet50 ranges step {step}", run, r_d, w_d, want)
        r, w = want[2], want[3]


@pytest.mark.parametrize("flags", [0, 1], ids=["sampled", "exact"])
def test_single_layer_ranges_mixed_layout(oracle, flags):
    """Every layer on its own, in reverse order, on a layout that has small,
    dense, full-sample and sampled layers (several finishing workgroups)."""
    import torch
    from layer_wise_top_amd import lags
    sizes = [700, 20000, 5000, 300000, 4096, 16385, 1, 1200000, 33, 90001]
    off = np.zeros(len(sizes) + 1, np.int64)
    off[1:] = np.cumsum(sizes)
    k = oracle.k_for_ratio(np.diff(off), 1, 100)
    k[1] = sizes[1]                           # a dense layer
    n, K, P = int(off[-1]), int(k.sum()), 3
    run = GpuRunner(off, k, P)
    rng = np.random.default_rng(7)
    g = rng.standard_normal(n).astype(np.float32)
    r = (0.1 * rng.standard_normal(n)).astype(np.float32)
    w = rng.standard_normal(n).astype(np.float32)
    oi, ov = _random_others(rng, off, k, P, K)
    run.set_others(oi, ov)
    g_d, r_d, w_d = to_dev(g), to_dev(r), to_dev(w)
    for l in reversed(range(len(sizes))):
        lags.lags_sparsify_range(run.layout, l, l + 1, g_d, r_d, run.msg_idx[0], run.msg_val[0],
                                 run.ws, flags)
    for l in range(len(sizes)):
        lags.lags_aggregate_range(run.layout, l, l + 1, w_d, run.msg_idx, run.msg_val, P, 0.05,
                                  run.ws)
    torch.cuda.synchronize()
    _compare("single-layer ranges", run, r_d, w_d, _expect(oracle, off, k, g, r, w, oi, ov, 0.05))


def test_disjoint_ranges_on_two_streams(oracle):
    """Two halves of the layout at once on two streams, one workspace."""
    import torch
    from layer_wise_top_amd import lags
    sizes = [97] * 200 + [5000] * 10 + [250000, 700000, 4100, 1500000, 60000]
    off = np.zeros(len(sizes) + 1, np.int64)
    off[1:] = np.cumsum(sizes)
    L = len(sizes)
    k = oracle.k_for_ratio(np.diff(off), 1, 200)
    n, K, P = int(off[-1]), int(k.sum()), 4
    run = GpuRunner(off, k, P)
    rng = np.random.default_rng(11)
    g = rng.standard_normal(n).astype(np.float32)
    r = (0.1 * rng.standard_normal(n)).astype(np.float32)
    w = rng.standard_normal(n).astype(np.float32)
    oi, ov = _random_others(rng, off, k, P, K)
    run.set_others(oi, ov)
    g_d, r_d, w_d = to_dev(g), to_dev(r), to_dev(w)
    main = torch.cuda.current_stream()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(main)
    s2.wait_stream(main)
    half = L - 3                               # the three largest tensors against the rest
    for s, (l0, l1) in ((s1, (0, half)), (s2, (half, L))):
        with torch.cuda.stream(s):
            lags.lags_sparsify_range(run.layout, l0, l1, g_d, r_d, run.msg_idx[0], run.msg_val[0],
                                     run.ws, 0, stream=s)
            lags.lags_aggregate_range(run.layout, l0, l1, w_d, run.msg_idx, run.msg_val, P, 0.1,
                                      run.ws, stream=s)
    main.wait_stream(s1)
    main.wait_stream(s2)
    torch.cuda.synchronize()
    _compare("two streams", run, r_d, w_d, _expect(oracle, off, k, g, r, w, oi, ov, 0.1))


def test_adaptive_sizes_then_pipelined_ranges(oracle):
    """VGG-16 with per-layer sizes from lags_adaptive_k (backward time
    proportional to tensor size, synthetic) and the step issued per range of
    the merged-message schedule, last range first: the oracle's results."""
    import torch
    from layer_wise_top_amd import lags
    wl = W.get("vgg16")
    off = wl.offsets()
    c = np.diff(off) * 66e-12
    k = lags.lags_adaptive_k(off, c, wl.P, 20e-6, 1.0 / 50e9, (1, 1000))
    assert k.tolist() == ratio_oracle.adaptive_k(np.diff(off).tolist(), c.tolist(), wl.P, 20e-6,
                                                 1.0 / 50e9, 1, 1000)
    runs, _ = lags.lags_merge_schedule(c, 8 * (wl.P - 1) * k, 20e-6, 1.0 / 50e9)
    _say(f"[vgg16 adaptive] K={int(k.sum())} runs={len(runs)}")
    P = wl.P
    run = GpuRunner(off, k, P)
    g = W.gen_grad(wl, 0)
    w = W.gen_weights(wl)
    r = np.zeros(wl.n, np.float32)
    oi, ov = W.gen_messages(wl, 0, k)
    run.set_others(oi, ov)
    g_d, r_d, w_d = to_dev(g), to_dev(r), to_dev(w)
    for l0, l1 in runs:
        lags.lags_sparsify_range(run.layout, l0, l1, g_d, r_d, run.msg_idx[0], run.msg_val[0], run.ws)
        lags.lags_aggregate_range(run.layout, l0, l1, w_d, run.msg_idx, run.msg_val, P, wl.lr, run.ws)
    torch.cuda.synchronize()
    _compare("vgg16 adaptive", run, r_d, w_d, _expect(oracle, off, k, g, r, w, oi, ov, wl.lr))
