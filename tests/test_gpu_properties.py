"""GPU properties through the C ABI: random layouts against the oracle, and
checkpoint/resume (the library keeps no state between calls apart from the
caller's residual and weights)."""
import zlib

import numpy as np
import pytest

from gpu_helpers import GpuRunner, assert_bits_equal, to_dev, to_np_f32
from layer_wise_top_amd import workloads as W

pytestmark = pytest.mark.gpu

KINDS = ["normal", "ties", "bf16", "zeros", "int", "equal"]


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("seed", list(range(8)))
def test_random_layouts(oracle, seed):
    """Random layer sizes (1 .. 400000), random k in [1, n], a random value
    kind per step, random P: messages, residuals and weights bit-exact, and
    the sparsify again in exact mode from the same residual, also bit-exact."""
    import torch
    rng = np.random.default_rng(zlib.crc32(f"random layout {seed}".encode()))
    L = int(rng.integers(1, 40))
    scale = rng.choice([300, 5000, 60000, 400000])
    sizes = rng.integers(1, scale + 1, size=L)
    off = np.zeros(L + 1, np.int64)
    off[1:] = np.cumsum(sizes)
    n = int(off[-1])
    mode = seed % 3
    if mode == 0:
        k = np.array([int(rng.integers(1, s + 1)) for s in sizes], np.int64)
    else:
        den = 100 if mode == 1 else 1000
        k = oracle.k_for_ratio(sizes, 1, den)
    P = int(rng.integers(1, 6))
    run = GpuRunner(off, k, P)
    K = int(k.sum())
    moff = np.concatenate([[0], np.cumsum(k)])
    r = np.zeros(n, np.float32)
    w = W.adversarial_values(1000 + seed, n, "normal")
    for step in range(2):
        kind = KINDS[int(rng.integers(0, len(KINDS)))]
        _say(f"[random layout {seed}] L={L} n={n} K={K} P={P} step {step} {kind}")
        g = W.adversarial_values(2000 + 10 * seed + step, n, kind)
        oi = np.empty((P - 1, K), np.uint32)
        ov = rng.standard_normal((P - 1, K)).astype(np.float32)
        for p in range(P - 1):
            for l in range(L):
                oi[p, moff[l]:moff[l + 1]] = np.sort(rng.choice(int(sizes[l]), int(k[l]), replace=False)) + off[l]
        g_d, r_d, w_d = to_dev(g), to_dev(r), to_dev(w)
        run.sparsify(g_d, r_d)
        if P > 1:
            run.set_others(oi, ov)
        run.aggregate(w_d, 0.05)
        torch.cuda.synchronize()
        mi_o, mv_o, r_o = oracle.sparsify(off, k, g, r)
        mi_g, mv_g = run.message()
        assert_bits_equal("msg_idx", mi_g, mi_o)
        assert_bits_equal("msg_val", mv_g, mv_o)
        assert_bits_equal("residual", to_np_f32(r_d), r_o)
        # exact mode from the same residual: the same bits
        from layer_wise_top_amd import lags
        r2 = to_dev(r)
        mi2 = torch.empty(max(K, 1), dtype=torch.int32, device="cuda")
        mv2 = torch.empty(max(K, 1), dtype=torch.float32, device="cuda")
        lags.lags_sparsify_layers(run.layout, g_d, r2, mi2[:K], mv2[:K], run.ws, lags.LAGS_SPARSIFY_EXACT)
        torch.cuda.synchronize()
        assert_bits_equal("exact-mode msg_idx", mi2[:K].cpu().numpy().view(np.uint32), mi_o)
        assert_bits_equal("exact-mode msg_val", to_np_f32(mv2[:K]), mv_o)
        assert_bits_equal("exact-mode residual", to_np_f32(r2), r_o)
        ai = np.concatenate([mi_o[None], oi], 0) if P > 1 else mi_o[None]
        av = np.concatenate([mv_o[None], ov], 0) if P > 1 else mv_o[None]
        w_o = oracle.aggregate(ai, av, w, 0.05)
        assert_bits_equal("weights", to_np_f32(w_d), w_o)
        r, w = r_o, w_o


SPECIAL_SIZES = [1, 2, 3, 4, 5, 63, 64, 65, 4095, 4096, 4097, 16383, 16384, 16385, 37888, 65537]


def _stratified_others(rng, off, k, P, collide):
    """Messages of workers 1..P-1: one index drawn in each of k_l equal strata
    of every layer (sorted and distinct); with `collide`, about half of the
    workers share one draw, so many indices carry several workers."""
    L, K = len(k), int(k.sum())
    moff = np.concatenate([[0], np.cumsum(k)])
    oi = np.empty((P - 1, K), np.uint32)
    for l in range(L):
        n_l, k_l = int(off[l + 1] - off[l]), int(k[l])
        lo = (np.arange(k_l, dtype=np.int64) * n_l) // k_l
        hi = (np.arange(1, k_l + 1, dtype=np.int64) * n_l) // k_l
        shared = lo + (rng.random(k_l) * (hi - lo)).astype(np.int64)
        for p in range(P - 1):
            own = shared if (collide and rng.random() < 0.5) else lo + (rng.random(k_l) * (hi - lo)).astype(np.int64)
            oi[p, moff[l]:moff[l + 1]] = own + off[l]
    return oi, rng.standard_normal((P - 1, K)).astype(np.float32)


@pytest.mark.parametrize("seed", list(range(12)))
def test_random_layouts_with_ranges(oracle, seed):
    """Random layouts (1 .. 30 layers, sizes log-uniform up to 1M entries or
    boundary sizes, k random, within 2 of n, or from a ratio), P up to 40
    with indices shared between workers, two steps, each issued as one call or
    as a random cut into layer ranges in random order: messages, residuals
    and weights bit-exact against the oracle, and exact mode from the same
    residual too."""
    import torch
    from layer_wise_top_amd import lags
    rng = np.random.default_rng(zlib.crc32(f"ranges layout {seed}".encode()))
    L = int(rng.integers(1, 31))
    sizes = np.array([int(rng.choice(SPECIAL_SIZES)) if rng.random() < 0.3
                      else int(np.exp(rng.uniform(0, np.log(1_000_000)))) + 1 for _ in range(L)], np.int64)
    off = np.zeros(L + 1, np.int64)
    off[1:] = np.cumsum(sizes)
    n = int(off[-1])
    mode = seed % 3
    if mode == 0:
        k = np.array([int(rng.integers(1, s + 1)) for s in sizes], np.int64)
    elif mode == 1:
        k = np.array([max(1, int(s) - int(rng.integers(0, 3))) for s in sizes], np.int64)
    else:
        k = oracle.k_for_ratio(sizes, 1, int(rng.choice([3, 100, 1000])))
    P = int(rng.choice([1, 2, 3, 8, 16, 33, 40]))
    collide = bool(seed % 2)
    K = int(k.sum())
    run = GpuRunner(off, k, P)
    r = np.zeros(n, np.float32)
    w = W.adversarial_values(3000 + seed, n, "normal")
    for step in range(2):
        kind = KINDS[int(rng.integers(0, len(KINDS)))]
        ranged = (step + seed) % 2 == 1 and L > 1
        _say(f"[ranges layout {seed}] L={L} n={n} K={K} P={P} step {step} {kind} ranges={ranged}")
        g = W.adversarial_values(4000 + 10 * seed + step, n, kind)
        g_d, r_d, w_d = to_dev(g), to_dev(r), to_dev(w)
        if P > 1:
            oi, ov = _stratified_others(rng, off, k, P, collide)
            run.set_others(oi, ov)
        if ranged:
            cuts = sorted(set([0, L] + [int(c) for c in rng.integers(1, L, size=int(rng.integers(1, min(L, 6))))]))
            parts = [(cuts[i], cuts[i + 1]) for i in range(len(cuts) - 1)]
            for j in rng.permutation(len(parts)):
                l0, l1 = parts[j]
                lags.lags_sparsify_range(run.layout, l0, l1, g_d, r_d, run.msg_idx[0], run.msg_val[0], run.ws)
                lags.lags_aggregate_range(run.layout, l0, l1, w_d, run.msg_idx, run.msg_val, P, 0.05, run.ws)
        else:
            run.sparsify(g_d, r_d)
            run.aggregate(w_d, 0.05)
        torch.cuda.synchronize()
        assert run.report()["bad_entries"] == 0
        mi_o, mv_o, r_o = oracle.sparsify(off, k, g, r)
        mi_g, mv_g = run.message()
        assert_bits_equal("msg_idx", mi_g, mi_o)
        assert_bits_equal("msg_val", mv_g, mv_o)
        assert_bits_equal("residual", to_np_f32(r_d), r_o)
        ai = np.concatenate([mi_o[None], oi], 0) if P > 1 else mi_o[None]
        av = np.concatenate([mv_o[None], ov], 0) if P > 1 else mv_o[None]
        w_o = oracle.aggregate(ai, av, w, 0.05)
        assert_bits_equal("weights", to_np_f32(w_d), w_o)
        r2 = to_dev(r)
        mi2 = torch.empty(K, dtype=torch.int32, device="cuda")
        mv2 = torch.empty(K, dtype=torch.float32, device="cuda")
        lags.lags_sparsify_layers(run.layout, g_d, r2, mi2, mv2, run.ws, lags.LAGS_SPARSIFY_EXACT)
        torch.cuda.synchronize()
        assert_bits_equal("exact-mode msg_idx", mi2.cpu().numpy().view(np.uint32), mi_o)
        assert_bits_equal("exact-mode msg_val", to_np_f32(mv2), mv_o)
        assert_bits_equal("exact-mode residual", to_np_f32(r2), r_o)
        r, w = r_o, w_o


def test_resume_equals_continuous_run():
    """ResNet-50: ten steps in one go equal five steps, a save of (weights,
    residual) to the host, a fresh layout and workspace, and five more steps
    — bit for bit."""
    import torch
    from layer_wise_top_amd import lags
    wl = W.get("resnet50")
    off = wl.offsets()
    num, den = wl.ratios()
    k = lags.k_table(off, num, den)
    P = wl.P
    grads = [to_dev(W.gen_grad(wl, s)) for s in range(10)]
    msgs = [W.gen_messages(wl, s, k) for s in range(10)]
    w0 = W.gen_weights(wl)

    def run_steps(run, r_d, w_d, steps):
        for s in steps:
            run.set_others(*msgs[s])
            run.sparsify(grads[s], r_d)
            run.aggregate(w_d, wl.lr)
        torch.cuda.synchronize()

    a = GpuRunner(off, k, P)
    r_a = torch.zeros(wl.n, dtype=torch.float32, device="cuda")
    w_a = to_dev(w0)
    run_steps(a, r_a, w_a, range(10))

    b = GpuRunner(off, k, P)
    r_b = torch.zeros(wl.n, dtype=torch.float32, device="cuda")
    w_b = to_dev(w0)
    run_steps(b, r_b, w_b, range(5))
    saved = (to_np_f32(r_b).copy(), to_np_f32(w_b).copy())
    del b
    c = GpuRunner(off, k, P)
    r_c, w_c = to_dev(saved[0]), to_dev(saved[1])
    run_steps(c, r_c, w_c, range(5, 10))
    assert_bits_equal("residual", to_np_f32(r_c), to_np_f32(r_a))
    assert_bits_equal("weights", to_np_f32(w_c), to_np_f32(w_a))
    mi_a, mv_a = a.message()
    mi_c, mv_c = c.message()
    assert_bits_equal("last message idx", mi_c, mi_a)
    assert_bits_equal("last message val", mv_c, mv_a)


def test_graph_capture_replays_match_eager():
    """After a first call has built the device tables, a step makes no
    allocation and no synchronisation, so it can be captured into a HIP graph.
    Each of three replays, with eager work and synchronisations between them,
    must equal the eager step from the same state."""
    import torch
    from layer_wise_top_amd import lags
    wl = W.get("vgg16")
    off = wl.offsets()
    num, den = wl.ratios()
    k = lags.k_table(off, num, den)
    P = wl.P
    run = GpuRunner(off, k, P)
    run.set_others(*W.gen_messages(wl, 0, k))
    g = to_dev(W.gen_grad(wl, 0))
    w0 = to_dev(W.gen_weights(wl))
    r = torch.zeros(wl.n, dtype=torch.float32, device="cuda")
    w = w0.clone()
    s = torch.cuda.Stream()

    def step():
        lags.lags_sparsify_layers(run.layout, g, r, run.msg_idx[0], run.msg_val[0], run.ws, 0, s)
        lags.lags_aggregate_apply(run.layout, w, run.msg_idx, run.msg_val, P, wl.lr, run.ws, s)

    with torch.cuda.stream(s):
        step()                                  # builds the device tables
    torch.cuda.synchronize()
    r_start, w_start = r.clone(), w.clone()
    torch.cuda.synchronize()                    # the copies are done before s starts
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    want = [to_np_f32(r).copy(), to_np_f32(w).copy(), run.message()]
    graph = torch.cuda.CUDAGraph()
    r.copy_(r_start)
    w.copy_(w_start)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=s):
        step()
    for rep in range(3):
        r.copy_(r_start)
        w.copy_(w_start)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _say(f"[graph] replay {rep}")
        assert_bits_equal("residual", to_np_f32(r), want[0])
        assert_bits_equal("weights", to_np_f32(w), want[1])
        mi, mv = run.message()
        assert_bits_equal("msg_idx", mi, want[2][0])
        assert_bits_equal("msg_val", mv, want[2][1])
        float(torch.ones(1000, device="cuda").sum())   # eager work between replays
