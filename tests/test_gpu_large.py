"""Full-size parity on the 1.3B-parameter transformer gradient (the benchmark's
workload, in the benchmark's launch configuration), layer-wise and as one
whole-model layer.

The oracle recomputes a sample of layers one by one (every layer's selection
depends only on that layer): the 103M-entry embedding, all eight tensors of
block 0, a middle qkv matrix and the last fc2.  Messages, residuals and
weights of those layers must match bit for bit.  Over all 193 layers the GPU
output is checked for the invariants that fix the selection (sizes, order,
range, residual bits, threshold order, tie prefix), and untouched weights
must keep their bits over the whole buffer.  A 2.3B-entry layout checks the
same beyond 2^31 entries (indices that only fit uint32).
"""
import numpy as np
import pytest

from gpu_helpers import GpuRunner, assert_bits_equal, bits, to_dev, to_np_f32, to_np_u32
from layer_wise_top_amd import workloads as W

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _exact_mode_agrees(run, g_d, r_d, sampled, tag):
    """Sparsify the same gradient again in exact mode (the multi-workgroup
    radix select; it shares no selection step with the sampled path) from a
    zero residual: messages and residual must equal the sampled path's bits."""
    import torch
    from layer_wise_top_amd import lags
    _say(f"{tag}: exact mode")
    K = run.layout.K
    r2 = torch.zeros_like(r_d)
    mi2 = torch.empty(K, dtype=torch.int32, device="cuda")
    mv2 = torch.empty(K, dtype=torch.float32, device="cuda")
    lags.lags_sparsify_layers(run.layout, g_d, r2, mi2, mv2, run.ws, lags.LAGS_SPARSIFY_EXACT)
    torch.cuda.synchronize()
    rep = run.report()
    assert rep["layers_exact"] == sampled and rep["bad_entries"] == 0, rep
    assert bool(torch.equal(mi2, run.msg_idx[0, :K])), f"{tag}: exact-mode msg_idx differs"
    assert bool(torch.equal(mv2.view(torch.int32), run.msg_val[0, :K].view(torch.int32))), \
        f"{tag}: exact-mode msg_val differs"
    assert bool(torch.equal(r2.view(torch.int32), r_d.view(torch.int32))), f"{tag}: exact-mode residual differs"
    del r2, mi2, mv2


@pytest.mark.timeout(1200)
def test_tfm1p3b_full_size(oracle):
    import torch
    wl = W.get("tfm1p3b")
    off = wl.offsets()
    num, den = wl.ratios()
    k = oracle.k_for_ratio(np.diff(off), num, den)
    moff = np.concatenate([[0], np.cumsum(k)])
    P = wl.P
    _say("generating inputs")
    g = W.gen_grad(wl, 0)
    w0 = W.gen_weights(wl)
    oi, ov = W.gen_messages(wl, 0, k)
    run = GpuRunner(off, k, P)
    g_d = to_dev(g)
    r_d = torch.zeros(wl.n, dtype=torch.float32, device="cuda")
    w_d = to_dev(w0)
    w0_d = w_d.clone()
    run.set_others(oi, ov)
    _say("running one step")
    run.sparsify(g_d, r_d)
    run.aggregate(w_d, wl.lr)
    torch.cuda.synchronize()
    rep = run.report()
    assert rep["layers_exact"] == 0 and rep["bad_entries"] == 0, rep

    # ---- invariants over every layer, on the device
    _say("invariants over all layers")
    mi = run.msg_idx[0, :run.layout.K].long() & 0xFFFFFFFF
    key_g = g_d.view(torch.int32) & 0x7FFFFFFF
    sent = torch.zeros(wl.n, dtype=torch.bool, device="cuda")
    sent[mi] = True
    assert int(sent.sum()) == run.layout.K
    r_bits = r_d.view(torch.int32)
    assert bool((r_bits[sent] == 0).all())
    assert bool((r_bits[~sent] == g_d.view(torch.int32)[~sent]).all())
    assert bool((run.msg_val[0, :run.layout.K].view(torch.int32) == g_d.view(torch.int32)[mi]).all())
    for l in range(wl.L):
        a, b = int(off[l]), int(off[l + 1])
        seg = mi[moff[l]:moff[l + 1]]
        assert bool((seg >= a).all()) and bool((seg < b).all())
        assert bool((seg[1:] > seg[:-1]).all())
        ks = key_g[a:b]
        s_l = sent[a:b]
        T = int(ks[s_l].min())
        assert int(ks[~s_l].max()) <= T
        tied_sent = torch.nonzero(s_l & (ks == T)).flatten()
        tied_unsent = torch.nonzero(~s_l & (ks == T)).flatten()
        if tied_unsent.numel():
            assert int(tied_sent.max()) < int(tied_unsent.min())

    del sent, key_g
    _exact_mode_agrees(run, g_d, r_d, rep["layers_sampled"], "tfm1p3b")

    # ---- untouched weights keep their bits (whole buffer)
    touched = torch.zeros(wl.n, dtype=torch.bool, device="cuda")
    touched[run.msg_idx.reshape(-1).long() & 0xFFFFFFFF] = True
    assert bool((w_d.view(torch.int32)[~touched] == w0_d.view(torch.int32)[~touched]).all())

    # ---- sampled layers against the oracle
    mi_h = to_np_u32(run.msg_idx[0, :run.layout.K])
    mv_h = to_np_f32(run.msg_val[0, :run.layout.K])
    r_h = to_np_f32(r_d)
    w_h = to_np_f32(w_d)
    blocks = [0] + list(range(1, 9)) + [1 + 8 * 12 + 2, wl.L - 1]   # emb, block 0, a qkv, last fc2
    for l in blocks:
        a, b = int(off[l]), int(off[l + 1])
        _say(f"oracle layer {l} ({wl.tensors[l].name}, {b - a} entries)")
        mi_o, mv_o, r_o = oracle.sparsify([0, b - a], [int(k[l])], g[a:b], np.zeros(b - a, np.float32))
        assert_bits_equal(f"layer {l} msg_idx", mi_h[moff[l]:moff[l + 1]], mi_o.astype(np.uint32) + a)
        assert_bits_equal(f"layer {l} msg_val", mv_h[moff[l]:moff[l + 1]], mv_o)
        assert_bits_equal(f"layer {l} residual", r_h[a:b], r_o)
        # aggregate restricted to this layer's index range: worker 0 from the
        # oracle's message, the others from the generated inputs
        ai = np.concatenate([np.zeros((1, run.layout.K), np.uint32), oi], 0)
        av = np.concatenate([np.zeros((1, run.layout.K), np.float32), ov], 0)
        ai[0, moff[l]:moff[l + 1]] = mi_o.astype(np.uint32) + a
        av[0, moff[l]:moff[l + 1]] = mv_o
        ai[0, :moff[l]] = 0xFFFFFFFF
        ai[0, moff[l + 1]:] = 0xFFFFFFFF
        w_o = oracle.aggregate(ai, av, w0[a:b], wl.lr, lo=a, hi=b)
        assert_bits_equal(f"layer {l} weights", w_h[a:b], w_o)

    # ---- the aggregate of every layer against the oracle: worker 0's
    # message is the GPU's own, which the invariants above pin on every layer
    # (the selected set is unique and its values are acc's bits)
    _say("oracle aggregate over all layers")
    ai = np.concatenate([mi_h[None], oi], 0)
    av = np.concatenate([mv_h[None], ov], 0)
    w_o = oracle.aggregate(ai, av, w0, wl.lr)
    assert_bits_equal("weights of all layers", w_h, w_o)


@pytest.mark.timeout(1200)
def test_slgs1p3b_full_size(oracle):
    """Whole-model selection (SLGS-SGD): the same 1.31B entries as one layer.
    The oracle's sort cannot take 1.31B keys in a test, so the expected
    selection comes from its definition evaluated on the host with a library
    partition (the k-th largest key, then the lowest-index ties): the GPU must
    send exactly that set, with the residual and value bits it implies, and
    its weights must match the oracle's aggregate on three windows of one
    million indices and over every index (worker 0's message taken from the
    host selection)."""
    import torch
    wl = W.get("slgs1p3b")
    off = wl.offsets()
    num, den = wl.ratios()
    k = oracle.k_for_ratio(np.diff(off), num, den)
    P = wl.P
    K = int(k[0])
    _say("generating inputs")
    g = W.gen_grad(wl, 0)
    w0 = W.gen_weights(wl)
    oi, ov = W.gen_messages(wl, 0, k)
    run = GpuRunner(off, k, P)
    g_d = to_dev(g)
    r_d = torch.zeros(wl.n, dtype=torch.float32, device="cuda")
    w_d = to_dev(w0)
    w0_d = w_d.clone()
    run.set_others(oi, ov)
    _say("running one step")
    run.sparsify(g_d, r_d)
    run.aggregate(w_d, wl.lr)
    torch.cuda.synchronize()
    rep = run.report()
    assert rep["layers_exact"] == 0 and rep["bad_entries"] == 0, rep
    _exact_mode_agrees(run, g_d, r_d, rep["layers_sampled"], "slgs1p3b")

    _say("host selection (acc = grad: the residual starts at zero)")
    key_h = g.view(np.int32) & np.int32(0x7FFFFFFF)
    T = int(np.partition(key_h, wl.n - K)[wl.n - K])       # the K-th largest key
    above = np.flatnonzero(key_h > T)
    tied = np.flatnonzero(key_h == T)
    e = K - above.size
    assert 1 <= e <= tied.size
    sel = np.sort(np.concatenate([above, tied[:e]])).astype(np.uint32)
    del key_h, above, tied

    _say("message, residual and untouched weights")
    assert_bits_equal("msg_idx", to_np_u32(run.msg_idx[0, :K]), sel)
    assert_bits_equal("msg_val", to_np_f32(run.msg_val[0, :K]), g[sel])
    sel_d = to_dev(sel).long() & 0xFFFFFFFF
    sent = torch.zeros(wl.n, dtype=torch.bool, device="cuda")
    sent[sel_d] = True
    rb = r_d.view(torch.int32)
    assert bool((rb[sent] == 0).all()) and bool((rb[~sent] == g_d.view(torch.int32)[~sent]).all())
    del sent, sel_d
    touched = torch.zeros(wl.n, dtype=torch.bool, device="cuda")
    touched[run.msg_idx.reshape(-1).long() & 0xFFFFFFFF] = True
    assert bool((w_d.view(torch.int32)[~touched] == w0_d.view(torch.int32)[~touched]).all())
    del touched

    _say("aggregate windows against the oracle")
    ai = np.full((P, K), 0xFFFFFFFF, np.uint32)
    av = np.zeros((P, K), np.float32)
    ai[0] = sel
    av[0] = g[sel]
    ai[1:] = oi
    av[1:] = ov
    for a in (0, wl.n // 2, wl.n - 1_000_000):
        b = a + 1_000_000
        wi = np.where((ai >= a) & (ai < b), ai, np.uint32(0xFFFFFFFF))
        w_o = oracle.aggregate(wi, av, w0[a:b], wl.lr, lo=a, hi=b)
        assert_bits_equal(f"weights [{a}, {b})", to_np_f32(w_d[a:b]), w_o)
    _say("oracle aggregate over every index")
    w_o = oracle.aggregate(ai, av, w0, wl.lr)
    assert_bits_equal("weights of every index", to_np_f32(w_d), w_o)


@pytest.mark.timeout(1200)
def test_layout_beyond_2_31_entries(oracle):
    """A 2.3B-entry layout (rho = 1/1000, P = 2): two 1.1B-entry layers, then
    four layers whose every index lies above 2^31 (the uint32 index range the
    boundary allows, beyond int32).  The four are recomputed by the oracle
    (messages, residual and, restricted to each layer, weights, bit for
    bit); every layer meets the selection's invariants; exact mode agrees bit
    for bit.  Inputs: seeded normal draws on the device (gradient, weights)
    and seeded stratified messages for the other worker."""
    import torch
    sizes = [1_100_000_003, 1_100_000_001, 20_000_001, 3, 30_000_000, 49_999_999]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    n, L = int(off[-1]), len(sizes)
    assert off[2] > 2 ** 31 and n < 2 ** 32 - 1
    k = oracle.k_for_ratio(np.diff(off), 1, 1000)
    moff = np.concatenate([[0], np.cumsum(k)])
    K, P = int(k.sum()), 2
    _say(f"[2^31] n={n:,} K={K:,}: inputs on the device")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2311)
    g_d = torch.randn(n, generator=gen, device="cuda")
    w_d = torch.randn(n, generator=gen, device="cuda")
    r_d = torch.zeros(n, dtype=torch.float32, device="cuda")
    rng = np.random.default_rng(2312)
    parts = []
    for l in range(L):
        n_l, k_l = int(sizes[l]), int(k[l])
        lo = (np.arange(k_l, dtype=np.int64) * n_l) // k_l
        hi = (np.arange(1, k_l + 1, dtype=np.int64) * n_l) // k_l
        parts.append(off[l] + lo + (rng.random(k_l) * (hi - lo)).astype(np.int64))
    oi = np.concatenate(parts).astype(np.uint32)[None]
    ov = rng.standard_normal((1, K)).astype(np.float32)
    a2 = int(off[2])
    g_tail = to_np_f32(g_d[a2:])
    w_tail = to_np_f32(w_d[a2:])
    w0_d = w_d.clone()
    run = GpuRunner(off, k, P)
    run.set_others(oi, ov)
    _say("[2^31] one step")
    run.sparsify(g_d, r_d)
    run.aggregate(w_d, 0.1)
    torch.cuda.synchronize()
    rep = run.report()
    assert rep["layers_exact"] == 0 and rep["bad_entries"] == 0, rep

    _say("[2^31] invariants over all layers")
    # every masked check is per layer: torch's boolean indexing fails beyond
    # 2^31 elements
    mi = run.msg_idx[0, :K].long() & 0xFFFFFFFF
    sent = torch.zeros(n, dtype=torch.bool, device="cuda")
    sent[mi] = True
    assert int(sent.sum()) == K
    touched = sent.clone()
    touched[torch.from_numpy(oi[0].astype(np.int64)).cuda()] = True
    g_bits, r_bits, w_bits, w0_bits = (t.view(torch.int32) for t in (g_d, r_d, w_d, w0_d))
    mv_bits = run.msg_val[0, :K].view(torch.int32)
    for l in range(L):
        a, b = int(off[l]), int(off[l + 1])
        seg = mi[moff[l]:moff[l + 1]]
        assert bool((seg >= a).all()) and bool((seg < b).all())
        assert bool((seg[1:] > seg[:-1]).all())
        assert bool((mv_bits[moff[l]:moff[l + 1]] == g_bits[seg]).all())
        s_l, gb, rb = sent[a:b], g_bits[a:b], r_bits[a:b]
        assert bool((rb[s_l] == 0).all())
        assert bool((rb[~s_l] == gb[~s_l]).all())
        ks = gb & 0x7FFFFFFF
        T = int(ks[s_l].min())
        if not bool(s_l.all()):
            assert int(ks[~s_l].max()) <= T
            tied_unsent = torch.nonzero(~s_l & (ks == T)).flatten()
            if tied_unsent.numel():
                assert int(torch.nonzero(s_l & (ks == T)).flatten().max()) < int(tied_unsent.min())
        u_l = ~touched[a:b]
        assert bool((w_bits[a:b][u_l] == w0_bits[a:b][u_l]).all())
        del s_l, gb, rb, ks, u_l
    del sent, touched, g_bits, r_bits, w_bits, w0_bits, w0_d

    mi_h = to_np_u32(run.msg_idx[0, :K])
    mv_h = to_np_f32(run.msg_val[0, :K])
    for l in range(2, L):
        a, b = int(off[l]), int(off[l + 1])
        _say(f"[2^31] oracle layer {l} ([{a:,}, {b:,}))")
        ga = g_tail[a - a2:b - a2]
        mi_o, mv_o, r_o = oracle.sparsify([0, b - a], [int(k[l])], ga, np.zeros(b - a, np.float32))
        assert_bits_equal(f"layer {l} msg_idx", mi_h[moff[l]:moff[l + 1]], mi_o.astype(np.uint32) + np.uint32(a))
        assert_bits_equal(f"layer {l} msg_val", mv_h[moff[l]:moff[l + 1]], mv_o)
        assert_bits_equal(f"layer {l} residual", to_np_f32(r_d[a:b]), r_o)
        ai = np.full((P, K), 0xFFFFFFFF, np.uint32)
        av = np.zeros((P, K), np.float32)
        ai[0, moff[l]:moff[l + 1]] = mi_o.astype(np.uint32) + np.uint32(a)
        av[0, moff[l]:moff[l + 1]] = mv_o
        ai[1, moff[l]:moff[l + 1]] = oi[0, moff[l]:moff[l + 1]]
        av[1, moff[l]:moff[l + 1]] = ov[0, moff[l]:moff[l + 1]]
        w_o = oracle.aggregate(ai, av, w_tail[a - a2:b - a2], 0.1, lo=a, hi=b)
        assert_bits_equal(f"layer {l} weights", to_np_f32(w_d[a:b]), w_o)
    _exact_mode_agrees(run, g_d, r_d, rep["layers_sampled"], "2^31 layout")
