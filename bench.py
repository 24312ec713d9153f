"""Benchmark of the LAGS-SGD hot path on one MI355X.

A step is one pass of the whole path for worker 0: lags_sparsify_layers
(error-compensated per-layer top-k, messages, residual) followed by
lags_aggregate_apply (P workers' messages summed in worker order and applied
to the weights).  The other P-1 workers' messages are seeded inputs, resident
in HBM with everything else before the timed region starts.

Prints one JSON line (rank 0).  Default workload: the 1.3B-parameter
transformer gradient (1,311,178,752 fp32 entries in 193 tensors, rho = 1/1000,
P = 16), the largest layout that fits one GPU.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME|all]
                  [--no-cpu-baseline] [--flush] [--pipeline] [--no-exact-mode]
                  [--no-per-config]

The line also carries "per_config": the pages' other workloads (ResNet-20,
VGG-16, ResNet-50, LSTM), each timed the same way in the same run (at least
20 steps), with their step time, rate, HBM fraction and kernel times.

--pipeline adds a second measurement of the same step issued layer range by
layer range (lags_sparsify_range / lags_aggregate_range, last layers first),
with the ranges of the merged-message schedule (lags_merge_schedule) under a
synthetic cost model stated in pipeline_model(), timed as issued from Python
and as one captured HIP graph replayed (the GPU's own cost, without the
host's per-call issue time; one replay is first checked bit for bit against
an eager step from the same state).

Every line also carries "exact_mode": the sparsify call with
LAGS_SPARSIFY_EXACT (multi-workgroup radix select) from the state after the
timed steps, its median time over five calls and whether its output equals
the sampled path's bit for bit.  It runs after the timed region;
--no-exact-mode leaves it out (profiles of the step alone).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Gelem/s layer-wise EC top-k sparsify+aggregate; % of HBM peak BW"
HBM_PEAK_GBS = 8000.0
DOMINANT = "k_main"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(n, K, P, U):
    """What the method must move per step: read grad and residual, write the
    residual (12 B/entry); write the own message (8 B per sent entry); read
    all P messages (8 B per entry); read-modify-write the touched weights."""
    return 12 * n + 8 * K + 8 * P * K + 8 * U


SMALL_MAX = 4096   # layers up to this size are finished outside the streaming pass


def main_kernel_bytes(wl, k):
    """Algorithmic bytes of one k_main launch: grad and residual read and the
    residual written for every entry of the layers it streams (all but the
    small ones), plus the message of the k == n layers it sends whole."""
    n = np.diff(wl.offsets())
    streamed = n > SMALL_MAX
    whole = streamed & (k == n)
    return int(12 * int(n[streamed].sum()) + 8 * int(k[whole].sum()))


def counters_traffic(workload):
    """HBM bytes per k_main launch from the committed rocprofv3 counter runs
    (FETCH_SIZE + WRITE_SIZE, each scaled by a 1 GiB copy), or None if they
    were taken on another workload or on a different kernel source."""
    import hashlib
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "k_main_counters.json")))[workload]
    except (OSError, KeyError, ValueError):
        return None
    src = os.path.join(ROOT, "layer_wise_top_amd", "csrc", "lags_kernels.hip")
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != rec.get("kernel_source_sha256"):
        return None
    return int(rec["traffic_bytes_per_launch"])


def cpu_baseline(wl, k, budget_s=20.0):
    """The oracle (single thread, as it stands) on a bounded sample of the
    same workload: the first layers of the table up to ~budget of CPU time
    (estimated from a small calibration run), sparsify + aggregate with P."""
    import oracle as O
    from layer_wise_top_amd import workloads as W
    orc = O.default()
    off = wl.offsets()
    if off[1] > 200_000_000:
        # one huge first tensor: time the same problem on its first 100M
        # entries as one layer of the same ratio
        from layer_wise_top_amd import lags
        m = 100_000_000
        num, den = wl.ratios()
        km = lags.lags_k_for_ratio(m, int(num[0]), int(den[0]))
        g = W.gen_grad_layer(wl, 0, 0, 0)[:m].copy()
        w = W.gen_weights_layer(wl, 0)[:m].copy()
        rng = np.random.default_rng(5)
        oi = np.stack([np.sort(rng.choice(m, km, replace=False)) for _ in range(wl.P - 1)]).astype(np.uint32)
        ov = rng.standard_normal(oi.shape).astype(np.float32) * np.float32(wl.const_std)
        t0 = time.perf_counter()
        orc.step(np.array([0, m]), np.array([km]), g, np.zeros(m, np.float32), oi, ov, w, wl.lr)
        t = time.perf_counter() - t0
        return {"value": round(m / t / 1e9, 6), "unit": "Gelem/s", "cores": 1, "kind": "oracle",
                "sample": f"{wl.name}: the first {m:,} entries of its single tensor as one layer "
                          f"(k = {km:,}), one sparsify + aggregate step with P={wl.P}, "
                          f"{t:.1f} s single-threaded on {cpu_model()}"}, None
    # calibrate on the smallest prefix with at least ~2M entries
    def run_prefix(nl):
        sub_off = off[: nl + 1]
        sub_k = k[:nl]
        n = int(sub_off[-1])
        g = np.concatenate([W.gen_grad_layer(wl, 0, 0, l) for l in range(nl)])
        r = np.zeros(n, np.float32)
        w = np.concatenate([W.gen_weights_layer(wl, l) for l in range(nl)])
        P = wl.P
        Ks = int(sub_k.sum())
        oi = np.empty((P - 1, Ks), np.uint32)
        ov = np.empty((P - 1, Ks), np.float32)
        moff = np.concatenate([[0], np.cumsum(sub_k)])
        for p in range(1, P):
            for l in range(nl):
                i, v = W.gen_message_layer(wl, 0, p, l, int(sub_k[l]))
                oi[p - 1, moff[l]:moff[l + 1]] = i
                ov[p - 1, moff[l]:moff[l + 1]] = v
        t0 = time.perf_counter()
        orc.step(sub_off, sub_k, g, r, oi, ov, w, wl.lr)
        return n, time.perf_counter() - t0
    nl = 1
    while nl < wl.L and off[nl] < 2_000_000:
        nl += 1
    n1, t1 = run_prefix(nl)
    rate = n1 / max(t1, 1e-9)
    target = rate * budget_s
    nl2 = nl
    while nl2 < wl.L and off[nl2 + 1] <= max(target, n1):
        nl2 += 1
    if nl2 > nl:
        n2, t2 = run_prefix(nl2)
    else:
        n2, t2 = n1, t1
    return {
        "value": round(n2 / t2 / 1e9, 6),
        "unit": "Gelem/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{wl.name}: first {nl2} of {wl.L} tensors ({n2:,} entries), one "
                  f"sparsify + aggregate step with P={wl.P}, {t2:.1f} s single-threaded "
                  f"on {cpu_model()}",
    }, run_prefix_threaded(wl, k, nl2)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def run_prefix_threaded(wl, k, nl):
    """The same oracle step on the same tensors, its per-layer selections and
    disjoint index windows of the aggregate run by a pool of threads (the
    oracle's C calls release the interpreter lock)."""
    import concurrent.futures as cf
    import oracle as O
    from layer_wise_top_amd import workloads as W
    orc = O.default()
    off = wl.offsets()
    sub_off = off[: nl + 1]
    n = int(sub_off[-1])
    threads = max(1, min(16, os.cpu_count() or 1))
    g = [W.gen_grad_layer(wl, 0, 0, l) for l in range(nl)]
    w = np.concatenate([W.gen_weights_layer(wl, l) for l in range(nl)])
    P = wl.P
    sub_k = k[:nl]
    Ks = int(sub_k.sum())
    moff = np.concatenate([[0], np.cumsum(sub_k)])
    oi = np.empty((P - 1, Ks), np.uint32)
    ov = np.empty((P - 1, Ks), np.float32)
    for p in range(1, P):
        for l in range(nl):
            i, v = W.gen_message_layer(wl, 0, p, l, int(sub_k[l]))
            oi[p - 1, moff[l]:moff[l + 1]] = i
            ov[p - 1, moff[l]:moff[l + 1]] = v
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda l: orc.sparsify([0, len(g[l])], [int(sub_k[l])], g[l],
                                                   np.zeros(len(g[l]), np.float32)), range(nl)))
        mi = np.concatenate([p_[0].astype(np.uint32) + np.uint32(sub_off[l]) for l, p_ in enumerate(parts)])
        mv = np.concatenate([p_[1] for p_ in parts])
        ai = np.concatenate([mi[None], oi], 0)
        av = np.concatenate([mv[None], ov], 0)
        cuts = np.linspace(0, n, threads + 1).astype(np.int64)
        list(ex.map(lambda t: orc.aggregate(ai, av, w[cuts[t]:cuts[t + 1]], wl.lr,
                                            lo=int(cuts[t]), hi=int(cuts[t + 1])),
                    [t for t in range(threads) if cuts[t + 1] > cuts[t]]))
    t = time.perf_counter() - t0
    return {
        "value": round(n / t / 1e9, 6), "unit": "Gelem/s", "cores": threads, "kind": "oracle",
        "sample": f"{wl.name}: the same {nl} tensors ({n:,} entries), per-layer selections and "
                  f"{threads} aggregate windows on {threads} threads, {t:.1f} s",
    }


def pipeline_model(wl, k):
    """Synthetic inputs of the merged-message schedule (the pages give no
    numbers): backward time of a tensor proportional to its size, 66 ps per
    parameter (a 1.3B-parameter model then takes ~86 ms, 4 * n * 16384 tokens
    at 1 PFLOP/s); each message costs a 50 us start-up plus its all-gather
    bytes, (P - 1) * 8 * k_l, at 50 GB/s."""
    n = np.diff(wl.offsets()).astype(np.float64)
    backward = n * 66e-12
    nbytes = (wl.P - 1) * 8 * np.asarray(k, np.int64)
    return backward, nbytes, 50e-6, 1.0 / 50e9


def torch_add_gbs(n, reps=5):
    """A reference stream of the same access pattern: torch.add over n fp32
    entries (read 2, write 1), in GB/s.  Not a ceiling: the streaming pass,
    whose workgroups each read one 16 KiB range per array in one step, runs
    faster than this looping elementwise kernel."""
    import torch
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.ones(n, dtype=torch.float32, device="cuda")
    c = torch.empty_like(a)
    torch.add(a, b, out=c)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.add(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b, c
    torch.cuda.empty_cache()
    return round(12 * n / (ms * 1e-3) / 1e9, 1)


def exact_mode(lay, g_d, r_d, msg_idx0, msg_val0, ws, stream, reps):
    """Sparsify in exact mode (the multi-workgroup radix select) from the
    current residual: equal bit for bit to the sampled path from the same
    state, and its time per call (events around each call; the residual is
    restored outside them).  Not part of the step."""
    import torch
    from layer_wise_top_amd import lags
    r0 = r_d.clone()
    outs = []
    for flags in (0, lags.LAGS_SPARSIFY_EXACT):
        r = r0.clone()
        mi = torch.empty_like(msg_idx0)
        mv = torch.empty_like(msg_val0)
        lags.lags_sparsify_layers(lay, g_d, r, mi, mv, ws, flags, stream)
        outs.append((mi, mv.view(torch.int32), r.view(torch.int32)))
    torch.cuda.synchronize()
    rep = lags.lags_workspace_report(lay, ws)
    same = all(bool(torch.equal(a, b)) for a, b in zip(outs[0], outs[1]))
    r = outs[1][2].view(torch.float32)
    mi, mv = outs[1][0], outs[1][1].view(torch.float32)
    times = []
    for _ in range(reps):
        r.copy_(r0)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        lags.lags_sparsify_layers(lay, g_d, r, mi, mv, ws, lags.LAGS_SPARSIFY_EXACT, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del outs, r0, r, mi, mv
    torch.cuda.empty_cache()
    return {"sparsify_ms_median": round(float(np.median(times)), 5), "calls": reps,
            "same_as_sampled": same, "layers_exact": rep["layers_exact"]}


def measure(name, steps, warmup, flush=False):
    """Inputs of one workload resident in HBM, W warm-up steps, then exactly K
    timed steps between two synchronisations (events on the launch stream),
    and K more steps with the library's per-kernel tracer.  Returns the state
    for further measurements and the metrics."""
    import torch
    from layer_wise_top_amd import lags, workloads as W

    wl = W.get(name)
    off = wl.offsets()
    num, den = wl.ratios()
    k = lags.k_table(off, num, den)
    lay = lags.Layout(off, k)
    P = wl.P
    dev = torch.device("cuda", 0)
    log(f"{name}: n={wl.n:,} L={wl.L} K={lay.K:,} P={P}: generating inputs")
    t0 = time.time()
    g = W.gen_grad(wl, 0)
    w0 = W.gen_weights(wl)
    oi, ov = W.gen_messages(wl, 0, k)
    log(f"inputs generated in {time.time() - t0:.1f} s; moving to HBM")
    g_d = torch.from_numpy(g).to(dev)
    del g
    w_d = torch.from_numpy(w0).to(dev)
    del w0
    r_d = torch.zeros(wl.n, dtype=torch.float32, device=dev)
    mi = torch.empty((P, lay.K), dtype=torch.int32, device=dev)
    mv = torch.empty((P, lay.K), dtype=torch.float32, device=dev)
    if P > 1:
        mi[1:].copy_(torch.from_numpy(oi.view(np.int32)))
        mv[1:].copy_(torch.from_numpy(ov))
    del oi, ov
    ws = lags.workspace(lay, P, device=dev)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if flush else None
    stream = torch.cuda.current_stream()

    def step():
        lags.lags_sparsify_layers(lay, g_d, r_d, mi[0], mv[0], ws, 0, stream)
        lags.lags_aggregate_apply(lay, w_d, mi, mv, P, wl.lr, ws, stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    rep = lags.lags_workspace_report(lay, ws)
    # distinct touched indices of one step (messages of the last warm step)
    U = int(torch.unique(mi.view(-1)).numel())

    # timed region: exactly `steps` steps bracketed by synchronisation; the
    # per-step events inside it add no synchronisation
    times = []
    if flush:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            scratch.fill_(i & 0xff)
            ev[i][0].record(stream)
            step()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        times = [a.elapsed_time(b) for a, b in ev]
        total_ms = sum(times)
    else:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for i in range(steps):
            step()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        total_ms = ev[0].elapsed_time(ev[-1])
        times = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    # per-kernel device time: the same steps again with the library's tracer,
    # which brackets every launch with HIP events on the launch stream
    lags.lags_trace_enable(lay, True)
    lags.lags_trace_read(lay)
    torch.cuda.synchronize()
    for _ in range(steps):
        if flush:
            scratch.fill_(0)
        step()
    trace = lags.lags_trace_read(lay)
    lags.lags_trace_enable(lay, False)
    ms_per_step = total_ms / steps
    kernels = {kname: round(ms / max(cnt, 1), 5) for kname, (ms, cnt) in trace.items() if cnt}
    main_ms = kernels[DOMINANT]
    b_main = main_kernel_bytes(wl, k)
    B = algorithmic_bytes(wl.n, lay.K, P, U)
    m = {
        "ms_per_step": round(ms_per_step, 5),
        "value": round(wl.n / (ms_per_step * 1e-3) / 1e9, 3),
        "hbm_frac_step": round(B / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "alg_bytes_step": B,
        "step_ms_min": round(min(times), 5),
        "step_ms_median": round(float(np.median(times)), 5),
        "k_main_ms": main_ms,
        "k_main_frac": round(b_main / (main_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "k_main_alg_bytes": b_main,
        "kernels_avg_ms": kernels,
        "sparsify_ms": round(sum(v for kk, v in kernels.items() if not kk.startswith("k_agg")), 5),
        "aggregate_ms": round(sum(v for kk, v in kernels.items() if kk.startswith("k_agg")), 5),
        "report": rep,
    }
    state = dict(wl=wl, k=k, lay=lay, g_d=g_d, r_d=r_d, w_d=w_d, mi=mi, mv=mv, ws=ws, P=P,
                 stream=stream, scratch=scratch, U=U, dev=dev)
    return state, m


def run_config(name, steps, warmup, do_cpu, flush, pipeline=False, exact=True, per_config=()):
    import torch
    from layer_wise_top_amd import lags, workloads as W

    st, m = measure(name, steps, warmup, flush)
    wl, k, lay, P, U = st["wl"], st["k"], st["lay"], st["P"], st["U"]
    g_d, r_d, w_d, mi, mv, ws = st["g_d"], st["r_d"], st["w_d"], st["mi"], st["mv"], st["ws"]
    stream, scratch, dev = st["stream"], st["scratch"], st["dev"]
    off = wl.offsets()
    main_ms = m["k_main_ms"]
    b_main = m["k_main_alg_bytes"]
    achieved = b_main / (main_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": m["value"],
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded numpy draws of the workload's shapes and distributions)",
        "config": {
            "workload": wl.name, "entries": wl.n, "tensors": wl.L, "sent_per_worker": lay.K,
            "workers": P, "touched": U, "rho": "adaptive" if wl.rho_rule == "adaptive"
            else f"{wl.rho_uniform[0]}/{wl.rho_uniform[1]}", "flush_infinity_cache": bool(flush),
        },
        "hbm_frac_step": m["hbm_frac_step"],
        "alg_bytes_step": m["alg_bytes_step"],
        "roofline": {
            "kernel": DOMINANT, "bound": "hbm", "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": counters_traffic(wl.name), "alg_bytes_per_launch": b_main,
            "avg_ms": main_ms,
        },
        "kernels_avg_ms": m["kernels_avg_ms"],
        "sparsify_ms": m["sparsify_ms"],
        "aggregate_ms": m["aggregate_ms"],
        "report": m["report"],
        "step_ms_min": m["step_ms_min"],
        "step_ms_median": m["step_ms_median"],
    }
    if exact:
        out["exact_mode"] = exact_mode(lay, g_d, r_d, mi[0], mv[0], ws, stream, 5)
    if pipeline:
        backward, nbytes, alpha, beta = pipeline_model(wl, k)
        runs, finish = lags.lags_merge_schedule(backward, nbytes, alpha, beta)

        def piped():
            for l0, l1 in runs:
                lags.lags_sparsify_range(lay, l0, l1, g_d, r_d, mi[0], mv[0], ws, 0, stream)
                lags.lags_aggregate_range(lay, l0, l1, w_d, mi, mv, P, wl.lr, ws, stream)

        for _ in range(warmup):
            piped()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            piped()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_piped = e0.elapsed_time(e1) / steps
        # the same issue captured once into a HIP graph and replayed: the
        # GPU's own cost per step, without the host's per-call issue time
        # (one replay is first checked bit for bit against an eager step
        # from the same state)
        gs = torch.cuda.Stream()

        def piped_on(s):
            for l0, l1 in runs:
                lags.lags_sparsify_range(lay, l0, l1, g_d, r_d, mi[0], mv[0], ws, 0, s)
                lags.lags_aggregate_range(lay, l0, l1, w_d, mi, mv, P, wl.lr, ws, s)

        torch.cuda.synchronize()
        r0, w0 = r_d.clone(), w_d.clone()
        torch.cuda.synchronize()              # the copies are done before gs starts
        with torch.cuda.stream(gs):
            piped_on(gs)
        torch.cuda.synchronize()
        want = (r_d.clone(), w_d.clone(), mi[0].clone(), mv[0].clone())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=gs):
            piped_on(gs)
        r_d.copy_(r0)
        w_d.copy_(w0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        graph_same = all(bool(torch.equal(a.view(torch.int32), b.view(torch.int32)))
                         for a, b in zip((r_d, w_d, mi[0], mv[0]), want))
        del r0, w0, want
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        ms_graph = e0.elapsed_time(e1) / steps
        del graph
        per_layer = [(l, l + 1) for l in range(wl.L - 1, -1, -1)]
        # the same, with per-layer sizes from each layer's overlap window
        k_ad = lags.lags_adaptive_k(off, backward, P, alpha, beta, (1, 1000))
        runs_ad, _ = lags.lags_merge_schedule(backward, (P - 1) * 8 * k_ad, alpha, beta)
        lay_ad = lags.Layout(off, k_ad)
        oi, ov = W.gen_messages(wl, 0, k_ad)
        mi_ad = torch.empty((P, lay_ad.K), dtype=torch.int32, device=dev)
        mv_ad = torch.empty((P, lay_ad.K), dtype=torch.float32, device=dev)
        if P > 1:
            mi_ad[1:].copy_(torch.from_numpy(oi.view(np.int32)))
            mv_ad[1:].copy_(torch.from_numpy(ov))
        del oi, ov
        ws_ad = lags.workspace(lay_ad, P, device=dev)

        def piped_ad():
            for l0, l1 in runs_ad:
                lags.lags_sparsify_range(lay_ad, l0, l1, g_d, r_d, mi_ad[0], mv_ad[0], ws_ad, 0, stream)
                lags.lags_aggregate_range(lay_ad, l0, l1, w_d, mi_ad, mv_ad, P, wl.lr, ws_ad, stream)

        for _ in range(warmup):
            piped_ad()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            piped_ad()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_ad = e0.elapsed_time(e1) / steps
        del mi_ad, mv_ad, ws_ad
        out["pipeline"] = {
            "runs": len(runs), "ms_per_step": round(ms_piped, 5),
            "ms_per_step_graph": round(ms_graph, 5), "graph_same_as_eager": graph_same,
            "model": "backward 66 ps/param, 50 us + all-gather bytes at 50 GB/s per message",
            "modelled_comm_finish_ms": {
                "merged": round(finish * 1e3, 4),
                "per_layer": round(lags.lags_schedule_finish(backward, nbytes, alpha, beta,
                                                             per_layer) * 1e3, 4),
                "one_message": round(lags.lags_schedule_finish(backward, nbytes, alpha, beta,
                                                               [(0, wl.L)]) * 1e3, 4),
            },
            "adaptive_k": {"sent_per_worker": int(k_ad.sum()), "runs": len(runs_ad),
                           "ms_per_step": round(ms_ad, 5)},
        }
    del g_d, w_d, r_d, mi, mv, ws, scratch, st
    torch.cuda.empty_cache()
    out["torch_add_gbs"] = torch_add_gbs(wl.n)
    if per_config:
        # the other workloads, timed the same way in the same run (the
        # headline fields above are the largest one's)
        out["per_config"] = {}
        for other in per_config:
            if other == name:
                continue
            st2, m2 = measure(other, max(steps, 20), warmup, flush)
            del st2
            torch.cuda.empty_cache()
            out["per_config"][other] = m2
    if do_cpu:
        log("timing the oracle on a bounded sample")
        out["cpu_baseline"], threaded = cpu_baseline(wl, k)
        if threaded is not None:
            out["cpu_baseline_threads"] = threaded
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="tfm1p3b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 1 GiB buffer a few times (reference for traffic counters)")
    ap.add_argument("--flush", action="store_true",
                    help="write 512 MiB between steps (outside the step events) to evict the "
                         "Infinity Cache; steps are then timed one by one")
    ap.add_argument("--pipeline", action="store_true",
                    help="also time the step issued per merged-message layer range")
    ap.add_argument("--no-exact-mode", action="store_true",
                    help="leave out the exact-mode sparsify measured after the timed steps")
    ap.add_argument("--no-per-config", action="store_true",
                    help="time only the chosen workload (by default the line also carries "
                         "per_config: every other workload of the pages, timed the same way)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path runs on one GPU's share; other workers' messages are inputs)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": {"read": 1 << 30, "write": 1 << 30},
                          "launches": 3}), flush=True)
        return
    from layer_wise_top_amd import workloads as W
    names = list(W.ORDER) + list(W.EXTRA) if args.config == "all" else [args.config]
    for nm in names:
        if nm not in W.WORKLOADS:
            print(f"unknown workload {nm}; choose from {', '.join(W.WORKLOADS)} or all", file=sys.stderr)
            sys.exit(2)
    per_config = () if (args.no_per_config or args.config == "all") else tuple(W.ORDER)
    for name in names:
        out = run_config(name, args.steps, args.warmup, not args.no_cpu_baseline, args.flush,
                         args.pipeline, not args.no_exact_mode, per_config)
        print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
