#!/usr/bin/env python3
"""Benchmark of the sparse latent-MoE decode step on one MI355X.

One step = one pass of the whole layer (router + top-k, latent-down, MXFP4
experts, combine, shared expert, latent-up) over one batch of synthetic
tokens.  The timed region is K launches of one-step HIP graphs (one graph per
input; the per-layer graph of a decode engine), back to back between two
synchronisations.  Inputs rotate through R pre-generated batches (different
routing each step) that are resident in HBM before the timed region starts.

Prints ONE JSON line:
  value        whole-step algorithmic HBM bytes / time (GB/s)
  ms_per_step  time per layer step over the K timed launches; p10/p50/p90
               from events between further launches; the same steps from
               graphs of 8 consecutive steps and as eager launches beside
  roofline     the kernel with the largest time of the library's default
               mode, its algorithmic bytes per launch over its average
               duration (HIP events attached to each kernel's dispatch on
               eager steps), against 8 TB/s
  expert_path  k_w13 + k_w2 of the four-launch step: the routed-expert
               kernels alone, bytes of the distinct experts the GPU selected
  modes        the same inputs in every execution mode
  cpu_baseline the binary64 CPU oracle on a bounded sample of the same inputs
  batch_sweep  the same K3 weights at batch 2, 8 (Zipf routing), 64
               (near-uniform routing), 64 (the batch-1 bias) and two
               speculative-decoding verify batches, each with the oracle on
               all host cores beside it
  c0_tiny_b1   the 64-expert layer at batch 1 (cache-resident: latency only)
  c4_x8        eight TP8-share layers in one graph at batch 1, 8 and 64: time
               per launch and per layer, one layer's kernels, expert path and
               roofline, the oracle on one layer at batch 1 and 64
With --workload c4_x8: the eight-layer graph at batch 1..64 in every mode.
"""
import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE decode layer µs/step + achieved HBM GB/s (% peak) at batch 1/8/64"
HBM_PEAK_GBS = 8000.0

# name -> (layer recipe, batch, top_k, description)
WORKLOADS = {
    "k3_b1": ("k3", 1, 16, "K3-scale layer, batch 1: hidden 7168, latent 2048, 896 MXFP4 "
              "experts (SwiGLU 2048->2048->2048), top-16, bias N(0,0.1), shared expert 4096"),
    "k3_zipf_b8": ("k3_zipf", 8, 16, "K3-scale layer, batch 8, Zipf(1.1) expert popularity"),
    "k3_flat_b64": ("k3_flat", 64, 16, "K3-scale layer, batch 64, near-uniform routing"),
    "k3_b64": ("k3", 64, 16, "K3-scale layer, batch 64, bias N(0,0.1)"),
    "k3_tp8_b1": ("k3_tp8", 1, 16, "one TP8 rank's share of the K3 layer, batch 1"),
    "tiny_b1": ("tiny", 1, 4, "64-expert layer, batch 1"),
}
KERNELS_BF16 = ("dense_in", "w13", "w2", "out")
KERNEL_SYMBOLS = {"dense_in": "k_dense_in", "w13": "k_w13", "w2": "k_w2", "out": "k_out",
                  "router_f32": "k_router_f32", "step": "k_step", "tail": "k_tail",
                  "shared_gu": "k_dense_in", "shared_down": "k_out_part", "lat_up": "k_out_part"}


MODE_FILTER = None  # names selected with --modes (None: all)
GRAPH_STEPS = 8     # consecutive steps (different inputs) per replayed graph


def modes():
    """Execution modes of the library by name (those selected with --modes,
    and the default one)."""
    from sparse_moe_decode_router_amd import binding
    allm = {"four_launches": binding.MODE_FOUR_LAUNCHES,
            "late_routing": binding.MODE_LATE_ROUTING,
            "dense_routing": binding.MODE_DENSE_ROUTING,
            "ordered": binding.MODE_ORDERED,
            "side_stream": binding.MODE_SIDE_STREAM,
            "two_launches": binding.MODE_TWO_LAUNCHES, "fused": binding.MODE_FUSED}
    if MODE_FILTER is None:
        return allm
    dflt = {v: n for n, v in allm.items()}[binding.DEFAULT_MODE]
    return {n: v for n, v in allm.items() if n in MODE_FILTER or n == dflt}


def default_mode():
    from sparse_moe_decode_router_amd import binding
    return {v: n for n, v in modes().items()}[binding.DEFAULT_MODE]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_bytes(d, B, k, D):
    """Algorithmic HBM bytes of each kernel of one step: weights read once
    (experts: only the D distinct active ones), activations in and out in the
    precision they are stored in (bf16 x/out, hi+lo bf16 intermediates, f32
    scores/keys/weights, i32 ids)."""
    H, L, E, I, Is = d.hidden, d.latent, d.n_experts, d.expert_inter, d.shared_inter
    P = B * k
    router = E * H * (4 if d.router_f32 else 2)
    expert13 = 2 * I * (L // 2 + L // 32)
    expert2 = L * (I // 2 + I // 32)
    b = {
        "dense_in": (0 if d.router_f32 else router) + L * H * 2 + 2 * Is * H * 2 + B * H * 2
        + B * L * 4 + B * Is * 4 + (0 if d.router_f32 else B * E * 8 + P * 8),
        "w13": D * expert13 + B * L * 4 + P * I * 4,
        "w2": D * expert2 + P * I * 4 + B * L * 4,
        "out": H * L * 2 + H * Is * 2 + B * L * 4 + B * Is * 4 + B * H * 2,
    }
    if d.router_f32:
        b["router_f32"] = router + B * H * 2 + B * E * 8 + P * 8
    return b


def kernel_bytes_side(d, B, k, D):
    """kernel_bytes split the way the side-stream step launches: dense-in
    (router + latent-down + routing), shared gate/up, gate/up, down,
    shared-down, latent-up."""
    H, L, E, Is = d.hidden, d.latent, d.n_experts, d.shared_inter
    b = kernel_bytes(d, B, k, D)
    shared_gu = 2 * Is * H * 2 + B * H * 2 + B * Is * 4
    shared_down = H * Is * 2 + B * Is * 4 + B * H * 4
    return {"dense_in": b["dense_in"] - shared_gu + B * H * 2, "shared_gu": shared_gu,
            "w13": b["w13"], "w2": b["w2"], "shared_down": shared_down,
            "lat_up": H * L * 2 + B * L * 4 + B * H * 4 + B * H * 2}


def load_traffic(kernel, workload):
    """HBM bytes per launch measured with rocprofv3 counters for this kernel
    source, from profiles/traffic.json; None when absent or stale."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    from sparse_moe_decode_router_amd.build import source_digest
    e = t.get(workload, {}).get(kernel)
    if not e or e.get("source_digest") != source_digest():
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(layer, xs, k, bytes_per_step, seconds):
    """The oracle as it stands, single-threaded, on whole steps of the same
    inputs until about `seconds` of work has been done."""
    import oracle
    oracle.lib()
    done, t_total = 0, 0.0
    for x in xs:
        t0 = time.perf_counter()
        oracle.moe_step(layer, x, rounding="output")
        t_total += time.perf_counter() - t0
        done += 1
        if t_total >= seconds:
            break
    per_step = t_total / done
    return {"value": bytes_per_step / per_step / 1e9, "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{done} of the {len(xs)} rotating input batches, whole steps "
                      f"(batch {xs[0].shape[0]}), {per_step:.3f} s per step single-threaded"}


def cpu_baseline_all_cores(layer, xs, k, bytes_per_step, seconds):
    """The same oracle on several host cores at once: one whole step per
    thread (the C oracle is reentrant and ctypes releases the interpreter
    lock during the call), rounds of as many steps as threads until about
    `seconds` have passed.  At most 16 threads, the host share of one GPU."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    oracle.lib()
    n = max(1, min(16, os.cpu_count() or 1))
    done, i = 0, 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=n) as pool:
        while time.perf_counter() - t0 < seconds:
            batch = [xs[(i + j) % len(xs)] for j in range(n)]
            i += n
            list(pool.map(lambda x: oracle.moe_step(layer, x, rounding="output"), batch))
            done += n
    elapsed = time.perf_counter() - t0
    return {"value": bytes_per_step * done / elapsed / 1e9, "unit": "GB/s", "cores": n,
            "kind": "oracle",
            "sample": f"{done} whole steps (batch {xs[0].shape[0]}) of the rotating inputs, "
                      f"{n} at a time on {n} threads, {elapsed:.1f} s"}


def cpu_oracle_sampled(layer, xs, bytes_per_step, seconds):
    """The oracle on all host cores (up to 16 threads) for a batch too large to
    time whole: single tokens of the rotating inputs, one per thread call,
    for about `seconds`.  Tokens are independent in the oracle, so a step of
    B tokens costs B token times; the figure is the step's bytes over that."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    oracle.lib()
    B = xs[0].shape[0]
    toks = [x[b:b + 1] for x in xs for b in range(B)]
    n = max(1, min(16, os.cpu_count() or 1))
    done, i = 0, 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=n) as pool:
        while time.perf_counter() - t0 < seconds:
            batch = [toks[(i + j) % len(toks)] for j in range(n)]
            i += n
            list(pool.map(lambda x: oracle.moe_step(layer, x, rounding="output"), batch))
            done += n
    elapsed = time.perf_counter() - t0
    s_step = B * elapsed / done
    return {"value": bytes_per_step / s_step / 1e9, "unit": "GB/s", "cores": n,
            "kind": "oracle", "us_per_step": round(s_step * 1e6, 1),
            "sample": f"{done} single tokens of the rotating batches on {n} threads in "
                      f"{elapsed:.1f} s, times {B} tokens per step"}


def device_info():
    """The GPU the figures come from, and the peak they are priced against."""
    import torch
    p = torch.cuda.get_device_properties(0)
    return {"name": torch.cuda.get_device_name(0), "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2**30, 1),
            "hbm_peak_assumed_gbs": HBM_PEAK_GBS}


def pct(v, q):
    import numpy as np
    return float(np.percentile(np.asarray(v), q))


def kernel_durations(ctx, names, kb, xd, k, out, idx, wts, steps, stream, out_staged):
    """Per-kernel durations: HIP events attached to each kernel's dispatch
    (start and stop of the kernel itself) on `steps` eager steps on `stream`,
    one event set per rotating input, read back before it is reused; each
    kernel's algorithmic bytes (kb[r][name]) over its average duration."""
    import torch
    R = len(xd)
    kev = []
    for r in range(R):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(names))]
        for x in e:
            x.record(stream)
        kev.append(e)
    torch.cuda.synchronize()
    sums = {n: 0.0 for n in names}
    kbytes = {n: 0.0 for n in names}
    pending = [False] * R

    def collect(r):
        e = kev[r]
        e[-1].synchronize()
        for j, n in enumerate(names):
            sums[n] += e[2 * j].elapsed_time(e[2 * j + 1])
            kbytes[n] += kb[r][n]

    for i in range(steps):
        r = i % R
        if pending[r]:
            collect(r)
        ctx.set_timing_events(kev[r])
        ctx.step(xd[r], k, out, idx, wts, stream=stream)
        pending[r] = True
    ctx.set_timing_events(None)
    torch.cuda.synchronize()
    for r in range(R):
        if pending[r]:
            collect(r)
    per_kernel = {}
    for n in names:
        avg_ms = sums[n] / steps
        avg_bytes = kbytes[n] / steps
        gbs = avg_bytes / (avg_ms * 1e-3) / 1e9
        sym = KERNEL_SYMBOLS[n]
        B = ctx.last_dispatch()["batch"]
        if n == "out":  # the output kernel's forms: K slices above 8 tokens, staged operands up to 8
            sym = "k_out_kx" if B > 8 else "k_out_st" if out_staged else sym
        elif n == "dense_in" and ctx.last_dispatch().get("in_staged") == 2:  # x per row group, K slices
            sym = "k_dense_in_kx"
        elif n == "dense_in" and ctx.last_dispatch().get("in_staged") == 1:  # x staged, up to 2 tokens
            sym = "k_dense_in_xl"
        elif n == "dense_in" and ctx.last_dispatch().get("in_staged") == 3:  # x staged, 3 to 8 tokens
            sym = "k_dense_in_xl8"
        per_kernel[n] = {"symbol": sym, "us": round(avg_ms * 1e3, 2),
                         "bytes": int(avg_bytes), "gbs": round(gbs, 1),
                         "frac": round(gbs / HBM_PEAK_GBS, 4)}
    return per_kernel


def expert_path(per_kernel):
    """k_w13 + k_w2 of the four-launch step: bytes of the distinct active
    experts (and their activations) over the two kernels' durations."""
    ex_us = per_kernel["w13"]["us"] + per_kernel["w2"]["us"]
    ex_bytes = per_kernel["w13"]["bytes"] + per_kernel["w2"]["bytes"]
    ex_gbs = ex_bytes / (ex_us * 1e-6) / 1e9
    return {"us": round(ex_us, 2), "gbs": round(ex_gbs, 1),
            "pct_hbm_peak": round(100 * ex_gbs / HBM_PEAK_GBS, 2),
            "from": "k_w13 + k_w2 of the four-launch step"}


def measure(dev, d, B, k, xs, steps, warmup, mode):
    """One configuration in one execution mode: graph replays (wall clock over
    `steps` replays, then per-replay events for percentiles) and eager steps
    with events attached to each kernel's dispatch (per-kernel durations; the
    fused step is one kernel).  Inputs rotate through xs."""
    import numpy as np
    import torch

    from sparse_moe_decode_router_amd import binding

    ctx = binding.MoEDecode(dev, B, k)
    ctx.set_mode(mode)
    R = len(xs)
    xd = [torch.from_numpy(x.view(np.int16)).cuda() for x in xs]
    out = torch.empty((B, d.hidden), dtype=torch.int16, device="cuda")
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((B, k), dtype=torch.float32, device="cuda")
    # Distinct experts each input actually selects on the GPU.
    Ds = []
    for r in range(R):
        ctx.step(xd[r], k, out, idx, wts)
        torch.cuda.synchronize()
        Ds.append(int(np.unique(idx.cpu().numpy()).size))
    disp = ctx.last_dispatch()
    fused = bool(disp["fused"])
    if disp["fused"] == 1:
        names = ("step",)
        kb = [{"step": sum(kernel_bytes(d, B, k, D).values())} for D in Ds]
    elif disp["fused"] == 3:
        names = (("router_f32",) if d.router_f32 else ()) + (
            "dense_in", "shared_gu", "w13", "w2", "shared_down", "lat_up")
        kb = [kernel_bytes_side(d, B, k, D) for D in Ds]
        if d.router_f32:
            for D, x in zip(Ds, kb):
                x["router_f32"] = kernel_bytes(d, B, k, D)["router_f32"]
    elif disp["fused"] == 2:
        names = ("dense_in", "tail")
        kb = []
        for D in Ds:
            b = kernel_bytes(d, B, k, D)
            kb.append({"dense_in": b["dense_in"], "tail": b["w13"] + b["w2"] + b["out"]})
    else:
        names = (("router_f32",) if d.router_f32 else ()) + KERNELS_BF16
        kb = [kernel_bytes(d, B, k, D) for D in Ds]
    step_bytes = [sum(b.values()) for b in kb]
    assert ctx.read_flags() == 0

    stream = torch.cuda.Stream()
    # The timed region: one graph per input, a graph launch per step (the
    # per-layer graph of a decode engine); `steps` launches back to back
    # between two synchronisations.
    graphs = [binding.Graph([ctx], [xd[r]], B, k, [out], [idx], [wts]) for r in range(R)]
    for i in range(warmup):
        graphs[i % R].launch(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % R].launch(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    mean_bytes = sum(step_bytes[i % R] for i in range(steps)) / steps
    # Per-launch spread, outside the timed region: an event between
    # consecutive launches, over at least 64 launches.
    n_ev = max(steps, 64)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev + 1)]
    evs[0].record(stream)
    for i in range(n_ev):
        graphs[i % R].launch(stream)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(n_ev)]
    # Graphs of G consecutive steps (G different inputs) for comparison: a
    # graph launch per G steps, as when many layers share one graph.
    G = GRAPH_STEPS if R % GRAPH_STEPS == 0 else 1
    NG = R // G
    graphs_g = [binding.Graph([ctx] * G, xd[G * q:G * q + G], B, k, [out] * G, [idx] * G,
                              [wts] * G) for q in range(NG)]
    reps = max(1, steps // G)
    for i in range(max(1, warmup // G)):
        graphs_g[i % NG].launch(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(reps):
        graphs_g[i % NG].launch(stream)
    torch.cuda.synchronize()
    ms_graph_g = (time.perf_counter() - t0) * 1e3 / (reps * G)
    for g in graphs_g:
        g.close()
    # Cold against warm: events around single one-step replays, each cold one
    # after a 1 GiB read on the same stream, which evicts the last-level cache
    # (256 MB on MI355X), so that no weight row comes from an earlier step;
    # the warm ones run the same way without the read.  (A scrub by writing
    # leaves up to the whole cache dirty, and the replay then pays for its
    # write-back: about 50 us at batch 1.)
    scrub = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    n_cold = min(steps, 32)
    cw = {}
    for kind in ("warm", "cold"):
        ce = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_cold)]
        for i in range(n_cold):
            if kind == "cold":
                with torch.cuda.stream(stream):
                    sink.add_(scrub.sum())
            ce[2 * i].record(stream)
            graphs[i % R].launch(stream)
            ce[2 * i + 1].record(stream)
        torch.cuda.synchronize()
        cw[kind] = pct([ce[2 * i].elapsed_time(ce[2 * i + 1]) * 1e3 for i in range(n_cold)], 50)
    del scrub, sink

    # Eager steps (launches without a graph), for comparison.
    for i in range(warmup):
        ctx.step(xd[i % R], k, out, idx, wts, stream=stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ctx.step(xd[i % R], k, out, idx, wts, stream=stream)
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t0) * 1e3 / steps

    per_kernel = kernel_durations(ctx, names, kb, xd, k, out, idx, wts, steps, stream,
                                  disp.get("out_staged"))
    expert = None if fused else expert_path(per_kernel)
    assert ctx.read_flags() == 0, "a bounded wait of the fused step ran out"
    for g in graphs:
        g.close()
    ctx.close()
    return {
        "ms": ms, "value": mean_bytes / (ms * 1e-3) / 1e9, "ms_eager": ms_eager,
        "ms_graph_g": ms_graph_g, "n_launches_timed": steps, "n_launches_percentiles": n_ev,
        "us_p10": pct(per, 10), "us_p50": pct(per, 50), "us_p90": pct(per, 90),
        "cold": {"us_warm": round(cw["warm"], 2), "us_cold": round(cw["cold"], 2),
                 "ratio": round(cw["cold"] / cw["warm"], 3),
                 "method": "median of one-step graph replays timed by events; cold ones "
                           "each after a 1 GiB read that evicts the last-level cache"},
        "Ds": Ds, "step_bytes": step_bytes, "per_kernel": per_kernel, "dispatch": disp,
        "names": names, "expert_path": expert,
    }


def summary(name, B, m, alt):
    """Figures of one configuration in the default mode, with every mode's
    time per step beside them."""
    return {"workload": name, "batch": B, "us_per_step": round(m["ms"] * 1e3, 2),
            "us_p10": round(m["us_p10"], 2), "us_p50": round(m["us_p50"], 2),
            "us_p90": round(m["us_p90"], 2), "tokens_per_s": round(B / (m["ms"] * 1e-3), 1),
            "gbs": round(m["value"], 1), "pct_hbm_peak": round(100 * m["value"] / HBM_PEAK_GBS, 2),
            "distinct_experts_mean": round(sum(m["Ds"]) / len(m["Ds"]), 1),
            "expert_path": alt.get("four_launches", m)["expert_path"],
            "cold": m["cold"],
            "us_per_step_by_mode": {n: round(x["ms"] * 1e3, 2) for n, x in alt.items()}}


# Batch sweep on the K3 layer's weights (the bias alone changes): name ->
# (bias recipe, batch).
SWEEP = (("k3_b2", "k3", 2, None), ("k3_zipf_b8", "k3_zipf", 8, None),
         ("k3_flat_b64", "k3_flat", 64, None), ("k3_b64", "k3", 64, None),
         # speculative-decoding verify batches: users x (drafts + 1) correlated tokens
         ("k3_spec_u1_d7", "k3", 8, (1, 7)), ("k3_spec_u8_d3", "k3", 32, (8, 3)))


def run_c4(args):
    """Eight TP8-share layers (own seeds, own inputs) captured in one graph,
    swept over the batch; value = algorithmic bytes of the eight layers over
    the time of one graph replay at batch 1."""
    import numpy as np
    import torch

    from sparse_moe_decode_router_amd import binding, synth

    recipe = synth.K3_TP8
    d = recipe.dims
    n_layers, k = 8, 16
    layers = []
    for l in range(n_layers):
        log(f"[bench] generating C4 layer {l}")
        layers.append(synth.make_layer(recipe, synth.TP8_STACK_SEED0 + l))
    devs = [binding.DeviceLayer(la) for la in layers]
    stream = torch.cuda.Stream()
    results = []
    def replay_ms(graphs, R):
        for i in range(args.warmup):
            graphs[i % R].launch(stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % R].launch(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps

    for B in (1, 2, 4, 8, 16, 32, 64):
        ctxs = [binding.MoEDecode(dv, B, k) for dv in devs]
        R = 4
        xd = [[torch.from_numpy(synth.make_tokens(d, synth.TP8_STACK_SEED0 + l, B, draw=r)
                                .view(np.int16)).cuda() for l in range(n_layers)] for r in range(R)]
        outs = [torch.empty((B, d.hidden), dtype=torch.int16, device="cuda") for _ in range(n_layers)]
        idxs = [torch.empty((B, k), dtype=torch.int32, device="cuda") for _ in range(n_layers)]
        wts = [torch.empty((B, k), dtype=torch.float32, device="cuda") for _ in range(n_layers)]
        graphs = [binding.Graph(ctxs, xd[r], B, k, outs, idxs, wts) for r in range(R)]
        Ds = []
        for r in range(R):
            graphs[r].launch(stream)
            torch.cuda.synchronize()
            Ds.append([int(np.unique(i.cpu().numpy()).size) for i in idxs])
        step_bytes = [sum(sum(kernel_bytes(d, B, k, D).values()) for D in ds) for ds in Ds]
        ms = replay_ms(graphs, R)
        mean_bytes = sum(step_bytes[i % R] for i in range(args.steps)) / args.steps
        by_mode = {}
        for name, mode in modes().items():
            for g in graphs:
                g.close()
            for c in ctxs:
                c.set_mode(mode)
            graphs = [binding.Graph(ctxs, xd[r], B, k, outs, idxs, wts) for r in range(R)]
            by_mode[name] = round(replay_ms(graphs, R) * 1e3 / n_layers, 2)
        # The default form with each layer prefetching the next one's router
        # and latent-down rows while it routes.
        for g in graphs:
            g.close()
        for c in ctxs:
            c.set_mode(binding.DEFAULT_MODE)
        graphs = [binding.Graph(ctxs, xd[r], B, k, outs, idxs, wts, prefetch_next=True)
                  for r in range(R)]
        by_mode["four_launches_prefetch"] = round(replay_ms(graphs, R) * 1e3 / n_layers, 2)
        assert all(c.read_flags() == 0 for c in ctxs), "a bounded wait of a persistent step ran out"
        results.append({"batch": B, "us_per_8_layers": round(ms * 1e3, 2),
                        "us_per_layer": round(ms * 1e3 / n_layers, 2),
                        "tokens_per_s": round(B / (ms * 1e-3), 1),
                        "gbs": round(mean_bytes / (ms * 1e-3) / 1e9, 1),
                        "distinct_experts_mean": round(float(np.mean(Ds)), 1),
                        "us_per_layer_by_mode": by_mode})
        log(f"[bench] C4 B={B}: {results[-1]}")
        for g in graphs:
            g.close()
        for c in ctxs:
            c.close()
    r1 = results[0]
    line = {
        "metric": METRIC, "value": r1["gbs"], "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(r1["us_per_8_layers"] / 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "c4_x8: eight TP8-share layers (hidden 7168, latent 2048, 896 "
                   "MXFP4 experts of inter 256, top-16, shared 512) in one HIP graph, batch 1",
                   "batch": 1, "layers": n_layers, "parallelism": "1 GPU"},
        "batch_sweep": results, "roofline": None, "cpu_baseline": None,
        "device": device_info(),
    }
    print(json.dumps(line), flush=True)


def c4_summary(args, batches=(1, 8, 64), oracle_batches=(1, 64)):
    """Eight TP8-share layers (own seeds and inputs) captured in one HIP graph,
    at each batch of `batches`: the time per graph launch (all eight layers,
    `args.steps` launches between two synchronisations), per layer, tokens/s
    and GB/s; the per-kernel durations of one layer's eager steps (events
    attached to each dispatch), its expert path and its kernel with the largest
    time against 8 TB/s; the oracle on one layer at `oracle_batches`."""
    import numpy as np
    import torch

    from sparse_moe_decode_router_amd import binding, synth

    recipe = synth.K3_TP8
    d = recipe.dims
    n_layers, k, R = 8, 16, 4
    t0 = time.time()
    layers = [synth.make_layer(recipe, synth.TP8_STACK_SEED0 + l) for l in range(n_layers)]
    devs = [binding.DeviceLayer(la) for la in layers]
    log(f"[bench] C4 layers generated and copied in {time.time() - t0:.1f} s")
    stream = torch.cuda.Stream()
    res = []
    for B in batches:
        ctxs = [binding.MoEDecode(dv, B, k) for dv in devs]
        xs = [[synth.make_tokens(d, synth.TP8_STACK_SEED0 + l, B, draw=r)
               for l in range(n_layers)] for r in range(R)]
        xd = [[torch.from_numpy(x.view(np.int16)).cuda() for x in row] for row in xs]
        outs = [torch.empty((B, d.hidden), dtype=torch.int16, device="cuda")
                for _ in range(n_layers)]
        idxs = [torch.empty((B, k), dtype=torch.int32, device="cuda") for _ in range(n_layers)]
        wts = [torch.empty((B, k), dtype=torch.float32, device="cuda") for _ in range(n_layers)]
        graphs = [binding.Graph(ctxs, xd[r], B, k, outs, idxs, wts) for r in range(R)]
        Ds = []
        for r in range(R):
            graphs[r].launch(stream)
            torch.cuda.synchronize()
            Ds.append([int(np.unique(i.cpu().numpy()).size) for i in idxs])
        step_bytes = [sum(sum(kernel_bytes(d, B, k, D).values()) for D in ds) for ds in Ds]
        for i in range(args.warmup):
            graphs[i % R].launch(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % R].launch(stream)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t1) * 1e3 / args.steps
        mean_bytes = sum(step_bytes[i % R] for i in range(args.steps)) / args.steps
        assert all(c.read_flags() == 0 for c in ctxs)
        for g in graphs:
            g.close()
        # The same graphs in the other multi-launch forms, for comparison.
        by_mode = {default_mode(): round(ms * 1e3 / n_layers, 2)}
        for name in ("four_launches", "late_routing", "dense_routing", "ordered"):
            if name == default_mode() or name not in modes():
                continue
            for c in ctxs:
                c.set_mode(modes()[name])
            gm = [binding.Graph(ctxs, xd[r], B, k, outs, idxs, wts) for r in range(R)]
            for i in range(args.warmup):
                gm[i % R].launch(stream)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            for i in range(args.steps):
                gm[i % R].launch(stream)
            torch.cuda.synchronize()
            by_mode[name] = round((time.perf_counter() - t1) * 1e6 / args.steps / n_layers, 2)
            for g in gm:
                g.close()
            for c in ctxs:
                c.set_mode(binding.DEFAULT_MODE)
        # One layer's kernels, eager, events on each dispatch.
        kb = [kernel_bytes(d, B, k, Ds[r][0]) for r in range(R)]
        per_kernel = kernel_durations(ctxs[0], KERNELS_BF16, kb, [xd[r][0] for r in range(R)],
                                      k, outs[0], idxs[0], wts[0], max(args.steps, 20), stream,
                                      ctxs[0].last_dispatch().get("out_staged"))
        dom = max(KERNELS_BF16, key=lambda n: per_kernel[n]["us"])
        pk = per_kernel[dom]
        entry = {"batch": B, "us_per_8_layers": round(ms * 1e3, 2),
                 "us_per_layer": round(ms * 1e3 / n_layers, 2),
                 "tokens_per_s": round(B / (ms * 1e-3), 1),
                 "gbs": round(mean_bytes / (ms * 1e-3) / 1e9, 1),
                 "pct_hbm_peak": round(100 * mean_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                 "distinct_experts_mean": round(float(np.mean(Ds)), 1),
                 "us_per_layer_by_mode": by_mode,
                 "layer_kernels": per_kernel, "expert_path": expert_path(per_kernel),
                 "roofline": {"bound": "hbm", "kernel": pk["symbol"], "achieved": pk["gbs"],
                              "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": pk["frac"],
                              "traffic": load_traffic(pk["symbol"], f"k3_tp8_b{B}")},
                 "timed": f"{args.steps} launches of the eight-layer graph"}
        if B in oracle_batches and not args.no_cpu_baseline:
            log(f"[bench] timing the CPU oracle on one C4 layer at batch {B}")
            entry["cpu_oracle_one_layer"] = cpu_oracle_sampled(
                layers[0], [xs[r][0] for r in range(R)], float(np.mean([b["dense_in"] + b["w13"]
                                                                        + b["w2"] + b["out"]
                                                                        for b in kb])),
                args.sweep_cpu_seconds)
        log(f"[bench] C4 B={B}: {entry['us_per_layer']} us per layer, "
            f"{entry['pct_hbm_peak']} % of peak")
        res.append(entry)
        for c in ctxs:
            c.close()
        del xd, outs, idxs, wts
    del devs
    torch.cuda.empty_cache()
    return {"workload": "eight TP8-share layers (hidden 7168, latent 2048, 896 MXFP4 experts of "
                        "inter 256, top-16, shared 512) in one HIP graph",
            "batches": res}


def c0_summary(args):
    """The 64-expert layer at batch 1 (its weights fit the last-level cache):
    time per step of one-step graph launches, and the oracle's."""
    import numpy as np

    from sparse_moe_decode_router_amd import binding, synth

    layer = synth.make_layer(synth.TINY, 0)
    d = layer.dims
    dev = binding.DeviceLayer(layer)
    xs = [synth.make_tokens(d, 0, 1, draw=r) for r in range(8)]
    m = measure(dev, d, 1, d.top_k, xs, max(args.steps, 20), args.warmup, binding.DEFAULT_MODE)
    res = {"workload": "64-expert layer, batch 1 (hidden 512, latent 256, top-4, f32 router)",
           "us_per_step": round(m["ms"] * 1e3, 2), "us_p50": round(m["us_p50"], 2),
           "us_p10": round(m["us_p10"], 2), "us_p90": round(m["us_p90"], 2),
           "kernels": {n: v["us"] for n, v in m["per_kernel"].items()},
           "note": "working set cache-resident: latency only, no % of HBM peak"}
    if not args.no_cpu_baseline:
        import oracle
        oracle.lib()
        t0, n = time.perf_counter(), 0
        while time.perf_counter() - t0 < 2.0:
            oracle.moe_step(layer, xs[n % len(xs)], rounding="output")
            n += 1
        res["cpu_oracle_us_per_step"] = round((time.perf_counter() - t0) / n * 1e6, 1)
        res["cpu_oracle_cores"] = 1
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="k3_b1", choices=sorted(WORKLOADS) + ["c4_x8"])
    ap.add_argument("--rotate", type=int, default=32, help="distinct input batches cycled")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--sweep-cpu-seconds", type=float, default=4.0,
                    help="oracle time per batch-sweep configuration (all host cores)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true", help="skip the batch sweep of the K3 layer")
    ap.add_argument("--no-c0", action="store_true", help="skip the 64-expert layer's latency")
    ap.add_argument("--no-c4", action="store_true",
                    help="skip the eight-layer TP8-share graph at batch 1, 8 and 64")
    ap.add_argument("--modes", default=None,
                    help="comma-separated execution modes to run (default: all; the "
                         "library's default mode is always run)")
    args = ap.parse_args()
    global MODE_FILTER
    if args.modes:
        MODE_FILTER = set(args.modes.split(","))

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the decode step on one GPU only; multi-GPU runs "
              f"(--gpus {args.gpus}, WORLD_SIZE {world}) are not supported: the library has no "
              "multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from sparse_moe_decode_router_amd import binding, synth

    torch.cuda.set_device(0)
    if args.workload == "c4_x8":
        run_c4(args)
        return

    recipe_name, B, k, desc = WORKLOADS[args.workload]
    recipe = synth.RECIPES[recipe_name]
    d = recipe.dims
    seed = synth.TP8_STACK_SEED0 if recipe_name == "k3_tp8" else 0
    log(f"[bench] generating {args.workload} layer (seed {seed})")
    t0 = time.time()
    layer = synth.make_layer(recipe, seed)
    log(f"[bench] generated in {time.time() - t0:.1f} s; copying to the GPU")
    dev = binding.DeviceLayer(layer)
    xs = [synth.make_tokens(d, seed, B, draw=r) for r in range(args.rotate)]
    log(f"[bench] timing {args.workload}: {args.steps} steps")
    alt = {}
    for name, mode in modes().items():
        log(f"[bench] mode {name}")
        alt[name] = measure(dev, d, B, k, xs, args.steps, args.warmup, mode)
    m = alt[default_mode()]
    log(f"[bench] distinct experts per input {m['Ds']}; dispatch {m['dispatch']}")
    per_kernel = m["per_kernel"]
    dom = max(m["names"], key=lambda n: per_kernel[n]["us"])
    pk = per_kernel[dom]

    sweep = None
    if not args.no_sweep and recipe_name == "k3" and B == 1:
        sweep = [summary(args.workload, B, m, alt)]
        for name, bias_recipe, Bs, spec in SWEEP:
            bias = synth.make_bias(synth.RECIPES[bias_recipe], 0)
            if spec:
                xs_s = [synth.make_spec_tokens(d, 0, spec[0], spec[1], draw=r)
                        for r in range(args.rotate)]
            else:
                xs_s = [synth.make_tokens(d, 0, Bs, draw=r) for r in range(args.rotate)]
            n_s = max(50, args.steps // 2)
            log(f"[bench] sweep {name}")
            dvb = dev.with_bias(bias)
            alt_s = {n: measure(dvb, d, Bs, k, xs_s, n_s, args.warmup, mode)
                     for n, mode in modes().items()}
            sweep.append(summary(name, Bs, alt_s[default_mode()], alt_s))
            if not args.no_cpu_baseline:
                log(f"[bench] timing the CPU oracle on {name}")
                sweep[-1]["cpu_oracle"] = cpu_oracle_sampled(
                    dataclasses.replace(layer, bias=bias), xs_s,
                    float(np.mean(alt_s[default_mode()]["step_bytes"])), args.sweep_cpu_seconds)

    c0 = c4 = None
    if not args.no_c0:
        log("[bench] 64-expert layer at batch 1")
        c0 = c0_summary(args)
    if not args.no_c4 and recipe_name == "k3" and B == 1:
        del dev
        log("[bench] eight TP8-share layers in one graph")
        c4 = c4_summary(args)

    cpu = cpu_all = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(layer, xs, k, float(np.mean(m["step_bytes"])), args.cpu_seconds)
        log("[bench] timing the CPU oracle on all host cores")
        cpu_all = cpu_baseline_all_cores(layer, xs, k, float(np.mean(m["step_bytes"])),
                                         args.cpu_seconds)

    ms = m["ms"]
    line = {
        "metric": METRIC, "value": round(m["value"], 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {desc}", "batch": B, "top_k": k,
                   "hidden": d.hidden, "latent": d.latent, "experts": d.n_experts,
                   "expert_inter": d.expert_inter, "shared_inter": d.shared_inter,
                   "weights": "MXFP4 experts, bf16 dense", "rotating_inputs": args.rotate,
                   "parallelism": "1 GPU"},
        "us_per_step": round(ms * 1e3, 2),
        "us_p10": round(m["us_p10"], 2), "us_p50": round(m["us_p50"], 2),
        "us_p90": round(m["us_p90"], 2),
        "tokens_per_s": round(B / (ms * 1e-3), 1),
        "pct_hbm_peak": round(100 * m["value"] / HBM_PEAK_GBS, 2),
        "distinct_experts": m["Ds"],
        "mode": default_mode(),
        "expert_path": alt.get("four_launches", m)["expert_path"],
        "cold": m["cold"],
        "device": device_info(),
        "kernels": per_kernel,
        "timed": f"{m['n_launches_timed']} launches of one-step graphs (a graph per input, "
                 f"{args.rotate} inputs rotating) between two synchronisations; percentiles "
                 f"from events between {m['n_launches_percentiles']} further launches",
        "ms_per_step_eager": round(m["ms_eager"], 5),
        f"ms_per_step_{GRAPH_STEPS}_step_graphs": round(m["ms_graph_g"], 5),
        "modes": {n: {"us_per_step": round(x["ms"] * 1e3, 2), "gbs": round(x["value"], 1),
                      "kernels": x["per_kernel"]} for n, x in alt.items()},
        "roofline": {"bound": "hbm", "kernel": pk["symbol"], "achieved": pk["gbs"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": pk["frac"],
                     "traffic": load_traffic(pk["symbol"], args.workload)},
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all,
        "batch_sweep": sweep,
        "c0_tiny_b1": c0,
        "c4_x8": c4,
        "dispatch": m["dispatch"],
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
