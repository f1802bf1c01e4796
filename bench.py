#!/usr/bin/env python3
"""Throughput of the neural-memory store + retrieve on one MI355X.

One step = one ``retrieved, mem_state = memory(seq)`` call of the README-sized
memory (dim 384, hidden 1536, depth 2, chunk 64) on a (2, 1024) token batch:
tm_state_init (fresh memory) + tm_forward (16 chunks: forward, backward,
theta-weighted gradient reduction with the fused momentum / forgetting write,
and the retrieval of every query).  Inputs are seeded synthetic bf16 arrays,
resident in HBM before timing starts.  Prints one JSON line.

The timed region runs the steps as a caller would (same buffers every step,
so the library replays each call as a HIP graph).  The same steps then run
once more with HIP events recorded around every kernel launch on the launch
stream (events force direct launches), which gives each kernel class's mean
duration.  ``roofline`` describes the class that takes the most time:
algorithmic bytes (or flops) per launch / its mean event-timed duration.
``roofline.traffic`` is the HBM traffic per launch from the committed
rocprofv3 counter summary of that kernel, used only while the kernel source
still hashes to the value recorded there.  The fp64 CPU oracle is timed on
the host as ``cpu_baseline``.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "memory tokens/sec (store+retrieve) at dim 384, chunk 64; MFMA util %"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3
# the sources of the chunk-step kernels: the device helpers, then the kernels
KERNEL_SOURCES = [os.path.join(ROOT, "test_trained_neural_amd", "csrc", f) for f in ("tm_device.h", "tm_kernels.hip")]


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# Algorithmic work of each launch (bytes a kernel must move at least once, and
# the flops of its products), for one tm_forward call of T tokens.

def first_layer_launches(wl, ns, T):
    """Bytes of every launch of the chunk-step kernel (chunk steps 0..C).

    Step c updates W_0 for chunk c-1 (M_0, S_0 read and written in fp32; its
    bf16 forward copy written on the call's last update only; the keys of
    chunk c-1, layer 1's Delta and SiLU' of chunk c-1 read; the in-place
    backward's rows of W_1 are the ones the same launch updates, counted
    there) and runs chunk c's first-layer forward of [queries of chunk c-1;
    keys of chunk c] (input rows read; activations, SiLU' and the transposed
    activations written).  The same launch carries chunk c-1's update of
    layers 1..L-1 (update_launch_bytes)."""
    e = 2 if wl.dtype == "bf16" else 4
    b, d = wl.chunk, wl.dim
    dims = wl.layer_dims()
    h1 = dims[0][1]
    C = T // b
    out = []
    for c in range(C + 1):
        upd, nq, nk = c >= 1, (b if c >= 1 else 0), (b if c < C else 0)
        x = 0
        if upd:
            x += 16 * d * h1 + d * b * e + 8 * b
            if c == C:
                x += 2 * d * h1
            if wl.depth >= 2:
                x += b * dims[1][1] * e + b * h1 * 4
            else:
                x += 2 * h1 * b * e
        else:
            x += (2 if wl.dtype == "bf16" else 4) * d * h1      # the layer's weights, read once
        x += (nq + nk) * d * e
        if wl.depth >= 2:
            x += (nq + nk) * h1 * e + nk * h1 * 4 + nk * h1 * e
        else:
            x += nq * d * 4 + nk * d * e + 2 * h1 * nk * e
        out.append(ns * x + (update_launch_bytes(wl, ns) if upd and wl.depth >= 2 else 0))
    return out


def update_launch_bytes(wl, ns):
    """Bytes of chunk c-1's update of layers 1..L-1 in one step launch: M, S
    read and written and the bf16 copy written (18 B per weight), the
    transposed activations and the two theta-weighted delta operands read."""
    e = 2 if wl.dtype == "bf16" else 4
    b = wl.chunk
    x = 0
    for l, (din, dout) in enumerate(wl.layer_dims()):
        if l == 0:
            continue
        x += 18 * din * dout + din * b * e + 2 * dout * b * e
    return ns * x


def fwd_flops(wl, ns, T):
    """Flops of the forward products of layers 1.. (the first layer's run in
    the step kernel): every key row once and every query row once."""
    return 2 * 2 * ns * T * sum(a * b for a, b in wl.layer_dims()[1:])


def bwd_flops(wl, ns, T):
    return 2 * ns * T * sum(a * b for a, b in wl.layer_dims()[2:])


def token_read_flops(wl, ns, T):
    """Flops of the per-token read's products (tm_forward_ex, read per
    token) over a call of T tokens: per chunk and stream, the scores
    2 b^2 d_in of every layer, the query rows' products with M and S
    (4 b d_in d_out) and the correction (2 b^2 d_out) of every layer, and
    layer 0's Delta (2 b d_1 h, or 2 b d d for depth 1)."""
    b = wl.chunk
    dims = wl.layer_dims()
    per = sum(2 * b * b * a + 4 * b * a * o + 2 * b * b * o for a, o in dims)
    per += 2 * b * dims[1][1] * dims[0][1] if len(dims) >= 2 else 2 * b * dims[0][0] * dims[0][1]
    return per * ns * (T // b)


def project_flops(wl, Bn, T):
    """Flops of the input side's projection kernel: k, v, q and the three
    gates from every token's model vector."""
    D, HD = wl.model_dim, wl.heads * wl.dim
    return 2 * Bn * T * D * (3 * HD + 3 * wl.heads)


def mfma_roofline(kind_flops, ms, n, dtype, kernel):
    """An MFMA roofline entry from event-timed launches of one class."""
    peak = BF16_PEAK_TFLOPS if dtype == "bf16" else FP32_PEAK_TFLOPS
    achieved = kind_flops / (ms / 1e3) / 1e12
    return {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
            "kernel": kernel, "launches": n, "avg_us": ms * 1e3 / max(n, 1),
            "timing": "HIP events recorded with each launch's own dispatch, second pass of the same steps"}


def read_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, or None."""
    path = os.path.join(ROOT, "profiles", "%s_%s_pmc.md" % (kernel, workload))
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel source sha256\[:16\][^`]*`([0-9a-f]+)`", text)
    t = re.search(r"HBM bytes per launch: ([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_source_hash():
        return None
    return float(t.group(1))


def host_info():
    """The host the CPU baselines ran on: logical CPUs and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


def cpu_baseline(wl, params, ci, min_seconds=10.0):
    """The fp64 oracle on a bounded sample of the same workload: the whole
    step (store + retrieve of every stream's tokens from the initial state),
    repeated until at least min_seconds of host time have been spent."""
    from oracle import tmref
    from test_trained_neural_amd import inputs as I
    streams = wl.batch * wl.heads
    tokens = wl.tokens_per_call
    threads = min(os.cpu_count() or 1, streams)
    reps = 0
    t0 = time.perf_counter()
    while True:
        st = I.initial_state(wl, params)
        tmref.forward(wl.dim, wl.depth, wl.expansion, wl.chunk, st, ci.k[:, :tokens], ci.v[:, :tokens],
                      ci.theta[:, :tokens], ci.eta[:, :tokens], ci.alpha[:, :tokens], q=ci.q[:, :tokens],
                      n_threads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": reps * wl.batch * tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%s: %d x the whole step (%d streams x %d tokens, store + retrieve from the initial "
                      "state), fp64 C oracle, one thread per stream, %.1f s" % (wl.name, reps, streams, tokens, dt),
            "host": host_info()}


def scan_bytes(wl, ns, T):
    """Bytes of the coefficient scan over a call of T tokens: the three gates
    read and c, d written (20 B per token), the chunk scalars (16 B per
    chunk), the keys and queries read once (2 d e) and written packed (rows
    of both and the keys transposed, 3 d e), per stream."""
    e = 2 if wl.dtype == "bf16" else 4
    return ns * (T * (20 + 5 * wl.dim * e) + (T // wl.chunk) * 16)


def other_workload(name, steps, calls=None, read=None, oracle=False, kernel_roof=False, oracle_tokens=None):
    """Throughput of another workload (tokens/s): state init + its calls in
    order, inputs resident in HBM, graph replay (each call's buffers repeat
    across steps).  calls: how many of the workload's calls to run (a prefix
    of the stream; None = all).  read: the queries' read order
    (tm_forward_ex), None for tm_forward."""
    import torch
    import test_trained_neural_amd as T
    from test_trained_neural_amd import inputs as I
    wl = I.WORKLOADS[name]
    n_calls = wl.calls if calls is None else calls
    Bn, Tn, H, d = wl.batch, wl.tokens_per_call, wl.heads, wl.dim
    params = I.make_params(wl, 0)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    bufs = []
    for j in range(n_calls):
        ci = I.make_call(wl, params, j, 0)
        bufs.append([torch.from_numpy(x).to(dev).to(tdt) for x in (ci.k, ci.v, ci.q)] +
                    [torch.from_numpy(x).to(dev) for x in (ci.theta, ci.eta, ci.alpha)])
    init = torch.from_numpy(params.init_weights).to(dev)
    ctx = T.tm_create(d, wl.depth, wl.expansion, wl.chunk)
    state = torch.empty(T.tm_state_bytes(ctx, Bn, H), dtype=torch.uint8, device=dev)
    ws = torch.empty(T.tm_workspace_bytes(ctx, Bn, H, Tn), dtype=torch.uint8, device=dev)
    y = torch.empty((Bn, Tn, H, d), dtype=torch.float32, device=dev)

    def step():
        T.tm_state_init(ctx, state, Bn, H, init)
        for (k, v, q, th, et, al) in bufs:
            if read is None:
                T.tm_forward(ctx, state, k, v, q, th, et, al, y, ws)
            else:
                T.tm_forward_ex(ctx, state, k, v, q, th, et, al, y, ws, read)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    tokens = Bn * Tn * n_calls
    out = {"tokens_per_s": tokens / dt, "ms_per_step": dt * 1e3, "steps": steps,
           "step": "tm_state_init + %d %s calls of (%d, %d) tokens, %d heads" % (
               n_calls, "tm_forward" if read is None else "tm_forward_ex(read=%d)" % read, Bn, Tn, H),
           "sample": "whole workload" if n_calls == wl.calls else "first %d of %d calls" % (n_calls, wl.calls)}
    if kernel_roof:
        # the coefficient scan and the chunk-step kernel, event-timed in a
        # second pass: their HBM rooflines at this workload's scale.  The
        # pass runs the calls as one chunk chain: with two batch groups the
        # launches of the two chains overlap, and the durations of
        # overlapping launches give no rate of either
        T.tm_store_groups_enable(0)
        T.tm_timing_enable((1 << T.K_SCAN) | (1 << T.K_FIRST))
        T.tm_timing_read(T.K_SCAN)
        T.tm_timing_read(T.K_FIRST)
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        T.tm_timing_enable(0)
        T.tm_store_groups_enable(1)
        out["kernels_timed_as"] = "one chunk chain (the throughput pass: two batch groups, overlapping)"
        kin = {}
        for nm, cls, kern, amount in (
                ("scan", T.K_SCAN, "scan_kernel", scan_bytes(wl, Bn * H, Tn) * n_calls),
                ("first", T.K_FIRST, "first_layer_kernel", sum(first_layer_launches(wl, Bn * H, Tn)) * n_calls)):
            ms, n = T.tm_timing_read(cls)
            gbs = amount * steps / (ms / 1e3) / 1e9
            kin[nm] = {"kernel": kern, "launches_per_step": n / steps, "us_per_launch": ms * 1e3 / max(n, 1),
                       "bytes_per_launch": amount * steps / max(n, 1), "GB_per_s": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}
        out["kernels"] = kin
    if read == T.TM_READ_PER_TOKEN:
        # the read's own launches, event-timed in a second pass
        T.tm_timing_enable(1 << T.K_TOKEN_READ)
        T.tm_timing_read(T.K_TOKEN_READ)
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        T.tm_timing_enable(0)
        ms, n = T.tm_timing_read(T.K_TOKEN_READ)
        out["roofline"] = mfma_roofline(token_read_flops(wl, Bn * H, Tn) * n_calls * steps, ms, n, wl.dtype,
                                        "r3_score_kernel + r3_layer_kernel")
    T.tm_destroy(ctx)
    if oracle:
        # the oracle on the workload's first call (or its first oracle_tokens
        # tokens), in the same read order, one thread per stream
        from oracle import tmref
        on = Tn if oracle_tokens is None else min(oracle_tokens, Tn)
        ci = I.make_call(wl, params, 0, 0, tokens=on)
        st = I.initial_state(wl, params)
        nt = min(os.cpu_count() or 1, Bn * H)
        t1 = time.perf_counter()
        tmref.forward(wl.dim, wl.depth, wl.expansion, wl.chunk, st, ci.k, ci.v, ci.theta, ci.eta, ci.alpha,
                      q=ci.q, n_threads=nt, read={None: "after", 1: "before", 2: "token"}[read])
        odt = time.perf_counter() - t1
        out["cpu_baseline"] = {"value": Bn * on / odt, "unit": "tokens/s", "cores": nt, "kind": "oracle",
                               "sample": "%s: %s (%d streams x %d tokens) from the initial state, fp64 C oracle, one "
                                         "thread per stream, %.1f s" % (wl.name, "one call" if on == Tn else
                                                                       "the first call's first %d tokens" % on,
                                                                       Bn * H, on, odt), "host": host_info()}
    return out


def backward_bytes(wl, ns, T):
    """Bytes of tm_backward's state-streaming launches over a call of T
    tokens, per layer and chunk: the recompute's write (M_0, S_0 read, M_end,
    S_end written: 16 B per weight; the key rows' layer input, Delta and the
    coefficients read) and the adjoint update (Mbar, Sbar read and written,
    M_0, S_0 read: 24 B per weight; the products' operands read)."""
    b = wl.chunk
    e = 2 if wl.dtype == "bf16" else 4
    per = 0
    for l, (din, dout) in enumerate(wl.layer_dims()):
        eh = e if l == 0 else 4
        per += 16 * din * dout + b * din * eh + b * dout * 4 + 8 * b
        per += 24 * din * dout + b * din * eh + b * dout * 4 + (8 * b * (din + dout) // 2 if l >= 1 else 0)
    return ns * (T // b) * per


def backward_flops(wl, ns, T):
    """Flops of tm_backward's other products over a call of T tokens (per
    chunk and stream: the key rows' forward and backward, the queries'
    forward, backprop and weight gradient, the surprise's adjoint (two
    accumulators, both directions), back through the key rows' backward and
    forward)."""
    b = wl.chunk
    P = wl.params
    dims = wl.layer_dims()
    P0, PL = dims[0][0] * dims[0][1], dims[-1][0] * dims[-1][1]
    per = 2 * b * (P + (P - P0) + (P - PL) + P + P + 2 * P + 2 * P + (P - P0) + P)
    return ns * (T // b) * per


def backward_line(name, steps, oracle=False):
    """tm_backward over the workload's first call (the gradient of a random
    outer loss on y; no gradient on the state after the call), inputs
    resident in HBM, graph replay; tokens/s, the dominant class's roofline,
    and the backward oracle on a bounded sample."""
    import numpy as np
    import torch
    import test_trained_neural_amd as T
    from test_trained_neural_amd import inputs as I
    wl = I.WORKLOADS[name]
    Bn, Tn, H, d = wl.batch, wl.tokens_per_call, wl.heads, wl.dim
    ns = Bn * H
    params = I.make_params(wl, 0)
    ci = I.make_call(wl, params, 0, 0)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    k, v, q = (torch.from_numpy(x).to(dev).to(tdt) for x in (ci.k, ci.v, ci.q))
    th, et, al = (torch.from_numpy(x).to(dev) for x in (ci.theta, ci.eta, ci.alpha))
    dy_np = np.random.default_rng(11).standard_normal(ci.k.shape).astype(np.float32)
    dy = torch.from_numpy(dy_np).to(dev)
    ctx = T.tm_create(d, wl.depth, wl.expansion, wl.chunk)
    state = torch.empty(T.tm_state_bytes(ctx, Bn, H), dtype=torch.uint8, device=dev)
    T.tm_state_init(ctx, state, Bn, H, torch.from_numpy(params.init_weights).to(dev))
    ws = torch.empty(T.tm_backward_workspace_bytes(ctx, Bn, H, Tn), dtype=torch.uint8, device=dev)
    dstate = torch.zeros((ns, 2 * wl.params), dtype=torch.float32, device=dev)
    dk, dv, dq = (torch.empty((Bn, Tn, H, d), dtype=torch.float32, device=dev) for _ in range(3))
    dth, det, dal = (torch.empty((Bn, Tn, H), dtype=torch.float32, device=dev) for _ in range(3))

    def step():
        dstate.zero_()
        T.tm_backward(ctx, state, k, v, q, th, et, al, dy, dstate, dk, dv, dq, dth, det, dal, ws)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    out = {"tokens_per_s": Bn * Tn / dt, "ms_per_step": dt * 1e3, "steps": steps,
           "step": "tm_backward of one tm_forward call of (%d, %d) tokens from the initial state (dstate "
                   "cleared first): recompute with every chunk-start state kept, reverse sweep, gate gradients"
                   % (Bn, Tn)}
    T.tm_timing_enable((1 << T.K_BACKWARD_STATE) | (1 << T.K_BACKWARD_REST))
    T.tm_timing_read(T.K_BACKWARD_STATE)
    T.tm_timing_read(T.K_BACKWARD_REST)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    T.tm_timing_enable(0)
    ms_s, n_s = T.tm_timing_read(T.K_BACKWARD_STATE)
    ms_r, n_r = T.tm_timing_read(T.K_BACKWARD_REST)
    by = backward_bytes(wl, ns, Tn) * steps
    fl = backward_flops(wl, ns, Tn) * steps
    gbs = by / (ms_s / 1e3) / 1e9
    tfl = fl / (ms_r / 1e3) / 1e12
    out["kernels"] = {
        "state_streaming": {"kernel": "bgemm_kernel (the write and adjoint-update epilogues)",
                            "launches_per_step": n_s / steps, "ms_per_step": ms_s / steps,
                            "us_per_launch": ms_s * 1e3 / max(n_s, 1), "GB_per_s": gbs, "hbm_frac": gbs / HBM_PEAK_GBS},
        "products_and_rest": {"kernel": "bgemm_kernel (other epilogues), belem_kernel, bcoef_kernel, export_kernel",
                              "launches_per_step": n_r / steps, "ms_per_step": ms_r / steps,
                              "us_per_launch": ms_r * 1e3 / max(n_r, 1), "tflops": tfl,
                              "fp32_frac": tfl / FP32_PEAK_TFLOPS},
    }
    if ms_s >= ms_r:
        out["roofline"] = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": gbs / HBM_PEAK_GBS, "kernel": "bgemm_kernel (state streaming)",
                           "launches": n_s, "avg_us": ms_s * 1e3 / max(n_s, 1), "bytes_per_launch": by / max(n_s, 1)}
    else:
        out["roofline"] = {"bound": "mfma", "achieved": tfl, "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": tfl / FP32_PEAK_TFLOPS, "kernel": "bgemm_kernel (products, fp32 matrix cores)",
                           "launches": n_r, "avg_us": ms_r * 1e3 / max(n_r, 1), "flops_per_launch": fl / max(n_r, 1)}
    out["roofline"]["timing"] = "HIP events recorded with each launch's own dispatch, second pass of the same steps"
    T.tm_destroy(ctx)
    if oracle:
        # the backward oracle on one stream's first 128 tokens, repeated for
        # at least 10 s
        import torch as _t
        from oracle import backward as BW
        n = min(128, Tn)
        sub = lambda a: np.ascontiguousarray(a[:1, :n, :1])
        st = I.initial_state(wl, params, batch=1)[:1]
        reps, t1 = 0, time.perf_counter()
        while True:
            BW.forward_backward(wl.dim, wl.depth, wl.expansion, wl.chunk, st, sub(ci.k), sub(ci.v), sub(ci.q),
                                sub(ci.theta), sub(ci.eta), sub(ci.alpha), sub(dy_np))
            reps += 1
            odt = time.perf_counter() - t1
            if odt >= 10.0:
                break
        out["cpu_baseline"] = {"value": reps * n / odt, "unit": "tokens/s", "cores": _t.get_num_threads(),
                               "kind": "oracle", "host": host_info(),
                               "sample": "%s backward: %d x one stream's first %d tokens (float64 autograd through "
                                         "the literal recurrence, PyTorch CPU), %.1f s" % (wl.name, reps, n, odt)}
    return out


def retrieval(name, steps, oracle=False):
    """Read-only retrieval (tm_retrieve: every query through the current
    memory, no write) of the workload's first call's queries, after storing
    that call; tokens/s and the products' MFMA roofline."""
    import torch
    import test_trained_neural_amd as T
    from test_trained_neural_amd import inputs as I
    wl = I.WORKLOADS[name]
    Bn, Tn, H, d = wl.batch, wl.tokens_per_call, wl.heads, wl.dim
    params = I.make_params(wl, 0)
    ci = I.make_call(wl, params, 0, 0)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    k, v, q = (torch.from_numpy(x).to(dev).to(tdt) for x in (ci.k, ci.v, ci.q))
    th, et, al = (torch.from_numpy(x).to(dev) for x in (ci.theta, ci.eta, ci.alpha))
    ctx = T.tm_create(d, wl.depth, wl.expansion, wl.chunk)
    state = torch.empty(T.tm_state_bytes(ctx, Bn, H), dtype=torch.uint8, device=dev)
    ws = torch.empty(T.tm_workspace_bytes(ctx, Bn, H, Tn), dtype=torch.uint8, device=dev)
    y = torch.empty((Bn, Tn, H, d), dtype=torch.float32, device=dev)
    T.tm_state_init(ctx, state, Bn, H, torch.from_numpy(params.init_weights).to(dev))
    T.tm_store(ctx, state, k, v, th, et, al, ws)

    def step():
        T.tm_retrieve(ctx, state, q, y, ws)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    T.tm_timing_enable(1 << T.K_FWD)
    T.tm_timing_read(T.K_FWD)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    T.tm_timing_enable(0)
    ms, n = T.tm_timing_read(T.K_FWD)
    flops = 2 * Bn * H * Tn * sum(a * b for a, b in wl.layer_dims()) * steps
    out = {"tokens_per_s": Bn * Tn / dt, "ms_per_step": dt * 1e3, "steps": steps,
           "step": "tm_retrieve of (%d, %d) queries through the memory after storing them" % (Bn, Tn),
           "roofline": mfma_roofline(flops, ms, n, wl.dtype, retrieve_kernel(wl, Tn))}
    T.tm_destroy(ctx)
    if oracle:
        from oracle import tmref
        st = I.initial_state(wl, params)
        tmref.forward(wl.dim, wl.depth, wl.expansion, wl.chunk, st, ci.k, ci.v, ci.theta, ci.eta, ci.alpha)
        nt = min(os.cpu_count() or 1, Bn * H)
        t1 = time.perf_counter()
        tmref.retrieve(wl.dim, wl.depth, wl.expansion, st, ci.q, n_threads=nt)
        odt = time.perf_counter() - t1
        out["cpu_baseline"] = {"value": Bn * Tn / odt, "unit": "tokens/s", "cores": nt, "kind": "oracle",
                               "sample": "%s: retrieve of one call's queries (%d streams x %d tokens), fp64 C "
                                         "oracle, %.2f s" % (wl.name, Bn * H, Tn, odt), "host": host_info()}
    return out


def retrieve_kernel(wl, n_tokens):
    """The kernel tm_retrieve launches for this memory: both layers in one
    launch (depth 2, bf16, width <= 128, hidden a multiple of 64), else one
    launch per layer, tiled from 256 rows a pass."""
    h = wl.dim * wl.expansion
    if wl.dtype == "bf16" and wl.depth == 2 and wl.dim <= 128 and h % 64 == 0:
        return "mlp2_kernel"
    return "rows_kernel" if wl.dtype == "bf16" and min(n_tokens, 2048) >= 256 else "gemm_kernel"


def input_side(name, steps, oracle=False):
    """The input side (tm_project: x -> k, v, q and the gates, 4-tap
    convolution) alone and chained with the memory step (tm_project +
    tm_state_init + tm_forward), on the workload's first call; tokens/s."""
    import numpy as np
    import torch
    import test_trained_neural_amd as T
    from test_trained_neural_amd import inputs as I
    wl = I.WORKLOADS[name]
    params = I.make_params(wl, 0)
    pi = I.make_prologue(wl, params, 0, 0, conv_len=4)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    Bn, Tn, H, d = wl.batch, wl.tokens_per_call, wl.heads, wl.dim
    x = torch.from_numpy(pi.x).to(dev).to(tdt).contiguous()
    w = torch.from_numpy(np.ascontiguousarray(pi.w_kvq.transpose(0, 2, 1))).to(dev).to(tdt).contiguous()
    conv = torch.from_numpy(pi.conv).to(dev).contiguous()
    wg = torch.from_numpy(np.ascontiguousarray(pi.w_gate.transpose(0, 2, 1))).to(dev).contiguous()
    gb = torch.from_numpy(pi.gate_bias).to(dev).contiguous()
    hist = torch.zeros((Bn, 3, 3, H * d), dtype=torch.float32, device=dev)
    k, v, q = (torch.empty((Bn, Tn, H, d), dtype=tdt, device=dev) for _ in range(3))
    g = [torch.empty((Bn, Tn, H), dtype=torch.float32, device=dev) for _ in range(3)]
    ctx = T.tm_create(d, wl.depth, wl.expansion, wl.chunk)
    state = torch.empty(T.tm_state_bytes(ctx, Bn, H), dtype=torch.uint8, device=dev)
    ws = torch.empty(T.tm_workspace_bytes(ctx, Bn, H, Tn), dtype=torch.uint8, device=dev)
    y = torch.empty((Bn, Tn, H, d), dtype=torch.float32, device=dev)
    init = torch.from_numpy(params.init_weights).to(dev)

    def project():
        T.tm_project(ctx, x, w, conv, wg, gb, hist, k, v, q, g[0], g[1], g[2], H)

    def chain():
        project()
        T.tm_state_init(ctx, state, Bn, H, init)
        T.tm_forward(ctx, state, k, v, q, g[0], g[1], g[2], y, ws)

    out = {}
    for nm, fn in (("input_side", project), ("from_tokens", chain)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        out[nm] = {"tokens_per_s": Bn * Tn / dt, "ms_per_step": dt * 1e3, "steps": steps}
    # the projection kernel, event-timed in a second pass
    T.tm_timing_enable(1 << T.K_PROJECT)
    T.tm_timing_read(T.K_PROJECT)
    for _ in range(steps):
        project()
    torch.cuda.synchronize()
    T.tm_timing_enable(0)
    ms, n = T.tm_timing_read(T.K_PROJECT)
    out["input_side"]["roofline"] = mfma_roofline(project_flops(wl, Bn, Tn) * steps, ms, n, wl.dtype,
                                                  "project_kernel")
    if oracle:
        from threadpoolctl import threadpool_limits
        from oracle import prologue
        with threadpool_limits(1):          # numpy's BLAS on one thread, as reported
            t1 = time.perf_counter()
            prologue.project(pi.x, pi.w_kvq, pi.conv, pi.w_gate, pi.gate_bias, H)
            odt = time.perf_counter() - t1
        out["input_side"]["cpu_baseline"] = {
            "value": Bn * Tn / odt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "%s input side: one call (%d x %d tokens of width %d), fp64 numpy oracle, %.2f s" % (
                wl.name, Bn, Tn, wl.model_dim, odt), "host": host_info()}
    out["input_side"]["step"] = "tm_project of (%d, %d) tokens of width %d, 4-tap convolution" % (Bn, Tn, wl.model_dim)
    out["from_tokens"]["step"] = "tm_project + tm_state_init + tm_forward of (%d, %d) tokens" % (Bn, Tn)
    T.tm_destroy(ctx)
    return out


def mac_wiring(name, steps, seg=128, n_persist=4, oracle=False):
    """The memory's side of memory as a context over the workload's first
    call, segment by segment from the initial state: the segment's
    projections (tm_project), its queries read before the write
    (tm_retrieve), the window (tm_mac_window), the caller's attention (here
    the segment's own rows passed through, one copy), the output's
    projections, its write (tm_store) and read (tm_retrieve), and the gate
    (tm_mac_gate); tokens/s, and the window kernel's HBM roofline."""
    import numpy as np
    import torch
    import test_trained_neural_amd as T
    from test_trained_neural_amd import inputs as I
    wl = I.WORKLOADS[name]
    params = I.make_params(wl, 0)
    pi = I.make_prologue(wl, params, 0, 0, conv_len=4)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    Bn, Tn, H, d = wl.batch, wl.tokens_per_call, wl.heads, wl.dim
    D, S, P = H * d, seg, n_persist
    assert Tn % S == 0 and S % wl.chunk == 0
    x = torch.from_numpy(pi.x).to(dev).to(tdt).contiguous()
    w = torch.from_numpy(np.ascontiguousarray(pi.w_kvq.transpose(0, 2, 1))).to(dev).to(tdt).contiguous()
    conv = torch.from_numpy(pi.conv).to(dev).contiguous()
    wg = torch.from_numpy(np.ascontiguousarray(pi.w_gate.transpose(0, 2, 1))).to(dev).contiguous()
    gb = torch.from_numpy(pi.gate_bias).to(dev).contiguous()
    pers = torch.from_numpy(np.random.default_rng(3).standard_normal((P, D)).astype(np.float32)).to(dev).to(tdt)
    hx = torch.zeros((Bn, 3, 3, D), dtype=torch.float32, device=dev)
    hy = torch.zeros_like(hx)
    mem = T.NeuralMemory(d, wl.depth, wl.expansion, wl.chunk, device=dev)
    init = torch.from_numpy(params.init_weights).to(dev)
    st = mem.init_state(Bn, H, init)
    segs = [x[:, i * S:(i + 1) * S].contiguous() for i in range(Tn // S)]

    def attention(window):
        return window[:, P + S:]

    def step():
        hx.zero_()
        hy.zero_()
        T.tm_state_init(mem.ctx, st.buf, Bn, H, init)
        for xs in segs:
            T.mac_segment(mem, st, xs, pers, attention, w, conv, wg, gb, H, hx, hy)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    out = {"tokens_per_s": Bn * Tn / dt, "ms_per_step": dt * 1e3, "steps": steps}
    # every kernel class of the step, event-timed in a second pass (direct
    # launches): where a step's time goes, and what the launches leave to
    # the host (the ctypes calls and launch gaps)
    cls = {"project_kernel": T.K_PROJECT, "scan_kernel": T.K_SCAN, "first_layer_kernel": T.K_FIRST,
           "gemm_kernel": T.K_FWD, "mac_window/gate_kernel": T.K_MAC}
    T.tm_timing_enable(sum(1 << c for c in cls.values()))
    for c in cls.values():
        T.tm_timing_read(c)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    T.tm_timing_enable(0)
    brk = {}
    for nm, c in cls.items():
        ms, n = T.tm_timing_read(c)
        brk[nm] = {"ms_per_step": ms / steps, "launches_per_step": n / steps, "us_per_launch": ms * 1e3 / max(n, 1)}
    kern_ms = sum(v["ms_per_step"] for v in brk.values())
    out["kernels"] = brk
    out["host_share"] = {"kernel_ms_per_step": kern_ms, "step_ms": dt * 1e3,
                         "host_frac": max(0.0, 1.0 - kern_ms / (dt * 1e3)),
                         "note": "1 - (summed event-timed kernel time) / (graph-replay step time)"}
    dom = max(brk, key=lambda nm: brk[nm]["ms_per_step"])
    nseg = Tn // S
    if dom == "project_kernel":
        flops = project_flops(wl, Bn, S) * 2 * nseg * steps
        out["roofline"] = mfma_roofline(flops, brk[dom]["ms_per_step"] * steps, brk[dom]["launches_per_step"] * steps,
                                        wl.dtype, dom)
    elif dom == "gemm_kernel":
        Pw = wl.params
        flops = (2 * 2 * Bn * H * S * Pw + 2 * Bn * H * S * sum(a * b for a, b in wl.layer_dims()[1:])) * nseg * steps
        out["roofline"] = mfma_roofline(flops, brk[dom]["ms_per_step"] * steps, brk[dom]["launches_per_step"] * steps,
                                        wl.dtype, dom)
    # the window kernel alone, event-timed
    rec = torch.randn((Bn, S, D), dtype=torch.float32, device=dev)
    win = torch.empty((Bn, P + 2 * S, D), dtype=tdt, device=dev)
    T.tm_timing_enable(1 << T.K_MAC)
    T.tm_timing_read(T.K_MAC)
    n_win = 20 * steps
    for _ in range(n_win):
        T.tm_mac_window(pers, rec, segs[0], win)
    torch.cuda.synchronize()
    T.tm_timing_enable(0)
    ms, n = T.tm_timing_read(T.K_MAC)
    es = 2 if wl.dtype == "bf16" else 4
    per_launch = Bn * S * D * 4 + Bn * S * D * es + P * D * es + Bn * (P + 2 * S) * D * es
    achieved = per_launch * n / (ms / 1e3) / 1e9
    win_roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": "mac_window_kernel",
                "launches": n, "avg_us": ms * 1e3 / max(n, 1), "bytes_per_launch": per_launch,
                "timing": "HIP events recorded with each launch's own dispatch"}
    out["window_kernel"] = win_roof
    out.setdefault("roofline", win_roof)
    if oracle:
        from threadpoolctl import threadpool_limits
        from oracle import mac, prologue, tmref
        xs = pi.x[:, :S].astype(np.float64)
        ref = I.initial_state(wl, params)
        lim = threadpool_limits(1)          # numpy's BLAS on one thread, as reported
        t1 = time.perf_counter()
        _, _, q, _, _, _, _ = prologue.project(xs, pi.w_kvq, pi.conv, pi.w_gate, pi.gate_bias, H)
        r = tmref.retrieve(d, wl.depth, wl.expansion, ref, q.astype(np.float32), n_threads=1)
        win_o = mac.window(pers.float().cpu().numpy(), r.reshape(Bn, S, D), xs, wl.dtype == "bf16")
        y = win_o[:, P + S:]
        k2, v2, q2, th, et, al, _ = prologue.project(y, pi.w_kvq, pi.conv, pi.w_gate, pi.gate_bias, H)
        tmref.forward(d, wl.depth, wl.expansion, wl.chunk, ref, k2, v2, th, et, al, n_threads=1)
        m2 = tmref.retrieve(d, wl.depth, wl.expansion, ref, q2.astype(np.float32), n_threads=1)
        mac.gate(y, m2.reshape(Bn, S, D))
        odt = time.perf_counter() - t1
        lim.restore_original_limits()
        out["cpu_baseline"] = {
            "value": Bn * S / odt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "%s memory-as-context wiring: the first segment (%d x %d tokens), fp64 oracles "
                      "(input side, memory, wiring), one thread, %.2f s" % (wl.name, Bn, S, odt),
            "host": host_info()}
    out["step"] = ("%d segments of %d tokens x %d streams, %d persistent tokens: tm_project, tm_retrieve, "
                   "tm_mac_window, pass-through attention, tm_project, tm_store, tm_retrieve, tm_mac_gate"
                   % (Tn // S, S, Bn, P))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mlp384")
    ap.add_argument("--read", choices=("after", "before", "token"), default="after",
                    help="the queries' read order (after the chunk's write: tm_forward, the headline step)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other", action="store_true", help="skip the other workloads' throughput")
    ap.add_argument("--lines", default=None,
                    help="comma-separated names of the other workloads' lines to run (default: all)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="finish with a plain 256 MiB device copy (scale reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the memory streams of this workload are independent "
              "and a multi-GPU run would only shard them; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import test_trained_neural_amd as T
    from test_trained_neural_amd import inputs as I

    wl = I.WORKLOADS[args.workload]
    Bn, Tn, H, d = wl.batch, wl.tokens_per_call, wl.heads, wl.dim
    ns = Bn * H
    params = I.make_params(wl, 0)
    ci = I.make_call(wl, params, 0, 0)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    k = torch.from_numpy(ci.k).to(dev).to(tdt)
    v = torch.from_numpy(ci.v).to(dev).to(tdt)
    q = torch.from_numpy(ci.q).to(dev).to(tdt)
    th = torch.from_numpy(ci.theta).to(dev)
    et = torch.from_numpy(ci.eta).to(dev)
    al = torch.from_numpy(ci.alpha).to(dev)
    init = torch.from_numpy(params.init_weights).to(dev)
    ctx = T.tm_create(d, wl.depth, wl.expansion, wl.chunk)
    state = torch.empty(T.tm_state_bytes(ctx, Bn, H), dtype=torch.uint8, device=dev)
    ws = torch.empty(T.tm_workspace_bytes(ctx, Bn, H, Tn), dtype=torch.uint8, device=dev)
    y = torch.empty((Bn, Tn, H, d), dtype=torch.float32, device=dev)

    read = {"after": None, "before": T.TM_READ_BEFORE_WRITE, "token": T.TM_READ_PER_TOKEN}[args.read]

    def step():
        T.tm_state_init(ctx, state, Bn, H, init)
        if read is None:
            T.tm_forward(ctx, state, k, v, q, th, et, al, y, ws)
        else:
            T.tm_forward_ex(ctx, state, k, v, q, th, et, al, y, ws, read)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    nf, pos = T.tm_state_check(ctx, state, Bn, H)
    if nf:
        print("warning: non-finite memory state", file=sys.stderr)

    # timed region: the steps as a caller runs them (repeated buffers, so the
    # chunk loop replays as a HIP graph)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # per-step spread: the same steps again, each between two events on the
    # stream (graph replay as above)
    step_ms = []
    for _ in range(args.steps):
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ea.record()
        step()
        eb.record()
        eb.synchronize()
        step_ms.append(ea.elapsed_time(eb))
    step_ms.sort()

    # the same steps again with HIP events around every launch (events force
    # direct launches): per-kernel durations for the roofline, as one chunk
    # chain (a call of two batch groups overlaps the two chains' launches,
    # and the durations of overlapping launches give no rate of either)
    groups = Bn % 2 == 0 and ns >= 16
    classes = (T.K_SCAN, T.K_FWD, T.K_BWD, T.K_FIRST)
    T.tm_store_groups_enable(0)
    T.tm_timing_enable(sum(1 << c for c in classes))
    for c in classes:
        T.tm_timing_read(c)
    torch.cuda.synchronize()
    e0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    e1 = time.perf_counter()
    T.tm_timing_enable(0)
    T.tm_store_groups_enable(1)
    names = {T.K_SCAN: "scan", T.K_FWD: "fwd", T.K_BWD: "bwd", T.K_FIRST: "first"}
    per = {nm: T.tm_timing_read(c) for c, nm in names.items()}

    # algorithmic work per step of each class
    fl = first_layer_launches(wl, ns, Tn)
    work = {
        "first": ("hbm", sum(fl)),
        "fwd": ("mfma", fwd_flops(wl, ns, Tn)),
        "bwd": ("mfma", bwd_flops(wl, ns, Tn)),
    }
    kernel_names = {"first": "first_layer_kernel", "fwd": "gemm_kernel",
                    "bwd": "gemm_kernel", "scan": "scan_kernel"}
    kernels = {}
    for nm, (ms, n) in per.items():
        kd = {"kernel": kernel_names[nm], "launches_per_step": n / args.steps,
              "us_per_launch": ms * 1e3 / max(n, 1), "ms_per_step": ms / args.steps}
        if nm in work and n > 0:
            kind, amount = work[nm]
            s_per_step = ms / 1e3 / args.steps
            if kind == "hbm":
                kd["GB_per_s"] = amount / s_per_step / 1e9
                kd["hbm_frac"] = kd["GB_per_s"] / HBM_PEAK_GBS
            else:
                peak = BF16_PEAK_TFLOPS if wl.dtype == "bf16" else FP32_PEAK_TFLOPS
                kd["tflops"] = amount / s_per_step / 1e12
                kd["mfma_util"] = kd["tflops"] / peak
        kernels[nm] = kd
    kernels["direct_launch_ms_per_step"] = (e1 - e0) / args.steps * 1e3

    dom = max((nm for nm in work if per[nm][1] > 0), key=lambda nm: per[nm][0])
    kind, amount = work[dom]
    dms, dn = per[dom]
    avg_s = dms / 1e3 / dn
    per_launch = amount / (dn / args.steps)
    if kind == "hbm":
        achieved = per_launch / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    else:
        peak = BF16_PEAK_TFLOPS if wl.dtype == "bf16" else FP32_PEAK_TFLOPS
        achieved = per_launch / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak}
    roof["traffic"] = read_traffic(kernel_names[dom], wl.name)
    roof.update({"kernel": kernel_names[dom], "launches": dn, "avg_us": avg_s * 1e6,
                 ("bytes_per_launch" if kind == "hbm" else "flops_per_launch"): per_launch,
                 "timing": "HIP events recorded with each launch's own dispatch (hipExtLaunchKernel) on its stream, second pass of the same steps",
                 "kernel_source_sha256_16": kernel_source_hash()})

    tokens = Bn * Tn * args.steps
    out = {
        "metric": METRIC,
        "value": tokens / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "step_ms": {"min": step_ms[0], "median": step_ms[len(step_ms) // 2],
                    "timing": "events around each step on its stream, a separate pass of the same steps"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; shapes of the README example, gates with fixed logit offsets)",
        "config": {"workload": wl.name, "batch": Bn, "seq": Tn, "heads": H, "dim": d,
                   "hidden": wl.hidden, "depth": wl.depth, "chunk": wl.chunk,
                   "step": "tm_state_init + tm_forward (store + retrieve)" if read is None else
                           "tm_state_init + tm_forward_ex(read=%s) (store + retrieve)" % args.read},
        "roofline": roof,
        "kernels": kernels,
    }
    if groups:
        out["kernels_timed_as"] = "one chunk chain (the throughput pass: two batch groups, overlapping)"

    if not args.no_other:
        # the other workloads of the pages' shapes, a few steps each (context;
        # the headline value is the workload above)
        orc = not args.no_cpu_baseline
        lines = {
            "linear64": lambda: other_workload("linear64", 20, oracle=orc),
            "mlp384_stream": lambda: other_workload("mlp384_stream", 3, oracle=orc),
            "multihead1024": lambda: other_workload("multihead1024", 3, kernel_roof=True, oracle=orc,
                                                    oracle_tokens=128),
            "deep512": lambda: other_workload("deep512", 2, calls=16, oracle=orc, oracle_tokens=64),
            # the same step with each chunk's queries read before its write
            "mlp384_read_before_write": lambda: other_workload("mlp384", 20, read=1, oracle=orc),
            # each query read right after its own token's write (the dual form)
            "mlp384_read_per_token": lambda: other_workload("mlp384", 20, read=2, oracle=orc),
            # read-only retrieval of the call's queries through the stored memory
            "mlp384_retrieve": lambda: retrieval("mlp384", 20, oracle=orc),
            # ... and at the multi-head workload's scale (64 streams x 32768 queries)
            "multihead1024_retrieve": lambda: retrieval("multihead1024", 3),
            # the backward through the store (gradients through one tm_forward call)
            "mlp384_backward": lambda: backward_line("mlp384", 10, oracle=orc),
            # the input side alone and chained with the memory (two lines)
            "mlp384_input_side": lambda: input_side("mlp384", 20, oracle=orc),
            # the memory's side of memory as a context, segment by segment
            "mlp384_mac": lambda: mac_wiring("mlp384", 10, oracle=orc),
        }
        want = list(lines) if args.lines is None else args.lines.split(",")
        out["other_workloads"] = {}
        for nm in want:
            r = lines[nm]()
            if nm == "mlp384_input_side":
                out["other_workloads"]["mlp384_input_side"] = r["input_side"]
                out["other_workloads"]["mlp384_from_tokens"] = r["from_tokens"]
            else:
                out["other_workloads"][nm] = r
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, params, ci)
        out["cpu_baseline"]["gpu_over_cpu"] = out["value"] / out["cpu_baseline"]["value"]
    if args.calib_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
