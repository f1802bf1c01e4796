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
stream (events force direct launches); ``roofline.achieved`` = the dominant
kernel's (the gradient-reduction + state-update kernel) algorithmic bytes per
launch / its mean event-timed duration.  The fp64 CPU oracle is timed on the
host as ``cpu_baseline``.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3


def algorithmic(wl, ns):
    """Per-launch algorithmic work of each kernel class for one chunk step."""
    P = wl.params
    b = wl.chunk
    dims = wl.layer_dims()
    # update: M, S read + written in fp32, bf16 copy of M written; plus the
    # chunk's activations (bf16) and deltas (fp32) read once
    upd_bytes = ns * (18 * P + sum(b * (din * 2 + dout * 4) for din, dout in dims))
    upd_flops = ns * 4 * b * P                      # two K=b reductions
    fwd_flops = ns * 2 * (2 * b) * P                # q rows of the previous chunk + k rows
    bwd_flops = ns * 2 * b * sum(din * dout for din, dout in dims[1:])
    return dict(upd_bytes=upd_bytes, upd_flops=upd_flops, fwd_flops=fwd_flops, bwd_flops=bwd_flops)


def cpu_baseline(wl, params, ci, seconds_hint):
    """The fp64 oracle on a bounded sample of the same workload."""
    from oracle import tmref
    from test_trained_neural_amd import inputs as I
    import numpy as np
    streams = wl.batch * wl.heads
    # ~12 ms per token per stream for this memory: the whole workload
    # (2 streams x 1024 tokens) is ~10-15 s on 2 threads
    tokens = wl.tokens_per_call
    st = I.initial_state(wl, params)
    threads = min(os.cpu_count() or 1, streams)
    t0 = time.perf_counter()
    tmref.forward(wl.dim, wl.depth, wl.expansion, wl.chunk, st, ci.k[:, :tokens], ci.v[:, :tokens],
                  ci.theta[:, :tokens], ci.eta[:, :tokens], ci.alpha[:, :tokens], q=ci.q[:, :tokens],
                  n_threads=threads)
    dt = time.perf_counter() - t0
    return {"value": wl.batch * tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%s: %d streams x %d tokens (the whole step), fp64 C oracle, %.1f s"
                      % (wl.name, streams, tokens, dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mlp384")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the memory streams of this workload are independent "
              "and a multi-GPU run would only shard them; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
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

    def step():
        T.tm_state_init(ctx, state, Bn, H, init)
        T.tm_forward(ctx, state, k, v, q, th, et, al, y, ws)

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
    t1 = time.perf_counter()
    elapsed = t1 - t0

    # the same steps again with HIP events around every launch (events force
    # direct launches): per-kernel durations for the roofline
    T.tm_timing_enable(0x1F)
    for c in range(5):
        T.tm_timing_read(c)
    torch.cuda.synchronize()
    e0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    e1 = time.perf_counter()
    T.tm_timing_enable(0)
    names = {T.K_SCAN: "scan", T.K_FWD: "fwd", T.K_BWD: "bwd", T.K_UPDATE: "update", T.K_FIRST: "first"}
    per = {}
    for c, nm in names.items():
        per[nm] = T.tm_timing_read(c)
    upd_ms, upd_n = per["update"]

    tokens = Bn * Tn * args.steps
    work = algorithmic(wl, ns)
    upd_avg_s = upd_ms / 1e3 / max(upd_n, 1)
    achieved = work["upd_bytes"] / upd_avg_s / 1e9
    kernels = {}
    for nm, (ms, n) in per.items():
        kernels[nm] = {"launches_per_step": n / args.steps, "us_per_launch": ms * 1e3 / max(n, 1),
                       "ms_per_step": ms / args.steps}
    fwd_s = per["fwd"][0] / 1e3 / args.steps
    bwd_s = per["bwd"][0] / 1e3 / args.steps
    # forward: every token row goes through the weights twice per call (as a
    # key of its chunk and as a query of the same chunk); backward: key rows
    # through layers 2..L
    fwd_flops = 2 * 2 * Bn * H * Tn * wl.params
    bwd_flops = 2 * Bn * H * Tn * sum(a * b for a, b in wl.layer_dims()[1:])
    kernels["fwd"]["tflops"] = fwd_flops / fwd_s / 1e12
    kernels["fwd"]["mfma_util"] = kernels["fwd"]["tflops"] / BF16_PEAK_TFLOPS
    if bwd_s > 0:
        kernels["bwd"]["tflops"] = bwd_flops / bwd_s / 1e12
        kernels["bwd"]["mfma_util"] = kernels["bwd"]["tflops"] / BF16_PEAK_TFLOPS
    kernels["direct_launch_ms_per_step"] = (e1 - e0) / args.steps * 1e3
    out = {
        "metric": "memory tokens/sec (store+retrieve) at dim 384, chunk 64; MFMA util %",
        "value": tokens / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; shapes of the README example)",
        "config": {"workload": wl.name, "batch": Bn, "seq": Tn, "heads": H, "dim": d,
                   "hidden": wl.hidden, "depth": wl.depth, "chunk": wl.chunk,
                   "step": "tm_state_init + tm_forward"},
        "roofline": {"bound": "hbm", "kernel": "update_kernel (gradient reduction + state update)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "launches": upd_n, "avg_us": upd_avg_s * 1e6,
                     "bytes_per_launch": work["upd_bytes"],
                     "timing": "HIP events around each launch, second pass of the same steps"},
        "kernels": kernels,
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, params, ci, 15.0)
        out["cpu_baseline"]["vs_gpu"] = out["value"] / out["cpu_baseline"]["value"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
