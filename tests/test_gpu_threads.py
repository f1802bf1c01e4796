"""One ctx shared by two host threads, each with its own state, workspace
and torch stream, calling at the same time: every result is bitwise that of
the same calls made by one thread.  The calls go through a first sighting
(direct launches), a capture and replays, and the 16-stream shape runs its
batch halves as two chunk chains, so the threads also exercise their own
extra streams and the shared graph cache.  2 x 8 heads of 128 -> 512 -> 128,
chunk 64, 256 tokens, bf16."""
import threading

import numpy as np
import pytest
import torch

import test_trained_neural_amd as T
from harness import dev_inputs, say
from test_trained_neural_amd import inputs as I

pytestmark = pytest.mark.gpu

WL = I.Workload("threads", batch=2, seq=256, heads=8, dim=128, depth=2, expansion=4, chunk=64, dtype="bf16",
                offsets=(-7.0, 2.0, -7.0))


def calls(ctx, d, init, out, stream):
    """The sequence of one user: set up a state, three tm_forward calls, a
    tm_store and a tm_retrieve; the outputs and the exported state go to out."""
    B, H, Tn = WL.batch, WL.heads, WL.seq
    with torch.cuda.stream(stream):
        state = torch.empty(T.tm_state_bytes(ctx, B, H), dtype=torch.uint8, device="cuda")
        ws = torch.empty(T.tm_workspace_bytes(ctx, B, H, Tn), dtype=torch.uint8, device="cuda")
        T.tm_state_init(ctx, state, B, H, init)
        for i in range(3):
            y = torch.empty((B, Tn, H, WL.dim), dtype=torch.float32, device="cuda")
            T.tm_forward(ctx, state, d["k"], d["v"], d["q"], d["theta"], d["eta"], d["alpha"], y, ws)
            out["y%d" % i] = y
        T.tm_store(ctx, state, d["k"], d["v"], d["theta"], d["eta"], d["alpha"], ws)
        r = torch.empty((B, Tn, H, WL.dim), dtype=torch.float32, device="cuda")
        T.tm_retrieve(ctx, state, d["q"], r, ws)
        out["r"] = r
        st = torch.empty((B * H, 2 * T.tm_param_count(ctx)), dtype=torch.float32, device="cuda")
        T.tm_state_export(ctx, state, B, H, st)
        out["st"] = st
    stream.synchronize()
    for k in list(out):
        out[k] = out[k].cpu().numpy()


def test_two_threads_share_a_ctx():
    say("case", WL)
    p = I.make_params(WL)
    ci = I.make_call(WL, p)
    d = dev_inputs(ci, "bf16")
    init = torch.from_numpy(np.ascontiguousarray(p.init_weights, np.float32)).to("cuda")
    ref_ctx = T.tm_create(WL.dim, WL.depth, WL.expansion, WL.chunk)
    ref = {}
    calls(ref_ctx, d, init, ref, torch.cuda.Stream())
    T.tm_destroy(ref_ctx)

    ctx = T.tm_create(WL.dim, WL.depth, WL.expansion, WL.chunk)
    outs = [{}, {}]
    errs = []

    def run(i):
        try:
            calls(ctx, d, init, outs[i], torch.cuda.Stream())
        except Exception as e:   # reported by the main thread
            errs.append(repr(e))

    ths = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in ths:
        t.start()
    for t in ths:
        t.join(timeout=100)
    assert not any(t.is_alive() for t in ths), "a thread did not finish"
    assert not errs, errs
    for i, o in enumerate(outs):
        assert sorted(o) == sorted(ref)
        for k in sorted(ref):
            assert np.array_equal(o[k], ref[k]), (i, k)
    torch.cuda.synchronize()
    T.tm_destroy(ctx)
    say("  both threads: %d outputs and the state bitwise equal to one thread's" % (len(ref) - 1))
