"""The full-size workloads through the C ABI, against the fp64 oracle.

The dim-384 stream is compared in full (all 16 calls, every stream); the
multi-head workload on all 64 streams over its first 2048 tokens, then on
its last chunk (the oracle's read of the GPU's final state, under reading
R1); the depth-4 workload over its first 2048 tokens, its full stream by
call-split invariance (bitwise), finiteness and its decay.  Comparisons are
element-wise in the sense of harness.yerr / compare_state: the worst of the
relative Frobenius error, the worst token row's relative error (y) and
max |diff| / max |ref|, under 2e-2 for bf16 inputs (2x for S) and 1e-4 for
the fp32 runs at the same memory shapes.
"""
import numpy as np
import pytest
import torch

from harness import GpuMemory, TOL, compare_state, dev_inputs, oracle_forward, relerr, say, yerr
from oracle import tmref
from test_trained_neural_amd import inputs as I

pytestmark = pytest.mark.gpu


def sub_call(ci, b0, b1, t0, t1, h0=None, h1=None):
    """Slice of a call's inputs: batch rows b0:b1, tokens t0:t1 (heads h0:h1)."""
    hs = slice(h0, h1)
    return I.CallInputs(*(np.ascontiguousarray(getattr(ci, n)[b0:b1, t0:t1, hs]) for n in
                          ("k", "v", "q", "theta", "eta", "alpha")))


def last_chunk_check(wl, g, ci, y_gpu, streams):
    """The last chunk's queries of the call just run: GPU y against the
    oracle's read of the GPU's final state, for the given (batch, head) streams."""
    b = wl.chunk
    T = ci.k.shape[1]
    st = g.export()
    worst = 0.0
    for (bi, hi) in streams:
        s = bi * wl.heads + hi
        q = np.ascontiguousarray(ci.q[bi:bi + 1, T - b:T, hi:hi + 1])
        yr = tmref.retrieve(wl.dim, wl.depth, wl.expansion, st[s:s + 1].astype(np.float64), q)
        e = yerr(y_gpu[bi:bi + 1, T - b:T, hi:hi + 1], yr)
        worst = max(worst, e)
    return worst, st


def test_mlp384_stream_workload():
    # 4 streams x 16 calls of 1024 tokens, state carried, every call on every
    # stream against the oracle:
    #   * carried: the oracle carries its own state from the start.  With
    #     bf16 operands the difference grows along the stream (fp32 does not,
    #     see the fp32 test below): measured 2e-3 on y over the first 5
    #     calls, 6.5e-3 at call 8, 4.3e-2 at call 16, as the memory's norm
    #     decays from 29 to 1.6 and each chunk's bf16 rounding is carried
    #     forward.  Asserted over the first 8 calls (8192 tokens per stream);
    #   * per call: the oracle restarted from the GPU's own state at the
    #     call's start, so each call's comparison holds that call's rounding
    #     only.  Asserted for all 16 calls.
    # Then the same stream as one 16384-token call (bitwise identical).
    wl = I.WORKLOADS["mlp384_stream"]
    say("case", wl)
    p = I.make_params(wl)
    g = GpuMemory(wl, p)
    ref = I.initial_state(wl, p)
    calls = [I.make_call(wl, p, j) for j in range(wl.calls)]
    ys = []
    for j, ci in enumerate(calls):
        st0 = g.export().astype(np.float64)
        y = g.forward(dev_inputs(ci, "bf16")).cpu().numpy()
        ys.append(y)
        st = g.export()
        yr = oracle_forward(wl, ref, ci)
        ey, (em, es) = yerr(y, yr), compare_state(wl, st, ref)
        yc = oracle_forward(wl, st0, ci)
        cy, (cm, cs) = yerr(y, yc), compare_state(wl, st, st0)
        say("  call %d: carried y %.2e  M %.2e  S %.2e | from the GPU's state y %.2e  M %.2e  S %.2e"
            % (j + 1, ey, em, es, cy, cm, cs))
        if j < 8:
            assert ey < TOL["bf16"] and em < TOL["bf16"] and es < 2 * TOL["bf16"]
        assert cy < TOL["bf16"] and cm < TOL["bf16"] and cs < 2 * TOL["bf16"]
    nf, pos = g.check()
    assert not nf and pos == wl.seq
    st = g.export()
    assert np.all(np.isfinite(st))
    # the same stream as one call
    whole = I.CallInputs(*(np.concatenate([getattr(c, n) for c in calls], axis=1) for n in
                           ("k", "v", "q", "theta", "eta", "alpha")))
    h = GpuMemory(wl, p)
    yw = h.forward(dev_inputs(whole, "bf16")).cpu().numpy()
    assert np.array_equal(h.export(), st)
    assert np.array_equal(yw, np.concatenate(ys, axis=1))
    g.close()
    h.close()


def test_mlp384_stream_fp32_carried():
    # the same 4 x 16 calls with fp32 inputs, the oracle carrying its own
    # state over all 16384 tokens of every stream: no drift (measured 1e-5)
    wl = I.WORKLOADS["mlp384_stream"].replace(name="mlp384_stream_f32", dtype="f32")
    say("case", wl)
    p = I.make_params(wl)
    g = GpuMemory(wl, p)
    ref = I.initial_state(wl, p)
    for j in range(wl.calls):
        ci = I.make_call(wl, p, j)
        y = g.forward(dev_inputs(ci, "f32")).cpu().numpy()
        yr = oracle_forward(wl, ref, ci)
        ey, (em, es) = yerr(y, yr), compare_state(wl, g.export(), ref)
        say("  call %d: y %.2e  M %.2e  S %.2e" % (j + 1, ey, em, es))
        assert ey < TOL["f32"] and em < TOL["f32"] and es < 2 * TOL["f32"]
    g.close()


def test_multihead1024_workload():
    # 8 x 32768 tokens, 8 heads of dim 128 = 64 streams.  Oracle: all 64
    # streams over the first 2048 tokens (y and state), then the last chunk's
    # retrieval of every stream against the oracle's read of the GPU's final
    # state; the whole call as one call and as 2048 + 30720 (bitwise
    # identical); a read-only retrieval of the whole call from the final state
    wl = I.WORKLOADS["multihead1024"]
    say("case", wl)
    p = I.make_params(wl)
    ci = I.make_call(wl, p)
    d = dev_inputs(ci, "bf16")
    g = GpuMemory(wl, p)
    pre = {k: v[:, :2048].contiguous() for k, v in d.items()}
    rest = {k: v[:, 2048:].contiguous() for k, v in d.items()}
    y_pre = g.forward(pre).cpu().numpy()
    st_pre = g.export()
    ref = I.initial_state(wl, p)
    yr = oracle_forward(wl, ref, sub_call(ci, 0, wl.batch, 0, 2048))
    ey = yerr(y_pre, yr)
    em, es = compare_state(wl, st_pre, ref)
    say("  64 streams, 2048 tokens: y %.2e  M %.2e  S %.2e" % (ey, em, es))
    assert ey < TOL["bf16"] and em < TOL["bf16"] and es < 2 * TOL["bf16"]
    y_rest = g.forward(rest).cpu().numpy()
    nf, pos = g.check()
    assert not nf and pos == wl.seq
    y_full = np.concatenate([y_pre, y_rest], axis=1)
    every = [(bi, hi) for bi in range(wl.batch) for hi in range(wl.heads)]
    e_last, st = last_chunk_check(wl, g, ci, y_full, every)
    say("  last chunk, every stream: y %.2e" % e_last)
    assert e_last < TOL["bf16"]
    h = GpuMemory(wl, p)
    y_one = h.forward(d).cpu().numpy()
    assert np.array_equal(h.export(), st)
    assert np.array_equal(y_one, y_full)
    h.close()
    # read-only retrieval of the whole call's queries (64 streams x 32768
    # rows, one launch) from the final state: every stream at 144 sampled
    # rows (128 random, the last 16) against the oracle's read of that state
    y_ret = g.retrieve(d["q"]).cpu().numpy()
    assert np.all(np.isfinite(y_ret))
    rng = np.random.default_rng(11)
    worst = 0.0
    for (bi, hi) in every:
        s = bi * wl.heads + hi
        rows = np.concatenate([np.sort(rng.choice(wl.seq - 16, 128, replace=False)), np.arange(wl.seq - 16, wl.seq)])
        q = np.ascontiguousarray(ci.q[bi:bi + 1, rows, hi:hi + 1])
        yr = tmref.retrieve(wl.dim, wl.depth, wl.expansion, st[s:s + 1].astype(np.float64), q)
        worst = max(worst, yerr(y_ret[bi:bi + 1, rows, hi:hi + 1], yr))
    say("  retrieve of the whole call, every stream at 144 rows: y %.2e" % worst)
    assert worst < TOL["bf16"]
    g.close()


def test_deep512_prefix():
    # depth 4 (512 -> 2048 -> 2048 -> 2048 -> 512), chunk 32: the backward
    # runs through three hidden layers.  Oracle: the first two calls (2048
    # tokens), the state carried between them, and call 2 again from the
    # GPU's state after call 1.  y and M are held to 2e-2 throughout.  S, the
    # momentum, is a difference of nearly equal terms whose bf16 error is the
    # largest at this depth: held to 4e-2 over the first call, reported after
    # the second (measured 4.7e-2 carried, by max |diff| / max |ref|); the
    # fp32 run at this shape holds S to 2e-4.
    wl = I.WORKLOADS["deep512"]
    say("case", wl)
    p = I.make_params(wl)
    g = GpuMemory(wl, p)
    ref = I.initial_state(wl, p)
    for j in range(2):
        ci = I.make_call(wl, p, j)
        st0 = g.export().astype(np.float64)
        y = g.forward(dev_inputs(ci, "bf16")).cpu().numpy()
        st = g.export()
        yr = oracle_forward(wl, ref, ci)
        ey, (em, es) = yerr(y, yr), compare_state(wl, st, ref)
        yc = oracle_forward(wl, st0, ci)
        cy, (cm, cs) = yerr(y, yc), compare_state(wl, st, st0)
        say("  call %d (1024 tokens): carried y %.2e  M %.2e  S %.2e | from the GPU's state y %.2e  M %.2e  S %.2e"
            % (j + 1, ey, em, es, cy, cm, cs))
        assert ey < TOL["bf16"] and em < TOL["bf16"] and cy < TOL["bf16"] and cm < TOL["bf16"]
        if j == 0:
            assert es < 2 * TOL["bf16"]
    g.close()


# fp32 inputs at the multi-head and depth-4 memory shapes, gated at 1e-4:
# an algorithm slip that bf16 rounding would hide shows here
F32_SHAPES = [
    I.WORKLOADS["multihead1024"].replace(name="multihead1024_f32", batch=2, seq=512, dtype="f32"),
    I.WORKLOADS["deep512"].replace(name="deep512_f32", seq=128, calls=1, dtype="f32"),
]


@pytest.mark.parametrize("wl", F32_SHAPES, ids=lambda w: w.name)
def test_fp32_at_workload_shapes(wl):
    say("case", wl)
    p = I.make_params(wl)
    ci = I.make_call(wl, p)
    g = GpuMemory(wl, p)
    y = g.forward(dev_inputs(ci, "f32")).cpu().numpy()
    ref = I.initial_state(wl, p)
    yr = oracle_forward(wl, ref, ci)
    ey = yerr(y, yr)
    em, es = compare_state(wl, g.export(), ref)
    say("  y %.2e  M %.2e  S %.2e" % (ey, em, es))
    assert ey < TOL["f32"] and em < TOL["f32"] and es < 2 * TOL["f32"]
    g.close()


def test_deep512_stream():
    # the whole 1,048,576-token stream in 1024 calls of 1024 tokens.  With
    # this workload's gate offsets the depth-4 memory shrinks towards the
    # zero fixed point (zero weights have zero gradient): it is still well
    # away from zero after 4 calls, where the last chunk's retrieval is
    # checked against the oracle's read of the GPU state, and it has decayed
    # to the bottom of the fp32 range long before the end of the stream,
    # where the state must be finite, below 1e-30 everywhere (a decay factor
    # close to 1 rounds the smallest subnormal back to itself, so isolated
    # entries stay there), the retrieval below 1e-30, and every token counted
    wl = I.WORKLOADS["deep512"]
    say("case", wl)
    p = I.make_params(wl)
    g = GpuMemory(wl, p)
    for j in range(wl.calls):
        ci = I.make_call(wl, p, j)
        y = g.forward(dev_inputs(ci, "bf16"))
        if j == 3:
            y4 = y.cpu().numpy()
            e4, st4 = last_chunk_check(wl, g, ci, y4, [(0, 0)])
            norms = [float(np.linalg.norm(st4[0, :wl.params]))]
            say("  call 4: last chunk y %.2e, |M| %.3g, |y| %.3g" % (e4, norms[0], np.linalg.norm(y4[0, -32:])))
            assert e4 < TOL["bf16"] and norms[0] > 1.0
        if j % 128 == 127:
            nf, pos = g.check()
            say("  call %d: position %d, non-finite %s" % (j + 1, pos, nf))
            assert not nf
    y = y.cpu().numpy()
    nf, pos = g.check()
    assert not nf and pos == wl.seq
    st = g.export()
    say("  end: max |state| %.3g, max |y| %.3g" % (np.abs(st).max(), np.abs(y).max()))
    assert np.all(np.isfinite(st)) and np.abs(st).max() < 1e-30 and np.abs(y).max() < 1e-30
    g.close()


MAX = [
    # the widest memory the library takes (dim 1024) at the largest chunk
    I.Workload("dim1024", batch=1, seq=128, heads=1, dim=1024, depth=2, expansion=2, chunk=64,
               dtype="bf16", offsets=(-5.0, 1.0, -5.0)),
    # the deepest memory (8 weight matrices)
    I.Workload("depth8", batch=1, seq=64, heads=2, dim=32, depth=8, expansion=2, chunk=8,
               dtype="bf16", offsets=(-4.0, 1.0, -4.0)),
    I.Workload("depth8_f32", batch=1, seq=64, heads=2, dim=32, depth=8, expansion=2, chunk=8,
               dtype="f32", offsets=(-4.0, 1.0, -4.0)),
]


@pytest.mark.parametrize("wl", MAX, ids=lambda w: w.name)
def test_maximum_sizes(wl):
    say("case", wl)
    p = I.make_params(wl)
    ci = I.make_call(wl, p)
    g = GpuMemory(wl, p)
    y = g.forward(dev_inputs(ci, wl.dtype)).cpu().numpy()
    ref = I.initial_state(wl, p)
    yr = oracle_forward(wl, ref, ci)
    ey = yerr(y, yr)
    em, es = compare_state(wl, g.export(), ref)
    say("  y %.2e  M %.2e  S %.2e" % (ey, em, es))
    tol = TOL[wl.dtype]
    assert np.all(np.isfinite(ref))
    assert ey < tol and em < tol and es < 2 * tol
    g.close()


def test_empty_call_is_a_no_op():
    wl = I.Workload("empty", batch=2, seq=0, heads=1, dim=64, depth=2, expansion=2, chunk=16, dtype="bf16",
                    offsets=(-4.0, 1.0, -4.0))
    p = I.make_params(wl)
    g = GpuMemory(wl, p)
    before = g.export()
    z = torch.empty((2, 0, 1, 64), dtype=torch.bfloat16, device="cuda")
    zg = torch.empty((2, 0, 1), dtype=torch.float32, device="cuda")
    y = g.forward({"k": z, "v": z, "q": z, "theta": zg, "eta": zg, "alpha": zg})
    torch.cuda.synchronize()
    assert y.shape == (2, 0, 1, 64)
    assert np.array_equal(g.export(), before)
    assert g.check() == (False, 0)
    g.close()
