"""The full-size workloads through the C ABI, against the fp64 oracle.

Where the oracle cannot run the whole workload in seconds, it runs a prefix
(or sampled streams) for element-wise parity, and the full-size GPU run is
checked on outputs the oracle can compute one by one: the last chunk's
retrieval equals the oracle's read of the GPU's final state (reading R1: the
queries of the last chunk read the weights after its write).  Full-size runs
are also checked for call-split invariance (bitwise) and finiteness.
Tolerances: relative Frobenius error, 2e-2 for bf16 inputs (2x for S).
"""
import numpy as np
import pytest
import torch

from harness import GpuMemory, TOL, compare_state, dev_inputs, oracle_forward, relerr, say
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
        e = relerr(y_gpu[bi:bi + 1, T - b:T, hi:hi + 1], yr)
        worst = max(worst, e)
    return worst, st


def test_mlp384_stream_workload():
    # 4 streams x 16 calls of 1024 tokens, state carried.  Oracle: the first
    # two calls on every stream; GPU: all sixteen, then the last chunk's
    # retrieval and a single 16384-token call (bitwise identical state)
    wl = I.WORKLOADS["mlp384_stream"]
    say("case", wl)
    p = I.make_params(wl)
    g = GpuMemory(wl, p)
    ref = I.initial_state(wl, p)
    calls = [I.make_call(wl, p, j) for j in range(wl.calls)]
    ys = []
    for j, ci in enumerate(calls):
        y = g.forward(dev_inputs(ci, "bf16")).cpu().numpy()
        ys.append(y)
        if j < 2:
            yr = oracle_forward(wl, ref, ci)
            ey = relerr(y, yr)
            em, es = compare_state(wl, g.export(), ref)
            say("  call %d: y %.2e  M %.2e  S %.2e" % (j, ey, em, es))
            assert ey < TOL["bf16"] and em < TOL["bf16"] and es < 2 * TOL["bf16"]
    nf, pos = g.check()
    assert not nf and pos == wl.seq
    e_last, st = last_chunk_check(wl, g, calls[-1], ys[-1], [(b, 0) for b in range(wl.batch)])
    say("  last chunk of call 16: y %.2e" % e_last)
    assert e_last < TOL["bf16"]
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


def test_multihead1024_workload():
    # 8 x 32768 tokens, 8 heads of dim 128 = 64 streams.  Oracle: the first
    # 2048 tokens of four sampled streams; GPU: the whole call, as one call
    # and as 2048 + 30720 (bitwise identical), then the last chunk's retrieval
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
    init = I.initial_state(wl, p)
    sampled = [(0, 0), (3, 5), (5, 2), (7, 7)]
    for (bi, hi) in sampled:
        s = bi * wl.heads + hi
        one = wl.replace(batch=1, heads=1)
        ref = np.ascontiguousarray(init[s:s + 1])
        yr = oracle_forward(one, ref, sub_call(ci, bi, bi + 1, 0, 2048, hi, hi + 1))
        ey = relerr(y_pre[bi:bi + 1, :, hi:hi + 1], yr)
        em, es = compare_state(one, st_pre[s:s + 1], ref)
        say("  stream (%d, %d), 2048 tokens: y %.2e  M %.2e  S %.2e" % (bi, hi, ey, em, es))
        assert ey < TOL["bf16"] and em < TOL["bf16"] and es < 2 * TOL["bf16"]
    y_rest = g.forward(rest).cpu().numpy()
    nf, pos = g.check()
    assert not nf and pos == wl.seq
    y_full = np.concatenate([y_pre, y_rest], axis=1)
    e_last, st = last_chunk_check(wl, g, ci, y_full, sampled)
    say("  last chunk: y %.2e" % e_last)
    assert e_last < TOL["bf16"]
    h = GpuMemory(wl, p)
    y_one = h.forward(d).cpu().numpy()
    assert np.array_equal(h.export(), st)
    assert np.array_equal(y_one, y_full)
    g.close()
    h.close()


def test_deep512_prefix():
    # depth 4 (512 -> 2048 -> 2048 -> 2048 -> 512), chunk 32: the backward
    # runs through three hidden layers.  Oracle: the first 128 tokens
    wl = I.WORKLOADS["deep512"]
    say("case", wl)
    p = I.make_params(wl)
    ci = I.make_call(wl, p, 0, tokens=128)
    g = GpuMemory(wl, p)
    y = g.forward(dev_inputs(ci, "bf16")).cpu().numpy()
    ref = I.initial_state(wl, p)
    yr = oracle_forward(wl, ref, ci)
    ey = relerr(y, yr)
    em, es = compare_state(wl, g.export(), ref)
    say("  128 tokens: y %.2e  M %.2e  S %.2e" % (ey, em, es))
    assert ey < TOL["bf16"] and em < TOL["bf16"] and es < 2 * TOL["bf16"]
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
    ey = relerr(y, yr)
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
