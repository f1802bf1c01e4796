"""Parity of the HIP path against the fp64 oracle, through the C ABI, on the
same seeded inputs.  Tolerances (relative Frobenius error per output tensor
and per weight matrix of every stream): fp32 inputs 1e-4, bf16 inputs 2e-2.
"""
import numpy as np
import pytest
import torch

from harness import GpuMemory, TOL, compare_state, dev_inputs, oracle_forward, relerr, say, yerr
from oracle import tmref
from test_trained_neural_amd import inputs as I

pytestmark = pytest.mark.gpu


def small(name, dim, depth, ex, chunk, B, H, T, dtype, offsets=(-4.0, 1.0, -4.0)):
    return I.Workload(name, batch=B, seq=T, heads=H, dim=dim, depth=depth, expansion=ex, chunk=chunk,
                      dtype=dtype, offsets=offsets)


# shapes spanning several 64-wide tiles, a ragged 32-wide tail (dim 96,
# hidden 288), chunks that are not a multiple of 32 (24, 5) and chunk 1
SMALL = [
    small("lin32", 32, 1, 1, 8, 2, 2, 32, "f32"),
    small("mlp64", 64, 2, 2, 16, 1, 2, 64, "f32"),
    small("mlp96", 96, 2, 3, 24, 2, 1, 96, "f32"),
    small("deep64", 64, 3, 2, 64, 1, 1, 192, "f32"),
    small("deep32x4", 32, 4, 4, 5, 1, 3, 40, "f32"),
    small("tok1", 32, 2, 2, 1, 1, 1, 12, "f32"),
    # long K, one 64-wide column tile: the products split K over workgroups
    small("wide512", 32, 2, 16, 32, 1, 2, 96, "f32"),
]


def run_pair(wl, seed=0, calls=1, mode="forward"):
    p = I.make_params(wl, seed)
    g = GpuMemory(wl, p)
    ref = I.initial_state(wl, p)
    ys_g, ys_r = [], []
    for j in range(calls):
        ci = I.make_call(wl, p, j, seed)
        d = dev_inputs(ci, wl.dtype)
        if mode == "forward":
            ys_g.append(g.forward(d).cpu().numpy())
            ys_r.append(oracle_forward(wl, ref, ci))
        else:
            g.store(d)
            oracle_forward(wl, ref, ci, with_q=False)
    st = g.export()
    nf, pos = g.check()
    g.close()
    return ys_g, ys_r, st, ref, nf, pos


@pytest.mark.parametrize("wl", SMALL + [w.replace(dtype="bf16", name=w.name + "_bf16") for w in SMALL],
                         ids=lambda w: w.name)
def test_small_parity(wl):
    say("case", wl)
    ys_g, ys_r, st, ref, nf, pos = run_pair(wl)
    tol = TOL[wl.dtype]
    ey = yerr(ys_g[0], ys_r[0])
    em, es = compare_state(wl, st, ref)
    say("  y %.2e  M %.2e  S %.2e" % (ey, em, es))
    assert not nf and pos == wl.seq
    assert np.all(np.isfinite(ref))
    assert ey < tol and em < tol
    assert es < 2 * tol


def test_store_only_matches_forward_state():
    wl = small("mlp64s", 64, 2, 2, 16, 2, 1, 64, "f32")
    say("case", wl)
    _, _, st_f, ref, _, _ = run_pair(wl)
    _, _, st_s, ref_s, _, _ = run_pair(wl, mode="store")
    assert np.array_equal(st_f, st_s)
    assert np.array_equal(ref, ref_s)


def test_state_init_and_export():
    wl = small("init", 64, 2, 2, 16, 2, 3, 16, "bf16", offsets=(0, 0, 0))
    say("case", wl)
    p = I.make_params(wl)
    g = GpuMemory(wl, p)
    st = g.export()
    ref = I.initial_state(wl, p)
    assert np.array_equal(st, ref.astype(np.float32))
    nf, pos = g.check()
    assert not nf and pos == 0
    g.close()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_theta_zero_alpha_zero_leaves_memory_unchanged(dtype):
    wl = small("th0", 64, 2, 2, 16, 1, 2, 64, dtype)
    say("case", wl)
    p = I.make_params(wl)
    g = GpuMemory(wl, p)
    ci = I.make_call(wl, p)
    ci.theta[:] = 0
    ci.alpha[:] = 0
    before = g.export()
    g.forward(dev_inputs(ci, dtype))
    after = g.export()
    assert np.array_equal(before, after)
    g.close()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_alpha_one_memory_equals_momentum(dtype):
    wl = small("al1", 64, 2, 2, 16, 1, 1, 64, dtype)
    say("case", wl)
    p = I.make_params(wl)
    g = GpuMemory(wl, p)
    ci = I.make_call(wl, p)
    ci.alpha[:] = 1
    g.forward(dev_inputs(ci, dtype))
    st = g.export()
    P = wl.params
    assert relerr(st[0, :P], st[0, P:]) < 1e-6
    ref = I.initial_state(wl, p)
    oracle_forward(wl, ref, ci)
    em, es = compare_state(wl, st, ref)
    assert em < TOL[dtype] and es < TOL[dtype]
    g.close()


def test_delta_rule_chunk_one():
    # linear memory, eta = alpha = 0, chunk 1: the delta rule
    wl = small("delta", 32, 1, 1, 1, 1, 1, 16, "f32")
    say("case", wl)
    p = I.make_params(wl)
    rng = np.random.default_rng(5)
    init = (rng.standard_normal((1, 32 * 32)) * 0.2).astype(np.float32)
    p.init_weights[:] = init
    g = GpuMemory(wl, p)
    ci = I.make_call(wl, p)
    ci.eta[:] = 0
    ci.alpha[:] = 0
    ci.theta[:] = 0.3
    g.forward(dev_inputs(ci, "f32"))
    st = g.export()
    W = init.reshape(32, 32).astype(np.float64)
    for t in range(16):
        k = ci.k[0, t, 0].astype(np.float64)
        v = ci.v[0, t, 0].astype(np.float64)
        W = W - float(np.float32(0.3)) * 2.0 * np.outer(k, k @ W - v)
    assert relerr(st[0, :32 * 32].reshape(32, 32), W) < 1e-5
    g.close()


def test_retrieve_is_read_only_and_matches_oracle():
    for dtype in ("f32", "bf16"):
        wl = small("ret", 96, 3, 2, 16, 2, 2, 48, dtype)
        say("case", wl)
        p = I.make_params(wl)
        g = GpuMemory(wl, p)
        ci = I.make_call(wl, p)
        d = dev_inputs(ci, dtype)
        g.forward(d)
        ref = I.initial_state(wl, p)
        oracle_forward(wl, ref, ci)
        before = g.export()
        y = g.retrieve(d["q"]).cpu().numpy()
        y2 = g.retrieve(d["q"]).cpu().numpy()
        after = g.export()
        assert np.array_equal(before, after) and np.array_equal(y, y2)
        yr = tmref.retrieve(wl.dim, wl.depth, wl.expansion, ref, ci.q)
        assert yerr(y, yr) < TOL[dtype]
        g.close()


# retrieve passes of many query rows (the tiled product): a full pass of 2048
# rows and a short second pass, a ragged row count inside one pass, a hidden
# width that is not a multiple of 64, depth 1 to 3
RET_CASES = [
    small("ret_rows_2pass", 64, 2, 4, 16, 1, 2, 2100, "bf16"),
    small("ret_rows_ragged", 96, 3, 3, 16, 2, 1, 1000, "bf16"),
    small("ret_rows_lin", 128, 1, 1, 16, 1, 1, 512, "bf16"),
    # depth 2 at widths up to 128: both layers in one launch (mlp2_kernel):
    # widths 32 to 128, hidden 64 (one 64-unit weight chunk), 192 (an odd
    # number of chunks) and 512, row counts with a ragged last row block or
    # under one 16-row block, 8 streams (grouped by XCD) and fewer
    small("ret_mlp2_d128", 128, 2, 4, 64, 2, 4, 600, "bf16"),
    small("ret_mlp2_d64_h192", 64, 2, 3, 16, 1, 2, 300, "bf16"),
    small("ret_mlp2_d96", 96, 2, 2, 16, 2, 1, 77, "bf16"),
    small("ret_mlp2_d32_h64", 32, 2, 2, 4, 1, 1, 5, "bf16"),
]


@pytest.mark.parametrize("wl", RET_CASES, ids=lambda w: w.name)
def test_retrieve_many_rows(wl):
    say("case", wl)
    p = I.make_params(wl)
    g = GpuMemory(wl, p)
    ci = I.make_call(wl, p)
    d = dev_inputs(ci, "bf16")
    # store a first chunk-aligned prefix, then read every query
    n = (min(wl.seq, 256) // wl.chunk) * wl.chunk
    pre = {k: v[:, :n].contiguous() for k, v in d.items()}
    g.store(pre)
    ref = I.initial_state(wl, p)
    cp = I.CallInputs(*(np.ascontiguousarray(getattr(ci, f)[:, :n]) for f in ("k", "v", "q", "theta", "eta", "alpha")))
    oracle_forward(wl, ref, cp, with_q=False)
    before = g.export()
    y = g.retrieve(d["q"]).cpu().numpy()
    assert np.array_equal(before, g.export())
    yr = tmref.retrieve(wl.dim, wl.depth, wl.expansion, ref, ci.q)
    e = yerr(y, yr)
    say("  y %.2e" % e)
    assert np.all(np.isfinite(y)) and e < TOL["bf16"]
    g.close()


def test_call_split_and_determinism():
    wl = small("split", 64, 2, 2, 16, 2, 1, 96, "bf16")
    say("case", wl)
    p = I.make_params(wl)
    ci = I.make_call(wl, p)
    d = dev_inputs(ci, "bf16")
    g1 = GpuMemory(wl, p)
    y1 = g1.forward(d).cpu().numpy()
    s1 = g1.export()
    g2 = GpuMemory(wl, p)
    ys = []
    for a, b in ((0, 32), (32, 48), (48, 96)):
        part = {k: v[:, a:b].contiguous() for k, v in d.items()}
        ys.append(g2.forward(part).cpu().numpy())
    s2 = g2.export()
    g3 = GpuMemory(wl, p)
    y3 = g3.forward(d).cpu().numpy()
    s3 = g3.export()
    assert np.array_equal(y1, y3) and np.array_equal(s1, s3)         # run to run
    assert np.array_equal(s1, s2)                                     # split calls
    assert np.array_equal(y1, np.concatenate(ys, axis=1))
    assert g2.check() == (False, 96)
    for g in (g1, g2, g3):
        g.close()


def test_export_import_resume():
    wl = small("resume", 64, 2, 2, 16, 1, 2, 64, "bf16")
    say("case", wl)
    p = I.make_params(wl)
    c0 = dev_inputs(I.make_call(wl, p, 0), "bf16")
    c1 = dev_inputs(I.make_call(wl, p, 1), "bf16")
    g = GpuMemory(wl, p)
    g.forward(c0)
    mid = g.export()
    y_a = g.forward(c1).cpu().numpy()
    end_a = g.export()
    h = GpuMemory(wl, p)
    h.import_(mid)
    y_b = h.forward(c1).cpu().numpy()
    assert np.array_equal(y_a, y_b) and np.array_equal(end_a, h.export())
    g.close()
    h.close()


def test_linear64_workload():
    wl = I.WORKLOADS["linear64"]
    say("case", wl)
    ys_g, ys_r, st, ref, nf, pos = run_pair(wl)
    ey = yerr(ys_g[0], ys_r[0])
    em, es = compare_state(wl, st, ref)
    say("  y %.2e  M %.2e  S %.2e" % (ey, em, es))
    assert ey < 1e-4 and em < 1e-4 and es < 1e-4


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mlp384_workload(dtype):
    # the README-sized memory: (2, 1024, 384), chunk 64, depth 2, hidden 1536
    wl = I.WORKLOADS["mlp384"].replace(dtype=dtype)
    say("case", wl)
    ys_g, ys_r, st, ref, nf, pos = run_pair(wl)
    ey = yerr(ys_g[0], ys_r[0])
    em, es = compare_state(wl, st, ref)
    say("  y %.2e  M %.2e  S %.2e" % (ey, em, es))
    assert not nf and pos == 1024
    assert ey < TOL[dtype] and em < TOL[dtype]
    assert es < 2 * TOL[dtype]


def test_literal_gates_raise_the_nonfinite_flag():
    # gate offsets (0, 0, 0) on the dim-384 MLP: the exact state leaves the
    # float32 range within the call (pinned on the oracle), so the flag is set
    wl = I.WORKLOADS["mlp384"].replace(batch=1, offsets=(0.0, 0.0, 0.0))
    say("case", wl)
    p = I.make_params(wl)
    g = GpuMemory(wl, p)
    g.forward(dev_inputs(I.make_call(wl, p), "bf16"))
    nf, pos = g.check()
    assert nf and pos == 1024
    g.close()


def test_graph_replay_matches_direct_launches():
    # repeated calls on the same buffers are captured once and replayed as a
    # HIP graph; every replay (with eager work and syncs in between) must
    # equal the directly launched result bit for bit
    import test_trained_neural_amd as T
    wl = small("graph", 64, 2, 2, 16, 2, 1, 64, "bf16")
    say("case", wl)
    p = I.make_params(wl)
    d = dev_inputs(I.make_call(wl, p), "bf16")
    g = GpuMemory(wl, p)
    y = torch.empty((2, 64, 1, 64), dtype=torch.float32, device="cuda")
    ws = torch.empty(T.tm_workspace_bytes(g.ctx, 2, 1, 64), dtype=torch.uint8, device="cuda")
    args = (g.ctx, g.state, d["k"], d["v"], d["q"], d["theta"], d["eta"], d["alpha"], y, ws)
    try:
        T.tm_graphs_enable(False)
        T.tm_state_init(g.ctx, g.state, 2, 1, g.init)
        T.tm_forward(*args)
        y_ref, s_ref = y.cpu().numpy().copy(), g.export()
        T.tm_graphs_enable(True)
        for rep in range(4):
            y.fill_(float("nan"))
            T.tm_state_init(g.ctx, g.state, 2, 1, g.init)
            T.tm_forward(*args)
            torch.cuda.synchronize()
            assert np.array_equal(y.cpu().numpy(), y_ref), rep
            assert np.array_equal(g.export(), s_ref), rep
            assert g.check() == (False, 64)
            torch.cuda.synchronize()
    finally:
        T.tm_graphs_enable(True)
        g.close()


# depth 2: W_1's update in workgroups of its own (M_1 alternating with a
# workspace buffer) against the update in place in the first-layer blocks;
# even and odd numbers of chunks per call, forward and store-only, fp32 and
# bf16, and a second call carrying the state
SPLIT_CASES = [
    (small("w1s_even", 96, 2, 3, 24, 2, 1, 96, "f32"), (96,), "forward"),
    (small("w1s_odd", 96, 2, 3, 24, 2, 1, 72, "f32"), (72,), "forward"),
    (small("w1s_bf16", 64, 2, 2, 16, 1, 2, 80, "bf16"), (48, 32), "forward"),
    (small("w1s_store", 64, 2, 2, 16, 2, 1, 80, "bf16"), (80, 48), "store"),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: c[0].name)
def test_w1_split_matches_in_place(case):
    import test_trained_neural_amd as T
    wl, calls, mode = case
    say("case", wl, calls, mode)
    p = I.make_params(wl)
    out = []
    try:
        for split in (True, False):
            T.tm_w1_split_enable(split)
            g = GpuMemory(wl, p)
            ys = []
            for j, n in enumerate(calls):
                d = {k: v[:, :n].contiguous() for k, v in dev_inputs(I.make_call(wl, p, j), wl.dtype).items()}
                if mode == "forward":
                    ys.append(g.forward(d).cpu().numpy())
                else:
                    g.store(d)
            out.append((ys, g.export(), g.check()))
            g.close()
    finally:
        T.tm_w1_split_enable(True)
    (ya, sa, ca), (yb, sb, cb) = out
    assert ca == cb == (False, sum(calls))
    assert np.array_equal(sa, sb)
    for u, v in zip(ya, yb):
        assert np.array_equal(u, v)


# queries read before their chunk's write (TM_READ_BEFORE_WRITE) against the
# oracle's read-before-write order, on the small shapes and mlp384, two calls
# carrying the state; the state matches the read-after-write call bitwise
RB_CASES = [SMALL[0], SMALL[2], SMALL[3], SMALL[5], SMALL[2].replace(dtype="bf16", name="mlp96_bf16"),
            SMALL[4].replace(dtype="bf16", name="deep32x4_bf16")]


@pytest.mark.parametrize("wl", RB_CASES, ids=lambda w: w.name)
def test_read_before_write_parity(wl):
    import test_trained_neural_amd as T
    say("case", wl)
    p = I.make_params(wl)
    g = GpuMemory(wl, p)
    h = GpuMemory(wl, p)
    ref = I.initial_state(wl, p)
    tol = TOL[wl.dtype]
    for j in range(2):
        ci = I.make_call(wl, p, j)
        d = dev_inputs(ci, wl.dtype)
        y = g.forward(d, read=T.TM_READ_BEFORE_WRITE).cpu().numpy()
        h.forward(d)
        yr = oracle_forward(wl, ref, ci, read="before")
        ey = yerr(y, yr)
        em, es = compare_state(wl, g.export(), ref)
        say("  call %d: y %.2e  M %.2e  S %.2e" % (j, ey, em, es))
        assert ey < tol and em < tol and es < 2 * tol
        assert np.array_equal(g.export(), h.export())
    assert g.check() == (False, 2 * wl.seq)
    g.close()
    h.close()


def test_read_before_write_mlp384():
    import test_trained_neural_amd as T
    wl = I.WORKLOADS["mlp384"]
    say("case", wl)
    p = I.make_params(wl)
    ci = I.make_call(wl, p)
    g = GpuMemory(wl, p)
    y = g.forward(dev_inputs(ci, "bf16"), read=T.TM_READ_BEFORE_WRITE).cpu().numpy()
    ref = I.initial_state(wl, p)
    yr = oracle_forward(wl, ref, ci, read="before")
    ey = yerr(y, yr)
    em, es = compare_state(wl, g.export(), ref)
    say("  y %.2e  M %.2e  S %.2e" % (ey, em, es))
    assert ey < TOL["bf16"] and em < TOL["bf16"] and es < 2 * TOL["bf16"]
    g.close()
