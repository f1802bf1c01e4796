"""Per-token read (TM_READ_PER_TOKEN: every query through the memory as its
own token's write left it, the gradients at the chunk start) against the
oracle's per-token order on y (per tensor, per token row and per element:
harness.yerr) and on the state after each call (per weight matrix and per
element: harness.compare_state).  The small shapes span ragged chunks (5, 24 tokens), a chunk of
one token, several streams and heads, depth 1 to 4, and both operand types;
mlp384 runs at full size.

Source: "Attack of the Titans" (synthesis.ai), the long-term memory section
and Technical Details / Parallel training; "Titans, explained" steps 3-6.
"""
import numpy as np
import pytest
import torch

from harness import GpuMemory, TOL, compare_state, dev_inputs, oracle_forward, relerr, say, yerr
from test_gpu_parity import SMALL, small
from test_gpu_workloads import MAX
from test_trained_neural_amd import inputs as I

pytestmark = pytest.mark.gpu

CASES = SMALL + [SMALL[2].replace(dtype="bf16", name="mlp96_bf16"),
                 SMALL[4].replace(dtype="bf16", name="deep32x4_bf16"),
                 SMALL[0].replace(dtype="bf16", name="lin32_bf16")]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_per_token_read_parity(wl):
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
        y = g.forward(d, read=T.TM_READ_PER_TOKEN).cpu().numpy()
        h.forward(d)
        yr = oracle_forward(wl, ref, ci, read="token")
        ey = yerr(y, yr)
        em, es = compare_state(wl, g.export(), ref)
        ed = relerr(g.export(), h.export())
        say("  call %d: y %.2e  M %.2e  S %.2e  state vs read-after-write %.2e" % (j, ey, em, es, ed))
        assert np.all(np.isfinite(y))
        assert ey < tol and em < tol and es < 2 * tol
        # the read takes nothing from the write: the state matches the
        # read-after-write call's (same products; W_1's update placement may
        # differ, which is bitwise neutral)
        assert np.array_equal(g.export(), h.export())
    assert g.check() == (False, 2 * wl.seq)
    g.close()
    h.close()


@pytest.mark.parametrize("wl", [w for w in MAX], ids=lambda w: w.name)
def test_per_token_read_maximum_sizes(wl):
    # the widest memory (dim 1024: layer 1's scores with K = 2048) and the
    # deepest (8 weight matrices, six of them in the row-major layout)
    import test_trained_neural_amd as T
    say("case", wl)
    p = I.make_params(wl)
    ci = I.make_call(wl, p)
    g = GpuMemory(wl, p)
    y = g.forward(dev_inputs(ci, wl.dtype), read=T.TM_READ_PER_TOKEN).cpu().numpy()
    ref = I.initial_state(wl, p)
    yr = oracle_forward(wl, ref, ci, read="token")
    ey = yerr(y, yr)
    em, es = compare_state(wl, g.export(), ref)
    say("  y %.2e  M %.2e  S %.2e" % (ey, em, es))
    tol = TOL[wl.dtype]
    assert np.all(np.isfinite(ref))
    assert ey < tol and em < tol and es < 2 * tol
    g.close()


def test_per_token_read_mlp384():
    import test_trained_neural_amd as T
    wl = I.WORKLOADS["mlp384"]
    say("case", wl)
    p = I.make_params(wl)
    ci = I.make_call(wl, p)
    g = GpuMemory(wl, p)
    y = g.forward(dev_inputs(ci, "bf16"), read=T.TM_READ_PER_TOKEN).cpu().numpy()
    ref = I.initial_state(wl, p)
    yr = oracle_forward(wl, ref, ci, read="token")
    ey = yerr(y, yr)
    em, es = compare_state(wl, g.export(), ref)
    say("  y %.2e  M %.2e  S %.2e" % (ey, em, es))
    assert ey < TOL["bf16"] and em < TOL["bf16"] and es < 2 * TOL["bf16"]
    g.close()


@pytest.mark.parametrize("depth", [1, 2, 3])
def test_per_token_read_graph_replay_matches_direct_launches(depth):
    # repeated per-token calls on the same buffers replay as a HIP graph;
    # every replay (eager work and syncs in between) equals the directly
    # launched result bit for bit
    import test_trained_neural_amd as T
    wl = small("graph_r3_d%d" % depth, 64, depth, 2, 16, 2, 1, 64, "bf16")
    say("case", wl)
    p = I.make_params(wl)
    d = dev_inputs(I.make_call(wl, p), "bf16")
    g = GpuMemory(wl, p)
    y = torch.empty((2, 64, 1, 64), dtype=torch.float32, device="cuda")
    ws = torch.empty(T.tm_workspace_bytes(g.ctx, 2, 1, 64), dtype=torch.uint8, device="cuda")
    args = (g.ctx, g.state, d["k"], d["v"], d["q"], d["theta"], d["eta"], d["alpha"], y, ws, T.TM_READ_PER_TOKEN)
    try:
        T.tm_graphs_enable(False)
        T.tm_state_init(g.ctx, g.state, 2, 1, g.init)
        T.tm_forward_ex(*args)
        y_ref, s_ref = y.cpu().numpy().copy(), g.export()
        T.tm_graphs_enable(True)
        for rep in range(4):
            y.fill_(float("nan"))
            T.tm_state_init(g.ctx, g.state, 2, 1, g.init)
            T.tm_forward_ex(*args)
            torch.cuda.synchronize()
            assert np.array_equal(y.cpu().numpy(), y_ref), rep
            assert np.array_equal(g.export(), s_ref), rep
            torch.cuda.synchronize()
    finally:
        T.tm_graphs_enable(True)
        g.close()
