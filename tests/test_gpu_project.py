"""The input side (tm_project) through the C ABI against the fp64 oracle
(oracle/prologue.py) on the same seeded inputs: keys, values, queries and the
gates, the history carried across calls, and the whole chain from the
tokens' model vectors to the memory's output (tm_project then tm_forward,
against the input oracle then the memory oracle).  Tolerances: relative
Frobenius error per tensor, 1e-4 for fp32, 2e-2 for bf16 (the outputs are
rounded to bf16); the fp32 gates 1e-4 in both."""
import numpy as np
import pytest
import torch

import test_trained_neural_amd as T
from harness import GpuMemory, TOL, compare_state, relerr, say, yerr
from oracle import prologue as PR
from oracle import tmref
from test_trained_neural_amd import inputs as I

pytestmark = pytest.mark.gpu


def wl_of(name, B, T, H, d, dtype):
    return I.Workload(name, batch=B, seq=T, heads=H, dim=d, depth=2, expansion=2, chunk=16, dtype=dtype,
                      offsets=(-4.0, 1.0, -4.0))


class GpuProject:
    def __init__(self, wl, pi):
        self.wl = wl
        self.ctx = T.tm_create(wl.dim, 2, 2, 16)
        dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        self.dt = dt
        # the GPU takes W as [3][H*d][D] (one row per output channel)
        self.w = torch.from_numpy(np.ascontiguousarray(pi.w_kvq.transpose(0, 2, 1))).to("cuda").to(dt).contiguous()
        self.conv = torch.from_numpy(pi.conv).to("cuda").contiguous()
        self.wg = torch.from_numpy(np.ascontiguousarray(pi.w_gate.transpose(0, 2, 1))).to("cuda").contiguous()
        self.gb = torch.from_numpy(pi.gate_bias).to("cuda").contiguous()
        K = pi.conv.shape[-1]
        self.hist = (torch.zeros((wl.batch, K - 1, 3, wl.model_dim), dtype=torch.float32, device="cuda")
                     if K > 1 else None)

    def __call__(self, x):
        B, Tn, D = x.shape
        H, d = self.wl.heads, self.wl.dim
        xd = torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(self.dt).contiguous()
        k, v, q = (torch.empty((B, Tn, H, d), dtype=self.dt, device="cuda") for _ in range(3))
        g = [torch.empty((B, Tn, H), dtype=torch.float32, device="cuda") for _ in range(3)]
        T.tm_project(self.ctx, xd, self.w, self.conv, self.wg, self.gb, self.hist, k, v, q, g[0], g[1], g[2], H)
        return [t.float().cpu().numpy() for t in (k, v, q)] + [t.cpu().numpy() for t in g]


CASES = [
    # the README shape: (2, 1024) tokens of width 384, one head
    (wl_of("p384", 2, 1024, 1, 384, "bf16"), 4),
    # 8 heads of 128 over a model width of 1024
    (wl_of("p8x128", 2, 96, 8, 128, "bf16"), 4),
    (wl_of("p_f32", 2, 40, 2, 32, "f32"), 3),
    # the widest head (dim 1024: 16-token tiles)
    (wl_of("p1024", 1, 48, 1, 1024, "f32"), 4),
    # one tap: no convolution
    (wl_of("p_k1", 1, 33, 2, 64, "bf16"), 1),
    # calls long enough for the 32-token tiles (their grid covers the compute
    # units): 8 heads of 128 with a ragged last tile; fp32 with two heads and
    # a ragged last tile
    (wl_of("p8x128_long", 2, 340, 8, 128, "bf16"), 4),
    (wl_of("p_f32_long", 4, 1000, 2, 64, "f32"), 3),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0].name)
def test_project_parity(case):
    wl, K = case
    say("case", wl, "taps", K)
    p = I.make_params(wl)
    pi = I.make_prologue(wl, p, conv_len=K)
    g = GpuProject(wl, pi)
    got = g(pi.x)
    ref = PR.project(pi.x, pi.w_kvq, pi.conv, pi.w_gate, pi.gate_bias, wl.heads)
    tol = TOL[wl.dtype]
    for n, a, r in zip(("k", "v", "q", "theta", "eta", "alpha"), got, ref[:6]):
        e = yerr(a, r)
        say("  %s %.2e" % (n, e))
        assert e < (tol if n in ("k", "v", "q") else 1e-4), n
    if K > 1:
        e = relerr(g.hist.cpu().numpy(), ref[6])
        say("  history %.2e" % e)
        assert e < 1e-4
    T.tm_destroy(g.ctx)


@pytest.mark.parametrize("wl,cuts", [
    # calls of 37, 2 (shorter than the history) and 57 tokens (16-token tiles)
    (wl_of("p_hist", 2, 96, 2, 64, "f32"), (0, 37, 39, 96)),
    # calls of 300, 2 and 405 tokens: the long ones on 32-token tiles
    (wl_of("p_hist_long", 4, 707, 2, 64, "f32"), (0, 300, 302, 707)),
], ids=lambda x: x.name if hasattr(x, "name") else "")
def test_project_history_across_calls(wl, cuts):
    # consecutive calls equal one call
    say("case", wl, cuts)
    p = I.make_params(wl)
    pi = I.make_prologue(wl, p, conv_len=4)
    ref = PR.project(pi.x, pi.w_kvq, pi.conv, pi.w_gate, pi.gate_bias, wl.heads)
    g = GpuProject(wl, pi)
    parts = [g(pi.x[:, a:b]) for a, b in zip(cuts[:-1], cuts[1:])]
    for i, n in enumerate(("k", "v", "q", "theta", "eta", "alpha")):
        e = yerr(np.concatenate([pp[i] for pp in parts], axis=1), ref[i])
        say("  %s %.2e" % (n, e))
        assert e < 1e-4, n
    assert relerr(g.hist.cpu().numpy(), ref[6]) < 1e-4
    T.tm_destroy(g.ctx)


def test_tokens_to_memory_output():
    # tm_project then tm_forward against the input oracle then the memory
    # oracle (the memory oracle fed the input oracle's fp64 keys and values
    # rounded as the GPU's are: to bf16).  The MLP workloads' gate offsets:
    # with larger write gates the memory diverges on these inputs, in the
    # oracle too
    wl = I.Workload("chain", batch=2, seq=256, heads=2, dim=64, depth=2, expansion=4, chunk=32, dtype="bf16",
                    offsets=(-7.0, 2.0, -7.0))
    say("case", wl)
    p = I.make_params(wl)
    pi = I.make_prologue(wl, p, conv_len=4)
    g = GpuProject(wl, pi)
    B, Tn, H, d = wl.batch, wl.seq, wl.heads, wl.dim
    xd = torch.from_numpy(pi.x).to("cuda").to(torch.bfloat16).contiguous()
    k, v, q = (torch.empty((B, Tn, H, d), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    gt = [torch.empty((B, Tn, H), dtype=torch.float32, device="cuda") for _ in range(3)]
    T.tm_project(g.ctx, xd, g.w, g.conv, g.wg, g.gb, g.hist, k, v, q, gt[0], gt[1], gt[2], H)
    mem = GpuMemory(wl, p)
    y = mem.forward({"k": k, "v": v, "q": q, "theta": gt[0], "eta": gt[1], "alpha": gt[2]}).cpu().numpy()
    rk, rv, rq, rth, ret, ral, _ = PR.project(pi.x, pi.w_kvq, pi.conv, pi.w_gate, pi.gate_bias, H)
    ci = I.CallInputs(*(I.round_bf16(a.astype(np.float32)) for a in (rk, rv, rq)),
                      *(a.astype(np.float32) for a in (rth, ret, ral)))
    ref = I.initial_state(wl, p)
    yr = tmref.forward(wl.dim, wl.depth, wl.expansion, wl.chunk, ref, ci.k, ci.v, ci.theta, ci.eta, ci.alpha,
                       q=ci.q)
    ey = yerr(y, yr)
    em, es = compare_state(wl, mem.export(), ref)
    say("  y %.2e  M %.2e  S %.2e" % (ey, em, es))
    assert ey < TOL["bf16"] and em < TOL["bf16"] and es < 2 * TOL["bf16"]
    mem.close()
    T.tm_destroy(g.ctx)
