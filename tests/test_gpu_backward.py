"""tm_backward (the backward through the store) through the C ABI against
the backward oracle (oracle/backward.py: float64 autograd through the
literal recurrence) on the same seeded inputs: dk, dv, dq, dtheta, deta,
dalpha and the gradient with respect to the state before the call, for
depth 1 to 4, chunks 1, 5, 8, 16 and 24, widths that are not multiples of
the 64-wide tiles, several streams and heads, both read orders, bf16 and
fp32 inputs, a nonzero starting momentum and a nonzero gradient arriving
for the state after the call; the dim-384 memory over a 256-token prefix;
two calls chained through dstate; graph replay and run-to-run determinism.

The backward runs fp32 arithmetic for both input types (bf16 inputs are
exact in fp32), so every case is held to the fp32 tolerance, 1e-4, by the
element-wise measures of tests/harness.py.

Source: "titans-pytorch analysis", Editorial conclusion; "Titans,
explained", steps 2-6.
"""
import numpy as np
import pytest
import torch

import test_trained_neural_amd as T
from harness import TOL, compare_state, say, yerr
from oracle import backward as BW
from test_trained_neural_amd import inputs as I

pytestmark = pytest.mark.gpu

NAMES = ("dk", "dv", "dq", "dtheta", "deta", "dalpha")


def case(name, dim, depth, ex, chunk, B, H, Tn, dtype, read="after", offsets=(-4.0, 1.0, -4.0)):
    return (I.Workload(name, batch=B, seq=Tn, heads=H, dim=dim, depth=depth, expansion=ex, chunk=chunk,
                       dtype=dtype, offsets=offsets), read)


CASES = [
    case("b_lin", 32, 1, 1, 8, 2, 1, 32, "f32"),
    case("b_mlp", 64, 2, 2, 16, 1, 2, 48, "f32"),
    case("b_mlp_bf16", 64, 2, 2, 16, 2, 1, 48, "bf16"),
    case("b_deep3", 32, 3, 2, 5, 1, 2, 20, "f32"),
    case("b_deep4", 32, 4, 2, 8, 1, 1, 24, "f32", "before"),
    case("b_ragged", 96, 2, 3, 24, 1, 1, 48, "f32"),
    case("b_chunk1", 32, 2, 2, 1, 1, 1, 6, "f32"),
    case("b_before_bf16", 64, 2, 2, 16, 1, 1, 32, "bf16", "before"),
]


class Setup:
    """A memory whose starting state (M from the workload's init, a random
    momentum S) is imported, the call's inputs, and a random dy and dstate."""

    def __init__(self, wl, seed=0, tokens=None, s_scale=0.05):
        self.wl = wl
        self.p = I.make_params(wl)
        self.ci = I.make_call(wl, self.p, 0, tokens=tokens)
        B, Tn, H, d = self.ci.k.shape
        self.B, self.Tn, self.H = B, Tn, H
        rng = np.random.default_rng([seed, 7])
        st = I.initial_state(wl, self.p)
        P = wl.params
        st[:, P:] = rng.standard_normal((B * H, P)) * s_scale / np.sqrt(wl.dim)
        self.st = st.astype(np.float32).astype(np.float64)
        self.dy = rng.standard_normal((B, Tn, H, d))
        self.dst = (rng.standard_normal((B * H, 2 * P)) * 0.1).astype(np.float32).astype(np.float64)
        self.ctx = T.tm_create(wl.dim, wl.depth, wl.expansion, wl.chunk)
        self.state = torch.empty(T.tm_state_bytes(self.ctx, B, H), dtype=torch.uint8, device="cuda")
        T.tm_state_import(self.ctx, self.state, B, H, torch.from_numpy(self.st.astype(np.float32)).cuda())
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        self.d = {n: torch.from_numpy(np.ascontiguousarray(getattr(self.ci, n))).cuda().to(tdt).contiguous()
                  for n in ("k", "v", "q")}
        for n in ("theta", "eta", "alpha"):
            self.d[n] = torch.from_numpy(np.ascontiguousarray(getattr(self.ci, n))).cuda().contiguous()
        self.ws = torch.empty(T.tm_backward_workspace_bytes(self.ctx, B, H, Tn), dtype=torch.uint8, device="cuda")

    def gpu(self, read="after", dst=None, dy=None):
        d = self.d
        dyt = torch.from_numpy((self.dy if dy is None else dy).astype(np.float32)).cuda().contiguous()
        dstate = torch.from_numpy((self.dst if dst is None else dst).astype(np.float32)).cuda().contiguous()
        out = {n: torch.empty_like(d["k"], dtype=torch.float32) for n in ("dk", "dv", "dq")}
        for n in ("dtheta", "deta", "dalpha"):
            out[n] = torch.empty_like(d["theta"])
        rd = T.TM_READ_AFTER_WRITE if read == "after" else T.TM_READ_BEFORE_WRITE
        T.tm_backward(self.ctx, self.state, d["k"], d["v"], d["q"], d["theta"], d["eta"], d["alpha"], dyt, dstate,
                      out["dk"], out["dv"], out["dq"], out["dtheta"], out["deta"], out["dalpha"], self.ws, rd)
        res = {n: t.cpu().numpy() for n, t in out.items()}
        res["dstate_in"] = dstate.cpu().numpy()
        return res

    def oracle(self, read="after"):
        ci = self.ci
        return BW.forward_backward(self.wl.dim, self.wl.depth, self.wl.expansion, self.wl.chunk, self.st, ci.k, ci.v,
                                   ci.q, ci.theta, ci.eta, ci.alpha, self.dy, self.dst, read=read)

    def close(self):
        T.tm_destroy(self.ctx)


def check(wl, got, ref, tol):
    errs = {n: yerr(got[n], ref[n]) for n in NAMES}
    em, es = compare_state(wl, got["dstate_in"], ref["dstate_in"])
    say("  " + "  ".join("%s %.1e" % (n, e) for n, e in errs.items()) + "  dM0 %.1e  dS0 %.1e" % (em, es))
    for n, e in errs.items():
        assert e < tol, n
    assert em < tol and es < tol


@pytest.mark.parametrize("c", CASES, ids=lambda c: c[0].name)
def test_backward_parity(c):
    wl, read = c
    say("case", wl, read)
    s = Setup(wl)
    before = s.state.clone()
    got = s.gpu(read)
    torch.cuda.synchronize()
    assert torch.equal(s.state, before)          # the starting state is read only
    check(wl, got, s.oracle(read), TOL["f32"])
    s.close()


def test_backward_mlp384_prefix():
    # the dim-384 memory (2 streams, bf16 inputs, chunk 64) over its first
    # 256 tokens (4 chunks), reading after the write
    wl = I.WORKLOADS["mlp384"]
    say("case", wl, "256 tokens")
    s = Setup(wl, tokens=256)
    check(wl, s.gpu(), s.oracle(), TOL["f32"])
    s.close()


def test_backward_chains_two_calls():
    # calls of 32 then 16 tokens: the second call's backward from the state
    # the first left, its dstate fed to the first's; against the oracle's
    # backward of the whole 48 tokens
    wl, _ = case("b_chain", 64, 2, 2, 16, 1, 2, 48, "f32")
    say("case", wl)
    s = Setup(wl)
    ref = s.oracle()
    d = s.d
    cut = lambda t, a, b: t[:, a:b].contiguous()
    # the state after the first call, from the forward (on a copy of the
    # starting state, set up by import)
    st1 = torch.empty_like(s.state)
    T.tm_state_import(s.ctx, st1, 1, 2, torch.from_numpy(s.st.astype(np.float32)).cuda())
    ws = torch.empty(T.tm_workspace_bytes(s.ctx, 1, 2, 32), dtype=torch.uint8, device="cuda")
    y1 = torch.empty((1, 32, 2, 64), device="cuda")
    T.tm_forward(s.ctx, st1, *(cut(d[n], 0, 32) for n in ("k", "v", "q", "theta", "eta", "alpha")), y1, ws)
    dst = torch.from_numpy(s.dst.astype(np.float32)).cuda().contiguous()
    outs = []
    for (a, b), stt in (((32, 48), st1), ((0, 32), s.state)):
        o = {n: torch.empty((1, b - a, 2, 64), device="cuda") for n in ("dk", "dv", "dq")}
        for n in ("dtheta", "deta", "dalpha"):
            o[n] = torch.empty((1, b - a, 2), device="cuda")
        wsb = torch.empty(T.tm_backward_workspace_bytes(s.ctx, 1, 2, b - a), dtype=torch.uint8, device="cuda")
        dyt = torch.from_numpy(s.dy[:, a:b].astype(np.float32)).cuda().contiguous()
        T.tm_backward(s.ctx, stt, *(cut(d[n], a, b) for n in ("k", "v", "q", "theta", "eta", "alpha")), dyt, dst,
                      o["dk"], o["dv"], o["dq"], o["dtheta"], o["deta"], o["dalpha"], wsb)
        outs.append({n: t.cpu().numpy() for n, t in o.items()})
    got = {n: np.concatenate([outs[1][n], outs[0][n]], axis=1) for n in NAMES}
    got["dstate_in"] = dst.cpu().numpy()
    check(wl, got, ref, TOL["f32"])
    s.close()


def test_backward_graph_replay_and_determinism():
    # the same call three times: the first launches directly, the second is
    # captured, the third replays; all bitwise equal
    wl, _ = case("b_graph", 64, 3, 2, 16, 2, 1, 48, "bf16")
    say("case", wl)
    s = Setup(wl)
    runs = [s.gpu() for _ in range(3)]
    for r in runs[1:]:
        for n in NAMES + ("dstate_in",):
            assert np.array_equal(r[n], runs[0][n]), n
    s.close()
