"""The memory-as-context wiring on the GPU against its oracle: the window and
the gate bit for bit on the same inputs, and two segments chained through
the memory (queries before the write, the attention output written, its read
gating it) against the oracle chain (the input-side oracle, the memory
oracle and the wiring oracle) with a fixed stand-in for attention.

Source: "Titans, explained" step 8; "Attack of the Titans", Technical
Details, memory as a context."""
import numpy as np
import pytest
import torch

from harness import TOL, relerr, say, yerr
from oracle import mac, prologue, tmref
from test_gpu_parity import small
from test_trained_neural_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,P", [("bf16", 4), ("f32", 0), ("bf16", 0)])
def test_window_and_gate_bit_exact(dtype, P):
    import test_trained_neural_amd as T
    rng = np.random.default_rng(5)
    B, S, D = 3, 24, 96
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    pers = rng.standard_normal((P, D)).astype(np.float32)
    rec = rng.standard_normal((B, S, D)).astype(np.float32)
    seg = rng.standard_normal((B, S, D)).astype(np.float32)
    if dtype == "bf16":
        pers, seg = mac.round_to_bf16(pers).astype(np.float32), mac.round_to_bf16(seg).astype(np.float32)
    dev = "cuda"
    tp = torch.from_numpy(pers).to(dev).to(tdt) if P else None
    tr = torch.from_numpy(rec).to(dev)
    ts = torch.from_numpy(seg).to(dev).to(tdt)
    w = torch.empty((B, P + 2 * S, D), dtype=tdt, device=dev)
    T.tm_mac_window(tp, tr, ts, w)
    want = mac.window(pers if P else None, rec, seg, dtype == "bf16")
    assert np.array_equal(w.float().cpu().numpy().astype(np.float64), want)
    out = torch.empty((B, S, D), dtype=torch.float32, device=dev)
    T.tm_mac_gate(ts, tr, out)
    # one fp32 rounding of an exact product on both sides
    assert np.array_equal(out.cpu().numpy(), (seg * rec).astype(np.float32))


def stand_in_attention(window, S):
    """A fixed stand-in for attention (the caller's in a model), fp64: each
    segment position mixes its own row with the window's mean row; the
    result is rounded to bfloat16, the dtype it is handed back in."""
    return mac.round_to_bf16(window[:, -S:] + 0.5 * window.mean(axis=1, keepdims=True))


def test_mac_segments_chain():
    import test_trained_neural_amd as T
    wl = small("mac", 64, 2, 2, 16, 2, 2, 64, "bf16", offsets=(-4.5, 1.0, -6.0))
    say("case", wl)
    H, d, S, P = wl.heads, wl.dim, 32, 4
    D = H * d
    p = I.make_params(wl)
    pi = I.make_prologue(wl, p, conv_len=2)
    x = pi.x                                             # [B][2S][D], bf16 values
    rng = np.random.default_rng(9)
    pers = mac.round_to_bf16(rng.standard_normal((P, D)).astype(np.float32))
    dev = "cuda"
    bf = torch.bfloat16
    mem = T.NeuralMemory(d, wl.depth, wl.expansion, wl.chunk, device=dev)
    st = mem.init_state(wl.batch, H, torch.from_numpy(p.init_weights))
    w_kvq = torch.from_numpy(np.ascontiguousarray(pi.w_kvq.transpose(0, 2, 1))).to(dev).to(bf)
    conv = torch.from_numpy(pi.conv).to(dev)
    wg = torch.from_numpy(np.ascontiguousarray(pi.w_gate.transpose(0, 2, 1))).to(dev)
    gb = torch.from_numpy(pi.gate_bias).to(dev)
    hx = torch.zeros((wl.batch, 1, 3, D), dtype=torch.float32, device=dev)
    hy = torch.zeros_like(hx)
    tpers = torch.from_numpy(pers.astype(np.float32)).to(dev).to(bf)

    def attention(window):
        w = window.float()
        return (w[:, -S:] + 0.5 * w.mean(dim=1, keepdim=True)).to(bf)

    # the oracle chain, fp64
    ref = I.initial_state(wl, p)
    rhx = rhy = None
    for sgi in range(2):
        xs = x[:, sgi * S:(sgi + 1) * S]
        out, st = T.mac_segment(mem, st, torch.from_numpy(np.ascontiguousarray(xs)).to(dev).to(bf), tpers,
                                attention, w_kvq, conv, wg, gb, H, hx, hy)
        kx, vx, qx, _, _, _, rhx = prologue.project(xs, pi.w_kvq, pi.conv, pi.w_gate, pi.gate_bias, H, rhx)
        rec = tmref.retrieve(d, wl.depth, wl.expansion, ref, qx.astype(np.float32)).reshape(wl.batch, S, D)
        win = mac.window(pers, rec, xs, bf16=True)
        y = stand_in_attention(win, S)
        ky, vy, qy, th, et, al, rhy = prologue.project(y, pi.w_kvq, pi.conv, pi.w_gate, pi.gate_bias, H, rhy)
        tmref.forward(d, wl.depth, wl.expansion, wl.chunk, ref, ky, vy, th, et, al)
        my = tmref.retrieve(d, wl.depth, wl.expansion, ref, qy.astype(np.float32)).reshape(wl.batch, S, D)
        want = mac.gate(y, my)
        e = yerr(out.cpu().numpy(), want)
        say("  segment %d: out %.2e" % (sgi, e))
        assert np.all(np.isfinite(want)) and e < TOL["bf16"]
    assert mem.check(st) == (False, 2 * S)


def test_mac_timing_class():
    """Both wiring kernels are counted under their timing class, and the
    timed launches give the same bytes."""
    import test_trained_neural_amd as T
    B, S, D, P = 2, 16, 64, 3
    g = torch.Generator().manual_seed(4)
    pers_c = torch.randn((P, D), generator=g, dtype=torch.float32).to(torch.bfloat16)
    rec_c = torch.randn((B, S, D), generator=g, dtype=torch.float32)
    seg_c = torch.randn((B, S, D), generator=g, dtype=torch.float32).to(torch.bfloat16)
    want_w = torch.cat([pers_c[None].expand(B, P, D), rec_c.to(torch.bfloat16), seg_c], dim=1)
    want_o = seg_c.float() * rec_c
    pers, rec, seg = pers_c.cuda(), rec_c.cuda(), seg_c.cuda()
    for mask in (0, 1 << T.K_MAC):
        T.tm_timing_enable(mask)
        T.tm_timing_read(T.K_MAC)
        w = torch.empty((B, P + 2 * S, D), dtype=torch.bfloat16, device="cuda")
        o = torch.empty((B, S, D), dtype=torch.float32, device="cuda")
        T.tm_mac_window(pers, rec, seg, w)
        T.tm_mac_gate(seg, rec, o)
        torch.cuda.synchronize()
        ms, n = T.tm_timing_read(T.K_MAC)
        T.tm_timing_enable(0)
        assert n == (2 if mask else 0) and (ms > 0) == bool(mask)
        bw = (w.cpu() != want_w).nonzero().tolist()
        bo = (o.cpu() != want_o).nonzero().tolist()
        say("mask %d: window mismatches %d %s, gate mismatches %d %s" % (mask, len(bw), bw[:4], len(bo), bo[:4]))
        assert not bw and not bo


def test_mac_segment_buffers():
    """mac_segment reuses the memory's buffers across segments: an output
    it returned is untouched by the next segment, a change of segment length
    takes new buffers, and every segment equals the same segment run by a
    memory with no buffers kept (the state carried alike)."""
    import test_trained_neural_amd as T
    wl = small("macbuf", 64, 2, 2, 16, 2, 2, 64, "bf16", offsets=(-4.5, 1.0, -6.0))
    H, d, P = wl.heads, wl.dim, 2
    D = H * d
    p = I.make_params(wl)
    pi = I.make_prologue(wl, p, conv_len=2)
    dev, bf = "cuda", torch.bfloat16
    x = torch.from_numpy(pi.x).to(dev).to(bf)
    w_kvq = torch.from_numpy(np.ascontiguousarray(pi.w_kvq.transpose(0, 2, 1))).to(dev).to(bf)
    conv = torch.from_numpy(pi.conv).to(dev)
    wg = torch.from_numpy(np.ascontiguousarray(pi.w_gate.transpose(0, 2, 1))).to(dev)
    gb = torch.from_numpy(pi.gate_bias).to(dev)
    pers = torch.from_numpy(np.random.default_rng(2).standard_normal((P, D)).astype(np.float32)).to(dev).to(bf)
    init = torch.from_numpy(p.init_weights)

    def attention(window):
        S = (window.shape[1] - P) // 2
        return window[:, P + S:] * 0.5 + window[:, P:P + S] * 0.25

    mem = T.NeuralMemory(d, wl.depth, wl.expansion, wl.chunk, device=dev)
    st = mem.init_state(wl.batch, H, init)
    hx = torch.zeros((wl.batch, 1, 3, D), dtype=torch.float32, device=dev)
    hy = torch.zeros_like(hx)
    ref_st = mem.init_state(wl.batch, H, init)
    rhx, rhy = torch.zeros_like(hx), torch.zeros_like(hx)
    outs, keep, t = [], [], 0
    for S in (32, 16, 16):
        xs = x[:, t:t + S].contiguous()
        t += S
        out, st = T.mac_segment(mem, st, xs, pers, attention, w_kvq, conv, wg, gb, H, hx, hy)
        outs.append(out)
        keep.append(out.clone())
        fresh = T.NeuralMemory(d, wl.depth, wl.expansion, wl.chunk, device=dev)   # no buffers kept
        want, ref_st = T.mac_segment(fresh, ref_st, xs, pers, attention, w_kvq, conv, wg, gb, H, rhx, rhy)
        assert torch.equal(out, want)
    torch.cuda.synchronize()
    for o, k in zip(outs, keep):
        assert torch.equal(o, k)
    assert mem.check(st) == (False, 64)
