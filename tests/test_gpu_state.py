"""The state header check (tm_state_check): a state made for one memory
configuration, batch and head count is refused for another, and a state
whose header is damaged is refused; the refusal is TM_ERR_STATE."""
import numpy as np
import pytest
import torch

from harness import GpuMemory, say
from test_gpu_parity import small
from test_trained_neural_amd import inputs as I

pytestmark = pytest.mark.gpu


def test_state_header_mismatch_is_refused():
    import test_trained_neural_amd as T
    wl = small("hdr", 64, 2, 2, 16, 2, 1, 32, "bf16")
    say("case", wl)
    p = I.make_params(wl)
    g = GpuMemory(wl, p)
    assert g.check() == (False, 0)
    other = T.tm_create(128, 2, 2, 16)   # another configuration
    try:
        for ctx, B, H in ((other, 2, 1), (g.ctx, 1, 1), (g.ctx, 2, 2)):
            with pytest.raises(T.TMError) as e:
                T.tm_state_check(ctx, g.state, B, H)
            assert e.value.code == T.TM_ERR_STATE
        # a damaged header (the magic word cleared)
        g.state[:4].zero_()
        torch.cuda.synchronize()
        with pytest.raises(T.TMError) as e:
            T.tm_state_check(g.ctx, g.state, 2, 1)
        assert e.value.code == T.TM_ERR_STATE
        # a fresh init restores it
        T.tm_state_init(g.ctx, g.state, 2, 1, g.init)
        assert T.tm_state_check(g.ctx, g.state, 2, 1) == (False, 0)
    finally:
        T.tm_destroy(other)
        g.close()


def test_nan_input_sets_the_nonfinite_flag():
    # a NaN in one key poisons the memory; the step kernels raise the sticky
    # non-finite flag, as the oracle's state turns non-finite too
    import test_trained_neural_amd as T
    from harness import dev_inputs, oracle_forward
    wl = small("nanflag", 64, 2, 2, 16, 1, 1, 64, "f32")
    say("case", wl)
    p = I.make_params(wl)
    ci = I.make_call(wl, p)
    ci.k[0, 20, 0, 3] = np.nan
    g = GpuMemory(wl, p)
    g.forward(dev_inputs(ci, "f32"))
    nf, pos = g.check()
    ref = I.initial_state(wl, p)
    oracle_forward(wl, ref, ci)
    assert not np.all(np.isfinite(ref))
    assert nf and pos == 64
    # the flag is sticky: a clean call after it leaves it set
    g.forward(dev_inputs(I.make_call(wl, p, 1), "f32"))
    assert g.check()[0]
    g.close()


def test_compute_calls_refuse_a_mismatched_state():
    # a state set up for batch 1 passed with batch 2 (or another head count,
    # or another configuration) is refused on the host with TM_ERR_STATE,
    # nothing launched: the state's bytes and the output stay as they were
    import ctypes
    import test_trained_neural_amd as T
    from harness import dev_inputs
    wl = small("mismatch", 64, 2, 2, 16, 1, 1, 32, "bf16")
    say("case", wl)
    p = I.make_params(wl)
    g = GpuMemory(wl, p)                      # batch 1
    d = dev_inputs(I.make_call(wl.replace(batch=2), p), "bf16")   # inputs of batch 2
    L = T.lib()
    y = torch.full((2, 32, 1, 64), 7.0, device="cuda")
    ws = torch.empty(T.tm_workspace_bytes(g.ctx, 2, 1, 32), dtype=torch.uint8, device="cuda")
    before = g.state.clone()
    torch.cuda.synchronize()
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = (ptr(d["k"]), ptr(d["v"]), ptr(d["q"]), ptr(d["theta"]), ptr(d["eta"]), ptr(d["alpha"]), ptr(y))
    assert L.tm_forward(g.ctx, ptr(g.state), *args, 2, 1, 32, T.TM_BF16, ptr(ws), st) == T.TM_ERR_STATE
    assert L.tm_forward_ex(g.ctx, ptr(g.state), *args, 1, 2, 32, T.TM_BF16, T.TM_READ_BEFORE_WRITE, ptr(ws),
                           st) == T.TM_ERR_STATE
    assert L.tm_store(g.ctx, ptr(g.state), *args[:2], *args[3:6], 2, 1, 32, T.TM_BF16, ptr(ws), st) == \
        T.TM_ERR_STATE
    assert L.tm_retrieve(g.ctx, ptr(g.state), args[2], ptr(y), 2, 1, 32, T.TM_BF16, ptr(ws), st) == T.TM_ERR_STATE
    other = T.tm_create(64, 2, 2, 32)        # same widths, another chunk: another configuration
    assert L.tm_retrieve(other, ptr(g.state), args[2], ptr(y), 1, 1, 32, T.TM_BF16, ptr(ws), st) == \
        T.TM_ERR_STATE
    torch.cuda.synchronize()
    assert torch.equal(g.state, before)
    assert bool((y == 7.0).all())
    # the binding refuses a short workspace or state before calling the library
    d1 = dev_inputs(I.make_call(wl, p), "bf16")
    y1 = torch.empty((1, 32, 1, 64), device="cuda")
    short = torch.empty(T.tm_workspace_bytes(g.ctx, 1, 1, 32) - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="workspace"):
        T.tm_forward(g.ctx, g.state, d1["k"], d1["v"], d1["q"], d1["theta"], d1["eta"], d1["alpha"], y1, short)
    with pytest.raises(ValueError, match="state"):
        T.tm_forward(g.ctx, g.state[:-256], d1["k"], d1["v"], d1["q"], d1["theta"], d1["eta"], d1["alpha"], y1,
                     ws)
    with pytest.raises(ValueError, match="dim"):
        T.tm_retrieve(g.ctx, g.state, d1["q"][..., :32].contiguous(), y1[..., :32].contiguous(), ws)
    torch.cuda.synchronize()
    assert torch.equal(g.state, before)
    # a state set up again for batch 2 is taken with batch 2 (its record replaced)
    big = torch.empty(T.tm_state_bytes(g.ctx, 2, 1), dtype=torch.uint8, device="cuda")
    T.tm_state_init(g.ctx, big, 2, 1, g.init)
    T.tm_forward(g.ctx, big, d["k"], d["v"], d["q"], d["theta"], d["eta"], d["alpha"], y, ws)
    assert T.tm_state_check(g.ctx, big, 2, 1) == (False, 32)
    T.tm_destroy(other)
    g.close()


def test_tm_log_prints_the_call_shape_and_plan():
    # TM_LOG=1: a new call shape and its launch plan are printed (stderr);
    # TM_LOG=2 also prints the capture and the replays
    import os
    import subprocess
    import sys
    code = ("import sys, os\n"
            "sys.path.insert(0, %r)\n"
            "from test_trained_neural_amd import inputs as I\n"
            "from tests.harness import GpuMemory, dev_inputs\n"
            "wl = I.Workload('log', batch=1, seq=32, heads=1, dim=32, depth=2, expansion=2, chunk=16, dtype='bf16',"
            " offsets=(-4.0, 1.0, -4.0))\n"
            "p = I.make_params(wl); g = GpuMemory(wl, p); d = dev_inputs(I.make_call(wl, p), 'bf16')\n"
            "for _ in range(3): g.forward(d)\n"
            "import torch; torch.cuda.synchronize()\n") % os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for lvl, want in (("1", ["[tm] new call shape: tm_forward", "[tm] plan: 2 chunks of 16"]),
                      ("2", ["[tm] capture call tm_forward", "[tm] replay call tm_forward"])):
        r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                           env=dict(os.environ, TM_LOG=lvl))
        assert r.returncode == 0, r.stderr[-2000:]
        for w in want:
            assert w in r.stderr, (lvl, w, r.stderr[-2000:])
