"""tm_forward_noalloc (the allocation-free forward) against tm_forward, the
entry point whose kernels it shares: bitwise equal outputs and states over
two calls in a row, the second with a smaller input, and a call too large for
the library's scratch array refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

from harness import GpuMemory, dev_inputs, say
from test_trained_neural_amd import inputs as I
import test_trained_neural_amd as T

pytestmark = pytest.mark.gpu


def noalloc(g, d):
    B, Tn, H, dim = d["k"].shape
    y = torch.empty((B, Tn, H, dim), dtype=torch.float32, device="cuda")
    T.tm_forward_noalloc(g.ctx, g.state, d["k"], d["v"], d["q"], d["theta"], d["eta"], d["alpha"], y)
    return y


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_noalloc_equals_forward(dtype):
    wl = I.WORKLOADS["mlp384"].replace(dtype=dtype)
    say("case", wl.name, dtype)
    p = I.make_params(wl)
    ref, na = GpuMemory(wl, p), GpuMemory(wl, p)
    # call 1: the whole 2 x 1024 call; call 2: 2 x 256 tokens more (smaller),
    # continuing from the state call 1 left
    for j, n in ((0, 1024), (1, 256)):
        d = dev_inputs(I.make_call(wl, p, j, tokens=n), dtype)
        y_ref = ref.forward(d)
        y_na = noalloc(na, d)
        torch.cuda.synchronize()
        say("  call %d (%d tokens): max |dy| %.3g" % (j + 1, n, float((y_na - y_ref).abs().max())))
        assert torch.equal(y_na, y_ref)
        assert np.array_equal(na.export(), ref.export())
    assert na.check() == ref.check() == (False, 1280)
    ref.close()
    na.close()


def test_forward_noalloc_refuses_a_call_beyond_its_scratch():
    # 4 streams of 1024 tokens at dim 384 need 48 MiB of workspace: more than
    # the 32 MiB scratch array, refused with TM_ERR_SCRATCH, nothing launched
    wl = I.WORKLOADS["mlp384"].replace(batch=4)
    p = I.make_params(wl)
    g = GpuMemory(wl, p)
    assert T.tm_workspace_bytes(g.ctx, 4, 1, 1024) > 32 << 20
    d = dev_inputs(I.make_call(wl, p), "bf16")
    before = g.state.clone()
    y = torch.full((4, 1024, 1, 384), 3.0, device="cuda")
    with pytest.raises(T.TMError) as e:
        T.tm_forward_noalloc(g.ctx, g.state, d["k"], d["v"], d["q"], d["theta"], d["eta"], d["alpha"], y)
    assert e.value.code == T.TM_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.equal(g.state, before) and bool((y == 3.0).all())
    g.close()
