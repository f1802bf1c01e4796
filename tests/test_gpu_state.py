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
