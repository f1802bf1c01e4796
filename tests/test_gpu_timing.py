"""Per-launch event timing (tm_timing_enable / tm_timing_read): every timed
launch records its pair with its own dispatch, launches are counted per
class, and results with timing on are bitwise those with timing off (the
timed path launches the same kernels directly instead of replaying a
graph)."""
import numpy as np
import pytest
import torch

from harness import GpuMemory, dev_inputs, say
from test_gpu_parity import small
from test_trained_neural_amd import inputs as I

pytestmark = pytest.mark.gpu

def read_all(T):
    return {c: T.tm_timing_read(c) for c in (T.K_SCAN, T.K_FWD, T.K_BWD, T.K_FIRST, T.K_TOKEN_READ)}


@pytest.mark.parametrize("depth,read", [(2, None), (3, None), (2, "token")])
def test_timed_launch_counts_and_results(depth, read):
    import test_trained_neural_amd as T
    wl = small("timing_d%d" % depth, 64, depth, 2, 16, 2, 1, 64, "bf16")
    say("case", wl, read)
    p = I.make_params(wl)
    d = dev_inputs(I.make_call(wl, p), "bf16")
    C = wl.seq // wl.chunk
    mode = None if read is None else T.TM_READ_PER_TOKEN
    g = GpuMemory(wl, p)
    y0 = g.forward(d, read=mode).cpu().numpy()
    s0 = g.export()
    g.close()
    g = GpuMemory(wl, p)
    try:
        T.tm_timing_enable(0x7F)
        read_all(T)
        y1 = g.forward(d, read=mode).cpu().numpy()
        torch.cuda.synchronize()
        got = read_all(T)
    finally:
        T.tm_timing_enable(0)
    assert np.array_equal(y0, y1) and np.array_equal(s0, g.export())
    g.close()
    ms = {c: v[0] for c, v in got.items()}
    n = {c: v[1] for c, v in got.items()}
    say("  launches", n, "ms", ms)
    assert n[T.K_SCAN] == 1
    assert n[T.K_FIRST] == C + 1                    # chunk steps 0 .. C
    # layers 1.. of each step with rows: every step for the read after the
    # write (its last step carries the last chunk's queries), all but the
    # last for the per-token read (its queries take their own launches)
    assert n[T.K_FWD] == (C + 1 if read is None else C) * (depth - 1)
    assert n[T.K_BWD] == C * max(depth - 2, 0)      # layers L-1 .. 2 of each chunk
    assert n[T.K_TOKEN_READ] == (C * depth + 1 if read == "token" else 0)
    for c in n:
        if n[c]:
            assert 0.0 < ms[c] < 1e3 * n[c]
