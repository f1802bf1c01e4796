"""The parity measures the GPU tests use (tests/harness.py), on the CPU:
an error confined to one token's output row, or to one 16 x 16 tile of a
weight matrix, slips under the whole-tensor Frobenius ratio at the bf16
tolerance but fails the row and element-wise measures; and the oracle's
threaded element loops give bitwise the results of one thread."""
import numpy as np
import pytest

from harness import TOL, compare_state, max_err, relerr, row_err, yerr
from oracle import tmref
from test_trained_neural_amd import inputs as I


def test_one_wrong_row_fails_the_row_measure():
    rng = np.random.default_rng(3)
    yr = rng.standard_normal((2, 1024, 1, 384))
    y = yr * (1 + 1e-3 * rng.standard_normal(yr.shape))     # bf16-like noise
    assert yerr(y, yr) < TOL["bf16"]
    bad = y.copy()
    bad[1, 517, 0] += 0.3 * yr[1, 517, 0]                   # one token's output off by 30%
    assert relerr(bad, yr) < TOL["bf16"]                     # the Frobenius ratio misses it
    assert row_err(bad, yr) > 0.25 and yerr(bad, yr) > TOL["bf16"]


def test_one_wrong_tile_fails_the_element_measure():
    wl = I.Workload("tile", batch=1, seq=64, heads=1, dim=384, depth=2, expansion=4, chunk=64, dtype="bf16",
                    offsets=(0, 0, 0))
    rng = np.random.default_rng(4)
    ref = rng.standard_normal((1, 2 * wl.params)) / 20
    gpu = ref * (1 + 1e-3 * rng.standard_normal(ref.shape))
    em, es = compare_state(wl, gpu, ref)
    assert em < TOL["bf16"] and es < TOL["bf16"]
    bad = gpu.copy()
    W0 = bad[0, :384 * 1536].reshape(384, 1536)
    W0[32:48, 160:176] *= 1.5                               # one 16 x 16 tile of W_0 off by 50%
    assert relerr(bad[0, :384 * 1536], ref[0, :384 * 1536]) < TOL["bf16"]   # missed by Frobenius
    assert max_err(bad[0, :384 * 1536], ref[0, :384 * 1536]) > TOL["bf16"]
    em, _ = compare_state(wl, bad, ref)
    assert em > TOL["bf16"]


@pytest.mark.parametrize("batch", [1, 3])
def test_oracle_threads_are_bitwise_one_thread(batch):
    # one stream split over 3 and 8 threads (its element loops), and 3
    # streams over 8 threads (a worker per stream, 2 threads splitting each
    # stream's loops), against one thread
    wl = I.Workload("thr", batch=batch, seq=64, heads=1, dim=96, depth=3, expansion=3, chunk=16, dtype="f32",
                    offsets=(-3.0, 1.0, -3.0))
    p = I.make_params(wl)
    ci = I.make_call(wl, p)
    outs = []
    for nt in (1, 3, 8):
        st = I.initial_state(wl, p)
        y = tmref.forward(wl.dim, wl.depth, wl.expansion, wl.chunk, st, ci.k, ci.v, ci.theta, ci.eta, ci.alpha,
                          q=ci.q, n_threads=nt)
        r = tmref.retrieve(wl.dim, wl.depth, wl.expansion, st, ci.q, n_threads=nt)
        outs.append((y, st, r))
    for y, st, r in outs[1:]:
        assert np.array_equal(y, outs[0][0]) and np.array_equal(st, outs[0][1]) and np.array_equal(r, outs[0][2])
