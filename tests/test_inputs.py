"""The seeded workload generator: deterministic, right shapes and
distributions, bf16 rounding identical to torch's round-to-nearest-even."""
import numpy as np
import torch

from test_trained_neural_amd import inputs as I


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, 65504.0, 3.0e38, -3.0e38, 1e-40], np.float32)]).astype(np.float32)
    ours = I.round_bf16(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_workload_shapes_and_determinism():
    wl = I.WORKLOADS["multihead1024"].replace(batch=2, seq=256)
    p = I.make_params(wl)
    a = I.make_call(wl, p, j=3)
    b = I.make_call(wl, p, j=3)
    assert a.k.shape == (2, 256, 8, 128) and a.theta.shape == (2, 256, 8)
    for x, y in zip((a.k, a.v, a.q, a.theta, a.eta, a.alpha), (b.k, b.v, b.q, b.theta, b.eta, b.alpha)):
        assert np.array_equal(x, y)
    # a subset of the batch draws the same values as the full batch
    c = I.make_call(wl, p, j=3, batch_rows=[1])
    assert np.array_equal(c.k[0], a.k[1]) and np.array_equal(c.alpha[0], a.alpha[1])
    # keys and queries unit norm per head (up to bf16 rounding); all bf16-exact
    n = np.linalg.norm(a.k.astype(np.float64), axis=-1)
    assert np.all(np.abs(n - 1) < 1e-2)
    assert np.array_equal(I.round_bf16(a.v), a.v)
    # gate offsets (-7, +2, -7): theta, alpha small, eta large
    assert 0.0 < a.theta.mean() < 0.01 and 0.8 < a.eta.mean() < 0.9 and a.alpha.mean() < 0.01
    assert a.theta.min() > 0 and a.eta.max() < 1


def test_initial_weights():
    wl = I.WORKLOADS["mlp384"]
    p = I.make_params(wl)
    assert p.init_weights.shape == (1, wl.params) == (1, 2 * 384 * 1536)
    w1 = p.init_weights[0, :384 * 1536]
    w2 = p.init_weights[0, 384 * 1536:]
    assert abs(w1.var() * 384 - 1) < 0.02 and abs(w2.var() * 1536 - 1) < 0.02
    lin = I.WORKLOADS["linear64"]
    assert np.all(I.make_params(lin).init_weights == 0)
    st = I.initial_state(wl, p)
    assert st.shape == (2, 2 * wl.params) and np.all(st[:, wl.params:] == 0)


def test_workload_table():
    W = I.WORKLOADS
    assert [W[n].params for n in W] == [4096, 1179648, 1179648, 131072, 10485760]
    assert W["deep512"].tokens_per_call == 1024 and W["mlp384_stream"].tokens_per_call == 1024
    assert W["multihead1024"].streams == 64
