"""Pins for the input-side oracle (oracle/prologue.py): brute force on tiny
inputs, the memory workloads' own input recipe as an independent
implementation, the convolution's impulse response, causality, the history
carried across calls, and the normalisation and gate invariants.

Source: "Titans, explained" (vibeengines.com) method steps 1 (projections,
short depthwise convolution, l2-normalised keys and queries), 4 (the gates
are computed from the input) and 5 (the query projection).
"""
import numpy as np

from oracle import prologue as PR
from test_trained_neural_amd import inputs as I


def rand_case(rng, B=2, T=7, D=6, H=2, d=3, K=3):
    x = rng.standard_normal((B, T, D))
    w = rng.standard_normal((3, D, H * d))
    conv = rng.standard_normal((3, H * d, K))
    wg = rng.standard_normal((3, D, H))
    gb = rng.standard_normal(3)
    return x, w, conv, wg, gb


def test_brute_force_tiny():
    # every output element from the definition, in plain loops
    rng = np.random.default_rng(1)
    B, T, D, H, d, K = 1, 5, 3, 2, 2, 3
    x, w, conv, wg, gb = rand_case(rng, B, T, D, H, d, K)
    hist = rng.standard_normal((B, K - 1, 3, H * d))
    k, v, q, th, et, al, nh = PR.project(x, w, conv, wg, gb, H, hist)
    outs = (k, v, q)
    for i in range(3):
        for t in range(T):
            rows = []
            for h in range(H):
                vals = []
                for e in range(d):
                    n = h * d + e
                    acc = 0.0
                    for j in range(K):
                        u = t - j
                        if u >= 0:
                            p = sum(x[0, u, a] * w[i, a, n] for a in range(D))
                        else:
                            p = hist[0, K - 1 + u, i, n]
                        acc += conv[i, n, j] * p
                    vals.append(acc)
                if i != 1:
                    nrm = max(sum(z * z for z in vals) ** 0.5, 1e-12)
                    vals = [z / nrm for z in vals]
                rows.append(vals)
            np.testing.assert_allclose(outs[i][0, t], np.array(rows), rtol=1e-12, atol=1e-13)
    for g, arr in enumerate((th, et, al)):
        for t in range(T):
            for h in range(H):
                z = sum(x[0, t, a] * wg[g, a, h] for a in range(D)) + gb[g]
                assert abs(arr[0, t, h] - 1.0 / (1.0 + np.exp(-z))) < 1e-14
    # the new history: the last K-1 projections of the call, oldest first
    for r in range(K - 1):
        for i in range(3):
            u = T - (K - 1) + r
            np.testing.assert_allclose(nh[0, r, i], x[0, u] @ w[i], rtol=1e-12, atol=1e-13)


def test_one_tap_identity_matches_the_memory_input_recipe():
    # with a single tap of 1 the input side is the memory workloads' recipe
    # (inputs.make_call, an independent float32 implementation)
    wl = I.Workload("p", batch=2, seq=16, heads=2, dim=8, depth=2, expansion=2, chunk=8, dtype="f32",
                    offsets=(-3.0, 1.0, -2.0))
    p = I.make_params(wl)
    pi = I.make_prologue(wl, p, conv_len=1)
    conv = np.ones((3, wl.model_dim, 1))
    k, v, q, th, et, al, _ = PR.project(pi.x, pi.w_kvq, conv, pi.w_gate, pi.gate_bias, wl.heads)
    ci = I.make_call(wl, p)
    for a, b in ((k, ci.k), (v, ci.v), (q, ci.q), (th, ci.theta), (et, ci.eta), (al, ci.alpha)):
        np.testing.assert_allclose(a, b, rtol=2e-5, atol=2e-6)


def test_impulse_response_is_the_taps():
    # one token with x = e_0 through identity projections and zero history:
    # the (unnormalised) values j tokens later are tap j of each channel
    D, H, K, T, t0 = 4, 1, 4, 9, 2
    x = np.zeros((1, T, D))
    x[0, t0, 0] = 1.0
    w = np.stack([np.eye(D)] * 3)
    rng = np.random.default_rng(2)
    conv = rng.standard_normal((3, D, K))
    _, v, _, _, _, _, _ = PR.project(x, w, conv, np.zeros((3, D, H)), np.zeros(3), H)
    for t in range(T):
        j = t - t0
        want = conv[1, 0, j] if 0 <= j < K else 0.0
        assert v[0, t, 0, 0] == want
        assert np.all(v[0, t, 0, 1:] == 0.0)


def test_causal():
    rng = np.random.default_rng(3)
    x, w, conv, wg, gb = rand_case(rng, T=9)
    a = PR.project(x, w, conv, wg, gb, 2)
    x2 = x.copy()
    x2[:, 5:] += rng.standard_normal(x2[:, 5:].shape)
    b = PR.project(x2, w, conv, wg, gb, 2)
    for u, v in zip(a[:6], b[:6]):
        assert np.array_equal(u[:, :5], v[:, :5])
        assert not np.allclose(u[:, 5:], v[:, 5:])


def test_history_carries_across_calls():
    # one call of T tokens equals calls of 3, 1 and T-4 tokens with the
    # history handed on (including a call shorter than the history)
    rng = np.random.default_rng(4)
    x, w, conv, wg, gb = rand_case(rng, T=11, K=4)
    whole = PR.project(x, w, conv, wg, gb, 2)
    h = None
    parts = []
    for sl in (slice(0, 3), slice(3, 4), slice(4, 11)):
        r = PR.project(x[:, sl], w, conv, wg, gb, 2, h)
        h = r[6]
        parts.append(r[:6])
    for i in range(6):
        np.testing.assert_allclose(whole[i], np.concatenate([p[i] for p in parts], axis=1), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(whole[6], h, rtol=1e-13, atol=1e-14)


def test_norms_and_gate_bias():
    rng = np.random.default_rng(5)
    x, w, conv, wg, gb = rand_case(rng)
    k, v, q, th, et, al, _ = PR.project(x, w, conv, np.zeros_like(wg), gb, 2)
    np.testing.assert_allclose(np.linalg.norm(k, axis=-1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(np.linalg.norm(q, axis=-1), 1.0, rtol=1e-13)
    assert not np.allclose(np.linalg.norm(v, axis=-1), 1.0)
    for g, arr in enumerate((th, et, al)):
        np.testing.assert_allclose(arr, 1.0 / (1.0 + np.exp(-gb[g])), rtol=1e-15)
    # a zero projection stays zero (the clamp, not a division by zero)
    k0, _, q0, _, _, _, _ = PR.project(np.zeros_like(x), w, conv, wg, gb, 2)
    assert np.all(k0 == 0.0) and np.all(q0 == 0.0)
