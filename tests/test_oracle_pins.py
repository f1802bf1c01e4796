"""Pins for the fp64 oracle: each test checks it against something other than
itself -- a closed form the pages state, a special case that reduces to a
textbook rule, finite differences, torch.autograd as an independent library
backprop, brute force on tiny inputs, or invariants of the definition.

Sources: "Titans, explained" (vibeengines.com) method steps 1-6 and its
paragraph on the extremes; "Attack of the Titans" (synthesis.ai), section
Technical Details / Parallel training.
"""
import numpy as np
import pytest
import torch

from oracle import tmref
from test_trained_neural_amd import inputs as I



@pytest.fixture(autouse=True)
def _float64_default():
    """torch's default dtype is float64 inside these pins, and restored
    after each (other modules build float32 tensors by default)."""
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(old)


# --------------------------------------------------------------------------
# independent helpers (torch autograd; nothing shared with the oracle)

def dims_of(dim, depth, expansion):
    h = dim * expansion if depth > 1 else dim
    if depth == 1:
        return [(dim, dim)]
    return [(dim, h)] + [(h, h)] * (depth - 2) + [(h, dim)]


def unflatten(W, dims):
    out, off = [], 0
    for a, b in dims:
        out.append(torch.tensor(W[off:off + a * b].reshape(a, b)))
        off += a * b
    return out


def torch_grad(W, k, v, dims):
    """Gradient of ||M(k) - v||^2 by torch.autograd (row-vector MLP, SiLU
    between layers, no bias)."""
    Ws = [w.clone().requires_grad_(True) for w in unflatten(W, dims)]
    h = torch.tensor(k)[None, :]
    for i, w in enumerate(Ws):
        h = h @ w
        if i < len(Ws) - 1:
            h = torch.nn.functional.silu(h)
    loss = ((h[0] - torch.tensor(v)) ** 2).sum()
    gs = torch.autograd.grad(loss, Ws)
    return np.concatenate([g.numpy().ravel() for g in gs])


def torch_fwd(W, x, dims):
    h = torch.tensor(x)[None, :]
    Ws = unflatten(W, dims)
    for i, w in enumerate(Ws):
        h = h @ w
        if i < len(Ws) - 1:
            h = torch.nn.functional.silu(h)
    return h[0].numpy()


def rand_inputs(rng, B, T, H, d, gate_lo=0.05, gate_hi=0.95):
    k = rng.standard_normal((B, T, H, d)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, d)).astype(np.float32)
    q = rng.standard_normal((B, T, H, d)).astype(np.float32)
    g = [rng.uniform(gate_lo, gate_hi, (B, T, H)).astype(np.float32) for _ in range(3)]
    return k, v, q, g


def rand_state(rng, ns, P, scale=0.5, s_scale=0.0):
    st = np.zeros((ns, 2 * P))
    st[:, :P] = rng.standard_normal((ns, P)) * scale
    st[:, P:] = rng.standard_normal((ns, P)) * s_scale
    return st


def rel(a, b):
    return np.linalg.norm(np.ravel(a - b)) / max(np.linalg.norm(np.ravel(b)), 1e-300)


# --------------------------------------------------------------------------
# the gradient (the momentary surprise, step 2)

def test_linear_gradient_closed_form():
    # The extremes paragraph of "Titans, explained": a linear memory has
    # gradient 2 (M k - v) k^T.  With row vectors y = k W that is the
    # transpose: dl/dW = k^T 2 (k W - v), an outer product.
    rng = np.random.default_rng(1)
    d = 7
    W = rng.standard_normal(d * d)
    k, v = rng.standard_normal(d), rng.standard_normal(d)
    G, loss = tmref.mlp_grad(d, 1, 1, W, k, v)
    e = k @ W.reshape(d, d) - v
    np.testing.assert_allclose(G.reshape(d, d), 2.0 * np.outer(k, e), rtol=1e-13, atol=1e-13)
    assert loss == pytest.approx(float(e @ e), rel=1e-13)


@pytest.mark.parametrize("depth,expansion", [(2, 2), (3, 2), (4, 3)])
def test_mlp_gradient_finite_differences(depth, expansion):
    # central differences of the loss itself, evaluated through the oracle's
    # forward pass only
    rng = np.random.default_rng(depth)
    d = 4
    P = tmref.param_count(d, depth, expansion)
    W = rng.standard_normal(P) * 0.7
    k, v = rng.standard_normal(d), rng.standard_normal(d)
    G, _ = tmref.mlp_grad(d, depth, expansion, W, k, v)

    def loss(Wx):
        y = tmref.mlp_forward(d, depth, expansion, Wx, k)
        return float(np.sum((y - v) ** 2))

    h = 1e-6
    fd = np.zeros(P)
    for p in range(P):
        Wp, Wm = W.copy(), W.copy()
        Wp[p] += h
        Wm[p] -= h
        fd[p] = (loss(Wp) - loss(Wm)) / (2 * h)
    assert rel(G, fd) < 1e-6


@pytest.mark.parametrize("depth,expansion,d", [(1, 1, 5), (2, 4, 6), (3, 2, 5), (4, 2, 8)])
def test_mlp_gradient_autograd(depth, expansion, d):
    rng = np.random.default_rng(10 + depth)
    dims = dims_of(d, depth, expansion)
    P = sum(a * b for a, b in dims)
    assert tmref.param_count(d, depth, expansion) == P
    W = rng.standard_normal(P) * 0.6
    k, v = rng.standard_normal(d), rng.standard_normal(d)
    G, _ = tmref.mlp_grad(d, depth, expansion, W, k, v)
    np.testing.assert_allclose(G, torch_grad(W, k, v, dims), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(tmref.mlp_forward(d, depth, expansion, W, k),
                               torch_fwd(W, k, dims), rtol=1e-12, atol=1e-12)


def test_zero_init_mlp_is_a_fixed_point():
    # SiLU(0) = 0 and there are no biases: an all-zero MLP memory outputs 0 and
    # every weight gradient is 0, so it never leaves zero.  (A bias anywhere
    # would break this.)
    rng = np.random.default_rng(3)
    d, depth, ex = 8, 3, 2
    P = tmref.param_count(d, depth, ex)
    k, v, q, (th, et, al) = rand_inputs(rng, 1, 32, 1, d)
    st = np.zeros((1, 2 * P))
    y = tmref.forward(d, depth, ex, 8, st, k, v, th, et, al, q=q)
    assert np.all(st == 0.0) and np.all(y == 0.0)


# --------------------------------------------------------------------------
# special cases of the update (extremes paragraph of "Titans, explained")

def test_delta_rule():
    # linear memory, eta = alpha = 0, chunk 1: DeltaNet's delta rule
    # W <- W - theta * 2 k^T (k W - v)
    rng = np.random.default_rng(4)
    d, T = 6, 40
    k, v, q, (th, _, _) = rand_inputs(rng, 1, T, 1, d)
    zero = np.zeros_like(th)
    W0 = rng.standard_normal((d, d)) * 0.3
    st = np.zeros((1, 2 * d * d))
    st[0, :d * d] = W0.ravel()
    tmref.forward(d, 1, 1, 1, st, k, v, th, zero, zero)
    W = W0.copy()
    for t in range(T):
        kt, vt = k[0, t, 0].astype(np.float64), v[0, t, 0].astype(np.float64)
        W = W - float(th[0, t, 0]) * 2.0 * np.outer(kt, kt @ W - vt)
    np.testing.assert_allclose(st[0, :d * d].reshape(d, d), W, rtol=1e-12, atol=1e-13)


def _token_sequential(W0, S0, k, v, th, et, al, dims):
    """The per-token definition (steps 2-4), gradients by autograd at the
    current weights."""
    M, S = W0.copy(), S0.copy()
    for t in range(k.shape[0]):
        G = torch_grad(M, k[t].astype(np.float64), v[t].astype(np.float64), dims)
        S = float(et[t]) * S - float(th[t]) * G
        M = (1.0 - float(al[t])) * M + S
    return M, S


@pytest.mark.parametrize("depth", [1, 2, 3])
def test_chunk_one_is_token_sequential(depth):
    rng = np.random.default_rng(20 + depth)
    d, ex, T = 5, 2, 24
    dims = dims_of(d, depth, ex)
    P = sum(a * b for a, b in dims)
    k, v, q, (th, et, al) = rand_inputs(rng, 1, T, 1, d, 0.05, 0.6)
    st = rand_state(rng, 1, P, 0.6, 0.1)
    M, S = _token_sequential(st[0, :P], st[0, P:], k[0, :, 0], v[0, :, 0],
                             th[0, :, 0], et[0, :, 0], al[0, :, 0], dims)
    tmref.forward(d, depth, ex, 1, st, k, v, th, et, al)
    np.testing.assert_allclose(st[0, :P], M, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(st[0, P:], S, rtol=1e-11, atol=1e-12)


def test_eta_zero_is_plain_gradient_step():
    # eta = 0: M_t = (1 - alpha_t) M_{t-1} - theta_t grad (the TTT form)
    rng = np.random.default_rng(5)
    d, ex, T, depth = 4, 3, 20, 2
    dims = dims_of(d, depth, ex)
    P = sum(a * b for a, b in dims)
    k, v, q, (th, _, al) = rand_inputs(rng, 1, T, 1, d)
    st = rand_state(rng, 1, P, 0.5, 0.3)   # S_0 is wiped by eta_1 = 0
    M = st[0, :P].copy()
    tmref.forward(d, depth, ex, 1, st, k, v, th, np.zeros_like(th), al)
    for t in range(T):
        G = torch_grad(M, k[0, t, 0].astype(np.float64), v[0, t, 0].astype(np.float64), dims)
        M = (1.0 - float(al[0, t, 0])) * M - float(th[0, t, 0]) * G
    np.testing.assert_allclose(st[0, :P], M, rtol=1e-11, atol=1e-12)


def test_alpha_one_wipes_memory():
    # alpha = 1: M_t = 0 * M_{t-1} + S_t, i.e. the memory is exactly the
    # momentum after every token
    rng = np.random.default_rng(6)
    d, ex, depth = 4, 2, 2
    P = tmref.param_count(d, depth, ex)
    k, v, q, (th, et, _) = rand_inputs(rng, 2, 16, 1, d)
    st = rand_state(rng, 2, P, 0.5, 0.2)
    tmref.forward(d, depth, ex, 4, st, k, v, th, et, np.ones_like(th))
    assert np.array_equal(st[:, :P], st[:, P:])


def test_theta_zero_turns_writing_off():
    rng = np.random.default_rng(7)
    d, ex, depth, T = 4, 2, 3, 32
    P = tmref.param_count(d, depth, ex)
    k, v, q, (_, et, al) = rand_inputs(rng, 1, T, 1, d)
    zero = np.zeros_like(et)
    st0 = rand_state(rng, 1, P, 0.5, 0.0)
    # alpha = 0 as well: the memory is bitwise unchanged
    st = st0.copy()
    tmref.forward(d, depth, ex, 8, st, k, v, zero, et, zero)
    assert np.array_equal(st, st0)
    # alpha > 0: M_T = prod(1 - alpha_t) M_0, S stays 0
    st = st0.copy()
    tmref.forward(d, depth, ex, 8, st, k, v, zero, et, al)
    decay = np.prod(1.0 - al[0, :, 0].astype(np.float64))
    np.testing.assert_allclose(st[0, :P], decay * st0[0, :P], rtol=1e-13)
    assert np.all(st[0, P:] == 0.0)


def test_write_hard_then_fade_under_silence():
    # One strong write (token 1), then theta = 0 with constant eta, alpha.
    # S_t = eta^(t-1) S_1 and M_n = (1-a)^(n-1) M_1 + S_1 sum_{j=1}^{n-1} (1-a)^(n-1-j) eta^j.
    rng = np.random.default_rng(8)
    d, n = 6, 30
    k, v, q, _ = rand_inputs(rng, 1, n, 1, d)
    th = np.zeros((1, n, 1), np.float32)
    th[0, 0, 0] = 0.9
    eta = np.float32(0.8)
    a = np.float32(0.1)
    et = np.full_like(th, eta)
    al = np.full_like(th, a)
    W0 = rng.standard_normal(d * d) * 0.2
    st = np.zeros((1, 2 * d * d))
    st[0, :d * d] = W0
    tmref.forward(d, 1, 1, 1, st, k, v, th, et, al)
    k0, v0 = k[0, 0, 0].astype(np.float64), v[0, 0, 0].astype(np.float64)
    G1 = 2.0 * np.outer(k0, k0 @ W0.reshape(d, d) - v0).ravel()
    e, oa = float(eta), 1.0 - float(a)
    S1 = -float(np.float32(0.9)) * G1
    M1 = oa * W0 + S1
    Mn = oa ** (n - 1) * M1 + S1 * sum(oa ** (n - 1 - j) * e ** j for j in range(1, n))
    np.testing.assert_allclose(st[0, :d * d], Mn, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(st[0, d * d:], e ** (n - 1) * S1, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# the chunked (mini-batch) form, step 6 and "Parallel training"

def _closed_form_chunks(W0, S0, k, v, th, et, al, b, dims):
    """Independent derivation of a whole chunk in one go.  With every
    gradient G_i taken at the chunk-start weights and the per-token
    recurrences unrolled:
        S_end = (prod eta) S_0 - sum_i theta_i (prod_{j>i} eta_j) G_i
        M_end = (prod (1-alpha)) M_0 + s0 S_0 - sum_i theta_i r_i G_i
    with A_i = prod_{j>i}(1-alpha_j), r_i = sum_{m>=i} A_m prod_{i<j<=m} eta_j,
    s0 = sum_m A_m prod_{j<=m} eta_j, all coefficient sums done by brute force."""
    M, S = W0.copy(), S0.copy()
    T = k.shape[0]
    for c0 in range(0, T, b):
        idx = range(c0, c0 + b)
        e = np.array([float(et[t]) for t in idx])
        oa = np.array([1.0 - float(al[t]) for t in idx])
        thc = np.array([float(th[t]) for t in idx])
        Gs = [torch_grad(M, k[t].astype(np.float64), v[t].astype(np.float64), dims) for t in idx]
        A = [np.prod(oa[i + 1:]) for i in range(b)]
        r = [sum(A[m] * np.prod(e[i + 1:m + 1]) for m in range(i, b)) for i in range(b)]
        s0 = sum(A[m] * np.prod(e[:m + 1]) for m in range(b))
        Mn = np.prod(oa) * M + s0 * S - sum(thc[i] * r[i] * Gs[i] for i in range(b))
        Sn = np.prod(e) * S - sum(thc[i] * np.prod(e[i + 1:]) * Gs[i] for i in range(b))
        M, S = Mn, Sn
    return M, S


@pytest.mark.parametrize("depth,b", [(1, 4), (2, 4), (2, 8), (3, 6)])
def test_chunked_form_matches_closed_form(depth, b):
    rng = np.random.default_rng(30 + depth * 10 + b)
    d, ex = 5, 2
    T = 4 * b
    dims = dims_of(d, depth, ex)
    P = sum(a * b_ for a, b_ in dims)
    k, v, q, (th, et, al) = rand_inputs(rng, 1, T, 1, d, 0.05, 0.7)
    st = rand_state(rng, 1, P, 0.5, 0.2)
    M, S = _closed_form_chunks(st[0, :P], st[0, P:], k[0, :, 0], v[0, :, 0],
                               th[0, :, 0], et[0, :, 0], al[0, :, 0], b, dims)
    tmref.forward(d, depth, ex, b, st, k, v, th, et, al)
    np.testing.assert_allclose(st[0, :P], M, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(st[0, P:], S, rtol=1e-10, atol=1e-12)


def test_page3_minibatch_form_linear_no_momentum():
    # "Attack of the Titans", Parallel training: without momentum the chunk
    # result is M_t = beta_t M_{t'} - sum_i theta_i (beta_t / beta_i) grad(M_{t'}; x_i)
    # with beta the running product of (1 - alpha) from the chunk start.
    rng = np.random.default_rng(9)
    d, b, T = 6, 8, 32
    k, v, q, (th, _, al) = rand_inputs(rng, 1, T, 1, d, 0.05, 0.3)
    zero = np.zeros_like(th)
    W = rng.standard_normal((d, d)) * 0.3
    st = np.zeros((1, 2 * d * d))
    st[0, :d * d] = W.ravel()
    tmref.forward(d, 1, 1, b, st, k, v, th, zero, al)
    for c0 in range(0, T, b):
        beta = np.cumprod([1.0 - float(al[0, t, 0]) for t in range(c0, c0 + b)])
        acc = beta[-1] * W
        for i, t in enumerate(range(c0, c0 + b)):
            kt, vt = k[0, t, 0].astype(np.float64), v[0, t, 0].astype(np.float64)
            G = 2.0 * np.outer(kt, kt @ W - vt)
            acc = acc - float(th[0, t, 0]) * (beta[-1] / beta[i]) * G
        W = acc
    np.testing.assert_allclose(st[0, :d * d].reshape(d, d), W, rtol=1e-11, atol=1e-13)


def test_retrieval_reads_the_freshly_written_memory():
    # in a store+retrieve call the queries of chunk c see the weights after
    # chunk c's write: identical to storing chunk c, then a read-only retrieve
    rng = np.random.default_rng(11)
    d, ex, depth, b, T = 4, 2, 2, 4, 16
    P = tmref.param_count(d, depth, ex)
    k, v, q, (th, et, al) = rand_inputs(rng, 2, T, 1, d)
    st0 = rand_state(rng, 2, P, 0.5, 0.1)
    st = st0.copy()
    y = tmref.forward(d, depth, ex, b, st, k, v, th, et, al, q=q)
    st2 = st0.copy()
    for c0 in range(0, T, b):
        s = slice(c0, c0 + b)
        tmref.forward(d, depth, ex, b, st2, k[:, s], v[:, s], th[:, s], et[:, s], al[:, s])
        y2 = tmref.retrieve(d, depth, ex, st2, q[:, s])
        assert np.array_equal(y[:, s], y2)
    assert np.array_equal(st, st2)


def test_read_before_write_linear_closed_form():
    # the queries read the memory before their chunk writes (the
    # memory-as-context order).  Linear memory from W_0 = 0 with eta = alpha =
    # 0: every gradient of chunk 1 is taken at W = 0, -2 k^T v, so after it
    # W_1 = sum_t theta_t 2 k_t^T v_t; chunk 1's queries read W_0 (zeros),
    # chunk 2's read W_1: y = q W_1 = sum_t 2 theta_t (q . k_t) v_t.  Read
    # after the write, chunk 1's queries would see W_1 instead.
    rng = np.random.default_rng(21)
    d, b = 4, 3
    k, v, q, (th, _, _) = rand_inputs(rng, 1, 2 * b, 1, d)
    zeros = np.zeros_like(th)
    st = np.zeros((1, 2 * d * d))
    y = tmref.forward(d, 1, 1, b, st, k, v, th, zeros, zeros, q=q, read="before")
    assert np.array_equal(y[0, :b], np.zeros((b, 1, d)))
    K = k[0, :b, 0].astype(np.float64)
    V = v[0, :b, 0].astype(np.float64)
    t1 = th[0, :b, 0].astype(np.float64)
    W1 = (2.0 * t1[:, None] * K).T @ V
    for t in range(b, 2 * b):
        np.testing.assert_allclose(y[0, t, 0], q[0, t, 0].astype(np.float64) @ W1, rtol=1e-12, atol=1e-14)
    st_a = np.zeros((1, 2 * d * d))
    y_a = tmref.forward(d, 1, 1, b, st_a, k, v, th, zeros, zeros, q=q, read="after")
    np.testing.assert_allclose(y_a[0, :b, 0], q[0, :b, 0].astype(np.float64) @ W1, rtol=1e-12, atol=1e-14)
    assert np.array_equal(st, st_a)   # the read order changes no write


def test_read_before_write_sees_the_chunk_start_weights():
    # read before the write: chunk c's queries equal a read-only retrieve
    # on the memory after chunks 1..c-1 (the first chunk's on the initial
    # memory, checked against torch), and without writes (theta = alpha = 0,
    # S_0 = 0) both read orders agree exactly
    rng = np.random.default_rng(22)
    d, ex, depth, b, T = 4, 2, 2, 4, 16
    dims = dims_of(d, depth, ex)
    P = tmref.param_count(d, depth, ex)
    k, v, q, (th, et, al) = rand_inputs(rng, 2, T, 1, d)
    st0 = rand_state(rng, 2, P, 0.5, 0.1)
    st = st0.copy()
    y = tmref.forward(d, depth, ex, b, st, k, v, th, et, al, q=q, read="before")
    for bi in range(2):
        for t in range(b):
            np.testing.assert_allclose(y[bi, t, 0], torch_fwd(st0[bi, :P], q[bi, t, 0].astype(np.float64), dims),
                                       rtol=1e-12, atol=1e-13)
    st2 = st0.copy()
    for c0 in range(0, T, b):
        s = slice(c0, c0 + b)
        y2 = tmref.retrieve(d, depth, ex, st2, q[:, s])
        assert np.array_equal(y[:, s], y2)
        tmref.forward(d, depth, ex, b, st2, k[:, s], v[:, s], th[:, s], et[:, s], al[:, s])
    assert np.array_equal(st, st2)
    z = np.zeros_like(th)
    sa = rand_state(rng, 2, P, 0.5, 0.0)
    sb = sa.copy()
    ya = tmref.forward(d, depth, ex, b, sa, k, v, z, et, z, q=q, read="after")
    yb = tmref.forward(d, depth, ex, b, sb, k, v, z, et, z, q=q, read="before")
    assert np.array_equal(ya, yb)


def chunk_coefficients(th, et, al):
    """Brute-force coefficients of the memory after token t of a chunk whose
    gradients all sit at the chunk-start weights (M_0, S_0), from unrolling
    S_u = eta_u S_{u-1} - theta_u G_u and M_u = (1 - alpha_u) M_{u-1} + S_u:
    M_t = pm[t] M_0 + ps[t] S_0 - sum_{i <= t} c[t, i] G_i, every product
    written out (no recurrence)."""
    b = len(th)
    prod = lambda xs: float(np.prod(xs)) if len(xs) else 1.0
    pm = np.array([prod(1.0 - al[:t + 1]) for t in range(b)])
    ps = np.array([sum(prod(1.0 - al[u + 1:t + 1]) * prod(et[:u + 1]) for u in range(t + 1)) for t in range(b)])
    c = np.zeros((b, b))
    for t in range(b):
        for i in range(t + 1):
            c[t, i] = th[i] * sum(prod(1.0 - al[u + 1:t + 1]) * prod(et[i + 1:u + 1]) for u in range(i, t + 1))
    return pm, ps, c


def test_per_token_read_linear_dual_form():
    # every query read right after its own token's write.  For the linear
    # memory this is a causal, linear-attention-like sum over the chunk's
    # earlier tokens and the token itself (the dual form): with
    # G_i = 2 k_i^T (k_i M_0 - v_i) at the chunk-start weights,
    #   y_t = pm_t q_t M_0 + ps_t q_t S_0 - sum_{i <= t} c_ti 2 (q_t . k_i)(k_i M_0 - v_i),
    # coefficients from the brute-force products above.  Checked over three
    # chunks with nonzero momentum, forgetting and S_0.
    rng = np.random.default_rng(23)
    d, b, C = 5, 4, 3
    k, v, q, (th, et, al) = rand_inputs(rng, 1, b * C, 1, d)
    st = rand_state(rng, 1, d * d, 0.5, 0.2)
    M = st[0, :d * d].reshape(d, d).copy()
    S = st[0, d * d:].reshape(d, d).copy()
    y = tmref.forward(d, 1, 1, b, st, k, v, th, et, al, q=q, read="token")
    for c0 in range(0, b * C, b):
        K = k[0, c0:c0 + b, 0].astype(np.float64)
        V = v[0, c0:c0 + b, 0].astype(np.float64)
        Q = q[0, c0:c0 + b, 0].astype(np.float64)
        pm, ps, cf = chunk_coefficients(*(g[0, c0:c0 + b, 0].astype(np.float64) for g in (th, et, al)))
        E = K @ M - V
        for t in range(b):
            want = pm[t] * Q[t] @ M + ps[t] * Q[t] @ S
            for i in range(t + 1):
                want = want - cf[t, i] * 2.0 * float(Q[t] @ K[i]) * E[i]
            np.testing.assert_allclose(y[0, c0 + t, 0], want, rtol=1e-11, atol=1e-13)
        # the chunk's end state from the same coefficients (c at t = b-1 and
        # the momentum's own products)
        G = [2.0 * np.outer(K[i], E[i]) for i in range(b)]
        pe = float(np.prod(et[0, c0:c0 + b, 0].astype(np.float64)))
        dS = [float(th[0, c0 + i, 0]) * float(np.prod(et[0, c0 + i + 1:c0 + b, 0].astype(np.float64)))
              for i in range(b)]
        M, S = (pm[-1] * M + ps[-1] * S - sum(cf[-1, i] * G[i] for i in range(b)),
                pe * S - sum(dS[i] * G[i] for i in range(b)))
    np.testing.assert_allclose(st[0, :d * d].reshape(d, d), M, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(st[0, d * d:].reshape(d, d), S, rtol=1e-11, atol=1e-13)


def test_per_token_read_delta_rule_special_case():
    # eta = alpha = 0, S_0 = 0: the memory after token t of the chunk is
    # M_0 - sum_{i <= t} theta_i G_i (the chunked delta rule), so
    # y_t = q_t M_0 - sum_{i <= t} 2 theta_i (q_t . k_i)(k_i M_0 - v_i);
    # token t's own write is included (i = t), later ones are not
    rng = np.random.default_rng(24)
    d, b = 4, 6
    k, v, q, (th, _, _) = rand_inputs(rng, 1, b, 1, d)
    z = np.zeros_like(th)
    st = rand_state(rng, 1, d * d, 0.5, 0.0)
    M0 = st[0, :d * d].reshape(d, d).copy()
    y = tmref.forward(d, 1, 1, b, st, k, v, th, z, z, q=q, read="token")
    K, V, Q = (a[0, :, 0].astype(np.float64) for a in (k, v, q))
    for t in range(b):
        want = Q[t] @ M0 - sum(2.0 * float(th[0, i, 0]) * float(Q[t] @ K[i]) * (K[i] @ M0 - V[i])
                               for i in range(t + 1))
        np.testing.assert_allclose(y[0, t, 0], want, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("depth", [2, 3])
def test_per_token_read_mlp_against_autograd(depth):
    # an MLP memory stepped token by token with torch.autograd gradients at
    # each chunk's start weights, every query read through the weights right
    # after its token; also: the read order changes no write, the last query
    # of each chunk reads what the after-the-write order reads, and a chunk
    # of one token makes the two orders the same
    rng = np.random.default_rng(25 + depth)
    d, ex, b, T = 4, 2, 4, 12
    dims = dims_of(d, depth, ex)
    P = tmref.param_count(d, depth, ex)
    k, v, q, (th, et, al) = rand_inputs(rng, 1, T, 1, d)
    st0 = rand_state(rng, 1, P, 0.5, 0.1)
    st = st0.copy()
    y = tmref.forward(d, depth, ex, b, st, k, v, th, et, al, q=q, read="token")
    M, S = st0[0, :P].copy(), st0[0, P:].copy()
    for c0 in range(0, T, b):
        M0 = M.copy()
        for t in range(c0, c0 + b):
            G = torch_grad(M0, k[0, t, 0].astype(np.float64), v[0, t, 0].astype(np.float64), dims)
            S = float(et[0, t, 0]) * S - float(th[0, t, 0]) * G
            M = (1.0 - float(al[0, t, 0])) * M + S
            np.testing.assert_allclose(y[0, t, 0], torch_fwd(M, q[0, t, 0].astype(np.float64), dims),
                                       rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(st[0], np.concatenate([M, S]), rtol=1e-11, atol=1e-13)
    sa = st0.copy()
    ya = tmref.forward(d, depth, ex, b, sa, k, v, th, et, al, q=q, read="after")
    assert np.array_equal(st, sa)
    for c0 in range(0, T, b):
        assert np.array_equal(y[:, c0 + b - 1], ya[:, c0 + b - 1])
    s1, s2 = st0.copy(), st0.copy()
    y1 = tmref.forward(d, depth, ex, 1, s1, k, v, th, et, al, q=q, read="token")
    y2 = tmref.forward(d, depth, ex, 1, s2, k, v, th, et, al, q=q, read="after")
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)


def test_retrieve_is_read_only_and_is_a_forward_pass():
    rng = np.random.default_rng(12)
    d, ex, depth = 5, 2, 3
    dims = dims_of(d, depth, ex)
    P = sum(a * b for a, b in dims)
    q = rng.standard_normal((1, 10, 2, d)).astype(np.float32)
    st = rand_state(rng, 2, P, 0.5, 0.3)
    st0 = st.copy()
    y = tmref.retrieve(d, depth, ex, st, q)
    assert np.array_equal(st, st0)
    for t in range(10):
        for h in range(2):
            np.testing.assert_allclose(y[0, t, h], torch_fwd(st[h, :P], q[0, t, h].astype(np.float64), dims),
                                       rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# invariants

def test_call_split_invariance():
    rng = np.random.default_rng(13)
    d, ex, depth, b, T = 4, 2, 2, 4, 32
    P = tmref.param_count(d, depth, ex)
    k, v, q, (th, et, al) = rand_inputs(rng, 2, T, 1, d)
    st = rand_state(rng, 2, P, 0.5)
    st2 = st.copy()
    y = tmref.forward(d, depth, ex, b, st, k, v, th, et, al, q=q)
    ys = []
    for s in (slice(0, 8), slice(8, 24), slice(24, 32)):
        ys.append(tmref.forward(d, depth, ex, b, st2, k[:, s], v[:, s], th[:, s], et[:, s], al[:, s], q=q[:, s]))
    assert np.array_equal(st, st2)
    assert np.array_equal(y, np.concatenate(ys, axis=1))


def test_streams_are_independent():
    # permuting the batch permutes the results; H heads equal H one-head
    # memories run on the head slices
    rng = np.random.default_rng(14)
    d, ex, depth, b, T, B, H = 4, 2, 2, 4, 16, 3, 2
    P = tmref.param_count(d, depth, ex)
    k, v, q, (th, et, al) = rand_inputs(rng, B, T, H, d)
    st = rand_state(rng, B * H, P, 0.5)
    st0 = st.copy()
    y = tmref.forward(d, depth, ex, b, st, k, v, th, et, al, q=q)
    perm = [2, 0, 1]
    sp = st0.reshape(B, H, -1)[perm].reshape(B * H, -1).copy()
    yp = tmref.forward(d, depth, ex, b, sp, k[perm], v[perm], th[perm], et[perm], al[perm], q=q[perm])
    assert np.array_equal(yp, y[perm])
    assert np.array_equal(sp, st.reshape(B, H, -1)[perm].reshape(B * H, -1))
    for h in range(H):
        sh = st0.reshape(B, H, -1)[:, h].copy()
        sl = (slice(None), slice(None), slice(h, h + 1))
        yh = tmref.forward(d, depth, ex, b, sh, k[sl], v[sl], th[:, :, h:h + 1], et[:, :, h:h + 1],
                           al[:, :, h:h + 1], q=q[sl])
        assert np.array_equal(yh[:, :, 0], y[:, :, h])


def test_rejects_ragged_token_count():
    st = np.zeros((1, 2 * 16))
    z = np.zeros((1, 6, 1, 4), np.float32)
    g = np.zeros((1, 6, 1), np.float32)
    with pytest.raises(ValueError):
        tmref.forward(4, 1, 1, 4, st, z, z, g, g, g)


@pytest.mark.slow
def test_literal_gates_diverge_on_mlp384():
    # The dim-384 MLP memory with gate offsets (0, 0, 0): median gates of 0.5
    # are a step size this memory cannot take.  Within the 1024-token call the
    # exact (fp64) state grows past the largest float32, so any fp32 state must
    # overflow (one stream is enough to show it).
    wl = I.WORKLOADS["mlp384"].replace(batch=1, offsets=(0.0, 0.0, 0.0))
    p = I.make_params(wl)
    ci = I.make_call(wl, p)
    st = I.initial_state(wl, p)
    tmref.forward(wl.dim, wl.depth, wl.expansion, wl.chunk, st, ci.k, ci.v, ci.theta, ci.eta, ci.alpha)
    assert tmref.nonfinite(st) or np.abs(st).max() > np.finfo(np.float32).max


def test_offset_gates_stay_finite_on_mlp384_prefix():
    wl = I.WORKLOADS["mlp384"].replace(batch=1)
    p = I.make_params(wl)
    ci = I.make_call(wl, p, tokens=256)
    st = I.initial_state(wl, p)
    y = tmref.forward(wl.dim, wl.depth, wl.expansion, wl.chunk, st, ci.k, ci.v, ci.theta, ci.eta, ci.alpha,
                      q=ci.q)
    assert not tmref.nonfinite(st) and np.all(np.isfinite(y))
    P = wl.params
    # the memory moved away from its init but is not exploding
    moved = np.linalg.norm(st[0, :P] - p.init_weights[0]) / np.linalg.norm(p.init_weights[0])
    assert 1e-4 < moved < 1.0


def _read_golden(name):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", name)
    out = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, vals = line.split(":", 1)
        out[key.strip()] = np.array([float(x) for x in vals.split()])
    return out


def test_hand_worked_linear_example():
    g = _read_golden("linear2_by_hand.txt")
    d, b = int(g["dim"][0]), int(g["chunk"][0])
    T = len(g["theta"])
    sh = (1, T, 1, d)
    st = np.zeros((1, 2 * d * d))
    st[0, :d * d] = g["M0"]
    y = tmref.forward(d, 1, 1, b, st, g["k"].reshape(sh), g["v"].reshape(sh),
                      g["theta"].reshape(1, T, 1), g["eta"].reshape(1, T, 1),
                      g["alpha"].reshape(1, T, 1), q=g["q"].reshape(sh))
    assert np.array_equal(y.ravel(), g["y"])
    assert np.array_equal(st[0, :d * d], g["M_final"])
    assert np.array_equal(st[0, d * d:], g["S_final"])
