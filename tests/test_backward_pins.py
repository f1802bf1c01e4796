"""Pins for the backward oracle (oracle/backward.py), on the CPU.  Each test
checks it against something other than itself:

  * its forward recurrence against the C oracle (oracle/tmref.c, an
    independent implementation of the same pages): y and the state after
    the call, both read orders;
  * its gradients against central finite differences, in random directions,
    of the loss through its own (pinned) forward, and of the gradient with
    respect to the starting state through the C oracle's forward;
  * closed forms for a linear memory and one token, worked out by hand from
    y = q M_1, M_1 = (1 - alpha) M_0 + eta S_0 - theta 2 k^T (k M_0 - v)
    ("Titans, explained", steps 2-5, and its closing remark on the linear
    memory's gradient);
  * writing switched off (theta = 0): no gradient reaches the keys and
    values, and the forgetting's gradient is that of a plain decay;
  * splitting a call in two and chaining the backward through the state
    changes nothing.
"""
import numpy as np
import pytest
import torch

from oracle import backward as BW
from oracle import tmref


@pytest.fixture(autouse=True)
def _float64_default():
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(old)


def rand_case(seed, B, T, H, d, depth, expansion, s_scale=0.1, gate=(0.1, 0.9)):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, T, H, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, d))
    q = rng.standard_normal((B, T, H, d))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    g = [rng.uniform(*gate, (B, T, H)) for _ in range(3)]
    P = sum(a * b for a, b in BW.layer_dims(d, depth, expansion))
    st = np.concatenate([rng.standard_normal((B * H, P)) * 0.4, rng.standard_normal((B * H, P)) * s_scale], 1)
    dy = rng.standard_normal((B, T, H, d))
    dst = rng.standard_normal((B * H, 2 * P)) * 0.3
    # the C oracle reads float32 token arrays: use float32-exact values
    f = lambda a: a.astype(np.float32).astype(np.float64)
    return f(k), f(v), f(q), [f(x) for x in g], st, dy, dst


@pytest.mark.parametrize("depth,chunk,read", [(1, 2, "after"), (2, 3, "after"), (3, 2, "before"), (2, 1, "before")])
def test_forward_matches_the_c_oracle(depth, chunk, read):
    d, ex, B, T, H = 6, 2, 2, 6, 1
    k, v, q, (th, et, al), st, _, _ = rand_case(1, B, T, H, d, depth, ex)
    y, end = BW.forward(d, depth, ex, chunk, st, k, v, q, th, et, al, read=read)
    ref = st.copy()
    yr = tmref.forward(d, depth, ex, chunk, ref, k, v, th, et, al, q=q, read=read)
    assert np.max(np.abs(y - yr)) < 1e-12 * max(1.0, np.max(np.abs(yr)))
    assert np.max(np.abs(end - ref)) < 1e-12 * max(1.0, np.max(np.abs(ref)))


def loss_of(d, depth, ex, chunk, st, k, v, q, th, et, al, dy, dst, read):
    y, end = BW.forward(d, depth, ex, chunk, st, k, v, q, th, et, al, read=read)
    return float(np.sum(dy * y) + np.sum(dst * end))


@pytest.mark.parametrize("depth,chunk,read", [(1, 2, "after"), (2, 2, "after"), (3, 3, "before"), (2, 1, "after")])
def test_gradients_match_finite_differences(depth, chunk, read):
    d, ex, B, T, H = 4, 2, 1, 6, 2
    k, v, q, (th, et, al), st, dy, dst = rand_case(2, B, T, H, d, depth, ex)
    g = BW.forward_backward(d, depth, ex, chunk, st, k, v, q, th, et, al, dy, dst, read=read)
    rng = np.random.default_rng(5)
    args = dict(k=k, v=v, q=q, th=th, et=et, al=al, st=st)
    names = dict(k="dk", v="dv", q="dq", th="dtheta", et="deta", al="dalpha", st="dstate_in")
    h = 1e-6
    for n, a in args.items():
        u = rng.standard_normal(a.shape)
        plus = dict(args, **{n: a + h * u})
        minus = dict(args, **{n: a - h * u})
        f = lambda kw: loss_of(d, depth, ex, chunk, kw["st"], kw["k"], kw["v"], kw["q"], kw["th"], kw["et"],
                               kw["al"], dy, dst, read)
        fd = (f(plus) - f(minus)) / (2 * h)
        an = float(np.sum(g[names[n]] * u))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (n, fd, an)


def test_state_gradient_matches_differences_of_the_c_oracle():
    # the C oracle's state is fp64: differences of its loss in the starting
    # state, against the gradient with respect to the state before the call
    d, depth, ex, chunk, B, T, H = 5, 2, 2, 2, 1, 4, 1
    k, v, q, (th, et, al), st, dy, dst = rand_case(3, B, T, H, d, depth, ex)
    g = BW.forward_backward(d, depth, ex, chunk, st, k, v, q, th, et, al, dy, dst)

    def c_loss(s0):
        s = s0.copy()
        y = tmref.forward(d, depth, ex, chunk, s, k, v, th, et, al, q=q)
        return float(np.sum(dy * y) + np.sum(dst * s))

    rng = np.random.default_rng(6)
    h = 1e-6
    for _ in range(3):
        u = rng.standard_normal(st.shape)
        fd = (c_loss(st + h * u) - c_loss(st - h * u)) / (2 * h)
        an = float(np.sum(g["dstate_in"] * u))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (fd, an)


def test_linear_one_token_closed_form():
    # y = q M_1 with M_1 = (1 - a) M_0 + e S_0 - th 2 k^T (k M_0 - v); the
    # gradients of L = <yb, y> + <Mb, M_1> + <Sb, S_1> worked out by hand
    rng = np.random.default_rng(7)
    d = 5
    k = rng.standard_normal(d); k /= np.linalg.norm(k)
    v, q, yb = rng.standard_normal(d), rng.standard_normal(d), rng.standard_normal(d)
    M0, S0, Mb, Sb = (rng.standard_normal((d, d)) for _ in range(4))
    th, e, a = 0.3, 0.6, 0.2
    f32 = lambda x: np.asarray(x, np.float32).astype(np.float64)
    k, v, q = f32(k), f32(v), f32(q)
    th, e, a = float(np.float32(th)), float(np.float32(e)), float(np.float32(a))
    r = k @ M0 - v                                  # the residual
    G = 2 * np.outer(k, r)                          # the linear memory's gradient
    S1 = e * S0 - th * G
    M1 = (1 - a) * M0 + S1
    qk = float(q @ k)
    Mt = np.outer(q, yb) + Mb                       # total adjoint of M_1
    St = Sb + Mt                                    # total adjoint of S_1
    want = {
        "dq": yb @ M1.T,
        "dv": 2 * th * (k @ St),
        # d/dk of <St, -th 2 k^T (k M0 - v)> = -2 th sum_ij k_i St_ij r_j, r = k M0 - v
        "dk": -2 * th * (St @ r + M0 @ (St.T @ k)),
        "dtheta": -np.sum(St * G),
        "deta": np.sum(St * S0),
        "dalpha": -np.sum(Mt * M0),
    }
    dM0 = (1 - a) * Mt - 2 * th * np.outer(k, k @ St)   # through the residual r = k M0 - v
    dS0 = e * St
    st = np.concatenate([M0.ravel(), S0.ravel()])[None]
    dst = np.concatenate([Mb.ravel(), Sb.ravel()])[None]
    r4 = lambda x: np.asarray(x).reshape(1, 1, 1, d)
    g1 = lambda x: np.full((1, 1, 1), x)
    g = BW.forward_backward(d, 1, 1, 1, st, r4(k), r4(v), r4(q), g1(th), g1(e), g1(a), r4(yb), dst)
    assert np.allclose(g["dq"].ravel(), want["dq"], rtol=1e-12, atol=1e-12)
    assert np.allclose(g["dv"].ravel(), want["dv"], rtol=1e-12, atol=1e-12)
    assert np.allclose(g["dk"].ravel(), want["dk"], rtol=1e-12, atol=1e-12)
    for n in ("dtheta", "deta", "dalpha"):
        assert abs(float(g[n].ravel()[0]) - float(want[n])) < 1e-12 * max(1, abs(want[n])), n
    assert np.allclose(g["dstate_in"][0, :d * d], dM0.ravel(), rtol=1e-12, atol=1e-12)
    assert np.allclose(g["dstate_in"][0, d * d:], dS0.ravel(), rtol=1e-12, atol=1e-12)


def test_writing_off_leaves_keys_and_values_without_gradient():
    # theta = 0: nothing is written, M_T = prod(1 - a_t) M_0 + (terms in S_0);
    # with S_0 = 0 and dS = 0: dk = dv = 0 and dalpha_t = -<dM, M_T> / (1 - a_t)
    d, depth, ex, chunk, B, T, H = 4, 3, 2, 2, 1, 6, 1
    k, v, q, (th, et, al), st, dy, dst = rand_case(8, B, T, H, d, depth, ex, s_scale=0.0)
    th = np.zeros_like(th)
    P = st.shape[1] // 2
    dst[:, P:] = 0.0
    g = BW.forward_backward(d, depth, ex, chunk, st, k, v, q, th, et, al, np.zeros_like(dy), dst)
    assert np.all(g["dk"] == 0) and np.all(g["dv"] == 0) and np.all(g["deta"] == 0)
    MT = np.prod(1 - al[0, :, 0]) * st[0, :P]
    assert np.allclose(g["state"][0, :P], MT, rtol=1e-12)
    want = -np.sum(dst[0, :P] * MT) / (1 - al[0, :, 0])
    assert np.allclose(g["dalpha"][0, :, 0], want, rtol=1e-10)


def test_split_call_chains_through_the_state():
    # one call of 6 tokens against calls of 4 then 2, the second call's
    # gradient with respect to its starting state fed to the first
    d, depth, ex, chunk, B, T, H = 4, 2, 2, 2, 1, 6, 1
    k, v, q, (th, et, al), st, dy, dst = rand_case(9, B, T, H, d, depth, ex)
    whole = BW.forward_backward(d, depth, ex, chunk, st, k, v, q, th, et, al, dy, dst)
    cut = lambda a, lo, hi: a[:, lo:hi]
    first = BW.forward(d, depth, ex, chunk, st, *(cut(a, 0, 4) for a in (k, v, q, th, et, al)))[1]
    g2 = BW.forward_backward(d, depth, ex, chunk, first, *(cut(a, 4, 6) for a in (k, v, q, th, et, al)),
                             cut(dy, 4, 6), dst)
    g1 = BW.forward_backward(d, depth, ex, chunk, st, *(cut(a, 0, 4) for a in (k, v, q, th, et, al)),
                             cut(dy, 0, 4), g2["dstate_in"])
    for n in ("dk", "dv", "dq", "dtheta", "deta", "dalpha"):
        assert np.allclose(np.concatenate([g1[n], g2[n]], axis=1), whole[n], rtol=1e-10, atol=1e-12), n
    assert np.allclose(g1["dstate_in"], whole["dstate_in"], rtol=1e-10, atol=1e-12)
