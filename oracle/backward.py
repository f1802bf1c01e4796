"""fp64 CPU oracle of the backward through the memory's store.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product library.  It shares no
code with the HIP path.

What it computes.  A call of tm_forward maps (the state before the call,
k, v, q, theta, eta, alpha) to (y, the state after the call); the training
of a model around the memory needs the gradient of an outer loss through that
map ("titans-pytorch analysis", Editorial conclusion: the loss must
backpropagate through the memory state; "Titans, explained", step 6: the
chunked form is what makes the memory trainable in parallel).  Given the
outer loss's gradients with respect to the outputs -- dy for y, and dM, dS for
the state after the call -- this module returns the gradients of

    L = sum(dy * y) + sum(dM * M_T) + sum(dS * S_T)

with respect to k, v, q, theta, eta, alpha and the state before the call
(M_0, S_0): the vector-Jacobian product of the call.

How.  The forward is the literal recurrence of the pages, token by token and
chunk by chunk, written with plain PyTorch CPU operations in float64:

  * the memory is an MLP without biases, SiLU between layers, row vectors
    (y = x W); the loss of a token is ||M(k_t) - v_t||^2 ("Titans,
    explained", step 2);
  * every token's surprise is the gradient of that loss with respect to the
    weights the chunk started with (step 6; "Attack of the Titans", Parallel
    training), obtained here from torch.autograd.grad with create_graph=True
    so that it stays differentiable;
  * S_t = eta_t S_{t-1} - theta_t grad, then M_t = (1 - alpha_t) M_{t-1} + S_t
    (steps 3 and 4);
  * the queries of chunk c read the memory after the chunk's write (read
    "after"), or the memory the chunk started with (read "before")
    (step 5).

torch.autograd then differentiates L through this recurrence (a library
primitive serving as a step: reverse-mode differentiation of the literal
program, second order through the per-token gradients).  Nothing is reordered,
blocked or rewritten in closed form.

State layout as in oracle/tmref.c: per stream 2P values, M_1..M_L then
S_1..S_L, each W_l row-major [d_in][d_out].  Token arrays are
[batch][n_tokens][heads][dim], gates [batch][n_tokens][heads].
"""
from __future__ import annotations

import numpy as np
import torch


def layer_dims(dim, depth, expansion):
    """(d_in, d_out) of each weight matrix, first layer first."""
    if depth == 1:
        return [(dim, dim)]
    h = dim * expansion
    return [(dim, h)] + [(h, h)] * (depth - 2) + [(h, dim)]


def _mlp(Ws, x):
    """Rows x through the memory: z = h W per layer, SiLU between layers."""
    h = x
    for i, W in enumerate(Ws):
        h = h @ W
        if i < len(Ws) - 1:
            h = torch.nn.functional.silu(h)
    return h


def _split(vec, dims):
    out, off = [], 0
    for a, b in dims:
        out.append(vec[off:off + a * b].reshape(a, b))
        off += a * b
    return out


def stream_forward(dims, chunk, M, S, k, v, q, theta, eta, alpha, read="after"):
    """The literal recurrence on one stream.  M, S: lists of [d_in][d_out]
    tensors (the state before the call); k, v, q: [T][d]; gates: [T].
    Returns (y [T][d], M after, S after).  Differentiable."""
    T = k.shape[0]
    y = [None] * T
    for c0 in range(0, T, chunk):
        M0 = list(M)                           # the weights the chunk started with
        if read == "before":
            y[c0:c0 + chunk] = list(_mlp(M0, q[c0:c0 + chunk]))
        for t in range(c0, c0 + chunk):
            loss = ((_mlp(M0, k[t:t + 1])[0] - v[t]) ** 2).sum()
            G = torch.autograd.grad(loss, M0, create_graph=True)
            S = [eta[t] * s_l - theta[t] * g_l for s_l, g_l in zip(S, G)]
            M = [(1 - alpha[t]) * m_l + s_l for m_l, s_l in zip(M, S)]
        if read == "after":
            y[c0:c0 + chunk] = list(_mlp(M, q[c0:c0 + chunk]))
    return torch.stack(y), M, S


def forward(dim, depth, expansion, chunk, state, k, v, q, theta, eta, alpha, read="after"):
    """The forward alone (numpy in, numpy out): y [B][T][H][d] and the state
    after the call [streams][2P]."""
    dims = layer_dims(dim, depth, expansion)
    B, T, H, d = k.shape
    P = sum(a * b for a, b in dims)
    y = np.zeros((B, T, H, d))
    out = np.zeros_like(np.asarray(state, np.float64))
    for s in range(B * H):
        bi, hi = divmod(s, H)
        st = torch.tensor(np.asarray(state[s], np.float64))
        M = [w.clone().requires_grad_(True) for w in _split(st[:P], dims)]
        S = _split(st[P:], dims)
        tk = lambda a: torch.tensor(np.asarray(a[bi, :, hi], np.float64))
        ys, Me, Se = stream_forward(dims, chunk, M, S, tk(k), tk(v), tk(q), tk(theta), tk(eta), tk(alpha), read)
        y[bi, :, hi] = ys.detach().numpy()
        out[s] = torch.cat([w.detach().reshape(-1) for w in Me + Se]).numpy()
    return y, out


def forward_backward(dim, depth, expansion, chunk, state, k, v, q, theta, eta, alpha, dy, dstate=None,
                     read="after"):
    """Gradients of L = sum(dy * y) + <dstate, state after the call> with
    respect to every input.  state, dstate: [streams][2P] (dstate None: the
    state after the call does not enter L).  Returns a dict with y, the
    state after the call, and dk, dv, dq ([B][T][H][d]), dtheta, deta,
    dalpha ([B][T][H]) and dstate_in ([streams][2P]: the gradient with
    respect to the state before the call)."""
    dims = layer_dims(dim, depth, expansion)
    B, T, H, d = k.shape
    P = sum(a * b for a, b in dims)
    out = {n: np.zeros((B, T, H, d)) for n in ("y", "dk", "dv", "dq")}
    for n in ("dtheta", "deta", "dalpha"):
        out[n] = np.zeros((B, T, H))
    out["state"] = np.zeros((B * H, 2 * P))
    out["dstate_in"] = np.zeros((B * H, 2 * P))
    for s in range(B * H):
        bi, hi = divmod(s, H)
        leaf = lambda a: torch.tensor(np.asarray(a[bi, :, hi], np.float64), requires_grad=True)
        tk, tv, tq, tth, tet, tal = (leaf(a) for a in (k, v, q, theta, eta, alpha))
        st = torch.tensor(np.asarray(state[s], np.float64), requires_grad=True)
        M = _split(st[:P], dims)
        S = _split(st[P:], dims)
        ys, Me, Se = stream_forward(dims, chunk, M, S, tk, tv, tq, tth, tet, tal, read)
        end = torch.cat([w.reshape(-1) for w in Me + Se])
        L = (torch.tensor(np.asarray(dy[bi, :, hi], np.float64)) * ys).sum()
        if dstate is not None:
            L = L + (torch.tensor(np.asarray(dstate[s], np.float64)) * end).sum()
        grads = torch.autograd.grad(L, [tk, tv, tq, tth, tet, tal, st], allow_unused=True)
        for n, g in zip(("dk", "dv", "dq"), grads[:3]):
            out[n][bi, :, hi] = 0.0 if g is None else g.numpy()
        for n, g in zip(("dtheta", "deta", "dalpha"), grads[3:6]):
            out[n][bi, :, hi] = 0.0 if g is None else g.numpy()
        out["dstate_in"][s] = grads[6].numpy()
        out["y"][bi, :, hi] = ys.detach().numpy()
        out["state"][s] = end.detach().numpy()
    return out
