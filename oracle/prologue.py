"""fp64 CPU oracle of the memory's input side: token -> key, value, query and
the three gates.

TEST INFRASTRUCTURE ONLY: imported by the tests and the benchmark's
CPU-baseline leg, never by the product library.  It shares no code with the
HIP path.

What it computes ("Titans, explained", method steps 1, 4 and 5):

* Projections k = x W_K, v = x W_V, q = x W_Q of each token's model vector x
  (row vectors; W is [D][H*d], head h owns columns h*d .. h*d + d - 1).
* A short depthwise convolution follows each projection: channel n of the
  output at token t is sum_j c[n][j] * p[t - j][n], j = 0 .. K-1, causal, per
  channel, no bias and no activation.  Tokens before the call come from the
  stream's history: the previous call's last K-1 projections (zeros at the
  stream start).
* Keys and queries are then l2-normalised per head (norm clamped below at
  1e-12); values are not.
* The gates theta, eta, alpha are sigmoid(x w_g + b_g) per token and head,
  with w_g [D][H] and one bias per gate.

The pages fix neither the convolution's length nor its history across calls,
nor the gates' form beyond "computed from the input"; the readings above are
the plainest ones (one bias per gate is the offset of the memory's input
recipe).
"""
from __future__ import annotations

import numpy as np


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def project(x, w_kvq, conv, w_gate, gate_bias, heads, history=None):
    """x [B][T][D]; w_kvq [3][D][H*d] (W_K, W_V, W_Q); conv [3][H*d][K];
    w_gate [3][D][H]; gate_bias [3]; history [B][K-1][3][H*d] (the previous
    call's last K-1 projections, oldest first) or None for the stream start.

    Returns (k, v, q [B][T][H][d], theta, eta, alpha [B][T][H], new history),
    all fp64."""
    x = np.asarray(x, np.float64)
    w_kvq = np.asarray(w_kvq, np.float64)
    conv = np.asarray(conv, np.float64)
    w_gate = np.asarray(w_gate, np.float64)
    B, T, D = x.shape
    HD = w_kvq.shape[2]
    d = HD // heads
    K = conv.shape[2]
    if history is None:
        history = np.zeros((B, K - 1, 3, HD))
    history = np.asarray(history, np.float64)
    # the projections, then the stream's past and this call's tokens in one
    # time axis: full[b, i, u] is projection i at time u - (K - 1)
    p = np.stack([x @ w_kvq[i] for i in range(3)], axis=1)            # [B][3][T][HD]
    full = np.concatenate([history.transpose(0, 2, 1, 3), p], axis=2)  # [B][3][K-1+T][HD]
    out = np.zeros_like(p)
    for j in range(K):
        # tap j multiplies the projection j tokens back
        out += conv[None, :, None, :, j] * full[:, :, K - 1 - j:K - 1 - j + T, :]
    k, v, q = (out[:, i].reshape(B, T, heads, d) for i in range(3))
    for a in (k, q):
        n = np.sqrt(np.sum(a * a, axis=-1, keepdims=True))
        a /= np.maximum(n, 1e-12)
    gates = [_sigmoid(x @ w_gate[g] + gate_bias[g]) for g in range(3)]
    new_history = full[:, :, T:, :].transpose(0, 2, 1, 3).copy()      # the last K-1 times
    return k, v, q, gates[0], gates[1], gates[2], new_history
