"""Seeded synthetic workloads for the neural long-term memory (Titans).

This module only draws random numbers and shapes them into the arrays that
the memory consumes: keys, values, queries, the three per-token gates and the
initial memory weights.  It holds none of the memory's own arithmetic (no
forward pass, no gradient, no momentum or forgetting), so the fp64 oracle and
the HIP library can both be fed from it without sharing any of the method.

Workload recipe (all draws from numpy's PCG64 ``default_rng``):

* Per token the input is a model vector x ~ N(0, 1) of width D = heads * dim.
* Keys, values and queries are linear projections, k = x W_K, v = x W_V,
  q = x W_Q, as in "Titans, explained", method step 1 (project each token to a
  key and a value; the query is the same kind of projection, step 5).  The
  projection entries are N(0, 1/D) (variance 1/D).
* Keys and queries are l2-normalised per head (step 1 again), with the norm
  clamped below at 1e-12.  Values are not normalised.  The short depthwise
  convolution of step 1 is left out: none of the workloads has one.
* The gates theta (write strength), eta (momentum) and alpha (forgetting) are
  sigmoid(x w + offset) per token and head, with w ~ N(0, 1/D) of shape
  [D][heads].  The pages only say the three controls are computed from the
  input ("Titans, explained", step 4); the fixed per-gate offset is the bias
  any such linear gate has and keeps the MLP memories finite and alive over
  the workload's length.
* The memory starts at S = 0 and either M = 0 (the linear memory) or, for an
  MLP, W_l ~ N(0, 1/fan_in) drawn per head, then per layer.
* Draw order: W_K, W_V, W_Q, w_theta, w_eta, w_alpha, then the memory init;
  the tokens of call j come from ``default_rng([seed, 1, j])``.
* For bf16 workloads k, v and q are rounded to bfloat16 (round to nearest
  even) here, on the host, and handed out as float32 arrays holding exactly
  those bf16 values, so both consumers see identical numbers.
"""
from __future__ import annotations

import dataclasses
import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seq: int              # tokens per stream over the whole workload
    heads: int
    dim: int              # per-head memory width d
    depth: int            # number of weight matrices in the memory MLP
    expansion: int        # hidden width = dim * expansion (depth >= 2)
    chunk: int            # b, tokens per mini-batch
    dtype: str            # "f32" or "bf16": type of k, v, q
    offsets: tuple        # gate logit offsets (theta, eta, alpha)
    calls: int = 1        # the stream is fed in this many equal calls
    zero_init: bool = False

    @property
    def model_dim(self) -> int:
        return self.heads * self.dim

    @property
    def hidden(self) -> int:
        return self.dim * self.expansion if self.depth > 1 else self.dim

    @property
    def tokens_per_call(self) -> int:
        return self.seq // self.calls

    @property
    def streams(self) -> int:
        return self.batch * self.heads

    def layer_dims(self):
        """(d_in, d_out) of each weight matrix, first layer first."""
        if self.depth == 1:
            return [(self.dim, self.dim)]
        h = self.hidden
        dims = [(self.dim, h)]
        dims += [(h, h)] * (self.depth - 2)
        dims += [(h, self.dim)]
        return dims

    @property
    def params(self) -> int:
        return sum(a * b for a, b in self.layer_dims())

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: a 64x64 linear memory; the README-sized 2-layer MLP
# (dim 384, chunk 64, a (2, 1024, 384) input); the same memory streamed over
# 16 calls; an 8-head memory over model dim 1024; a 4-layer memory over a
# 1,048,576-token stream.
WORKLOADS = {
    "linear64": Workload("linear64", batch=1, seq=256, heads=1, dim=64, depth=1,
                         expansion=1, chunk=16, dtype="f32", offsets=(0.0, 0.0, 0.0),
                         zero_init=True),
    "mlp384": Workload("mlp384", batch=2, seq=1024, heads=1, dim=384, depth=2,
                       expansion=4, chunk=64, dtype="bf16", offsets=(-7.0, 2.0, -7.0)),
    "mlp384_stream": Workload("mlp384_stream", batch=4, seq=16384, heads=1, dim=384,
                              depth=2, expansion=4, chunk=64, dtype="bf16",
                              offsets=(-7.0, 2.0, -7.0), calls=16),
    "multihead1024": Workload("multihead1024", batch=8, seq=32768, heads=8, dim=128,
                              depth=2, expansion=4, chunk=64, dtype="bf16",
                              offsets=(-7.0, 2.0, -7.0)),
    "deep512": Workload("deep512", batch=1, seq=1048576, heads=1, dim=512, depth=4,
                        expansion=4, chunk=32, dtype="bf16", offsets=(-6.0, 2.0, -7.0),
                        calls=1024),
}


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns
    float32 holding the rounded values.  NaN stays NaN."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    return np.where(np.isnan(a), a, out)


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


@dataclasses.dataclass
class Params:
    W_K: np.ndarray
    W_V: np.ndarray
    W_Q: np.ndarray
    w_gate: tuple           # (w_theta, w_eta, w_alpha), each [D][heads]
    init_weights: np.ndarray  # [heads][P] float32, canonical row-major layers


def make_params(wl: Workload, seed: int = 0) -> Params:
    """Projection, gate and memory-init parameters in the fixed draw order."""
    rng = np.random.default_rng(seed)
    D = wl.model_dim
    sd = 1.0 / np.sqrt(D)
    W_K = rng.standard_normal((D, D)) * sd
    W_V = rng.standard_normal((D, D)) * sd
    W_Q = rng.standard_normal((D, D)) * sd
    w_gate = tuple(rng.standard_normal((D, wl.heads)) * sd for _ in range(3))
    init = np.zeros((wl.heads, wl.params), dtype=np.float32)
    if not wl.zero_init:
        for h in range(wl.heads):
            off = 0
            for din, dout in wl.layer_dims():
                w = rng.standard_normal((din, dout)) / np.sqrt(din)
                init[h, off:off + din * dout] = w.astype(np.float32).ravel()
                off += din * dout
    return Params(W_K, W_V, W_Q, w_gate, init)


@dataclasses.dataclass
class CallInputs:
    k: np.ndarray      # [B][T][H][d] float32 (bf16-exact values for bf16 workloads)
    v: np.ndarray
    q: np.ndarray
    theta: np.ndarray  # [B][T][H] float32
    eta: np.ndarray
    alpha: np.ndarray


def make_call(wl: Workload, params: Params, j: int = 0, seed: int = 0,
              batch_rows=None, tokens=None, offsets=None) -> CallInputs:
    """Inputs of call j.  ``batch_rows`` optionally restricts the draw to a
    subset of the batch (the draws of the other rows are still made, so the
    values do not depend on the subset).  ``tokens`` overrides the call length,
    ``offsets`` the gate offsets."""
    T = wl.tokens_per_call if tokens is None else tokens
    B, H, d, D = wl.batch, wl.heads, wl.dim, wl.model_dim
    offs = wl.offsets if offsets is None else offsets
    rng = np.random.default_rng([seed, 1, j])
    rows = range(B) if batch_rows is None else list(batch_rows)
    nb = len(rows)
    k = np.empty((nb, T, H, d), np.float32)
    v = np.empty_like(k)
    q = np.empty_like(k)
    gates = [np.empty((nb, T, H), np.float32) for _ in range(3)]
    W = [params.W_K.astype(np.float32), params.W_V.astype(np.float32),
         params.W_Q.astype(np.float32)]
    wg = [g.astype(np.float32) for g in params.w_gate]
    want = set(rows)
    slot = 0
    for b in range(B):
        x = rng.standard_normal((T, D), dtype=np.float64).astype(np.float32)
        if b not in want:
            continue
        kk, vv, qq = (x @ Wm for Wm in W)
        kk = kk.reshape(T, H, d)
        qq = qq.reshape(T, H, d)
        for a in (kk, qq):
            n = np.sqrt(np.sum(a.astype(np.float64) ** 2, axis=-1, keepdims=True))
            a /= np.maximum(n, 1e-12).astype(np.float32)
        k[slot], v[slot], q[slot] = kk, vv.reshape(T, H, d), qq
        for g, w, o in zip(gates, wg, offs):
            g[slot] = _sigmoid((x @ w).astype(np.float64) + o).astype(np.float32)
        slot += 1
    if wl.dtype == "bf16":
        k, v, q = round_bf16(k), round_bf16(v), round_bf16(q)
    return CallInputs(k, v, q, *gates)


def initial_state(wl: Workload, params: Params, batch: int | None = None) -> np.ndarray:
    """Initial memory as fp64 [streams][2P]: M = init (broadcast over batch),
    S = 0.  Stream index = batch_index * heads + head."""
    B = wl.batch if batch is None else batch
    P = wl.params
    st = np.zeros((B * wl.heads, 2 * P), np.float64)
    for b in range(B):
        for h in range(wl.heads):
            st[b * wl.heads + h, :P] = params.init_weights[h]
    return st


@dataclasses.dataclass
class PrologueInputs:
    x: np.ndarray        # [B][T][D] float32 (bf16-exact for bf16 workloads)
    w_kvq: np.ndarray    # [3][D][H*d] float32 (bf16-exact for bf16): W_K, W_V, W_Q
    conv: np.ndarray     # [3][H*d][K] float32: per-channel taps, tap j for j tokens back
    w_gate: np.ndarray   # [3][D][H] float32: theta, eta, alpha
    gate_bias: np.ndarray  # [3] float32: the gate offsets


def make_prologue(wl: Workload, params: Params, j: int = 0, seed: int = 0, conv_len: int = 4,
                  tokens=None) -> PrologueInputs:
    """The token vectors of call j (the same draws as make_call) with the
    projection and gate weights of ``params``, and per-channel convolution
    taps ~ N(0, 1/conv_len) from their own generator.  Draws only: the input
    side's arithmetic is not done here."""
    T = wl.tokens_per_call if tokens is None else tokens
    B, D = wl.batch, wl.model_dim
    rng = np.random.default_rng([seed, 1, j])
    x = np.stack([rng.standard_normal((T, D), dtype=np.float64).astype(np.float32) for _ in range(B)])
    w = np.stack([params.W_K, params.W_V, params.W_Q]).astype(np.float32)
    crng = np.random.default_rng([seed, 2])
    conv = (crng.standard_normal((3, D, conv_len)) / np.sqrt(conv_len)).astype(np.float32)
    wg = np.stack(params.w_gate).astype(np.float32)
    if wl.dtype == "bf16":
        x, w = round_bf16(x), round_bf16(w)
    return PrologueInputs(x, w, conv, wg, np.asarray(wl.offsets, np.float32))
