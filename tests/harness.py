"""Test harness: run a workload through the HIP library (via the C ABI) and
through the fp64 oracle on the same seeded host arrays."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

from oracle import tmref
from test_trained_neural_amd import inputs as I
import test_trained_neural_amd as T


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def relerr(a, b):
    """Relative Frobenius error ||a - b|| / ||b|| over the whole tensor."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def row_err(a, b):
    """Worst row's relative error, a row being one vector along the last
    axis (one token's output): max_r ||a_r - b_r|| / max(||b_r||, rms), rms
    the root-mean-square row norm of b.  The floor: a row's rounding error
    scales with the weights and the input row, not with the output row's
    own norm, so a row far smaller than typical is measured against the
    typical row (a wholly wrong row still scores its norm over rms)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if b.size == 0:
        return 0.0
    a2 = a.reshape(-1, b.shape[-1])
    b2 = b.reshape(-1, b.shape[-1])
    nb = np.linalg.norm(b2, axis=1)
    rms = float(np.sqrt(np.mean(nb ** 2)))
    floor = rms if rms > 0 else 1.0
    return float(np.max(np.linalg.norm(a2 - b2, axis=1) / np.maximum(nb, floor)))


def max_err(a, b):
    """max |a - b| / max |b| (element-wise, over the whole tensor)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if b.size == 0:
        return 0.0
    mb = float(np.max(np.abs(b)))
    return float(np.max(np.abs(a - b)) / (mb if mb > 0 else 1.0))


# A single row's rounding error is bounded by the unit roundoff times the
# condition number of its sums, which varies from row to row; the worst of
# a few thousand rows sits a few times above the tensor-wide ratio.  The row
# measure is therefore held to ROW_SLACK times the tolerance.
ROW_SLACK = 2.0


def yerr(a, b):
    """Parity measure of an output tensor against its reference, compared
    with the tolerance: the worst of the relative Frobenius error,
    max |a - b| / max |b| and the worst row's relative error (row_err)
    divided by ROW_SLACK.  NaN anywhere gives NaN, which fails every
    comparison."""
    return float(np.max([relerr(a, b), max_err(a, b), row_err(a, b) / ROW_SLACK]))


def dev_inputs(ci: I.CallInputs, dtype: str):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {}
    for name in ("k", "v", "q"):
        out[name] = torch.from_numpy(np.ascontiguousarray(getattr(ci, name))).to("cuda").to(tdt).contiguous()
    for name in ("theta", "eta", "alpha"):
        out[name] = torch.from_numpy(np.ascontiguousarray(getattr(ci, name))).to("cuda").contiguous()
    return out


class GpuMemory:
    """A memory of batch*heads streams held in a device state blob."""

    def __init__(self, wl: I.Workload, params: I.Params, batch=None, init_weights=None):
        self.wl = wl
        self.B = wl.batch if batch is None else batch
        self.H = wl.heads
        self.ctx = T.tm_create(wl.dim, wl.depth, wl.expansion, wl.chunk)
        self.P = T.tm_param_count(self.ctx)
        assert self.P == wl.params
        self.state = torch.empty(T.tm_state_bytes(self.ctx, self.B, self.H), dtype=torch.uint8, device="cuda")
        w = params.init_weights if init_weights is None else init_weights
        self.init = torch.from_numpy(np.ascontiguousarray(w, np.float32)).to("cuda")
        T.tm_state_init(self.ctx, self.state, self.B, self.H, self.init)
        self.ws = None

    def _ws(self, n):
        need = T.tm_workspace_bytes(self.ctx, self.B, self.H, n)
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        return self.ws

    def forward(self, d, read=None):
        B, Tn, H, dim = d["k"].shape
        y = torch.empty((B, Tn, H, dim), dtype=torch.float32, device="cuda")
        if read is None:
            T.tm_forward(self.ctx, self.state, d["k"], d["v"], d["q"], d["theta"], d["eta"], d["alpha"], y,
                         self._ws(Tn))
        else:
            T.tm_forward_ex(self.ctx, self.state, d["k"], d["v"], d["q"], d["theta"], d["eta"], d["alpha"], y,
                            self._ws(Tn), read)
        return y

    def store(self, d):
        T.tm_store(self.ctx, self.state, d["k"], d["v"], d["theta"], d["eta"], d["alpha"],
                   self._ws(d["k"].shape[1]))

    def retrieve(self, q):
        B, Tn, H, dim = q.shape
        y = torch.empty((B, Tn, H, dim), dtype=torch.float32, device="cuda")
        T.tm_retrieve(self.ctx, self.state, q, y, self._ws(Tn))
        return y

    def export(self):
        out = torch.empty((self.B * self.H, 2 * self.P), dtype=torch.float32, device="cuda")
        T.tm_state_export(self.ctx, self.state, self.B, self.H, out)
        return out.cpu().numpy()

    def import_(self, arr):
        src = torch.from_numpy(np.ascontiguousarray(arr, np.float32)).to("cuda")
        T.tm_state_import(self.ctx, self.state, self.B, self.H, src)
        torch.cuda.synchronize()

    def check(self):
        return T.tm_state_check(self.ctx, self.state, self.B, self.H)

    def close(self):
        T.tm_destroy(self.ctx)
        self.ctx = None


def oracle_forward(wl: I.Workload, state: np.ndarray, ci: I.CallInputs, with_q=True, threads=None,
                   read="after"):
    return tmref.forward(wl.dim, wl.depth, wl.expansion, wl.chunk, state, ci.k, ci.v, ci.theta, ci.eta,
                         ci.alpha, q=ci.q if with_q else None, n_threads=threads, read=read)


def compare_state(wl: I.Workload, gpu_state, ref_state):
    """(error of M, error of S): the worst over streams and weight matrices
    of both ||X_gpu - X_ref||_F / ||X_ref||_F and max |X_gpu - X_ref| /
    max |X_ref| (element-wise) per matrix."""
    P = wl.params
    em, es = [], []
    for s in range(ref_state.shape[0]):
        off = 0
        for din, dout in wl.layer_dims():
            n = din * dout
            gm, rm = gpu_state[s, off:off + n], ref_state[s, off:off + n]
            gs, rs = gpu_state[s, P + off:P + off + n], ref_state[s, P + off:P + off + n]
            em.append(max(relerr(gm, rm), max_err(gm, rm)))
            es.append(max(relerr(gs, rs), max_err(gs, rs)))
            off += n
    # np.max propagates NaN (a NaN anywhere must fail the comparison)
    return float(np.max(em)), float(np.max(es))


TOL = {"f32": 1e-4, "bf16": 2e-2}
