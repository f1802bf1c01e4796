"""ctypes wrapper around the fp64 CPU oracle (``oracle/tmref.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product library.  It shares no code
with the HIP path; the two only meet in the seeded input generator.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tmref.c")
_LIB = os.path.join(_HERE, "libtmref.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)


def build() -> str:
    """Compile the oracle with gcc (plain -O2: no fast-math, so every sum runs
    in the order written)."""
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-fopenmp",
                           "-o", tmp, _SRC, "-lm", "-lpthread"])
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        L.tmref_param_count.restype = ctypes.c_long
        L.tmref_param_count.argtypes = [ctypes.c_int] * 3
        L.tmref_mlp_forward.argtypes = [ctypes.c_int] * 3 + [_dp, _dp, _dp]
        L.tmref_mlp_grad.argtypes = [ctypes.c_int] * 3 + [_dp, _dp, _dp, _dp, _dp]
        L.tmref_forward.argtypes = ([ctypes.c_int] * 7 + [_fp] * 6 + [_dp, _dp, ctypes.c_int])
        L.tmref_forward_read.argtypes = ([ctypes.c_int] * 7 + [_fp] * 6 + [_dp, _dp, ctypes.c_int, ctypes.c_int])
        L.tmref_retrieve.argtypes = ([ctypes.c_int] * 6 + [_dp, _fp, _dp, ctypes.c_int])
        _lib = L
    return _lib


def _d(a):
    return a.ctypes.data_as(_dp)


def _f(a):
    return None if a is None else a.ctypes.data_as(_fp)


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def param_count(dim, depth, expansion):
    return lib().tmref_param_count(dim, depth, expansion)


def mlp_forward(dim, depth, expansion, W, x):
    """One row through the memory MLP (fp64)."""
    W = np.ascontiguousarray(W, np.float64)
    x = np.ascontiguousarray(x, np.float64)
    y = np.zeros(dim, np.float64)
    rc = lib().tmref_mlp_forward(dim, depth, expansion, _d(W), _d(x), _d(y))
    assert rc == 0, rc
    return y


def mlp_grad(dim, depth, expansion, W, k, v):
    """(gradient of ||M(k) - v||^2 w.r.t. the flat weights, loss)."""
    W = np.ascontiguousarray(W, np.float64)
    k = np.ascontiguousarray(k, np.float64)
    v = np.ascontiguousarray(v, np.float64)
    G = np.zeros_like(W)
    loss = np.zeros(1, np.float64)
    rc = lib().tmref_mlp_grad(dim, depth, expansion, _d(W), _d(k), _d(v), _d(G), _d(loss))
    assert rc == 0, rc
    return G, float(loss[0])


READ_MODES = {"after": 0, "before": 1, "token": 2}


def default_threads():
    """Threads for the oracle: the host's cores, at most 16 (a GPU host's
    share per device).  Streams get a thread each; spare threads split each
    stream's element loops (bitwise the same results)."""
    return max(1, min(os.cpu_count() or 1, 16))


def forward(dim, depth, expansion, chunk, state, k, v, theta, eta, alpha, q=None,
            n_threads=None, read="after"):
    """Store the call's tokens into ``state`` (fp64 [streams][2P], updated in
    place); if ``q`` is given also return y [B][T][H][d] read chunk by chunk,
    through the memory after the chunk's write (read="after") or the memory
    the chunk started with (read="before"), or each query through the memory
    as its own token's write left it (read="token").  k, v, q: [B][T][H][d];
    gates [B][T][H]."""
    k, v, q = _f32(k), _f32(v), _f32(q)
    theta, eta, alpha = _f32(theta), _f32(eta), _f32(alpha)
    B, T, H, d = k.shape
    assert d == dim and state.dtype == np.float64 and state.flags.c_contiguous
    assert state.shape == (B * H, 2 * param_count(dim, depth, expansion))
    y = np.zeros((B, T, H, d), np.float64) if q is not None else None
    nt = n_threads or default_threads()
    rc = lib().tmref_forward_read(dim, depth, expansion, chunk, B, H, T, _f(k), _f(v), _f(q),
                                  _f(theta), _f(eta), _f(alpha), _d(state),
                                  _d(y) if y is not None else None, READ_MODES[read], nt)
    if rc != 0:
        raise ValueError("tmref_forward failed: %d" % rc)
    return y


def retrieve(dim, depth, expansion, state, q, n_threads=None):
    """y = M(q) for every query; the state is not written."""
    q = _f32(q)
    B, T, H, d = q.shape
    state = np.ascontiguousarray(state, np.float64)
    y = np.zeros((B, T, H, d), np.float64)
    nt = n_threads or default_threads()
    rc = lib().tmref_retrieve(dim, depth, expansion, B, H, T, _d(state), _f(q), _d(y), nt)
    if rc != 0:
        raise ValueError("tmref_retrieve failed: %d" % rc)
    return y


def nonfinite(state) -> bool:
    return not bool(np.all(np.isfinite(state)))
