"""Titans neural long-term memory on MI355X: Python binding of ``libtm.so``.

Argument marshalling only: every step of the store / retrieve path runs in
the HIP kernels behind the C ABI declared in ``include/tm.h``.  PyTorch
supplies device memory (tensors) and the HIP stream.  The functions carry the
C names; batch, heads and n_tokens are read off the [batch][n_tokens][heads]
[dim] token tensors, and the dtype off their element type (bfloat16 or
float32).  ``NeuralMemory`` wraps them into the pages' call
``retrieved, mem_state = memory(...)``.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtm.so")

TM_OK, TM_ERR_INVALID, TM_ERR_SHAPE, TM_ERR_DTYPE, TM_ERR_STATE, TM_ERR_HIP, TM_ERR_SCRATCH = 0, -1, -2, -3, -4, -5, -6
TM_F32, TM_BF16 = 0, 1
TM_READ_AFTER_WRITE, TM_READ_BEFORE_WRITE, TM_READ_PER_TOKEN = 0, 1, 2

EXPORTED = ("tm_create", "tm_destroy", "tm_param_count", "tm_state_bytes", "tm_workspace_bytes",
            "tm_state_init", "tm_store", "tm_retrieve", "tm_forward", "tm_state_export",
            "tm_state_import", "tm_state_check", "tm_status_str", "tm_timing_enable", "tm_timing_read",
            "tm_graphs_enable", "tm_w1_split_enable", "tm_store_groups_enable", "tm_forward_ex", "tm_project",
            "tm_mac_window", "tm_mac_gate", "tm_config", "tm_forward_noalloc", "tm_backward",
            "tm_backward_workspace_bytes")

# kernel classes of tm_timing_enable / tm_timing_read (3 is unused); 8 and 9
# are tm_backward's state-streaming launches and its other launches
K_SCAN, K_FWD, K_BWD, K_FIRST, K_TOKEN_READ, K_PROJECT, K_MAC = 0, 1, 2, 4, 5, 6, 7
K_BACKWARD_STATE, K_BACKWARD_REST = 8, 9

_lib = None
_vp = ctypes.c_void_p
_i = ctypes.c_int


class TMError(RuntimeError):
    def __init__(self, fn, code):
        msg = lib().tm_status_str(code).decode() if _lib is not None else str(code)
        super().__init__("%s failed: %s (%d)" % (fn, msg, code))
        self.code = code


def lib():
    """Load libtm.so.  Raises if it has not been built: there is no other
    implementation to fall back to."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libtm.so is not built (run python -m test_trained_neural_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        L.tm_create.restype = _i
        L.tm_create.argtypes = [_i, _i, _i, _i, ctypes.POINTER(_vp)]
        L.tm_destroy.restype = None
        L.tm_destroy.argtypes = [_vp]
        L.tm_param_count.restype = ctypes.c_size_t
        L.tm_param_count.argtypes = [_vp]
        L.tm_config.restype = _i
        L.tm_config.argtypes = [_vp] + [ctypes.POINTER(_i)] * 4
        L.tm_state_bytes.restype = ctypes.c_size_t
        L.tm_state_bytes.argtypes = [_vp, _i, _i]
        L.tm_workspace_bytes.restype = ctypes.c_size_t
        L.tm_workspace_bytes.argtypes = [_vp, _i, _i, _i]
        L.tm_state_init.restype = _i
        L.tm_state_init.argtypes = [_vp, _vp, _i, _i, _vp, _vp]
        L.tm_store.restype = _i
        L.tm_store.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp]
        L.tm_retrieve.restype = _i
        L.tm_retrieve.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp]
        L.tm_forward.restype = _i
        L.tm_forward.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp]
        L.tm_forward_ex.restype = _i
        L.tm_backward.restype = _i
        L.tm_backward.argtypes = [_vp] * 16 + [_i, _i, _i, _i, _i, _vp, _vp]
        L.tm_backward_workspace_bytes.restype = ctypes.c_size_t
        L.tm_backward_workspace_bytes.argtypes = [_vp, _i, _i, _i]
        L.tm_forward_noalloc.restype = _i
        L.tm_forward_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp]
        L.tm_project.restype = _i
        L.tm_project.argtypes = [_vp, _vp, _i, _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _i, _i, _i, _i, _vp]
        L.tm_forward_ex.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp]
        L.tm_mac_window.restype = _i
        L.tm_mac_window.argtypes = [_vp, _i, _vp, _vp, _vp, _i, _i, _i, _i, _vp]
        L.tm_mac_gate.restype = _i
        L.tm_mac_gate.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _vp]
        L.tm_state_export.restype = _i
        L.tm_state_export.argtypes = [_vp, _vp, _i, _i, _vp, _vp]
        L.tm_state_import.restype = _i
        L.tm_state_import.argtypes = [_vp, _vp, _i, _i, _vp, _vp]
        L.tm_state_check.restype = _i
        L.tm_state_check.argtypes = [_vp, _vp, _i, _i, ctypes.POINTER(_i),
                                     ctypes.POINTER(ctypes.c_longlong), _vp]
        L.tm_timing_enable.restype = _i
        L.tm_timing_enable.argtypes = [_i]
        L.tm_timing_read.restype = _i
        L.tm_timing_read.argtypes = [_i, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_longlong)]
        L.tm_graphs_enable.restype = _i
        L.tm_graphs_enable.argtypes = [_i]
        L.tm_w1_split_enable.restype = _i
        L.tm_w1_split_enable.argtypes = [_i]
        L.tm_store_groups_enable.restype = _i
        L.tm_store_groups_enable.argtypes = [_i]
        L.tm_status_str.restype = ctypes.c_char_p
        L.tm_status_str.argtypes = [_i]
        _lib = L
    return _lib


def _check(fn, rc):
    if rc != TM_OK:
        raise TMError(fn, rc)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return _vp(stream.cuda_stream)


def _ptr(t):
    return None if t is None else _vp(t.data_ptr())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return TM_BF16
    if t.dtype == torch.float32:
        return TM_F32
    raise TypeError("token tensors must be bfloat16 or float32, got %s" % t.dtype)


def _tok(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda or not t.is_contiguous():
                raise ValueError("token and gate tensors must be contiguous device tensors")


def _same(dtype, *named):
    """Each (name, tensor) pair holds ``dtype`` (None tensors are skipped)."""
    for name, t in named:
        if t is not None and t.dtype != dtype:
            raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))


def _shape(name, t, shape):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _nbytes(t):
    return t.numel() * t.element_size()


def _blob(name, t, need):
    """t is a contiguous device tensor of at least ``need`` bytes (the state
    blob and the workspace are untyped bytes the kernels index by the call's
    sizes: a short buffer would be read or written past its end)."""
    if t is None or not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous device tensor" % name)
    if need == 0 or _nbytes(t) < need:
        raise ValueError("%s holds %d bytes; this call needs %d" % (name, _nbytes(t), need))


def _memory_sizes(ctx, state, workspace, B, H, T, d):
    """The token width matches the memory's dim; the state and workspace
    hold what tm_state_bytes / tm_workspace_bytes give for this call."""
    dim = tm_config(ctx)[0]
    if d != dim:
        raise ValueError("token vectors are %d wide; the memory's dim is %d" % (d, dim))
    _blob("state", state, tm_state_bytes(ctx, B, H))
    if workspace is not False:
        _blob("workspace", workspace, tm_workspace_bytes(ctx, B, H, T))


def _memory_call(k, v, q, theta, eta, alpha, y):
    """The token, gate and output tensors of a memory call: k, v, q
    [B][T][H][d] of one operand type, the gates [B][T][H] and y [B][T][H][d]
    fp32."""
    lead = k if k is not None else q
    _dtype_code(lead)
    _same(lead.dtype, ("v", v), ("q", q), ("k", k))
    _same(torch.float32, ("theta", theta), ("eta", eta), ("alpha", alpha), ("y", y))
    for name, t in (("v", v), ("q", q), ("y", y)):
        _shape(name, t, lead.shape)
    for name, t in (("theta", theta), ("eta", eta), ("alpha", alpha)):
        _shape(name, t, lead.shape[:3])


# ---------------------------------------------------------------------------
# the C calls, one to one

def tm_create(dim, depth, expansion, chunk):
    h = _vp()
    _check("tm_create", lib().tm_create(dim, depth, expansion, chunk, ctypes.byref(h)))
    return h


def tm_destroy(ctx):
    _forget(ctx)
    lib().tm_destroy(ctx)


def tm_param_count(ctx):
    return _cached(ctx, ("params",), lambda: lib().tm_param_count(ctx))


def tm_config(ctx):
    """(dim, depth, expansion, chunk) of the memory configuration."""
    def query():
        v = [_i(0) for _ in range(4)]
        _check("tm_config", lib().tm_config(ctx, *[ctypes.byref(x) for x in v]))
        return tuple(int(x.value) for x in v)
    return _cached(ctx, ("config",), query)


# The size queries and tm_config are pure functions of a ctx's (immutable)
# configuration and their arguments: the binding's argument checks, made on
# every call, remember them per ctx (forgotten by tm_destroy, so an address
# reused by a later ctx starts afresh).
_memo = {}


def _cached(ctx, key, fn):
    k = (ctx.value if isinstance(ctx, ctypes.c_void_p) else ctx,) + key
    v = _memo.get(k)
    if v is None:
        v = _memo[k] = fn()
    return v


def _forget(ctx):
    c = ctx.value if isinstance(ctx, ctypes.c_void_p) else ctx
    for k in [k for k in _memo if k[0] == c]:
        del _memo[k]


def tm_state_bytes(ctx, batch, heads):
    return _cached(ctx, ("state", batch, heads), lambda: lib().tm_state_bytes(ctx, batch, heads))


def tm_workspace_bytes(ctx, batch, heads, n_tokens):
    return _cached(ctx, ("ws", batch, heads, n_tokens), lambda: lib().tm_workspace_bytes(ctx, batch, heads, n_tokens))


def tm_state_init(ctx, state, batch, heads, init_weights, stream=None):
    _same(torch.float32, ("init_weights", init_weights))
    _tok(init_weights)
    _blob("state", state, tm_state_bytes(ctx, batch, heads))
    if init_weights.numel() != heads * tm_param_count(ctx):
        raise ValueError("init_weights must hold heads * P = %d values, got %d"
                         % (heads * tm_param_count(ctx), init_weights.numel()))
    _check("tm_state_init", lib().tm_state_init(ctx, _ptr(state), batch, heads, _ptr(init_weights),
                                                _stream(stream)))


def tm_store(ctx, state, k, v, theta, eta, alpha, workspace, stream=None):
    _memory_call(k, v, None, theta, eta, alpha, None)
    _tok(k, v, theta, eta, alpha)
    B, T, H, d = k.shape
    _memory_sizes(ctx, state, workspace, B, H, T, d)
    _check("tm_store", lib().tm_store(ctx, _ptr(state), _ptr(k), _ptr(v), _ptr(theta), _ptr(eta),
                                      _ptr(alpha), B, H, T, _dtype_code(k), _ptr(workspace),
                                      _stream(stream)))


def tm_retrieve(ctx, state, q, y, workspace, stream=None):
    _memory_call(None, None, q, None, None, None, y)
    _tok(q, y)
    B, T, H, d = q.shape
    _memory_sizes(ctx, state, workspace, B, H, T, d)
    _check("tm_retrieve", lib().tm_retrieve(ctx, _ptr(state), _ptr(q), _ptr(y), B, H, T,
                                            _dtype_code(q), _ptr(workspace), _stream(stream)))


def tm_forward(ctx, state, k, v, q, theta, eta, alpha, y, workspace, stream=None):
    _memory_call(k, v, q, theta, eta, alpha, y)
    _tok(k, v, q, theta, eta, alpha, y)
    B, T, H, d = k.shape
    _memory_sizes(ctx, state, workspace, B, H, T, d)
    _check("tm_forward", lib().tm_forward(ctx, _ptr(state), _ptr(k), _ptr(v), _ptr(q), _ptr(theta),
                                          _ptr(eta), _ptr(alpha), _ptr(y), B, H, T, _dtype_code(k),
                                          _ptr(workspace), _stream(stream)))


def tm_backward_workspace_bytes(ctx, batch, heads, n_tokens):
    return _cached(ctx, ("bws", batch, heads, n_tokens),
                   lambda: lib().tm_backward_workspace_bytes(ctx, batch, heads, n_tokens))


def tm_backward(ctx, state, k, v, q, theta, eta, alpha, dy, dstate, dk, dv, dq, dtheta, deta, dalpha, workspace,
                read=TM_READ_AFTER_WRITE, stream=None):
    """Gradients through one tm_forward call (see include/tm.h): ``state``
    is the state blob as it was before the call (read only); dy [B][T][H][d]
    fp32; dstate [B*H][2P] fp32, on entry the gradient with respect to the
    state after the call, on return the one with respect to the state
    before it; dk, dv, dq, dtheta, deta, dalpha are written."""
    _memory_call(k, v, q, theta, eta, alpha, None)
    _same(torch.float32, ("dy", dy), ("dk", dk), ("dv", dv), ("dq", dq), ("dtheta", dtheta), ("deta", deta),
          ("dalpha", dalpha), ("dstate", dstate))
    for name, t in (("dy", dy), ("dk", dk), ("dv", dv), ("dq", dq)):
        _shape(name, t, k.shape)
    for name, t in (("dtheta", dtheta), ("deta", deta), ("dalpha", dalpha)):
        _shape(name, t, k.shape[:3])
    _tok(k, v, q, theta, eta, alpha, dy, dk, dv, dq, dtheta, deta, dalpha)
    B, T, H, d = k.shape
    _memory_sizes(ctx, state, False, B, H, T, d)
    _canonical("dstate", dstate, ctx, B, H)
    _blob("workspace", workspace, tm_backward_workspace_bytes(ctx, B, H, T))
    _check("tm_backward", lib().tm_backward(ctx, _ptr(state), _ptr(k), _ptr(v), _ptr(q), _ptr(theta), _ptr(eta),
                                            _ptr(alpha), _ptr(dy), _ptr(dstate), _ptr(dk), _ptr(dv), _ptr(dq),
                                            _ptr(dtheta), _ptr(deta), _ptr(dalpha), B, H, T, _dtype_code(k),
                                            int(read), _ptr(workspace), _stream(stream)))


def tm_forward_noalloc(ctx, state, k, v, q, theta, eta, alpha, y, stream=None):
    """tm_forward with the library's own scratch array as the workspace (no
    device allocation; calls on one GPU must not overlap)."""
    _memory_call(k, v, q, theta, eta, alpha, y)
    _tok(k, v, q, theta, eta, alpha, y)
    B, T, H, d = k.shape
    _memory_sizes(ctx, state, False, B, H, T, d)
    _check("tm_forward_noalloc", lib().tm_forward_noalloc(ctx, _ptr(state), _ptr(k), _ptr(v), _ptr(q), _ptr(theta),
                                                          _ptr(eta), _ptr(alpha), _ptr(y), B, H, T,
                                                          _dtype_code(k), _stream(stream)))


def tm_forward_ex(ctx, state, k, v, q, theta, eta, alpha, y, workspace, read, stream=None):
    """read: TM_READ_AFTER_WRITE (as tm_forward), TM_READ_BEFORE_WRITE or
    TM_READ_PER_TOKEN."""
    _memory_call(k, v, q, theta, eta, alpha, y)
    _tok(k, v, q, theta, eta, alpha, y)
    B, T, H, d = k.shape
    _memory_sizes(ctx, state, workspace, B, H, T, d)
    _check("tm_forward_ex", lib().tm_forward_ex(ctx, _ptr(state), _ptr(k), _ptr(v), _ptr(q), _ptr(theta),
                                                _ptr(eta), _ptr(alpha), _ptr(y), B, H, T, _dtype_code(k),
                                                int(read), _ptr(workspace), _stream(stream)))


def tm_mac_window(persistent, recalled, segment, window, stream=None):
    """window [B][P+2S][D] = [persistent [P][D]; recalled [B][S][D] (fp32,
    rounded to the segment's dtype); segment [B][S][D]]."""
    _dtype_code(segment)
    _same(segment.dtype, ("persistent", persistent), ("window", window))
    _same(torch.float32, ("recalled", recalled))
    B, S, D = segment.shape
    P = 0 if persistent is None else persistent.shape[0]
    _shape("persistent", persistent, (P, D))
    _shape("recalled", recalled, (B, S, D))
    _shape("window", window, (B, P + 2 * S, D))
    _tok(recalled, segment, window)
    if persistent is not None:
        _tok(persistent)
    _check("tm_mac_window", lib().tm_mac_window(_ptr(persistent), P, _ptr(recalled), _ptr(segment), _ptr(window),
                                                B, S, D, _dtype_code(segment), _stream(stream)))


def tm_mac_gate(y, mem, out, stream=None):
    """out [B][S][D] fp32 = y * mem element-wise."""
    _dtype_code(y)
    _same(torch.float32, ("mem", mem), ("out", out))
    _shape("mem", mem, y.shape)
    _shape("out", out, y.shape)
    _tok(y, mem, out)
    B, S, D = y.shape
    _check("tm_mac_gate", lib().tm_mac_gate(_ptr(y), _ptr(mem), _ptr(out), B, S, D, _dtype_code(y),
                                            _stream(stream)))


def tm_project(ctx, x, w_kvq, conv, w_gate, gate_bias, history, k, v, q, theta, eta, alpha, heads,
               stream=None):
    """The input side: x [B][T][D] -> k, v, q [B][T][H][d] (x's dtype) and
    the gates [B][T][H] fp32; history [B][K-1][3][H*d] fp32 is read and
    rewritten (None for K = 1)."""
    _dtype_code(x)
    _same(x.dtype, ("w_kvq", w_kvq))
    _same(torch.float32, ("conv", conv), ("w_gate", w_gate), ("gate_bias", gate_bias), ("history", history))
    B, T, D = x.shape
    K = conv.shape[-1]
    HD = w_kvq.shape[1]
    _shape("w_kvq", w_kvq, (3, HD, D))
    _shape("conv", conv, (3, HD, K))
    _shape("w_gate", w_gate, (3, heads, D))
    _shape("gate_bias", gate_bias, (3,))
    if K > 1:
        _shape("history", history, (B, K - 1, 3, HD))
    _memory_call(k, v, q, theta, eta, alpha, None)
    dim = tm_config(ctx)[0]
    if HD != heads * dim:
        raise ValueError("w_kvq has %d output rows; heads * dim is %d" % (HD, heads * dim))
    _shape("k", k, (B, T, heads, dim))
    _tok(x, w_kvq, conv, w_gate, gate_bias, k, v, q, theta, eta, alpha)
    if history is not None:
        _tok(history)
    _check("tm_project", lib().tm_project(ctx, _ptr(x), D, _ptr(w_kvq), _ptr(conv), K, _ptr(w_gate),
                                          _ptr(gate_bias), _ptr(history) if history is not None else None,
                                          _ptr(k), _ptr(v), _ptr(q), _ptr(theta), _ptr(eta), _ptr(alpha),
                                          B, heads, T, _dtype_code(x), _stream(stream)))


def _canonical(name, t, ctx, batch, heads):
    n = batch * heads * 2 * tm_param_count(ctx)
    if t is None or not t.is_cuda or not t.is_contiguous() or t.numel() != n:
        raise ValueError("%s must be a contiguous device tensor of batch * heads * 2P = %d values" % (name, n))


def tm_state_export(ctx, state, batch, heads, dst, stream=None):
    _same(torch.float32, ("dst", dst))
    _canonical("dst", dst, ctx, batch, heads)
    _blob("state", state, tm_state_bytes(ctx, batch, heads))
    _check("tm_state_export", lib().tm_state_export(ctx, _ptr(state), batch, heads, _ptr(dst),
                                                    _stream(stream)))


def tm_state_import(ctx, state, batch, heads, src, stream=None):
    _same(torch.float32, ("src", src))
    _canonical("src", src, ctx, batch, heads)
    _blob("state", state, tm_state_bytes(ctx, batch, heads))
    _check("tm_state_import", lib().tm_state_import(ctx, _ptr(state), batch, heads, _ptr(src),
                                                    _stream(stream)))


def tm_state_check(ctx, state, batch, heads, stream=None):
    _blob("state", state, 256)   # the header
    nf = _i(0)
    pos = ctypes.c_longlong(0)
    _check("tm_state_check", lib().tm_state_check(ctx, _ptr(state), batch, heads, ctypes.byref(nf),
                                                  ctypes.byref(pos), _stream(stream)))
    return bool(nf.value), int(pos.value)


def tm_graphs_enable(on):
    _check("tm_graphs_enable", lib().tm_graphs_enable(1 if on else 0))


def tm_w1_split_enable(on):
    _check("tm_w1_split_enable", lib().tm_w1_split_enable(1 if on else 0))


def tm_store_groups_enable(on):
    _check("tm_store_groups_enable", lib().tm_store_groups_enable(1 if on else 0))


def tm_timing_enable(class_mask):
    _check("tm_timing_enable", lib().tm_timing_enable(class_mask))


def tm_timing_read(kernel_class):
    """(summed milliseconds, launches) of one kernel class since its last read."""
    ms = ctypes.c_double(0)
    n = ctypes.c_longlong(0)
    _check("tm_timing_read", lib().tm_timing_read(kernel_class, ctypes.byref(ms), ctypes.byref(n)))
    return float(ms.value), int(n.value)


# ---------------------------------------------------------------------------
# convenience wrapper: retrieved, mem_state = memory(...)

class MemState:
    """Opaque memory state of batch*heads streams (device bytes)."""

    def __init__(self, mem, batch, heads, device):
        self.batch, self.heads = batch, heads
        self.buf = torch.empty(tm_state_bytes(mem.ctx, batch, heads), dtype=torch.uint8, device=device)


def mac_segment(mem, state, x, persistent, attention, w_kvq, conv, w_gate, gate_bias, heads, hist_x=None,
                hist_y=None):
    """One segment of memory as a context, on the memory's side (argument
    marshalling over the C calls).  x [B][S][D] (D = heads * dim; S a
    multiple of the chunk) is the segment's model vectors; ``attention`` is
    the caller's: window [B][P+2S][D] (x's dtype) -> y [B][S][D] for the
    segment's positions, x's dtype.  The segment's queries (projections of x)
    read the memory before the segment is written; y is written (its keys,
    values and gates from the same projections) and read back through its
    queries to gate y.  Returns (out [B][S][D] fp32, state).  hist_x, hist_y:
    the two projection streams' convolution histories (see tm_project).
    The window handed to ``attention`` and the other intermediates are
    buffers the memory keeps and reuses: calls on one memory run on one
    stream at a time (as its state does), and ``attention`` keeps no
    reference to the window past its call."""
    B, S, D = x.shape
    dev, dt, d = x.device, x.dtype, mem.dim
    P = 0 if persistent is None else persistent.shape[0]
    # the intermediates live in buffers the memory keeps for its last
    # segment shape (reused in stream order); only the output is new
    key = (B, S, D, P, heads, dt, str(dev))
    if mem._mac is None or mem._mac[0] != key:
        f32 = torch.float32
        kvq = [torch.empty((B, S, heads, d), dtype=dt, device=dev) for _ in range(3)]
        g = [torch.empty((B, S, heads), dtype=f32, device=dev) for _ in range(3)]
        reads = [torch.empty((B, S, heads, d), dtype=f32, device=dev) for _ in range(2)]
        window = torch.empty((B, P + 2 * S, D), dtype=dt, device=dev)
        mem._mac = (key, kvq, g, reads, window)
    _, (k, v, q), g, (recalled, my), window = mem._mac
    ws = mem.workspace(B, heads, S)

    tm_project(mem.ctx, x, w_kvq, conv, w_gate, gate_bias, hist_x, k, v, q, g[0], g[1], g[2], heads)
    tm_retrieve(mem.ctx, state.buf, q, recalled, ws)
    tm_mac_window(persistent, recalled.view(B, S, D), x, window)
    y = attention(window).contiguous()
    tm_project(mem.ctx, y, w_kvq, conv, w_gate, gate_bias, hist_y, k, v, q, g[0], g[1], g[2], heads)
    tm_store(mem.ctx, state.buf, k, v, g[0], g[1], g[2], ws)
    tm_retrieve(mem.ctx, state.buf, q, my, ws)
    out = torch.empty((B, S, D), dtype=torch.float32, device=dev)
    tm_mac_gate(y, my.view(B, S, D), out)
    return out, state


class NeuralMemory:
    def __init__(self, dim, depth=2, expansion=4, chunk=64, device="cuda"):
        self.dim, self.depth, self.expansion, self.chunk = dim, depth, expansion, chunk
        self.device = torch.device(device)
        self.ctx = tm_create(dim, depth, expansion, chunk)
        self.params = tm_param_count(self.ctx)
        self._ws = None
        self._mac = None   # mac_segment's intermediates for its last segment shape

    def __del__(self):
        try:
            if self.ctx is not None and _lib is not None:
                tm_destroy(self.ctx)
        except Exception:
            pass

    def workspace(self, batch, heads, n_tokens):
        need = tm_workspace_bytes(self.ctx, batch, heads, n_tokens)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._ws

    def init_state(self, batch, heads, init_weights):
        st = MemState(self, batch, heads, self.device)
        w = init_weights.to(self.device, torch.float32).contiguous()
        assert w.numel() == heads * self.params
        tm_state_init(self.ctx, st.buf, batch, heads, w)
        return st

    def store(self, state, k, v, theta, eta, alpha):
        B, T, H, _ = k.shape
        tm_store(self.ctx, state.buf, k, v, theta, eta, alpha, self.workspace(B, H, T))
        return state

    def retrieve(self, state, q):
        B, T, H, d = q.shape
        y = torch.empty((B, T, H, d), dtype=torch.float32, device=self.device)
        tm_retrieve(self.ctx, state.buf, q, y, self.workspace(B, H, T))
        return y

    def __call__(self, state, k, v, q, theta, eta, alpha, read=TM_READ_AFTER_WRITE):
        """Store + retrieve; read: when each chunk's queries read the memory
        (TM_READ_AFTER_WRITE, the default, TM_READ_BEFORE_WRITE or
        TM_READ_PER_TOKEN)."""
        B, T, H, d = k.shape
        y = torch.empty((B, T, H, d), dtype=torch.float32, device=self.device)
        tm_forward_ex(self.ctx, state.buf, k, v, q, theta, eta, alpha, y, self.workspace(B, H, T), read)
        return y, state

    def export(self, state):
        out = torch.empty((state.batch * state.heads, 2 * self.params), dtype=torch.float32,
                          device=self.device)
        tm_state_export(self.ctx, state.buf, state.batch, state.heads, out)
        return out

    def import_(self, state, src):
        tm_state_import(self.ctx, state.buf, state.batch, state.heads, src.contiguous())
        return state

    def check(self, state):
        return tm_state_check(self.ctx, state.buf, state.batch, state.heads)
