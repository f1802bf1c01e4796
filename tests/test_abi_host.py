"""Host side of the C ABI, no GPU needed: the library loads, exports every
entry point include/tm.h declares, and rejects bad arguments on the host
before anything is launched (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import test_trained_neural_amd as T

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "tm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tm_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    syms = declared_symbols()
    assert len(syms) == 26
    assert set(syms) == set(T.EXPORTED)
    L = ctypes.CDLL(T.LIB_PATH)
    for s in syms:
        assert hasattr(L, s), s


def test_create_validation():
    for args in [(48, 2, 4, 64), (2048, 2, 4, 64), (0, 2, 4, 64), (64, 0, 4, 64), (64, 9, 4, 64), (64, 2, 0, 64),
                 (64, 2, 4, 0), (64, 2, 4, 65)]:
        with pytest.raises(T.TMError) as e:
            T.tm_create(*args)
        assert e.value.code == T.TM_ERR_INVALID
    assert T.lib().tm_create(64, 1, 1, 16, None) == T.TM_ERR_INVALID


def test_sizes():
    c = T.tm_create(384, 2, 4, 64)
    P = 2 * 384 * 1536
    assert T.tm_param_count(c) == P
    # header + M + S (fp32) + bf16 copy, each 256-aligned
    assert T.tm_state_bytes(c, 2, 1) == 256 + 2 * P * 4 * 2 + 2 * P * 2
    assert T.tm_state_bytes(c, 0, 1) == 0
    c1 = T.tm_create(64, 1, 7, 16)   # depth 1 ignores the expansion
    assert T.tm_param_count(c1) == 64 * 64
    c4 = T.tm_create(512, 4, 4, 32)
    assert T.tm_param_count(c4) == 512 * 2048 * 2 + 2048 * 2048 * 2
    assert T.tm_workspace_bytes(c, 2, 1, 1024) > 0
    for h in (c, c1, c4):
        T.tm_destroy(h)


def test_call_validation_before_launch():
    # fake, aligned "device" addresses: every call below must be rejected on
    # the host, so nothing is dereferenced or launched
    L = T.lib()
    c = T.tm_create(64, 2, 2, 16)
    A = ctypes.c_void_p(1 << 20)
    G = ctypes.c_void_p((1 << 20) + 4096)
    st = ctypes.c_void_p(None)
    # n_tokens not a multiple of the chunk
    assert L.tm_store(c, A, A, A, G, G, G, 1, 1, 24, T.TM_BF16, A, st) == T.TM_ERR_SHAPE
    assert L.tm_forward(c, A, A, A, A, G, G, G, A, 1, 1, 17, T.TM_F32, A, st) == T.TM_ERR_SHAPE
    # bad dtype
    assert L.tm_store(c, A, A, A, G, G, G, 1, 1, 16, 7, A, st) == T.TM_ERR_DTYPE
    # null / misaligned pointers, bad sizes
    assert L.tm_store(c, None, A, A, G, G, G, 1, 1, 16, T.TM_BF16, A, st) == T.TM_ERR_INVALID
    assert L.tm_store(c, A, ctypes.c_void_p((1 << 20) + 2), A, G, G, G, 1, 1, 16, T.TM_BF16, A, st) == \
        T.TM_ERR_INVALID
    assert L.tm_store(c, ctypes.c_void_p((1 << 20) + 16), A, A, G, G, G, 1, 1, 16, T.TM_BF16, A, st) == \
        T.TM_ERR_INVALID
    assert L.tm_store(c, A, A, A, G, G, G, 0, 1, 16, T.TM_BF16, A, st) == T.TM_ERR_INVALID
    assert L.tm_store(c, A, A, A, G, G, G, 1, 1, -16, T.TM_BF16, A, st) == T.TM_ERR_INVALID
    assert L.tm_retrieve(c, A, None, A, 1, 1, 16, T.TM_BF16, A, st) == T.TM_ERR_INVALID
    assert L.tm_forward(c, A, A, A, None, G, G, G, A, 1, 1, 16, T.TM_BF16, A, st) == T.TM_ERR_INVALID
    assert L.tm_state_init(c, None, 1, 1, A, st) == T.TM_ERR_INVALID
    assert L.tm_state_export(c, A, 0, 1, A, st) == T.TM_ERR_INVALID
    # empty calls are no-ops that succeed without touching anything
    assert L.tm_store(c, A, A, A, G, G, G, 1, 1, 0, T.TM_BF16, A, st) == T.TM_OK
    assert L.tm_retrieve(c, A, A, A, 1, 1, 0, T.TM_BF16, A, st) == T.TM_OK
    # ... also with the (empty) token arrays given as null pointers
    assert L.tm_store(c, A, None, None, None, None, None, 1, 1, 0, T.TM_BF16, A, st) == T.TM_OK
    assert L.tm_forward(c, A, None, None, None, None, None, None, None, 1, 1, 0, T.TM_BF16, A, st) == T.TM_OK
    assert L.tm_retrieve(c, A, None, None, 1, 1, 0, T.TM_F32, A, st) == T.TM_OK
    # the read order: only the two defined values
    for bad in (-1, 3):
        assert L.tm_forward_ex(c, A, A, A, A, G, G, G, A, 1, 1, 16, T.TM_BF16, bad, A, st) == T.TM_ERR_INVALID
    assert L.tm_forward_ex(c, A, A, A, A, G, G, G, A, 1, 1, 17, T.TM_BF16, T.TM_READ_BEFORE_WRITE, A, st) == \
        T.TM_ERR_SHAPE
    assert L.tm_forward_ex(c, A, A, A, A, G, G, G, A, 1, 1, 17, T.TM_F32, T.TM_READ_PER_TOKEN, A, st) == \
        T.TM_ERR_SHAPE
    assert L.tm_forward_ex(c, A, None, None, None, None, None, None, None, 1, 1, 0, T.TM_BF16,
                           T.TM_READ_BEFORE_WRITE, A, st) == T.TM_OK
    # the input side: sizes, dtype, alignment, all on the host
    P = L.tm_project
    assert P(c, A, 64, A, G, 4, G, G, G, A, A, A, G, G, G, 1, 1, 16, 7, st) == T.TM_ERR_DTYPE
    assert P(c, A, 48, A, G, 4, G, G, G, A, A, A, G, G, G, 1, 1, 16, T.TM_BF16, st) == T.TM_ERR_INVALID
    assert P(c, A, 64, A, G, 5, G, G, G, A, A, A, G, G, G, 1, 1, 16, T.TM_BF16, st) == T.TM_ERR_INVALID
    assert P(c, A, 64, A, G, 0, G, G, G, A, A, A, G, G, G, 1, 1, 16, T.TM_BF16, st) == T.TM_ERR_INVALID
    assert P(c, A, 64, A, G, 4, G, G, None, A, A, A, G, G, G, 1, 1, 16, T.TM_BF16, st) == T.TM_ERR_INVALID
    assert P(c, ctypes.c_void_p((1 << 20) + 2), 64, A, G, 4, G, G, G, A, A, A, G, G, G, 1, 1, 16, T.TM_BF16,
             st) == T.TM_ERR_INVALID
    assert P(c, A, 64, A, G, 4, G, G, G, None, A, A, G, G, G, 1, 1, 16, T.TM_BF16, st) == T.TM_ERR_INVALID
    assert P(c, A, 64, A, G, 4, G, G, G, A, A, A, G, G, G, 0, 1, 16, T.TM_BF16, st) == T.TM_ERR_INVALID
    # empty: a no-op (outputs and, for one tap, the history may be null)
    assert P(c, A, 64, A, G, 1, G, G, None, None, None, None, None, None, None, 1, 1, 0, T.TM_BF16, st) == T.TM_OK
    # the memory-as-context wiring: sizes, dtype, alignment, all on the host
    W, G = L.tm_mac_window, L.tm_mac_gate
    assert W(A, 2, A, A, A, 1, 4, 64, 7, st) == T.TM_ERR_DTYPE
    assert W(A, 2, A, A, A, 1, 4, 48, T.TM_BF16, st) == T.TM_ERR_INVALID
    assert W(A, -1, A, A, A, 1, 4, 64, T.TM_BF16, st) == T.TM_ERR_INVALID
    assert W(None, 2, A, A, A, 1, 4, 64, T.TM_BF16, st) == T.TM_ERR_INVALID
    assert W(A, 2, A, A, A, 1, 0, 64, T.TM_BF16, st) == T.TM_ERR_INVALID
    assert W(A, 2, ctypes.c_void_p((1 << 20) + 4), A, A, 1, 4, 64, T.TM_BF16, st) == T.TM_ERR_INVALID
    assert G(A, A, A, 1, 4, 64, 7, st) == T.TM_ERR_DTYPE
    assert G(A, A, None, 1, 4, 64, T.TM_F32, st) == T.TM_ERR_INVALID
    assert G(A, A, A, 0, 4, 64, T.TM_F32, st) == T.TM_ERR_INVALID
    assert L.tm_status_str(T.TM_ERR_SHAPE).decode().startswith("n_tokens")
    # every argument valid, but the state was never set up by tm_state_init /
    # tm_state_import: refused before any launch
    assert L.tm_store(c, A, A, A, G, G, G, 1, 1, 16, T.TM_BF16, A, st) == T.TM_ERR_STATE
    assert L.tm_forward(c, A, A, A, A, G, G, G, A, 1, 1, 16, T.TM_F32, A, st) == T.TM_ERR_STATE
    assert L.tm_forward_ex(c, A, A, A, A, G, G, G, A, 1, 1, 16, T.TM_BF16, T.TM_READ_PER_TOKEN, A, st) == \
        T.TM_ERR_STATE
    assert L.tm_retrieve(c, A, A, A, 1, 1, 5, T.TM_BF16, A, st) == T.TM_ERR_STATE
    assert L.tm_state_export(c, A, 1, 1, A, st) == T.TM_ERR_STATE
    T.tm_destroy(c)


def test_config_getter():
    c = T.tm_create(128, 3, 2, 32)
    assert T.tm_config(c) == (128, 3, 2, 32)
    c1 = T.tm_create(64, 1, 7, 16)
    assert T.tm_config(c1) == (64, 1, 1, 16)
    assert T.lib().tm_config(None, None, None, None, None) == T.TM_ERR_INVALID
    T.tm_destroy(c)
    T.tm_destroy(c1)


def test_binding_checks_dtypes_and_shapes():
    """The binding refuses tensors of the wrong element type or shape before
    it passes any pointer on (the C calls take untyped pointers)."""
    import torch
    import test_trained_neural_amd as T
    bf, f32, f64 = torch.bfloat16, torch.float32, torch.float64
    B, S, D, P = 2, 4, 32, 1
    seg = torch.zeros((B, S, D), dtype=bf)
    with pytest.raises(TypeError, match="recalled"):
        T.tm_mac_window(torch.zeros((P, D), dtype=bf), torch.zeros((B, S, D), dtype=f64), seg,
                        torch.zeros((B, P + 2 * S, D), dtype=bf))
    with pytest.raises(TypeError, match="window"):
        T.tm_mac_window(None, torch.zeros((B, S, D)), seg, torch.zeros((B, 2 * S, D), dtype=f32))
    with pytest.raises(ValueError, match="window"):
        T.tm_mac_window(None, torch.zeros((B, S, D)), seg, torch.zeros((B, 2 * S + 1, D), dtype=bf))
    with pytest.raises(TypeError, match="mem"):
        T.tm_mac_gate(seg, torch.zeros((B, S, D), dtype=bf), torch.zeros((B, S, D)))
    with pytest.raises(ValueError, match="out"):
        T.tm_mac_gate(seg, torch.zeros((B, S, D)), torch.zeros((B, S, D + 1)))
    k = torch.zeros((1, 8, 2, 32), dtype=bf)
    g = torch.zeros((1, 8, 2))
    y = torch.zeros((1, 8, 2, 32))
    with pytest.raises(TypeError, match="theta"):
        T.tm_forward(None, None, k, k, k, g.double(), g, g, y, None)
    with pytest.raises(TypeError, match="q"):
        T.tm_forward(None, None, k, k, k.float(), g, g, g, y, None)
    with pytest.raises(TypeError, match="y"):
        T.tm_retrieve(None, None, k, y.to(bf), None)
    with pytest.raises(ValueError, match="alpha"):
        T.tm_store(None, None, k, k, g, g, g[:, :4], None)
    with pytest.raises(TypeError, match="bfloat16 or float32"):
        T.tm_store(None, None, k.half(), k.half(), g, g, g, None)
    with pytest.raises(TypeError, match="init_weights"):
        T.tm_state_init(None, None, 1, 2, torch.zeros((2, 10), dtype=f64))


def test_backward_validation_before_launch():
    L = T.lib()
    c = T.tm_create(64, 2, 2, 16)
    A = ctypes.c_void_p(1 << 20)
    G = ctypes.c_void_p((1 << 20) + 4096)
    st = ctypes.c_void_p(None)
    args = lambda n, read, dstate=A: (c, A, A, A, A, G, G, G, A, dstate, A, A, A, G, G, G, 1, 1, n, T.TM_F32, read,
                                      A, st)
    assert L.tm_backward(*args(16, T.TM_READ_PER_TOKEN)) == T.TM_ERR_INVALID
    assert L.tm_backward(*args(16, 5)) == T.TM_ERR_INVALID
    assert L.tm_backward(*args(16, T.TM_READ_AFTER_WRITE, None)) == T.TM_ERR_INVALID
    assert L.tm_backward(*args(17, T.TM_READ_AFTER_WRITE)) == T.TM_ERR_SHAPE
    assert L.tm_backward(*args(16, T.TM_READ_BEFORE_WRITE)) == T.TM_ERR_STATE   # never set up
    assert L.tm_backward(*args(0, T.TM_READ_AFTER_WRITE)) == T.TM_OK             # the identity
    assert T.tm_backward_workspace_bytes(c, 2, 1, 64) > T.tm_backward_workspace_bytes(c, 2, 1, 32) > 0
    T.tm_destroy(c)
