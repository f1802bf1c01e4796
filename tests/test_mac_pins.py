"""Pins for the memory-as-context wiring oracle (oracle/mac.py): the window's
row order and the gate by hand, and bfloat16 rounding against torch's own
conversion.

Source: "Titans, explained" step 8; "Attack of the Titans", Technical
Details, memory as a context."""
import numpy as np
import torch

from oracle import mac


def test_window_rows_in_order():
    P, B, S, D = 2, 2, 3, 4
    pers = np.arange(P * D, dtype=np.float64).reshape(P, D) + 100
    rec = np.arange(B * S * D, dtype=np.float64).reshape(B, S, D) + 200
    seg = np.arange(B * S * D, dtype=np.float64).reshape(B, S, D) + 300
    w = mac.window(pers, rec, seg, bf16=False)
    assert w.shape == (B, P + 2 * S, D)
    for b in range(B):
        for r in range(P):
            assert np.array_equal(w[b, r], pers[r])
        for r in range(S):
            assert np.array_equal(w[b, P + r], rec[b, r])
            assert np.array_equal(w[b, P + S + r], seg[b, r])
    # no persistent tokens
    assert np.array_equal(mac.window(None, rec, seg, False), np.concatenate([rec, seg], axis=1))


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(4096) * 10.0 ** rng.integers(-8, 8, 4096)).astype(np.float32)
    x[:4] = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -9, -0.0, np.inf]   # ties and specials
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(mac.round_to_bf16(x), want)


def test_gate_by_hand():
    y = np.array([[[1.0, -2.0, 0.5, 0.0]]])
    m = np.array([[[3.0, 0.25, -4.0, 7.0]]])
    assert np.array_equal(mac.gate(y, m), np.array([[[3.0, -0.5, -2.0, 0.0]]]))
