"""fp64 CPU oracle of the memory-side wiring of memory as a context (MAC).

TEST INFRASTRUCTURE ONLY: imported by the tests, never by the product
library.  It shares no code with the HIP path.

What it computes ("Titans, explained", step 8; "Attack of the Titans",
Technical Details, memory as a context), per segment of S tokens:
  1. the segment's queries read the memory as the previous segments left it;
  2. the attention window is [persistent tokens; the recalled vectors; the
     segment], in that order (the extended input is the concatenation of the
     persistent memory, the contextual memory's lookup results and x);
  3. attention runs over the window (the caller's; any function here);
  4. its output y for the segment's positions is written into the memory;
  5. the final output is y gated by the memory's read of y, taken here as the
     element-wise product y * M(y): the pages fix no form for the gate, and
     the product is the plainest reading.
The window's recalled rows carry the dtype of the segment: for bfloat16 they
are rounded to nearest even, as the memory's inputs are.
"""
from __future__ import annotations

import numpy as np


def round_to_bf16(a):
    """float32 -> the nearest bfloat16 value (ties to even), as float64."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    keep = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    out = keep.astype(np.uint32).view(np.float32)
    out = np.where(np.isnan(a), a, out)
    return out.astype(np.float64)


def window(persistent, recalled, segment, bf16):
    """persistent [P][D] (or None), recalled [B][S][D], segment [B][S][D] ->
    [B][P+2S][D]."""
    recalled = np.asarray(recalled, np.float64)
    segment = np.asarray(segment, np.float64)
    B, S, D = segment.shape
    if bf16:
        recalled = round_to_bf16(recalled)
    parts = []
    if persistent is not None and len(persistent):
        parts.append(np.broadcast_to(np.asarray(persistent, np.float64)[None], (B,) + np.shape(persistent)))
    parts += [recalled, segment]
    return np.concatenate(parts, axis=1)


def gate(y, mem):
    """The final output: y * M(y), element-wise."""
    return np.asarray(y, np.float64) * np.asarray(mem, np.float64)
