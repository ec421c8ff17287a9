"""Storage formats of the oracle: bf16 and fp16 rounding, written out.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

bf16 is the top half of an IEEE float32; rounding float32 to bf16 is
round-to-nearest, ties-to-even on the 16 dropped bits.  fp16 is IEEE
binary16; numpy's float32 -> float16 cast rounds to nearest even directly from
float32, which is the reading used by both quantisers (one rounding, no
intermediate float64).
"""
from __future__ import annotations

import numpy as np


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16, nearest-even; returns uint16 patterns.

    Finite inputs only (the quantisers never see NaN/Inf by contract)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_f16_bits(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(b) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)
