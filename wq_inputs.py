"""Seeded synthetic inputs for the weight-quantised GEMV/GEMM path.

This module is the only code shared by the CPU oracle (``oracle/``) and the
HIP path (``gemm_wq_quantize_amd``).  It draws raw values only: integer codes,
trits, scales, activations.  It holds none of the method's arithmetic: no
packing, no quantisation, no block encoding, no dot products.  Each side turns
these raw values into its own packed bytes.

Every array is drawn from ``numpy.random.default_rng(seed)`` (a fresh
generator per workload, seed 0 unless stated) in the order written in each
function.  Half-precision values are the round-to-nearest-even rounding of the
float32 draws, done with torch's CPU casts (input preparation only).

Workload shapes follow the pages:
  * the Vulkan int4 GEMV post (section 2, the GLSL shader): per-row fp32 scale
    and zero point, fp32 activations;
  * the ternary-compression post (section 3, MMVQ): Qwen layer widths
    K in {5120, 17280} and a batch of a few activation columns;
  * the Helion int4 GEMM issue (the example's test): A 8192 x 8192 bf16 and a
    B of 8192 x 8192 int4 codes.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = [
    "to_bf16_bits", "to_f16_bits", "bf16_bits_to_f32", "f16_bits_to_f32",
    "tiny_int4", "decode_int4", "small_batch_int4", "large_gemm", "grouped_gemm",
    "ternary_gemv", "ternary_correlated_scales", "DECODE_SHAPES", "SMALL_BATCH_SHAPES",
]

# (K, N) pairs: the two projections of one transformer layer at these widths.
DECODE_SHAPES = ((5120, 17280), (17280, 5120))
SMALL_BATCH_SHAPES = ((4096, 11008), (11008, 4096))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 draws -> bf16 bit patterns (uint16), RNE via torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_f16_bits(a: np.ndarray) -> np.ndarray:
    """float32 draws -> fp16 bit patterns (uint16), RNE."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


@dataclass
class Int4Problem:
    """Raw int4 GEMV/GEMM operands.

    codes   uint8 [N][K], values 0..15 (one code per byte, logical layout)
    scales  float32 [N][K/group] holding exactly representable values of
            ``scale_dtype`` ("f32" or "bf16"); ``scale_bits`` has the uint16
            bf16 patterns when scale_dtype == "bf16"
    zeros   float32 [N][K/group] or None (then ``zero_const`` applies)
    x       float32 [c][K] (exact values of ``x_dtype``); ``x_bits`` has the
            bf16 patterns when x_dtype == "bf16"
    w_f16   optional fp16 weights (uint16 bits) [N][K] for the quantiser
    """
    n: int
    k: int
    group: int
    codes: np.ndarray | None
    scales: np.ndarray | None
    scale_dtype: str
    zeros: np.ndarray | None
    zero_const: float
    x: np.ndarray
    x_dtype: str
    x_bits: np.ndarray | None = None
    scale_bits: np.ndarray | None = None
    w_f16: np.ndarray | None = None
    extra: dict = field(default_factory=dict)


def tiny_int4(seed: int = 0) -> Int4Problem:
    """256 x 512 int4 GEMV, per-row fp32 scale U(0.005,0.02) and zero U(6,9),
    fp32 x ~ N(0,1), one column.  Then, from the same generator, fp16 weights
    N(0, 0.02) for the quantise + pack round trip."""
    rng = np.random.default_rng(seed)
    n, k = 256, 512
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    scales = rng.uniform(0.005, 0.02, n).astype(np.float32).reshape(n, 1)
    zeros = rng.uniform(6.0, 9.0, n).astype(np.float32).reshape(n, 1)
    x = rng.standard_normal((1, k)).astype(np.float32)
    w_f16 = to_f16_bits(0.02 * rng.standard_normal((n, k)))
    return Int4Problem(n, k, k, codes, scales, "f32", zeros, 8.0, x, "f32",
                       w_f16=w_f16)


def decode_int4(k: int, n: int, cmax: int = 4, seed: int = 0) -> Int4Problem:
    """Decode-shape W4A16 GEMV: codes U{0..15}, group 128, bf16 scales
    U(0.002, 0.02), zero 8, bf16 x ~ N(0,1) with ``cmax`` columns (a batch of
    c <= cmax uses the first c columns)."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    sbits = to_bf16_bits(rng.uniform(0.002, 0.02, (n, k // 128)))
    xbits = to_bf16_bits(rng.standard_normal((cmax, k)))
    return Int4Problem(n, k, 128, codes, bf16_bits_to_f32(sbits), "bf16", None, 8.0,
                       bf16_bits_to_f32(xbits), "bf16", x_bits=xbits, scale_bits=sbits)


def small_batch_int4(k: int, n: int, cmax: int = 32, seed: int = 0) -> Int4Problem:
    """Small-batch W4A16: fp16 weights N(0, 0.02) to be quantised (group 128,
    bf16 scales) by each side, bf16 x ~ N(0,1) with ``cmax`` columns."""
    rng = np.random.default_rng(seed)
    w_f16 = to_f16_bits(0.02 * rng.standard_normal((n, k)))
    xbits = to_bf16_bits(rng.standard_normal((cmax, k)))
    return Int4Problem(n, k, 128, None, None, "bf16", None, 8.0,
                       bf16_bits_to_f32(xbits), "bf16", x_bits=xbits, w_f16=w_f16)


@dataclass
class GemmProblem:
    m: int
    n: int
    k: int
    a_bits: np.ndarray      # bf16 patterns [M][K]
    codes: np.ndarray       # uint8 [N][K]: code of logical B[k][n] stored at [n][k]
    scale_bits: np.ndarray  # bf16 patterns [N] (one scale per output column)
    zero_const: float
    rows: np.ndarray        # sorted sample of output rows the oracle checks


def large_gemm(m: int = 8192, n: int = 8192, k: int = 8192, n_rows: int = 256,
               seed: int = 0) -> GemmProblem:
    """W4A16 GEMM: A bf16 ~ N(0,1); int4 codes U{0..15}; per-column bf16 scale
    0.01; zero 8; a sorted random sample of output rows."""
    rng = np.random.default_rng(seed)
    a_bits = to_bf16_bits(rng.standard_normal((m, k), dtype=np.float32))
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    scale_bits = to_bf16_bits(np.full(n, 0.01, dtype=np.float32))
    rows = np.sort(rng.choice(m, min(n_rows, m), replace=False))
    return GemmProblem(m, n, k, a_bits, codes, scale_bits, 8.0, rows)


def grouped_gemm(m: int, n: int, k: int, group: int = 128, seed: int = 0) -> GemmProblem:
    """W4A16 GEMM with group scales, shaped like the decode workload's weights:
    A bf16 ~ N(0,1); int4 codes U{0..15}; bf16 scales U(0.002, 0.02) per
    (column, group of ``group`` k) as [N][K/group]; zero 8; every row."""
    rng = np.random.default_rng(seed)
    a_bits = to_bf16_bits(rng.standard_normal((m, k), dtype=np.float32))
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    scale_bits = to_bf16_bits(rng.uniform(0.002, 0.02, (n, k // group)).astype(np.float32))
    return GemmProblem(m, n, k, a_bits, codes, scale_bits, 8.0, np.arange(m))


@dataclass
class TernaryProblem:
    n: int
    k: int
    trits: np.ndarray   # int8 [N][K], values -1, 0, 1
    d_bits: np.ndarray  # fp16 patterns [N][K/128], one scale per 128-trit block
    x: np.ndarray       # float32 [c][K] activations (quantised by each side)


def ternary_gemv(k: int = 5120, n: int = 17280, cmax: int = 8, seed: int = 0,
                 unit_scale: bool = False) -> TernaryProblem:
    """Ternary GEMV: trits U{-1,0,1}; fp16 block scale U(0.01, 0.05); fp32
    x ~ N(0,1).  ``unit_scale`` makes every block scale 1.0 and x integer in
    [-127, 127] with a +-127 in every block of 32, so the activation blocks
    quantise with scale exactly 1 and every output is an exact integer."""
    rng = np.random.default_rng(seed)
    trits = rng.integers(-1, 2, (n, k), dtype=np.int8)
    if unit_scale:
        d_bits = to_f16_bits(np.ones((n, k // 128), dtype=np.float32))
        xi = rng.integers(-127, 128, (cmax, k))
        xi = xi.reshape(cmax, k // 32, 32)
        xi[:, :, 0] = np.where(rng.integers(0, 2, (cmax, k // 32)) == 0, 127, -127)
        x = xi.reshape(cmax, k).astype(np.float32)
    else:
        d_bits = to_f16_bits(rng.uniform(0.01, 0.05, (n, k // 128)))
        x = rng.standard_normal((cmax, k)).astype(np.float32)
    return TernaryProblem(n, k, trits, d_bits, x)


def ternary_correlated_scales(k: int = 5120, n: int = 17280, cmax: int = 8, seed: int = 0,
                              p_change: float = 0.075) -> TernaryProblem:
    """Ternary GEMV whose block scales have the exponent statistics the
    ternary post reports for trained weights (section 2: the sign is always
    positive, the exponents of neighbouring blocks rarely differ, and eight
    consecutive blocks almost never leave a set of 768 exponent patterns).

    Draws: trits U{-1,0,1} [N][K]; per row a starting fp16 exponent field
    U{8, 9, 10} (scales in [2^-7, 2^-4), the range of the U(0.01, 0.05)
    scales of the plain ternary workload); along the row, each next block's
    exponent moves by -1 or +1 with probability p_change / 2 each (a running
    sum, clipped to [7, 11]); a 10-bit mantissa U{0..1023} per block; fp32
    x ~ N(0,1).  The fp16 scale bits are (exponent << 10) | mantissa.
    p_change = 0.075 leaves about 3 in 10^4 superblocks outside the 767 most
    common patterns at K=5120, N=17280 (the post: about 1 in 10^4)."""
    rng = np.random.default_rng(seed)
    trits = rng.integers(-1, 2, (n, k), dtype=np.int8)
    nb = k // 128
    e0 = rng.integers(8, 11, n)
    u = rng.random((n, max(nb - 1, 0)))
    step = np.where(u < p_change / 2, -1, np.where(u < p_change, 1, 0))
    e = np.concatenate([e0[:, None], e0[:, None] + np.cumsum(step, axis=1)], axis=1)
    e = np.clip(e, 7, 11)
    mant = rng.integers(0, 1024, (n, nb))
    d_bits = ((e << 10) | mant).astype(np.uint16)
    x = rng.standard_normal((cmax, k)).astype(np.float32)
    return TernaryProblem(n, k, trits, d_bits, x)
