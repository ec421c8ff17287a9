"""Oracle for the int4 path: quantise, pack, interleave, GEMV and GEMM.

TEST INFRASTRUCTURE (see ``oracle/__init__``): slow, plain and obviously
correct; never imported by the product path.

Definitions followed (short page names are listed in ``oracle/__init__``):

* Codes and dequantisation.  A weight is an unsigned 4-bit code q in 0..15;
  its value is (q - zero) * scale, with the code read as unsigned so no sign
  bit interferes (Vulkan post, section 2 core GLSL shader and section 3 key
  points).
* Packing.  Two codes share one byte along K: the even k in the low nibble,
  the odd k in the high nibble (Paddle PR, "int4量化kernel"; Helion issue,
  the low/high nibble split of ``matmul_bf16_int4``).  Read as a
  little-endian 32-bit word, eight consecutive k sit with element 0 in the
  lowest nibble (Vulkan post, section 1 packing strategy).
* Interleave.  The Paddle PR ("int4 permute kernel") stores the eight nibbles
  of a word in the order 0 2 4 6 1 3 5 7 so that a register trick can unpack
  them into elements 0..7.  The gfx950 layout of this library uses that same
  within-word order; nothing else moves.
* GEMV / GEMM.  d[c, r] = sum_k W[r, k] * x[c, k] (Ternary post, section 3
  MMVQ, the batched form with x indexed [c][k]); the GEMM is the same sum
  with A's rows as the columns c (Helion issue, ``matmul_bf16_int4``).

The quantiser formula is not on the pages.  Reading adopted (parity
unpinned -- only invariants and a hand-worked case pin it): symmetric,
zero = 8, scale = absmax / 7 computed in float32 and rounded to the scale's
storage dtype before use, code = clamp(rint(w / scale), -8, 7) + 8 with a
float32 IEEE divide and ties-to-even; an all-zero group stores scale 0 and
codes 8.
"""
from __future__ import annotations

import numpy as np

from . import fpformat

LAYOUT_PLAIN = 0
LAYOUT_GFX950 = 1

# Within each 32-bit word of eight consecutive k: nibble position p holds
# element GFX950_ORDER[p] of that word (the fast-dequant order of the Paddle
# PR's permute section).
GFX950_ORDER = (0, 2, 4, 6, 1, 3, 5, 7)


# --------------------------------------------------------------------------
# quantise
# --------------------------------------------------------------------------
def quantize_int4(w_f16_bits: np.ndarray, group: int, scale_dtype: str):
    """fp16 weights [N][K] -> (codes uint8 [N][K], scales float32 [N][K/group],
    scale bits).  ``scale_dtype`` is "f32" or "bf16"; for "bf16" the returned
    bits are the uint16 patterns, for "f32" the uint32 patterns.

    Reading of the unstated formula (parity unpinned): see module docstring.
    """
    w = fpformat.f16_bits_to_f32(w_f16_bits)
    n, k = w.shape
    assert k % group == 0
    ng = k // group
    codes = np.empty((n, k), dtype=np.uint8)
    scales = np.empty((n, ng), dtype=np.float32)
    bits = np.empty((n, ng), dtype=np.uint16 if scale_dtype == "bf16" else np.uint32)
    seven = np.float32(7.0)
    for g in range(ng):
        blk = w[:, g * group:(g + 1) * group]
        absmax = np.max(np.abs(blk), axis=1)                 # exact
        s32 = (absmax / seven).astype(np.float32)            # fp32 IEEE divide
        if scale_dtype == "bf16":
            b = fpformat.f32_to_bf16_bits(s32)
            s = fpformat.bf16_bits_to_f32(b)
        elif scale_dtype == "f32":
            s = s32
            b = s32.view(np.uint32)
        else:
            raise ValueError(scale_dtype)
        scales[:, g] = s
        bits[:, g] = b
        zero = s == 0.0
        safe = np.where(zero, np.float32(1.0), s)
        quot = (blk / safe[:, None]).astype(np.float32)      # fp32 IEEE divide
        q = np.clip(np.rint(quot), -8, 7).astype(np.int32) + 8
        q[zero, :] = 8                                       # all-zero group
        codes[:, g * group:(g + 1) * group] = q.astype(np.uint8)
    return codes, scales, bits


# --------------------------------------------------------------------------
# pack / unpack / interleave
# --------------------------------------------------------------------------
def pack_plain(codes: np.ndarray) -> np.ndarray:
    """codes [N][K] (0..15) -> bytes [N][K/2]; byte i = q[2i] | q[2i+1] << 4."""
    codes = np.asarray(codes, dtype=np.uint8)
    assert codes.shape[-1] % 2 == 0 and int(codes.max(initial=0)) < 16
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack_plain(packed: np.ndarray) -> np.ndarray:
    """Inverse of ``pack_plain``: bytes [N][K/2] -> codes [N][K]."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out


def permute_groups(seq: np.ndarray, order) -> np.ndarray:
    """Gather within consecutive groups of len(order) along the last axis:
    out[..., G*i + p] = seq[..., G*i + order[p]]."""
    seq = np.asarray(seq)
    g = len(order)
    assert seq.shape[-1] % g == 0
    v = seq.reshape(seq.shape[:-1] + (seq.shape[-1] // g, g))
    return v[..., list(order)].reshape(seq.shape)


def inverse_order(order):
    inv = [0] * len(order)
    for p, e in enumerate(order):
        inv[e] = p
    return tuple(inv)


def pack(codes: np.ndarray, layout: int) -> np.ndarray:
    """codes [N][K] -> packed bytes [N][K/2] in the given layout.

    Plain: nibble sequence index == k.  gfx950: within each group of eight
    nibbles (one little-endian word), nibble p holds element GFX950_ORDER[p].
    """
    if layout == LAYOUT_PLAIN:
        return pack_plain(codes)
    if layout == LAYOUT_GFX950:
        assert codes.shape[-1] % 8 == 0
        return pack_plain(permute_groups(codes, GFX950_ORDER))
    raise ValueError(layout)


def unpack(packed: np.ndarray, layout: int) -> np.ndarray:
    """packed bytes [N][K/2] in ``layout`` -> codes [N][K] in k order."""
    seq = unpack_plain(packed)
    if layout == LAYOUT_PLAIN:
        return seq
    if layout == LAYOUT_GFX950:
        return permute_groups(seq, inverse_order(GFX950_ORDER))
    raise ValueError(layout)


# --------------------------------------------------------------------------
# dequantise, GEMV, GEMM
# --------------------------------------------------------------------------
def dequantize(codes: np.ndarray, scales: np.ndarray, zeros, zero_const: float,
               group: int) -> np.ndarray:
    """W[r, k] = (q[r, k] - zero[r, k // group]) * scale[r, k // group] in fp64."""
    codes = np.asarray(codes)
    n, k = codes.shape
    s = np.repeat(np.asarray(scales, dtype=np.float64).reshape(n, k // group), group, axis=1)
    if zeros is None:
        z = np.float64(zero_const)
    else:
        z = np.repeat(np.asarray(zeros, dtype=np.float64).reshape(n, k // group), group, axis=1)
    return (codes.astype(np.float64) - z) * s


def gemv_w4(packed: np.ndarray, layout: int, scales: np.ndarray, zeros,
            zero_const: float, group: int, x: np.ndarray) -> np.ndarray:
    """d[c, r] = sum_k (q[r,k] - z) * s * x[c, k] in fp64; returns [c][N]."""
    codes = unpack(packed, layout)
    w = dequantize(codes, scales, zeros, zero_const, group)
    xx = np.asarray(x, dtype=np.float64)
    return xx @ w.T


def gemm_w4a16_rows(a_rows: np.ndarray, packed: np.ndarray, layout: int,
                    scales: np.ndarray, zero_const: float, group: int,
                    zeros=None) -> np.ndarray:
    """Selected rows of C = A * dequant(B)^T in fp64: C[m, n] = sum_k A[m, k] *
    (q[n, k] - z) * s[n, k // group], z the stored zero of the group when
    ``zeros`` is given, else ``zero_const``.  B is stored output-major
    [N][K/2]."""
    codes = unpack(packed, layout)
    w = dequantize(codes, scales, zeros, zero_const, group)
    return np.asarray(a_rows, dtype=np.float64) @ w.T


def gemm_w4a16_rows_bf16w(a_rows: np.ndarray, packed: np.ndarray, layout: int,
                          scales: np.ndarray, zero_const: float, group: int,
                          zeros=None) -> np.ndarray:
    """Selected rows of C = A * W^T in fp64 where every weight is first
    rounded to bf16: W[n, k] = bf16_rne((q[n, k] - z) * s[n, k // group]).

    This is the matrix-core path with group scales: the bf16 multiply takes
    bf16 operands (Helion issue, ``matmul_bf16_int4``: B is converted to
    bf16 before the dot), so a group scale that varies along K is applied to
    the weight before the multiply, and the weight is rounded once.  (q - z)
    * s is exact in float32 for bf16 s and an integer or bf16 z (at most
    about 17 significant bits), so the rounding here is the one bf16 rounding
    of the exact product.  ``zeros``: stored zeros per group (Vulkan post,
    section 2: (q - zero) * scale), else ``zero_const``."""
    codes = unpack(packed, layout)
    w = dequantize(codes, scales, zeros, zero_const, group)
    w16 = fpformat.bf16_bits_to_f32(fpformat.f32_to_bf16_bits(w.astype(np.float32)))
    return np.asarray(a_rows, dtype=np.float64) @ w16.astype(np.float64).T
