"""Oracle for the ternary path: PTQ1_0 blocks, q8_1 activation blocks, GEMV.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

Formats, from the Ternary post (short page names in ``oracle/__init__``):

* PTQ1_0 block (section 2): 128 trits in 28 bytes -- ``qs[24]`` holding 120
  trits five to a byte, ``qh[2]`` holding the last 8 trits at 2 bits each,
  and an fp16 scale ``d``.  Byte order in memory: qs, qh, d (little endian).
* Trit placement (section 3.2): for element e < 80 the trit sits in qs byte
  e & 15 at digit e >> 4 (so byte 0 holds elements 0, 16, 32, 48, 64); for
  element 80 + e (e < 40) in qs byte 16 + (e & 7) at digit e >> 3; the last
  eight are the 2-bit qh trits.
* block_q8_1 (section 3.1): fp16 d, fp16 s = d * sum(qs), int8 qs[32];
  36 bytes, d then s then qs.
* GEMV (section 3): d[r, c] = sum_k W[r, k] x[c, k].

Readings where the post is silent or garbled (parity unpinned for the first
two; they are pinned by round trips and by the post's byte-0 example only):
  R-digit  A trit t is stored as the digit u = t + 1 in {0, 1, 2}; a qs byte
           is sum_j u_j * 3**j with digit 0 least significant (max 242).
  R-qh     Tail element 120 + e lives in qh[e & 1] at bits 2*(e >> 1) .. +1
           as the 2-bit value u -- the same "byte = e mod bytes, slot =
           e div bytes" stride the two qs sections use.
  R-q8     The post says "d is an integer", but declares d as fp16; read: qs
           are the integers, d and s are fp16.  Quantiser: amax over the 32
           floats; d = fp16(amax / 127) (float32 divide, then RNE to fp16);
           q = clamp(rint(x / float(d)), -127, 127) with a float32 divide;
           s = fp16(float32(float(d) * sum(q))); amax == 0 gives d = 0, q = 0.
  R-sum    The product is computed from the exact integer sub-block sums
           S[r, c, b] = sum_i t * q over each block of 32 (s is stored for
           fidelity; the exact path never uses it):
           y[c, r] = sum_b d_w[r, b // 4] * d_x[c, b] * S[r, c, b].
"""
from __future__ import annotations

import numpy as np

from . import fpformat

QK = 128          # trits per PTQ1_0 block
BLOCK_BYTES = 28  # 24 qs + 2 qh + 2 d
Q8_QK = 32        # values per q8_1 block
Q8_BYTES = 36     # 2 d + 2 s + 32 qs


def trit_position(e: int):
    """Where element e (0..127) of a PTQ1_0 block lives.

    Returns ("qs", byte, digit) or ("qh", byte, bit_offset)."""
    if e < 80:
        return "qs", e & 15, e >> 4
    if e < 120:
        f = e - 80
        return "qs", 16 + (f & 7), f >> 3
    f = e - 120
    return "qh", 24 + (f & 1), 2 * (f >> 1)


def encode_ptq1_0(trits: np.ndarray, d_bits: np.ndarray) -> np.ndarray:
    """trits int8 [N][K] in {-1,0,1}, d fp16 bits [N][K/128] -> uint8
    [N][K/128][28]."""
    trits = np.asarray(trits, dtype=np.int64)
    n, k = trits.shape
    assert k % QK == 0
    nb = k // QK
    u = (trits + 1).reshape(n, nb, QK)
    assert u.min(initial=0) >= 0 and u.max(initial=0) <= 2
    out = np.zeros((n, nb, BLOCK_BYTES), dtype=np.int64)
    for e in range(QK):
        kind, byte, pos = trit_position(e)
        if kind == "qs":
            out[:, :, byte] += u[:, :, e] * (3 ** pos)
        else:
            out[:, :, byte] |= u[:, :, e] << pos
    d = np.asarray(d_bits, dtype=np.uint16).reshape(n, nb)
    out[:, :, 26] = d & 0xFF
    out[:, :, 27] = d >> 8
    assert out[:, :, :24].max(initial=0) <= 242
    return out.astype(np.uint8)


def decode_ptq1_0(blocks: np.ndarray):
    """uint8 [N][NB][28] -> (trits int8 [N][NB*128], d fp16 bits [N][NB])."""
    b = np.asarray(blocks, dtype=np.int64)
    n, nb, _ = b.shape
    t = np.empty((n, nb, QK), dtype=np.int64)
    for e in range(QK):
        kind, byte, pos = trit_position(e)
        if kind == "qs":
            u = (b[:, :, byte] // (3 ** pos)) % 3
        else:
            u = (b[:, :, byte] >> pos) & 3
        t[:, :, e] = u - 1
    d = (b[:, :, 26] | (b[:, :, 27] << 8)).astype(np.uint16)
    return t.reshape(n, nb * QK).astype(np.int8), d


def quantize_q8_1(x: np.ndarray) -> np.ndarray:
    """float32 x [c][K] -> block_q8_1 bytes [c][K/32][36] (reading R-q8)."""
    x = np.asarray(x, dtype=np.float32)
    c, k = x.shape
    assert k % Q8_QK == 0
    nb = k // Q8_QK
    xb = x.reshape(c, nb, Q8_QK)
    amax = np.max(np.abs(xb), axis=2)                                   # exact
    d16 = fpformat.f32_to_f16_bits((amax / np.float32(127.0)).astype(np.float32))
    d = fpformat.f16_bits_to_f32(d16)
    q = np.zeros((c, nb, Q8_QK), dtype=np.int64)
    nz = d != 0
    quot = (xb / np.where(nz, d, np.float32(1.0))[:, :, None]).astype(np.float32)
    q[nz] = np.clip(np.rint(quot[nz]), -127, 127).astype(np.int64)
    qsum = q.sum(axis=2)
    s16 = fpformat.f32_to_f16_bits((d * qsum.astype(np.float32)).astype(np.float32))
    out = np.zeros((c, nb, Q8_BYTES), dtype=np.uint8)
    out[:, :, 0] = d16 & 0xFF
    out[:, :, 1] = d16 >> 8
    out[:, :, 2] = s16 & 0xFF
    out[:, :, 3] = s16 >> 8
    out[:, :, 4:] = q.astype(np.int8).view(np.uint8)
    return out


def decode_q8_1(blocks: np.ndarray):
    """uint8 [c][NB][36] -> (q int8 [c][NB*32], d bits [c][NB], s bits [c][NB])."""
    b = np.asarray(blocks, dtype=np.uint8)
    c, nb, _ = b.shape
    d = (b[:, :, 0].astype(np.uint16) | (b[:, :, 1].astype(np.uint16) << 8))
    s = (b[:, :, 2].astype(np.uint16) | (b[:, :, 3].astype(np.uint16) << 8))
    q = b[:, :, 4:].copy().view(np.int8).reshape(c, nb * Q8_QK)
    return q, d, s


def subblock_sums(trits: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Exact S[r, c, b] = sum_{i<32} t[r, 32b+i] * q[c, 32b+i] (int64)."""
    t = np.asarray(trits, dtype=np.int64)
    qq = np.asarray(q, dtype=np.int64)
    n, k = t.shape
    c = qq.shape[0]
    nb = k // Q8_QK
    t3 = t.reshape(n, nb, Q8_QK)
    q3 = qq.reshape(c, nb, Q8_QK)
    out = np.empty((n, c, nb), dtype=np.int64)
    for j in range(c):
        out[:, j, :] = np.einsum("rbi,bi->rb", t3, q3[j])
    return out


def gemv_ternary(w_blocks: np.ndarray, x_blocks: np.ndarray) -> np.ndarray:
    """y[c, r] = sum_b d_w[r, b // 4] * d_x[c, b] * S[r, c, b] in fp64.

    w_blocks uint8 [N][K/128][28]; x_blocks uint8 [c][K/32][36]."""
    trits, dw_bits = decode_ptq1_0(w_blocks)
    q, dx_bits, _ = decode_q8_1(x_blocks)
    S = subblock_sums(trits, q).astype(np.float64)                  # [N][c][K/32]
    dw = fpformat.f16_bits_to_f32(dw_bits).astype(np.float64)       # [N][K/128]
    dx = fpformat.f16_bits_to_f32(dx_bits).astype(np.float64)       # [c][K/32]
    dw32 = np.repeat(dw, QK // Q8_QK, axis=1)                       # [N][K/32]
    y = np.einsum("rcb,rb,cb->cr", S, dw32, dx)
    return y
