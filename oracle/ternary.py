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

PT plane layout of the activations (section 3.1): the q8_1 data of one
column regrouped by 128-element block i (K/128 of them) into nine planes of
K/128 16-byte slots.  Element e (0..127) of block i sits at byte
16 (floor(e / 16) * K/128 + i) + e mod 16 -- plane floor(e / 16) -- and plane
8 holds the four (d, s) pairs of each block.  The post draws plane 8 only as
"all (d, s)" of the block; reading (parity unpinned beyond the sizes, the
plane picture and the round trip):
  R-pt     Slot i of plane 8 holds the (d, s) words of the block's four q8_1
           sub-blocks in order, each as in block_q8_1 (fp16 d, then fp16 s):
           sub-block j of block i at byte 16 (8 K/128 + i) + 4 j.  K must be a
           multiple of 128.  A batch of c columns is c consecutive PT arrays
           of 9 K / 8 bytes (the size of the column's q8_1 blocks).

PTQ1_1 superblock (section 2, struct ptq1_1; section 3.1, sb = kbx >> 3,
sub = kbx & 7): eight consecutive PTQ1_0 blocks of a row in 216 bytes --
qs[192], qh[13], eight 10-bit mantissas, one exponent byte.  The post fixes
the sizes and the idea (the sign of d is always +; the eight 5-bit exponents
become an index into 768 patterns made of the exponent byte and the free
trit of qh, 767 meaning "look the superblock up in an external table"),
not the bit positions.  Readings (parity unpinned beyond the round trips,
sizes and hand-worked bytes of the tests):
  R-sb     A row's K/128 blocks form K/1024 superblocks of 8 consecutive
           blocks (block kbx is sub-block kbx & 7 of superblock kbx >> 3);
           K must be a multiple of 1024.  Superblocks are [N][K/1024].
  R-sbqs   Bytes 0..191: the qs[24] of sub-blocks 0..7 in order, unchanged
           (section 3.1 reads qs of sub-block sub as a uint8_t[24] at sub).
  R-sbqh   Bytes 192..204 (qh[13]): the 64 tail trits (elements 120..127 of
           each sub-block, digit u = t + 1) in sub-block order, tail trit
           8 sub + e in byte (8 sub + e) // 5 at base-3 digit
           (8 sub + e) % 5, digit 0 least significant -- five to a byte as in
           qs; digit 4 of qh[12] is the free trit.
  R-sbm    Bytes 205..214: the ten bytes of an 80-bit little-endian field
           holding mantissa sub (the low 10 bits of d) at bits 10 sub.
  R-sbe    Byte 215 and the free trit: pattern index P = byte + 256 * free
           digit (0..767).  P < 767 selects row P of a 767 x 8 codebook of
           exponent fields; P = 767 means the superblock's 8 exponents come
           from the escape table (superblock indices row * K/1024 + sb in
           ascending order, with their 8 exponents).  d = (e << 10) | m.
  R-sbcb   Codebook (the encoder's choice; the post builds it from the
           statistics of trained weights): the exponent patterns of the
           tensor by decreasing count, ties by increasing pattern (e_0..e_7
           compared in order), the first min(767, #patterns) of them; unused
           rows are zero; every other superblock escapes.
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


# --------------------------------------------------------------------------
# PTQ1_1 superblocks
# --------------------------------------------------------------------------
SB_BLOCKS = 8        # PTQ1_0 blocks per superblock
SB_BYTES = 216       # 192 qs + 13 qh + 10 mantissa + 1 exponent byte
SB_QH = 192          # byte offset of qh[13]
SB_MANT = 205        # byte offset of the 80-bit mantissa field
SB_EXP = 215         # byte offset of the exponent (pattern) byte
CODEBOOK_ROWS = 767  # pattern indices 0..766; 767 is the escape
ESCAPE = 767


def tail_position(t: int):
    """Tail trit t (0..63, = 8 sub + e) of a superblock -> (qh byte, digit).
    Position 64 (byte 12, digit 4) is the free trit."""
    return t // 5, t % 5


def pattern_fields(p: int):
    """Pattern index (0..767) -> (exponent byte, free-trit digit)."""
    return p & 0xFF, p >> 8


def pattern_index(byte: int, digit: int) -> int:
    """(exponent byte, free-trit digit) -> pattern index; inverse of
    ``pattern_fields``."""
    return byte + 256 * digit


def mantissa_bytes(mant) -> np.ndarray:
    """Eight 10-bit mantissas -> the 10 bytes of the little-endian 80-bit
    field, mantissa sub at bit 10 sub."""
    field = 0
    for sub, m in enumerate(mant):
        field |= (int(m) & 0x3FF) << (10 * sub)
    return np.frombuffer(field.to_bytes(10, "little"), dtype=np.uint8).copy()


def mantissas(field_bytes) -> list:
    """Inverse of ``mantissa_bytes``."""
    field = int.from_bytes(bytes(np.asarray(field_bytes, dtype=np.uint8)), "little")
    return [(field >> (10 * sub)) & 0x3FF for sub in range(SB_BLOCKS)]


def superblock_index(row: int, sb: int, nsb: int) -> int:
    """Global index of superblock sb of a row (the key of the escape table)."""
    return row * nsb + sb


def exponent_patterns(d_bits: np.ndarray) -> np.ndarray:
    """fp16 scale bits [N][K/128] -> exponent fields [N][K/1024][8].  The sign
    must be 0 (the post drops it: d is always positive)."""
    d = np.asarray(d_bits, dtype=np.uint16)
    n, nb = d.shape
    assert nb % SB_BLOCKS == 0, "K must be a multiple of 1024"
    assert not np.any(d >> 15), "PTQ1_1 stores no sign: every d must be >= +0"
    return ((d >> 10) & 0x1F).astype(np.int64).reshape(n, nb // SB_BLOCKS, SB_BLOCKS)


def codebook_order(counts: dict) -> list:
    """Reading R-sbcb: patterns by decreasing count, ties by increasing
    pattern."""
    return [pat for pat, _ in sorted(counts.items(), key=lambda kv: (-kv[1], kv[0]))]


def build_codebook(patterns: np.ndarray):
    """The 767 first patterns of ``codebook_order``.  Returns (codebook uint8
    [767][8], {pattern: row})."""
    counts = {}
    for row in np.asarray(patterns).reshape(-1, SB_BLOCKS):
        pat = tuple(int(v) for v in row)
        counts[pat] = counts.get(pat, 0) + 1
    book = np.zeros((CODEBOOK_ROWS, SB_BLOCKS), dtype=np.uint8)
    index = {}
    for row, pat in enumerate(codebook_order(counts)[:CODEBOOK_ROWS]):
        book[row] = pat
        index[pat] = row
    return book, index


def encode_ptq1_1(blocks: np.ndarray):
    """PTQ1_0 blocks uint8 [N][K/128][28] -> (superblocks uint8
    [N][K/1024][216], codebook uint8 [767][8], escape indices int64 [n_esc],
    escape patterns uint8 [n_esc][8])."""
    b = np.asarray(blocks, dtype=np.uint8)
    n, nb, _ = b.shape
    assert nb % SB_BLOCKS == 0, "K must be a multiple of 1024"
    nsb = nb // SB_BLOCKS
    d = (b[:, :, 26].astype(np.int64) | (b[:, :, 27].astype(np.int64) << 8))
    pats = exponent_patterns(d.astype(np.uint16))
    book, index = build_codebook(pats)
    out = np.zeros((n, nsb, SB_BYTES), dtype=np.uint8)
    esc = []
    for r in range(n):
        for sb in range(nsb):
            blk = b[r, sb * SB_BLOCKS:(sb + 1) * SB_BLOCKS]
            dd = d[r, sb * SB_BLOCKS:(sb + 1) * SB_BLOCKS]
            sup = out[r, sb]
            # qs: the eight qs[24] arrays in sub-block order
            sup[:SB_QH] = blk[:, :24].reshape(-1)
            # tail trits: element 120 + e of sub-block sub is qh[e & 1] bits
            # 2 (e >> 1) of that block (reading R-qh); it is tail trit 8 sub + e
            qh = [0] * 13
            for sub in range(SB_BLOCKS):
                for e in range(8):
                    u = (int(blk[sub, 24 + (e & 1)]) >> (2 * (e >> 1))) & 3
                    byte, digit = tail_position(8 * sub + e)
                    qh[byte] += u * 3 ** digit
            pat = tuple(int(v) for v in pats[r, sb])
            p = index.get(pat, ESCAPE)
            ebyte, free = pattern_fields(p)
            byte, digit = tail_position(64)
            qh[byte] += free * 3 ** digit
            sup[SB_QH:SB_MANT] = qh
            sup[SB_MANT:SB_EXP] = mantissa_bytes(dd & 0x3FF)
            sup[SB_EXP] = ebyte
            if p == ESCAPE:
                esc.append((superblock_index(r, sb, nsb), pat))
    esc.sort()
    return (out, book, np.array([g for g, _ in esc], dtype=np.int64),
            np.array([pt for _, pt in esc], dtype=np.uint8).reshape(-1, SB_BLOCKS))


def superblock_pattern(sup: np.ndarray, gidx: int, codebook, esc_idx, esc_pat):
    """The eight exponent fields of superblock ``sup`` (216 bytes), global
    index gidx (section 3.1: the pattern lookup takes the superblock's index,
    the codebook and the escape table)."""
    byte, digit = tail_position(64)
    free = (int(sup[SB_QH + byte]) // 3 ** digit) % 3
    p = pattern_index(int(sup[SB_EXP]), free)
    if p < ESCAPE:
        return [int(v) for v in codebook[p]]
    j = int(np.searchsorted(esc_idx, gidx))
    assert j < len(esc_idx) and int(esc_idx[j]) == gidx, "escaped superblock missing from the table"
    return [int(v) for v in esc_pat[j]]


def decode_ptq1_1(sup: np.ndarray, codebook, esc_idx, esc_pat) -> np.ndarray:
    """Superblocks uint8 [N][K/1024][216] -> the PTQ1_0 blocks uint8
    [N][K/128][28] they hold (section 3.1: qs of sub-block sub, its eight
    tail trits, its scale -- "the same as the PTQ1_0 format")."""
    s = np.asarray(sup, dtype=np.uint8)
    n, nsb, _ = s.shape
    out = np.zeros((n, nsb * SB_BLOCKS, BLOCK_BYTES), dtype=np.uint8)
    for r in range(n):
        for sb in range(nsb):
            x = s[r, sb]
            exps = superblock_pattern(x, superblock_index(r, sb, nsb), codebook, esc_idx, esc_pat)
            mant = mantissas(x[SB_MANT:SB_EXP])
            for sub in range(SB_BLOCKS):
                blk = out[r, sb * SB_BLOCKS + sub]
                blk[:24] = x[24 * sub:24 * sub + 24]
                qh = [0, 0]
                for e in range(8):
                    byte, digit = tail_position(8 * sub + e)
                    u = (int(x[SB_QH + byte]) // 3 ** digit) % 3
                    qh[e & 1] |= u << (2 * (e >> 1))
                blk[24], blk[25] = qh
                dbits = (exps[sub] << 10) | mant[sub]
                blk[26], blk[27] = dbits & 0xFF, dbits >> 8
    return out


def gemv_ternary_ptq1_1(sup, codebook, esc_idx, esc_pat, x_blocks) -> np.ndarray:
    """y[c, r] for PTQ1_1 weights: the PTQ1_0 GEMV of the decoded blocks."""
    return gemv_ternary(decode_ptq1_1(sup, codebook, esc_idx, esc_pat), x_blocks)


# ---------------------------------------------------------------- PT planes
PT_PLANES = 9     # eight planes of q, one of (d, s)
PT_SLOT = 16      # bytes per block per plane


def pt_offset(e: int, i: int, k: int) -> int:
    """Byte of element e (0..127) of 128-element block i in a column's PT
    array (Ternary post, section 3.1: plane floor(e / 16), slot i)."""
    return PT_SLOT * ((e // 16) * (k // QK) + i) + e % 16


def pt_ds_offset(j: int, i: int, k: int) -> int:
    """Byte of the (d, s) pair of sub-block j (0..3) of block i: plane 8
    (reading R-pt)."""
    return PT_SLOT * (8 * (k // QK) + i) + 4 * j


def q8_1_to_pt(blocks: np.ndarray) -> np.ndarray:
    """block_q8_1 bytes [c][K/32][36] -> PT arrays uint8 [c][9 K / 8]."""
    b = np.asarray(blocks, dtype=np.uint8)
    c, nsb, _ = b.shape
    k = nsb * Q8_QK
    assert k % QK == 0
    nb = k // QK
    q = b[:, :, 4:].reshape(c, k)          # q of element 128 i + e, as bytes
    out = np.zeros((c, PT_PLANES * nb * PT_SLOT), dtype=np.uint8)
    e = np.arange(QK)
    for i in range(nb):
        offs = np.array([pt_offset(int(v), i, k) for v in e])
        out[:, offs] = q[:, QK * i + e]
        for j in range(QK // Q8_QK):
            o = pt_ds_offset(j, i, k)
            out[:, o:o + 4] = b[:, 4 * i + j, 0:4]
    return out


def pt_to_q8_1(pt: np.ndarray) -> np.ndarray:
    """Inverse of ``q8_1_to_pt``: PT arrays [c][9 K / 8] -> [c][K/32][36]."""
    p = np.asarray(pt, dtype=np.uint8)
    c, nbytes = p.shape
    assert nbytes % (PT_PLANES * PT_SLOT) == 0
    nb = nbytes // (PT_PLANES * PT_SLOT)
    k = nb * QK
    out = np.zeros((c, k // Q8_QK, Q8_BYTES), dtype=np.uint8)
    e = np.arange(QK)
    for i in range(nb):
        offs = np.array([pt_offset(int(v), i, k) for v in e])
        out[:, 4 * i:4 * i + 4, 4:] = p[:, offs].reshape(c, 4, Q8_QK)
        for j in range(QK // Q8_QK):
            o = pt_ds_offset(j, i, k)
            out[:, 4 * i + j, 0:4] = p[:, o:o + 4]
    return out
