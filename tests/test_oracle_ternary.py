"""Pins of the ternary oracle against the Ternary post and closed forms."""
import numpy as np
import pytest

from oracle import fpformat, ternary
from conftest import load_golden

import wq_inputs


def _ints(v):
    return [int(t) for t in v]


def test_format_sizes():
    g = load_golden("ptq1_0_layout.txt")
    assert ternary.BLOCK_BYTES == int(g["block_bytes"][0])
    assert ternary.Q8_BYTES == int(g["q8_1_bytes"][0])
    blk = ternary.encode_ptq1_0(np.zeros((1, 128), np.int8), np.zeros((1, 1), np.uint16))
    assert blk.shape == (1, 1, 28)
    # trit counts per section: 16 bytes x 5 + 8 bytes x 5 = 120, and 8 in qh
    kinds = [ternary.trit_position(e)[0] for e in range(128)]
    assert kinds.count("qs") == int(g["qs_trits"][0]) and kinds.count("qh") == int(g["qh_trits"][0])
    # superblock arithmetic: 192 + 13 + 10 (eight 10-bit mantissas) + 1 bytes
    sb = 192 + 13 + 8 * 10 // 8 + 1
    assert sb == int(g["superblock_bytes"][0])
    assert 8 * ternary.BLOCK_BYTES == int(g["plain_bytes_per_1024"][0])
    assert (8 * ternary.BLOCK_BYTES - sb) * 28 == 8 * ternary.BLOCK_BYTES


def test_trit_positions_match_post():
    g = load_golden("ptq1_0_layout.txt")
    for digit, e in enumerate(_ints(g["qs_byte0_elements"])):
        assert ternary.trit_position(e) == ("qs", 0, digit)
    for digit, e in enumerate(_ints(g["qs_byte16_elements"])):
        assert ternary.trit_position(e) == ("qs", 16, digit)
    # every (byte, slot) is used exactly once
    slots = {ternary.trit_position(e) for e in range(128)}
    assert len(slots) == 128


def test_digit_placement_by_value():
    # trit +1 (digit 2) at element 32 only, 0 (digit 1) elsewhere: byte 0 is
    # 1 + 3 + 2*9 + 27 + 81 = 130; every other qs byte is 121; qh bytes 0x55
    t = np.zeros((1, 128), np.int8)
    t[0, 32] = 1
    b = ternary.encode_ptq1_0(t, np.array([[0x3C00]], np.uint16))[0, 0]
    assert b[0] == 130 and all(v == 121 for v in b[1:24])
    assert b[24] == 0x55 and b[25] == 0x55 and b[26] == 0x00 and b[27] == 0x3C
    # the tail: element 121 -> qh[1] bits 0..1; element 126 -> qh[0] bits 6..7
    t = np.full((1, 128), -1, np.int8)
    t[0, 121] = 1
    t[0, 126] = 0
    b = ternary.encode_ptq1_0(t, np.zeros((1, 1), np.uint16))[0, 0]
    assert b[24] == 0x40 and b[25] == 0x02 and all(v == 0 for v in b[:24])


def test_ptq1_0_round_trip_exhaustive_bytes():
    # every byte value 0..242 decodes to five digits and re-encodes to itself
    blocks = np.zeros((1, 243, 28), np.uint8)
    for v in range(243):
        blocks[0, v, :24] = v
        blocks[0, v, 24:26] = 0x55
    t, d = ternary.decode_ptq1_0(blocks)
    assert np.array_equal(ternary.encode_ptq1_0(t, d), blocks)
    for v in range(243):
        digits = [(v // 3 ** j) % 3 for j in range(5)]
        assert sum(u * 3 ** j for j, u in enumerate(digits)) == v
        assert int(t[0, 128 * v + 0]) + 1 == digits[0]
        assert int(t[0, 128 * v + 64]) + 1 == digits[4]


def test_ptq1_0_round_trip_random():
    p = wq_inputs.ternary_gemv(k=512, n=9, cmax=1)
    blk = ternary.encode_ptq1_0(p.trits, p.d_bits)
    t, d = ternary.decode_ptq1_0(blk)
    assert np.array_equal(t, p.trits) and np.array_equal(d, p.d_bits)
    assert blk[:, :, :24].max() <= 242


def test_q8_1_closed_forms():
    # integer x with amax 127: d = 1 exactly, q = x, s = sum(x)
    x = np.zeros((2, 64), np.float32)
    x[0, :32] = np.arange(-16, 16)
    x[0, 5] = 127
    x[0, 32:] = 0                       # an all-zero block: d = 0, q = 0
    x[1, :32] = np.arange(32) * 2.0 - 31.0
    x[1, 0] = -63.5                     # amax 63.5 -> d = 0.5, q = 2x
    x[1, 32:] = 127.0
    blk = ternary.quantize_q8_1(x)
    q, d, s = ternary.decode_q8_1(blk)
    assert d[0, 0] == 0x3C00 and np.array_equal(q[0, :32], x[0, :32].astype(np.int8))
    assert fpformat.f16_bits_to_f32(s[0, :1])[0] == x[0, :32].sum()
    assert d[0, 1] == 0 and s[0, 1] == 0 and np.all(q[0, 32:] == 0)
    assert d[1, 0] == 0x3800 and np.array_equal(q[1, :32], (2 * x[1, :32]).astype(np.int8))
    assert np.all(q[1, 32:] == 127) and d[1, 1] == 0x3C00


def test_q8_1_ties_and_bounds():
    # d = 1: ties 0.5 1.5 2.5 -0.5 -1.5 round to even
    x = np.zeros((1, 32), np.float32)
    x[0, :6] = [127, 0.5, 1.5, 2.5, -0.5, -1.5]
    q, _, _ = ternary.decode_q8_1(ternary.quantize_q8_1(x))
    assert list(q[0, :6]) == [127, 0, 2, 2, 0, -2]
    rng = np.random.default_rng(3)
    xr = rng.standard_normal((4, 1024)).astype(np.float32)
    q, d, _ = ternary.decode_q8_1(ternary.quantize_q8_1(xr))
    dd = np.repeat(fpformat.f16_bits_to_f32(d), 32, axis=1)
    assert np.abs(q.astype(np.int32)).max() <= 127
    assert np.all(np.abs(xr - q * dd) <= dd / 2 * (1 + 1e-3))


def test_ternary_unit_scale_exact():
    p = wq_inputs.ternary_gemv(k=512, n=20, cmax=3, unit_scale=True)
    wb = ternary.encode_ptq1_0(p.trits, p.d_bits)
    xb = ternary.quantize_q8_1(p.x)
    q, d, _ = ternary.decode_q8_1(xb)
    assert np.all(d == 0x3C00) and np.array_equal(q, p.x.astype(np.int8))
    y = ternary.gemv_ternary(wb, xb)
    exact = p.x.astype(np.int64) @ p.trits.astype(np.int64).T
    assert np.array_equal(y, exact.astype(np.float64))


def test_ternary_special_cases():
    rng = np.random.default_rng(11)
    k, n = 256, 4
    x = rng.standard_normal((2, k)).astype(np.float32)
    xb = ternary.quantize_q8_1(x)
    q, dbits, _ = ternary.decode_q8_1(xb)
    dx = np.repeat(fpformat.f16_bits_to_f32(dbits).astype(np.float64), 32, axis=1)
    dw = rng.uniform(0.01, 0.05, (n, k // 128)).astype(np.float32)
    dwb = fpformat.f32_to_f16_bits(dw)
    dwf = fpformat.f16_bits_to_f32(dwb).astype(np.float64)
    # all trits zero -> 0
    y = ternary.gemv_ternary(ternary.encode_ptq1_0(np.zeros((n, k), np.int8), dwb), xb)
    assert np.all(y == 0)
    # all trits +1 -> sum over blocks of d_w * d_x * q
    y = ternary.gemv_ternary(ternary.encode_ptq1_0(np.ones((n, k), np.int8), dwb), xb)
    ref = np.einsum("ck,rk->cr", dx * q, np.repeat(dwf, 128, axis=1))
    np.testing.assert_allclose(y, ref, rtol=1e-12)
    # one nonzero trit picks out one product
    t = np.zeros((n, k), np.int8)
    t[2, 77] = -1
    y = ternary.gemv_ternary(ternary.encode_ptq1_0(t, dwb), xb)
    for c in range(2):
        assert y[c, 2] == -dwf[2, 0] * dx[c, 77] * q[c, 77]
        assert np.all(np.delete(y[c], 2) == 0)


# ---- PTQ1_1 superblocks (Ternary post, section 2 struct ptq1_1; section 3.1)
def test_ptq1_1_sizes_match_post():
    g = load_golden("ptq1_0_layout.txt")
    assert ternary.SB_BYTES == int(g["superblock_bytes"][0])
    # trits: qs + qh = 205 bytes against 8 * (24 + 2) = 208
    assert ternary.SB_MANT == int(g["superblock_trit_bytes"][0])
    assert 8 * 26 == int(g["plain_trit_bytes_per_1024"][0])
    # scales: 10 mantissa bytes + 1 exponent byte = 11 against 8 * 2 = 16
    assert ternary.SB_BYTES - ternary.SB_MANT == int(g["superblock_scale_bytes"][0])
    assert 8 * 2 == int(g["plain_scale_bytes_per_8"][0])
    # 256 exponent-byte values x 3 free-trit digits; the last is the escape
    assert 256 * 3 == int(g["superblock_patterns"][0])
    assert ternary.ESCAPE == int(g["superblock_escape_index"][0]) == ternary.CODEBOOK_ROWS
    # 13 bytes hold 65 trits: the 64 tail trits and one free trit
    assert 13 * 5 == 8 * 8 + 1 and ternary.tail_position(64) == (12, 4)
    sup, _, _, _ = ternary.encode_ptq1_1(ternary.encode_ptq1_0(np.zeros((2, 2048), np.int8),
                                                               np.full((2, 16), 0x3C00, np.uint16)))
    assert sup.shape == (2, 2, 216)


def test_ptq1_1_handworked_single_superblock():
    g = load_golden("ptq1_1_handworked.txt")
    t = np.zeros((1, 1024), np.int8)
    t[0, 128 + 121] = 1                     # sub-block 1, element 121
    d = np.full((1, 8), 0x3C00, np.uint16)
    d[0, 7] = 0x3801
    sup, book, ei, ep = ternary.encode_ptq1_1(ternary.encode_ptq1_0(t, d))
    s = sup[0, 0]
    assert all(int(v) == 121 for v in s[:192])
    assert _ints(s[192:205]) == _ints(g["a_qh"])
    assert _ints(s[205:215]) == _ints(g["a_mantissa_bytes"])
    assert int(s[215]) == int(g["a_exponent_byte"][0])
    assert _ints(book[0]) == _ints(g["a_codebook_row0"]) and not book[1:].any()
    assert len(ei) == 0 and ep.shape == (0, 8)


def test_ptq1_1_handworked_escape():
    g = load_golden("ptq1_1_handworked.txt")
    nsb = 768
    e = np.zeros((nsb, 8), np.int64)
    j = np.arange(767)
    e[:767, 6] = j // 31
    e[:767, 7] = j % 31
    e[767, :] = 30
    d = (e.reshape(1, nsb * 8) << 10).astype(np.uint16)
    t = np.zeros((1, nsb * 1024), np.int8)
    sup, book, ei, ep = ternary.encode_ptq1_1(ternary.encode_ptq1_0(t, d))
    esc = sup[0, 767]
    assert int(esc[204]) == int(g["b_escape_qh12"][0])
    assert int(esc[215]) == int(g["b_escape_exponent_byte"][0])
    assert _ints(ei) == _ints(g["b_escape_index"])
    assert _ints(ep[0]) == _ints(g["b_escape_pattern"])
    assert _ints(book[5]) == _ints(g["b_row5_pattern"])
    assert int(sup[0, 5, 215]) == int(g["b_sb5_exponent_byte"][0])
    assert int(sup[0, 5, 204]) == int(g["b_sb5_qh12"][0])
    # and the decoder finds the escaped scales again
    blocks = ternary.decode_ptq1_1(sup, book, ei, ep)
    _, d2 = ternary.decode_ptq1_0(blocks)
    assert np.array_equal(d2, d)


def test_ptq1_1_tail_positions_exhaustive():
    # each of the 64 tail trits set alone to +1 (digit 2, the rest digit 1)
    # raises exactly one qh byte by 3^digit at the reading's position
    for tt in range(64):
        sub, e = divmod(tt, 8)
        t = np.zeros((1, 1024), np.int8)
        t[0, 128 * sub + 120 + e] = 1
        sup, _, _, _ = ternary.encode_ptq1_1(ternary.encode_ptq1_0(t, np.full((1, 8), 0x3C00, np.uint16)))
        qh = sup[0, 0, 192:205].astype(int)
        byte, digit = ternary.tail_position(tt)
        base = np.array([121] * 12 + [40])
        base[byte] += 3 ** digit
        assert np.array_equal(qh, base), tt
        assert qh.max() <= 242


@pytest.mark.parametrize("independent,n,k", [(False, 40, 5120), (True, 240, 8192)])
def test_ptq1_1_round_trip(independent, n, k):
    # correlated scales (few patterns, no escape) and independent exponents
    # (many more patterns than codebook rows: most superblocks escape)
    p = wq_inputs.ternary_correlated_scales(k, n, 1, seed=n)
    d = p.d_bits
    if independent:
        rng = np.random.default_rng(k)
        d = ((rng.integers(5, 13, d.shape) << 10) | rng.integers(0, 1024, d.shape)).astype(np.uint16)
    blocks = ternary.encode_ptq1_0(p.trits, d)
    sup, book, ei, ep = ternary.encode_ptq1_1(blocks)
    if independent:
        assert len(ei) >= n * k // 1024 - 2 * 767  # (a few patterns repeat)
    assert np.array_equal(ternary.decode_ptq1_1(sup, book, ei, ep), blocks)
    assert sup[:, :, 192:205].max() <= 242
    assert np.all(np.diff(ei) > 0)
    # the GEMV of the superblocks is the GEMV of the blocks they hold
    xq = ternary.quantize_q8_1(p.x)
    assert np.array_equal(ternary.gemv_ternary_ptq1_1(sup, book, ei, ep, xq),
                          ternary.gemv_ternary(blocks, xq))


def test_ptq1_1_rejects_negative_scale():
    d = np.full((1, 8), 0x3C00, np.uint16)
    d[0, 3] = 0xBC00
    with pytest.raises(AssertionError):
        ternary.encode_ptq1_1(ternary.encode_ptq1_0(np.zeros((1, 1024), np.int8), d))


# ---------------------------------------------------------------- PT planes
def _q8_blocks(c, k, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 256, (c, k // 32, 36), dtype=np.uint8)


def test_pt_sizes_match_post():
    g = load_golden("ptq1_0_layout.txt")
    k = int(g["pt_example_k"][0])
    nb = k // 128
    assert nb == int(g["pt_example_blocks_per_plane"][0])
    assert 128 // 32 == int(g["pt_ds_pairs_per_block"][0])
    pt = ternary.q8_1_to_pt(_q8_blocks(1, k, 1))
    planes, slot = int(g["pt_planes"][0]), int(g["pt_slot_bytes"][0])
    assert pt.shape == (1, planes * nb * slot)
    # the same bytes as the column's q8_1 blocks: 9 K / 8 = 36 K / 32
    assert pt.shape[1] == (k // 32) * ternary.Q8_BYTES == 9 * k // 8
    # the four (d, s) pairs of a block fill its 16-byte slot of plane 8
    assert int(g["pt_ds_pairs_per_block"][0]) * 4 == slot
    assert int(g["pt_elements_per_plane_slot"][0]) * (planes - 1) == 128


def test_pt_offset_is_a_bijection():
    # planes 0..7: every (block, element) to its own byte of [0, 8 * 16 * K/128)
    for k in (128, 1024, 5120):
        nb = k // 128
        offs = sorted(ternary.pt_offset(e, i, k) for i in range(nb) for e in range(128))
        assert offs == list(range(8 * 16 * nb))
        ds = sorted(ternary.pt_ds_offset(j, i, k) + b for i in range(nb) for j in range(4) for b in range(4))
        assert ds == list(range(8 * 16 * nb, 9 * 16 * nb))


def test_pt_matches_plane_picture():
    # the post's picture read directly: plane p = [block 0][block 1]... with
    # elements 16p .. 16p + 15 of each block, then plane 8 = the (d, s) words
    c, k = 3, 1024
    blk = _q8_blocks(c, k, 2)
    pt = ternary.q8_1_to_pt(blk)
    nb = k // 128
    q = blk[:, :, 4:].reshape(c, nb, 8, 16)        # [col][block][plane][16]
    planes = q.transpose(0, 2, 1, 3).reshape(c, 8 * nb * 16)
    assert np.array_equal(pt[:, :8 * nb * 16], planes)
    ds = blk[:, :, 0:4].reshape(c, nb, 16)         # four (d, s) words per block
    assert np.array_equal(pt[:, 8 * nb * 16:], ds.reshape(c, nb * 16))


def test_pt_handworked_offsets():
    # K = 256 (two blocks per plane): element 17 of block 1 is plane 1, slot
    # 1, byte 1 -> 16 * (1 * 2 + 1) + 1 = 49; element 127 of block 0 is
    # plane 7, slot 0, byte 15 -> 16 * 14 + 15 = 239; the (d, s) pair of
    # sub-block 3 of block 1 starts at 16 * (8 * 2 + 1) + 12 = 284
    assert ternary.pt_offset(17, 1, 256) == 49
    assert ternary.pt_offset(127, 0, 256) == 239
    assert ternary.pt_ds_offset(3, 1, 256) == 284
    blk = np.zeros((1, 8, 36), np.uint8)
    blk[0, 4, 4 + 17] = 0xAB      # block 1 = sub-blocks 4..7; element 17 is in sub-block 4
    blk[0, 3, 4 + 31] = 0xCD      # element 127 of block 0: sub-block 3, q[31]
    blk[0, 7, 0:4] = [1, 2, 3, 4]
    pt = ternary.q8_1_to_pt(blk)[0]
    assert pt[49] == 0xAB and pt[239] == 0xCD and list(pt[284:288]) == [1, 2, 3, 4]
    assert np.count_nonzero(pt) == 6


def test_pt_round_trip():
    for c, k in ((1, 128), (2, 5120), (3, 17280 // 128 * 128)):
        blk = _q8_blocks(c, k, 3)
        assert np.array_equal(ternary.pt_to_q8_1(ternary.q8_1_to_pt(blk)), blk)
