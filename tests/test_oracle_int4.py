"""Pins of the int4 oracle against what the pages and the mathematics fix.

Every test here runs on the CPU.  Each check is chosen so that a plausible
mistake in the oracle (swapped nibbles, a transposed operand, a dropped zero
point, a wrong rounding) fails at least one of them.
"""
import numpy as np
import pytest
import torch

from oracle import fpformat, int4
from conftest import load_golden

import wq_inputs


def _ints(v):
    return [int(t) for t in v]


# ---------------------------------------------------------------- bf16 / fp16
def test_bf16_rounding_known_values():
    # 0.01 = 1.28 * 2^-7: mantissa 0.28 * 128 = 35.84 -> 36 (0x24), exponent 120
    assert fpformat.f32_to_bf16_bits(np.float32(0.01))[()] == 0x3C24
    # exact ties round to even: 1 + 2^-8 -> 1.0 ; 1 + 3 * 2^-8 -> 1 + 2^-6
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000], dtype=np.uint32).view(np.float32)
    assert list(fpformat.f32_to_bf16_bits(ties)) == [0x3F80, 0x3F82, 0xBF80]
    # just above a tie rounds up
    above = np.array([0x3F808001], dtype=np.uint32).view(np.float32)
    assert fpformat.f32_to_bf16_bits(above)[0] == 0x3F81
    # carry into the exponent
    carry = np.array([0x3FFFFFFF], dtype=np.uint32).view(np.float32)
    assert fpformat.f32_to_bf16_bits(carry)[0] == 0x4000


def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(5)
    a = (rng.standard_normal(100000) * np.exp(rng.uniform(-30, 30, 100000))).astype(np.float32)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(fpformat.f32_to_bf16_bits(a), ref)


# ---------------------------------------------------------------- packing
def test_pack_unpack_exhaustive():
    every_byte = np.arange(256, dtype=np.uint8).reshape(1, 256)
    assert np.array_equal(int4.pack_plain(int4.unpack_plain(every_byte)), every_byte)
    pairs = np.array([[a, b] for a in range(16) for b in range(16)], dtype=np.uint8)
    packed = int4.pack_plain(pairs)
    assert np.array_equal(int4.unpack_plain(packed), pairs)
    # low nibble = even k (Helion issue: b & 0x0F is the first of each pair)
    assert np.array_equal(packed[:, 0] & 0x0F, pairs[:, 0])
    assert np.array_equal(packed[:, 0] >> 4, pairs[:, 1])


def test_vulkan_word_formula():
    g = load_golden("vulkan_packing.txt")
    codes = np.array([_ints(g["codes"])], dtype=np.uint8)
    word = int4.pack(codes, int4.LAYOUT_PLAIN).view("<u4")[0, 0]
    assert word == int(g["word_hex"][0], 16)
    # the post's word formula on random codes: word = sum_j w_j << 4j
    rng = np.random.default_rng(1)
    c = rng.integers(0, 16, (3, 64), dtype=np.uint8)
    words = int4.pack(c, int4.LAYOUT_PLAIN).view("<u4")
    for r in range(3):
        for m in range(8):
            expect = 0
            for j in range(8):
                expect |= int(c[r, 8 * m + j]) << (4 * j)
            assert int(words[r, m]) == expect


def test_gfx950_worked_case_and_unpack_pairs():
    codes = np.arange(8, dtype=np.uint8).reshape(1, 8)
    w = int(int4.pack(codes, int4.LAYOUT_GFX950).view("<u4")[0, 0])
    assert w == 0x75316420
    # the register unpack this order exists for: (w >> 4j) & 0x000F000F
    # yields elements (2j, 2j+1) in the two 16-bit halves
    rng = np.random.default_rng(2)
    c = rng.integers(0, 16, (4, 256), dtype=np.uint8)
    words = int4.pack(c, int4.LAYOUT_GFX950).view("<u4")
    for r in range(4):
        for m in range(32):
            wd = int(words[r, m])
            for j in range(4):
                pair = (wd >> (4 * j)) & 0x000F000F
                assert pair & 0xFFFF == c[r, 8 * m + 2 * j]
                assert pair >> 16 == c[r, 8 * m + 2 * j + 1]
                # OR-ing 0x4300 makes the bf16 of 128 + code
                bf = np.array([(pair & 0xFFFF) | 0x4300], dtype=np.uint16)
                assert fpformat.bf16_bits_to_f32(bf)[0] == 128 + c[r, 8 * m + 2 * j]


def test_gfx950_bijection():
    rng = np.random.default_rng(3)
    c = rng.integers(0, 16, (7, 512), dtype=np.uint8)
    p = int4.pack(c, int4.LAYOUT_GFX950)
    assert np.array_equal(int4.unpack(p, int4.LAYOUT_GFX950), c)
    iota = (np.arange(512) % 16).astype(np.uint8).reshape(1, 512)
    assert np.array_equal(int4.unpack(int4.pack(iota, 1), 1), iota)
    # same bytes as a set per word (a permutation of nibbles within words)
    plain = int4.unpack_plain(int4.pack(c, 0)).reshape(7, 64, 8)
    inter = int4.unpack_plain(p).reshape(7, 64, 8)
    assert np.array_equal(np.sort(plain, axis=2), np.sort(inter, axis=2))
    assert int4.inverse_order(int4.inverse_order(int4.GFX950_ORDER)) == int4.GFX950_ORDER


def test_paddle_printed_sequences():
    """The permutation machinery reproduces the Paddle PR's printed values."""
    g = {k: _ints(v) for k, v in load_golden("paddle_permute_sequences.txt").items()}
    order = tuple(g["fast_dequant_order"])
    assert order == int4.GFX950_ORDER
    out = np.array(g["dequant_output"])
    before = int4.permute_groups(out, order)
    assert list(before) == g["before_dequant"]
    # undoing the store order gives the dequant output back
    assert list(int4.permute_groups(before, int4.inverse_order(order))) == g["dequant_output"]
    # byte form -> pair indices -> the int4 permute_kk is the inverse map
    bf = g["byte_form"]
    pair_idx = [bf[2 * i] // 2 for i in range(16)]
    assert pair_idx == g["byte_index"]
    assert [pair_idx.index(i) for i in range(16)] == g["permute_kk_int4"]
    assert list(int4.inverse_order(tuple(g["byte_index"]))) == g["permute_kk_int4"]
    # int8 -> int4 permute_kk: regroup, then (t % 8) * 2, +1 on the second half
    kk8 = g["permute_kk_int8"]
    regrouped = kk8[0:4] + kk8[8:12] + kk8[4:8] + kk8[12:16]
    assert regrouped == g["permute_kk_int8_regrouped"]
    mod8 = [(t % 8) * 2 for t in regrouped]
    assert mod8 == g["permute_kk_mod8_times2"]
    assert mod8[:8] + [t + 1 for t in mod8[8:]] == g["permute_kk_int4"]
    # "simple bit ops": within each 4-byte word swap the high nibble of byte 0
    # with the low nibble of byte 2, and byte 1's high with byte 3's low
    def to_words(seq):
        v = np.array(seq, dtype=np.uint32).reshape(-1, 8)
        return [sum(int(v[i, j]) << (4 * j) for j in range(8)) for i in range(len(v))]
    src = to_words([t % 16 for t in bf])
    dst = to_words([t % 16 for t in g["before_dequant"]])
    for xs, xd in zip(src, dst):
        t = ((xs >> 12) ^ xs) & 0x0000F0F0
        assert (xs ^ t ^ (t << 12)) == xd
    # row interleave index (section "int4 row interval") is a bijection when
    # total_k is the packed bytes per row
    n_rows, total_k = 8, 64
    idx = sorted(pk % 32 + pk // 32 * 128 + 32 * (n % 4) + total_k * 4 * (n // 4)
                 for n in range(n_rows) for pk in range(total_k))
    assert idx == list(range(n_rows * total_k))


# ---------------------------------------------------------------- quantiser
def test_quantize_handworked():
    g = load_golden("quantize_handworked.txt")
    w = np.array([int(h, 16) for h in g["w_f16_hex"]], dtype=np.uint16).reshape(1, 8)
    codes, scales, bits = int4.quantize_int4(w, 8, "bf16")
    assert bits[0, 0] == int(g["scale_bf16_hex"][0], 16)
    assert scales[0, 0] == np.float32(0.010009765625)
    assert list(codes[0]) == _ints(g["codes"])
    plain = int4.pack(codes, int4.LAYOUT_PLAIN)
    assert [f"{b:02x}" for b in plain[0]] == g["plain_bytes_hex"]
    word = int4.pack(codes, int4.LAYOUT_GFX950).view("<u4")[0, 0]
    assert f"{int(word):08x}" == g["gfx950_word_hex"][0]


@pytest.mark.parametrize("group,sdt", [(128, "bf16"), (512, "f32"), (32, "bf16")])
def test_quantize_invariants(group, sdt):
    rng = np.random.default_rng(4)
    w = wq_inputs.to_f16_bits(0.02 * rng.standard_normal((16, 512)))
    w[3, :group] = 0                                    # an all-zero group
    codes, scales, _ = int4.quantize_int4(w, group, sdt)
    wf = fpformat.f16_bits_to_f32(w).astype(np.float64)
    assert codes.min() >= 0 and codes.max() <= 15
    assert np.all(codes[3, :group] == 8) and scales[3, 0] == 0
    s = np.repeat(scales.astype(np.float64), group, axis=1)
    err = np.abs(wf - (codes.astype(np.float64) - 8) * s)
    assert np.all(err <= s / 2 * (1 + 1e-6) + 1e-30)
    # the absmax element of each group lands on code 1 or 15
    for r in range(16):
        for gi in range(512 // group):
            blk = wf[r, gi * group:(gi + 1) * group]
            if np.all(blk == 0):
                continue
            j = int(np.argmax(np.abs(blk)))
            assert codes[r, gi * group + j] in (1, 15)
    if sdt == "bf16":  # stored scale is a bf16 value
        assert np.array_equal(fpformat.bf16_bits_to_f32(fpformat.f32_to_bf16_bits(scales)), scales)


def test_quantize_exact_ties_round_to_even():
    # absmax 7 -> scale exactly 1 (bf16 and f32): w / s is w itself, so the
    # ties 0.5, 1.5, 2.5, -0.5, -2.5 round to 0, 2, 2, -0, -2
    w = np.array([[7.0, 0.5, 1.5, 2.5, -0.5, -2.5, 3.25, -6.75]], dtype=np.float32)
    wb = w.astype(np.float16).view(np.uint16)
    codes, scales, _ = int4.quantize_int4(wb, 8, "bf16")
    assert scales[0, 0] == 1.0
    assert list(codes[0].astype(int) - 8) == [7, 0, 2, 2, 0, -2, 3, -7]


# ---------------------------------------------------------------- GEMV / GEMM
def test_gemv_handworked():
    g = load_golden("gemv_handworked.txt")
    codes = np.array([_ints(g["codes_row0"]), _ints(g["codes_row1"])], dtype=np.uint8)
    codes = np.concatenate([codes, np.full((2, 24), 0, np.uint8)], axis=1)  # pad K to 32
    x = np.concatenate([np.array([[float(t) for t in g["x"]]]), np.zeros((1, 24))], axis=1)
    scale = np.array([[float(t)] for t in g["scale"]])
    zero = np.array([[float(t)] for t in g["zero"]])
    for layout in (0, 1):
        d = int4.gemv_w4(int4.pack(codes, layout), layout, scale, zero, 0.0, 32, x)
        assert list(d[0]) == [float(t) for t in g["out"]]


def _brute_gemv(codes, scales, zeros, zc, group, x):
    n, k = codes.shape
    out = [[0.0] * n for _ in range(x.shape[0])]
    for c in range(x.shape[0]):
        for r in range(n):
            acc = 0.0
            for kk in range(k):
                z = zc if zeros is None else float(zeros[r][kk // group])
                acc += (int(codes[r][kk]) - z) * float(scales[r][kk // group]) * float(x[c][kk])
            out[c][r] = acc
    return np.array(out)


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("k,group,with_zeros", [(16, 16, True), (128, 128, False), (256, 128, True)])
def test_gemv_brute_force_tiny(layout, k, group, with_zeros):
    rng = np.random.default_rng(7)
    n, c = 8, 3
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    scales = rng.uniform(0.01, 0.1, (n, k // group))
    zeros = rng.uniform(6, 9, (n, k // group)) if with_zeros else None
    x = rng.standard_normal((c, k))
    got = int4.gemv_w4(int4.pack(codes, layout), layout, scales, zeros, 8.0, group, x)
    ref = _brute_gemv(codes, scales, zeros, 8.0, group, x)
    assert got.shape == (c, n)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_gemv_closed_forms():
    rng = np.random.default_rng(8)
    n, k = 12, 256
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    scales = rng.uniform(0.01, 0.1, (n, 2))
    p = int4.pack(codes, 1)
    # one-hot x picks out one dequantised column exactly
    for kk in (0, 5, 130, 255):
        x = np.zeros((1, k)); x[0, kk] = 1.0
        d = int4.gemv_w4(p, 1, scales, None, 8.0, 128, x)
        assert np.array_equal(d[0], (codes[:, kk].astype(np.float64) - 8) * scales[:, kk // 128])
    # codes equal to the zero point give exactly 0
    z = np.full((n, k), 8, np.uint8)
    x = rng.standard_normal((2, k))
    assert np.all(int4.gemv_w4(int4.pack(z, 1), 1, scales, None, 8.0, 128, x) == 0)
    # integer exactness: s = 1, z = 8, integer x gives the exact integer sum
    xi = rng.integers(-2, 3, (2, k)).astype(np.float64)
    d = int4.gemv_w4(p, 1, np.ones((n, 2)), None, 8.0, 128, xi)
    exact = xi.astype(np.int64) @ (codes.astype(np.int64) - 8).T
    assert np.array_equal(d, exact.astype(np.float64))


def test_gemm_rows_closed_forms():
    rng = np.random.default_rng(9)
    m, n, k = 6, 10, 64
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    p = int4.pack(codes, 1)
    s = rng.uniform(0.005, 0.02, (n, 1))
    a = np.zeros((m, k))
    for i in range(m):
        a[i, 3 * i] = 1.0
    c = int4.gemm_w4a16_rows(a, p, 1, s, 8.0, k)
    for i in range(m):
        # one-hot A row i picks B's logical row k = 3i: C[i, n] = (q[n, 3i] - 8) s_n
        assert np.array_equal(c[i], (codes[:, 3 * i].astype(np.float64) - 8) * s[:, 0])
    ai = rng.integers(-4, 5, (m, k))
    c = int4.gemm_w4a16_rows(ai.astype(np.float64), p, 1, np.ones((n, 1)), 8.0, k)
    assert np.array_equal(c, (ai @ (codes.astype(np.int64) - 8).T).astype(np.float64))


def test_gemm_bf16_weights_handworked():
    # one column, group 64, scale bf16 0x3C24 = 1.28125 * 2^-7: (q - 8) = 7
    # gives 8.96875 * 2^-7 = (1 + 15.5/128) * 2^-4, a tie that rounds to even
    # (16/128) -> 0.0703125; q - 8 = 3 gives 3.84375 * 2^-7, exact in bf16;
    # q - 8 = -7 mirrors the tie.  One-hot rows of A read single weights.
    s = fpformat.bf16_bits_to_f32(np.array([[0x3C24]], np.uint16)).astype(np.float64)
    assert s[0, 0] == 0.010009765625
    codes = np.full((1, 64), 8, np.uint8)
    codes[0, 0], codes[0, 1], codes[0, 2] = 15, 11, 1
    a = np.eye(64)[:3]
    c = int4.gemm_w4a16_rows_bf16w(a, int4.pack(codes, 1), 1, s, 8.0, 64)
    assert c[:, 0].tolist() == [0.0703125, 0.030029296875, -0.0703125]
    exact = int4.gemm_w4a16_rows(a, int4.pack(codes, 1), 1, s, 8.0, 64)
    assert exact[:, 0].tolist() == [7 * 0.010009765625, 3 * 0.010009765625, -7 * 0.010009765625]


def test_gemm_bf16_weights_equal_exact_for_power_of_two_scales():
    # (q - 8) * 2^e is exact in bf16, so rounding the weights changes nothing;
    # a wrong group index (scale taken from another group) would still differ
    # from the exact oracle because the exponents vary per group.
    rng = np.random.default_rng(12)
    m, n, k, group = 5, 12, 512, 128
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    s = 2.0 ** rng.integers(-3, 3, (n, k // group))
    a = rng.standard_normal((m, k))
    p = int4.pack(codes, 1)
    got = int4.gemm_w4a16_rows_bf16w(a, p, 1, s, 8.0, group)
    ref = int4.gemm_w4a16_rows(a, p, 1, s, 8.0, group)
    assert np.array_equal(got, ref)
    # and against a per-element brute force of the group lookup
    w = np.array([[(int(codes[r, kk]) - 8) * s[r, kk // group] for kk in range(k)] for r in range(n)])
    assert np.allclose(ref, a @ w.T, rtol=0, atol=1e-12)


def test_gemm_stored_zeros_brute_force():
    # stored zeros per group (bf16-like fractional values): per-element brute
    # force of (q - z[n, g]) * s[n, g]; and the bf16-weight variant rounds
    # exactly those products
    rng = np.random.default_rng(13)
    m, n, k, group = 4, 9, 256, 64
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    s = fpformat.bf16_bits_to_f32(fpformat.f32_to_bf16_bits(rng.uniform(0.002, 0.02, (n, k // group)).astype(np.float32))).astype(np.float64)
    z = fpformat.bf16_bits_to_f32(fpformat.f32_to_bf16_bits(rng.uniform(6, 9, (n, k // group)).astype(np.float32))).astype(np.float64)
    a = rng.standard_normal((m, k))
    p = int4.pack(codes, 1)
    got = int4.gemm_w4a16_rows(a, p, 1, s, 8.0, group, zeros=z)
    w = np.array([[(int(codes[r, kk]) - z[r, kk // group]) * s[r, kk // group] for kk in range(k)]
                  for r in range(n)])
    assert np.allclose(got, a @ w.T, rtol=0, atol=1e-12)
    # the product is exact in float32, so the bf16 variant is the RNE of it
    assert np.array_equal(w.astype(np.float32).astype(np.float64), w)
    w16 = fpformat.bf16_bits_to_f32(fpformat.f32_to_bf16_bits(w.astype(np.float32))).astype(np.float64)
    assert np.allclose(int4.gemm_w4a16_rows_bf16w(a, p, 1, s, 8.0, group, zeros=z), a @ w16.T,
                       rtol=0, atol=1e-12)
