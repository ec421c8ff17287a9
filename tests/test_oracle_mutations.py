"""The pins catch plausible mistakes in the oracle.

Each case below plants one mistake in the oracle (on the CPU, through
monkeypatch, for the duration of the test) -- a swapped nibble, a transposed
operand, a dropped zero point, a wrong divisor or rounding, a misplaced digit
or sign -- then runs the oracle's pin tests and requires at least one of them
to fail.  A case that no pin catches marks a gap in the pins.
"""
import numpy as np
import pytest

import test_oracle_int4 as pins_int4
import test_oracle_ternary as pins_ternary
from oracle import fpformat, int4, ternary


def _int4_pins():
    out = [f for name, f in sorted(vars(pins_int4).items())
           if name.startswith("test_") and f.__code__.co_argcount == 0]
    out.append(lambda: pins_int4.test_quantize_invariants(128, "bf16"))
    out.append(lambda: pins_int4.test_quantize_invariants(32, "bf16"))
    for layout in (0, 1):
        for args in ((16, 16, True), (128, 128, False), (256, 128, True)):
            out.append(lambda layout=layout, args=args: pins_int4.test_gemv_brute_force_tiny(layout, *args))
    return out


def _ternary_pins():
    out = [f for name, f in sorted(vars(pins_ternary).items())
           if name.startswith("test_") and f.__code__.co_argcount == 0]
    out.append(lambda: pins_ternary.test_ptq1_1_round_trip(False, 40, 5120))
    out.append(lambda: pins_ternary.test_ptq1_1_round_trip(True, 240, 8192))
    return out


# ------------------------------------------------------------ planted mistakes
def _swap_nibbles(mp):
    orig_pack, orig_unpack = int4.pack_plain, int4.unpack_plain

    def pack_plain(codes):
        p = orig_pack(codes)
        return ((p >> 4) | (p << 4)).astype(np.uint8)

    def unpack_plain(packed):
        p = np.asarray(packed, dtype=np.uint8)
        return orig_unpack(((p >> 4) | (p << 4)).astype(np.uint8))
    mp.setattr(int4, "pack_plain", pack_plain)
    mp.setattr(int4, "unpack_plain", unpack_plain)


def _inverse_interleave(mp):
    mp.setattr(int4, "GFX950_ORDER", int4.inverse_order(int4.GFX950_ORDER))


def _drop_zero(mp):
    orig = int4.dequantize
    mp.setattr(int4, "dequantize", lambda codes, scales, zeros, zc, group: orig(codes, scales, None, 0.0, group))


def _group_by_modulo(mp):
    def dequantize(codes, scales, zeros, zero_const, group):
        codes = np.asarray(codes)
        n, k = codes.shape
        s = np.tile(np.asarray(scales, dtype=np.float64).reshape(n, k // group), (1, group))
        z = np.float64(zero_const) if zeros is None else np.tile(
            np.asarray(zeros, dtype=np.float64).reshape(n, k // group), (1, group))
        return (codes.astype(np.float64) - z) * s
    mp.setattr(int4, "dequantize", dequantize)


def _transposed_gemv(mp):
    def gemv_w4(packed, layout, scales, zeros, zero_const, group, x):
        w = int4.dequantize(int4.unpack(packed, layout), scales, zeros, zero_const, group)
        return np.asarray(x, dtype=np.float64)[:, ::-1] @ w.T  # k reversed in x
    mp.setattr(int4, "gemv_w4", gemv_w4)


def _quantizer(divisor=7.0, rounding=np.rint, divide_by_rounded=True):
    """The oracle's quantiser with one knob turned."""
    def quantize_int4(w_f16_bits, group, scale_dtype):
        w = fpformat.f16_bits_to_f32(w_f16_bits)
        n, k = w.shape
        ng = k // group
        codes = np.empty((n, k), dtype=np.uint8)
        scales = np.empty((n, ng), dtype=np.float32)
        bits = np.empty((n, ng), dtype=np.uint16 if scale_dtype == "bf16" else np.uint32)
        for g in range(ng):
            blk = w[:, g * group:(g + 1) * group]
            s32 = (np.max(np.abs(blk), axis=1) / np.float32(divisor)).astype(np.float32)
            if scale_dtype == "bf16":
                b = fpformat.f32_to_bf16_bits(s32)
                s = fpformat.bf16_bits_to_f32(b)
            else:
                s, b = s32, s32.view(np.uint32)
            scales[:, g], bits[:, g] = s, b
            sd = s if divide_by_rounded else s32
            zero = sd == 0.0
            quot = (blk / np.where(zero, np.float32(1.0), sd)[:, None]).astype(np.float32)
            q = np.clip(rounding(quot), -8, 7).astype(np.int32) + 8
            q[zero, :] = 8
            codes[:, g * group:(g + 1) * group] = q.astype(np.uint8)
        return codes, scales, bits
    return quantize_int4


def _quant_divisor_8(mp):
    mp.setattr(int4, "quantize_int4", _quantizer(divisor=8.0))


def _quant_truncate(mp):
    mp.setattr(int4, "quantize_int4", _quantizer(rounding=np.trunc))


def _quant_half_up(mp):
    mp.setattr(int4, "quantize_int4", _quantizer(rounding=lambda v: np.floor(v + np.float32(0.5))))


def _quant_unrounded_scale(mp):
    mp.setattr(int4, "quantize_int4", _quantizer(divide_by_rounded=False))


def _digits_reversed(mp):
    orig = ternary.trit_position

    def trit_position(e):
        kind, byte, pos = orig(e)
        return (kind, byte, 4 - pos) if kind == "qs" else (kind, byte, pos)
    mp.setattr(ternary, "trit_position", trit_position)


def _trit_sign_flipped(mp):
    orig = ternary.decode_ptq1_0

    def decode_ptq1_0(blocks):
        t, d = orig(blocks)
        return (-t).astype(np.int8), d
    mp.setattr(ternary, "decode_ptq1_0", decode_ptq1_0)


def _weight_scale_per_32(mp):
    def gemv_ternary(w_blocks, x_blocks):
        trits, dw_bits = ternary.decode_ptq1_0(w_blocks)
        q, dx_bits, _ = ternary.decode_q8_1(x_blocks)
        S = ternary.subblock_sums(trits, q).astype(np.float64)
        dw = fpformat.f16_bits_to_f32(dw_bits).astype(np.float64)
        dx = fpformat.f16_bits_to_f32(dx_bits).astype(np.float64)
        dw32 = np.tile(dw, (1, 4))   # block b of 128 paired with the wrong 32-k sub-blocks
        return np.einsum("rcb,rb,cb->cr", S, dw32, dx)
    mp.setattr(ternary, "gemv_ternary", gemv_ternary)


def _q8_divisor_128(mp):
    orig = ternary.quantize_q8_1
    mp.setattr(ternary, "quantize_q8_1", lambda x: orig(np.asarray(x, np.float32) * np.float32(127.0 / 128.0)))


def _subblock_off_by_one(mp):
    orig = ternary.subblock_sums

    def subblock_sums(trits, q):
        S = orig(trits, q)
        return S + (S != 0)  # off by one wherever the sum is not zero
    mp.setattr(ternary, "subblock_sums", subblock_sums)


def _sb_tail_strided(mp):
    # the stride of the PTQ1_0 sections (byte t % 13, digit t // 13) instead
    # of five consecutive tail trits per byte
    mp.setattr(ternary, "tail_position", lambda t: (t % 13, t // 13))


def _sb_pattern_3b(mp):
    # pattern index 3 * byte + digit instead of byte + 256 * digit
    mp.setattr(ternary, "pattern_fields", lambda p: (p // 3, p % 3))
    mp.setattr(ternary, "pattern_index", lambda byte, digit: 3 * byte + digit)


def _sb_mantissa_big_endian(mp):
    def mantissa_bytes(mant):
        field = 0
        for sub, m in enumerate(mant):
            field |= (int(m) & 0x3FF) << (10 * sub)
        return np.frombuffer(field.to_bytes(10, "big"), dtype=np.uint8).copy()

    def mantissas(field_bytes):
        field = int.from_bytes(bytes(np.asarray(field_bytes, dtype=np.uint8)), "big")
        return [(field >> (10 * sub)) & 0x3FF for sub in range(8)]
    mp.setattr(ternary, "mantissa_bytes", mantissa_bytes)
    mp.setattr(ternary, "mantissas", mantissas)


def _sb_ties_descending(mp):
    mp.setattr(ternary, "codebook_order",
               lambda counts: [pat for pat, _ in sorted(counts.items(), key=lambda kv: (-kv[1], tuple(-v for v in kv[0])))])


def _sb_escape_key_without_row(mp):
    mp.setattr(ternary, "superblock_index", lambda row, sb, nsb: sb)


def _pt_block_major(mp):
    # block i's eight 16-byte slots together (16 (8 i + plane) + e mod 16)
    # instead of plane-major slots
    mp.setattr(ternary, "pt_offset", lambda e, i, k: 16 * (8 * i + e // 16) + e % 16)


def _pt_ds_reversed(mp):
    # the four (d, s) pairs of a block in reverse sub-block order
    mp.setattr(ternary, "pt_ds_offset", lambda j, i, k: 16 * (8 * (k // 128) + i) + 4 * (3 - j))


CASES = {
    "int4: low nibble holds the odd k": (_swap_nibbles, _int4_pins),
    "int4: gfx950 order replaced by its inverse": (_inverse_interleave, _int4_pins),
    "int4: zero point dropped": (_drop_zero, _int4_pins),
    "int4: group index k % groups instead of k // group": (_group_by_modulo, _int4_pins),
    "int4: x reversed along k in the GEMV": (_transposed_gemv, _int4_pins),
    "int4: scale absmax / 8": (_quant_divisor_8, _int4_pins),
    "int4: quotient truncated instead of rounded to even": (_quant_truncate, _int4_pins),
    "int4: ties rounded half up instead of to even": (_quant_half_up, _int4_pins),
    "int4: divide by the scale before its bf16 rounding": (_quant_unrounded_scale, _int4_pins),
    "ternary: base-3 digit order reversed": (_digits_reversed, _ternary_pins),
    "ternary: trit sign flipped on decode": (_trit_sign_flipped, _ternary_pins),
    "ternary: weight scale paired with the wrong sub-blocks": (_weight_scale_per_32, _ternary_pins),
    "ternary: q8_1 scale amax / 128": (_q8_divisor_128, _ternary_pins),
    "ternary: sub-block sum off by one": (_subblock_off_by_one, _ternary_pins),
    "ptq1_1: tail trits strided over qh": (_sb_tail_strided, _ternary_pins),
    "ptq1_1: pattern index 3 * byte + free digit": (_sb_pattern_3b, _ternary_pins),
    "ptq1_1: mantissa field big-endian": (_sb_mantissa_big_endian, _ternary_pins),
    "ptq1_1: codebook ties by decreasing pattern": (_sb_ties_descending, _ternary_pins),
    "ptq1_1: escape table keyed by the superblock within its row": (_sb_escape_key_without_row, _ternary_pins),
    "pt: slots block-major instead of plane-major": (_pt_block_major, _ternary_pins),
    "pt: (d, s) pairs of a block in reverse order": (_pt_ds_reversed, _ternary_pins),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_pins_catch_planted_mistake(case, monkeypatch):
    plant, pins = CASES[case]
    plant(monkeypatch)
    caught = []
    for pin in pins():
        try:
            pin()
        except Exception as e:  # an assertion, or the mistake breaking a shape
            caught.append(f"{getattr(pin, '__name__', 'pin')}: {type(e).__name__}")
    assert caught, f"no pin fails with the planted mistake: {case}"


def test_pins_pass_without_a_planted_mistake():
    # the control: the same pin lists, nothing planted
    for pins in (_int4_pins, _ternary_pins):
        for pin in pins():
            pin()
