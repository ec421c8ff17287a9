"""GPU parity: the W4A16 MFMA GEMM against the oracle."""
import numpy as np
import pytest
import torch

import wq_inputs
from oracle import fpformat, int4 as o4
from tolerances import check_bf16_rownorm, check_bf16_rows

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def G():
    import gemm_wq_quantize_amd as g
    return g


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).cuda()


def run(a_bits, codes, scale_bits, zc=8.0, group=None):
    g = G()
    m, k = a_bits.shape
    n = codes.shape[0]
    b = torch.empty((n, k // 2), dtype=torch.uint8, device="cuda")
    g.wq_pack_int4(torch.from_numpy(codes).cuda(), 1, b)
    c = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    g.wq_gemm_w4a16(bf16_dev(a_bits), b, 1, bf16_dev(scale_bits), group or k, zc, c)
    torch.cuda.synchronize()
    return c


@pytest.mark.parametrize("m,n,k", [(300, 520, 512), (256, 256, 64), (64, 8, 128), (1, 1000, 192),
                                   (513, 257, 1088), (320, 640, 256), (200, 300, 704)])
def test_gemm_ragged(m, n, k):
    say("gemm", m, n, k)
    p = wq_inputs.large_gemm(m, n, k, n_rows=m, seed=m + n)
    c = run(p.a_bits, p.codes, p.scale_bits).float().cpu().numpy()
    a = fpformat.bf16_bits_to_f32(p.a_bits)
    s = fpformat.bf16_bits_to_f32(p.scale_bits).reshape(n, 1)
    ref = o4.gemm_w4a16_rows(a, o4.pack(p.codes, 1), 1, s, 8.0, k)
    check_bf16_rows(c, ref)


def test_gemm_integer_exact():
    say("gemm integer exact")
    rng = np.random.default_rng(4)
    m, n, k = 320, 384, 1024
    a = rng.integers(-4, 5, (m, k)).astype(np.float32)
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    ones = fpformat.f32_to_bf16_bits(np.ones(n, np.float32))
    c = run(fpformat.f32_to_bf16_bits(a), codes, ones)
    exact = a.astype(np.int64) @ (codes.astype(np.int64) - 8).T
    want = fpformat.f32_to_bf16_bits(exact.astype(np.float32))
    assert np.array_equal(c.view(torch.int16).cpu().numpy().view(np.uint16), want)


def test_gemm_zero_point_other_than_8():
    say("gemm zero point 5")
    rng = np.random.default_rng(6)
    m, n, k = 128, 256, 256
    a = rng.integers(-3, 4, (m, k)).astype(np.float32)
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    ones = fpformat.f32_to_bf16_bits(np.ones(n, np.float32))
    c = run(fpformat.f32_to_bf16_bits(a), codes, ones, zc=5.0)
    exact = a.astype(np.int64) @ (codes.astype(np.int64) - 5).T
    want = fpformat.f32_to_bf16_bits(exact.astype(np.float32))
    assert np.array_equal(c.view(torch.int16).cpu().numpy().view(np.uint16), want)


def test_gemm_8192_sampled_rows():
    p = wq_inputs.large_gemm()
    say("gemm 8192^3, sampled rows", len(p.rows))
    c = run(p.a_bits, p.codes, p.scale_bits)
    rows = torch.from_numpy(p.rows).cuda()
    got = c.index_select(0, rows).float().cpu().numpy()
    a = fpformat.bf16_bits_to_f32(p.a_bits[p.rows])
    s = fpformat.bf16_bits_to_f32(p.scale_bits).reshape(-1, 1)
    ref = o4.gemm_w4a16_rows(a, o4.pack(p.codes, 1), 1, s, 8.0, p.k)
    check_bf16_rows(got, ref)
    # every other row: finite and of the expected magnitude (property at any size)
    allc = c.float()
    assert torch.isfinite(allc).all()
    rms = allc.pow(2).mean(dim=1).sqrt().cpu().numpy()
    expect = float(np.sqrt(np.mean(ref ** 2)))
    assert np.all(np.abs(rms / expect - 1) < 0.1)


def test_gemm_8192_group128_sampled_rows():
    # the timed group-scale workload (8192^3, group 128) checked on a seeded
    # sample of 128 output rows
    p = wq_inputs.grouped_gemm(8192, 8192, 8192, 128, seed=3)
    rows = np.sort(np.random.default_rng(3).choice(8192, 128, replace=False))
    say("gemm 8192^3 group 128, sampled rows", len(rows))
    c = run(p.a_bits, p.codes, p.scale_bits, group=128)
    got = c.index_select(0, torch.from_numpy(rows).cuda()).float().cpu().numpy()
    a = fpformat.bf16_bits_to_f32(p.a_bits[rows])
    s = fpformat.bf16_bits_to_f32(p.scale_bits)
    packed = o4.pack(p.codes, 1)
    check_bf16_rows(got, o4.gemm_w4a16_rows_bf16w(a, packed, 1, s, 8.0, 128))
    # and against the plain product (no rounding of the weights), normwise
    check_bf16_rownorm(got, o4.gemm_w4a16_rows(a, packed, 1, s, 8.0, 128))
    assert torch.isfinite(c.float()).all()


# ---- group scales ([N][K/group] bf16; each weight rounded to bf16 before the
# multiply, as the oracle's ``gemm_w4a16_rows_bf16w`` states)
@pytest.mark.parametrize("m,n,k,group", [(300, 520, 512, 128), (256, 256, 256, 64),
                                         (129, 333, 1152, 128), (200, 300, 704, 64),
                                         (513, 257, 2048, 256), (64, 1000, 1024, 512)])
def test_gemm_group_scales(m, n, k, group):
    # (129, 333, 1152): 9 groups and 333 columns, an odd number of scales,
    # so the last scale sits in the low half of a word that ends past the array
    say("gemm group scales", m, n, k, group)
    p = wq_inputs.grouped_gemm(m, n, k, group, seed=m + n)
    c = run(p.a_bits, p.codes, p.scale_bits, group=group).float().cpu().numpy()
    a = fpformat.bf16_bits_to_f32(p.a_bits)
    s = fpformat.bf16_bits_to_f32(p.scale_bits)
    packed = o4.pack(p.codes, 1)
    check_bf16_rows(c, o4.gemm_w4a16_rows_bf16w(a, packed, 1, s, 8.0, group))
    check_bf16_rownorm(c, o4.gemm_w4a16_rows(a, packed, 1, s, 8.0, group))


@pytest.mark.parametrize("zc", [8.0, 7.5, -3.25, 0.0])
def test_gemm_group_scales_integer_exact(zc):
    # power-of-two scales that change per group: every weight is exact in
    # bf16 and every partial sum a multiple of 1/8 below 2^21, so C must be
    # the RNE bf16 of the exact sum; taking a scale from the wrong group or
    # the wrong half of a scale word changes the result.  Constant zeros that
    # are multiples of 1/32 (integer, half-integer, negative, zero) take the
    # fp16-magic dequantisation.
    say("gemm group scales, integer exact, zero", zc)
    rng = np.random.default_rng(14)
    m, n, k, group = 256, 264, 1408, 128
    a = rng.integers(-4, 5, (m, k)).astype(np.float32)
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    e = rng.integers(-2, 3, (n, k // group))
    s_bits = fpformat.f32_to_bf16_bits((2.0 ** e).astype(np.float32))
    c = run(fpformat.f32_to_bf16_bits(a), codes, s_bits, zc=zc, group=group)
    w = (codes.astype(np.float64) - zc) * np.repeat(2.0 ** e, group, axis=1)
    exact = a.astype(np.float64) @ w.T
    want = fpformat.f32_to_bf16_bits(exact.astype(np.float32))
    assert np.array_equal(c.view(torch.int16).cpu().numpy().view(np.uint16), want)


@pytest.mark.parametrize("zc", [7.3, 0.1, 1500.0])
@pytest.mark.parametrize("m,n,k,group", [(300, 520, 512, 128), (129, 333, 1152, 64)])
def test_gemm_group_scales_any_zero(m, n, k, group, zc):
    # constant zeros that are not multiples of 1/32 below 1024 keep the
    # float32 code convert and one FMA per weight; zc is the float32 the
    # entry point receives.  For 7.3f and 0.1f, z * s is not exact in float32,
    # so a weight can sit one bf16 ulp from bf16_rne((q - z) * s): the bar is
    # the bf16 one, 1e-2 of the row norm of the exact product.  1500 is an
    # integer (the weights are exact before their bf16 rounding), and with
    # every weight near -1500 s that rounding alone is about 1% of the row
    # norm, so it is held to the elementwise bound against the rounded weights
    say("gemm group scales, zero", m, n, k, group, zc)
    zc = float(np.float32(zc))
    p = wq_inputs.grouped_gemm(m, n, k, group, seed=m + n + 2)
    c = run(p.a_bits, p.codes, p.scale_bits, zc=zc, group=group).float().cpu().numpy()
    a = fpformat.bf16_bits_to_f32(p.a_bits)
    s = fpformat.bf16_bits_to_f32(p.scale_bits)
    packed = o4.pack(p.codes, 1)
    if zc == int(zc):
        check_bf16_rows(c, o4.gemm_w4a16_rows_bf16w(a, packed, 1, s, zc, group))
    else:
        check_bf16_rownorm(c, o4.gemm_w4a16_rows(a, packed, 1, s, zc, group))


def test_gemm_on_quantiser_output():
    # the quantiser's group-128 output (codes and bf16 scales) feeds the GEMM
    # directly; the oracle quantises the same fp16 weights itself
    say("gemm on wq_quantize_pack_int4 output, 64 x 4096 x 11008")
    g = G()
    m, n, k = 64, 4096, 11008
    rng = np.random.default_rng(15)
    w16 = wq_inputs.to_f16_bits(0.02 * rng.standard_normal((n, k), dtype=np.float32))
    a_bits = wq_inputs.to_bf16_bits(rng.standard_normal((m, k), dtype=np.float32))
    packed = torch.empty((n, k // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((n, k // 128), dtype=torch.bfloat16, device="cuda")
    g.wq_quantize_pack_int4(torch.from_numpy(w16).view(torch.float16).cuda(), 128, 1, packed, scales)
    c = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    g.wq_gemm_w4a16(bf16_dev(a_bits), packed, 1, scales, 128, 8.0, c)
    torch.cuda.synchronize()
    codes, s, _ = o4.quantize_int4(w16, 128, "bf16")
    assert np.array_equal(packed.cpu().numpy(), o4.pack(codes, 1))
    a = fpformat.bf16_bits_to_f32(a_bits)
    got = c.float().cpu().numpy()
    packed_ref = o4.pack(codes, 1)
    check_bf16_rows(got, o4.gemm_w4a16_rows_bf16w(a, packed_ref, 1, s, 8.0, 128))
    check_bf16_rownorm(got, o4.gemm_w4a16_rows(a, packed_ref, 1, s, 8.0, 128))


# ---- stored zero points (wq_gemm_w4a16_zp)
def run_zp(a_bits, codes, scale_bits, zero_bits, group):
    g = G()
    m, k = a_bits.shape
    n = codes.shape[0]
    b = torch.empty((n, k // 2), dtype=torch.uint8, device="cuda")
    g.wq_pack_int4(torch.from_numpy(codes).cuda(), 1, b)
    c = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    g.wq_gemm_w4a16_zp(bf16_dev(a_bits), b, 1, bf16_dev(scale_bits), bf16_dev(zero_bits), group, c)
    torch.cuda.synchronize()
    return c


@pytest.mark.parametrize("m,n,k,group", [(300, 520, 512, 128), (129, 333, 1152, 128),
                                         (256, 200, 704, 704), (64, 1000, 2048, 2048)])
def test_gemm_stored_zeros(m, n, k, group):
    # zeros bf16 U(6, 9) of the scales' shape: group scales (weights rounded
    # once to bf16) and one scale and zero per column (folded exactly)
    say("gemm stored zeros", m, n, k, group)
    p = wq_inputs.grouped_gemm(m, n, k, group, seed=m + n + 1)
    rng = np.random.default_rng(m + k)
    z_bits = fpformat.f32_to_bf16_bits(rng.uniform(6, 9, p.scale_bits.shape).astype(np.float32))
    c = run_zp(p.a_bits, p.codes, p.scale_bits, z_bits, group).float().cpu().numpy()
    a = fpformat.bf16_bits_to_f32(p.a_bits)
    s = fpformat.bf16_bits_to_f32(p.scale_bits).reshape(n, k // group)
    z = fpformat.bf16_bits_to_f32(z_bits).reshape(n, k // group)
    packed = o4.pack(p.codes, 1)
    exact = o4.gemm_w4a16_rows(a, packed, 1, s, 8.0, group, zeros=z)
    if group == k:
        check_bf16_rows(c, exact)
    else:
        check_bf16_rows(c, o4.gemm_w4a16_rows_bf16w(a, packed, 1, s, 8.0, group, zeros=z))
        check_bf16_rownorm(c, exact)


@pytest.mark.parametrize("group", [128, 1024])
def test_gemm_stored_zeros_integer_exact(group):
    # integer zeros 3..12 and power-of-two scales per group (or per column):
    # exact weights and sums, so C is the RNE bf16 of the exact product
    say("gemm stored zeros, integer exact", group)
    rng = np.random.default_rng(17 + group)
    m, n, k = 192, 264, 1024
    a = rng.integers(-4, 5, (m, k)).astype(np.float32)
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    e = rng.integers(-2, 3, (n, k // group))
    zi = rng.integers(3, 13, (n, k // group))
    c = run_zp(fpformat.f32_to_bf16_bits(a), codes,
               fpformat.f32_to_bf16_bits((2.0 ** e).astype(np.float32)),
               fpformat.f32_to_bf16_bits(zi.astype(np.float32)), group)
    w = (codes.astype(np.float64) - np.repeat(zi, group, axis=1)) * np.repeat(2.0 ** e, group, axis=1)
    want = fpformat.f32_to_bf16_bits((a.astype(np.float64) @ w.T).astype(np.float32))
    assert np.array_equal(c.view(torch.int16).cpu().numpy().view(np.uint16), want)


def test_gemm_repeatable():
    # every output is summed by one wave in a fixed order: bitwise repeatable,
    # with one scale per column and with group scales
    say("gemm bitwise repeatable")
    p = wq_inputs.grouped_gemm(512, 768, 2048, 128, seed=21)
    for group, sbits in ((2048, p.scale_bits[:, :1].copy()), (128, p.scale_bits)):
        outs = [run(p.a_bits, p.codes, sbits, group=group).view(torch.int16).cpu().numpy()
                for _ in range(3)]
        assert all(np.array_equal(outs[0], o) for o in outs[1:]), group
