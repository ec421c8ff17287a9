"""GPU parity: int4 packing, quantise + pack and the W4 GEMV against the oracle.

Integer results (codes, packed bytes, scales) must be bit-exact; float
results meet the bars in tests/tolerances.py.  Every input comes from the
seeded generators in wq_inputs; each side packs and quantises on its own.
"""
import numpy as np
import pytest
import torch

import wq_inputs
from oracle import fpformat, int4 as o4
from tolerances import check_bf16_rows, check_f32

pytestmark = pytest.mark.gpu

G = None


def setup_module():
    global G
    import gemm_wq_quantize_amd as g
    G = g
    torch.cuda.init()


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def say(*a):
    print("[case]", *a, flush=True)


def gpu_pack(codes, layout):
    n, k = codes.shape
    out = torch.empty((n, k // 2), dtype=torch.uint8, device="cuda")
    G.wq_pack_int4(dev(codes), layout, out)
    return out


def x_dev(x_f32, x_dtype):
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if x_dtype == "bf16" else t


def scales_dev(s_f32, sdt):
    t = torch.from_numpy(np.ascontiguousarray(s_f32, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if sdt == "bf16" else t


def run_gemv(packed_dev, layout, s_dev, z_dev, zc, k, group, x_d, c, n, out_dtype):
    out = torch.empty((c, n), dtype=out_dtype, device="cuda")
    G.wq_gemv_w4(packed_dev, layout, s_dev, z_dev, zc, k, group, x_d, out)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


# ---------------------------------------------------------------- packing
@pytest.mark.parametrize("n,k", [(1, 8), (37, 264), (256, 512), (5120, 17280)])
@pytest.mark.parametrize("layout", [0, 1])
def test_pack_int4_bit_exact(n, k, layout):
    say("pack", n, k, layout)
    rng = np.random.default_rng(n + k)
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    got = gpu_pack(codes, layout).cpu().numpy()
    assert np.array_equal(got, o4.pack(codes, layout))


# ---------------------------------------------------------------- quantiser
def _quant_case(w_bits, group, sdt, layout):
    n, k = w_bits.shape
    packed = torch.empty((n, k // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((n, k // group), dtype=torch.bfloat16 if sdt == "bf16" else torch.float32,
                         device="cuda")
    G.wq_quantize_pack_int4(dev(w_bits, torch.float16), group, layout, packed, scales)
    torch.cuda.synchronize()
    codes, s_ref, bits_ref = o4.quantize_int4(w_bits, group, sdt)
    assert np.array_equal(packed.cpu().numpy(), o4.pack(codes, layout))
    if sdt == "bf16":
        got_bits = scales.view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        got_bits = scales.view(torch.int32).cpu().numpy().view(np.uint32)
    assert np.array_equal(got_bits, bits_ref)
    return packed, scales, codes, s_ref


@pytest.mark.parametrize("layout", [0, 1])
def test_quantize_tiny_per_row(layout):
    p = wq_inputs.tiny_int4()
    say("quantize tiny per-row", layout)
    _quant_case(p.w_f16, p.k, "f32", layout)


@pytest.mark.parametrize("k,n", wq_inputs.SMALL_BATCH_SHAPES)
def test_quantize_small_batch_group128(k, n):
    p = wq_inputs.small_batch_int4(k, n, cmax=1)
    say("quantize group128", k, n)
    _quant_case(p.w_f16, 128, "bf16", 1)


@pytest.mark.parametrize("group,sdt", [(32, "bf16"), (64, "f32"), (128, "f32"), (4352, "bf16")])
def test_quantize_edge_cases(group, sdt):
    rng = np.random.default_rng(group)
    n, k = 19, 4352
    w = 0.02 * rng.standard_normal((n, k))
    w[0, :group] = 0.0                     # all-zero group
    w[1, :] *= 1e-6                        # fp16 subnormal range
    w[2, :8] = [7.0, 0.5, 1.5, 2.5, -0.5, -2.5, 3.25, -6.75]  # exact ties
    w[3, 0] = 60000.0                      # large magnitudes
    w[4, :] = -w[4, :]
    say("quantize edge", group, sdt)
    _quant_case(wq_inputs.to_f16_bits(w), group, sdt, 1)


@pytest.mark.parametrize("group,k", [(32, 256), (64, 512), (256, 1024), (512, 2048), (96, 96),
                                     (1024, 1024), (2048, 2048), (4096, 4096), (4352, 4352)])
def test_quantize_every_team_shape(group, k):
    # one case per register layout of the single-pass quantiser (4, 8 or 64
    # lanes per group holding 1..8 words each; 96 = a per-row group of 12
    # words, not a multiple of the lanes) and the two-pass kernel past 512
    # words; exact ties and a zero group in every case
    rng = np.random.default_rng(group + k)
    n = 37
    w = 0.02 * rng.standard_normal((n, k))
    w[0, :min(group, k)] = 0.0
    w[1, :8] = [7.0, 0.5, 1.5, 2.5, -0.5, -2.5, 3.25, -6.75]
    w[2, -8:] = [-7.0, 3.5, -4.5, 5.5, 6.5, -1.5, 0.0, 2.0]
    say("quantize team shape", group, k)
    for sdt in ("bf16", "f32"):
        _quant_case(wq_inputs.to_f16_bits(w), group, sdt, 1)


# ---------------------------------------------------------------- GEMV
def test_gemv_tiny_per_row_fp32():
    p = wq_inputs.tiny_int4()
    for layout in (0, 1):
        say("gemv tiny", layout)
        packed = gpu_pack(p.codes, layout)
        ref = o4.gemv_w4(o4.pack(p.codes, layout), layout, p.scales, p.zeros, 0.0, p.k, p.x)
        got = run_gemv(packed, layout, scales_dev(p.scales, "f32"), scales_dev(p.zeros, "f32"),
                       0.0, p.k, p.k, x_dev(p.x, "f32"), 1, p.n, torch.float32)
        check_f32(got, ref)


def test_gemv_tiny_quantized_round_trip():
    p = wq_inputs.tiny_int4()
    say("gemv tiny quantised")
    packed, scales, codes, s_ref = _quant_case(p.w_f16, p.k, "f32", 1)
    ref = o4.gemv_w4(o4.pack(codes, 1), 1, s_ref, None, 8.0, p.k, p.x)
    got = run_gemv(packed, 1, scales, None, 8.0, p.k, p.k, x_dev(p.x, "f32"), 1, p.n, torch.float32)
    check_f32(got, ref)
    # the dequantised weights approximate the fp16 originals: out ~ W x
    wf = fpformat.f16_bits_to_f32(p.w_f16).astype(np.float64)
    approx = p.x.astype(np.float64) @ wf.T
    assert np.sqrt(np.mean((got - approx) ** 2)) < 0.2 * np.sqrt(np.mean(approx ** 2))


@pytest.mark.parametrize("k,n", wq_inputs.DECODE_SHAPES)
def test_gemv_decode_shapes(k, n):
    p = wq_inputs.decode_int4(k, n, cmax=4)
    packed = gpu_pack(p.codes, 1)
    s_d = dev(p.scale_bits, torch.bfloat16)
    xb = dev(p.x_bits, torch.bfloat16)
    ref_all = o4.gemv_w4(o4.pack(p.codes, 1), 1, p.scales, None, 8.0, 128, p.x)
    for c in (1, 2, 4):
        say("gemv decode", k, n, c)
        got = run_gemv(packed, 1, s_d, None, 8.0, k, 128, xb[:c].contiguous(), c, n, torch.bfloat16)
        check_bf16_rows(got, ref_all[:c])


@pytest.mark.parametrize("k,n", wq_inputs.SMALL_BATCH_SHAPES)
def test_gemv_small_batch(k, n):
    p = wq_inputs.small_batch_int4(k, n, cmax=32)
    packed, scales, codes, s_ref = _quant_case(p.w_f16, 128, "bf16", 1)
    xb = dev(p.x_bits, torch.bfloat16)
    ref_all = o4.gemv_w4(o4.pack(codes, 1), 1, s_ref, None, 8.0, 128, p.x)
    for c in (8, 16, 32):
        say("gemv small batch", k, n, c)
        got = run_gemv(packed, 1, scales, None, 8.0, k, 128, xb[:c].contiguous(), c, n, torch.bfloat16)
        check_bf16_rows(got, ref_all[:c])


RAGGED = [
    # n, k, group, c, x dtype, scale dtype, zeros, out dtype, layout
    (1001, 1056, 32, 1, "bf16", "bf16", False, torch.float32, 1),
    (77, 4224, 128, 3, "bf16", "f32", True, torch.bfloat16, 1),
    (5, 2080, 2080, 5, "f32", "f32", True, torch.float32, 0),
    (300, 1024, 64, 17, "bf16", "bf16", True, torch.float32, 0),
    (9, 33792, 128, 32, "bf16", "bf16", False, torch.bfloat16, 1),
    (260, 96, 32, 2, "f32", "bf16", False, torch.float32, 1),
    (1, 32, 32, 1, "f32", "f32", False, torch.float32, 1),
    (515, 2048, 2048, 12, "f32", "f32", True, torch.float32, 1),
    (2050, 4160, 4160, 6, "bf16", "f32", True, torch.bfloat16, 1),
    (33, 2080, 32, 9, "bf16", "f32", False, torch.float32, 0),
]


@pytest.mark.parametrize("case", RAGGED, ids=[f"n{c[0]}k{c[1]}g{c[2]}c{c[3]}" for c in RAGGED])
def test_gemv_ragged_and_dtypes(case):
    n, k, group, c, xdt, sdt, with_z, odt, layout = case
    say("gemv ragged", case)
    rng = np.random.default_rng(n * 7 + k)
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    s = rng.uniform(0.002, 0.02, (n, k // group)).astype(np.float32)
    if sdt == "bf16":
        s = fpformat.bf16_bits_to_f32(fpformat.f32_to_bf16_bits(s))
    z = rng.uniform(6, 9, (n, k // group)).astype(np.float32) if with_z else None
    if z is not None and sdt == "bf16":
        z = fpformat.bf16_bits_to_f32(fpformat.f32_to_bf16_bits(z))
    x = rng.standard_normal((c, k)).astype(np.float32)
    if xdt == "bf16":
        x = fpformat.bf16_bits_to_f32(fpformat.f32_to_bf16_bits(x))
    ref = o4.gemv_w4(o4.pack(codes, layout), layout, s, z, 8.0, group, x)
    got = run_gemv(gpu_pack(codes, layout), layout, scales_dev(s, sdt),
                   None if z is None else scales_dev(z, sdt), 8.0, k, group, x_dev(x, xdt), c, n, odt)
    if odt == torch.float32:
        check_f32(got, ref)
    else:
        check_bf16_rows(got, ref)


# One case per launch path of wq_gemv_w4 that the workloads above do not
# reach.  bf16 x: the matrix-core kernel at c = 4 past the quad kernel's LDS
# (K = 28672), on plain-layout weights (1 and 2 blocks of 16 columns, stored
# zeros, fp32 scales) and on one group per row whose K is not a multiple of
# 128 (a partial last item); the quad kernel on plain-layout weights with
# stored zeros (groups of 128 and 64 k); with groups of 64 k, which the
# matrix-core kernel leaves to the others, the streaming kernel when x is
# too large for the quad kernel's LDS (c = 3 and 4 at K = 28672).  fp32 x:
# N >= 16384 (two rows per half-wave) and c > 16 (passes of 16).
PATHS = [
    # n, k, group, c, x dtype, scale dtype, zeros, out dtype, layout
    (2048, 28672, 128, 4, "bf16", "bf16", False, torch.bfloat16, 1),
    (500, 2048, 128, 2, "bf16", "bf16", True, torch.bfloat16, 0),
    (777, 2048, 128, 16, "bf16", "f32", True, torch.float32, 0),
    (1000, 1024, 256, 20, "bf16", "bf16", True, torch.bfloat16, 0),
    (333, 160, 160, 5, "bf16", "f32", False, torch.float32, 1),
    (500, 2048, 64, 2, "bf16", "bf16", True, torch.bfloat16, 0),
    (2048, 28672, 64, 3, "bf16", "bf16", False, torch.bfloat16, 1),
    (2048, 28672, 64, 4, "bf16", "f32", False, torch.float32, 1),
    (16400, 1024, 128, 3, "f32", "f32", False, torch.float32, 1),
    (16400, 1024, 64, 8, "f32", "bf16", True, torch.float32, 0),
    (300, 1024, 64, 24, "f32", "f32", True, torch.float32, 1),
    (131, 2048, 2048, 32, "f32", "bf16", False, torch.bfloat16, 1),
]


@pytest.mark.parametrize("case", PATHS, ids=[f"n{c[0]}k{c[1]}g{c[2]}c{c[3]}{c[4]}l{c[8]}" for c in PATHS])
def test_gemv_launch_paths(case):
    test_gemv_ragged_and_dtypes(case)


@pytest.mark.parametrize("xdt,c", [("bf16", 4), ("f32", 4), ("bf16", 16)])
def test_gemv_integer_exact(xdt, c):
    say("gemv integer exact", xdt, c)
    rng = np.random.default_rng(21)
    n, k = 700, 5120
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    x = rng.integers(-2, 3, (c, k)).astype(np.float32)
    exact = x.astype(np.int64) @ (codes.astype(np.int64) - 8).T
    ones = np.ones((n, k // 128), np.float32)
    packed = gpu_pack(codes, 1)
    got = run_gemv(packed, 1, scales_dev(ones, "bf16"), None, 8.0, k, 128, x_dev(x, xdt), c, n,
                   torch.float32)
    assert np.array_equal(got, exact.astype(np.float64))
    got = run_gemv(packed, 1, scales_dev(ones, "bf16"), None, 8.0, k, 128, x_dev(x, xdt), c, n,
                   torch.bfloat16)
    want = fpformat.bf16_bits_to_f32(fpformat.f32_to_bf16_bits(exact.astype(np.float32)))
    assert np.array_equal(got, want.astype(np.float64))


def test_gemv_closed_forms():
    say("gemv one-hot / zero codes")
    n, k = 64, 1024
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    s = rng.uniform(0.01, 0.1, (n, k // 128)).astype(np.float32)
    x = np.zeros((3, k), np.float32)
    x[0, 0] = 1.0; x[1, 517] = 1.0; x[2, 1023] = 1.0
    got = run_gemv(gpu_pack(codes, 1), 1, scales_dev(s, "f32"), None, 8.0, k, 128,
                   x_dev(x, "bf16"), 3, n, torch.float32)
    for j, kk in enumerate((0, 517, 1023)):
        want = (codes[:, kk].astype(np.float32) - 8) * s[:, kk // 128]
        assert np.array_equal(got[j], want.astype(np.float64))
    # codes equal to the zero point: 0 up to the float32 rounding of the
    # offset fold sum (128 + q) x - 136 sum x (bounded by 2^-16 * 143 * s * sum|x|)
    zcodes = np.full((n, k), 8, np.uint8)
    xz = fpformat.bf16_bits_to_f32(fpformat.f32_to_bf16_bits(rng.standard_normal((2, k))))
    got = run_gemv(gpu_pack(zcodes, 1), 1, scales_dev(s, "f32"), None, 8.0, k, 128,
                   x_dev(xz, "bf16"), 2, n, torch.float32)
    bound = 2.0 ** -16 * 143 * s.max() * np.abs(xz).sum(axis=1, keepdims=True)
    assert np.all(np.abs(got) <= bound)


@pytest.mark.parametrize("k,n,c", [(5120, 4096, 4), (5120, 4096, 8), (4096, 11008, 8),
                                   (4096, 4096, 16), (5120, 1000, 32)])
def test_gemv_repeatable(k, n, c):
    # fixed-order sums in every path: the persistent decode kernel (c <= 4)
    # and the wide-batch kernel in each of its forms (x staged once or per
    # tile, one or two column sets) give the same bits on every call
    say("gemv bitwise repeatable", k, n, c)
    p = wq_inputs.decode_int4(k, n, cmax=c, seed=3)
    packed = gpu_pack(p.codes, 1)
    s_d = dev(p.scale_bits, torch.bfloat16)
    xb = dev(p.x_bits, torch.bfloat16)
    outs = []
    for _ in range(3):
        out = torch.empty((c, n), dtype=torch.float32, device="cuda")
        G.wq_gemv_w4(packed, 1, s_d, None, 8.0, k, 128, xb, out)
        outs.append(out.cpu().numpy().copy())
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_gemv_rejects_bad_arguments():
    say("gemv argument errors")
    packed = torch.zeros((8, 64), dtype=torch.uint8, device="cuda")
    s = torch.ones((8, 1), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((33, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full((33, 8), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(G.WqError) as e:
        G.wq_gemv_w4(packed, 1, s, None, 8.0, 128, 128, x, out)
    assert e.value.status == G.WQ_ESHAPE
    assert torch.all(out == 7.0)
