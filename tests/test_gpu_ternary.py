"""GPU parity: PTQ1_0 packing, q8_1 quantiser and the ternary GEMV."""
import numpy as np
import pytest
import torch

import wq_inputs
from oracle import ternary as ot
from tolerances import check_f32

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def G():
    import gemm_wq_quantize_amd as g
    return g


def gpu_blocks(trits, d_bits):
    n, k = trits.shape
    out = torch.empty((n, k // 128, 28), dtype=torch.uint8, device="cuda")
    G().wq_pack_ptq1_0(torch.from_numpy(trits).cuda(),
                       torch.from_numpy(d_bits).view(torch.int16).cuda(), out)
    return out


def gpu_q8(x):
    c, k = x.shape
    out = torch.empty((c, k // 32, 36), dtype=torch.uint8, device="cuda")
    G().wq_quantize_q8_1(torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda(), out)
    return out


def gpu_gemv(wb, xq, k):
    n, c = wb.shape[0], xq.shape[0]
    out = torch.empty((c, n), dtype=torch.float32, device="cuda")
    G().wq_gemv_ternary(wb, xq, k, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("n,k", [(1, 128), (33, 1024), (17280, 5120)])
def test_pack_ptq1_0_bit_exact(n, k):
    say("ptq1_0 pack", n, k)
    p = wq_inputs.ternary_gemv(k, n, cmax=1, seed=n)
    got = gpu_blocks(p.trits, p.d_bits).cpu().numpy()
    assert np.array_equal(got, ot.encode_ptq1_0(p.trits, p.d_bits))


@pytest.mark.parametrize("c,k", [(1, 32), (3, 4096), (8, 5120)])
def test_quantize_q8_1_bit_exact(c, k):
    say("q8_1", c, k)
    rng = np.random.default_rng(c * k)
    x = rng.standard_normal((c, k)).astype(np.float32)
    x[0, :32] = 0.0                                   # zero block
    if k >= 64:
        x[0, 32:64] = np.arange(32) - 15.5            # ties at d = 16/127...
    assert np.array_equal(gpu_q8(x).cpu().numpy(), ot.quantize_q8_1(x))


@pytest.mark.parametrize("k,n", [(5120, 17280), (17280, 1000), (384, 77)])
def test_ternary_gemv(k, n):
    p = wq_inputs.ternary_gemv(k, n, cmax=16)
    wb = gpu_blocks(p.trits, p.d_bits)
    wref = ot.encode_ptq1_0(p.trits, p.d_bits)
    cs = (1, 2, 4, 8) if k == 5120 else (1, 3, 5, 16)
    for c in cs:
        say("ternary gemv", k, n, c)
        xq = gpu_q8(p.x[:c])
        xref = ot.quantize_q8_1(p.x[:c])
        assert np.array_equal(xq.cpu().numpy(), xref)
        check_f32(gpu_gemv(wb, xq, k), ot.gemv_ternary(wref, xref))


@pytest.mark.parametrize("k,n,c", [(5120, 4000, 8), (17280, 300, 8), (5120, 4000, 1), (384, 77, 1),
                                   (17280, 300, 1), (65536, 40, 1), (17280, 300, 6), (12288, 300, 8),
                                   (24576, 200, 3)])
def test_ternary_unit_scale_exact(k, n, c):
    # one column: the kernel that splits each row's blocks between two
    # waves (k = 384: three blocks, so the second wave of a row has none);
    # 8 columns: the matrix-core kernel where x and its digit table fit in
    # LDS (k = 5120), past it the persistent vector kernel (k = 12288; and
    # 3 columns at k = 24576), past that the tiled vector kernel (8 and 6
    # columns at k = 17280)
    say("ternary unit scale", k, n, c)
    p = wq_inputs.ternary_gemv(k, n, cmax=8, unit_scale=True)
    wb = gpu_blocks(p.trits, p.d_bits)
    xq = gpu_q8(p.x[:c])
    got = gpu_gemv(wb, xq, k)
    exact = p.x[:c].astype(np.int64) @ p.trits.astype(np.int64).T
    assert np.array_equal(got, exact.astype(np.float64))


def test_ternary_special_cases():
    say("ternary all-zero / all-one trits")
    k, n = 1024, 40
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, k)).astype(np.float32)
    d = wq_inputs.to_f16_bits(rng.uniform(0.01, 0.05, (n, k // 128)))
    xq = gpu_q8(x)
    xref = ot.quantize_q8_1(x)
    for t in (np.zeros((n, k), np.int8), np.ones((n, k), np.int8), -np.ones((n, k), np.int8)):
        got = gpu_gemv(gpu_blocks(t, d), xq, k)
        ref = ot.gemv_ternary(ot.encode_ptq1_0(t, d), xref)
        if not t.any():
            assert np.all(got == 0)
        else:
            check_f32(got, ref)


@pytest.mark.parametrize("k,n,c", [(1024, 300, 24), (5120, 2000, 40), (384, 77, 63)])
def test_ternary_gemv_passes_of_16(k, n, c):
    # 17..63 columns run as passes of at most 16 columns (the last one ragged)
    say("ternary gemv in passes", k, n, c)
    p = wq_inputs.ternary_gemv(k, n, cmax=c, seed=c + k)
    wb = gpu_blocks(p.trits, p.d_bits)
    xq = gpu_q8(p.x)
    xref = ot.quantize_q8_1(p.x)
    assert np.array_equal(xq.cpu().numpy(), xref)
    check_f32(gpu_gemv(wb, xq, k), ot.gemv_ternary(ot.encode_ptq1_0(p.trits, p.d_bits), xref))
    u = wq_inputs.ternary_gemv(k, n, cmax=c, seed=c, unit_scale=True)
    got = gpu_gemv(gpu_blocks(u.trits, u.d_bits), gpu_q8(u.x), k)
    exact = u.x.astype(np.int64) @ u.trits.astype(np.int64).T
    assert np.array_equal(got, exact.astype(np.float64))


# ---- 64 or more columns: the fp4 x fp8 matrix-core kernel on unpacked operands
@pytest.mark.parametrize("k,n,c", [(1024, 256, 64), (640, 333, 200), (5120, 2048, 128),
                                   (384, 77, 130)])
def test_ternary_gemm(k, n, c):
    # ragged tiles in both directions; n = 333 and 77 take the scalar stores
    say("ternary gemm", k, n, c)
    p = wq_inputs.ternary_gemv(k, n, cmax=c, seed=c + n)
    wb = gpu_blocks(p.trits, p.d_bits)
    xq = gpu_q8(p.x)
    xref = ot.quantize_q8_1(p.x)
    assert np.array_equal(xq.cpu().numpy(), xref)
    check_f32(gpu_gemv(wb, xq, k), ot.gemv_ternary(ot.encode_ptq1_0(p.trits, p.d_bits), xref))


def test_ternary_gemm_timed_shape_sampled_columns():
    # the timed matrix-core workload (K=5120, N=17280, 4096 columns), checked
    # on a seeded sample of 8 columns against the oracle, the rest finite
    k, n, c = 5120, 17280, 4096
    say("ternary gemm", k, n, c, "sampled columns")
    p = wq_inputs.ternary_gemv(k, n, cmax=c, seed=11)
    wb = gpu_blocks(p.trits, p.d_bits)
    xq = gpu_q8(p.x)
    got = gpu_gemv(wb, xq, k)
    cols = np.sort(np.random.default_rng(11).choice(c, 8, replace=False))
    xref = ot.quantize_q8_1(p.x[cols])
    assert np.array_equal(xq.cpu().numpy()[cols], xref)
    check_f32(got[cols], ot.gemv_ternary(ot.encode_ptq1_0(p.trits, p.d_bits), xref))
    assert np.isfinite(got).all()


@pytest.mark.parametrize("k,n,c", [(1024, 300, 64), (5120, 200, 129)])
def test_ternary_gemm_unit_scale_exact(k, n, c):
    # unit scales and integer x (a +-127 in every block): the products' sums
    # (exact integers in float32) and the scaled sums are exact, so the result
    # is the integer product bit for bit
    say("ternary gemm unit scale", k, n, c)
    p = wq_inputs.ternary_gemv(k, n, cmax=c, unit_scale=True)
    wb = gpu_blocks(p.trits, p.d_bits)
    got = gpu_gemv(wb, gpu_q8(p.x), k)
    exact = p.x.astype(np.int64) @ p.trits.astype(np.int64).T
    assert np.array_equal(got, exact.astype(np.float64))


@pytest.mark.parametrize("c", [1, 4, 8, 96])
def test_ternary_repeatable(c):
    # fixed-order sums in every path (the split row groups of one column, the
    # persistent kernel, the matrix-core kernel): bitwise repeatable
    say("ternary bitwise repeatable", c)
    p = wq_inputs.ternary_gemv(5120, 2000, cmax=c, seed=5)
    wb = gpu_blocks(p.trits, p.d_bits)
    xq = gpu_q8(p.x)
    outs = [gpu_gemv(wb, xq, 5120) for _ in range(3)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
