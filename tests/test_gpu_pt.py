"""GPU parity: activations in the PT plane layout (Ternary post, section 3.1).

The quantiser's PT output must be the oracle's PT arrangement of the oracle's
q8_1 blocks, byte for byte; the GEMVs that read x in the PT layout must give
the same bits as the same kernels reading the blocks in record order, and
agree with the oracle.  The shapes reach every kernel that stages x: the
K-split kernel (one column), the matrix-core kernel (2..8 columns while x
and its 62 KiB digit table fit in LDS), the persistent vector kernel (x past
that but within its own LDS: k = 12288 at 8 columns, 24576 at 4), the tiled
vector kernel (x past every staging kernel's LDS, or 9..16 columns), passes
of 16 columns, and the matrix-core GEMM (64 columns or more)."""
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


def quantise(x, pt):
    c, k = x.shape
    xs = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    if pt:
        out = torch.empty((c, 9 * k // 8), dtype=torch.uint8, device="cuda")
        G().wq_quantize_q8_1_pt(xs, out)
    else:
        out = torch.empty((c, k // 32, 36), dtype=torch.uint8, device="cuda")
        G().wq_quantize_q8_1(xs, out)
    return out


def run(fn, *args, n, c):
    out = torch.empty((c, n), dtype=torch.float32, device="cuda")
    fn(*args, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("c,k", [(1, 128), (3, 5120), (8, 17280), (2, 131072)])
def test_quantize_q8_1_pt_bit_exact(c, k):
    say("q8_1 pt", c, k)
    rng = np.random.default_rng(c + k)
    x = rng.standard_normal((c, k)).astype(np.float32)
    x[0, :32] = 0.0                                   # zero block
    if k >= 128:
        x[-1, 96:128] = np.arange(32) - 15.5          # ties
    want = ot.q8_1_to_pt(ot.quantize_q8_1(x))
    assert np.array_equal(quantise(x, True).cpu().numpy(), want)


@pytest.mark.parametrize("k,n,c", [(5120, 1000, 1), (5120, 1000, 3), (5120, 1000, 8), (12288, 300, 8),
                                   (24576, 200, 4), (17280, 300, 8), (17280, 300, 16), (131072, 40, 1),
                                   (5120, 500, 40), (1024, 256, 96), (384, 77, 130)])
def test_gemv_ternary_pt_matches_rows(k, n, c):
    say("ternary gemv pt", k, n, c)
    p = wq_inputs.ternary_gemv(k, n, cmax=c, seed=k + c)
    blocks = ot.encode_ptq1_0(p.trits, p.d_bits)
    wb = torch.from_numpy(blocks).cuda()
    rows, pt = quantise(p.x, False), quantise(p.x, True)
    xref = ot.quantize_q8_1(p.x)
    assert np.array_equal(pt.cpu().numpy(), ot.q8_1_to_pt(xref))
    got_rows = run(G().wq_gemv_ternary, wb, rows, k, n=n, c=c)
    got_pt = run(G().wq_gemv_ternary_pt, wb, pt, k, n=n, c=c)
    assert np.array_equal(got_pt, got_rows)
    check_f32(got_pt, ot.gemv_ternary(blocks, xref))


def test_gemv_ternary_pt_unit_scale_exact():
    # unit scales: the results are the exact integer products
    k, n, c = 5120, 700, 4
    say("ternary gemv pt unit scale", k, n, c)
    p = wq_inputs.ternary_gemv(k, n, cmax=c, unit_scale=True)
    wb = torch.from_numpy(ot.encode_ptq1_0(p.trits, p.d_bits)).cuda()
    got = run(G().wq_gemv_ternary_pt, wb, quantise(p.x, True), k, n=n, c=c)
    exact = p.x.astype(np.int64) @ p.trits.astype(np.int64).T
    assert np.array_equal(got, exact.astype(np.float64))


@pytest.mark.parametrize("k,n,c", [(5120, 500, 1), (5120, 500, 4), (5120, 500, 8), (10240, 100, 8),
                                   (65536, 24, 1), (16384, 40, 13), (5120, 333, 96)])
def test_gemv_ternary_ptq1_1_pt_matches_rows(k, n, c):
    say("ptq1_1 gemv pt", k, n, c)
    p = wq_inputs.ternary_correlated_scales(k, n, cmax=c)
    blocks = ot.encode_ptq1_0(p.trits, p.d_bits)
    sup, book, ei, ep = G().wq_ptq1_1_encode(blocks)
    dev = [torch.from_numpy(a).cuda() for a in (sup, book, ei, ep)]
    rows, pt = quantise(p.x, False), quantise(p.x, True)
    got_rows = run(G().wq_gemv_ternary_ptq1_1, *dev, rows, k, n=n, c=c)
    got_pt = run(G().wq_gemv_ternary_ptq1_1_pt, *dev, pt, k, n=n, c=c)
    assert np.array_equal(got_pt, got_rows)
    check_f32(got_pt, ot.gemv_ternary(blocks, ot.quantize_q8_1(p.x)))
