"""GPU parity: the ternary GEMV on PTQ1_1 superblocks against the oracle.

The superblocks come from the library's host encoder; the oracle encodes
the same PTQ1_0 blocks itself (and the bytes must agree), then its GEMV is
the PTQ1_0 GEMV of its own decoded blocks."""
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


def encode_both(trits, d_bits):
    blocks = ot.encode_ptq1_0(trits, d_bits)
    sup, book, ei, ep = G().wq_ptq1_1_encode(blocks)
    ref = ot.encode_ptq1_1(blocks)
    assert np.array_equal(sup, ref[0]) and np.array_equal(book, ref[1])
    assert np.array_equal(ei.astype(np.int64), ref[2]) and np.array_equal(ep, ref[3])
    dev = [torch.from_numpy(a).cuda() for a in (sup, book, ei, ep)]
    return dev, ref


def gpu_q8(x):
    c, k = x.shape
    out = torch.empty((c, k // 32, 36), dtype=torch.uint8, device="cuda")
    G().wq_quantize_q8_1(torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda(), out)
    return out


def gemv(dev, xq, k, n):
    out = torch.empty((xq.shape[0], n), dtype=torch.float32, device="cuda")
    G().wq_gemv_ternary_ptq1_1(dev[0], dev[1], dev[2], dev[3], xq, k, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_ptq1_1_gemv_timed_shape():
    # K=5120, N=17280, block scales with the post's exponent statistics
    k, n = 5120, 17280
    p = wq_inputs.ternary_correlated_scales(k, n, cmax=8)
    dev, ref = encode_both(p.trits, p.d_bits)
    say("ptq1_1 gemv", k, n, "escapes", len(ref[2]))
    for c in (1, 4, 8):
        say("ptq1_1 gemv", k, n, c)
        xq = gpu_q8(p.x[:c])
        xref = ot.quantize_q8_1(p.x[:c])
        assert np.array_equal(xq.cpu().numpy(), xref)
        check_f32(gemv(dev, xq, k, n), ot.gemv_ternary_ptq1_1(*ref, xref))


@pytest.mark.parametrize("k,n", [(8192, 300), (1024, 77), (16384, 40), (65536, 24)])
def test_ptq1_1_gemv_escapes_and_passes(k, n):
    # independent exponents: most superblocks escape; widths that take every
    # pass shape (1, 2, 3 columns; 5..8; more than 8 in passes); k = 65536
    # is past the matrix-core kernel's LDS, so its passes run on the vector
    # kernels (one column: the K-split kernel)
    p = wq_inputs.ternary_gemv(k, n, cmax=16, seed=k + n)
    rng = np.random.default_rng(n)
    d = ((rng.integers(5, 13, p.d_bits.shape) << 10) | rng.integers(0, 1024, p.d_bits.shape)).astype(np.uint16)
    dev, ref = encode_both(p.trits, d)
    say("ptq1_1 gemv escapes", k, n, len(ref[2]))
    for c in (1, 2, 3, 5, 9, 16):
        say("ptq1_1 gemv", k, n, c)
        xq = gpu_q8(p.x[:c])
        check_f32(gemv(dev, xq, k, n), ot.gemv_ternary_ptq1_1(*ref, ot.quantize_q8_1(p.x[:c])))


@pytest.mark.parametrize("k,n,c", [(5120, 500, 64), (2048, 333, 130), (8192, 77, 96)])
def test_ptq1_1_prefill(k, n, c):
    # 64 or more columns: the superblocks unpacked, then the matrix-core
    # product; ragged tiles in both directions, most superblocks escaped
    p = wq_inputs.ternary_gemv(k, n, cmax=c, seed=k + c)
    rng = np.random.default_rng(c)
    d = ((rng.integers(5, 13, p.d_bits.shape) << 10) | rng.integers(0, 1024, p.d_bits.shape)).astype(np.uint16)
    dev, ref = encode_both(p.trits, d)
    say("ptq1_1 prefill", k, n, c, "escapes", len(ref[2]))
    xq = gpu_q8(p.x)
    check_f32(gemv(dev, xq, k, n), ot.gemv_ternary_ptq1_1(*ref, ot.quantize_q8_1(p.x)))


def test_ptq1_1_prefill_timed_shape_sampled_columns():
    # the ternary GEMM's workload on superblocks with the post's exponent
    # statistics; 8 seeded columns against the oracle, the rest finite
    k, n, c = 5120, 17280, 4096
    p = wq_inputs.ternary_correlated_scales(k, n, cmax=c, seed=3)
    dev, ref = encode_both(p.trits, p.d_bits)
    say("ptq1_1 prefill", k, n, c, "sampled columns")
    got = gemv(dev, gpu_q8(p.x), k, n)
    cols = np.sort(np.random.default_rng(3).choice(c, 8, replace=False))
    check_f32(got[cols], ot.gemv_ternary_ptq1_1(*ref, ot.quantize_q8_1(p.x[cols])))
    assert np.isfinite(got).all()


@pytest.mark.parametrize("c", [1, 4, 8, 96])
def test_ptq1_1_unit_scale_exact(c):
    # every d = 1.0 (one pattern) and integer activations with +-127 in each
    # block of 32: the exact integer product, bit for bit
    k, n = 5120, 4000
    say("ptq1_1 unit scale", k, n, c)
    p = wq_inputs.ternary_gemv(k, n, cmax=max(c, 8), unit_scale=True)
    dev, _ = encode_both(p.trits, p.d_bits)
    got = gemv(dev, gpu_q8(p.x[:c]), k, n)
    exact = p.x[:c].astype(np.int64) @ p.trits.astype(np.int64).T
    assert np.array_equal(got, exact.astype(np.float64))


def test_ptq1_1_repeatable():
    k, n = 5120, 2000
    say("ptq1_1 bitwise repeatable")
    p = wq_inputs.ternary_correlated_scales(k, n, cmax=4, seed=7)
    dev, _ = encode_both(p.trits, p.d_bits)
    xq = gpu_q8(p.x)
    outs = [gemv(dev, xq, k, n) for _ in range(3)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
