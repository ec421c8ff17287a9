"""GPU parity over seeded random shapes.

Each case draws its sizes and options from its own seed (printed before the
GPU call) and compares the entry point with the oracle: ragged row and
column counts, every group size, both nibble layouts, f32 / bf16 scales,
activations and outputs, optional stored zeros, every batch width the
kernels split on (1..32 for the int4 GEMV; 1..200 for the ternary path, with
the PT plane layout bit-identical to record order), and GEMM tiles with
ragged edges.  Sizes stay small enough for the fp64 oracle.
"""
import numpy as np
import pytest
import torch

from oracle import fpformat, int4 as o4, ternary as ot
from tolerances import check_bf16_rownorm, check_bf16_rows, check_f32

pytestmark = pytest.mark.gpu

MAX_NK = 3 << 20  # n * k per case (the oracle dequantises W in fp64)


def G():
    import gemm_wq_quantize_amd as g
    return g


def say(*a):
    print("[case]", *a, flush=True)


def _round(v, dtype):
    v = np.asarray(v, dtype=np.float32)
    if dtype == "bf16":
        return fpformat.bf16_bits_to_f32(fpformat.f32_to_bf16_bits(v))
    return v


def _dev(v, dtype):
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


@pytest.mark.parametrize("case", range(24))
def test_gemv_w4_random_shapes(case):
    rng = np.random.default_rng(7000 + case)
    group = int(rng.choice([32, 64, 128, 256, 0]))  # 0: one scale per row
    k = group * int(rng.integers(1, 48)) if group else 32 * int(rng.integers(1, 400))
    group = group or k
    n = int(rng.integers(1, max(2, min(3000, MAX_NK // k))))
    c = int(rng.integers(1, 33))
    layout = int(rng.integers(0, 2))
    sdt, xdt, odt = (str(rng.choice(["f32", "bf16"])) for _ in range(3))
    with_zeros = bool(rng.random() < 0.3)
    say("gemv_w4", dict(n=n, k=k, group=group, c=c, layout=layout, scales=sdt, x=xdt, out=odt, zeros=with_zeros))
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    s = _round(rng.uniform(0.002, 0.02, (n, k // group)), sdt)
    z = _round(rng.integers(0, 16, (n, k // group)), sdt) if with_zeros else None
    x = _round(rng.standard_normal((c, k)), xdt)
    g = G()
    packed = torch.empty((n, k // 2), dtype=torch.uint8, device="cuda")
    g.wq_pack_int4(torch.from_numpy(codes).cuda(), layout, packed)
    out = torch.empty((c, n), dtype=torch.bfloat16 if odt == "bf16" else torch.float32, device="cuda")
    g.wq_gemv_w4(packed, layout, _dev(s, sdt), _dev(z, sdt) if with_zeros else None, 8.0, k, group,
                 _dev(x, xdt), out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    ref = o4.gemv_w4(o4.pack(codes, layout), layout, s, z, 8.0, group, x)
    if odt == "bf16":
        check_bf16_rows(got, ref)
    else:
        check_f32(got, ref)


@pytest.mark.parametrize("case", range(12))
def test_gemv_ternary_random_shapes(case):
    rng = np.random.default_rng(8000 + case)
    k = 128 * int(rng.integers(1, 100))
    n = int(rng.integers(1, max(2, min(2500, MAX_NK // k))))
    c = int(rng.choice([int(rng.integers(1, 9)), int(rng.integers(9, 64)), int(rng.integers(64, 201))]))
    say("gemv_ternary", dict(n=n, k=k, c=c))
    trits = rng.integers(-1, 2, (n, k), dtype=np.int8)
    d_bits = fpformat.f32_to_f16_bits(rng.uniform(0.005, 0.05, (n, k // 128)).astype(np.float32))
    x = rng.standard_normal((c, k)).astype(np.float32)
    g = G()
    wb = torch.empty((n, k // 128, 28), dtype=torch.uint8, device="cuda")
    g.wq_pack_ptq1_0(torch.from_numpy(trits).cuda(), torch.from_numpy(d_bits).view(torch.int16).cuda(), wb)
    xs = torch.from_numpy(x).cuda()
    xq = torch.empty((c, k // 32, 36), dtype=torch.uint8, device="cuda")
    g.wq_quantize_q8_1(xs, xq)
    xp = torch.empty((c, 9 * k // 8), dtype=torch.uint8, device="cuda")
    g.wq_quantize_q8_1_pt(xs, xp)
    out = torch.empty((c, n), dtype=torch.float32, device="cuda")
    out_pt = torch.empty_like(out)
    g.wq_gemv_ternary(wb, xq, k, out)
    g.wq_gemv_ternary_pt(wb, xp, k, out_pt)
    torch.cuda.synchronize()
    xref = ot.quantize_q8_1(x)
    blocks = ot.encode_ptq1_0(trits, d_bits)
    assert np.array_equal(wb.cpu().numpy(), blocks)
    assert np.array_equal(xq.cpu().numpy(), xref)
    assert np.array_equal(xp.cpu().numpy(), ot.q8_1_to_pt(xref))
    got = out.cpu().numpy()
    assert np.array_equal(out_pt.cpu().numpy(), got)
    check_f32(got, ot.gemv_ternary(blocks, xref))


@pytest.mark.parametrize("case", range(10))
def test_gemm_w4a16_random_shapes(case):
    rng = np.random.default_rng(9000 + case)
    k = 64 * int(rng.integers(1, 48))
    groups = [k] + [gr for gr in (64, 128, 256) if gr < k and k % gr == 0]
    group = int(rng.choice(groups))
    m = int(rng.integers(1, 600))
    n = int(rng.integers(1, max(2, min(1500, MAX_NK // k))))
    say("gemm_w4a16", dict(m=m, n=n, k=k, group=group))
    a = _round(rng.standard_normal((m, k)), "bf16")
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    s = _round(rng.uniform(0.002, 0.02, (n, k // group)), "bf16")
    g = G()
    b = torch.empty((n, k // 2), dtype=torch.uint8, device="cuda")
    g.wq_pack_int4(torch.from_numpy(codes).cuda(), 1, b)
    cm = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    g.wq_gemm_w4a16(_dev(a, "bf16"), b, 1, _dev(s.reshape(-1) if group == k else s, "bf16"), group, 8.0, cm)
    torch.cuda.synchronize()
    got = cm.float().cpu().numpy()
    packed = o4.pack(codes, 1)
    exact = o4.gemm_w4a16_rows(a, packed, 1, s, 8.0, group)
    if group == k:
        check_bf16_rows(got, exact)
    else:
        check_bf16_rows(got, o4.gemm_w4a16_rows_bf16w(a, packed, 1, s, 8.0, group))
        check_bf16_rownorm(got, exact)
