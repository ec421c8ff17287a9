"""wq_gemv_ternary_noalloc (the entry point that allocates nothing) against
wq_gemv_ternary, through the C ABI: two calls in a row on the matrix-core
path, the second smaller, then one below 64 columns.  Both entry points run
the same kernels, so the outputs must match bit for bit; the first call is
also checked against the oracle on sampled columns."""
import ctypes

import numpy as np
import pytest
import torch

import wq_inputs
from oracle import ternary as ot
from tolerances import check_f32

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def operands(k, n, c, seed):
    import gemm_wq_quantize_amd as g
    p = wq_inputs.ternary_gemv(k, n, cmax=c, seed=seed)
    wb = torch.empty((n, k // 128, 28), dtype=torch.uint8, device="cuda")
    g.wq_pack_ptq1_0(torch.from_numpy(p.trits).cuda(), torch.from_numpy(p.d_bits).view(torch.int16).cuda(), wb)
    xq = torch.empty((c, k // 32, 36), dtype=torch.uint8, device="cuda")
    g.wq_quantize_q8_1(torch.from_numpy(np.ascontiguousarray(p.x[:c], np.float32)).cuda(), xq)
    return p, wb, xq


def call(name, wb, xq, n, k, c, out):
    import gemm_wq_quantize_amd as g
    fn = getattr(g.lib, name)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = fn(ctypes.c_void_p(wb.data_ptr()), ctypes.c_void_p(xq.data_ptr()), n, k, c,
            ctypes.c_void_p(out.data_ptr()), st)
    assert rc == 0, (name, rc)


def test_noalloc_matches_allocating_entry_point():
    # workspaces: 4096 x 5120 + 2 x 512 x 5120 ~ 26 MB, then ~ 5 MB (limit 64 MiB)
    for (k, n, c, seed) in [(5120, 4096, 512, 3), (2048, 1500, 200, 4), (2048, 1000, 40, 5)]:
        say("noalloc vs allocating", k, n, c)
        p, wb, xq = operands(k, n, c, seed)
        a = torch.empty((c, n), dtype=torch.float32, device="cuda")
        b = torch.full((c, n), float("nan"), dtype=torch.float32, device="cuda")
        call("wq_gemv_ternary", wb, xq, n, k, c, a)
        call("wq_gemv_ternary_noalloc", wb, xq, n, k, c, b)
        torch.cuda.synchronize()
        assert torch.equal(a, b), float((a - b).abs().max())
        if seed == 3:  # sampled columns against the oracle
            xq_h = xq.cpu().numpy()
            blocks = wb.cpu().numpy()
            for j in (0, 257, c - 1):
                ref = ot.gemv_ternary(blocks, xq_h[j:j + 1])
                check_f32(b[j:j + 1].cpu().numpy(), ref)
