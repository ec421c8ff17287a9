"""The library's PTQ1_1 encoder (host C++, wq_ptq1_1_encode) against the
oracle's: every byte of the superblocks, the codebook and the escape table.
Host code only, so it runs without a GPU."""
import numpy as np
import pytest

import wq_inputs
from oracle import ternary as ot


def g():
    import gemm_wq_quantize_amd as gg
    import os
    if not os.path.exists(gg.LIB_PATH):
        from gemm_wq_quantize_amd import build
        build.build()
    return gg


def _compare(blocks):
    sup, book, ei, ep = g().wq_ptq1_1_encode(blocks)
    rs, rb, ri, rp = ot.encode_ptq1_1(blocks)
    assert np.array_equal(sup, rs)
    assert np.array_equal(book, rb)
    assert np.array_equal(ei.astype(np.int64), ri)
    assert np.array_equal(ep, rp)
    return len(ei)


@pytest.mark.parametrize("n,k,independent", [(40, 5120, False), (7, 1024, False), (300, 8192, True)])
def test_encoder_matches_oracle(n, k, independent):
    p = wq_inputs.ternary_correlated_scales(k, n, 1, seed=n + k)
    d = p.d_bits
    if independent:  # many more exponent patterns than codebook rows
        rng = np.random.default_rng(n)
        d = ((rng.integers(5, 13, d.shape) << 10) | rng.integers(0, 1024, d.shape)).astype(np.uint16)
    n_esc = _compare(ot.encode_ptq1_0(p.trits, d))
    if independent:
        assert n_esc > 1000


def test_encoder_rejects_negative_scale():
    gg = g()
    d = np.full((2, 16), 0x3C00, np.uint16)
    d[1, 9] = 0xBC00
    with pytest.raises(gg.WqError) as e:
        gg.wq_ptq1_1_encode(ot.encode_ptq1_0(np.zeros((2, 2048), np.int8), d))
    assert e.value.status == gg.WQ_EINVAL
