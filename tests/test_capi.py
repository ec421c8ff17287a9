"""CPU checks of the C-ABI library: it builds, loads, exports every symbol
that include/wq.h declares, and rejects bad arguments before any HIP call
(so no GPU is needed: every call below fails validation)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    import gemm_wq_quantize_amd as g
    if not os.path.exists(g.LIB_PATH):
        from gemm_wq_quantize_amd import build
        build.build()
    return g.load_library()


def declared_functions():
    inc = os.path.join(ROOT, "include")
    text = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    return sorted(set(re.findall(r"^(?:const\s+)?\w+\**\s+\**(wq_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("wq_pack_int4", "wq_quantize_pack_int4", "wq_gemv_w4", "wq_gemm_w4a16",
                 "wq_pack_ptq1_0", "wq_quantize_q8_1", "wq_gemv_ternary", "wq_gemv_ternary_noalloc", "wq_status_string",
                 "wq_quantize_q8_1_pt", "wq_gemv_ternary_pt", "wq_gemv_ternary_ptq1_1_pt",
                 "wq_abi_version", "wq_peak_read", "wq_peak_read_sink_words", "wq_peak_mfma_bf16",
                 "wq_peak_valu_fma"):
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    import gemm_wq_quantize_amd as g
    assert g.wq_abi_version() == 1
    for st in (0, -1, -2, -3, -4, -5):
        assert g.status_string(st).startswith("WQ_")
    assert g.status_string(-99) == "unknown wq_status"


P = ctypes.c_void_p
FAKE = P(0x1000)      # never dereferenced: validation fails first
ODD = P(0x1001)


def test_validation_errors_without_gpu(lib):
    import gemm_wq_quantize_amd as g
    # empty problems are no-ops that succeed without touching pointers
    assert lib.wq_gemv_w4(None, 1, None, 2, None, 8.0, 0, 128, 128, None, 2, 1, None, 2, None) == 0
    assert lib.wq_gemv_ternary(None, None, 10, 128, 0, None, None) == 0
    assert lib.wq_pack_int4(None, 0, 8, 1, None, None) == 0
    assert lib.wq_quantize_pack_int4(None, 4, 0, 128, 1, None, None, 2, None) == 0
    assert lib.wq_gemm_w4a16(None, None, 1, None, 128, 8.0, 0, 64, 128, None, None) == 0
    assert lib.wq_gemm_w4a16_zp(None, None, 1, None, None, 128, 64, 0, 128, None, None) == 0
    assert lib.wq_pack_ptq1_0(None, None, 0, 128, None, None) == 0
    assert lib.wq_quantize_q8_1(None, 0, 64, None, None) == 0
    # null pointers / bad enums / negative sizes
    assert lib.wq_pack_int4(None, 4, 8, 1, FAKE, None) == g.WQ_EINVAL
    assert lib.wq_pack_int4(FAKE, 4, 8, 7, FAKE, None) == g.WQ_EINVAL
    assert lib.wq_pack_int4(FAKE, -1, 8, 1, FAKE, None) == g.WQ_EINVAL
    assert lib.wq_gemv_w4(FAKE, 1, FAKE, 5, None, 8.0, 4, 128, 128, FAKE, 2, 1, FAKE, 2, None) == g.WQ_EINVAL
    # shapes
    assert lib.wq_pack_int4(FAKE, 4, 12, 1, FAKE, None) == g.WQ_ESHAPE
    assert lib.wq_quantize_pack_int4(FAKE, 4, 256, 96, 1, FAKE, FAKE, 2, None) == g.WQ_ESHAPE
    assert lib.wq_quantize_pack_int4(FAKE, 4, 48, 48, 1, FAKE, FAKE, 2, None) == g.WQ_ESHAPE
    assert lib.wq_gemv_w4(FAKE, 1, FAKE, 2, None, 8.0, 4, 256, 128, FAKE, 2, 33, FAKE, 2, None) == g.WQ_ESHAPE
    assert lib.wq_gemv_w4(FAKE, 1, FAKE, 2, None, 8.0, 4, 250, 250, FAKE, 2, 1, FAKE, 2, None) == g.WQ_ESHAPE
    big = (1 << 24) + 32  # beyond the 32-bit offset bound
    assert lib.wq_gemv_w4(FAKE, 1, FAKE, 2, None, 8.0, 4, big, big, FAKE, 2, 1, FAKE, 2, None) == g.WQ_ESHAPE
    assert lib.wq_gemm_w4a16(FAKE, FAKE, 1, FAKE, (1 << 22) + 64, 8.0, 64, 64, (1 << 22) + 64, FAKE,
                             None) == g.WQ_ESHAPE
    assert lib.wq_gemm_w4a16(FAKE, FAKE, 1, FAKE, 96, 8.0, 64, 64, 96, FAKE, None) == g.WQ_ESHAPE
    assert lib.wq_gemv_ternary(FAKE, FAKE, 4, 100, 1, FAKE, None) == g.WQ_ESHAPE
    # 32-bit offsets of the matrix-core path: 2^22 rows of 32 blocks is 3.8 GB
    # of weights; 2^20 columns of 128 q8_1 blocks is 4.8 GB of activations
    assert lib.wq_gemv_ternary(FAKE, FAKE, 1 << 22, 4096, 64, FAKE, None) == g.WQ_ESHAPE
    assert lib.wq_gemv_ternary(FAKE, FAKE, 64, 4096, 1 << 20, FAKE, None) == g.WQ_ESHAPE
    # the entry point that allocates nothing: the same checks, and a workspace
    # (about n k + 2 c k bytes) beyond its 64 MiB scratch is refused up front
    assert lib.wq_gemv_ternary_noalloc(FAKE, FAKE, 4, 100, 1, FAKE, None) == g.WQ_ESHAPE
    assert lib.wq_gemv_ternary_noalloc(FAKE, FAKE, 64, 4096, 1 << 20, FAKE, None) == g.WQ_ESHAPE
    assert lib.wq_gemv_ternary_noalloc(FAKE, FAKE, 17280, 5120, 4096, FAKE, None) == g.WQ_ESHAPE
    assert lib.wq_gemv_ternary_noalloc(None, None, 10, 128, 0, None, None) == 0
    assert lib.wq_pack_ptq1_0(FAKE, FAKE, 2, 64, FAKE, None) == g.WQ_ESHAPE
    # sizes whose products overflow int64 are rejected, not wrapped round
    huge = 1 << 40
    assert lib.wq_pack_int4(FAKE, huge, huge, 1, FAKE, None) == g.WQ_ESHAPE
    assert lib.wq_quantize_pack_int4(FAKE, huge, 1 << 39, 1 << 39, 1, FAKE, FAKE, 2, None) == g.WQ_ESHAPE
    assert lib.wq_gemm_w4a16(FAKE, FAKE, 1, FAKE, 128, 8.0, huge, huge, 128, FAKE, None) == g.WQ_ESHAPE
    assert lib.wq_pack_ptq1_0(FAKE, FAKE, huge, 1 << 39, FAKE, None) == g.WQ_ESHAPE
    assert lib.wq_quantize_q8_1(FAKE, huge, 1 << 39, FAKE, None) == g.WQ_ESHAPE
    assert lib.wq_gemv_ternary(FAKE, FAKE, huge, 1 << 39, 64, FAKE, None) == g.WQ_ESHAPE
    assert lib.wq_quantize_q8_1(FAKE, 2, 48, FAKE, None) == g.WQ_ESHAPE
    # unsupported combinations
    assert lib.wq_gemm_w4a16(FAKE, FAKE, 0, FAKE, 128, 8.0, 64, 64, 128, FAKE, None) == g.WQ_EUNSUPPORTED
    # group scales: a power of two >= 64 dividing k (k = 256 or 192 here)
    assert lib.wq_gemm_w4a16(FAKE, FAKE, 1, FAKE, 32, 8.0, 64, 64, 256, FAKE, None) == g.WQ_EUNSUPPORTED
    assert lib.wq_gemm_w4a16(FAKE, FAKE, 1, FAKE, 96, 8.0, 64, 64, 192, FAKE, None) == g.WQ_ESHAPE
    assert lib.wq_gemm_w4a16(FAKE, FAKE, 1, FAKE, 512, 8.0, 64, 64, 256, FAKE, None) == g.WQ_ESHAPE
    # alignment
    assert lib.wq_gemv_w4(ODD, 1, FAKE, 2, None, 8.0, 4, 128, 128, FAKE, 2, 1, FAKE, 2, None) == g.WQ_EALIGN
    assert lib.wq_quantize_pack_int4(FAKE, 4, 256, 128, 1, ODD, FAKE, 2, None) == g.WQ_EALIGN
    assert lib.wq_gemm_w4a16(ODD, FAKE, 1, FAKE, 128, 8.0, 64, 64, 128, FAKE, None) == g.WQ_EALIGN
    # stored zeros are required by the _zp entry point, aligned like the scales
    assert lib.wq_gemm_w4a16_zp(FAKE, FAKE, 1, FAKE, None, 128, 64, 64, 256, FAKE, None) == g.WQ_EINVAL
    assert lib.wq_gemm_w4a16_zp(FAKE, FAKE, 1, FAKE, P(0x1002), 128, 64, 64, 256, FAKE, None) == g.WQ_EALIGN
    # group scales are read as aligned 4-byte words
    assert lib.wq_gemm_w4a16(FAKE, FAKE, 1, P(0x1002), 128, 8.0, 64, 64, 256, FAKE, None) == g.WQ_EALIGN
    assert lib.wq_gemv_ternary(ODD, FAKE, 4, 128, 1, FAKE, None) == g.WQ_EALIGN
    assert lib.wq_gemv_ternary(FAKE, FAKE, 4, 128, 64, P(0x1004), None) == g.WQ_EALIGN


def test_calibration_kernels_validate_without_gpu(lib):
    import gemm_wq_quantize_amd as g
    words = lib.wq_peak_read_sink_words()
    assert words >= 4096 * 16
    assert lib.wq_peak_read(None, 0, None, 0, None) == g.WQ_OK
    assert lib.wq_peak_read(None, 64, FAKE, words, None) == g.WQ_EINVAL
    assert lib.wq_peak_read(FAKE, -16, FAKE, words, None) == g.WQ_EINVAL
    assert lib.wq_peak_read(P(0x1008), 64, FAKE, words, None) == g.WQ_EALIGN
    assert lib.wq_peak_read(FAKE, 72, FAKE, words, None) == g.WQ_ESHAPE
    assert lib.wq_peak_read(FAKE, 64, FAKE, words - 1, None) == g.WQ_ESHAPE
    assert lib.wq_peak_read(FAKE, 1 << 40, FAKE, words, None) == g.WQ_ESHAPE
    for fn in (lib.wq_peak_mfma_bf16, lib.wq_peak_valu_fma):
        assert fn(0, 10, None, 0, None) == g.WQ_OK
        assert fn(4, 10, None, 1024, None) == g.WQ_EINVAL
        assert fn(-1, 10, FAKE, 1024, None) == g.WQ_EINVAL
        assert fn(4, 10, ODD, 1024, None) == g.WQ_EALIGN
        assert fn(4, 0, FAKE, 1024, None) == g.WQ_ESHAPE
        assert fn(4, 10, FAKE, 1023, None) == g.WQ_ESHAPE
        assert fn((1 << 20) + 1, 10, FAKE, 1 << 40, None) == g.WQ_ESHAPE


def test_ptq1_1_validation_without_gpu(lib):
    import gemm_wq_quantize_amd as g
    n_esc = ctypes.c_int64(0)
    # the host encoder: shape and argument errors
    assert lib.wq_ptq1_1_encode(FAKE, 4, 512, FAKE, FAKE, None, None, 0, None) == g.WQ_EINVAL
    assert lib.wq_ptq1_1_encode(FAKE, -1, 1024, FAKE, FAKE, None, None, 0, ctypes.byref(n_esc)) == g.WQ_EINVAL
    # the GEMV: k a multiple of 1024, at most 65536, at most 2048 escapes
    args = lambda k, ne, c=1: (FAKE, FAKE, FAKE, FAKE, ne, FAKE, 8, k, c, FAKE, None)
    assert lib.wq_gemv_ternary_ptq1_1(*args(512, 0)) == g.WQ_ESHAPE
    assert lib.wq_gemv_ternary_ptq1_1(*args(65536 + 1024, 0)) == g.WQ_ESHAPE
    assert lib.wq_gemv_ternary_ptq1_1(*args(1024, 2049)) == g.WQ_EUNSUPPORTED
    assert lib.wq_gemv_ternary_ptq1_1(*args(1024, -1)) == g.WQ_EINVAL
    assert lib.wq_gemv_ternary_ptq1_1(FAKE, FAKE, None, None, 3, FAKE, 8, 1024, 1, FAKE, None) == g.WQ_EINVAL
    assert lib.wq_gemv_ternary_ptq1_1(ODD, FAKE, FAKE, FAKE, 0, FAKE, 8, 1024, 1, FAKE, None) == g.WQ_EALIGN
    assert lib.wq_gemv_ternary_ptq1_1(*args(1024, 0, c=0)) == 0


def test_pt_layout_validation_without_gpu(lib):
    # the PT-layout entry points: the checks of their row-layout twins, and
    # the quantiser's k a multiple of 128 (whole 128-element blocks)
    import gemm_wq_quantize_amd as g
    assert lib.wq_quantize_q8_1_pt(None, 0, 128, None, None) == 0
    assert lib.wq_quantize_q8_1_pt(FAKE, 2, 96, FAKE, None) == g.WQ_ESHAPE
    assert lib.wq_quantize_q8_1_pt(FAKE, 2, 256, None, None) == g.WQ_EINVAL
    assert lib.wq_quantize_q8_1_pt(ODD, 2, 256, FAKE, None) == g.WQ_EALIGN
    assert lib.wq_quantize_q8_1_pt(FAKE, 1, (1 << 30) + 128, FAKE, None) == g.WQ_ESHAPE
    assert lib.wq_gemv_ternary_pt(None, None, 10, 128, 0, None, None) == 0
    assert lib.wq_gemv_ternary_pt(FAKE, FAKE, 4, 100, 1, FAKE, None) == g.WQ_ESHAPE
    assert lib.wq_gemv_ternary_pt(FAKE, ODD, 4, 128, 1, FAKE, None) == g.WQ_EALIGN
    assert lib.wq_gemv_ternary_pt(FAKE, FAKE, 64, 4096, 1 << 20, FAKE, None) == g.WQ_ESHAPE
    args = lambda k, ne, c=1: (FAKE, FAKE, FAKE, FAKE, ne, FAKE, 8, k, c, FAKE, None)
    assert lib.wq_gemv_ternary_ptq1_1_pt(*args(512, 0)) == g.WQ_ESHAPE
    assert lib.wq_gemv_ternary_ptq1_1_pt(*args(1024, 2049)) == g.WQ_EUNSUPPORTED
    assert lib.wq_gemv_ternary_ptq1_1_pt(*args(1024, 0, c=0)) == 0
