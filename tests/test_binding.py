"""Host-side checks of the Python binding: size and dtype mismatches raise
ValueError before any GPU call (the sizes bound what the kernels touch)."""
import pytest
import torch

import gemm_wq_quantize_amd as g


def t(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def test_gemm_scale_count_is_checked():
    a, b, c = t((64, 256), torch.bfloat16), t((64, 128), torch.uint8), t((64, 64), torch.bfloat16)
    with pytest.raises(ValueError, match="scales"):
        g.wq_gemm_w4a16(a, b, 1, t((63,), torch.bfloat16), 256, 8.0, c)
    with pytest.raises(ValueError, match="scales"):
        g.wq_gemm_w4a16(a, b, 1, t((64, 1), torch.bfloat16), 128, 8.0, c)  # needs 64 x 2
    with pytest.raises(ValueError, match="zeros"):
        g.wq_gemm_w4a16_zp(a, b, 1, t((64, 2), torch.bfloat16), t((64, 1), torch.bfloat16), 128, c)


def test_output_and_packed_sizes_are_checked():
    with pytest.raises(ValueError, match="c_out"):
        g.wq_gemm_w4a16(t((64, 256), torch.bfloat16), t((64, 128), torch.uint8), 1,
                        t((64,), torch.bfloat16), 256, 8.0, t((64, 63), torch.bfloat16))
    with pytest.raises(ValueError, match="packed"):
        g.wq_gemv_w4(t((8, 63), torch.uint8), 1, t((8, 1), torch.bfloat16), None, 8.0, 128, 128,
                     t((1, 128), torch.bfloat16), t((1, 8), torch.float32))
    with pytest.raises(ValueError, match="x is"):
        g.wq_gemv_w4(t((8, 64), torch.uint8), 1, t((8, 1), torch.bfloat16), None, 8.0, 128, 128,
                     t((1, 120), torch.bfloat16), t((1, 8), torch.float32))
    with pytest.raises(ValueError, match="packed"):
        g.wq_quantize_pack_int4(t((4, 256), torch.float16), 128, 1, t((4, 127), torch.uint8),
                                t((4, 2), torch.bfloat16))
    with pytest.raises(ValueError, match="out"):
        g.wq_gemv_ternary(t((4, 1, 28), torch.uint8), t((2, 4, 36), torch.uint8), 128,
                          t((2, 3), torch.float32))
    with pytest.raises(ValueError, match="x_q8"):
        g.wq_quantize_q8_1(t((2, 64), torch.float32), t((2, 2, 35), torch.uint8))
    with pytest.raises(ValueError, match="blocks"):
        g.wq_pack_ptq1_0(t((2, 128), torch.int8), t((2, 1), torch.float16), t((2, 1, 27), torch.uint8))


def test_zero_group_is_rejected():
    with pytest.raises(ValueError, match="scales"):
        g.wq_gemv_w4(t((8, 64), torch.uint8), 1, t((8, 1), torch.bfloat16), None, 8.0, 128, 0,
                     t((1, 128), torch.bfloat16), t((1, 8), torch.float32))


def test_calibration_bindings_check_sink_sizes():
    with pytest.raises(ValueError, match="sink"):
        g.wq_peak_read(t((1024,), torch.uint8), t((16,), torch.int32))
    with pytest.raises(ValueError, match="sink"):
        g.wq_peak_mfma_bf16(4, 8, t((4 * 256 - 1,), torch.float32))
    with pytest.raises(ValueError, match="sink"):
        g.wq_peak_valu_fma(4, 8, t((4 * 256,), torch.int32))
