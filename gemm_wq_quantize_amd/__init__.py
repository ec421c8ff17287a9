"""Python binding of libwq (gfx950 weight-quantised GEMV / GEMM).

Argument marshalling only: every entry point takes torch tensors that live
on the GPU, checks their dtypes and shapes, and calls the C function of the
same name in ``libwq.so`` (declared in ``include/wq.h``) on torch's current
HIP stream.  All arithmetic runs in the library's HIP kernels; there is no
CPU path.  The first call raises ImportError if the library has not been built
(``python -m gemm_wq_quantize_amd.build``).
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libwq.so")

WQ_OK, WQ_EINVAL, WQ_EALIGN, WQ_ESHAPE, WQ_EUNSUPPORTED, WQ_EHIP = 0, -1, -2, -3, -4, -5
WQ_F32, WQ_F16, WQ_BF16 = 0, 1, 2
LAYOUT_PLAIN, LAYOUT_GFX950 = 0, 1

_p, _i64, _i, _f = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
_SIGS = {
    "wq_abi_version": ([], _i),
    "wq_status_string": ([_i], ctypes.c_char_p),
    "wq_pack_int4": ([_p, _i64, _i64, _i, _p, _p], _i),
    "wq_quantize_pack_int4": ([_p, _i64, _i64, _i64, _i, _p, _p, _i, _p], _i),
    "wq_gemv_w4": ([_p, _i, _p, _i, _p, _f, _i64, _i64, _i64, _p, _i, _i64, _p, _i, _p], _i),
    "wq_gemm_w4a16": ([_p, _p, _i, _p, _i64, _f, _i64, _i64, _i64, _p, _p], _i),
    "wq_gemm_w4a16_zp": ([_p, _p, _i, _p, _p, _i64, _i64, _i64, _i64, _p, _p], _i),
    "wq_pack_ptq1_0": ([_p, _p, _i64, _i64, _p, _p], _i),
    "wq_quantize_q8_1": ([_p, _i64, _i64, _p, _p], _i),
    "wq_gemv_ternary": ([_p, _p, _i64, _i64, _i64, _p, _p], _i),
}
_LIB = None


def load_library():
    """Load libwq.so once; raises ImportError if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m gemm_wq_quantize_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _LIB = lib
    return _LIB


class _Lazy:
    def __getattr__(self, name):
        return getattr(load_library(), name)


lib = _Lazy()


class WqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {lib.wq_status_string(status).decode()} ({status})")
        self.status = status


def _check(fn: str, status: int) -> None:
    if status != WQ_OK:
        raise WqError(fn, status)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("wq: tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("wq: tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


_DT = {torch.float32: WQ_F32, torch.float16: WQ_F16, torch.bfloat16: WQ_BF16}


def _dtype(t, allowed=(torch.float32, torch.bfloat16)):
    if t.dtype not in allowed:
        raise TypeError(f"wq: dtype {t.dtype} not in {allowed}")
    return _DT[t.dtype]


def status_string(status: int) -> str:
    return lib.wq_status_string(status).decode()


def wq_abi_version() -> int:
    return lib.wq_abi_version()


def wq_pack_int4(codes, layout, packed, stream=None):
    """codes uint8 [n][k] -> packed uint8 [n][k/2] in ``layout``."""
    n, k = codes.shape
    assert codes.dtype == torch.uint8 and packed.dtype == torch.uint8
    assert packed.numel() == n * k // 2
    _check("wq_pack_int4", lib.wq_pack_int4(_ptr(codes), n, k, layout, _ptr(packed), _stream(stream)))


def wq_quantize_pack_int4(w, group, layout, packed, scales, stream=None):
    """fp16 w [n][k] -> packed uint8 [n][k/2] + scales [n][k/group] (f32 or bf16)."""
    n, k = w.shape
    assert w.dtype in (torch.float16, torch.int16, torch.uint16) and packed.dtype == torch.uint8
    assert packed.numel() == n * k // 2 and scales.numel() == n * (k // group)
    _check("wq_quantize_pack_int4",
           lib.wq_quantize_pack_int4(_ptr(w), n, k, group, layout, _ptr(packed), _ptr(scales),
                                     _dtype(scales), _stream(stream)))


def wq_gemv_w4(packed, layout, scales, zeros, zero_const, k, group, x, out, stream=None):
    """out[c][n] = sum_k (q - z) s x[c][k]; n = packed rows, c = x rows."""
    n = packed.shape[0]
    c = x.shape[0]
    assert packed.dtype == torch.uint8 and packed.numel() == n * k // 2
    assert x.shape[-1] == k and out.numel() == c * n
    assert scales.numel() == n * (k // group)
    if zeros is not None:
        assert zeros.dtype == scales.dtype and zeros.numel() == scales.numel()
    _check("wq_gemv_w4",
           lib.wq_gemv_w4(_ptr(packed), layout, _ptr(scales), _dtype(scales), _ptr(zeros),
                          float(zero_const), n, k, group, _ptr(x), _dtype(x), c, _ptr(out),
                          _dtype(out), _stream(stream)))


def wq_gemm_w4a16(a, b, layout, scales, group, zero_const, c_out, stream=None):
    """C[m][n] = sum_k A[m][k] (q[n][k] - z) s[n]; a bf16 [m][k], b uint8 [n][k/2]."""
    m, k = a.shape
    n = b.shape[0]
    assert a.dtype == torch.bfloat16 and c_out.dtype == torch.bfloat16 and b.dtype == torch.uint8
    assert b.numel() == n * k // 2 and c_out.numel() == m * n and scales.dtype == torch.bfloat16
    _check("wq_gemm_w4a16",
           lib.wq_gemm_w4a16(_ptr(a), _ptr(b), layout, _ptr(scales), group, float(zero_const),
                             m, n, k, _ptr(c_out), _stream(stream)))


def wq_gemm_w4a16_zp(a, b, layout, scales, zeros, group, c_out, stream=None):
    """C[m][n] = sum_k A[m][k] (q[n][k] - z[n][k/group]) s[n][k/group] with stored
    bf16 zeros of the scales' shape."""
    m, k = a.shape
    n = b.shape[0]
    assert a.dtype == torch.bfloat16 and c_out.dtype == torch.bfloat16 and b.dtype == torch.uint8
    assert b.numel() == n * k // 2 and c_out.numel() == m * n
    assert scales.dtype == torch.bfloat16 and zeros.dtype == torch.bfloat16
    assert zeros.numel() == scales.numel() == n * (k // group)
    _check("wq_gemm_w4a16_zp",
           lib.wq_gemm_w4a16_zp(_ptr(a), _ptr(b), layout, _ptr(scales), _ptr(zeros), group,
                                m, n, k, _ptr(c_out), _stream(stream)))


def wq_pack_ptq1_0(trits, d, blocks, stream=None):
    """trits int8 [n][k], d fp16 [n][k/128] -> PTQ1_0 blocks uint8 [n][k/128][28]."""
    n, k = trits.shape
    assert trits.dtype == torch.int8 and blocks.dtype == torch.uint8
    assert d.numel() == n * (k // 128) and blocks.numel() == n * (k // 128) * 28
    _check("wq_pack_ptq1_0",
           lib.wq_pack_ptq1_0(_ptr(trits), _ptr(d), n, k, _ptr(blocks), _stream(stream)))


def wq_quantize_q8_1(x, x_q8, stream=None):
    """fp32 x [c][k] -> block_q8_1 uint8 [c][k/32][36]."""
    c, k = x.shape
    assert x.dtype == torch.float32 and x_q8.dtype == torch.uint8
    assert x_q8.numel() == c * (k // 32) * 36
    _check("wq_quantize_q8_1", lib.wq_quantize_q8_1(_ptr(x), c, k, _ptr(x_q8), _stream(stream)))


def wq_gemv_ternary(w_blocks, x_q8, k, out, stream=None):
    """out fp32 [c][n] from PTQ1_0 weights [n][k/128][28] and q8_1 x [c][k/32][36]."""
    n = w_blocks.shape[0]
    c = x_q8.shape[0]
    assert w_blocks.numel() == n * (k // 128) * 28 and x_q8.numel() == c * (k // 32) * 36
    assert out.dtype == torch.float32 and out.numel() == c * n
    _check("wq_gemv_ternary",
           lib.wq_gemv_ternary(_ptr(w_blocks), _ptr(x_q8), n, k, c, _ptr(out), _stream(stream)))
