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
    "wq_quantize_q8_1_pt": ([_p, _i64, _i64, _p, _p], _i),
    "wq_gemv_ternary": ([_p, _p, _i64, _i64, _i64, _p, _p], _i),
    "wq_gemv_ternary_pt": ([_p, _p, _i64, _i64, _i64, _p, _p], _i),
    "wq_gemv_ternary_noalloc": ([_p, _p, _i64, _i64, _i64, _p, _p], _i),
    "wq_ptq1_1_encode": ([_p, _i64, _i64, _p, _p, _p, _p, _i64, _p], _i),
    "wq_gemv_ternary_ptq1_1": ([_p, _p, _p, _p, _i64, _p, _i64, _i64, _i64, _p, _p], _i),
    "wq_gemv_ternary_ptq1_1_pt": ([_p, _p, _p, _p, _i64, _p, _i64, _i64, _i64, _p, _p], _i),
    # calibration kernels (include/wq_peaks.h)
    "wq_peak_read_sink_words": ([], _i64),
    "wq_peak_read": ([_p, _i64, _p, _i64, _p], _i),
    "wq_peak_mfma_bf16": ([_i, _i, _p, _i64, _p], _i),
    "wq_peak_valu_fma": ([_i, _i, _p, _i64, _p], _i),
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


def _require(cond: bool, msg: str) -> None:
    """Argument check that survives ``python -O`` (unlike assert): the sizes
    checked here bound what the kernels read and write."""
    if not cond:
        raise ValueError(f"wq: {msg}")


def _ptr(t, dev=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("wq: tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("wq: tensors must be contiguous")
    if dev is not None and t.device != dev:
        raise ValueError(f"wq: tensor on {t.device}, stream on {dev}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    return stream if stream is not None else torch.cuda.current_stream()


def _sptr(s):
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
    _require(codes.dtype == torch.uint8 and packed.dtype == torch.uint8, "codes and packed are uint8")
    _require(packed.numel() == n * k // 2, "packed holds n * k / 2 bytes")
    st = _stream(stream)
    _check("wq_pack_int4", lib.wq_pack_int4(_ptr(codes, st.device), n, k, layout,
                                            _ptr(packed, st.device), _sptr(st)))


def wq_quantize_pack_int4(w, group, layout, packed, scales, stream=None):
    """fp16 w [n][k] -> packed uint8 [n][k/2] + scales [n][k/group] (f32 or bf16)."""
    n, k = w.shape
    _require(w.dtype in (torch.float16, torch.int16, torch.uint16), "w is fp16 (or its bits)")
    _require(packed.dtype == torch.uint8 and packed.numel() == n * k // 2,
             "packed is uint8 with n * k / 2 bytes")
    _require(group > 0 and scales.numel() == n * (k // group), "scales hold n * (k / group) values")
    st = _stream(stream)
    _check("wq_quantize_pack_int4",
           lib.wq_quantize_pack_int4(_ptr(w, st.device), n, k, group, layout, _ptr(packed, st.device),
                                     _ptr(scales, st.device), _dtype(scales), _sptr(st)))


def wq_gemv_w4(packed, layout, scales, zeros, zero_const, k, group, x, out, stream=None):
    """out[c][n] = sum_k (q - z) s x[c][k]; n = packed rows, c = x rows."""
    n = packed.shape[0]
    c = x.shape[0]
    _require(packed.dtype == torch.uint8 and packed.numel() == n * k // 2,
             "packed is uint8 with n * k / 2 bytes")
    _require(x.numel() == c * k and out.numel() == c * n, "x is [c][k] and out [c][n]")
    _require(group > 0 and scales.numel() == n * (k // group), "scales hold n * (k / group) values")
    if zeros is not None:
        _require(zeros.dtype == scales.dtype and zeros.numel() == scales.numel(),
                 "zeros match the scales in dtype and shape")
    st = _stream(stream)
    d = st.device
    _check("wq_gemv_w4",
           lib.wq_gemv_w4(_ptr(packed, d), layout, _ptr(scales, d), _dtype(scales), _ptr(zeros, d),
                          float(zero_const), n, k, group, _ptr(x, d), _dtype(x), c, _ptr(out, d),
                          _dtype(out), _sptr(st)))


def _gemm_shapes(a, b, scales, group, c_out):
    m, k = a.shape
    n = b.shape[0]
    _require(a.dtype == torch.bfloat16 and c_out.dtype == torch.bfloat16, "a and c_out are bf16")
    _require(b.dtype == torch.uint8 and b.numel() == n * k // 2, "b is uint8 with n * k / 2 bytes")
    _require(c_out.numel() == m * n, "c_out is [m][n]")
    _require(scales.dtype == torch.bfloat16, "scales are bf16")
    _require(group > 0 and scales.numel() == (n if group == k else n * (k // group)),
             "scales hold n (group == k) or n * (k / group) values")
    return m, n, k


def wq_gemm_w4a16(a, b, layout, scales, group, zero_const, c_out, stream=None):
    """C[m][n] = sum_k A[m][k] (q[n][k] - z) s[n]; a bf16 [m][k], b uint8 [n][k/2]."""
    m, n, k = _gemm_shapes(a, b, scales, group, c_out)
    st = _stream(stream)
    d = st.device
    _check("wq_gemm_w4a16",
           lib.wq_gemm_w4a16(_ptr(a, d), _ptr(b, d), layout, _ptr(scales, d), group, float(zero_const),
                             m, n, k, _ptr(c_out, d), _sptr(st)))


def wq_gemm_w4a16_zp(a, b, layout, scales, zeros, group, c_out, stream=None):
    """C[m][n] = sum_k A[m][k] (q[n][k] - z[n][k/group]) s[n][k/group] with stored
    bf16 zeros of the scales' shape."""
    m, n, k = _gemm_shapes(a, b, scales, group, c_out)
    _require(zeros is not None and zeros.dtype == torch.bfloat16 and zeros.numel() == scales.numel(),
             "zeros are bf16 of the scales' shape")
    st = _stream(stream)
    d = st.device
    _check("wq_gemm_w4a16_zp",
           lib.wq_gemm_w4a16_zp(_ptr(a, d), _ptr(b, d), layout, _ptr(scales, d), _ptr(zeros, d), group,
                                m, n, k, _ptr(c_out, d), _sptr(st)))


def wq_pack_ptq1_0(trits, d, blocks, stream=None):
    """trits int8 [n][k], d fp16 [n][k/128] -> PTQ1_0 blocks uint8 [n][k/128][28]."""
    n, k = trits.shape
    _require(trits.dtype == torch.int8 and blocks.dtype == torch.uint8, "trits int8, blocks uint8")
    _require(d.dtype in (torch.float16, torch.int16, torch.uint16), "d is fp16 (or its bits)")
    _require(d.numel() == n * (k // 128), "d holds n * k / 128 fp16 values")
    _require(blocks.numel() == n * (k // 128) * 28, "blocks hold n * k / 128 * 28 bytes")
    st = _stream(stream)
    dv = st.device
    _check("wq_pack_ptq1_0",
           lib.wq_pack_ptq1_0(_ptr(trits, dv), _ptr(d, dv), n, k, _ptr(blocks, dv), _sptr(st)))


def _quantize_q8_1(name, x, x_q8, stream):
    c, k = x.shape
    _require(x.dtype == torch.float32 and x_q8.dtype == torch.uint8, "x fp32, x_q8 uint8")
    _require(x_q8.numel() == c * (k // 32) * 36, "x_q8 holds c * k / 32 * 36 bytes")
    st = _stream(stream)
    _check(name, getattr(lib, name)(_ptr(x, st.device), c, k, _ptr(x_q8, st.device), _sptr(st)))


def wq_quantize_q8_1(x, x_q8, stream=None):
    """fp32 x [c][k] -> block_q8_1 uint8 [c][k/32][36]."""
    _quantize_q8_1("wq_quantize_q8_1", x, x_q8, stream)


def wq_quantize_q8_1_pt(x, x_pt, stream=None):
    """fp32 x [c][k] -> the same q8_1 blocks in the PT plane layout, uint8
    [c][9k/8]."""
    _quantize_q8_1("wq_quantize_q8_1_pt", x, x_pt, stream)


def _ternary_args(w_blocks, x_q8, k, out):
    n = w_blocks.shape[0]
    c = x_q8.shape[0]
    _require(w_blocks.dtype == torch.uint8 and x_q8.dtype == torch.uint8, "blocks are uint8")
    _require(w_blocks.numel() == n * (k // 128) * 28 and x_q8.numel() == c * (k // 32) * 36,
             "w_blocks [n][k/128][28], x_q8 [c][k/32][36]")
    _require(out.dtype == torch.float32 and out.numel() == c * n, "out is fp32 [c][n]")
    return n, c


def wq_gemv_ternary(w_blocks, x_q8, k, out, stream=None):
    """out fp32 [c][n] from PTQ1_0 weights [n][k/128][28] and q8_1 x [c][k/32][36]."""
    n, c = _ternary_args(w_blocks, x_q8, k, out)
    st = _stream(stream)
    d = st.device
    _check("wq_gemv_ternary",
           lib.wq_gemv_ternary(_ptr(w_blocks, d), _ptr(x_q8, d), n, k, c, _ptr(out, d), _sptr(st)))


def wq_gemv_ternary_pt(w_blocks, x_pt, k, out, stream=None):
    """wq_gemv_ternary with x in the PT plane layout, uint8 [c][9k/8]."""
    n, c = _ternary_args(w_blocks, x_pt, k, out)
    st = _stream(stream)
    d = st.device
    _check("wq_gemv_ternary_pt",
           lib.wq_gemv_ternary_pt(_ptr(w_blocks, d), _ptr(x_pt, d), n, k, c, _ptr(out, d), _sptr(st)))


def wq_gemv_ternary_noalloc(w_blocks, x_q8, k, out, stream=None):
    """wq_gemv_ternary with no device allocation (workspace in the library's
    static scratch; a larger workspace raises)."""
    n, c = _ternary_args(w_blocks, x_q8, k, out)
    st = _stream(stream)
    d = st.device
    _check("wq_gemv_ternary_noalloc",
           lib.wq_gemv_ternary_noalloc(_ptr(w_blocks, d), _ptr(x_q8, d), n, k, c, _ptr(out, d), _sptr(st)))


def wq_ptq1_1_encode(blocks):
    """PTQ1_0 blocks (host numpy uint8 [n][k/128][28]) -> PTQ1_1 superblocks
    on the host: (superblocks uint8 [n][k/1024][216], codebook uint8 [767][8],
    escape indices int32 [n_esc], escape patterns uint8 [n_esc][8])."""
    import numpy as np
    b = np.ascontiguousarray(blocks, dtype=np.uint8)
    _require(b.ndim == 3 and b.shape[2] == 28, "blocks are [n][k/128][28]")
    n, nb = b.shape[0], b.shape[1]
    k = nb * 128
    _require(nb % 8 == 0, "k is a multiple of 1024")
    sup = np.empty((n, nb // 8, 216), dtype=np.uint8)
    book = np.empty((767, 8), dtype=np.uint8)
    n_esc = ctypes.c_int64(0)
    cap = n * (nb // 8)
    idx = np.empty(max(cap, 1), dtype=np.int32)
    patt = np.empty((max(cap, 1), 8), dtype=np.uint8)
    _check("wq_ptq1_1_encode",
           lib.wq_ptq1_1_encode(b.ctypes.data_as(_p), n, k, sup.ctypes.data_as(_p),
                                book.ctypes.data_as(_p), idx.ctypes.data_as(_p),
                                patt.ctypes.data_as(_p), cap, ctypes.byref(n_esc)))
    m = n_esc.value
    return sup, book, idx[:m].copy(), patt[:m].copy()


def wq_gemv_ternary_ptq1_1(superblocks, codebook, esc_idx, esc_patt, x_q8, k, out, stream=None):
    """out fp32 [c][n] from PTQ1_1 superblocks [n][k/1024][216] (device), the
    codebook [767][8] and escape table (device), and q8_1 x [c][k/32][36]."""
    _gemv_ternary_ptq1_1("wq_gemv_ternary_ptq1_1", superblocks, codebook, esc_idx, esc_patt, x_q8, k, out,
                         stream)


def wq_gemv_ternary_ptq1_1_pt(superblocks, codebook, esc_idx, esc_patt, x_pt, k, out, stream=None):
    """wq_gemv_ternary_ptq1_1 with x in the PT plane layout, uint8 [c][9k/8]."""
    _gemv_ternary_ptq1_1("wq_gemv_ternary_ptq1_1_pt", superblocks, codebook, esc_idx, esc_patt, x_pt, k, out,
                         stream)


def _gemv_ternary_ptq1_1(name, superblocks, codebook, esc_idx, esc_patt, x_q8, k, out, stream):
    n = superblocks.shape[0]
    c = x_q8.shape[0]
    n_esc = esc_idx.numel()
    _require(superblocks.dtype == torch.uint8 and codebook.dtype == torch.uint8 and
             x_q8.dtype == torch.uint8 and esc_patt.dtype == torch.uint8, "byte tensors are uint8")
    _require(esc_idx.dtype == torch.int32, "escape indices are int32")
    _require(superblocks.numel() == n * (k // 1024) * 216, "superblocks [n][k/1024][216]")
    _require(codebook.numel() == 767 * 8, "codebook [767][8]")
    _require(esc_patt.numel() == n_esc * 8, "escape patterns [n_esc][8]")
    _require(x_q8.numel() == c * (k // 32) * 36, "x_q8 [c][k/32][36]")
    _require(out.dtype == torch.float32 and out.numel() == c * n, "out is fp32 [c][n]")
    st = _stream(stream)
    d = st.device
    _check(name, getattr(lib, name)(_ptr(superblocks, d), _ptr(codebook, d),
                                    _ptr(esc_idx, d) if n_esc else None,
                                    _ptr(esc_patt, d) if n_esc else None, n_esc,
                                    _ptr(x_q8, d), n, k, c, _ptr(out, d), _sptr(st)))


# ---- calibration kernels (include/wq_peaks.h): practical ceilings of the
# device, for setting kernel times against what it sustains

def wq_peak_read_sink_words() -> int:
    return lib.wq_peak_read_sink_words()


def wq_peak_read(buf, sink, stream=None):
    """Stream all bytes of ``buf`` (any dtype, 16-byte multiple) through one
    1024-lane workgroup per CU; ``sink`` is uint32-sized storage of at least
    ``wq_peak_read_sink_words()`` words (overwritten)."""
    nbytes = buf.numel() * buf.element_size()
    _require(sink.element_size() == 4 and sink.numel() >= wq_peak_read_sink_words(),
             "sink holds wq_peak_read_sink_words() 32-bit words")
    st = _stream(stream)
    _check("wq_peak_read", lib.wq_peak_read(_ptr(buf, st.device), nbytes, _ptr(sink, st.device),
                                            sink.numel(), _sptr(st)))


def wq_peak_mfma_bf16(workgroups, iters, sink, stream=None):
    """bf16 matrix-core loop; flops = workgroups * 4 * iters * 8 * 32768 (2 * 32 * 32 * 16 per product)."""
    _require(sink.dtype == torch.float32 and sink.numel() >= workgroups * 256, "sink fp32, workgroups * 256")
    st = _stream(stream)
    _check("wq_peak_mfma_bf16", lib.wq_peak_mfma_bf16(workgroups, iters, _ptr(sink, st.device), sink.numel(),
                                                      _sptr(st)))


def wq_peak_valu_fma(workgroups, iters, sink, stream=None):
    """fp32 FMA loop; flops = workgroups * 256 * iters * 8 * 2."""
    _require(sink.dtype == torch.float32 and sink.numel() >= workgroups * 256, "sink fp32, workgroups * 256")
    st = _stream(stream)
    _check("wq_peak_valu_fma", lib.wq_peak_valu_fma(workgroups, iters, _ptr(sink, st.device), sink.numel(),
                                                    _sptr(st)))
