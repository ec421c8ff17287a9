"""Parity bars between the HIP path and the oracle (float results).

fp32 outputs: |y - y*| <= 1e-3 * max(|y*|, rms(y*[c, :])) -- relative, with the
denominator floored at the RMS of that output vector so that results near
zero from cancellation do not fail spuriously.

bf16 outputs: max_j |y_j - y*_j| <= 1e-2 * rms(y*_row), a row being one
output vector (out[c, :] or C[m, :]).
"""
import numpy as np

REL_F32 = 1e-3
REL_BF16_ROW = 1e-2


def check_f32(got, ref, rel=REL_F32):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    denom = np.maximum(np.abs(ref), rms)
    bad = np.abs(got - ref) > rel * denom
    assert not bad.any(), (f"{int(bad.sum())} of {bad.size} outside {rel} relative; "
                           f"worst {float((np.abs(got - ref) / np.maximum(denom, 1e-300)).max()):.3g}")


def check_bf16_rows(got, ref, rel=REL_BF16_ROW):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    rms = np.sqrt(np.mean(ref * ref, axis=-1))
    err = np.abs(got - ref).max(axis=-1)
    bad = err > rel * rms
    assert not bad.any(), (f"{int(bad.sum())} of {bad.size} rows outside {rel} of row RMS; "
                           f"worst {float((err / np.maximum(rms, 1e-300)).max()):.3g}")
