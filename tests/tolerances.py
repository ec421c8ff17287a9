"""Parity bars between the HIP path and the oracle (float results).

fp32 outputs: |y - y*| <= 1e-3 * max(|y*|, rms(y*[c, :])) -- relative, with the
denominator floored at the RMS of that output vector so that results near
zero from cancellation do not fail spuriously.

bf16 outputs ("1e-2 relative to the row norm"), a row being one output
vector (out[c, :] or C[m, :]), two conditions:
  * normwise: ||y - y*||_2 <= 1e-2 * ||y*||_2 per row;
  * elementwise: |y_j - y*_j| <= 2^-8 * |y*_j| + 1e-3 * rms(y*_row).  Rounding
    a float32 result to bf16 (8 significant bits, RNE) moves it by at most
    half an ulp <= 2^-8 of its magnitude; the second term budgets the float32
    accumulation.  A bound of 1e-2 * rms alone is not met even by the exact
    result rounded to bf16 (an output at 5 rms may move by 2^-8 * 5 rms).
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


BF16_HALF_ULP = 2.0 ** -8
ACC_BUDGET = 1e-3


def check_bf16_rows(got, ref, rel=REL_BF16_ROW):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    diff = got - ref
    norm_err = np.sqrt(np.sum(diff * diff, axis=-1))
    norm_ref = np.sqrt(np.sum(ref * ref, axis=-1))
    bad = norm_err > rel * norm_ref
    assert not bad.any(), (f"{int(bad.sum())} of {bad.size} rows beyond {rel} normwise; worst "
                           f"{float((norm_err / np.maximum(norm_ref, 1e-300)).max()):.3g}")
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    bound = BF16_HALF_ULP * np.abs(ref) + ACC_BUDGET * rms
    badel = np.abs(diff) > bound
    assert not badel.any(), (f"{int(badel.sum())} of {badel.size} elements beyond "
                             f"2^-8|y*| + {ACC_BUDGET} rms; worst excess "
                             f"{float((np.abs(diff) / np.maximum(bound, 1e-300)).max()):.3g}x")


def check_bf16_rownorm(got, ref, rel=REL_BF16_ROW):
    """The normwise half of ``check_bf16_rows`` alone: ||y - y*|| <= rel ||y*||
    per row, for a reference that is not the kernel's own rounding chain."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = np.sqrt(np.sum((got - ref) ** 2, axis=-1))
    nrm = np.sqrt(np.sum(ref * ref, axis=-1))
    bad = err > rel * nrm
    assert not bad.any(), (f"{int(bad.sum())} of {bad.size} rows beyond {rel} normwise; worst "
                           f"{float((err / np.maximum(nrm, 1e-300)).max()):.3g}")
