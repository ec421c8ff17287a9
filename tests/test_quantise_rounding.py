"""Host check of the rounding argument the int4 quantiser kernel relies on.

The kernel forms t = RN32(w * r + (8.5 + 2^-18)) with r = RN32(1 / s) in one
FMA and takes floor(t) as the code, falling back to the IEEE quotient when
fract(t) <= 2^-17.  The claim: whenever floor(t) differs from
clamp(rint(RN32(w / s)), -8, 7) + 8 (the definition the oracle follows),
fract(t) <= 2^-17.  Checked here over every finite fp16 weight against
scales s = bf16(absmax / 7) and s = float32(absmax / 7) for many absmax,
with the FMA emulated exactly in float64 (w r has at most 35 significant
bits) and one rounding to float32.  GPU parity of the kernel itself is in
tests/test_gpu_int4.py.
"""
import numpy as np


def _bf16_rne(x32):
    u = x32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32)


def _check(s32):
    w = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    w = w[np.isfinite(w)].astype(np.float32)
    w = w[np.abs(w) <= s32 * np.float32(7.0) * np.float32(1.0 + 2.0 ** -8)]  # |w| <= absmax
    q = np.rint(w / s32)                                     # RN32 quotient, then RNE
    want = (np.clip(q, -8, 7) + 8).astype(np.int64)
    r = np.float32(1.0) / s32
    c = np.float64(8.5) + np.float64(2.0 ** -18)
    t = (w.astype(np.float64) * np.float64(r) + c).astype(np.float32)  # one rounding
    got = np.floor(t).astype(np.int64)
    near = (t - np.floor(t)) <= np.float32(2.0 ** -17)
    bad = (got != want) & ~near
    assert not bad.any(), (s32, w[bad][:5], t[bad][:5], want[bad][:5])
    return int(near.sum()), w.size


def test_fast_code_path_is_exact_or_flagged():
    rng = np.random.default_rng(7)
    amax = np.concatenate([rng.uniform(1e-3, 0.2, 60), rng.uniform(0.2, 60000.0, 20),
                           np.array([2.0 ** -14, 6.0, 7.0, 0.5, 1.0, 3.5], dtype=np.float64)])
    flagged = total = 0
    for a in amax.astype(np.float32):
        s32 = a / np.float32(7.0)
        for s in (s32, _bf16_rne(np.array([s32], np.float32))[0]):
            if s == 0:
                continue
            f, n = _check(np.float32(s))
            flagged += f
            total += n
    # the fallback is rare: exact half-integer quotients (ties) and near-ties
    assert total > 1_000_000 and flagged < total // 100
