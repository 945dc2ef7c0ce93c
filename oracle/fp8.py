"""Oracle: the 8-bit float format E4M3 and the quantisation steps of the fp8 path.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The fp8 variant pairs ISPA with 8-bit arithmetic, as the technical summary's
results do when it combines ISPA with W8A8 post-training quantisation
("Technical Summary: Instance-Specific Parametric Absorption (ISPA) for
Memory-Efficient Video Generation", section 4 "Results").  The pages give no
format or scaling; the reading taken here is:

* format: E4M3 with the OCP "FN" encoding: 1 sign bit, 4 exponent bits with
  bias 7, 3 mantissa bits, subnormals below 2^-6 (spacing 2^-9), largest
  finite value 448 (bits S.1111.110), no infinities, S.1111.111 is NaN;
* rounding: to nearest, ties to even, of the float32 value x / scale;
* scale: amax / 448 in float32 over the block the scale covers (1 if amax = 0),
  so the largest magnitude maps to 448 exactly.

Codes are computed from the definition (exponent and mantissa split), not by a
library cast; the tests pin them against torch's float8_e4m3fn.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_encode(x) -> np.ndarray:
    """Codes (uint8) of float32 values |x| <= 448 rounded to nearest E4M3, ties to even."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)  # exact widening
    if np.any(np.isnan(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode: |x| must be <= 448 and not NaN")
    sign = (np.signbit(x)).astype(np.uint8) << 7
    a = np.abs(x)
    # exponent of the value's binade, clamped to the subnormal range (2^-6 and below share spacing 2^-9)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    step = np.exp2(e - 3.0)
    m = a / step                                   # in [0, 16): significand in units of the spacing
    r = np.floor(m)
    frac = m - r
    r = r + ((frac > 0.5) | ((frac == 0.5) & (np.mod(r, 2.0) == 1.0)))  # nearest, ties to even
    # r == 16 carries into the next binade (value step * 16 = 2^(e+1))
    carry = r >= 16.0
    e = np.where(carry, e + 1.0, e)
    r = np.where(carry, 8.0, r)
    sub = r < 8.0                                  # only possible when e == -6: subnormal
    exp_field = np.where(sub, 0.0, e + 7.0)
    man_field = np.where(sub, r, r - 8.0)
    code = (exp_field.astype(np.uint8) << 3) | man_field.astype(np.uint8)
    return (code | sign).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    """Float64 values of E4M3 codes (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    mf = c & 0x7
    val = np.where(ef == 0, mf * 2.0 ** -9, (1.0 + mf / 8.0) * np.exp2(ef - 7.0))
    val = np.where((ef == 15) & (mf == 7), np.nan, val)
    return s * val


def absmax_scale(x, axis=None) -> np.ndarray:
    """float32 scale amax / 448 over `axis` (1 where amax is 0)."""
    a = np.max(np.abs(np.asarray(x, dtype=np.float32)), axis=axis)
    a = np.asarray(a, dtype=np.float32)
    return np.where(a > 0, a / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)


def quantize(x, scale) -> np.ndarray:
    """Codes of x / scale (division in float32, as the format's input is a float32 value)."""
    q = np.asarray(x, dtype=np.float32) / np.asarray(scale, dtype=np.float32)
    return e4m3_encode(np.clip(q, -E4M3_MAX, E4M3_MAX))


def quantize_per_head(x) -> tuple:
    """[n, H, D] tensor -> (codes [n, H, D], scale [H]): one scale per head over all rows and dims."""
    x = np.asarray(x, dtype=np.float32)
    s = absmax_scale(x, axis=(0, 2))
    return quantize(x, s[None, :, None]), s


def dequantize(codes, scale) -> np.ndarray:
    """codes * scale in float64 (exact: both factors have few significant bits)."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)


def w8a8_matmul(a, w) -> np.ndarray:
    """W8A8 product y = deq(A8) deq(W8) in float64: A [n, d] quantised per row (token), W [d, d_out]
    per column (output channel), each with its own absmax scale."""
    a = np.asarray(a, dtype=np.float32)
    w = np.asarray(w, dtype=np.float32)
    sa = absmax_scale(a, axis=1)          # [n]
    sw = absmax_scale(w, axis=0)          # [d_out]
    a8 = quantize(a, sa[:, None])
    w8 = quantize(w, sw[None, :])
    return dequantize(a8, sa[:, None]) @ dequantize(w8, sw[None, :])
