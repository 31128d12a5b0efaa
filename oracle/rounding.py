"""Rounding to the storage and quantisation formats, from their definitions.

Test infrastructure only (see the package docstring).

* bfloat16: the upper 16 bits of an IEEE-754 binary32, rounded to nearest,
  ties to even, on the 16 discarded bits.
* binary16: IEEE-754 half precision; numpy's float16 cast is a correctly
  rounded (ties-to-even) conversion and serves as the library primitive.
* e4m3fn (OCP 8-bit floating point, E4M3 flavour): 1 sign, 4 exponent bits
  with bias 7, 3 mantissa bits; no infinities, S.1111.111 is NaN, largest
  finite value 448 = 1.75 * 2**8, smallest normal 2**-6, subnormals
  m * 2**-9 for m = 1..7.  Conversion rounds to nearest even; values beyond
  448 in magnitude saturate to 448 (the saturating conversion the variant
  needs, since its inputs are bounded by 448 by construction).
"""
from __future__ import annotations

import numpy as np


def f32_to_bf16_bits(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even; NaN stays NaN."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    if nan.any():
        r = np.where(nan, ((b >> 16) | 0x40).astype(np.uint16), r)
    return r


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """Value of x after rounding to bf16, as float64 (exact)."""
    return bf16_bits_to_f64(f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def f32_to_f16_bits(x) -> np.ndarray:
    """fp32 -> IEEE binary16 bit patterns (uint16), numpy's correctly rounded cast."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def round_f16(x) -> np.ndarray:
    """Value of x after rounding to IEEE binary16, as float64 (exact)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float64)


# ---- e4m3fn ---------------------------------------------------------------

E4M3_MAX = 448.0
_E4M3_BIAS = 7


def e4m3_bits_to_f64(bits) -> np.ndarray:
    """Decode e4m3fn bit patterns (uint8) to float64."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    normal = s * (1.0 + m / 8.0) * np.exp2(e - _E4M3_BIAS)
    sub = s * (m / 8.0) * np.exp2(1 - _E4M3_BIAS)
    v = np.where(e == 0, sub, normal)
    return np.where((e == 0xF) & (m == 0x7), np.nan, v)


# All 127 non-negative finite e4m3 magnitudes in increasing order (code = index).
_E4M3_POS = e4m3_bits_to_f64(np.arange(0, 0x7F, dtype=np.uint8))


def e4m3_nearest_by_search(x) -> np.ndarray:
    """Round to the nearest e4m3fn value (ties to the even code), saturating at
    448, by searching the table of all finite values.  Slow; used to pin
    ``round_e4m3``."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.minimum(np.searchsorted(_E4M3_POS, a, side="left"), len(_E4M3_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    vhi, vlo = _E4M3_POS[hi], _E4M3_POS[lo]
    dhi, dlo = vhi - a, a - vlo
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0)) | (vhi == a)
    v = np.where(pick_hi, vhi, vlo)
    v = np.where(np.signbit(x), -v, v)
    return np.where(np.isnan(x), np.nan, v)


def round_e4m3(x) -> np.ndarray:
    """Value of x after rounding to e4m3fn (ties to even, saturating at 448), as float64.

    Within a binade [2^e, 2^(e+1)) with e >= -6 the e4m3 values are spaced
    2^(e-3) (3 mantissa bits); below 2^-6 (subnormals) the spacing is 2^-9.
    Dividing by the spacing, rounding half to even and multiplying back is
    exact in float64.  Results beyond 448 saturate to 448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 2.0 * E4M3_MAX)   # keeps the exponent field finite
    e = (a.view(np.uint64) >> np.uint64(52)).astype(np.int64) - 1023   # binade of a
    e = np.maximum(e, -6)                     # subnormal range shares the 2^-6 spacing
    quantum = ((e - 3 + 1023).astype(np.uint64) << np.uint64(52)).view(np.float64)
    r = np.rint(a / quantum) * quantum
    r = np.minimum(r, E4M3_MAX)
    r = np.where(np.signbit(x), -r, r)
    return np.where(np.isnan(x), np.nan, r)


def f64_to_e4m3_bits(x) -> np.ndarray:
    """e4m3fn bit patterns of round_e4m3(x)."""
    v = round_e4m3(x)
    a = np.abs(v)
    code = np.searchsorted(_E4M3_POS, np.nan_to_num(a)).astype(np.uint8)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
    return np.where(np.isnan(v), np.uint8(0x7F), code | sign).astype(np.uint8)
