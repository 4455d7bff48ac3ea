"""OCP OFP8 E4M3 codec (the "e4m3fn" encoding), written from the format definition.

Format (OCP 8-bit Floating Point Specification, E4M3): 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits. Exponent field 0 encodes subnormals
m * 2^-9. The all-ones exponent with mantissa 111 is NaN (both signs); there is
no infinity, so S.1111.110 = 448 is the largest finite magnitude.

Encoding used by the method (SageAttention pages: P and V go to FP8 for the PV
product -- thu-ml/SageAttention repo card, "How it works"; jisaku.com glossary,
概要): round to nearest, ties to even mantissa, saturating to +-448 for
magnitudes beyond the largest finite value (the OCP "saturate" conversion mode).
Inputs here are always scaled so that |x| <= 448 * (1 + 2^-22); saturation only
guards the last ulp.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_BIAS = 7
_MIN_NORMAL_EXP = 1 - E4M3_BIAS          # -6
_SUBNORMAL_QUANTUM_EXP = _MIN_NORMAL_EXP - 3  # 2^-9


def e4m3_decode(codes) -> np.ndarray:
    """Decode uint8 codes to float64 values (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.ldexp(1.0, e - E4M3_BIAS)
    sub = m * np.ldexp(1.0, _SUBNORMAL_QUANTUM_EXP)
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return sign * val


def e4m3_round(x) -> np.ndarray:
    """Round float32 values to the nearest finite E4M3 value (RNE, saturating).

    Returns float64 values that are exactly representable in E4M3.
    """
    a64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    if np.isnan(a64).any():
        raise ValueError("e4m3_round: NaN input")
    mag = np.abs(a64)
    # floor(log2 |x|) exactly, via frexp: |x| = f * 2^e with f in [0.5, 1).
    _, e = np.frexp(mag)
    expo = np.maximum(e - 1, _MIN_NORMAL_EXP)        # subnormal range shares 2^-6's quantum
    quantum = np.ldexp(1.0, expo - 3)                  # one mantissa ulp at that exponent
    r = np.rint(mag / quantum) * quantum               # exact scaling; np.rint is ties-to-even
    r = np.minimum(r, E4M3_MAX)                        # saturate (480 would be the NaN code)
    return np.copysign(r, a64)


def e4m3_encode(x) -> np.ndarray:
    """Encode float32 values to uint8 E4M3 codes (RNE, saturating)."""
    r = e4m3_round(x)
    sign = np.signbit(r).astype(np.int64)
    mag = np.abs(r)
    _, e = np.frexp(mag)
    expo = e - 1
    is_normal = mag >= np.ldexp(1.0, _MIN_NORMAL_EXP)
    exp_field = np.where(is_normal, expo + E4M3_BIAS, 0)
    mant_normal = np.where(is_normal, mag / np.ldexp(1.0, np.where(is_normal, expo, 0) - 3) - 8.0, 0)
    mant_sub = mag / np.ldexp(1.0, _SUBNORMAL_QUANTUM_EXP)
    mant = np.where(is_normal, mant_normal, mant_sub)
    mant_i = mant.astype(np.int64)
    assert np.all(mant_i == mant) and np.all((mant_i >= 0) & (mant_i < 8))
    code = (sign << 7) | (exp_field.astype(np.int64) << 3) | mant_i
    return code.astype(np.uint8)
