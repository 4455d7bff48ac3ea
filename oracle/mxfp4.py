"""OCP Microscaling FP4 (MXFP4) codec, written from the format definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Element format, FP4 E2M1 (OCP Microscaling Formats (MX) Specification v1.0,
element data types): 1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit.
Exponent field 0 holds the subnormals m * 0.5; there is no infinity and no NaN.
Magnitudes: 0, 0.5, 1, 1.5, 2, 3, 4, 6 (largest normal 1.5 * 2^2).

Scale format, E8M0: an 8-bit biased exponent, bias 127, value 2^(E - 127)
(0xFF is NaN and never produced here).

MX block (same specification, conversion to MX): k = 32 elements share one
scale X = 2^(floor(log2(max_i |v_i|)) - emax_elem), emax_elem = 2 for E2M1 (the
exponent of its largest normal), clamped to the E8M0 range; each element is
v_i / X rounded to E2M1 with round-half-to-even, magnitudes beyond 6
saturating to 6. A block of zeros gets the smallest scale, 2^-127.

The SageAttention pages name FP4 microscaling for SageAttention3 (heatdrop.ai
review, "Key highlights"; cnnetsun.cn guide, 序列长度优化技巧) without a format;
this package reads it as MXFP4 (see ``sage_ref.sage_attention_fp4``).
"""
from __future__ import annotations

import numpy as np

E2M1_MAX = 6.0
E2M1_EMAX = 2
MX_BLOCK = 32
E8M0_BIAS = 127
E8M0_MIN_EXP = -127
E8M0_MAX_EXP = 127


def e2m1_decode(codes) -> np.ndarray:
    """Decode 4-bit codes (low nibble of each uint8) to float64 values."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64) & 0xF
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    normal = (1.0 + m / 2.0) * np.ldexp(1.0, e - 1)
    sub = m * 0.5
    return sign * np.where(e == 0, sub, normal)


def e2m1_round(x) -> np.ndarray:
    """Round values to the nearest E2M1 value (ties to even, saturating at +-6).

    The representable magnitudes are the multiples of 0.5 below 2, of 1 in
    [2, 4) and of 2 in [4, 6]; an even multiple has an even code, so rounding
    |x| / quantum half to even is round-half-to-even on the codes.
    """
    a = np.asarray(x, dtype=np.float64)
    if np.isnan(a).any():
        raise ValueError("e2m1_round: NaN input")
    mag = np.abs(a)
    quantum = np.where(mag < 2.0, 0.5, np.where(mag < 4.0, 1.0, 2.0))
    r = np.minimum(np.rint(mag / quantum) * quantum, E2M1_MAX)
    return np.copysign(r, a)


def e2m1_encode(x) -> np.ndarray:
    """E2M1 codes (uint8, low nibble) of values, rounded as e2m1_round."""
    r = e2m1_round(x)
    mag = np.abs(r)
    # code magnitude index: 0, 0.5, 1, 1.5, 2, 3, 4, 6 -> 0..7
    table = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    idx = np.searchsorted(table, mag)
    assert np.all(table[idx] == mag)
    return ((np.signbit(r).astype(np.int64) << 3) | idx).astype(np.uint8)


def mx_block_exponent(amax) -> np.ndarray:
    """Shared-scale exponent of MX blocks with the given max magnitudes:
    floor(log2 amax) - emax_elem, clamped to the E8M0 range; -127 for zero."""
    a = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(np.where(a > 0, a, 1.0))          # a = f 2^e, f in [0.5, 1): floor(log2 a) = e - 1
    x = np.clip(e - 1 - E2M1_EMAX, E8M0_MIN_EXP, E8M0_MAX_EXP)
    return np.where(a > 0, x, E8M0_MIN_EXP).astype(np.int64)


def mxfp4_quantize(x, axis: int):
    """MXFP4 quantisation of x (float64/float32) in blocks of 32 consecutive
    elements along ``axis``, from index 0 (a last partial block is a block of
    its own elements). Returns (codes uint8 like x, exponents int64 with the
    axis reduced to its block count, dequantised float64 like x)."""
    a = np.moveaxis(np.asarray(x, dtype=np.float64), axis, -1)
    n = a.shape[-1]
    nb = -(-n // MX_BLOCK)
    pad = nb * MX_BLOCK - n
    ap = np.concatenate([a, np.zeros(a.shape[:-1] + (pad,))], axis=-1) if pad else a
    blocks = ap.reshape(a.shape[:-1] + (nb, MX_BLOCK))
    ex = mx_block_exponent(np.abs(blocks).max(axis=-1))
    scale = np.ldexp(1.0, ex)[..., None]
    q = e2m1_round(blocks / scale)                       # exact division by a power of two
    codes = e2m1_encode(q).reshape(ap.shape)[..., :n]
    deq = (q * scale).reshape(ap.shape)[..., :n]
    return np.moveaxis(codes, -1, axis), np.moveaxis(ex, -1, axis), np.moveaxis(deq, -1, axis)
