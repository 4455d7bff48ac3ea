"""Host check of the fused attention kernel's score representation.

In FP8 mode the kernel starts every INT32 QK^T product chain from the integer
0x4B400000 instead of zero and reads the results as fp32 bit patterns: the
float 1.5 * 2^23 + S, from which one fp32 subtraction recovers float(S). This
holds exactly when every score lies in [-2^22, 2^22], and the integer order of
the offset codes must be that of S (the row maximum runs on the integers).
The check covers every score a d = 128 tile can produce from INT8 codes,
-128 included (|S| <= 128 * 128 * 128 = 2^21), and the limits of the binade.
"""
import numpy as np

OFFSET = 0x4B400000
OFFSET_F = np.float32(12582912.0)


def _recovered(s):
    bits = (np.int64(OFFSET) + s.astype(np.int64)).astype(np.int32)
    return bits.view(np.float32) - OFFSET_F


def test_offset_codes_are_exact_floats():
    s = np.arange(-(1 << 21), (1 << 21) + 1, dtype=np.int32)
    assert np.array_equal(_recovered(s), s.astype(np.float32))


def test_offset_binade_limits():
    inside = np.array([-(1 << 22), (1 << 22)], dtype=np.int32)
    assert np.array_equal(_recovered(inside), inside.astype(np.float32))
    # one step past either end leaves the unit-spaced floats: the pattern no longer means 1.5 * 2^23 + S
    for v in (-(1 << 22) - 1, (1 << 22) + 1):
        assert _recovered(np.array([v], dtype=np.int32))[0] != np.float32(v)


def test_offset_codes_keep_the_integer_order():
    rng = np.random.default_rng(7)
    s = rng.integers(-(1 << 21), (1 << 21) + 1, size=100_000).astype(np.int32)
    codes = (np.int64(OFFSET) + s.astype(np.int64)).astype(np.int32)
    assert codes.min() > np.iinfo(np.int32).min       # the mask value stays below every score
    order = np.argsort(s, kind="stable")
    assert np.array_equal(np.argsort(codes, kind="stable"), order)
    assert np.array_equal(np.argsort(codes.view(np.float32), kind="stable"), order)
