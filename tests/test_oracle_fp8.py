"""Pins for the oracle's E4M3 codec (CPU only).

The codec is checked against (1) the code points the OCP OFP8 specification
fixes, (2) hand-worked rounding cases, (3) a brute-force nearest-value search
over the decoded table -- a different algorithm from the oracle's arithmetic
rounding -- and (4) PyTorch's own float8_e4m3fn cast where that cast is defined
(|x| <= 464; above it torch returns NaN instead of saturating).
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle.fp8_e4m3 import e4m3_decode, e4m3_encode, e4m3_round

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def test_decode_spec_points():
    for code, val in _read("e4m3_spec_points.txt"):
        got = e4m3_decode(np.array([int(code, 16)], np.uint8))[0]
        if val == "nan":
            assert math.isnan(got), code
        else:
            assert got == float(val), (code, got, val)
            assert math.copysign(1.0, got) == math.copysign(1.0, float(val))


def test_decode_exhaustive_structure():
    vals = e4m3_decode(np.arange(256, dtype=np.uint8))
    assert np.isnan(vals).sum() == 2                      # only S.1111.111
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0)                       # monotonic over 0x00..0x7E
    assert np.array_equal(vals[0x80:0xFF], -vals[:0x7F])  # sign-magnitude symmetric
    assert pos.max() == 448.0
    # subnormal step 2^-9, and the normal range has 8 values per binade
    assert np.allclose(np.diff(pos[:9]), 2.0 ** -9)
    for e in range(1, 15):
        binade = pos[e * 8:(e + 1) * 8]
        assert np.all((binade >= 2.0 ** (e - 7)) & (binade < 2.0 ** (e - 6)))


def test_encode_worked_examples():
    for x, code in _read("e4m3_rounding_worked.txt"):
        got = int(e4m3_encode(np.array([float(x)], np.float32))[0])
        assert got == int(code, 16), (x, hex(got), code)


def _brute_force(xs):
    """Nearest finite E4M3 value by exhaustive search; ties -> even mantissa."""
    codes = np.arange(256, dtype=np.uint8)
    vals = e4m3_decode(codes)
    finite = ~np.isnan(vals)
    codes, vals = codes[finite], vals[finite]
    out = []
    for x in np.asarray(xs, np.float64):
        dist = np.abs(vals - x)
        best = dist.min()
        cand = codes[dist == best]
        cand_vals = vals[dist == best]
        if len(cand) > 1:
            even = [(c, v) for c, v in zip(cand, cand_vals) if (int(c) & 1) == 0]
            # +-0 both at distance |x|: keep the sign of x
            if all(v == 0 for _, v in even):
                c = 0x80 if math.copysign(1.0, x) < 0 else 0x00
                out.append(c)
                continue
            assert len(even) == 1
            out.append(int(even[0][0]))
        else:
            out.append(int(cand[0]))
    return np.array(out, np.uint8)


def _sweep_points():
    vals = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[1:] + vals[:-1]) / 2
    pts = [mids, vals, [464.0, 470.0, 480.0, 500.0, 1e4]]
    base = np.concatenate([np.asarray(p, np.float64) for p in pts]).astype(np.float32)
    up = np.nextafter(base, np.float32(np.inf))
    dn = np.nextafter(base, np.float32(0))
    allp = np.concatenate([base, up, dn])
    return np.concatenate([allp, -allp]).astype(np.float32)


def test_encode_matches_brute_force_at_every_midpoint():
    xs = _sweep_points()
    got = e4m3_encode(xs)
    want = _brute_force(xs)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(xs[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


def test_encode_matches_brute_force_random():
    rng = np.random.default_rng(0)
    xs = np.concatenate([
        rng.standard_normal(3000) * 50,
        rng.uniform(-1, 1, 3000) * 2.0 ** -6,
        np.exp2(rng.uniform(-12, 9, 3000)) * rng.choice([-1, 1], 3000),
    ]).astype(np.float32)
    assert np.array_equal(e4m3_encode(xs), _brute_force(xs))


def test_encode_matches_torch_cast_where_defined():
    rng = np.random.default_rng(1)
    xs = np.concatenate([_sweep_points(), (rng.standard_normal(100000) * 40).astype(np.float32)])
    xs = xs[np.abs(xs) <= 464].astype(np.float32)
    t = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(xs), t)


def test_round_is_decode_of_encode():
    rng = np.random.default_rng(2)
    xs = (rng.standard_normal(20000) * 100).astype(np.float32)
    assert np.array_equal(e4m3_round(xs), e4m3_decode(e4m3_encode(xs)))


def test_saturates_instead_of_nan():
    xs = np.array([448.0, 463.99, 464.0, 464.01, 479.0, 1e30, -1e30], np.float32)
    assert np.array_equal(e4m3_round(xs), [448, 448, 448, 448, 448, 448, -448])
    with pytest.raises(ValueError):
        e4m3_round(np.array([np.nan], np.float32))
