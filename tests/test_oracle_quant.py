"""Pins for the oracle's quantisation stages (CPU only).

* K channel mean: against an exact summation (math.fsum) and exact rational
  division, so the fp64 sum is shown to be exact on these inputs.
* INT8 per-block quantisation: hand-worked ties, the invariants any correct
  symmetric absmax quantiser satisfies (range, an extreme code of +-127 in every
  non-zero block, half-step reconstruction error), block locality and the
  ragged tail block.
* Smoothing: the smoothed K the oracle quantises has (dequantised) channel mean
  ~0 -- a dropped or sign-flipped smoothing step breaks it.
* V to FP8: range, per-channel extreme code, layout (keys contiguous per channel).
* INT32 QK^T: brute-force pure-Python integer dot products.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import workloads as W
from oracle import sage_ref
from oracle.fp8_e4m3 import e4m3_decode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _inputs(w):
    q, k, v = W.generate(w)
    return tuple(sage_ref.as_hnd(x.float().numpy(), w.layout) for x in (q, k, v))


SMALL = W.TINY.with_(B=2, Hq=4, Hkv=2, N=200, d=64)


def test_k_mean_is_exact_sum_correctly_divided():
    for w in (SMALL, SMALL.with_(dtype="bf16", d=128, N=333)):
        _, k, _ = _inputs(w)
        mu = sage_ref.k_channel_mean(k)
        B, H, N, d = k.shape
        for b in range(B):
            for h in range(H):
                for c in range(0, d, 7):
                    col = [float(x) for x in k[b, h, :, c]]
                    exact = Fraction(math.fsum(col))          # fsum is exact-then-rounded
                    assert float(exact) == float(np.sum(np.asarray(col, np.float64))), "fp64 sum not exact"
                    want = np.float32(float(exact / N))       # within one fp32 rounding of the exact mean
                    got = mu[b, h, c]
                    assert abs(float(got) - float(want)) <= float(np.spacing(np.float32(abs(want)))), (b, h, c)


def test_k_mean_is_exact_where_fp64_addition_would_round():
    """A channel whose plain fp64 running sum loses a term (2^60 + 1 - 2^60, all
    bf16-exact) still gets the exact mean; a channel within the fp64 bound is
    summed plainly and agrees with math.fsum."""
    k = np.zeros((1, 1, 3, 2), np.float32)
    k[0, 0, :, 0] = [2.0 ** 60, 1.0, -(2.0 ** 60)]
    k[0, 0, :, 1] = [0.5, 0.25, -0.125]
    assert float(np.sum(np.asarray(k[0, 0, :, 0], np.float64))) == 0.0     # the plain sum drops the 1
    mu = sage_ref.k_channel_mean(k)
    assert mu[0, 0, 0] == np.float32(1.0 / 3.0)
    assert mu[0, 0, 1] == np.float32(0.625 / 3.0)


def test_int8_worked_examples():
    with open(os.path.join(GOLDEN, "int8_rne_worked.txt")) as f:
        lines = [ln for ln in f if ln.strip() and not ln.startswith("#")]
    for ln in lines:
        vals, codes, scale = (part.split() for part in ln.split("|"))
        x = np.array([float(t) for t in vals], np.float32).reshape(1, 1, -1, 1)
        c, s = sage_ref.quant_int8_blocks(x, blk=x.shape[2])
        assert c.ravel().tolist() == [int(t) for t in codes], ln
        assert float(s.ravel()[0]) == float(scale[0])


@pytest.mark.parametrize("blk", [1, 16, 64, 128])
def test_int8_invariants(blk):
    rng = np.random.default_rng(blk)
    x = (rng.standard_normal((2, 3, 301, 64)) * rng.uniform(0.01, 100, (2, 3, 1, 64))).astype(np.float32)
    x[0, 0, :blk] = 0                                     # an all-zero block [R4]
    codes, scale = sage_ref.quant_int8_blocks(x, blk)
    nblk = -(-301 // blk)
    assert codes.dtype == np.int8 and scale.shape == (2, 3, nblk)
    assert np.abs(codes.astype(np.int32)).max() <= 127
    assert scale[0, 0, 0] == 0 and not codes[0, 0, :blk].any()
    for b in range(2):
        for h in range(3):
            for i in range(nblk):
                xb = x[b, h, i * blk:(i + 1) * blk].astype(np.float64)
                cb = codes[b, h, i * blk:(i + 1) * blk].astype(np.float64)
                s = float(scale[b, h, i])
                if not np.any(xb):
                    continue
                assert np.abs(cb).max() == 127                       # extreme element maps to +-127
                assert abs(s - np.abs(xb).max() / 127) <= 1e-7 * s   # s = a/127 to fp32 precision
                err = np.abs(xb - cb * s).max()
                assert err <= s * (0.5 + 1e-5), (b, h, i, err / s)   # half a step (+ fp32 roundings)


def test_int8_block_locality_and_tail():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((1, 1, 130, 16)).astype(np.float32)
    c0, s0 = sage_ref.quant_int8_blocks(x, 64)
    x2 = x.copy()
    x2[0, 0, 129, 3] = 1000.0                        # only the tail block (tokens 128..129) changes
    c1, s1 = sage_ref.quant_int8_blocks(x2, 64)
    assert s1.shape == (1, 1, 3)
    assert np.array_equal(c0[:, :, :128], c1[:, :, :128]) and np.array_equal(s0[:, :, :2], s1[:, :, :2])
    assert s1[0, 0, 2] == np.float32(np.float32(1000.0) / np.float32(127.0))
    assert c1[0, 0, 129, 3] == 127


def test_smoothed_k_has_zero_channel_mean():
    """Channel smoothing (glossary 概要) removes the per-channel offset."""
    w = SMALL.with_(N=512, k_off_var=25.0)
    q, k, v = _inputs(w)
    parts = sage_ref.quant_qk(q, k)
    blk = sage_ref.BLK_K
    deq = parts["k8"].astype(np.float64) * np.repeat(parts["k_scale"], blk, axis=2)[:, :, :k.shape[2], None]
    chan_mean = deq.mean(axis=2)
    half_step = parts["k_scale"].max(axis=2)[:, :, None] / 2
    assert np.all(np.abs(chan_mean) <= half_step + 1e-6)
    offset = k.astype(np.float64).mean(axis=2)
    assert np.abs(offset).max() > 5 * half_step.max()      # the offset was large before smoothing


def test_v_fp8_invariants_and_layout():
    w = SMALL.with_(N=300)
    _, _, v = _inputs(w)
    codes, scale = sage_ref.quant_v_fp8(v)
    B, H, N, d = v.shape
    assert codes.shape == (B, H, d, N) and codes.dtype == np.uint8
    vals = e4m3_decode(codes)
    assert not np.isnan(vals).any()
    assert np.all(np.abs(vals).max(axis=3) == 448.0)          # per-channel extreme code
    recon = np.swapaxes(vals, 2, 3) * scale[:, :, None, :]
    err = np.abs(recon - v)
    # half an e4m3 ulp: 2^-4 relative in the normal range, 2^-10 (code units) below 2^-6
    bound = 2.0 ** -4 * np.abs(v) * (1 + 1e-6) + scale[:, :, None, :] * 2.0 ** -10
    assert np.all(err <= bound)


def test_int32_qk_brute_force():
    rng = np.random.default_rng(3)
    for d in (64, 128):
        q8 = rng.integers(-127, 128, (9, d)).astype(np.int8)
        k8 = rng.integers(-127, 128, (13, d)).astype(np.int8)
        q8[0] = 127
        k8[0] = -127                                           # the extreme |S| = d * 127^2
        s = sage_ref.qk_int32(q8, k8)
        for i in range(9):
            for j in range(13):
                want = sum(int(a) * int(b) for a, b in zip(q8[i], k8[j]))
                assert s[i, j] == want
        assert s[0, 0] == -d * 127 * 127
