"""Pins for the oracle's MXFP4 codec and its FP4 attention variant (CPU only).

Codec (oracle/mxfp4.py), against the OCP Microscaling Formats (MX)
Specification v1.0:
  * every E2M1 code point the specification fixes (golden table);
  * hand-worked shared exponents and block quantisations (golden files), with
    every kind of rounding tie, saturation, signed zero, a zero block and a
    ragged last block;
  * a brute-force nearest-value search over the decoded code table -- a
    different algorithm from the oracle's quantum arithmetic.

Attention variant (sage_ref.sage_attention_fp4):
  * closed forms: Q = 0 (uniform weights: every P~ is 1, whose FP4 code is
    exact), causal row 0 (only key 0 is visible), identical keys (smoothing
    zeroes K), a single key;
  * V built exactly representable in MXFP4 per channel and 32 keys reaches the
    PV product unchanged (fails if V were blocked along the channels);
  * a hand-worked two-block P example: the P scale is per query row and 32
    keys, not per row or per tile, and the online rescale composes with it;
  * method accuracy against fp64 exact attention, with a K channel offset that
    only smoothing removes;
  * planted mistakes: each of several plausible codec or variant bugs fails one
    of the pins above.
"""
import math
import os

import numpy as np
import pytest

import workloads as W
from oracle import exact, sage_ref
from oracle import mxfp4 as mx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def _num(s):
    return float.fromhex(s) if s.lower().startswith(("0x", "-0x")) else float(s)


def cos(a, b):
    a, b = np.ravel(a).astype(np.float64), np.ravel(b).astype(np.float64)
    return float(a @ b / np.sqrt((a @ a) * (b @ b)))


# --------------------------------------------------------------------------- codec
def test_decode_spec_points():
    rows = _read("e2m1_spec_points.txt")
    assert len(rows) == 16
    for code, val in rows:
        got = mx.e2m1_decode(np.array([int(code, 16)], np.uint8))[0]
        assert got == float(val), (code, got, val)
        assert math.copysign(1.0, got) == math.copysign(1.0, float(val)), code


def test_encode_decode_round_trip_over_all_codes():
    codes = np.arange(16, dtype=np.uint8)
    vals = mx.e2m1_decode(codes)
    assert np.array_equal(mx.e2m1_encode(vals), codes)
    assert np.array_equal(mx.e2m1_round(vals), vals)


def _nearest_by_search(x):
    """Nearest E2M1 value by enumerating the 16 codes: smallest distance, a tie
    to the code with mantissa bit 0; magnitudes beyond 6 saturate."""
    codes = np.arange(16)
    table = mx.e2m1_decode(codes.astype(np.uint8))
    out = []
    for v in np.ravel(x):
        same_sign = [c for c in codes if (c >> 3) == (1 if math.copysign(1.0, v) < 0 else 0)]
        if abs(v) >= 6.0:
            best = max(same_sign, key=lambda c: abs(table[c]))
        else:
            dist = {c: abs(abs(v) - abs(table[c])) for c in same_sign}
            dmin = min(dist.values())
            ties = [c for c in same_sign if dist[c] == dmin]
            best = [c for c in ties if c % 2 == 0][0] if len(ties) > 1 else ties[0]
        out.append(table[best])
    return np.array(out).reshape(np.shape(x))


def test_round_equals_brute_force_search():
    rng = np.random.default_rng(5)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    grid = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 10), np.arange(0, 8.01, 1 / 64),
                           rng.uniform(0, 9, 3000), [6.0, 6.5, 7.0, 100.0, 1e30]])
    x = np.concatenate([grid, -grid])
    got = mx.e2m1_round(x)
    want = _nearest_by_search(x)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_round_refuses_nan():
    with pytest.raises(ValueError):
        mx.e2m1_round(np.array([1.0, np.nan]))


def test_block_exponent_worked_examples():
    for amax, e in _read("mx_scale_worked.txt"):
        got = int(mx.mx_block_exponent(np.array([_num(amax)]))[0])
        assert got == int(e), (amax, got, e)


def _worked_vector():
    blocks, vals, codes = [], [], []
    for row in _read("mxfp4_block_worked.txt"):
        if row[0] == "block":
            blocks.append(int(row[1]))
        else:
            vals.append(float(row[0]))
            codes.append(int(row[1], 16))
    return np.array(vals, np.float32), np.array(codes, np.uint8), np.array(blocks)


def test_block_quantisation_worked_example():
    x, codes, exps = _worked_vector()
    assert x.size == 104 and exps.size == 4
    c, e, dq = mx.mxfp4_quantize(x, axis=0)
    assert np.array_equal(e, exps), e
    assert np.array_equal(c, codes), [(float(v), int(a), int(b)) for v, a, b in zip(x, c, codes) if a != b]
    scale = np.ldexp(1.0, np.repeat(exps, 32)[:104])
    assert np.array_equal(dq, mx.e2m1_decode(codes) * scale)


def test_block_quantisation_follows_the_axis():
    """Blocks run along the given axis from index 0; the other axes are
    independent (a 2-D case built from the worked vector)."""
    x, codes, exps = _worked_vector()
    x2 = np.stack([x, 2 * x])                     # row 1: every exponent one higher, same codes
    c, e, dq = mx.mxfp4_quantize(x2.T, axis=0)    # [104, 2], blocks along axis 0
    assert np.array_equal(c[:, 0], codes) and np.array_equal(c[:, 1], codes)
    want_e = np.stack([exps, np.where(exps == -127, -127, exps + 1)], axis=1)
    assert np.array_equal(e, want_e)
    c1, e1, _ = mx.mxfp4_quantize(x2, axis=1)
    assert np.array_equal(c1, c.T) and np.array_equal(e1, e.T)


# --------------------------------------------------------------------------- attention variant
SMALL = W.TINY.with_(B=2, Hq=4, Hkv=2, N=200, d=64)


def _inputs(w):
    q, k, v = W.generate(w)
    return tuple(sage_ref.as_hnd(x.float().numpy(), w.layout) for x in (q, k, v))


def _fp4(q, k, v, causal, **kw):
    return sage_ref.sage_attention_fp4(q, k, v, dtype="fp16", is_causal=causal, sm_scale=q.shape[-1] ** -0.5,
                                       return_fp64=True, **kw)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_q_gives_mean_of_values(causal):
    q, k, v = _inputs(SMALL)
    q = np.zeros_like(q)
    out = _fp4(q, k, v, causal)
    vd = sage_ref.quant_v_fp4(v)[2]
    G = q.shape[1] // k.shape[1]
    for h in range(q.shape[1]):
        vh = vd[:, h // G]
        want = (np.cumsum(vh, axis=1) / np.arange(1, vh.shape[1] + 1)[None, :, None]) if causal else \
            np.broadcast_to(vh.mean(axis=1, keepdims=True), vh.shape)
        np.testing.assert_allclose(out[:, h], want, rtol=1e-12, atol=1e-12)


def test_causal_row0_is_value0():
    q, k, v = _inputs(SMALL)
    out = _fp4(q, k, v, True)
    vd = sage_ref.quant_v_fp4(v)[2]
    G = q.shape[1] // k.shape[1]
    for h in range(q.shape[1]):
        np.testing.assert_array_equal(out[:, h, 0], vd[:, h // G, 0])


def test_identical_keys_give_uniform_attention():
    q, k, v = _inputs(SMALL)
    k = np.broadcast_to(k[:, :, :1], k.shape).copy()
    out = _fp4(q, k, v, False)
    vd = sage_ref.quant_v_fp4(v)[2]
    G = q.shape[1] // k.shape[1]
    for h in range(q.shape[1]):
        np.testing.assert_allclose(out[:, h], np.broadcast_to(vd[:, h // G].mean(axis=1, keepdims=True),
                                                              out[:, h].shape), rtol=1e-12, atol=1e-12)


def test_single_key_returns_its_value():
    q, k, v = _inputs(SMALL)
    out = _fp4(q, k[:, :, :1], v[:, :, :1], False)
    vd = sage_ref.quant_v_fp4(v[:, :, :1])[2]
    G = q.shape[1] // k.shape[1]
    for h in range(q.shape[1]):
        np.testing.assert_array_equal(out[:, h], np.broadcast_to(vd[:, h // G, :1], out[:, h].shape))


def _mx_exact(shape, axis, rng):
    """Values exactly representable in MXFP4 with blocks of 32 along ``axis``:
    E2M1 values times a random power of two per block, each block holding a
    +-6 (so its shared exponent is the block's own)."""
    a = np.moveaxis(np.zeros(shape), axis, -1)
    n = a.shape[-1]
    nb = -(-n // 32)
    e = rng.integers(-6, 4, size=a.shape[:-1] + (nb,))
    vals = mx.e2m1_decode(rng.integers(0, 16, size=a.shape).astype(np.uint8))
    vals[..., ::32] = np.where(rng.random(vals[..., ::32].shape) < 0.5, 6.0, -6.0)
    a = vals * np.ldexp(1.0, np.repeat(e, 32, axis=-1)[..., :n])
    return np.moveaxis(a, -1, axis).astype(np.float32)


def test_mx_representable_operands_pass_unchanged():
    """Q and smoothed K exact per token and 32 channels, V exact per channel and
    32 keys: the codec is the identity on them, so each operand must come back
    bit for bit -- and would not with the blocks along another axis."""
    rng = np.random.default_rng(3)
    q = _mx_exact((1, 2, 100, 64), 3, rng)
    v = _mx_exact((1, 2, 100, 64), 2, rng)
    k = _mx_exact((1, 2, 100, 64), 3, rng)
    # sm_scale = 1 / log2(e): the score factor applied to Q is exactly 1
    unit = 1.0 / sage_ref.LOG2E
    assert sage_ref.fp4_score_factor(unit) == np.float32(1.0)
    parts = sage_ref.quant_qk_fp4(q, k, sm_scale=unit, k_mean=np.zeros((1, 2, 64), np.float32))
    np.testing.assert_array_equal(parts["qd"], q)
    np.testing.assert_array_equal(parts["kd"], k)
    np.testing.assert_array_equal(sage_ref.quant_v_fp4(v)[2], v)
    # the score factor scales Q before the quantisation: Q * 2 (a power of two)
    # gives the same codes one exponent up, and dequantises to 2 Q exactly
    two = sage_ref.quant_qk_fp4(q, k, sm_scale=2.0 * unit, k_mean=np.zeros((1, 2, 64), np.float32))
    np.testing.assert_array_equal(two["q4"], parts["q4"])
    np.testing.assert_array_equal(two["q_exp"], parts["q_exp"] + 1)
    np.testing.assert_array_equal(two["qd"], 2.0 * q)
    # and the Q = 0 closed form then reaches the plain mean of V
    out = _fp4(np.zeros_like(q), k, v, False)
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(v[0, 0].astype(np.float64).mean(axis=0), (100, 64)),
                               rtol=1e-13, atol=1e-13)


def _p_worked(order):
    """One query row over 64 keys in two 32-key blocks, log2-domain scores
    block A: -j and block B: -5 - j (j = 0..31), V = the 64 x 64 identity.
    ``order`` "AB" or "BA" puts block A first or second; ``bkv`` 32 makes each
    block its own KV tile."""
    a = -np.arange(32, dtype=np.float32)
    s2 = np.concatenate([a, a - 5] if order == "AB" else [a - 5, a])[None, :]
    return s2, np.eye(64)


@pytest.mark.parametrize("order,bkv", [("AB", 64), ("AB", 32), ("BA", 32), ("BA", 128)])
def test_p_fp4_worked_example(order, bkv):
    """Hand-worked: in block A, P~ = 2^-j and the block's max is 1, so its
    exponent is -2 and P~ / 2^-2 = 4, 2, 1, 0.5, 0.25 (tie -> 0), ...: the P
    entering PV is 1, 1/2, 1/4, 1/8 and then zeros. Block B's max is 2^-5
    (exponent -7): the same codes, values 2^-5 .. 2^-8. Row sum
    (1 + 1/32) * 15/8 = 1.93359375. With V = I the output row is P / l. When
    block B comes first in a tile of its own, the running max moves and alpha =
    2^-5 rescales it: the same result. (One scale per row or per tile would
    round every value of block B to 0.)"""
    s2, vals = _p_worked(order)
    o, l = sage_ref.online_softmax_pv(s2, vals, bkv=bkv, p_codec=sage_ref._p_codec_fp4, work_dtype=np.float32)
    head = np.array([1.0, 0.5, 0.25, 0.125])
    pa = np.concatenate([head, np.zeros(28)])
    pb = pa / 32.0
    want_p = np.concatenate([pa, pb] if order == "AB" else [pb, pa])
    assert l[0] == 1.93359375
    np.testing.assert_array_equal(o[0], want_p)


def _offset_workload(nk=256, d=64, off=8.0, seed=11):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, 2, nk, d)).astype(np.float32)
    k = (rng.standard_normal((1, 2, nk, d)) + off * rng.standard_normal((1, 2, 1, d))).astype(np.float32)
    v = rng.standard_normal((1, 2, nk, d)).astype(np.float32)
    return q, k, v


FP4_ACCURACY = [("offset", False, 0.96), ("offset", True, 0.96), ("small", False, 0.96)]


@pytest.mark.parametrize("which,causal,bound", FP4_ACCURACY)
def test_fp4_method_accuracy_vs_fp64(which, causal, bound):
    """The FP4 variant stays close to exact attention (cosine similarity over the
    output), also with a K channel offset eight times the per-token spread,
    which without smoothing would swamp the per-token part of K in 4-bit
    codes; it is less accurate than the INT8 method on the same input."""
    q, k, v = _offset_workload() if which == "offset" else _inputs(SMALL)
    sm = q.shape[-1] ** -0.5
    ref = exact.exact_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), is_causal=causal,
                          sm_scale=sm)
    got = _fp4(q, k, v, causal)
    c4 = cos(got, ref)
    assert c4 >= bound, c4
    c8 = cos(sage_ref.sage_attention(q, k, v, dtype="fp16", is_causal=causal, sm_scale=sm, pv="fp8",
                                     return_fp64=True), ref)
    assert c8 > c4


# --------------------------------------------------------------------------- planted mistakes
def _fails(check):
    try:
        check()
    except AssertionError:
        return True
    return False


def test_planted_mistakes_are_caught(monkeypatch):
    # 1. shared exponent off by one either way (emax 1 or 3)
    for off in (1, -1):
        orig = mx.mx_block_exponent
        with monkeypatch.context() as m:
            m.setattr(mx, "mx_block_exponent", lambda a, o=off, f=orig: np.clip(f(a) + o, -127, 127))
            assert _fails(test_block_exponent_worked_examples)
            assert _fails(test_block_quantisation_worked_example)
    # 2. ties rounded away from zero
    with monkeypatch.context() as m:
        m.setattr(mx.np, "rint", lambda x: np.trunc(np.asarray(x) + 0.5))
        assert _fails(test_block_quantisation_worked_example)
        assert _fails(test_round_equals_brute_force_search)
    # 3. no saturation (magnitudes above 6 kept, as a wider format would)
    orig_round = mx.e2m1_round
    with monkeypatch.context() as m:
        m.setattr(mx, "E2M1_MAX", 8.0)
        assert _fails(test_round_equals_brute_force_search)
    # 4. sign dropped on values that round to zero
    with monkeypatch.context() as m:
        m.setattr(mx, "e2m1_round", lambda x: np.where(orig_round(x) == 0, 0.0, orig_round(x)))
        assert _fails(test_block_quantisation_worked_example)
    # 5. P scaled once per row of the tile instead of per 32 keys
    with monkeypatch.context() as m:
        m.setattr(sage_ref, "_p_codec_fp4", _per_row_p)
        assert _fails(lambda: test_p_fp4_worked_example("AB", 64))
    # 6. V blocked along the channels instead of the keys
    orig_qv = sage_ref.quant_v_fp4
    with monkeypatch.context() as m:
        m.setattr(sage_ref, "quant_v_fp4", lambda v: mx.mxfp4_quantize(np.asarray(v, np.float32), axis=3))
        assert _fails(test_mx_representable_operands_pass_unchanged)
    # 7. Q blocked along the tokens instead of the channels
    orig_qk = sage_ref.quant_qk_fp4
    with monkeypatch.context() as m:
        def qk_token_blocks(q, k, *, sm_scale, k_mean=None):
            p = orig_qk(q, k, sm_scale=sm_scale, k_mean=k_mean)
            qs = (np.asarray(q, np.float32) * sage_ref.fp4_score_factor(sm_scale)).astype(np.float32)
            p["q4"], p["q_exp"], p["qd"] = mx.mxfp4_quantize(qs, axis=2)
            return p
        m.setattr(sage_ref, "quant_qk_fp4", qk_token_blocks)
        assert _fails(test_mx_representable_operands_pass_unchanged)
    # 8. K smoothing dropped in the FP4 variant
    with monkeypatch.context() as m:
        m.setattr(sage_ref, "smooth_k", lambda k, mu: np.asarray(k, np.float32))
        assert _fails(lambda: test_fp4_method_accuracy_vs_fp64(*FP4_ACCURACY[0]))
    # 9. log2(e) dropped from the score factor
    with monkeypatch.context() as m:
        m.setattr(sage_ref, "LOG2E", 1.0)
        assert _fails(lambda: test_fp4_method_accuracy_vs_fp64(*FP4_ACCURACY[2]))
    assert orig_qv is sage_ref.quant_v_fp4


def _per_row_p(p):
    """One MX scale for the whole row of the tile (the planted mistake 5)."""
    p = p.astype(np.float64)
    e = mx.mx_block_exponent(np.abs(p).max(axis=1))
    sc = np.ldexp(1.0, e)[:, None]
    return mx.e2m1_round(p / sc) * sc
