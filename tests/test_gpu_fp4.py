"""GPU parity of the FP4 microscaling variant against the oracle.

* The MXFP4 stages (K mean, Q/K codes and E8M0 scales, V^T codes and scales,
  padding included) are compared with oracle/mxfp4 + sage_ref bit for bit: the
  rounding decisions are integer results, taken in the same precision on both
  sides (fp32 inputs, exact power-of-two scaling, round half to even).
* The attention output is compared with sage_ref.sage_attention_fp4 on every
  row at small sizes (several tiles, ragged tails, GQA, causal, both layouts
  and dtypes) and on one row per work-group and head at the full size of every
  large workload,
  at the method's bars (cosine >= 0.9999 and relative L1 <= 1e-3 against the
  oracle). Against fp64 exact attention the variant is checked to land where
  the oracle lands (FP4 is a coarser method: its own accuracy is the bound).
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import exact, sage_ref
from tests.parity_util import COS_ORACLE, RL1_ORACLE, check_heads, cos, rel_l1, rows_per_head, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sage():
    import quantized_attention_channel_amd as m
    return m


def _hnd(t, layout):
    return sage_ref.as_hnd(t.float().cpu().numpy(), layout)


def _pack(codes):
    """One E2M1 code per byte -> two per byte, element 2i in the low nibble."""
    c = np.asarray(codes, np.uint8)
    return ((c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)).astype(np.uint8)


def _unpack(packed):
    p = np.asarray(packed, np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def check_fp4_stages(got, qn, kn, vn, sm_scale):
    """Every MXFP4 stage bit for bit; returns the oracle's parts (with vd)."""
    parts = sage_ref.quant_qk_fp4(qn, kn, sm_scale=sm_scale)
    v4, vexp, vd = sage_ref.quant_v_fp4(vn)
    N = kn.shape[2]
    assert np.array_equal(got["k_mean"].cpu().numpy().view(np.uint32), parts["k_mean"].view(np.uint32))
    assert np.array_equal(got["q_codes"].cpu().numpy(), _pack(parts["q4"]))
    assert np.array_equal(got["q_scale"].cpu().numpy(), (parts["q_exp"] + 127).astype(np.uint8))
    assert np.array_equal(got["k_codes"].cpu().numpy(), _pack(parts["k4"]))
    assert np.array_equal(got["k_scale"].cpu().numpy(), (parts["k_exp"] + 127).astype(np.uint8))
    vc = _unpack(got["v_codes"].cpu().numpy())                       # [B,H,d,npad]
    assert np.array_equal(vc[..., :N], np.swapaxes(v4, 2, 3))
    assert not vc[..., N:].any(), "padding keys must be code 0"
    vs = got["v_scale"].cpu().numpy()                                # [B,H,npad/128,d,4]
    vs = np.swapaxes(vs, 2, 3).reshape(vs.shape[0], vs.shape[1], vs.shape[3], -1)   # [B,H,d,npad/32]
    nb = vexp.shape[2]
    assert np.array_equal(vs[..., :nb], np.swapaxes(vexp + 127, 2, 3).astype(np.uint8))
    assert not vs[..., nb:].any(), "blocks past the keys must have scale byte 0"
    parts["vd"] = vd
    return parts


QUANT_CASES = [
    W.TINY,                                                              # d=64 fp16 HND, 2 tiles
    W.TINY.with_(B=2, Hq=4, Hkv=2, N=200, d=64, dtype="bf16", layout="NHD"),
    W.TINY.with_(Hq=2, Hkv=1, N=300, d=128),                             # ragged, GQA
    W.TINY.with_(Hq=4, Hkv=4, N=129, d=128, dtype="bf16", k_off_var=40.0),
    W.TINY.with_(Hq=1, Hkv=1, N=1, d=128),                               # one token
    W.TINY.with_(Hq=2, Hkv=2, N=33, d=64, layout="NHD", outliers=3),     # one full and one 1-key block
]


@pytest.mark.parametrize("w", QUANT_CASES, ids=lambda w: f"{w.N}x{w.d}_{w.dtype}_{w.layout}_h{w.Hq}k{w.Hkv}")
def test_fp4_quant_stages_bit_exact(sage, w):
    say("fp4 quant", w)
    q, k, v = W.generate(w)
    got = sage.sage_quant_fp4(q.cuda(), k.cuda(), v.cuda(), tensor_layout=w.layout, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    check_fp4_stages(got, *(_hnd(t, w.layout) for t in (q, k, v)), w.sm_scale)


def test_fp4_quant_scale_edges(sage):
    """Blocks at the edges of the scale rule (bf16 inputs, which reach the
    clamp): all zeros (scale byte 0), values that saturate, every rounding tie
    of E2M1, small normals, a block whose maximum 2^-125 puts the exponent at
    the E8M0 floor, and a block of subnormals below it."""
    d = 64
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
    tie_row = np.tile(np.concatenate([ties, -ties]), d // 16)
    rows = [np.zeros(d), np.full(d, 6.0), np.concatenate([[4.0], np.full(d - 1, 5.0)]), tie_row,
            tie_row * 2.0 ** -14, np.concatenate([[2.0 ** -125], np.full(d - 1, -(2.0 ** -127))]),
            np.tile([2.0 ** -130, -(2.0 ** -131)], d // 2), tie_row[::-1] * 3.0, tie_row * 1e4]
    x = np.array(rows, np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16).reshape(1, 1, x.shape[0], d)
    # score factor exactly 1 (Q's blocks hit the listed edges unscaled), then
    # an ordinary one
    for sm in (1.0 / sage_ref.LOG2E, 0.125):
        got = sage.sage_quant_fp4(t.cuda(), t.cuda(), t.cuda(), sm_scale=sm)
        torch.cuda.synchronize()
        tn = t.float().numpy()
        check_fp4_stages(got, tn, tn, tn, sm)


ATTN_CASES = [
    (W.TINY, False),
    (W.TINY, True),
    (W.TINY.with_(B=2, Hq=4, Hkv=2, N=200, d=64, dtype="bf16", layout="NHD"), False),
    (W.TINY.with_(B=2, Hq=4, Hkv=2, N=200, d=64, dtype="bf16", layout="NHD"), True),
    (W.TINY.with_(Hq=2, Hkv=1, N=300, d=128), False),
    (W.TINY.with_(Hq=2, Hkv=1, N=300, d=128), True),
    (W.TINY.with_(Hq=4, Hkv=2, N=1000, d=128, dtype="bf16"), True),
    (W.TINY.with_(Hq=2, Hkv=2, N=640, d=128, outliers=4), False),
    (W.TINY.with_(Hq=2, Hkv=2, N=129, d=64), True),
    (W.TINY.with_(Hq=1, Hkv=1, N=1, d=128), False),
    # d = 64 with an odd key count, seen by every row: the last key's two K scale
    # bytes share a 4-byte word with the bytes past the head's range
    (W.TINY.with_(Hq=2, Hkv=1, N=257, d=64, dtype="bf16"), False),
    (W.TINY.with_(B=2, Hq=2, Hkv=1, N=129, d=64, layout="NHD", k_off_var=40.0), False),
]


def _attn_case(sage, w, causal):
    q, k, v = W.generate(w)
    o = sage.sage_attn_fwd_fp4(q.cuda(), k.cuda(), v.cuda(), is_causal=causal, sm_scale=w.sm_scale,
                               tensor_layout=w.layout)
    torch.cuda.synchronize()
    qn, kn, vn = (_hnd(t, w.layout) for t in (q, k, v))
    ref = sage_ref.sage_attention_fp4(qn, kn, vn, dtype=w.dtype, is_causal=causal, sm_scale=w.sm_scale)
    return q, k, v, _hnd(o, w.layout), ref, (qn, kn, vn)


@pytest.mark.parametrize("w,causal", ATTN_CASES,
                         ids=lambda x: x if isinstance(x, bool) else f"{x.N}x{x.d}_{x.dtype}_{x.layout}_h{x.Hq}k{x.Hkv}")
def test_fp4_attention_matches_oracle(sage, w, causal):
    say("fp4 attention", w, "causal" if causal else "")
    q, k, v, got, ref, (qn, kn, vn) = _attn_case(sage, w, causal)
    assert np.isfinite(got).all()
    c, r = cos(got, ref), rel_l1(got, ref)
    wc, wr = check_heads([got[b, h] for b in range(w.B) for h in range(w.Hq)],
                         [ref[b, h] for b in range(w.B) for h in range(w.Hq)])
    ex = exact.exact_attention(qn, kn, vn, is_causal=causal, sm_scale=w.sm_scale)
    ce, ce_oracle = cos(got, ex), cos(ref, ex)
    say(f"   cos={c:.7f} rel_l1={r:.2e} worst head cos={wc:.7f}; vs fp64: HIP {ce:.5f} oracle {ce_oracle:.5f}")
    assert c >= COS_ORACLE and r <= RL1_ORACLE
    assert abs(ce - ce_oracle) <= 1e-3


def test_fp4_codes_entry_equals_whole_forward(sage):
    w = W.TINY.with_(Hq=4, Hkv=2, N=300, d=128, dtype="bf16")
    q, k, v = (t.cuda() for t in W.generate(w))
    whole = sage.sage_attn_fwd_fp4(q, k, v, is_causal=True, sm_scale=w.sm_scale)
    codes = sage.sage_quant_fp4(q, k, v, sm_scale=w.sm_scale)
    o = torch.empty_like(q)
    sage.sage_attn_fwd_fp4_codes(sage.shape_of(q, k, "HND"), codes, o, is_causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, whole)
    again = sage.sage_attn_fwd_fp4(q, k, v, is_causal=True, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(again, whole), "deterministic"


def test_fp4_codes_entry_at_d64_with_an_odd_scale_count(sage):
    """d = 64 and B * Hkv * Nk odd: the K scales end 2 bytes into a 4-byte word.
    The codes entry point (buffers from fp4_buffers, padded to whole words)
    equals the whole forward and the oracle; a K scale tensor without the
    padding is refused by the binding before any library call."""
    w = W.TINY.with_(Hq=2, Hkv=1, N=257, d=64)
    q, k, v = (t.cuda() for t in W.generate(w))
    whole = sage.sage_attn_fwd_fp4(q, k, v, sm_scale=w.sm_scale)
    codes = sage.sage_quant_fp4(q, k, v, sm_scale=w.sm_scale)
    o = torch.empty_like(q)
    shape = sage.shape_of(q, k, "HND")
    sage.sage_attn_fwd_fp4_codes(shape, codes, o)
    torch.cuda.synchronize()
    assert torch.equal(o, whole)
    ref = sage_ref.sage_attention_fp4(*(t.float().cpu().numpy() for t in (q, k, v)), dtype=w.dtype, is_causal=False,
                                      sm_scale=w.sm_scale)
    got = o.float().cpu().numpy()
    assert cos(got, ref) >= COS_ORACLE and rel_l1(got, ref) <= RL1_ORACLE
    exact_size = dict(codes, k_scale=codes["k_scale"].clone())
    with pytest.raises(ValueError, match="4-byte words"):
        sage.sage_attn_fwd_fp4_codes(shape, exact_size, o)


def test_fp4_zero_q_gives_mean_of_quantised_values(sage):
    """Q = 0: every score is 0, every P~ is 1 (an exact FP4 code), so each row is
    the mean of the dequantised V over the visible keys (closed form)."""
    w = W.TINY.with_(Hq=2, Hkv=2, N=300, d=128)
    q, k, v = W.generate(w)
    q = torch.zeros_like(q)
    for causal in (False, True):
        o = sage.sage_attn_fwd_fp4(q.cuda(), k.cuda(), v.cuda(), is_causal=causal, sm_scale=w.sm_scale)
        torch.cuda.synchronize()
        vd = sage_ref.quant_v_fp4(v.float().numpy())[2]
        want = (np.cumsum(vd, axis=2) / np.arange(1, w.N + 1)[None, None, :, None]) if causal else \
            np.broadcast_to(vd.mean(axis=2, keepdims=True), vd.shape)
        want = sage_ref._round_to(want, w.dtype)
        np.testing.assert_allclose(o.float().cpu().numpy(), want, rtol=2e-3, atol=1e-5)


def test_sageattn_fp4_routes_to_the_variant(sage):
    w = W.TINY.with_(Hq=2, Hkv=2, N=200, d=64, layout="NHD")
    q, k, v = (t.cuda() for t in W.generate(w))
    a = sage.sageattn(q, k, v, tensor_layout="NHD", is_causal=True, pv_dtype="fp4")
    b = sage.sage_attn_fwd_fp4(q, k, v, tensor_layout="NHD", is_causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    with pytest.raises(ValueError):
        sage.sageattn(q, k, v, tensor_layout="NHD", pv_dtype="fp4", qk_quant_gran="per_thread")


# ------------------------------------------------------------------ full size
FULL_SIZE = [W.MID_OUTLIER, W.GQA_CAUSAL, W.LONG_D64, W.PEAK]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("w", FULL_SIZE, ids=lambda w: w.name)
def test_fp4_full_size_workloads(sage, w):
    """Every large workload (the outlier workload, GQA causal NHD bf16, d = 64,
    and the benchmark's peak workload): the MXFP4 stages bit for bit for every
    (batch, head), and the output on one row of every work-group of every head
    plus the edge rows, per head and pooled."""
    say("fp4 full workload", w.name)
    q, k, v = W.generate(w)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    o = sage.sage_attn_fwd_fp4(qg, kg, vg, is_causal=w.causal, sm_scale=w.sm_scale, tensor_layout=w.layout)
    codes = sage.sage_quant_fp4(qg, kg, vg, tensor_layout=w.layout, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    del qg, kg, vg
    rows = rows_per_head(w.N, w.B * w.Hq)
    o_all = _hnd(o, w.layout)
    qa, ka, va = (_hnd(t, w.layout) for t in (q, k, v))
    G = w.Hq // w.Hkv
    got, ref, ex = [], [], []
    for b in range(w.B):
        bs = slice(b, b + 1)
        for h in range(w.Hq):
            hs, ks = slice(h, h + 1), slice(h // G, h // G + 1)
            one = {"q_codes": codes["q_codes"][bs, hs], "q_scale": codes["q_scale"][bs, hs]}
            one.update({n: codes[n][bs, ks] for n in ("k_codes", "k_scale", "k_mean", "v_codes", "v_scale")})
            qn, kn, vn = qa[bs, hs], ka[bs, ks], va[bs, ks]
            parts = check_fp4_stages(one, qn, kn, vn, w.sm_scale)
            r_h = rows[b * w.Hq + h]
            r = sage_ref.sage_attention_fp4(qn, kn, vn, dtype=w.dtype, is_causal=w.causal, sm_scale=w.sm_scale,
                                            rows=r_h, parts=parts)
            ref.append(r[0, 0])
            got.append(o_all[b, h, r_h])
            ex.append(exact.exact_attention(qn, kn, vn, is_causal=w.causal, sm_scale=w.sm_scale, rows=r_h)[0, 0])
        say(f"   batch {b}: {w.Hq} heads checked")
    assert all(np.isfinite(g).all() for g in got)
    wc, wr = check_heads(got, ref)
    Gt, R, E = (np.concatenate([np.ravel(x) for x in xs]) for xs in (got, ref, ex))
    c, r, ce, ceo = cos(Gt, R), rel_l1(Gt, R), cos(Gt, E), cos(R, E)
    say(f"   {sum(len(x) for x in rows)} rows: cos={c:.7f} rel_l1={r:.2e} worst head cos={wc:.7f} rel_l1={wr:.2e};"
        f" vs fp64: HIP {ce:.5f} oracle {ceo:.5f}")
    assert c >= COS_ORACLE and r <= RL1_ORACLE
    assert abs(ce - ceo) <= 1e-3


# ------------------------------------------------------------------ the longest sequence the ABI accepts
@pytest.mark.parametrize("d,causal", [(128, False), (64, True)], ids=["d128_noncausal", "d64_causal"])
def test_fp4_maximum_sequence_length(sage, d, causal):
    """N = 2^20 keys and queries (the ABI's limit): every MXFP4 stage in full,
    the output on rows at both ends and in between (buffer offsets, tile
    counts, the V^T padding and its tile-major scales at their largest)."""
    n = 1 << 20
    w = W.PEAK.with_(B=1, Hq=1, Hkv=1, N=n, d=d, causal=causal)
    say("fp4 maximum length", n, d, "causal" if causal else "")
    q, k, v = W.generate(w)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    o = sage.sage_attn_fwd_fp4(qg, kg, vg, is_causal=causal, sm_scale=w.sm_scale)
    codes = sage.sage_quant_fp4(qg, kg, vg, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    del qg, kg, vg
    qn, kn, vn = (_hnd(t, "HND") for t in (q, k, v))
    parts = check_fp4_stages(codes, qn, kn, vn, w.sm_scale)
    rows = np.array([0, 1, 127, 128, n // 2 + 77, n - 129, n - 1])
    got = o.float().cpu().numpy()[:, :, rows]
    ref = sage_ref.sage_attention_fp4(qn, kn, vn, dtype=w.dtype, is_causal=causal, sm_scale=w.sm_scale,
                                      rows=rows, parts=parts)
    ex = exact.exact_attention(qn, kn, vn, is_causal=causal, sm_scale=w.sm_scale, rows=rows)
    c, r, ce, ceo = cos(got, ref), rel_l1(got, ref), cos(got, ex), cos(ref, ex)
    say(f"   cos={c:.7f} rel_l1={r:.2e}; vs fp64: HIP {ce:.5f} oracle {ceo:.5f}")
    assert np.isfinite(got).all()
    assert c >= COS_ORACLE and r <= RL1_ORACLE
    assert abs(ce - ceo) <= 1e-3
