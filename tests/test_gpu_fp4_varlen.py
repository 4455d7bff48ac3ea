"""GPU parity of the FP4 microscaling variant over packed variable-length
batches (sage_attn_fwd_fp4_varlen, sage_quant_fp4_varlen) [R21-R24].

Each sequence of a packed batch is one independent FP4 attention: the oracle
runs sage_ref's FP4 stages and sage_attention_fp4 on every sequence as a batch
of one. The MXFP4 stages (K mean, Q/K codes and E8M0 scales, V^T codes and
scales at the sequence's padded columns, with their zero padding) must match bit
for bit; the output must meet cosine >= 0.9999 and relative L1 <= 1e-3 against
the oracle on the whole batch and on every sequence, and land where the oracle
lands against fp64 attention (FP4 is the coarser method). Mixes cover empty
sequences (no queries, or queries without keys), single tokens, lengths off
every 32-key block and 128-key tile, grouped-query heads, causal masking with
equal and unequal query and key counts, both head dims and both input dtypes.
One packed sequence must equal the dense FP4 entry point on the same tokens bit
for bit.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import exact, sage_ref
from tests.parity_util import COS_ORACLE, RL1_ORACLE, cos, rel_l1, say

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

if torch.cuda.is_available():
    import quantized_attention_channel_amd as sage

MIX = (0, 1, 17, 128, 129, 300, 1000)
CASES = [
    W.VarlenWorkload("fp4_mix_d128", MIX, MIX, Hq=2, Hkv=2, d=128, dtype="fp16", causal=False, pv="fp4"),
    W.VarlenWorkload("fp4_mix_d128_causal", MIX, MIX, Hq=2, Hkv=2, d=128, dtype="fp16", causal=True, pv="fp4"),
    W.VarlenWorkload("fp4_mix_bf16_gqa_causal", MIX, MIX, Hq=4, Hkv=2, d=128, dtype="bf16", causal=True, pv="fp4"),
    W.VarlenWorkload("fp4_gqa_d64_causal", (513, 2, 64, 255), (513, 2, 64, 255), Hq=4, Hkv=1, d=64, dtype="fp16",
                     causal=True, pv="fp4"),
    W.VarlenWorkload("fp4_cross", (5, 300, 0, 64, 40), (700, 1, 33, 0, 257), Hq=2, Hkv=2, d=128, dtype="fp16",
                     causal=False, pv="fp4"),
    W.VarlenWorkload("fp4_cross_d64_causal", (200, 50, 129), (100, 300, 129), Hq=2, Hkv=2, d=64, dtype="bf16",
                     causal=True, pv="fp4"),
    # d = 64, odd key counts seen by every row (the last key's K scales end
    # 2 bytes into a 4-byte word)
    W.VarlenWorkload("fp4_cross_d64_odd_keys", (5, 300, 64, 40), (701, 1, 33, 257), Hq=4, Hkv=2, d=64,
                     dtype="fp16", causal=False, pv="fp4"),
]


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


def _seq_hnd(x, a, b):
    """Tokens a..b-1 of a packed [total, H, d] array as a [1, H, n, d] batch."""
    return np.ascontiguousarray(x[a:b].transpose(1, 0, 2))[None]


def oracle_fp4_varlen(qn, kn, vn, cq, ck, *, dtype, is_causal, sm_scale):
    """The oracle's FP4 attention on every sequence as a batch of one; rows of
    sequences without queries or keys stay zero. Returns [total_q, Hq, d]."""
    out = np.zeros(qn.shape, np.float64)
    for b in range(len(cq) - 1):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        if q1 == q0 or k1 == k0:
            continue
        o = sage_ref.sage_attention_fp4(_seq_hnd(qn, q0, q1), _seq_hnd(kn, k0, k1), _seq_hnd(vn, k0, k1),
                                        dtype=dtype, is_causal=is_causal, sm_scale=sm_scale)
        out[q0:q1] = o[0].transpose(1, 0, 2)
    return out


def _run_gpu(w, q, k, v, cq, ck):
    o = sage.sage_attn_fwd_fp4_varlen(q.cuda(), k.cuda(), v.cuda(), cq.cuda(), ck.cuda(), max(w.lens_q),
                                      max(w.lens_k), is_causal=w.causal, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_fp4_varlen_all_rows(w):
    say("fp4 varlen", w.name, w.lens_q, w.lens_k)
    q, k, v, cq, ck = W.generate_varlen(w)
    got = _run_gpu(w, q, k, v, cq, ck)
    qn, kn, vn = (t.float().numpy() for t in (q, k, v))
    cqs, cks = cq.tolist(), ck.tolist()
    ref = oracle_fp4_varlen(qn, kn, vn, cqs, cks, dtype=w.dtype, is_causal=w.causal, sm_scale=w.sm_scale)
    assert np.isfinite(got).all()
    for b in range(w.B):
        if w.lens_k[b] == 0:
            assert not got[cqs[b]:cqs[b + 1]].any(), ("rows of a sequence without keys must be zero", b)
    c, r = cos(got, ref), rel_l1(got, ref)
    live = [b for b in range(w.B) if w.lens_q[b] and w.lens_k[b]]
    worst = min(cos(got[cqs[b]:cqs[b + 1]], ref[cqs[b]:cqs[b + 1]]) for b in live)
    ex = exact.exact_attention_varlen(qn, kn, vn, cqs, cks, is_causal=w.causal, sm_scale=w.sm_scale)
    ce, ce_oracle = cos(got, ex), cos(ref, ex)
    say(f"   cos={c:.7f} rel_l1={r:.2e} worst_sequence={worst:.7f}; vs fp64: HIP {ce:.5f} oracle {ce_oracle:.5f}")
    assert c >= COS_ORACLE and r <= RL1_ORACLE and worst >= COS_ORACLE
    assert abs(ce - ce_oracle) <= 1e-3


@pytest.mark.parametrize("causal,d,dtype", [(False, 128, "bf16"), (True, 128, "fp16"), (True, 64, "bf16")])
def test_one_packed_sequence_equals_the_dense_fp4_entry_point(causal, d, dtype):
    w = W.VarlenWorkload("one", (777,), (777,), Hq=4, Hkv=2, d=d, dtype=dtype, causal=causal, pv="fp4")
    say("fp4 varlen vs dense", causal, d, dtype)
    q, k, v, cq, ck = W.generate_varlen(w)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    o_var = sage.sage_attn_fwd_fp4_varlen(qg, kg, vg, cq.cuda(), ck.cuda(), 777, 777, is_causal=causal,
                                          sm_scale=w.sm_scale)
    o_dense = sage.sage_attn_fwd_fp4(qg[None], kg[None], vg[None], is_causal=causal, sm_scale=w.sm_scale,
                                     tensor_layout="NHD")
    torch.cuda.synchronize()
    assert torch.equal(o_var, o_dense[0])


def test_fp4_varlen_is_deterministic_and_ignores_workspace_contents():
    w = CASES[1]
    q, k, v, cq, ck = (t.cuda() for t in W.generate_varlen(w))
    shape = sage.varlen_shape_of(q, k, cq, max(w.lens_q), max(w.lens_k))
    ws = torch.full((sage.sage_fp4_varlen_workspace_bytes(shape),), 0x7F, dtype=torch.uint8, device="cuda")
    a = sage.sage_attn_fwd_fp4_varlen(q, k, v, cq, ck, max(w.lens_q), max(w.lens_k), is_causal=True,
                                      sm_scale=w.sm_scale, workspace=ws)
    b = sage.sage_attn_fwd_fp4_varlen(q, k, v, cq, ck, max(w.lens_q), max(w.lens_k), is_causal=True,
                                      sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.isfinite(a.float()).all()


def test_sageattn_varlen_routes_fp4():
    w = CASES[2]
    q, k, v, cq, ck = (t.cuda() for t in W.generate_varlen(w))
    a = sage.sageattn_varlen(q, k, v, cq, ck, max(w.lens_q), max(w.lens_k), is_causal=True, pv_dtype="fp4")
    b = sage.sage_attn_fwd_fp4_varlen(q, k, v, cq, ck, max(w.lens_q), max(w.lens_k), is_causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    with pytest.raises(ValueError):
        sage.sageattn_varlen(q, k, v, cq, ck, max(w.lens_q), max(w.lens_k), pv_dtype="fp4",
                             qk_quant_gran="per_thread")


# ------------------------------------------------------------------ MXFP4 stages per sequence, bit for bit
def check_fp4_varlen_quant(w):
    q, k, v, cq, ck = W.generate_varlen(w)
    got = sage.sage_quant_fp4_varlen(q.cuda(), k.cuda(), v.cuda(), cq.cuda(), ck.cuda(), max(w.lens_q),
                                     max(w.lens_k), sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    got = {n: t.cpu().numpy() for n, t in got.items()}
    qn, kn, vn = (t.float().numpy() for t in (q, k, v))
    vc = _unpack(got["v_codes"])                                        # [Hkv, d, npad]
    vs = got["v_scale"]                                                 # [Hkv, npad/128, d, 4]
    vs = np.swapaxes(vs, 1, 2).reshape(vs.shape[0], vs.shape[2], -1)    # [Hkv, d, npad/32]
    p = 0                                                               # first V column of the sequence
    for b in range(w.B):
        q0, q1, k0, k1 = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
        nq, nk = q1 - q0, k1 - k0
        kh = _seq_hnd(kn, k0, k1) if nk else np.zeros((1, w.Hkv, 1, w.d), np.float32)
        if nq:
            parts = sage_ref.quant_qk_fp4(_seq_hnd(qn, q0, q1), kh, sm_scale=w.sm_scale)
            assert np.array_equal(got["q_codes"][:, q0:q1], _pack(parts["q4"][0])), ("q codes", b)
            assert np.array_equal(got["q_scale"][:, q0:q1], (parts["q_exp"][0] + 127).astype(np.uint8)), b
        if nk:
            parts = sage_ref.quant_qk_fp4(np.zeros((1, w.Hq, 1, w.d), np.float32), kh, sm_scale=w.sm_scale)
            assert np.array_equal(got["k_mean"][b].view(np.uint32), parts["k_mean"][0].view(np.uint32)), b
            assert np.array_equal(got["k_codes"][:, k0:k1], _pack(parts["k4"][0])), ("k codes", b)
            assert np.array_equal(got["k_scale"][:, k0:k1], (parts["k_exp"][0] + 127).astype(np.uint8)), b
            v4, vexp, _ = sage_ref.quant_v_fp4(_seq_hnd(vn, k0, k1))
            pad = -(-nk // 128) * 128
            nb = vexp.shape[2]
            assert np.array_equal(vc[:, :, p:p + nk], np.swapaxes(v4[0], 1, 2)), ("v codes", b)
            assert not vc[:, :, p + nk:p + pad].any(), ("v padding", b)
            assert np.array_equal(vs[:, :, p // 32:p // 32 + nb], np.swapaxes(vexp[0] + 127, 1, 2).astype(np.uint8))
            assert not vs[:, :, p // 32 + nb:(p + pad) // 32].any(), ("v scale padding", b)
            p += pad
        else:
            assert not got["k_mean"][b].any(), ("k mean of a sequence without keys", b)


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_fp4_varlen_quant_stages_bit_exact(w):
    say("fp4 varlen quant stages", w.name)
    check_fp4_varlen_quant(w)


# ------------------------------------------------------------------ the serving mix at full size
@pytest.mark.timeout(900)
def test_fp4_varlen_serving_mix_full_size():
    """The serving mix (16 causal GQA sequences, 256 to 16384 tokens, bf16) at
    full size: the MXFP4 stages of every sequence bit for bit, and sampled rows
    of the longest, a middle and the shortest sequence against the oracle."""
    w = W.VARLEN_PREFILL.with_(pv="fp4")
    say("fp4 varlen full size", w.name)
    check_fp4_varlen_quant(w)
    q, k, v, cq, ck = W.generate_varlen(w)
    got = _run_gpu(w, q, k, v, cq, ck)
    assert np.isfinite(got).all()
    qn, kn, vn = (t.float().numpy() for t in (q, k, v))
    lens = list(w.lens_q)
    picks = [lens.index(max(lens)), lens.index(sorted(lens)[len(lens) // 2]), lens.index(min(lens))]
    for b in picks:
        q0, q1, k0, k1 = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
        rows = np.array(W.sample_rows(q1 - q0, 24, 128))
        qs, ks, vs = _seq_hnd(qn, q0, q1), _seq_hnd(kn, k0, k1), _seq_hnd(vn, k0, k1)
        ref = sage_ref.sage_attention_fp4(qs, ks, vs, dtype=w.dtype, is_causal=True, sm_scale=w.sm_scale,
                                          rows=rows)
        ex = exact.exact_attention(qs, ks, vs, is_causal=True, sm_scale=w.sm_scale, rows=rows)
        g = got[q0:q1][rows].transpose(1, 0, 2)[None]
        c, r, ce, ce_oracle = cos(g, ref), rel_l1(g, ref), cos(g, ex), cos(ref, ex)
        say(f"   seq {b} (len {q1 - q0}): cos={c:.7f} rel_l1={r:.2e}; vs fp64: HIP {ce:.5f} oracle {ce_oracle:.5f}")
        assert c >= COS_ORACLE and r <= RL1_ORACLE
        assert abs(ce - ce_oracle) <= 1e-3


# ------------------------------------------------------------------ bounds and degenerate batches
@pytest.mark.parametrize("fp4", [False, True])
def test_varlen_loose_bounds_give_the_same_output(fp4):
    """max_seqlen_q/k are bounds, not the exact maxima: looser bounds (a larger
    work list, more V tiles per sequence) change nothing in the output."""
    w = CASES[2]
    q, k, v, cq, ck = (t.cuda() for t in W.generate_varlen(w))
    mq, mk = max(w.lens_q), max(w.lens_k)
    say("varlen loose bounds", "fp4" if fp4 else "fp8", mq, mk)
    if fp4:
        run = lambda a, b: sage.sage_attn_fwd_fp4_varlen(q, k, v, cq, ck, a, b, is_causal=True)
    else:
        run = lambda a, b: sage.sage_attn_fwd_varlen(q, k, v, cq, ck, a, b, is_causal=True)
    exact_bounds = run(mq, mk)
    loose = run(3 * mq + 5, 2 * mk + 129)
    torch.cuda.synchronize()
    assert torch.equal(exact_bounds, loose)


@pytest.mark.parametrize("fp4", [False, True])
def test_varlen_without_any_keys_gives_zero_rows(fp4):
    """Queries but not a single key in the batch (total_k = 0): every output
    row is exactly zero, as for a sequence without keys."""
    w = W.VarlenWorkload("no_keys", (5, 300, 1), (0, 0, 0), Hq=4, Hkv=2, d=128, dtype="bf16", causal=False,
                         pv="fp4" if fp4 else "fp8")
    say("varlen without keys", w.pv)
    q, k, v, cq, ck = (t.cuda() for t in W.generate_varlen(w))
    assert k.shape[0] == 0
    for max_k in (0, 64):
        if fp4:
            o = sage.sage_attn_fwd_fp4_varlen(q, k, v, cq, ck, 300, max_k)
        else:
            o = sage.sage_attn_fwd_varlen(q, k, v, cq, ck, 300, max_k)
        torch.cuda.synchronize()
        assert o.shape == q.shape and not o.float().abs().sum().item(), max_k
