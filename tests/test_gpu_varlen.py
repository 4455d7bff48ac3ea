"""GPU parity of packed variable-length batches (sage_attn_fwd_varlen) [R21].

Each sequence of a packed batch is one independent attention by the method;
the HIP path must meet the same bar per packed batch as the dense path:
cosine >= 0.9999 and sum|o-r|/sum|r| <= 1e-3 against the oracle, cosine >=
0.999 against fp64 exact attention. Mixes cover empty sequences (no queries,
or queries without keys), single tokens, lengths off every block and tile
boundary, grouped-query heads, causal masking with equal and unequal query
and key counts, both head dims, both input dtypes, both PV precisions and
per-thread scales. One packed sequence must equal the dense entry point on the
same tokens bit for bit.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import exact, sage_ref
from tests.parity_util import COS_EXACT, COS_ORACLE, RL1_ORACLE, cos, rel_l1, say

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

if torch.cuda.is_available():
    import quantized_attention_channel_amd as sage

GRAN_BLK = {"per_block": (sage_ref.BLK_Q, sage_ref.BLK_K),
            "per_thread": (sage_ref.PER_THREAD_BLK_Q, sage_ref.PER_THREAD_BLK_K)}

MIX = (0, 1, 17, 128, 129, 300, 1000)
CASES = [
    (W.VarlenWorkload("mix_d128_fp8", MIX, MIX, Hq=2, Hkv=2, d=128, dtype="fp16", causal=False, pv="fp8"),
     "per_block"),
    (W.VarlenWorkload("mix_d128_fp8_causal", MIX, MIX, Hq=2, Hkv=2, d=128, dtype="fp16", causal=True, pv="fp8"),
     "per_block"),
    (W.VarlenWorkload("mix_bf16_fp16_causal", MIX, MIX, Hq=4, Hkv=2, d=128, dtype="bf16", causal=True, pv="fp16"),
     "per_block"),
    (W.VarlenWorkload("gqa_d64_fp8_causal", (513, 2, 64, 255), (513, 2, 64, 255), Hq=4, Hkv=1, d=64,
                      dtype="fp16", causal=True, pv="fp8"), "per_block"),
    (W.VarlenWorkload("cross_fp16", (5, 300, 0, 64, 40), (700, 1, 33, 0, 257), Hq=2, Hkv=2, d=128, dtype="fp16",
                      causal=False, pv="fp16"), "per_block"),
    (W.VarlenWorkload("cross_fp8_causal", (200, 50, 129), (100, 300, 129), Hq=2, Hkv=2, d=64, dtype="fp16",
                      causal=True, pv="fp8"), "per_block"),
    (W.VarlenWorkload("mix_per_thread", MIX, MIX, Hq=2, Hkv=2, d=128, dtype="fp16", causal=True, pv="fp8"),
     "per_thread"),
    (W.VarlenWorkload("d64_per_thread", (77, 1, 333), (77, 1, 333), Hq=2, Hkv=2, d=64, dtype="bf16", causal=False,
                      pv="fp16"), "per_thread"),
]


def _run_gpu(w, gran, q, k, v, cq, ck):
    o = sage.sage_attn_fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cq.cuda(), ck.cuda(), max(w.lens_q),
                                  max(w.lens_k), is_causal=w.causal, sm_scale=w.sm_scale, pv_dtype=w.pv,
                                  qk_gran=gran)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("w,gran", CASES, ids=[f"{w.name}-{g}" for w, g in CASES])
def test_varlen_all_rows(w, gran):
    say("varlen", w.name, gran, w.lens_q, w.lens_k)
    q, k, v, cq, ck = W.generate_varlen(w)
    got = _run_gpu(w, gran, q, k, v, cq, ck)
    qn, kn, vn = (t.float().numpy() for t in (q, k, v))
    bq, bk = GRAN_BLK[gran]
    ref = sage_ref.sage_attention_varlen(qn, kn, vn, cq.tolist(), ck.tolist(), dtype=w.dtype, is_causal=w.causal,
                                         sm_scale=w.sm_scale, pv=w.pv, blk_q=bq, blk_k=bk)
    ex = exact.exact_attention_varlen(qn, kn, vn, cq.tolist(), ck.tolist(), is_causal=w.causal,
                                      sm_scale=w.sm_scale)
    assert np.isfinite(got).all()
    # rows of sequences without keys are exactly zero
    for b in range(w.B):
        if w.lens_k[b] == 0:
            assert not got[cq[b]:cq[b + 1]].any()
    c, r, ce = cos(got, ref), rel_l1(got, ref), cos(got, ex)
    worst = min(cos(got[cq[b]:cq[b + 1]], ref[cq[b]:cq[b + 1]]) for b in range(w.B)
                if w.lens_q[b] and w.lens_k[b])
    say(f"   cos={c:.7f} rel_l1={r:.2e} cos_exact={ce:.6f} worst_sequence={worst:.7f}")
    assert c >= COS_ORACLE and r <= RL1_ORACLE and worst >= COS_ORACLE
    assert ce >= COS_EXACT


@pytest.mark.parametrize("causal,pv,gran", [(False, "fp8", "per_block"), (True, "fp16", "per_block"),
                                            (True, "fp8", "per_thread")])
def test_one_packed_sequence_equals_the_dense_entry_point(causal, pv, gran):
    w = W.VarlenWorkload("one", (777,), (777,), Hq=4, Hkv=2, d=128, dtype="bf16", causal=causal, pv=pv)
    say("varlen vs dense", causal, pv, gran)
    q, k, v, cq, ck = W.generate_varlen(w)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    o_var = sage.sage_attn_fwd_varlen(qg, kg, vg, cq.cuda(), ck.cuda(), 777, 777, is_causal=causal,
                                      sm_scale=w.sm_scale, pv_dtype=pv, qk_gran=gran)
    o_dense = sage.sage_attn_fwd(qg[None], kg[None], vg[None], is_causal=causal, sm_scale=w.sm_scale,
                                 pv_dtype=pv, tensor_layout="NHD", qk_gran=gran)
    torch.cuda.synchronize()
    assert torch.equal(o_var, o_dense[0])


def test_varlen_is_deterministic_and_ignores_workspace_contents():
    w = CASES[1][0]
    q, k, v, cq, ck = (t.cuda() for t in W.generate_varlen(w))
    need = sage.sage_varlen_workspace_bytes(sage.varlen_shape_of(q, k, cq, max(w.lens_q), max(w.lens_k)), "fp8")
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")       # stale bytes: NaN-like floats
    a = sage.sage_attn_fwd_varlen(q, k, v, cq, ck, max(w.lens_q), max(w.lens_k), is_causal=True,
                                  sm_scale=w.sm_scale, workspace=ws)
    b = sage.sage_attn_fwd_varlen(q, k, v, cq, ck, max(w.lens_q), max(w.lens_k), is_causal=True,
                                  sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.isfinite(a.float()).all()


def test_sageattn_varlen_wrapper():
    w = CASES[0][0]
    q, k, v, cq, ck = (t.cuda() for t in W.generate_varlen(w))
    a = sage.sageattn_varlen(q, k, v, cq, ck, max(w.lens_q), max(w.lens_k), sm_scale=w.sm_scale)
    b = sage.sage_attn_fwd_varlen(q, k, v, cq, ck, max(w.lens_q), max(w.lens_k), sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    with pytest.raises(TypeError):
        sage.sageattn_varlen(q, k, v, cq.long(), ck.long(), max(w.lens_q), max(w.lens_k))


def test_varlen_serving_mix_full_size():
    """The benchmark's serving mix at full size; sampled rows of the longest,
    a middle and the shortest sequence against the oracle."""
    w = W.VARLEN_PREFILL
    say("varlen full size", w.name)
    q, k, v, cq, ck = W.generate_varlen(w)
    got = _run_gpu(w, "per_block", q, k, v, cq, ck)
    assert np.isfinite(got).all()
    qn, kn, vn = (t.float().numpy() for t in (q, k, v))
    lens = list(w.lens_q)
    picks = [lens.index(max(lens)), lens.index(sorted(lens)[len(lens) // 2]), lens.index(min(lens))]
    for b in picks:
        q0, q1, k0, k1 = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
        rows = np.array(W.sample_rows(q1 - q0, 24, sage_ref.BLK_Q))
        ref = sage_ref.sage_attention(qn[None, q0:q1], kn[None, k0:k1], vn[None, k0:k1], dtype=w.dtype,
                                      is_causal=w.causal, sm_scale=w.sm_scale, pv=w.pv, layout="NHD", rows=rows)
        ex = exact.exact_attention(qn[None, q0:q1].transpose(0, 2, 1, 3), kn[None, k0:k1].transpose(0, 2, 1, 3),
                                   vn[None, k0:k1].transpose(0, 2, 1, 3), is_causal=w.causal, sm_scale=w.sm_scale,
                                   rows=rows)
        g = got[q0:q1][rows].transpose(1, 0, 2)[None]
        c, r, ce = cos(g, ref), rel_l1(g, ref), cos(g, ex)
        say(f"   seq {b} (len {q1 - q0}): cos={c:.7f} rel_l1={r:.2e} cos_exact={ce:.6f}")
        assert c >= COS_ORACLE and r <= RL1_ORACLE and ce >= COS_EXACT


def test_varlen_longest_sequence():
    """A packed batch whose longest sequence is the limit (2^20 tokens) between
    two short ones: spans, packed offsets, padded V^T columns and the work list
    at their largest, one query head (the plain round-robin order). Rows at both
    ends and in the middle of the long sequence, and every row of a short one,
    against the oracle."""
    n = 1 << 20
    w = W.VarlenWorkload("longest", (300, n, 77), (300, n, 77), Hq=1, Hkv=1, d=128, dtype="fp16", causal=True,
                         pv="fp8")
    say("varlen longest sequence", n)
    q, k, v, cq, ck = W.generate_varlen(w)
    got = _run_gpu(w, "per_block", q, k, v, cq, ck)
    assert np.isfinite(got).all()
    qn, kn, vn = (t.float().numpy() for t in (q, k, v))
    for b, rows in ((1, np.array([0, 1, 127, 128, n // 2 + 77, n - 129, n - 1])), (2, np.arange(77))):
        q0, q1, k0, k1 = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
        ref = sage_ref.sage_attention(qn[None, q0:q1], kn[None, k0:k1], vn[None, k0:k1], dtype=w.dtype,
                                      is_causal=True, sm_scale=w.sm_scale, pv=w.pv, layout="NHD", rows=rows)
        ex = exact.exact_attention(qn[None, q0:q1].transpose(0, 2, 1, 3), kn[None, k0:k1].transpose(0, 2, 1, 3),
                                   vn[None, k0:k1].transpose(0, 2, 1, 3), is_causal=True, sm_scale=w.sm_scale,
                                   rows=rows)
        g = got[q0:q1][rows].transpose(1, 0, 2)[None]
        c, r, ce = cos(g, ref), rel_l1(g, ref), cos(g, ex)
        say(f"   seq {b}: cos={c:.7f} rel_l1={r:.2e} cos_exact={ce:.6f}")
        assert c >= COS_ORACLE and r <= RL1_ORACLE and ce >= COS_EXACT


# ------------------------------------------------------------------ integer stages per sequence, bit for bit
def check_varlen_quant(w, gran):
    """sage_quant_varlen against the oracle, sequence by sequence: K mean, Q/K
    codes and scales, V e4m3 codes (with their zero padding) and scales, or the
    transposed 16-bit V in FP16 mode, all bit for bit [R21]."""
    q, k, v, cq, ck = W.generate_varlen(w)
    got = sage.sage_quant_varlen(q.cuda(), k.cuda(), v.cuda(), cq.cuda(), ck.cuda(), max(w.lens_q), max(w.lens_k),
                                 pv_dtype=w.pv, qk_gran=gran)
    torch.cuda.synchronize()
    got = {n: t.cpu() for n, t in got.items()}
    bq, bk = GRAN_BLK[gran]
    qn, kn, vn = (t.float().numpy() for t in (q, k, v))
    p = 0                                              # first V column of the sequence
    for b in range(w.B):
        q0, q1, k0, k1 = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
        nq, nk = q1 - q0, k1 - k0
        if nq:
            ref = sage_ref.quant_int8_blocks(np.ascontiguousarray(qn[q0:q1].transpose(1, 0, 2))[None], bq)
            assert np.array_equal(got["q_codes"][:, q0:q1].numpy(), ref[0][0]), ("q codes", b)
            assert np.array_equal(got["q_scale"][b, :, :ref[1].shape[2]].numpy(), ref[1][0]), ("q scale", b)
        if nk:
            kh = np.ascontiguousarray(kn[k0:k1].transpose(1, 0, 2))[None]
            ref = sage_ref.quant_qk(np.zeros_like(kh[:, :, :1]), kh, blk_q=bq, blk_k=bk)
            assert np.array_equal(got["k_mean"][b].numpy(), ref["k_mean"][0]), ("k mean", b)
            assert np.array_equal(got["k_codes"][:, k0:k1].numpy(), ref["k8"][0]), ("k codes", b)
            assert np.array_equal(got["k_scale"][b, :, :ref["k_scale"].shape[2]].numpy(), ref["k_scale"][0]), b
            vh = np.ascontiguousarray(vn[k0:k1].transpose(1, 0, 2))[None]
            pad = -(-nk // 128) * 128
            if w.pv == "fp8":
                c, s = sage_ref.quant_v_fp8(vh)
                assert np.array_equal(got["v_codes"][:, :, p:p + nk].numpy(), c[0]), ("v codes", b)
                assert not got["v_codes"][:, :, p + nk:p + pad].numpy().any(), ("v padding", b)
                assert np.array_equal(got["v_scale"][b].numpy(), s[0]), ("v scale", b)
            else:
                want = v[k0:k1].transpose(0, 1).transpose(1, 2)            # [Hkv, d, nk], the input bits
                assert torch.equal(got["v_t"][:, :, p:p + nk], want), ("v transposed", b)
                assert not got["v_t"][:, :, p + nk:p + pad].float().abs().sum(), ("v padding", b)
            p += pad
        else:
            assert not got["k_mean"][b].numpy().any(), ("k mean of a sequence without keys", b)


@pytest.mark.parametrize("w,gran", CASES, ids=[f"{w.name}-{g}" for w, g in CASES])
def test_varlen_quant_stages_bit_exact(w, gran):
    say("varlen quant stages", w.name, gran)
    check_varlen_quant(w, gran)


def test_varlen_quant_stages_serving_mix():
    say("varlen quant stages, serving mix")
    check_varlen_quant(W.VARLEN_PREFILL, "per_block")
    check_varlen_quant(W.VARLEN_PREFILL, "per_thread")
