"""GPU parity over seeded random configurations (valid inputs only).

The hand-picked cases elsewhere cover each switch on its own; these draw
combinations: batch, heads and GQA ratio, query and key counts (1 to ~1.5k,
independent for non-causal), head dim, input dtype, layout, causal masking, PV
precision and scale granularity -- and, for packed batches, random length mixes
with empty and single-token sequences. Every row is compared with the oracle at
the method's bar (cosine >= 0.9999, sum|o-r|/sum|r| <= 1e-3) and with fp64
exact attention (cosine >= 0.999).
"""
import random

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


def _dense_config(i):
    r = random.Random(1000 + i)
    hkv = r.choice([1, 2, 3])
    causal = r.random() < 0.5
    nk = r.choice([1, 2, r.randint(3, 300), r.randint(300, 1500)])
    nq = nk if causal else r.choice([1, r.randint(2, 400), r.randint(400, 1500)])
    return dict(B=r.choice([1, 2]), Hkv=hkv, Hq=hkv * r.choice([1, 2, 4]), nq=nq, nk=nk, d=r.choice([64, 128]),
                dtype=r.choice(["fp16", "bf16"]), layout=r.choice(["HND", "NHD"]), causal=causal,
                pv=r.choice(["fp8", "fp16"]), gran=r.choice(["per_block", "per_thread"]),
                k_off_var=r.choice([0.0, 4.0, 40.0]))


DENSE = [_dense_config(i) for i in range(48)]


def _cut(t, n, layout):
    return (t[:, :, :n] if layout == "HND" else t[:, :n]).contiguous()


@pytest.mark.parametrize("i", range(len(DENSE)))
def test_random_dense_config(i):
    c = DENSE[i]
    say("random dense", i, c)
    n = max(c["nq"], c["nk"])
    w = W.TINY.with_(B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], N=n, d=c["d"], dtype=c["dtype"], layout=c["layout"],
                     causal=c["causal"], k_off_var=c["k_off_var"], seed=i)
    q, k, v = W.generate(w)
    q, k, v = _cut(q, c["nq"], c["layout"]), _cut(k, c["nk"], c["layout"]), _cut(v, c["nk"], c["layout"])
    o = sage.sage_attn_fwd(q.cuda(), k.cuda(), v.cuda(), is_causal=c["causal"], sm_scale=w.sm_scale, pv_dtype=c["pv"],
                           tensor_layout=c["layout"], qk_gran=c["gran"])
    torch.cuda.synchronize()
    got = sage_ref.as_hnd(o.float().cpu().numpy(), c["layout"])
    qn, kn, vn = (sage_ref.as_hnd(t.float().numpy(), c["layout"]) for t in (q, k, v))
    bq, bk = GRAN_BLK[c["gran"]]
    ref = sage_ref.sage_attention(qn, kn, vn, dtype=c["dtype"], is_causal=c["causal"], sm_scale=w.sm_scale,
                                  pv=c["pv"], blk_q=bq, blk_k=bk)
    ex = exact.exact_attention(qn, kn, vn, is_causal=c["causal"], sm_scale=w.sm_scale)
    cc, r, ce = cos(got, ref), rel_l1(got, ref), cos(got, ex)
    say(f"   cos={cc:.7f} rel_l1={r:.2e} cos_exact={ce:.6f}")
    assert np.isfinite(got).all()
    assert cc >= COS_ORACLE and r <= RL1_ORACLE and ce >= COS_EXACT


def _varlen_config(i):
    r = random.Random(5000 + i)
    B = r.randint(1, 9)
    causal = r.random() < 0.5
    lens_k = tuple(r.choice([0, 1, r.randint(2, 130), r.randint(130, 900)]) for _ in range(B))
    lens_q = lens_k if causal else tuple(r.choice([0, 1, r.randint(2, 400)]) for _ in range(B))
    if not any(a and b for a, b in zip(lens_q, lens_k)):      # at least one sequence with rows and keys
        lens_k = (max(lens_k[0], 7),) + lens_k[1:]
        lens_q = lens_k if causal else (max(lens_q[0], 5),) + lens_q[1:]
    hkv = r.choice([1, 2])
    return W.VarlenWorkload(f"rand{i}", lens_q, lens_k, Hq=hkv * r.choice([1, 2, 4]), Hkv=hkv, d=r.choice([64, 128]),
                            dtype=r.choice(["fp16", "bf16"]), causal=causal, pv=r.choice(["fp8", "fp16"]),
                            k_off_var=r.choice([1.0, 9.0]), seed=i), r.choice(["per_block", "per_thread"])


VARLEN = [_varlen_config(i) for i in range(24)]


@pytest.mark.parametrize("i", range(len(VARLEN)))
def test_random_varlen_config(i):
    w, gran = VARLEN[i]
    say("random varlen", i, w.lens_q, w.lens_k, w.Hq, w.Hkv, w.d, w.dtype, w.causal, w.pv, gran)
    q, k, v, cq, ck = W.generate_varlen(w)
    o = sage.sage_attn_fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cq.cuda(), ck.cuda(), max(w.lens_q), max(w.lens_k),
                                  is_causal=w.causal, sm_scale=w.sm_scale, pv_dtype=w.pv, qk_gran=gran)
    torch.cuda.synchronize()
    got = o.float().cpu().numpy().astype(np.float64)
    qn, kn, vn = (t.float().numpy() for t in (q, k, v))
    bq, bk = GRAN_BLK[gran]
    ref = sage_ref.sage_attention_varlen(qn, kn, vn, cq.tolist(), ck.tolist(), dtype=w.dtype, is_causal=w.causal,
                                         sm_scale=w.sm_scale, pv=w.pv, blk_q=bq, blk_k=bk)
    ex = exact.exact_attention_varlen(qn, kn, vn, cq.tolist(), ck.tolist(), is_causal=w.causal, sm_scale=w.sm_scale)
    assert np.isfinite(got).all()
    for b in range(w.B):
        if w.lens_k[b] == 0:
            assert not got[cq[b]:cq[b + 1]].any()
    cc, r, ce = cos(got, ref), rel_l1(got, ref), cos(got, ex)
    say(f"   cos={cc:.7f} rel_l1={r:.2e} cos_exact={ce:.6f}")
    assert cc >= COS_ORACLE and r <= RL1_ORACLE and ce >= COS_EXACT


@pytest.mark.parametrize("i", range(len(VARLEN)))
def test_random_varlen_quant_stages(i):
    """The same 24 packed mixes: every sequence's integer stages bit for bit."""
    from tests.test_gpu_varlen import check_varlen_quant
    w, gran = VARLEN[i]
    say("random varlen quant stages", i, w.lens_q, w.lens_k, w.Hq, w.Hkv, w.d, w.dtype, w.pv, gran)
    check_varlen_quant(w, gran)


# ------------------------------------------------------------------ the FP4 microscaling variant
def _fp4_dense_config(i):
    r = random.Random(7000 + i)
    hkv = r.choice([1, 2, 3])
    causal = r.random() < 0.5
    nk = r.choice([1, r.randint(2, 300), r.randint(300, 1500)])
    nq = nk if causal else r.choice([1, r.randint(2, 400), r.randint(400, 1500)])
    return dict(B=r.choice([1, 2]), Hkv=hkv, Hq=hkv * r.choice([1, 2, 4]), nq=nq, nk=nk, d=r.choice([64, 128]),
                dtype=r.choice(["fp16", "bf16"]), layout=r.choice(["HND", "NHD"]), causal=causal,
                k_off_var=r.choice([0.0, 4.0, 40.0]))


FP4_DENSE = [_fp4_dense_config(i) for i in range(24)]


@pytest.mark.parametrize("i", range(len(FP4_DENSE)))
def test_random_fp4_dense_config(i):
    """The FP4 variant on a random dense configuration: every row against the
    oracle's FP4 attention at the bars, and as close to fp64 attention as the
    oracle (MXFP4 is the coarser method)."""
    c = FP4_DENSE[i]
    say("random fp4 dense", i, c)
    n = max(c["nq"], c["nk"])
    w = W.TINY.with_(B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], N=n, d=c["d"], dtype=c["dtype"], layout=c["layout"],
                     k_off_var=c["k_off_var"], seed=7000 + i)
    q, k, v = W.generate(w)
    q, k, v = _cut(q, c["nq"], c["layout"]), _cut(k, c["nk"], c["layout"]), _cut(v, c["nk"], c["layout"])
    o = sage.sage_attn_fwd_fp4(q.cuda(), k.cuda(), v.cuda(), is_causal=c["causal"], sm_scale=w.sm_scale,
                               tensor_layout=c["layout"])
    torch.cuda.synchronize()
    got = sage_ref.as_hnd(o.float().cpu().numpy(), c["layout"])
    qn, kn, vn = (sage_ref.as_hnd(t.float().numpy(), c["layout"]) for t in (q, k, v))
    ref = sage_ref.sage_attention_fp4(qn, kn, vn, dtype=c["dtype"], is_causal=c["causal"], sm_scale=w.sm_scale)
    ex = exact.exact_attention(qn, kn, vn, is_causal=c["causal"], sm_scale=w.sm_scale)
    cc, r, ce, ce_oracle = cos(got, ref), rel_l1(got, ref), cos(got, ex), cos(ref, ex)
    say(f"   cos={cc:.7f} rel_l1={r:.2e}; vs fp64: HIP {ce:.5f} oracle {ce_oracle:.5f}")
    assert np.isfinite(got).all()
    assert cc >= COS_ORACLE and r <= RL1_ORACLE and abs(ce - ce_oracle) <= 1e-3


FP4_VARLEN = [_varlen_config(100 + i)[0] for i in range(24)]


@pytest.mark.parametrize("i", range(len(FP4_VARLEN)))
def test_random_fp4_varlen_config(i):
    """The FP4 variant on a random packed mix: every sequence's MXFP4 stages bit
    for bit, every row against the oracle's FP4 attention run per sequence."""
    from tests.test_gpu_fp4_varlen import check_fp4_varlen_quant, oracle_fp4_varlen
    w = FP4_VARLEN[i].with_(pv="fp4")
    say("random fp4 varlen", i, w.lens_q, w.lens_k, w.Hq, w.Hkv, w.d, w.dtype, w.causal)
    check_fp4_varlen_quant(w)
    q, k, v, cq, ck = W.generate_varlen(w)
    o = sage.sage_attn_fwd_fp4_varlen(q.cuda(), k.cuda(), v.cuda(), cq.cuda(), ck.cuda(), max(w.lens_q),
                                      max(w.lens_k), is_causal=w.causal, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    got = o.float().cpu().numpy().astype(np.float64)
    qn, kn, vn = (t.float().numpy() for t in (q, k, v))
    ref = oracle_fp4_varlen(qn, kn, vn, cq.tolist(), ck.tolist(), dtype=w.dtype, is_causal=w.causal,
                            sm_scale=w.sm_scale)
    assert np.isfinite(got).all()
    for b in range(w.B):
        if w.lens_k[b] == 0:
            assert not got[cq[b]:cq[b + 1]].any()
    cc, r = cos(got, ref), rel_l1(got, ref)
    say(f"   cos={cc:.7f} rel_l1={r:.2e}")
    assert cc >= COS_ORACLE and r <= RL1_ORACLE


# ------------------------------------------------------------------ longer random shapes, every path
def _long_config(i):
    r = random.Random(9000 + i)
    hkv = r.choice([1, 2])
    causal = r.random() < 0.5
    nk = r.randint(1500, 6000)
    nq = nk if causal else r.choice([r.randint(1, 300), r.randint(1500, 6000)])
    pv = r.choice(["fp8", "fp16", "fp4"])
    return dict(B=1, Hkv=hkv, Hq=hkv * r.choice([1, 2]), nq=nq, nk=nk, d=r.choice([64, 128]),
                dtype=r.choice(["fp16", "bf16"]), layout=r.choice(["HND", "NHD"]), causal=causal, pv=pv,
                gran="per_block" if pv == "fp4" else r.choice(["per_block", "per_thread"]),
                k_off_var=r.choice([0.0, 4.0, 40.0]))


LONG = [_long_config(i) for i in range(12)]


@pytest.mark.parametrize("i", range(len(LONG)))
def test_random_long_config(i):
    """Longer random shapes (1.5k to 6k keys, ragged tails) on every path
    (FP8 or FP16 PV at either granularity, or the FP4 variant): every row
    against the oracle."""
    c = LONG[i]
    say("random long", i, c)
    n = max(c["nq"], c["nk"])
    w = W.TINY.with_(B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], N=n, d=c["d"], dtype=c["dtype"], layout=c["layout"],
                     k_off_var=c["k_off_var"], seed=9000 + i)
    q, k, v = W.generate(w)
    q, k, v = _cut(q, c["nq"], c["layout"]), _cut(k, c["nk"], c["layout"]), _cut(v, c["nk"], c["layout"])
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    if c["pv"] == "fp4":
        o = sage.sage_attn_fwd_fp4(qg, kg, vg, is_causal=c["causal"], sm_scale=w.sm_scale, tensor_layout=c["layout"])
    else:
        o = sage.sage_attn_fwd(qg, kg, vg, is_causal=c["causal"], sm_scale=w.sm_scale, pv_dtype=c["pv"],
                               tensor_layout=c["layout"], qk_gran=c["gran"])
    torch.cuda.synchronize()
    got = sage_ref.as_hnd(o.float().cpu().numpy(), c["layout"])
    qn, kn, vn = (sage_ref.as_hnd(t.float().numpy(), c["layout"]) for t in (q, k, v))
    ex = exact.exact_attention(qn, kn, vn, is_causal=c["causal"], sm_scale=w.sm_scale)
    if c["pv"] == "fp4":
        ref = sage_ref.sage_attention_fp4(qn, kn, vn, dtype=c["dtype"], is_causal=c["causal"], sm_scale=w.sm_scale)
    else:
        bq, bk = GRAN_BLK[c["gran"]]
        ref = sage_ref.sage_attention(qn, kn, vn, dtype=c["dtype"], is_causal=c["causal"], sm_scale=w.sm_scale,
                                      pv=c["pv"], blk_q=bq, blk_k=bk)
    cc, r, ce, ce_oracle = cos(got, ref), rel_l1(got, ref), cos(got, ex), cos(ref, ex)
    say(f"   cos={cc:.7f} rel_l1={r:.2e}; vs fp64: HIP {ce:.6f} oracle {ce_oracle:.6f}")
    assert np.isfinite(got).all()
    assert cc >= COS_ORACLE and r <= RL1_ORACLE
    if c["pv"] == "fp4":
        assert abs(ce - ce_oracle) <= 1e-3
    else:
        assert ce >= COS_EXACT


# ------------------------------------------------------------------ quantisation stages on random shapes
def _quant_config(i):
    r = random.Random(11000 + i)
    hkv = r.choice([1, 2, 3])
    return dict(B=r.choice([1, 2, 3]), Hkv=hkv, Hq=hkv * r.choice([1, 2, 4]), nq=r.randint(1, 2000),
                nk=r.randint(1, 2000), d=r.choice([64, 128]), dtype=r.choice(["fp16", "bf16"]),
                layout=r.choice(["HND", "NHD"]), gran=r.choice(["per_block", "per_thread"]),
                k_off_var=r.choice([0.0, 4.0, 40.0]))


QUANT = [_quant_config(i) for i in range(24)]


@pytest.mark.parametrize("i", range(len(QUANT)))
def test_random_quant_stages(i):
    """Every quantisation stage on a random shape (independent query and key
    counts), bit for bit against the oracle: the K mean, Q/K INT8 codes and
    scales at the drawn granularity, V e4m3 codes (with the zero padding) and
    scales, and every MXFP4 stage."""
    from tests.test_gpu_fp4 import check_fp4_stages
    c = QUANT[i]
    say("random quant stages", i, c)
    n = max(c["nq"], c["nk"])
    w = W.TINY.with_(B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], N=n, d=c["d"], dtype=c["dtype"], layout=c["layout"],
                     k_off_var=c["k_off_var"], seed=11000 + i)
    q, k, v = W.generate(w)
    q, k, v = _cut(q, c["nq"], c["layout"]), _cut(k, c["nk"], c["layout"]), _cut(v, c["nk"], c["layout"])
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    qk = sage.sage_quant_qk(qg, kg, tensor_layout=c["layout"], qk_gran=c["gran"])
    vc, vs = sage.sage_quant_v(vg, tensor_layout=c["layout"])
    f4 = sage.sage_quant_fp4(qg, kg, vg, tensor_layout=c["layout"], sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    qn, kn, vn = (sage_ref.as_hnd(t.float().numpy(), c["layout"]) for t in (q, k, v))
    bq, bk = GRAN_BLK[c["gran"]]
    ref = sage_ref.quant_qk(qn, kn, blk_q=bq, blk_k=bk)
    assert np.array_equal(qk["k_mean"].cpu().numpy(), ref["k_mean"])
    assert np.array_equal(qk["q_scale"].cpu().numpy(), ref["q_scale"])
    assert np.array_equal(qk["k_scale"].cpu().numpy(), ref["k_scale"])
    assert np.array_equal(qk["q_codes"].cpu().numpy(), ref["q8"])
    assert np.array_equal(qk["k_codes"].cpu().numpy(), ref["k8"])
    rc, rs = sage_ref.quant_v_fp8(vn)
    vc = vc.cpu().numpy()
    assert np.array_equal(vs.cpu().numpy(), rs)
    assert np.array_equal(vc[..., :c["nk"]], rc) and not vc[..., c["nk"]:].any()
    check_fp4_stages({n_: t for n_, t in f4.items()}, qn, kn, vn, w.sm_scale)
