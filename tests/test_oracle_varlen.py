"""Pins for the oracle's packed variable-length batches (CPU only) [R21].

Every sequence of a packed batch is one independent attention by the method.
The pins check that from outside the definition:
* one sequence packed alone equals the dense oracle on the same tokens;
* independence: changing the other sequences (a large K offset, a V scale, a
  different length) leaves a sequence's output bit-identical -- a K mean, a V
  channel scale or a quantisation block shared across sequences would not;
* closed forms per sequence: Q = 0 gives the mean of that sequence's values,
  the first causal row is that sequence's first value row, a sequence without
  keys gets zero rows;
* reordering the sequences reorders the output rows;
* accuracy against fp64 exact attention per sequence.
"""
import numpy as np
import pytest

import workloads as W
from oracle import exact, sage_ref
from oracle.fp8_e4m3 import e4m3_decode

SMALL = W.VarlenWorkload("t", lens_q=(0, 1, 17, 129, 300), lens_k=(0, 1, 17, 129, 300), Hq=4, Hkv=2, d=64,
                         dtype="fp16", causal=False, pv="fp8")


def _np(w):
    q, k, v, cq, ck = W.generate_varlen(w)
    return q.float().numpy(), k.float().numpy(), v.float().numpy(), cq.tolist(), ck.tolist()


def _run(q, k, v, cq, ck, w, pv=None, causal=None, fp64=True):
    return sage_ref.sage_attention_varlen(q, k, v, cq, ck, dtype=w.dtype, pv=pv or w.pv,
                                          is_causal=w.causal if causal is None else causal, sm_scale=w.sm_scale,
                                          return_fp64=fp64)


@pytest.mark.parametrize("pv", ["fp8", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_one_sequence_equals_the_dense_oracle(pv, causal):
    w = SMALL.with_(lens_q=(300,), lens_k=(300,))
    q, k, v, cq, ck = _np(w)
    o = _run(q, k, v, cq, ck, w, pv=pv, causal=causal)
    dense = sage_ref.sage_attention(q[None], k[None], v[None], dtype="fp16", is_causal=causal, sm_scale=w.sm_scale,
                                    pv=pv, layout="NHD", return_fp64=True)
    assert np.array_equal(o, dense[0].transpose(1, 0, 2))


@pytest.mark.parametrize("pv", ["fp8", "fp16"])
def test_sequences_are_independent(pv):
    q, k, v, cq, ck = _np(SMALL)
    base = _run(q, k, v, cq, ck, SMALL, pv=pv)
    # disturb every sequence but the last (tokens cq[-2]: / ck[-2]:)
    k2, v2, q2 = k.copy(), v.copy(), q.copy()
    k2[:ck[-2]] += 37.0
    v2[:ck[-2]] *= 50.0
    q2[:cq[-2]] = -q2[:cq[-2]]
    o = _run(q2, k2, v2, cq, ck, SMALL, pv=pv)
    assert np.array_equal(o[cq[-2]:], base[cq[-2]:])
    # a different neighbour length shifts the last sequence in the packing only
    wq = SMALL.with_(lens_q=(5, 300), lens_k=(9, 300))
    qa, ka, va, cqa, cka = _np(wq)
    qa[5:], ka[9:], va[9:] = q[cq[-2]:], k[ck[-2]:], v[ck[-2]:]
    oa = _run(qa, ka, va, cqa, cka, wq, pv=pv)
    assert np.array_equal(oa[5:], base[cq[-2]:])


@pytest.mark.parametrize("causal", [False, True])
def test_zero_q_gives_each_sequence_its_mean_value(causal):
    q, k, v, cq, ck = _np(SMALL)
    q[:] = 0
    o = _run(q, k, v, cq, ck, SMALL, pv="fp16", causal=causal)
    for b in range(SMALL.B):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        if q1 == q0:
            continue
        vb = np.repeat(v[k0:k1].astype(np.float64), 2, axis=1)          # GQA: 2 query heads per kv head
        if causal:
            want = np.cumsum(vb, axis=0) / np.arange(1, k1 - k0 + 1)[:, None, None]
        else:
            want = np.broadcast_to(vb.mean(axis=0, keepdims=True), vb.shape)
        assert np.allclose(o[q0:q1], want[: q1 - q0], rtol=1e-12, atol=1e-12 * np.abs(vb).max())


def test_zero_q_with_fp8_values_uses_each_sequence_own_scales():
    q, k, v, cq, ck = _np(SMALL)
    q[:] = 0
    v[:ck[-2]] *= 100.0                                            # other sequences: far larger values
    o = _run(q, k, v, cq, ck, SMALL, pv="fp8")
    k0, k1 = ck[-2], ck[-1]
    codes, scale = sage_ref.quant_v_fp8(v[None, k0:k1].transpose(0, 2, 1, 3))
    vd = np.swapaxes(e4m3_decode(codes), 2, 3)[0] * scale[0][:, None, :].astype(np.float64)   # [Hkv, N, d]
    want = np.repeat(vd.mean(axis=1), 2, axis=0)                   # [Hq, d]
    got = o[cq[-2]:]
    assert np.allclose(got, np.broadcast_to(want, got.shape), rtol=1e-12, atol=1e-14)


def test_causal_first_row_of_each_sequence_is_its_first_value():
    q, k, v, cq, ck = _np(SMALL)
    o = _run(q, k, v, cq, ck, SMALL, pv="fp16", causal=True)
    for b in range(SMALL.B):
        if cq[b + 1] > cq[b]:
            assert np.array_equal(o[cq[b]], np.repeat(v[ck[b]].astype(np.float64), 2, axis=0))


def test_sequence_without_keys_gets_zero_rows():
    w = SMALL.with_(lens_q=(3, 40, 7), lens_k=(50, 0, 20))
    q, k, v, cq, ck = _np(w)
    o = _run(q, k, v, cq, ck, w)
    assert not o[3:43].any() and np.abs(o[:3]).sum() > 0 and np.abs(o[43:]).sum() > 0


def test_reordering_sequences_reorders_rows():
    q, k, v, cq, ck = _np(SMALL)
    base = _run(q, k, v, cq, ck, SMALL)
    order = [4, 2, 0, 3, 1]
    qs = np.concatenate([q[cq[b]:cq[b + 1]] for b in order])
    ks = np.concatenate([k[ck[b]:ck[b + 1]] for b in order])
    vs = np.concatenate([v[ck[b]:ck[b + 1]] for b in order])
    w2 = SMALL.with_(lens_q=tuple(SMALL.lens_q[b] for b in order), lens_k=tuple(SMALL.lens_k[b] for b in order))
    cq2, ck2 = w2.cu_seqlens()
    o = _run(qs, ks, vs, cq2, ck2, w2)
    assert np.array_equal(o, np.concatenate([base[cq[b]:cq[b + 1]] for b in order]))


@pytest.mark.parametrize("pv", ["fp8", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_accuracy_vs_fp64(pv, causal):
    w = SMALL.with_(lens_q=(1, 200, 513, 64), lens_k=(1, 200, 513, 64), d=128)
    q, k, v, cq, ck = _np(w)
    o = _run(q, k, v, cq, ck, w, pv=pv, causal=causal, fp64=False)
    e = exact.exact_attention_varlen(q, k, v, cq, ck, is_causal=causal, sm_scale=w.sm_scale)
    c = float((o * e).sum() / np.sqrt((o * o).sum() * (e * e).sum()))
    assert c >= 0.999


def test_workload_offsets_and_ops():
    w = W.VarlenWorkload("t", lens_q=(3, 5), lens_k=(4, 2), Hq=2, Hkv=1, d=8, dtype="fp16", causal=True, pv="fp8")
    assert w.cu_seqlens() == ([0, 3, 8], [0, 4, 6])
    # causal top-left pairs: seq 0 rows see 1, 2, 3 keys; seq 1 rows see 1, 2, 2, 2, 2
    assert w.attention_ops() == 4.0 * 2 * 8 * (6 + 9)
    assert w.with_(causal=False).attention_ops() == 4.0 * 2 * 8 * (12 + 10)
