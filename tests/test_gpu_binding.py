"""GPU checks of the binding's buffer handling.

The attention kernel from precomputed codes (sage_attn_fwd_codes) must equal
the whole path bit for bit, in both PV precisions; caller-supplied outputs and
workspaces are used as given; buffers of the wrong size, dtype or device are
rejected before anything is launched.
"""
import pytest
import torch

import workloads as W
from tests.parity_util import say

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

if torch.cuda.is_available():
    import quantized_attention_channel_amd as sage


def _inputs(causal=False, dtype="fp16", layout="HND"):
    w = W.TINY.with_(B=2, Hq=4, Hkv=2, N=333, d=128, dtype=dtype, layout=layout, causal=causal)
    q, k, v = (t.cuda() for t in W.generate(w))
    return w, q, k, v


@pytest.mark.parametrize("pv,causal,layout", [("fp8", False, "HND"), ("fp16", True, "NHD")])
def test_codes_entry_point_equals_the_whole_path(pv, causal, layout):
    w, q, k, v = _inputs(causal, "bf16" if pv == "fp16" else "fp16", layout)
    say("codes path", pv, causal, layout)
    s = sage.shape_of(q, k, layout)
    qk = sage.sage_quant_qk(q, k, tensor_layout=layout)
    if pv == "fp8":
        vp, vs = sage.sage_quant_v(v, tensor_layout=layout)
    else:
        vp, vs = sage.sage_transpose_v(v, tensor_layout=layout), None
    o = torch.empty_like(q)
    sage.sage_attn_fwd_codes(s, qk["q_codes"], qk["q_scale"], qk["k_codes"], qk["k_scale"], vp, vs, o,
                             is_causal=causal, sm_scale=w.sm_scale, pv_dtype=pv)
    want = sage.sage_attn_fwd(q, k, v, is_causal=causal, sm_scale=w.sm_scale, pv_dtype=pv, tensor_layout=layout)
    torch.cuda.synchronize()
    assert torch.equal(o, want)


def test_codes_entry_point_rejects_mismatched_buffers():
    w, q, k, v = _inputs()
    s = sage.shape_of(q, k, "HND")
    qk = sage.sage_quant_qk(q, k)
    vp, vs = sage.sage_quant_v(v)
    o = torch.empty_like(q)
    args = [qk["q_codes"], qk["q_scale"], qk["k_codes"], qk["k_scale"], vp, vs, o]
    bad = [
        (0, qk["q_codes"][:, :, :-1].contiguous(), ValueError),      # one query row short
        (1, qk["q_scale"].double(), TypeError),
        (2, qk["k_codes"].float(), TypeError),
        (3, qk["k_scale"][..., :-1].contiguous(), ValueError),
        (4, vp[..., :128].contiguous(), ValueError),                 # V codes without their padding
        (5, vs.cpu(), ValueError),
        (6, torch.empty(2, 4, 333, 64, dtype=torch.float16, device="cuda"), ValueError),
    ]
    for i, t, exc in bad:
        a = list(args)
        a[i] = t
        with pytest.raises(exc):
            sage.sage_attn_fwd_codes(s, *a, sm_scale=w.sm_scale)
    torch.cuda.synchronize()


def test_given_output_and_workspace_are_used_and_checked():
    w, q, k, v = _inputs()
    o = torch.full_like(q, float("nan"))
    ws = torch.empty(sage.sage_workspace_bytes(sage.shape_of(q, k, "HND")), dtype=torch.uint8, device="cuda")
    got = sage.sage_attn_fwd(q, k, v, sm_scale=w.sm_scale, out=o, workspace=ws)
    want = sage.sage_attn_fwd(q, k, v, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    assert got is o and torch.equal(o, want)
    with pytest.raises(ValueError, match="shape"):
        sage.sage_attn_fwd(q, k, v, out=torch.empty_like(q)[:, :, :-1])
    with pytest.raises(TypeError, match="uint8"):
        sage.sage_attn_fwd(q, k, v, workspace=torch.empty(ws.numel(), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError, match="batch or head_dim"):
        sage.sage_attn_fwd(q, k[:1].contiguous(), v[:1].contiguous())


def test_many_batch_heads_with_short_sequences():
    """131072 (batch, head) pairs of 5 tokens: every quantisation launch puts
    the pairs in its second grid dimension, past 65535. Heads are independent,
    so the first and last batches are checked against the oracle on their own."""
    import numpy as np
    from oracle import exact, sage_ref
    from tests.parity_util import COS_EXACT, COS_ORACLE, RL1_ORACLE, cos, rel_l1

    w = W.TINY.with_(B=512, Hq=256, Hkv=256, N=5, d=64, dtype="fp16", pv="fp8", seed=11)
    say("many heads", w.B * w.Hq)
    q, k, v = W.generate(w)
    o = sage.sage_attn_fwd(q.cuda(), k.cuda(), v.cuda(), sm_scale=w.sm_scale, pv_dtype="fp8")
    torch.cuda.synchronize()
    got = o.float().cpu().numpy()
    for sl in (slice(0, 2), slice(w.B - 2, w.B)):
        qn, kn, vn = (t[sl].float().numpy() for t in (q, k, v))
        ref = sage_ref.sage_attention(qn, kn, vn, dtype="fp16", is_causal=False, sm_scale=w.sm_scale, pv="fp8")
        ex = exact.exact_attention(qn, kn, vn, is_causal=False, sm_scale=w.sm_scale)
        g = got[sl].astype(np.float64)
        assert cos(g, ref) >= COS_ORACLE and rel_l1(g, ref) <= RL1_ORACLE and cos(g, ex) >= COS_EXACT
