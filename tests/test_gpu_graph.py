"""Capture in a HIP graph (torch.cuda.CUDAGraph on ROCm).

Every library call enqueues kernels only (no allocation, no memset, no host
synchronisation), so a forward captured once replays on new contents of the
same buffers. Each replay is checked bit for bit against an eager call on the
same inputs, with eager work and synchronisations between the replays.
A packed batch keeps its offsets on the device: one captured graph serves
different length mixes with the same totals and bounds.
"""
import pytest
import torch

import workloads as W
from tests.parity_util import say

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

if torch.cuda.is_available():
    import quantized_attention_channel_amd as sage


def _capture(fn):
    """Warm up on a side stream (default priority), then capture one call."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("pv,causal,gran", [("fp8", False, "per_block"), ("fp16", True, "per_thread")])
def test_dense_forward_replays_equal_eager(pv, causal, gran):
    w = W.TINY.with_(B=2, Hq=4, Hkv=2, N=777, d=128, dtype="bf16", causal=causal, pv=pv)
    say("graph dense", pv, causal, gran)
    q, k, v = (t.cuda() for t in W.generate(w))
    o = torch.empty_like(q)
    ws = torch.empty(sage.sage_workspace_bytes(sage.shape_of(q, k, "HND", gran), pv), dtype=torch.uint8,
                     device="cuda")
    kw = dict(is_causal=causal, sm_scale=w.sm_scale, pv_dtype=pv, qk_gran=gran)
    g = _capture(lambda: sage.sage_attn_fwd(q, k, v, out=o, workspace=ws, **kw))
    for rep in range(4):
        q2, k2, v2 = (t.cuda() for t in W.generate(w.with_(seed=100 + rep)))
        q.copy_(q2)
        k.copy_(k2)
        v.copy_(v2)
        o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        want = sage.sage_attn_fwd(q2, k2, v2, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o, want), f"replay {rep}"


def test_packed_forward_replays_new_length_mixes():
    mixes = [(100, 300, 200), (300, 100, 200), (1, 299, 300), (300, 0, 300)]
    w0 = W.VarlenWorkload("graph", mixes[0], mixes[0], Hq=4, Hkv=2, d=128, dtype="fp16", causal=True, pv="fp8")
    say("graph varlen", mixes)
    q, k, v, cq, ck = (t.cuda() for t in W.generate_varlen(w0))
    o = torch.empty_like(q)
    mq = mk = max(max(m) for m in mixes)
    shape = sage.varlen_shape_of(q, k, cq, mq, mk)
    ws = torch.empty(sage.sage_varlen_workspace_bytes(shape, "fp8"), dtype=torch.uint8, device="cuda")
    kw = dict(is_causal=True, sm_scale=w0.sm_scale, pv_dtype="fp8")
    g = _capture(lambda: sage.sage_attn_fwd_varlen(q, k, v, cq, ck, mq, mk, out=o, workspace=ws, **kw))
    for rep, mix in enumerate(mixes):
        w = w0.with_(lens_q=mix, lens_k=mix, seed=7 + rep)
        q2, k2, v2, cq2, ck2 = (t.cuda() for t in W.generate_varlen(w))
        for dst, src in ((q, q2), (k, k2), (v, v2), (cq, cq2), (ck, ck2)):
            dst.copy_(src)
        o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        want = sage.sage_attn_fwd_varlen(q2, k2, v2, cq2, ck2, mq, mk, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o, want), f"replay {rep} {mix}"


def test_fp4_dense_forward_replays_equal_eager():
    w = W.TINY.with_(B=2, Hq=4, Hkv=2, N=777, d=128, dtype="bf16", layout="NHD")
    say("graph fp4 dense")
    q, k, v = (t.cuda() for t in W.generate(w))
    o = torch.empty_like(q)
    ws = torch.empty(sage.sage_fp4_workspace_bytes(sage.shape_of(q, k, "NHD")), dtype=torch.uint8, device="cuda")
    kw = dict(is_causal=True, sm_scale=w.sm_scale, tensor_layout="NHD")
    g = _capture(lambda: sage.sage_attn_fwd_fp4(q, k, v, out=o, workspace=ws, **kw))
    for rep in range(4):
        q2, k2, v2 = (t.cuda() for t in W.generate(w.with_(seed=200 + rep)))
        q.copy_(q2)
        k.copy_(k2)
        v.copy_(v2)
        o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        want = sage.sage_attn_fwd_fp4(q2, k2, v2, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o, want), f"replay {rep}"


def test_fp4_packed_forward_replays_new_length_mixes():
    mixes = [(100, 300, 200), (300, 100, 200), (1, 299, 300), (300, 0, 300)]
    w0 = W.VarlenWorkload("graph4", mixes[0], mixes[0], Hq=4, Hkv=2, d=64, dtype="bf16", causal=True, pv="fp4")
    say("graph fp4 varlen", mixes)
    q, k, v, cq, ck = (t.cuda() for t in W.generate_varlen(w0))
    o = torch.empty_like(q)
    mq = mk = max(max(m) for m in mixes)
    shape = sage.varlen_shape_of(q, k, cq, mq, mk)
    ws = torch.empty(sage.sage_fp4_varlen_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    kw = dict(is_causal=True, sm_scale=w0.sm_scale)
    g = _capture(lambda: sage.sage_attn_fwd_fp4_varlen(q, k, v, cq, ck, mq, mk, out=o, workspace=ws, **kw))
    for rep, mix in enumerate(mixes):
        w = w0.with_(lens_q=mix, lens_k=mix, seed=17 + rep)
        q2, k2, v2, cq2, ck2 = (t.cuda() for t in W.generate_varlen(w))
        for dst, src in ((q, q2), (k, k2), (v, v2), (cq, cq2), (ck, ck2)):
            dst.copy_(src)
        o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        want = sage.sage_attn_fwd_fp4_varlen(q2, k2, v2, cq2, ck2, mq, mk, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o, want), f"replay {rep} {mix}"
