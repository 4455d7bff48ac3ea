"""Framework integration: the custom operator and the guarded SDPA drop-in.

CPU: the operator is registered and its fake implementation propagates shapes
(meta tensors); the guard names a reason for every call the method does not
implement; the patch restores the original function, raises on unsupported
calls by default and hands them to the original function when asked.
GPU: a routed call equals the library's own entry point bit for bit, the
operator passes torch.library's checks, and a captured graph (torch.compile,
aot_eager backend: no generated kernels) equals eager execution.
"""
import pytest
import torch
import torch.nn.functional as F

import quantized_attention_channel_amd as sage
from quantized_attention_channel_amd.integration import attn_fwd_op, attn_fwd_varlen_op, patch_sdpa, sdpa_supported


def _meta(*shape, dtype=torch.float16):
    return torch.empty(shape, dtype=dtype, device="meta")


def test_operator_is_registered_with_a_fake_implementation():
    assert hasattr(torch.ops.sage_mi355x, "attn_fwd")
    q, k = _meta(2, 8, 100, 64), _meta(2, 4, 300, 64)
    out = torch.ops.sage_mi355x.attn_fwd(q, k, k, False, 0.125, "fp8", "HND", "per_block")
    assert out.shape == q.shape and out.dtype == q.dtype and out.device.type == "meta"


def test_varlen_operator_is_registered_with_a_fake_implementation():
    assert hasattr(torch.ops.sage_mi355x, "attn_fwd_varlen")
    q, k = _meta(700, 8, 128, dtype=torch.bfloat16), _meta(900, 2, 128, dtype=torch.bfloat16)
    cu = torch.empty(4, dtype=torch.int32, device="meta")
    out = torch.ops.sage_mi355x.attn_fwd_varlen(q, k, k, cu, cu, 400, 500, True, 0.088, "fp4", "per_block")
    assert out.shape == q.shape and out.dtype == q.dtype and out.device.type == "meta"


@pytest.mark.parametrize("kw,reason", [
    (dict(attn_mask=_meta(1, 1, 100, 100)), "masks"),
    (dict(dropout_p=0.1), "dropout"),
    (dict(q=_meta(8, 100, 64)), "4-D"),
    (dict(q=_meta(2, 8, 100, 64, dtype=torch.float32)), "float16"),
    (dict(q=_meta(2, 8, 100, 96), k=_meta(2, 8, 300, 96)), "head_dim"),
    (dict(v=_meta(2, 8, 299, 64)), "value"),
    (dict(k=_meta(2, 4, 300, 64)), "enable_gqa"),
    (dict(k=_meta(2, 3, 300, 64), enable_gqa=True), "enable_gqa"),
    (dict(is_causal=True), "causal"),
    (dict(scale=float("nan")), "scale"),
    (dict(), "GPU"),
])
def test_sdpa_guard_names_the_reason(kw, reason):
    q = kw.pop("q", _meta(2, 8, 100, 64))
    k = kw.pop("k", _meta(2, 8, 300, 64))
    v = kw.pop("v", k)
    got = sdpa_supported(q, k, v, **kw)
    assert got is not None and reason in got


def test_sdpa_guard_rejects_inputs_that_need_gradients():
    q = torch.empty(1, 2, 16, 64, dtype=torch.float16, requires_grad=True)
    assert "backward" in sdpa_supported(q, q.detach(), q.detach())
    with torch.no_grad():
        assert "GPU" in sdpa_supported(q, q.detach(), q.detach())


def test_patch_restores_and_guards_on_the_cpu():
    orig = F.scaled_dot_product_attention
    q = torch.randn(1, 2, 16, 64)
    mask = torch.zeros(16, 16)
    with patch_sdpa() as p:
        assert F.scaled_dot_product_attention is not orig
        with pytest.raises(NotImplementedError, match="masks"):
            F.scaled_dot_product_attention(q, q, q, attn_mask=mask)
        assert p.routed == 0 and p.passed == 0
    assert F.scaled_dot_product_attention is orig
    with patch_sdpa(passthrough=True) as p:
        got = F.scaled_dot_product_attention(q, q, q, attn_mask=mask)
    assert p.passed == 1 and p.routed == 0
    assert torch.equal(got, orig(q, q, q, attn_mask=mask))
    assert F.scaled_dot_product_attention is orig


def test_patch_rejects_settings_the_kernels_do_not_have():
    with pytest.raises(ValueError, match="pv_dtype"):
        patch_sdpa(pv_dtype="fp6")
    with pytest.raises(ValueError, match="MX blocks"):
        patch_sdpa(pv_dtype="fp4", qk_quant_gran="per_thread")


# ------------------------------------------------------------------ GPU
@pytest.mark.gpu
@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
@pytest.mark.parametrize("causal,gqa,pv,gran", [(False, False, "fp8", "per_block"), (True, True, "fp8", "per_block"),
                                               (True, False, "fp16", "per_thread"), (True, True, "fp4", "per_block")])
def test_patched_sdpa_routes_to_the_kernels(causal, gqa, pv, gran):
    g = torch.Generator().manual_seed(3)
    hkv = 2 if gqa else 4
    q = torch.randn(2, 4, 300, 128, generator=g).half().cuda()
    k = torch.randn(2, hkv, 300, 128, generator=g).half().cuda()
    v = torch.randn(2, hkv, 300, 128, generator=g).half().cuda()
    with torch.no_grad(), patch_sdpa(pv_dtype=pv, qk_quant_gran=gran) as p:
        got = F.scaled_dot_product_attention(q, k, v, is_causal=causal, enable_gqa=gqa)
    if pv == "fp4":
        want = sage.sage_attn_fwd_fp4(q, k, v, is_causal=causal, sm_scale=128 ** -0.5)
    else:
        want = sage.sage_attn_fwd(q, k, v, is_causal=causal, sm_scale=128 ** -0.5, pv_dtype=pv, qk_gran=gran)
    torch.cuda.synchronize()
    assert p.routed == 1 and torch.equal(got, want)
    # and against the oracle (SDPA's default scale 1/sqrt(d)), not only the library itself
    _against_oracle(got, q, k, v, causal=causal, sm_scale=128 ** -0.5, pv=pv, gran=gran)


def _against_oracle(got, q, k, v, *, causal, sm_scale, pv, gran, dtype="fp16"):
    from oracle import exact, sage_ref
    from tests.parity_util import COS_EXACT, COS_ORACLE, RL1_ORACLE, cos, rel_l1, worst_head_cos
    blk = ((sage_ref.PER_THREAD_BLK_Q, sage_ref.PER_THREAD_BLK_K) if gran == "per_thread"
           else (sage_ref.BLK_Q, sage_ref.BLK_K))
    qn, kn, vn = (t.float().cpu().numpy() for t in (q, k, v))
    if pv == "fp4":
        ref = sage_ref.sage_attention_fp4(qn, kn, vn, dtype=dtype, is_causal=causal, sm_scale=sm_scale)
    else:
        ref = sage_ref.sage_attention(qn, kn, vn, dtype=dtype, is_causal=causal, sm_scale=sm_scale, pv=pv,
                                      blk_q=blk[0], blk_k=blk[1])
    g = got.float().cpu().numpy()
    assert cos(g, ref) >= COS_ORACLE and rel_l1(g, ref) <= RL1_ORACLE and worst_head_cos(g, ref) >= COS_ORACLE
    ex = exact.exact_attention(qn, kn, vn, is_causal=causal, sm_scale=sm_scale)
    if pv == "fp4":     # (a coarser method: the kernel lands where the oracle lands)
        assert abs(cos(g, ex) - cos(ref, ex)) <= 1e-3
    else:
        assert cos(g, ex) >= COS_EXACT


@pytest.mark.gpu
@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
def test_operator_passes_torch_library_checks():
    g = torch.Generator().manual_seed(4)
    q, k, v = (torch.randn(1, 2, 200, 64, generator=g).half().cuda() for _ in range(3))
    torch.library.opcheck(attn_fwd_op, (q, k, v, True, 0.125, "fp8", "HND", "per_thread"),
                          test_utils=("test_schema", "test_faketensor"))


@pytest.mark.gpu
@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
def test_captured_graph_equals_eager():
    g = torch.Generator().manual_seed(5)
    q, k, v = (torch.randn(1, 4, 257, 128, generator=g).bfloat16().cuda() for _ in range(3))

    def f(q, k, v):
        o = torch.ops.sage_mi355x.attn_fwd(q * 2, k, v, True, 0.0625, "fp8", "HND", "per_block")
        return o.float().sum(dim=-1)

    eager = f(q, k, v)
    compiled = torch.compile(f, backend="aot_eager", fullgraph=True)(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(eager, compiled)
    # the operator's output inside the compiled graph against the oracle
    def g_(q, k, v):
        o = torch.ops.sage_mi355x.attn_fwd(q * 2, k, v, True, 0.0625, "fp8", "HND", "per_block")
        return o

    out = torch.compile(g_, backend="aot_eager", fullgraph=True)(q, k, v)
    torch.cuda.synchronize()
    _against_oracle(out, q * 2, k, v, causal=True, sm_scale=0.0625, pv="fp8", gran="per_block", dtype="bf16")


@pytest.mark.gpu
@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
def test_compiled_fp4_operator_against_oracle():
    """The FP4 variant through the custom operator inside a torch.compile graph."""
    g = torch.Generator().manual_seed(7)
    q, k, v = (torch.randn(1, 2, 333, 128, generator=g).half().cuda() for _ in range(3))

    def f(q, k, v):
        return torch.ops.sage_mi355x.attn_fwd(q, k, v, True, 0.09, "fp4", "HND", "per_block")

    out = torch.compile(f, backend="aot_eager", fullgraph=True)(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(out, sage.sage_attn_fwd_fp4(q, k, v, is_causal=True, sm_scale=0.09))
    _against_oracle(out, q, k, v, causal=True, sm_scale=0.09, pv="fp4", gran="per_block")


@pytest.mark.gpu
@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
@pytest.mark.parametrize("backend", ["inductor", "aot_eager"])
def test_compiled_model_against_oracle(backend):
    """A small attention block compiled with torch.compile: the projections run
    in torch, the attention in the custom operator (one opaque graph node); the
    result is checked against the same block with the oracle's attention."""
    g = torch.Generator().manual_seed(6)
    B, H, N, d = 1, 4, 300, 64
    x = torch.randn(B, N, H * d, generator=g).half().cuda()
    wq, wk, wv = (torch.randn(H * d, H * d, generator=g).mul(0.05).half().cuda() for _ in range(3))

    def block(x):
        q, k, v = (torch.matmul(x, w).view(B, N, H, d).transpose(1, 2).contiguous() for w in (wq, wk, wv))
        return torch.ops.sage_mi355x.attn_fwd(q, k, v, False, d ** -0.5, "fp16", "HND", "per_block"), q, k, v

    try:
        fn = torch.compile(block, backend=backend, fullgraph=True)
        o, q, k, v = fn(x)
    except Exception as e:  # noqa: BLE001 -- a backend that cannot build here is reported, not hidden
        if backend == "inductor":
            pytest.skip(f"inductor backend unavailable on this machine: {type(e).__name__}: {e}")
        raise
    torch.cuda.synchronize()
    _against_oracle(o, q, k, v, causal=False, sm_scale=d ** -0.5, pv="fp16", gran="per_block")


@pytest.mark.gpu
@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
@pytest.mark.parametrize("pv", ["fp8", "fp4"])
def test_compiled_varlen_operator_against_oracle(pv):
    """The packed-batch operator inside a torch.compile graph (aot_eager), with
    torch work on both sides of it: passes torch.library's checks, equals
    sageattn_varlen bit for bit, and meets the parity bars against the oracle
    run per sequence."""
    import numpy as np
    import workloads as W
    from oracle import sage_ref
    from tests.parity_util import COS_ORACLE, RL1_ORACLE, cos, rel_l1
    w = W.VarlenWorkload("compiled", (300, 1, 129, 0, 77), (300, 1, 129, 0, 77), Hq=4, Hkv=2, d=128,
                         dtype="bf16", causal=True, pv=pv)
    q, k, v, cq, ck = (t.cuda() for t in W.generate_varlen(w))
    mq = mk = max(w.lens_q)
    torch.library.opcheck(attn_fwd_varlen_op, (q, k, v, cq, ck, mq, mk, True, w.sm_scale, pv, "per_block"),
                          test_utils=("test_schema", "test_faketensor"))

    def f(q, k, v):
        o = torch.ops.sage_mi355x.attn_fwd_varlen(q * 1.5, k, v, cq, ck, mq, mk, True, w.sm_scale, pv, "per_block")
        return o, o.float().sum(dim=-1)

    o, rowsum = torch.compile(f, backend="aot_eager", fullgraph=True)(q, k, v)
    want = sage.sageattn_varlen(q * 1.5, k, v, cq, ck, mq, mk, is_causal=True, sm_scale=w.sm_scale, pv_dtype=pv)
    torch.cuda.synchronize()
    assert torch.equal(o, want) and torch.equal(rowsum, want.float().sum(dim=-1))
    qn, kn, vn = ((q * 1.5).float().cpu().numpy(), k.float().cpu().numpy(), v.float().cpu().numpy())
    got = o.float().cpu().numpy().astype(np.float64)
    cqs, cks = cq.tolist(), ck.tolist()
    if pv == "fp4":
        ref = np.zeros(qn.shape, np.float64)
        for b in range(w.B):
            q0, q1, k0, k1 = cqs[b], cqs[b + 1], cks[b], cks[b + 1]
            if q1 > q0 and k1 > k0:
                seq = [np.ascontiguousarray(x[a:e].transpose(1, 0, 2))[None]
                       for x, a, e in ((qn, q0, q1), (kn, k0, k1), (vn, k0, k1))]
                r = sage_ref.sage_attention_fp4(*seq, dtype=w.dtype, is_causal=True, sm_scale=w.sm_scale)
                ref[q0:q1] = r[0].transpose(1, 0, 2)
    else:
        ref = sage_ref.sage_attention_varlen(qn, kn, vn, cqs, cks, dtype=w.dtype, is_causal=True,
                                             sm_scale=w.sm_scale, pv=pv)
    assert cos(got, ref) >= COS_ORACLE and rel_l1(got, ref) <= RL1_ORACLE
