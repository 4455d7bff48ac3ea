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
from quantized_attention_channel_amd.integration import attn_fwd_op, patch_sdpa, sdpa_supported


def _meta(*shape, dtype=torch.float16):
    return torch.empty(shape, dtype=dtype, device="meta")


def test_operator_is_registered_with_a_fake_implementation():
    assert hasattr(torch.ops.sage_mi355x, "attn_fwd")
    q, k = _meta(2, 8, 100, 64), _meta(2, 4, 300, 64)
    out = torch.ops.sage_mi355x.attn_fwd(q, k, k, False, 0.125, "fp8", "HND", "per_block")
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


# ------------------------------------------------------------------ GPU
@pytest.mark.gpu
@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
@pytest.mark.parametrize("causal,gqa,pv,gran", [(False, False, "fp8", "per_block"), (True, True, "fp8", "per_block"),
                                               (True, False, "fp16", "per_thread")])
def test_patched_sdpa_routes_to_the_kernels(causal, gqa, pv, gran):
    g = torch.Generator().manual_seed(3)
    hkv = 2 if gqa else 4
    q = torch.randn(2, 4, 300, 128, generator=g).half().cuda()
    k = torch.randn(2, hkv, 300, 128, generator=g).half().cuda()
    v = torch.randn(2, hkv, 300, 128, generator=g).half().cuda()
    with torch.no_grad(), patch_sdpa(pv_dtype=pv, qk_quant_gran=gran) as p:
        got = F.scaled_dot_product_attention(q, k, v, is_causal=causal, enable_gqa=gqa)
    want = sage.sage_attn_fwd(q, k, v, is_causal=causal, sm_scale=128 ** -0.5, pv_dtype=pv, qk_gran=gran)
    torch.cuda.synchronize()
    assert p.routed == 1 and torch.equal(got, want)


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
