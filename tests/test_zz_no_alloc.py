"""sage_attn_fwd_noalloc (the library's fixed workspace, no allocation) against
sage_attn_fwd with a caller workspace: bit-identical outputs, through the C ABI,
on two calls in a row, the second with a smaller input (the fixed array keeps
the first call's contents, which must not leak into the second)."""
import ctypes

import pytest
import torch

import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

if torch.cuda.is_available():
    import quantized_attention_channel_amd as sage


def _both(w, pv):
    q, k, v = (t.cuda() for t in W.generate(w))
    want = sage.sage_attn_fwd(q, k, v, is_causal=w.causal, sm_scale=w.sm_scale, pv_dtype=pv, tensor_layout=w.layout)
    s = sage.shape_of(q, k, w.layout)
    assert sage.sage_workspace_bytes(s, pv) <= sage.NOALLOC_MAX_WORKSPACE_BYTES
    got = torch.full_like(q, float("nan"))
    st = sage.lib.sage_attn_fwd_noalloc(ctypes.byref(s), sage._ptr(q), sage._ptr(k), sage._ptr(v), sage._ptr(got),
                                        int(w.causal), float(w.sm_scale), sage.PV_DTYPES[pv],
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == sage.SAGE_OK, sage.lib.sage_status_string(st)
    return got, want


@pytest.mark.parametrize("pv", ["fp8", "fp16"])
def test_noalloc_equals_workspace_entry_point(pv):
    big = W.PEAK.with_(B=1, Hq=16, Hkv=8, N=4096, causal=True)         # workspace 16.2 (FP8) or 20.2 MiB of 32
    small = W.TINY.with_(B=2, Hq=4, Hkv=2, N=333, d=128, dtype="bf16", layout="NHD")
    for w in (big, small):
        print("noalloc", w.name, w.B, w.Hq, w.Hkv, w.N, w.d, pv, flush=True)
        got, want = _both(w, pv)
        assert torch.equal(got, want)


def test_noalloc_refuses_a_workspace_beyond_its_limit():
    w = W.PEAK.with_(B=1, Hq=32, Hkv=32, N=8192)                      # ~ 70 MB of workspace
    q = torch.empty(1, 32, 8192, 128, dtype=torch.float16, device="cuda")
    s = sage.shape_of(q, q, "HND")
    assert sage.sage_workspace_bytes(s, "fp8") > sage.NOALLOC_MAX_WORKSPACE_BYTES
    with pytest.raises(sage.SageError) as e:
        sage.sage_attn_fwd_noalloc(q, q, q, torch.empty_like(q), sm_scale=w.sm_scale)
    assert e.value.status == sage.SAGE_ERR_WORKSPACE
