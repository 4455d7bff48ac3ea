"""Host-side checks of the C ABI (CPU only, no GPU needed).

The library loads on a machine without a GPU, exports every function the header
declares, and rejects every invalid request on the host with the documented
status before making any HIP call (fake device addresses are therefore safe
here: validation never dereferences them).
"""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest
import torch

import quantized_attention_channel_amd as sage
from oracle import sage_ref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sage.h")

FAKE = 0x7F0000000000          # a 256-byte aligned address that is never dereferenced
G = 1 << 30

# The tests marked with this hand fake device addresses to entry points, and
# every such call must be rejected on the host. Were a check missing on a
# machine with a GPU, kernels would run on those addresses, so these tests run
# only where no GPU is visible (device_count does not initialise the runtime).
FAKE_ADDRESSES = pytest.mark.skipif(torch.cuda.device_count() > 0, reason="fake device addresses: CPU-only test")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sage_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("sage_quant_qk", "sage_quant_v", "sage_attn_fwd", "sage_workspace_bytes",
              "sage_block_sizes", "sage_status_string", "sage_debug_qk_i32"):
        assert n in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", sage.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (sage_[a-z0-9_]+)$", out, flags=re.M))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        getattr(sage.lib, n)                        # dlsym succeeds


def test_binding_covers_the_header():
    assert set(declared_functions()) == set(sage._SIGNATURES)


def test_block_sizes_match_the_oracle_readings():
    for d in (64, 128):
        assert sage.sage_block_sizes(d) == (sage_ref.BLK_Q, sage_ref.BLK_K, sage_ref.BKV[d])
        assert sage.sage_block_sizes(d, "per_thread") == (sage_ref.PER_THREAD_BLK_Q, sage_ref.PER_THREAD_BLK_K,
                                                          sage_ref.BKV[d])
    with pytest.raises(sage.SageError) as e:
        sage.sage_block_sizes(96)
    assert e.value.status == sage.SAGE_ERR_UNSUPPORTED
    assert sage.lib.sage_block_sizes(64, 0, None, None, None) == sage.SAGE_OK
    assert sage.lib.sage_block_sizes(64, 2, None, None, None) == sage.SAGE_ERR_INVALID_ARGUMENT
    assert sage.lib.sage_block_sizes(64, -1, None, None, None) == sage.SAGE_ERR_INVALID_ARGUMENT


def test_status_strings():
    for st in range(5):
        assert sage.lib.sage_status_string(st)
    assert b"unknown" in sage.lib.sage_status_string(99)


def test_v_codes_stride():
    assert sage.sage_v_codes_stride(0) == 0
    assert sage.sage_v_codes_stride(1) == 128
    assert sage.sage_v_codes_stride(128) == 128
    assert sage.sage_v_codes_stride(129) == 256


def _shape(**kw):
    base = dict(B=2, Hq=4, Hkv=2, Nq=300, Nk=300, d=128, layout="HND", gran="per_block")
    base.update(kw)
    return sage.make_shape(base["B"], base["Hq"], base["Hkv"], base["Nq"], base["Nk"], base["d"], base["layout"],
                           qk_gran=base["gran"])


def test_shape_struct_matches_the_header():
    # nine int32 fields in header order; a zero-initialised granularity is per-block
    assert ctypes.sizeof(sage.SageShape) == 9 * 4
    assert [f[0] for f in sage.SageShape._fields_][-1] == "qk_gran"
    assert sage.SageShape(1, 1, 1, 8, 8, 64, 0, 0).qk_gran == 0 == sage.QK_GRANS["per_block"]


def test_per_thread_workspace_holds_the_finer_scales():
    pb, pt = _shape(), _shape(gran="per_thread")
    for pv in ("fp8", "fp16"):
        grow = sage.sage_workspace_bytes(pt, pv) - sage.sage_workspace_bytes(pb, pv)
        # q scales: 300 per head instead of 3; k scales: 19 per head instead of 5
        assert grow >= 4 * (2 * 4 * (300 - 3) + 2 * 2 * (19 - 5))


def test_workspace_size_grows_with_the_problem():
    s = _shape()
    w8, w16 = sage.sage_workspace_bytes(s, "fp8"), sage.sage_workspace_bytes(s, "fp16")
    codes = 2 * 4 * 300 * 128 + 2 * 2 * 300 * 128
    assert w8 >= codes + 2 * 2 * 128 * 384 and w16 >= codes + 2 * 2 * 128 * 384 * 2
    assert w8 % 256 == 0 and w16 % 256 == 0
    assert sage.sage_workspace_bytes(_shape(Nq=600, Nk=600), "fp8") > w8
    assert sage.lib.sage_workspace_bytes(None, 1) == 0
    assert sage.lib.sage_workspace_bytes(ctypes.byref(s), 7) == 0
    assert sage.lib.sage_workspace_bytes(ctypes.byref(_shape(d=96)), 1) == 0


def _attn(shape, q=FAKE, k=FAKE + 2 ** 30, v=FAKE + 2 ** 31, o=FAKE + 3 * 2 ** 30, causal=0, scale=0.1,
          pv=1, ws=FAKE + 2 ** 33, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = sage.lib.sage_workspace_bytes(ctypes.byref(shape), pv) if shape is not None else 0
    sp = None if shape is None else ctypes.byref(shape)
    return sage.lib.sage_attn_fwd(sp, q, k, v, o, causal, scale, pv, ws, ws_bytes, None)


@FAKE_ADDRESSES
@pytest.mark.parametrize("case,kw,want", [
    ("null shape", dict(shape=None), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("Hq % Hkv", dict(shape=_shape(Hq=3, Hkv=2)), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("bad layout", dict(shape=sage.SageShape(1, 1, 1, 8, 8, 64, 5, 0)), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("bad dtype", dict(shape=sage.SageShape(1, 1, 1, 8, 8, 64, 0, 9)), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("bad qk_gran", dict(shape=sage.SageShape(1, 1, 1, 8, 8, 64, 0, 0, 7)), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("per-thread, no queries", dict(shape=_shape(gran="per_thread", Nq=0), q=None, o=None), sage.SAGE_OK),
    ("per-thread, per-block workspace", dict(shape=_shape(gran="per_thread"),
                                             ws_bytes=sage.lib.sage_workspace_bytes(ctypes.byref(_shape()), 1)),
     sage.SAGE_ERR_WORKSPACE),
    ("negative seq", dict(shape=_shape(Nq=-1)), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("too long", dict(shape=_shape(Nq=(1 << 20) + 1, Nk=(1 << 20) + 1)), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("head dim 96", dict(shape=_shape(d=96)), sage.SAGE_ERR_UNSUPPORTED),
    ("causal Nq != Nk", dict(shape=_shape(Nq=100, Nk=300), causal=1), sage.SAGE_ERR_UNSUPPORTED),
    ("causal flag 2", dict(shape=_shape(), causal=2), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("sm_scale nan", dict(shape=_shape(), scale=float("nan")), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("sm_scale 0", dict(shape=_shape(), scale=0.0), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("sm_scale inf", dict(shape=_shape(), scale=float("inf")), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("bad pv", dict(shape=_shape(), pv=3), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("null q", dict(shape=_shape(), q=None), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("null o", dict(shape=_shape(), o=None), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("null workspace", dict(shape=_shape(), ws=None), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("misaligned q", dict(shape=_shape(), q=FAKE + 8), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("misaligned ws", dict(shape=_shape(), ws=FAKE + 2 ** 33 + 64), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("small workspace", dict(shape=_shape(), ws_bytes=1024), sage.SAGE_ERR_WORKSPACE),
    ("o aliases q", dict(shape=_shape(), o=FAKE + 4096), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("o aliases workspace", dict(shape=_shape(), o=FAKE + 2 ** 33 + 256), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("workspace aliases k", dict(shape=_shape(), ws=FAKE + 2 ** 30 + 256), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("workspace aliases v", dict(shape=_shape(), ws=FAKE + 2 ** 31), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("no keys", dict(shape=_shape(Nk=0)), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("no queries is a no-op", dict(shape=_shape(Nq=0), q=None, o=None), sage.SAGE_OK),
    ("empty batch is a no-op", dict(shape=_shape(B=0)), sage.SAGE_OK),
])
def test_attn_fwd_validation(case, kw, want):
    assert _attn(**kw) == want, case


@FAKE_ADDRESSES
def test_quant_entry_points_validate():
    s = _shape()
    sp = ctypes.byref(s)
    ws = FAKE + 2 ** 33
    ok_ws = sage.lib.sage_quant_qk_workspace_bytes(sp)
    assert ok_ws > 0
    # null outputs, misalignment, small workspace
    assert sage.lib.sage_quant_qk(sp, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, ws, ok_ws, None) == \
        sage.SAGE_ERR_INVALID_ARGUMENT
    assert sage.lib.sage_quant_qk(sp, FAKE, FAKE, FAKE, FAKE + 2, FAKE, FAKE, FAKE, ws, ok_ws, None) == \
        sage.SAGE_ERR_INVALID_ARGUMENT
    assert sage.lib.sage_quant_qk(sp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, 16, None) == \
        sage.SAGE_ERR_WORKSPACE
    vws = sage.lib.sage_quant_v_workspace_bytes(sp)
    assert vws > 0
    assert sage.lib.sage_quant_v(sp, FAKE, None, FAKE, ws, vws, None) == sage.SAGE_ERR_INVALID_ARGUMENT
    assert sage.lib.sage_quant_v(sp, FAKE, FAKE, FAKE, ws, 16, None) == sage.SAGE_ERR_WORKSPACE
    assert sage.lib.sage_quant_v(ctypes.byref(_shape(d=32)), FAKE, FAKE, FAKE, ws, vws, None) == \
        sage.SAGE_ERR_UNSUPPORTED
    assert sage.lib.sage_debug_qk_i32(sp, None, FAKE, FAKE, None) == sage.SAGE_ERR_INVALID_ARGUMENT
    assert sage.lib.sage_debug_qk_i32(sp, FAKE + 1, FAKE, FAKE, None) == sage.SAGE_ERR_INVALID_ARGUMENT


@FAKE_ADDRESSES
@pytest.mark.parametrize("case,change", [
    ("q codes on q", dict(qc=FAKE + 4096)),
    ("k codes on k", dict(kc=FAKE + G)),
    ("k scale inside q", dict(ks=FAKE + 600000)),
    ("q scale on k codes", dict(qs=FAKE + 4 * G + 16)),
    ("k mean inside the workspace", dict(km=FAKE + 8 * G + 256)),
    ("workspace on k", dict(ws=FAKE + G)),
])
def test_quant_qk_rejects_aliased_writes(case, change):
    sp = ctypes.byref(_shape())
    a = dict(q=FAKE, k=FAKE + G, qc=FAKE + 2 * G, qs=FAKE + 3 * G, kc=FAKE + 4 * G, ks=FAKE + 5 * G, km=FAKE + 6 * G,
             ws=FAKE + 8 * G)
    a.update(change)
    n = sage.lib.sage_quant_qk_workspace_bytes(sp)
    assert sage.lib.sage_quant_qk(sp, a["q"], a["k"], a["qc"], a["qs"], a["kc"], a["ks"], a["km"], a["ws"], n,
                                  None) == sage.SAGE_ERR_INVALID_ARGUMENT, case


@FAKE_ADDRESSES
def test_other_entry_points_reject_aliased_writes():
    s = _shape()
    sp = ctypes.byref(s)
    bad = sage.SAGE_ERR_INVALID_ARGUMENT
    n = sage.lib.sage_quant_v_workspace_bytes(sp)
    v, vc, vs, ws = FAKE, FAKE + G, FAKE + 2 * G, FAKE + 3 * G
    assert sage.lib.sage_quant_v(sp, v, v + 4096, vs, ws, n, None) == bad           # codes on v
    assert sage.lib.sage_quant_v(sp, v, vc, ws, ws, n, None) == bad                 # scale in the workspace
    assert sage.lib.sage_quant_v(sp, v, vc, vs, v + 2 ** 18, n, None) == bad        # workspace inside v
    assert sage.lib.sage_transpose_v(sp, v, v + 4096, None) == bad
    # attention from codes: o may not cover any of the codes or scales it reads
    qc, qs, kc, ks, vp, vsc = (FAKE + i * G for i in range(6))
    for o in (qs, ks, vsc, vp + 4096):
        assert sage.lib.sage_attn_fwd_codes(sp, qc, qs, kc, ks, vp, vsc, o, 0, 0.1, 1, None) == bad
    # v_scale is read as 16-byte vectors: a 4-byte-aligned one is refused
    assert sage.lib.sage_attn_fwd_codes(sp, qc, qs, kc, ks, vp, vsc + 4, FAKE + 7 * G, 0, 0.1, 1, None) == bad
    # the INT32 hook: s_out on the codes, and a product of sizes past 2^64 bytes
    assert sage.lib.sage_debug_qk_i32(sp, FAKE, FAKE + G, FAKE + 64, None) == bad
    huge = ctypes.byref(_shape(B=1 << 10, Hq=1 << 14, Hkv=1 << 14, Nq=1 << 20, Nk=1 << 20))
    assert sage.lib.sage_debug_qk_i32(huge, FAKE + (1 << 44), FAKE + (1 << 45), FAKE, None) == bad


@FAKE_ADDRESSES
def test_noalloc_entry_point_checks_before_any_hip_call():
    """The allocation-free forward refuses shapes whose workspace exceeds its
    fixed array, and bad arguments, before it touches the device."""
    big = _shape(B=1, Hq=32, Hkv=32, Nq=8192, Nk=8192, d=128)
    assert sage.lib.sage_workspace_bytes(ctypes.byref(big), 1) > sage.NOALLOC_MAX_WORKSPACE_BYTES
    assert sage.lib.sage_attn_fwd_noalloc(ctypes.byref(big), FAKE, FAKE + G, FAKE + 2 * G, FAKE + 3 * G, 0, 0.1, 1,
                                          None) == sage.SAGE_ERR_WORKSPACE
    sp = ctypes.byref(_shape())
    bad = sage.SAGE_ERR_INVALID_ARGUMENT
    assert sage.lib.sage_attn_fwd_noalloc(sp, None, FAKE + G, FAKE + 2 * G, FAKE + 3 * G, 0, 0.1, 1, None) == bad
    assert sage.lib.sage_attn_fwd_noalloc(sp, FAKE, FAKE + G, FAKE + 2 * G, FAKE + 8, 0, 0.1, 1, None) == bad
    assert sage.lib.sage_attn_fwd_noalloc(sp, FAKE, FAKE + G, FAKE + 2 * G, FAKE + 3 * G, 0, -1.0, 1, None) == bad
    assert sage.lib.sage_attn_fwd_noalloc(sp, FAKE, FAKE + G, FAKE + 2 * G, FAKE, 0, 0.1, 1, None) == bad   # o on q


def test_fp4_workspace_holds_the_mx_buffers():
    s = _shape()
    B, Hq, Hkv, N, d = 2, 4, 2, 300, 128
    npad = sage.sage_v_codes_stride(N)
    need = (B * Hq * N * d // 2 + B * Hq * N * d // 32 + B * Hkv * N * d // 2 + B * Hkv * N * d // 32
            + B * Hkv * d * 4 + B * Hkv * d * npad // 2 + B * Hkv * d * npad // 32)
    assert sage.lib.sage_fp4_workspace_bytes(ctypes.byref(s)) >= need
    assert sage.lib.sage_quant_fp4_workspace_bytes(ctypes.byref(s)) == sage.lib.sage_quant_qk_workspace_bytes(
        ctypes.byref(s))
    # the MX blocks are fixed: per-thread granularity is not offered, bad enums are invalid
    assert sage.lib.sage_fp4_workspace_bytes(ctypes.byref(_shape(gran="per_thread"))) == 0
    assert sage.lib.sage_fp4_workspace_bytes(ctypes.byref(_shape(d=96))) == 0


@FAKE_ADDRESSES
def test_fp4_entry_points_validate():
    sp = ctypes.byref(_shape())
    bad, ws = sage.SAGE_ERR_INVALID_ARGUMENT, FAKE + 2 ** 33
    n = sage.lib.sage_fp4_workspace_bytes(sp)
    q, k, v, o = (FAKE + i * G for i in range(4))
    fwd = sage.lib.sage_attn_fwd_fp4
    assert fwd(sp, q, k, v, o, 0, 0.1, ws, n - 1, None) == sage.SAGE_ERR_WORKSPACE
    assert fwd(sp, None, k, v, o, 0, 0.1, ws, n, None) == bad
    assert fwd(sp, q, k, v, o + 8, 0, 0.1, ws, n, None) == bad                      # misaligned o
    assert fwd(sp, q, k, v, q, 0, 0.1, ws, n, None) == bad                          # o on q
    assert fwd(sp, q, k, v, o, 2, 0.1, ws, n, None) == bad
    assert fwd(sp, q, k, v, o, 0, float("nan"), ws, n, None) == bad
    assert fwd(sp, q, k, v, o, 0, 0.1, ws + 16, n, None) == bad                     # workspace alignment
    assert fwd(sp, q, k, v, o, 0, 0.1, k + 4096, n, None) == bad                    # workspace inside k
    assert fwd(ctypes.byref(_shape(Nk=200)), q, k, v, o, 1, 0.1, ws, n, None) == sage.SAGE_ERR_UNSUPPORTED
    assert fwd(ctypes.byref(_shape(gran="per_thread")), q, k, v, o, 0, 0.1, ws, n, None) == sage.SAGE_ERR_UNSUPPORTED
    assert fwd(ctypes.byref(_shape(d=32)), q, k, v, o, 0, 0.1, ws, n, None) == sage.SAGE_ERR_UNSUPPORTED
    assert fwd(ctypes.byref(_shape(Nq=0)), None, None, None, None, 0, 0.1, None, 0, None) == sage.SAGE_OK
    # quantisation: null, misaligned and aliased outputs, small workspace
    qc, qs, kc, ks, km, vc, vs = (FAKE + i * G for i in range(4, 11))
    qw = sage.lib.sage_quant_fp4_workspace_bytes(sp)
    quant = sage.lib.sage_quant_fp4
    assert quant(sp, q, k, v, 0.1, None, qs, kc, ks, km, vc, vs, ws, qw, None) == bad
    assert quant(sp, q, k, v, 0.1, qc, qs, kc, ks, km, vc, vs + 4, ws, qw, None) == bad   # v_scale needs 16 bytes
    assert quant(sp, q, k, v, 0.1, qc, qs, kc, ks, km, vc, vs, ws, qw - 1, None) == sage.SAGE_ERR_WORKSPACE
    assert quant(sp, q, k, v, 0.1, qc, qs, kc, ks, km, v + 4096, vs, ws, qw, None) == bad  # codes on v
    assert quant(sp, q, k, v, 0.1, qc, qs, kc, qc + 16, km, vc, vs, ws, qw, None) == bad   # k scale on q codes
    assert quant(sp, q, k, v, float("inf"), qc, qs, kc, ks, km, vc, vs, ws, qw, None) == bad
    assert quant(sp, q, k, v, -0.1, qc, qs, kc, ks, km, vc, vs, ws, qw, None) == bad
    # attention from codes: o may not cover what it reads; v_scale 16-byte aligned
    codes = sage.lib.sage_attn_fwd_fp4_codes
    for oo in (qs, ks, vs, vc + 4096):
        assert codes(sp, qc, qs, kc, ks, vc, vs, oo, 0, None) == bad
    assert codes(sp, qc, qs, kc, ks, vc, vs + 4, o, 0, None) == bad
    assert codes(sp, qc, qs, kc, ks, None, vs, o, 0, None) == bad
    assert codes(sp, qc, qs, kc, ks, vc, vs, o, 3, None) == bad


def test_python_wrapper_rejects_unsupported_sdpa_arguments():
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.float16)
    with pytest.raises(NotImplementedError):
        sage.sageattn(q, q, q, attn_mask=torch.ones(4, 4))
    with pytest.raises(NotImplementedError):
        sage.sageattn(q, q, q, dropout_p=0.1)
    with pytest.raises(TypeError):
        sage.sageattn(q, q, q, bogus=1)
    with pytest.raises(ValueError):                       # CPU tensors never reach the library
        sage.sageattn(q, q, q)


# ------------------------------------------------------------------ packed variable-length batches
def _vshape(**kw):
    base = dict(B=3, Hq=4, Hkv=2, d=128, tq=500, tk=700, mq=300, mk=400, dtype=0, gran=0)
    base.update(kw)
    return sage.SageVarlenShape(base["B"], base["Hq"], base["Hkv"], base["d"], base["tq"], base["tk"], base["mq"],
                                base["mk"], base["dtype"], base["gran"])


def test_varlen_shape_struct_matches_the_header():
    assert ctypes.sizeof(sage.SageVarlenShape) == 10 * 4
    assert [f[0] for f in sage.SageVarlenShape._fields_] == [
        "batch", "heads_q", "heads_kv", "head_dim", "total_q", "total_k", "max_seqlen_q", "max_seqlen_k", "dtype",
        "qk_gran"]


def test_varlen_workspace_holds_the_packed_intermediates():
    s = _vshape()
    w8 = sage.sage_varlen_workspace_bytes(s, "fp8")
    # codes [H][total][d], V^T [Hkv][d][padded total], the span table
    assert w8 >= 4 * 500 * 128 + 2 * 700 * 128 + 2 * 128 * (700 + 127 * 3) + 3 * 32
    assert sage.sage_varlen_workspace_bytes(s, "fp16") > w8
    assert sage.sage_varlen_workspace_bytes(_vshape(gran=1), "fp8") > w8      # finer scales
    assert sage.lib.sage_varlen_workspace_bytes(None, 1) == 0
    assert sage.lib.sage_varlen_workspace_bytes(ctypes.byref(_vshape(d=96)), 1) == 0


def _vattn(shape, q=FAKE, k=FAKE + 2 ** 30, v=FAKE + 2 ** 31, cq=FAKE + 2 ** 34, ck=FAKE + 2 ** 34 + 64,
           o=FAKE + 3 * 2 ** 30, causal=0, scale=0.1, pv=1, ws=FAKE + 2 ** 33, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = sage.lib.sage_varlen_workspace_bytes(ctypes.byref(shape), pv) if shape is not None else 0
    sp = None if shape is None else ctypes.byref(shape)
    return sage.lib.sage_attn_fwd_varlen(sp, q, k, v, cq, ck, o, causal, scale, pv, ws, ws_bytes, None)


@FAKE_ADDRESSES
@pytest.mark.parametrize("case,kw,want", [
    ("null shape", dict(shape=None), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("Hq % Hkv", dict(shape=_vshape(Hq=3)), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("bad dtype", dict(shape=_vshape(dtype=5)), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("bad qk_gran", dict(shape=_vshape(gran=3)), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("negative total", dict(shape=_vshape(tk=-1)), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("max seqlen too long", dict(shape=_vshape(mq=(1 << 20) + 1)), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("padded keys too many", dict(shape=_vshape(tk=(1 << 24) - 300)), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("head dim 96", dict(shape=_vshape(d=96)), sage.SAGE_ERR_UNSUPPORTED),
    ("causal flag 2", dict(shape=_vshape(), causal=2), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("sm_scale nan", dict(shape=_vshape(), scale=float("nan")), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("bad pv", dict(shape=_vshape(), pv=2), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("null cu_seqlens_q", dict(shape=_vshape(), cq=None), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("null cu_seqlens_k", dict(shape=_vshape(), ck=None), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("misaligned cu_seqlens", dict(shape=_vshape(), cq=FAKE + 2 ** 34 + 2), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("null o", dict(shape=_vshape(), o=None), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("null k with keys", dict(shape=_vshape(), k=None), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("null k, v without keys reach the device", dict(shape=_vshape(tk=0), k=None, v=None), sage.SAGE_ERR_HIP),
    ("misaligned v", dict(shape=_vshape(), v=FAKE + 2 ** 31 + 8), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("small workspace", dict(shape=_vshape(), ws_bytes=4096), sage.SAGE_ERR_WORKSPACE),
    ("o aliases q", dict(shape=_vshape(), o=FAKE + 4096), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("workspace aliases q", dict(shape=_vshape(), ws=FAKE + 4096), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("workspace aliases cu_seqlens_q", dict(shape=_vshape(), ws=FAKE + 2 ** 34 - 256), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("o aliases cu_seqlens_k", dict(shape=_vshape(), o=FAKE + 2 ** 34 + 64), sage.SAGE_ERR_INVALID_ARGUMENT),
    ("no sequences is a no-op", dict(shape=_vshape(B=0), q=None, o=None), sage.SAGE_OK),
    ("no queries is a no-op", dict(shape=_vshape(tq=0), q=None, o=None), sage.SAGE_OK),
])
def test_attn_fwd_varlen_validation(case, kw, want):
    assert _vattn(**kw) == want, case


def test_fp4_varlen_workspace_holds_the_mx_buffers():
    s = _vshape()
    npad = sage.varlen_v_codes_stride(700, 3)
    need = (4 * 500 * 128 // 2 + 4 * 500 * 128 // 32 + 2 * 700 * 128 // 2 + 2 * 700 * 128 // 32
            + 3 * 2 * 128 * 4 + 2 * 128 * npad // 2 + 2 * 128 * npad // 32 + 3 * 32)
    assert sage.sage_fp4_varlen_workspace_bytes(s) >= need
    assert 0 < sage.lib.sage_quant_fp4_varlen_workspace_bytes(ctypes.byref(s)) < need
    # fixed MX blocks: per-thread granularity is unsupported, bad shapes invalid
    for bad in (_vshape(gran=1), _vshape(d=96), _vshape(Hq=3)):
        assert sage.sage_fp4_varlen_workspace_bytes(bad) == 0
        assert sage.lib.sage_quant_fp4_varlen_workspace_bytes(ctypes.byref(bad)) == 0
    assert sage.lib.sage_fp4_varlen_workspace_bytes(None) == 0


@FAKE_ADDRESSES
def test_fp4_varlen_entry_points_validate():
    s = _vshape()
    sp = ctypes.byref(s)
    bad, ws = sage.SAGE_ERR_INVALID_ARGUMENT, FAKE + 2 ** 33
    q, k, v, o = FAKE, FAKE + G, FAKE + 2 * G, FAKE + 3 * G
    cq, ck = FAKE + 2 ** 34, FAKE + 2 ** 34 + 64
    n = sage.sage_fp4_varlen_workspace_bytes(s)
    fwd = sage.lib.sage_attn_fwd_fp4_varlen
    assert fwd(sp, q, k, v, cq, ck, o, 0, 0.1, ws, n - 1, None) == sage.SAGE_ERR_WORKSPACE
    assert fwd(sp, None, k, v, cq, ck, o, 0, 0.1, ws, n, None) == bad
    assert fwd(sp, q, k, v, None, ck, o, 0, 0.1, ws, n, None) == bad
    assert fwd(sp, q, k, v, cq + 2, ck, o, 0, 0.1, ws, n, None) == bad               # misaligned cu_seqlens
    assert fwd(sp, q, k, v, cq, ck, o + 8, 0, 0.1, ws, n, None) == bad               # misaligned o
    assert fwd(sp, q, k, v, cq, ck, q + 4096, 0, 0.1, ws, n, None) == bad            # o on q
    assert fwd(sp, q, k, v, cq, ck, o, 0, 0.1, cq - 256, n, None) == bad             # workspace on cu_seqlens
    assert fwd(sp, q, k, v, cq, ck, o, 2, 0.1, ws, n, None) == bad
    assert fwd(sp, q, k, v, cq, ck, o, 0, float("nan"), ws, n, None) == bad
    assert fwd(ctypes.byref(_vshape(gran=1)), q, k, v, cq, ck, o, 0, 0.1, ws, n, None) == sage.SAGE_ERR_UNSUPPORTED
    assert fwd(ctypes.byref(_vshape(d=96)), q, k, v, cq, ck, o, 0, 0.1, ws, n, None) == sage.SAGE_ERR_UNSUPPORTED
    assert fwd(ctypes.byref(_vshape(tq=0)), None, None, None, None, None, None, 0, 0.1, None, 0, None) == sage.SAGE_OK
    assert fwd(sp, q, None, v, cq, ck, o, 0, 0.1, ws, n, None) == bad                  # null k with keys
    nok = _vshape(tk=0, mk=0)
    assert fwd(ctypes.byref(nok), q, None, None, cq, ck, o, 0, 0.1, ws, sage.sage_fp4_varlen_workspace_bytes(nok),
               None) == sage.SAGE_ERR_HIP                                                # no keys: reaches the device
    # quantisation alone
    qc, qs, kc, ks, km, vc, vs = (FAKE + i * G for i in range(4, 11))
    qw = sage.lib.sage_quant_fp4_varlen_workspace_bytes(sp)
    quant = sage.lib.sage_quant_fp4_varlen
    args = [sp, q, k, v, cq, ck, 0.1, qc, qs, kc, ks, km, vc, vs, ws, qw, None]

    def call(**change):
        a = list(args)
        for i, val in change.items():
            a[int(i[1:])] = val
        return quant(*a)
    assert call(a15=qw - 1) == sage.SAGE_ERR_WORKSPACE
    assert call(a7=None) == bad                                                    # q_codes
    assert call(a13=vs + 4) == bad                                                 # v_scale needs 16 bytes
    assert call(a12=v + 4096) == bad                                               # v codes on v
    assert call(a10=qc + 16) == bad                                                # k scale on q codes
    assert call(a14=ck - 64) == bad                                                # workspace on cu_seqlens
    assert call(a6=-0.1) == bad
    assert call(a0=ctypes.byref(_vshape(gran=1))) == sage.SAGE_ERR_UNSUPPORTED
    # no keys: the K and V outputs may be NULL (the call then reaches the device)
    nok = ctypes.byref(_vshape(tk=0, mk=0))
    assert quant(nok, q, None, None, cq, ck, 0.1, qc, qs, None, None, None, None, None, ws,
                 sage.lib.sage_quant_fp4_varlen_workspace_bytes(nok), None) == sage.SAGE_ERR_HIP
    assert quant(ctypes.byref(_vshape(B=0)), None, None, None, cq, ck, 0.1, *([None] * 7), ws, 0,
                 None) == sage.SAGE_OK


def _plan_model(cq, ck, total_q, total_k, max_q, max_k, n_pad, owner=None):
    """The span rules of the plan kernel: clamp, pack the padded keys, and list
    each sequence's query pairs (256 queries) in a work list of bounded size."""
    n_owner = total_q // 256 + (len(cq) - 1)
    spans, carry, carryq = [], 0, 0
    table = [None] * n_owner
    for b in range(len(cq) - 1):
        q0 = min(max(cq[b], 0), total_q)
        q1 = min(max(cq[b + 1], q0), total_q)
        k0 = min(max(ck[b], 0), total_k)
        k1 = min(max(ck[b + 1], k0), total_k)
        nq, nk = min(q1 - q0, max_q), min(k1 - k0, max_k)
        padded, pairs = -(-nk // 128) * 128, -(-nq // 256)
        kp0, qp0 = carry, carryq
        carry += padded
        carryq += pairs
        if kp0 + padded > n_pad:
            nk, kp0 = 0, 0
        for i in range(qp0, min(qp0 + pairs, n_owner)):
            table[i] = b
        spans.append((q0, nq, k0, nk, kp0, min(qp0, n_owner)))
    for i in range(carryq, n_owner):
        table[i] = -1
    if owner is not None:
        owner.extend(table)
    return spans


def test_varlen_plan_clamps_every_span_into_bounds():
    rng = np.random.default_rng(5)
    for trial in range(300):
        B = int(rng.integers(1, 40))
        total_q, total_k = int(rng.integers(0, 5000)), int(rng.integers(0, 5000))
        max_q, max_k = int(rng.integers(0, 3000)), int(rng.integers(0, 3000))
        n_pad = -(-(total_k + 127 * B) // 128) * 128 or 128
        if trial % 3 == 0:                               # well-formed tables
            cuts = np.sort(rng.integers(0, total_k + 1, B - 1))
            ck = [0, *cuts.tolist(), total_k]
            cq = ck if total_q == total_k else [0, *np.sort(rng.integers(0, total_q + 1, B - 1)).tolist(), total_q]
        else:                                            # arbitrary, also negative and decreasing
            cq = rng.integers(-100, total_q + 200, B + 1).tolist()
            ck = rng.integers(-100, total_k + 200, B + 1).tolist()
        padded_cols = set()
        owner = []
        spans = _plan_model(cq, ck, total_q, total_k, max_q, max_k, n_pad, owner)
        for q0, nq, k0, nk, kp0, qp0 in spans:
            assert 0 <= q0 and q0 + nq <= total_q and 0 <= nq <= max_q
            assert 0 <= k0 and k0 + nk <= total_k and 0 <= nk <= max_k
            assert 0 <= kp0 and kp0 + -(-nk // 128) * 128 <= n_pad
            cols = set(range(kp0, kp0 + -(-nk // 128) * 128))
            assert not cols & padded_cols                # V^T column slots never overlap
            padded_cols |= cols
        # every work-list entry is filled; an entry names a sequence whose
        # pair index (entry - qp0) lies inside that sequence's pairs
        assert all(e is not None for e in owner)
        for i, b in enumerate(owner):
            if b >= 0:
                q0, nq, _, _, _, qp0 = spans[b]
                assert 0 <= i - qp0 < -(-nq // 256)
        if trial % 3 == 0 and max(np.diff(ck)) <= max_k and max(np.diff(cq)) <= max_q:
            # well-formed: nothing is dropped, every query pair is listed once
            assert [s[3] for s in spans] == np.diff(ck).tolist()
            listed = sorted((b, i - spans[b][5]) for i, b in enumerate(owner) if b >= 0)
            assert listed == [(b, p) for b in range(B) for p in range(-(-(cq[b + 1] - cq[b]) // 256))]


def test_binding_fails_loudly_without_the_library(tmp_path):
    """No fallback: importing the binding with the library missing raises."""
    env = dict(os.environ, SAGE_LIB_PATH=str(tmp_path / "missing" / "libsage.so"))
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", "import quantized_attention_channel_amd"], cwd=root, env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and "ImportError" in r.stderr and "not built" in r.stderr


C_USER = r"""
#include <stdio.h>
#include "sage.h"
int main(void) {
  sage_shape s = {2, 4, 2, 300, 300, 128, SAGE_LAYOUT_HND, SAGE_DTYPE_F16, SAGE_QK_PER_BLOCK};
  sage_varlen_shape vs = {3, 4, 2, 128, 500, 700, 300, 400, SAGE_DTYPE_BF16, SAGE_QK_PER_THREAD};
  int32_t bq = 0, bk = 0, bkv = 0;
  if (sage_block_sizes(128, SAGE_QK_PER_THREAD, &bq, &bk, &bkv) != SAGE_OK) return 1;
  if (sage_workspace_bytes(&s, SAGE_PV_FP8_E4M3) == 0 || sage_varlen_workspace_bytes(&vs, SAGE_PV_FP16) == 0) return 2;
  /* host validation runs before any HIP call: null tensors are rejected without a GPU */
  if (sage_attn_fwd(&s, 0, 0, 0, 0, 0, 0.1f, SAGE_PV_FP8_E4M3, 0, 0, 0) != SAGE_ERR_INVALID_ARGUMENT) return 3;
  printf("%d %d %d %d\n", bq, bk, bkv, (int)sizeof(sage_varlen_shape));
  return 0;
}
"""


def test_header_is_plain_c_and_the_library_links_from_c(tmp_path):
    """The boundary is a C ABI: the header compiles as strict C99 and a C program
    links against libsage.so and calls its host-side entry points."""
    import shutil
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    pkg = os.path.join(root, "quantized_attention_channel_amd")
    src = tmp_path / "use_sage.c"
    src.write_text(C_USER)
    exe = tmp_path / "use_sage"
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(root, "include"),
                        str(src), "-L", pkg, "-lsage", f"-Wl,-rpath,{pkg}", "-o", str(exe)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, (r.returncode, r.stderr)
    assert r.stdout.split() == [str(sage_ref.PER_THREAD_BLK_Q), str(sage_ref.PER_THREAD_BLK_K),
                                str(sage_ref.BKV[128]), str(10 * 4)]


def test_binding_checks_shapes_before_any_library_call():
    """The binding rejects tensors whose sizes would let a kernel run past a
    buffer (checked on CPU tensors: the checks precede every library call)."""
    q = torch.empty(2, 4, 100, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="batch or head_dim"):
        sage.shape_of(q, torch.empty(1, 2, 100, 64, dtype=torch.float16), "HND")      # k's batch smaller
    with pytest.raises(ValueError, match="batch or head_dim"):
        sage.shape_of(q, torch.empty(2, 2, 100, 32, dtype=torch.float16), "HND")      # k's head_dim smaller
    with pytest.raises(TypeError, match="one dtype"):
        sage.shape_of(q, torch.empty(2, 2, 100, 64, dtype=torch.bfloat16), "HND")
    with pytest.raises(ValueError, match="batch or head_dim"):
        sage.shape_of(q.transpose(1, 2), torch.empty(2, 100, 2, 128, dtype=torch.float16), "NHD")
    # packed batches
    cq = torch.tensor([0, 50, 100], dtype=torch.int32)
    with pytest.raises(ValueError, match="head_dim"):
        sage.varlen_shape_of(torch.empty(100, 4, 64, dtype=torch.float16),
                             torch.empty(100, 2, 128, dtype=torch.float16), cq, 50, 50)
    # outputs and workspaces handed in by the caller
    cpu = torch.device("cpu")
    with pytest.raises(ValueError, match="shape"):
        sage._out_like(q, torch.empty(2, 4, 99, 64, dtype=torch.float16))
    with pytest.raises(TypeError, match="float16"):
        sage._out_like(q, torch.empty(2, 4, 100, 64, dtype=torch.float32))
    with pytest.raises(ValueError, match="contiguous"):
        sage._out_like(q, torch.empty(2, 100, 4, 64, dtype=torch.float16).transpose(1, 2))
    assert sage._out_like(q, None).shape == q.shape
    with pytest.raises(TypeError, match="uint8"):
        sage._workspace_for(torch.empty(4096, dtype=torch.float32), 1024, cpu)
    with pytest.raises(ValueError, match="must be on"):
        sage._workspace_for(torch.empty(4096, dtype=torch.uint8), 1024, torch.device("meta"))
    ws = torch.empty(4096, dtype=torch.uint8)
    assert sage._workspace_for(ws, 1024, cpu) is ws
    assert sage._workspace_for(ws, 8192, cpu).numel() == 8192
    with pytest.raises(ValueError, match="elements"):
        sage._expect(torch.empty(10, dtype=torch.int8), "q_codes", torch.int8, 11, cpu)
    # the codes entry point checks every buffer against the shape (o first: it must be a GPU tensor)
    s = sage.make_shape(1, 2, 2, 100, 100, 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        sage.sage_attn_fwd_codes(s, None, None, None, None, None, None, torch.empty(1, 2, 100, 64, dtype=torch.float16))
