"""Python binding of libsage (include/sage.h): MI355X quantised attention forward.

Argument marshalling only. Every step of the computation runs in the gfx950 HIP
kernels behind the C ABI; PyTorch supplies device memory and the current stream.
There is no fallback: if ``libsage.so`` is missing or fails to load, importing
the binding raises.

Entry points (same names as the C ABI):
  sage_block_sizes, sage_v_codes_stride, sage_workspace_bytes,
  sage_quant_qk, sage_quant_v, sage_transpose_v, sage_attn_fwd,
  sage_attn_fwd_codes, sage_debug_qk_i32, sage_varlen_workspace_bytes,
  sage_attn_fwd_varlen, sage_quant_varlen, sage_quant_varlen_workspace_bytes,
  sage_attn_fwd_noalloc, sage_quant_fp4, sage_quant_fp4_workspace_bytes,
  sage_fp4_workspace_bytes, sage_attn_fwd_fp4_codes, sage_attn_fwd_fp4,
  sage_fp4_varlen_workspace_bytes, sage_attn_fwd_fp4_varlen,
  sage_quant_fp4_varlen_workspace_bytes, sage_quant_fp4_varlen.
User-facing wrapper:
  sageattn(q, k, v, tensor_layout="HND", is_causal=False, sm_scale=None,
           pv_dtype="fp8", qk_quant_gran="per_block") -- the call shape the
  SageAttention pages show (cnnetsun.cn guide, basic usage; thu-ml/SageAttention
  repo card, "How to use"); qk_quant_gran="per_thread" selects the per-thread
  Q/K scales (heatdrop.ai review, "The interesting bit").
  sageattn_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                  max_seqlen_k, ...) -- packed variable-length batches
  (heatdrop.ai review, "Key highlights").
  pv_dtype="fp4" in sageattn and sageattn_varlen selects the FP4 microscaling
  variant (MXFP4 Q, K, P and V; heatdrop.ai review, "Key highlights";
  cnnetsun.cn guide, 序列长度优化技巧).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SAGE_LIB_PATH selects another build of the same library (same ABI); default: in-tree.
LIB_PATH = os.environ.get("SAGE_LIB_PATH") or os.path.join(_HERE, "libsage.so")

SAGE_OK, SAGE_ERR_INVALID_ARGUMENT, SAGE_ERR_UNSUPPORTED, SAGE_ERR_WORKSPACE, SAGE_ERR_HIP = range(5)
LAYOUTS = {"HND": 0, "NHD": 1}
DTYPES = {torch.float16: 0, torch.bfloat16: 1}
PV_DTYPES = {"fp16": 0, "fp8": 1, "fp8_e4m3": 1}
QK_GRANS = {"per_block": 0, "per_thread": 1}

# Every function the header declares, with its ctypes signature.
_c_shape_p = ctypes.c_void_p
_vp = ctypes.c_void_p
_SIGNATURES = {
    "sage_block_sizes": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp]),
    "sage_v_codes_stride": (ctypes.c_int64, [ctypes.c_int32]),
    "sage_quant_qk_workspace_bytes": (ctypes.c_size_t, [_c_shape_p]),
    "sage_quant_v_workspace_bytes": (ctypes.c_size_t, [_c_shape_p]),
    "sage_workspace_bytes": (ctypes.c_size_t, [_c_shape_p, ctypes.c_int32]),
    "sage_quant_qk": (ctypes.c_int, [_c_shape_p, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "sage_quant_v": (ctypes.c_int, [_c_shape_p, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "sage_attn_fwd": (ctypes.c_int, [_c_shape_p, _vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_float,
                                     ctypes.c_int32, _vp, ctypes.c_size_t, _vp]),
    "sage_transpose_v": (ctypes.c_int, [_c_shape_p, _vp, _vp, _vp]),
    "sage_attn_fwd_codes": (ctypes.c_int, [_c_shape_p, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32,
                                           ctypes.c_float, ctypes.c_int32, _vp]),
    "sage_debug_qk_i32": (ctypes.c_int, [_c_shape_p, _vp, _vp, _vp, _vp]),
    "sage_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "sage_varlen_workspace_bytes": (ctypes.c_size_t, [_c_shape_p, ctypes.c_int32]),
    "sage_attn_fwd_varlen": (ctypes.c_int, [_c_shape_p, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32,
                                            ctypes.c_float, ctypes.c_int32, _vp, ctypes.c_size_t, _vp]),
    "sage_attn_fwd_noalloc": (ctypes.c_int, [_c_shape_p, _vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_float,
                                             ctypes.c_int32, _vp]),
    "sage_quant_varlen_workspace_bytes": (ctypes.c_size_t, [_c_shape_p]),
    "sage_quant_varlen": (ctypes.c_int, [_c_shape_p, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                         _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "sage_quant_fp4_workspace_bytes": (ctypes.c_size_t, [_c_shape_p]),
    "sage_fp4_workspace_bytes": (ctypes.c_size_t, [_c_shape_p]),
    "sage_quant_fp4": (ctypes.c_int, [_c_shape_p, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _vp, _vp, ctypes.c_size_t, _vp]),
    "sage_attn_fwd_fp4_codes": (ctypes.c_int, [_c_shape_p, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32,
                                               _vp]),
    "sage_attn_fwd_fp4": (ctypes.c_int, [_c_shape_p, _vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_float, _vp,
                                         ctypes.c_size_t, _vp]),
    "sage_fp4_varlen_workspace_bytes": (ctypes.c_size_t, [_c_shape_p]),
    "sage_attn_fwd_fp4_varlen": (ctypes.c_int, [_c_shape_p, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32,
                                                ctypes.c_float, _vp, ctypes.c_size_t, _vp]),
    "sage_quant_fp4_varlen_workspace_bytes": (ctypes.c_size_t, [_c_shape_p]),
    "sage_quant_fp4_varlen": (ctypes.c_int, [_c_shape_p, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp,
                                             _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
}
# the workspace limit of sage_attn_fwd_noalloc (SAGE_NOALLOC_MAX_WORKSPACE_BYTES in sage.h)
NOALLOC_MAX_WORKSPACE_BYTES = 32 * 1024 * 1024


class SageShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "heads_q", "heads_kv", "seq_q", "seq_k", "head_dim", "layout", "dtype", "qk_gran")]


class SageVarlenShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "heads_q", "heads_kv", "head_dim", "total_q", "total_k", "max_seqlen_q", "max_seqlen_k",
                 "dtype", "qk_gran")]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run quantized_attention_channel_amd/build.py "
                          "(or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class SageError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib.sage_status_string(status).decode()}")


def _check(status: int, where: str):
    if status != SAGE_OK:
        raise SageError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def make_shape(B, Hq, Hkv, Nq, Nk, d, layout="HND", dtype=torch.float16, qk_gran="per_block") -> SageShape:
    return SageShape(B, Hq, Hkv, Nq, Nk, d, LAYOUTS[layout], DTYPES[dtype], QK_GRANS[qk_gran])


def shape_of(q: torch.Tensor, k: torch.Tensor, layout: str, qk_gran: str = "per_block") -> SageShape:
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be 4-D")
    if layout == "HND":
        B, Hq, Nq, d = q.shape
        _, Hkv, Nk, _ = k.shape
    elif layout == "NHD":
        B, Nq, Hq, d = q.shape
        _, Nk, Hkv, _ = k.shape
    else:
        raise ValueError(f"tensor_layout must be HND or NHD, got {layout!r}")
    if q.dtype not in DTYPES:
        raise TypeError(f"q/k/v must be float16 or bfloat16, got {q.dtype}")
    if k.dtype != q.dtype:
        raise TypeError("q and k must have one dtype")
    if k.shape[0] != B or k.shape[-1] != d:
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} differ in batch or head_dim")
    return make_shape(B, Hq, Hkv, Nq, Nk, d, layout, q.dtype, qk_gran)


def _ref(s: SageShape):
    return ctypes.byref(s)


# ------------------------------------------------------------------ queries
def sage_block_sizes(head_dim: int, qk_gran: str = "per_block"):
    bq, bk, bkv = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib.sage_block_sizes(head_dim, QK_GRANS[qk_gran], ctypes.byref(bq), ctypes.byref(bk),
                                ctypes.byref(bkv)), "sage_block_sizes")
    return bq.value, bk.value, bkv.value


def sage_v_codes_stride(seq_k: int) -> int:
    return int(lib.sage_v_codes_stride(seq_k))


def sage_workspace_bytes(shape: SageShape, pv_dtype: str = "fp8") -> int:
    return int(lib.sage_workspace_bytes(_ref(shape), PV_DTYPES[pv_dtype]))


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _expect(t: Optional[torch.Tensor], name: str, dtype: torch.dtype, numel: int, device: torch.device):
    """A tensor the library reads or writes as a dense buffer of `numel`
    elements of `dtype` on `device`."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _out_like(q: torch.Tensor, out: Optional[torch.Tensor]) -> torch.Tensor:
    if out is None:
        return torch.empty_like(q)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError(f"out must have q's shape {tuple(q.shape)}, got {tuple(out.shape)}")
    _expect(out, "out", q.dtype, q.numel(), q.device)
    return out


def _workspace_for(workspace: Optional[torch.Tensor], need: int, device: torch.device) -> torch.Tensor:
    """The caller's workspace (a contiguous uint8 tensor on `device`) if it
    holds `need` bytes, else a fresh one."""
    if workspace is None:
        return _workspace(need, device)
    _expect(workspace, "workspace", torch.uint8, workspace.numel(), device)
    return workspace if workspace.numel() >= need else _workspace(need, device)


def _check_inputs(*ts):
    dev = ts[0].device
    for t in ts:
        if not t.is_cuda or t.device != dev:
            raise ValueError("all tensors must be on the same GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous in the stated layout")


# ------------------------------------------------------------------ entry points
def sage_quant_qk(q: torch.Tensor, k: torch.Tensor, tensor_layout: str = "HND", qk_gran: str = "per_block"):
    """Returns dict(q_codes, q_scale, k_codes, k_scale, k_mean) (canonical HND order)."""
    _check_inputs(q, k)
    s = shape_of(q, k, tensor_layout, qk_gran)
    blk_q, blk_k, _ = sage_block_sizes(s.head_dim, qk_gran)
    dev = q.device
    out = dict(
        q_codes=torch.empty((s.batch, s.heads_q, s.seq_q, s.head_dim), dtype=torch.int8, device=dev),
        q_scale=torch.empty((s.batch, s.heads_q, -(-s.seq_q // blk_q)), dtype=torch.float32, device=dev),
        k_codes=torch.empty((s.batch, s.heads_kv, s.seq_k, s.head_dim), dtype=torch.int8, device=dev),
        k_scale=torch.empty((s.batch, s.heads_kv, -(-s.seq_k // blk_k)), dtype=torch.float32, device=dev),
        k_mean=torch.empty((s.batch, s.heads_kv, s.head_dim), dtype=torch.float32, device=dev),
    )
    ws = _workspace(lib.sage_quant_qk_workspace_bytes(_ref(s)), dev)
    _check(lib.sage_quant_qk(_ref(s), _ptr(q), _ptr(k), _ptr(out["q_codes"]), _ptr(out["q_scale"]),
                             _ptr(out["k_codes"]), _ptr(out["k_scale"]), _ptr(out["k_mean"]),
                             _ptr(ws), ws.numel(), _stream(dev)), "sage_quant_qk")
    return out


def sage_quant_v(v: torch.Tensor, tensor_layout: str = "HND"):
    """Returns (v_codes uint8 [B,Hkv,d,Nk_pad], v_scale fp32 [B,Hkv,d])."""
    _check_inputs(v)
    s = shape_of(v, v, tensor_layout)
    dev = v.device
    npad = sage_v_codes_stride(s.seq_k)
    codes = torch.empty((s.batch, s.heads_kv, s.head_dim, npad), dtype=torch.uint8, device=dev)
    scale = torch.empty((s.batch, s.heads_kv, s.head_dim), dtype=torch.float32, device=dev)
    ws = _workspace(lib.sage_quant_v_workspace_bytes(_ref(s)), dev)
    _check(lib.sage_quant_v(_ref(s), _ptr(v), _ptr(codes), _ptr(scale), _ptr(ws), ws.numel(), _stream(dev)),
           "sage_quant_v")
    return codes, scale


def sage_transpose_v(v: torch.Tensor, tensor_layout: str = "HND") -> torch.Tensor:
    """16-bit V transposed to [B,Hkv,d,Nk_pad] (the FP16-PV operand layout)."""
    _check_inputs(v)
    s = shape_of(v, v, tensor_layout)
    vt = torch.empty((s.batch, s.heads_kv, s.head_dim, sage_v_codes_stride(s.seq_k)), dtype=v.dtype,
                     device=v.device)
    _check(lib.sage_transpose_v(_ref(s), _ptr(v), _ptr(vt), _stream(v.device)), "sage_transpose_v")
    return vt


def sage_attn_fwd_codes(shape: SageShape, q_codes, q_scale, k_codes, k_scale, v_prepared, v_scale, o, *,
                        is_causal: bool = False, sm_scale: Optional[float] = None, pv_dtype: str = "fp8"):
    """The fused attention kernel alone, from the outputs of sage_quant_qk and
    sage_quant_v (FP8) or sage_transpose_v (FP16). Writes into ``o``."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(shape.head_dim)
    if pv_dtype not in PV_DTYPES:
        raise ValueError(f"pv_dtype must be one of {sorted(PV_DTYPES)}, got {pv_dtype!r}")
    fp8 = PV_DTYPES[pv_dtype] == 1
    in_dtype = {v: k for k, v in DTYPES.items()}.get(shape.dtype)
    if in_dtype is None:
        raise ValueError(f"shape.dtype must be one of {sorted(DTYPES.values())}, got {shape.dtype}")
    gran = {v: k for k, v in QK_GRANS.items()}.get(shape.qk_gran)
    if gran is None:
        raise ValueError(f"shape.qk_gran must be one of {sorted(QK_GRANS.values())}, got {shape.qk_gran}")
    bq, bk, _ = sage_block_sizes(shape.head_dim, gran)
    B, Hq, Hkv, Nq, Nk, d = shape.batch, shape.heads_q, shape.heads_kv, shape.seq_q, shape.seq_k, shape.head_dim
    if not isinstance(o, torch.Tensor) or not o.is_cuda:
        raise ValueError("o must be a GPU tensor")
    dev = o.device
    _expect(o, "o", in_dtype, B * Hq * Nq * d, dev)
    _expect(q_codes, "q_codes", torch.int8, B * Hq * Nq * d, dev)
    _expect(q_scale, "q_scale", torch.float32, B * Hq * -(-Nq // bq), dev)
    _expect(k_codes, "k_codes", torch.int8, B * Hkv * Nk * d, dev)
    _expect(k_scale, "k_scale", torch.float32, B * Hkv * -(-Nk // bk), dev)
    _expect(v_prepared, "v_prepared", torch.uint8 if fp8 else in_dtype, B * Hkv * d * sage_v_codes_stride(Nk), dev)
    if fp8:
        _expect(v_scale, "v_scale", torch.float32, B * Hkv * d, dev)
    _check(lib.sage_attn_fwd_codes(_ref(shape), _ptr(q_codes), _ptr(q_scale), _ptr(k_codes), _ptr(k_scale),
                                   _ptr(v_prepared), _ptr(v_scale), _ptr(o), int(bool(is_causal)),
                                   float(sm_scale), PV_DTYPES[pv_dtype], _stream(o.device)),
           "sage_attn_fwd_codes")
    return o


def sage_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, is_causal: bool = False,
                  sm_scale: Optional[float] = None, pv_dtype: str = "fp8", tensor_layout: str = "HND",
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  qk_gran: str = "per_block") -> torch.Tensor:
    _check_inputs(q, k, v)
    s = shape_of(q, k, tensor_layout, qk_gran)
    if tuple(v.shape) != tuple(k.shape) or v.dtype != q.dtype or k.dtype != q.dtype:
        raise ValueError("v must have k's shape and all inputs one dtype")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(s.head_dim)
    dev = q.device
    o = _out_like(q, out)
    ws = _workspace_for(workspace, sage_workspace_bytes(s, pv_dtype), dev)
    _check(lib.sage_attn_fwd(_ref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(o), int(bool(is_causal)),
                             float(sm_scale), PV_DTYPES[pv_dtype], _ptr(ws), ws.numel(), _stream(dev)),
           "sage_attn_fwd")
    return o


def sage_attn_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, *,
                          is_causal: bool = False, sm_scale: Optional[float] = None, pv_dtype: str = "fp8",
                          tensor_layout: str = "HND", qk_gran: str = "per_block") -> torch.Tensor:
    """sage_attn_fwd with the library's own fixed workspace (no allocation by
    the call; the caller passes ``out``). Shapes whose workspace exceeds
    NOALLOC_MAX_WORKSPACE_BYTES raise SageError(SAGE_ERR_WORKSPACE)."""
    if out is None:
        raise ValueError("sage_attn_fwd_noalloc needs the caller's output tensor")
    _check_inputs(q, k, v)
    s = shape_of(q, k, tensor_layout, qk_gran)
    if tuple(v.shape) != tuple(k.shape) or v.dtype != q.dtype or k.dtype != q.dtype:
        raise ValueError("v must have k's shape and all inputs one dtype")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(s.head_dim)
    o = _out_like(q, out)
    _check(lib.sage_attn_fwd_noalloc(_ref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(o), int(bool(is_causal)),
                                     float(sm_scale), PV_DTYPES[pv_dtype], _stream(q.device)),
           "sage_attn_fwd_noalloc")
    return o


def varlen_shape_of(q: torch.Tensor, k: torch.Tensor, cu_seqlens_q: torch.Tensor, max_seqlen_q: int,
                    max_seqlen_k: int, qk_gran: str = "per_block") -> SageVarlenShape:
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("packed q, k, v must be 3-D: [total, heads, head_dim]")
    if q.dtype not in DTYPES:
        raise TypeError(f"q/k/v must be float16 or bfloat16, got {q.dtype}")
    if cu_seqlens_q.dim() != 1 or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens must be 1-D with B + 1 entries")
    if k.dtype != q.dtype or k.shape[2] != q.shape[2]:
        raise ValueError(f"packed q {tuple(q.shape)} and k {tuple(k.shape)} differ in dtype or head_dim")
    return SageVarlenShape(cu_seqlens_q.numel() - 1, q.shape[1], k.shape[1], q.shape[2], q.shape[0], k.shape[0],
                           int(max_seqlen_q), int(max_seqlen_k), DTYPES[q.dtype], QK_GRANS[qk_gran])


def sage_varlen_workspace_bytes(shape: SageVarlenShape, pv_dtype: str = "fp8") -> int:
    return int(lib.sage_varlen_workspace_bytes(_ref(shape), PV_DTYPES[pv_dtype]))


def sage_attn_fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                         cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int, *,
                         is_causal: bool = False, sm_scale: Optional[float] = None, pv_dtype: str = "fp8",
                         qk_gran: str = "per_block", out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Packed variable-length batch: q [total_q, Hq, d], k/v [total_k, Hkv, d],
    cu_seqlens int32 device tensors of B + 1 offsets. Returns o like q."""
    _check_inputs(q, k, v, cu_seqlens_q, cu_seqlens_k)
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if cu_seqlens_k.numel() != cu_seqlens_q.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    if tuple(v.shape) != tuple(k.shape) or v.dtype != q.dtype or k.dtype != q.dtype:
        raise ValueError("v must have k's shape and all inputs one dtype")
    s = varlen_shape_of(q, k, cu_seqlens_q, max_seqlen_q, max_seqlen_k, qk_gran)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(s.head_dim)
    dev = q.device
    o = _out_like(q, out)
    ws = _workspace_for(workspace, sage_varlen_workspace_bytes(s, pv_dtype), dev)
    _check(lib.sage_attn_fwd_varlen(_ref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                    _ptr(o), int(bool(is_causal)), float(sm_scale), PV_DTYPES[pv_dtype], _ptr(ws),
                                    ws.numel(), _stream(dev)), "sage_attn_fwd_varlen")
    return o


def varlen_v_codes_stride(total_k: int, batch: int) -> int:
    """Columns of the packed V operand rows: every sequence's keys rounded up to 128."""
    return max(128, -(-(total_k + 127 * batch) // 128) * 128)


def sage_quant_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                      cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int, *, pv_dtype: str = "fp8",
                      qk_gran: str = "per_block") -> dict:
    """The quantisation stages of a packed batch, per sequence (see sage.h):
    q_codes [Hq,total_q,d], q_scale [B,Hq,nbq], k_codes [Hkv,total_k,d],
    k_scale [B,Hkv,nbk], k_mean [B,Hkv,d], v_codes (FP8) or v_t (FP16)
    [Hkv,d,n_pad] and v_scale [B,Hkv,d] (FP8)."""
    _check_inputs(q, k, v, cu_seqlens_q, cu_seqlens_k)
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if cu_seqlens_k.numel() != cu_seqlens_q.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    if tuple(v.shape) != tuple(k.shape) or v.dtype != q.dtype or k.dtype != q.dtype:
        raise ValueError("v must have k's shape and all inputs one dtype")
    s = varlen_shape_of(q, k, cu_seqlens_q, max_seqlen_q, max_seqlen_k, qk_gran)
    blk_q, blk_k, _ = sage_block_sizes(s.head_dim, qk_gran)
    B, dev, d = s.batch, q.device, s.head_dim
    nbq = max(1, -(-int(max_seqlen_q) // blk_q))
    nbk = max(1, -(-int(max_seqlen_k) // blk_k))
    npad = varlen_v_codes_stride(s.total_k, B)
    out = {"q_codes": torch.zeros((s.heads_q, s.total_q, d), dtype=torch.int8, device=dev),
           "q_scale": torch.zeros((B, s.heads_q, nbq), dtype=torch.float32, device=dev),
           "k_codes": torch.zeros((s.heads_kv, s.total_k, d), dtype=torch.int8, device=dev),
           "k_scale": torch.zeros((B, s.heads_kv, nbk), dtype=torch.float32, device=dev),
           "k_mean": torch.zeros((B, s.heads_kv, d), dtype=torch.float32, device=dev)}
    if PV_DTYPES[pv_dtype] == 1:
        out["v_codes"] = torch.zeros((s.heads_kv, d, npad), dtype=torch.uint8, device=dev)
        out["v_scale"] = torch.zeros((B, s.heads_kv, d), dtype=torch.float32, device=dev)
        vp, vs = out["v_codes"], out["v_scale"]
    else:
        out["v_t"] = torch.zeros((s.heads_kv, d, npad), dtype=q.dtype, device=dev)
        vp, vs = out["v_t"], None
    ws = _workspace_for(None, int(lib.sage_quant_varlen_workspace_bytes(_ref(s))), dev)
    _check(lib.sage_quant_varlen(_ref(s), PV_DTYPES[pv_dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q),
                                 _ptr(cu_seqlens_k), _ptr(out["q_codes"]), _ptr(out["q_scale"]),
                                 _ptr(out["k_codes"]), _ptr(out["k_scale"]), _ptr(out["k_mean"]), _ptr(vp),
                                 _ptr(vs), _ptr(ws), ws.numel(), _stream(dev)), "sage_quant_varlen")
    return out


# ------------------------------------------------------------------ FP4 microscaling variant
def sage_fp4_workspace_bytes(shape: SageShape) -> int:
    return int(lib.sage_fp4_workspace_bytes(_ref(shape)))


def fp4_buffers(shape: SageShape, device) -> dict:
    """Empty MXFP4 buffers of ``shape`` (layouts of sage.h): codes two per byte,
    E8M0 scale bytes; V transposed and padded to sage_v_codes_stride(Nk) keys,
    its scales per 128-key tile."""
    B, Hq, Hkv, Nq, Nk, d = shape.batch, shape.heads_q, shape.heads_kv, shape.seq_q, shape.seq_k, shape.head_dim
    npad = sage_v_codes_stride(Nk)
    u8 = dict(dtype=torch.uint8, device=device)
    nks = B * Hkv * Nk * (d // 32)
    # (the attention kernel reads the K scales in whole 4-byte words: keep the
    #  storage readable up to the next multiple of 4 bytes)
    k_scale = torch.empty(nks + (-nks) % 4, **u8)[:nks].view(B, Hkv, Nk, d // 32)
    return dict(q_codes=torch.empty((B, Hq, Nq, d // 2), **u8), q_scale=torch.empty((B, Hq, Nq, d // 32), **u8),
                k_codes=torch.empty((B, Hkv, Nk, d // 2), **u8), k_scale=k_scale,
                k_mean=torch.empty((B, Hkv, d), dtype=torch.float32, device=device),
                v_codes=torch.empty((B, Hkv, d, npad // 2), **u8),
                v_scale=torch.empty((B, Hkv, npad // 128, d, 4), **u8))


def sage_quant_fp4(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, tensor_layout: str = "HND",
                   sm_scale: Optional[float] = None) -> dict:
    """MXFP4 quantisation of Q (times sm_scale * log2 e), smoothed K and V;
    returns fp4_buffers' dict."""
    _check_inputs(q, k, v)
    s = shape_of(q, k, tensor_layout)
    if tuple(v.shape) != tuple(k.shape) or v.dtype != q.dtype:
        raise ValueError("v must have k's shape and all inputs one dtype")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(s.head_dim)
    dev = q.device
    out = fp4_buffers(s, dev)
    ws = _workspace(int(lib.sage_quant_fp4_workspace_bytes(_ref(s))), dev)
    _check(lib.sage_quant_fp4(_ref(s), _ptr(q), _ptr(k), _ptr(v), float(sm_scale), _ptr(out["q_codes"]),
                              _ptr(out["q_scale"]),
                              _ptr(out["k_codes"]), _ptr(out["k_scale"]), _ptr(out["k_mean"]), _ptr(out["v_codes"]),
                              _ptr(out["v_scale"]), _ptr(ws), ws.numel(), _stream(dev)), "sage_quant_fp4")
    return out


def sage_attn_fwd_fp4_codes(shape: SageShape, codes: dict, o: torch.Tensor, *, is_causal: bool = False) -> torch.Tensor:
    """The FP4 attention kernel alone, from sage_quant_fp4's buffers (the
    softmax temperature is already in the Q codes). Writes into ``o``."""
    in_dtype = {v: k for k, v in DTYPES.items()}.get(shape.dtype)
    if in_dtype is None:
        raise ValueError(f"shape.dtype must be one of {sorted(DTYPES.values())}, got {shape.dtype}")
    if not isinstance(o, torch.Tensor) or not o.is_cuda:
        raise ValueError("o must be a GPU tensor")
    dev = o.device
    B, Hq, Hkv, Nq, Nk, d = shape.batch, shape.heads_q, shape.heads_kv, shape.seq_q, shape.seq_k, shape.head_dim
    npad = sage_v_codes_stride(Nk)
    sizes = dict(q_codes=B * Hq * Nq * d // 2, q_scale=B * Hq * Nq * d // 32, k_codes=B * Hkv * Nk * d // 2,
                 k_scale=B * Hkv * Nk * d // 32, v_codes=B * Hkv * d * npad // 2, v_scale=B * Hkv * d * npad // 32)
    _expect(o, "o", in_dtype, B * Hq * Nq * d, dev)
    for name, n in sizes.items():
        _expect(codes.get(name), name, torch.uint8, n, dev)
    ks = codes["k_scale"]
    if ks.untyped_storage().nbytes() - ks.storage_offset() < sizes["k_scale"] + (-sizes["k_scale"]) % 4:
        raise ValueError("k_scale is read in whole 4-byte words: its storage needs 2 more bytes (see fp4_buffers)")
    _check(lib.sage_attn_fwd_fp4_codes(_ref(shape), _ptr(codes["q_codes"]), _ptr(codes["q_scale"]),
                                       _ptr(codes["k_codes"]), _ptr(codes["k_scale"]), _ptr(codes["v_codes"]),
                                       _ptr(codes["v_scale"]), _ptr(o), int(bool(is_causal)), _stream(dev)),
           "sage_attn_fwd_fp4_codes")
    return o


def sage_attn_fwd_fp4(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, is_causal: bool = False,
                      sm_scale: Optional[float] = None, tensor_layout: str = "HND",
                      out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The whole FP4 microscaling forward (quantisation and attention)."""
    _check_inputs(q, k, v)
    s = shape_of(q, k, tensor_layout)
    if tuple(v.shape) != tuple(k.shape) or v.dtype != q.dtype:
        raise ValueError("v must have k's shape and all inputs one dtype")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(s.head_dim)
    dev = q.device
    o = _out_like(q, out)
    ws = _workspace_for(workspace, sage_fp4_workspace_bytes(s), dev)
    _check(lib.sage_attn_fwd_fp4(_ref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(o), int(bool(is_causal)),
                                 float(sm_scale), _ptr(ws), ws.numel(), _stream(dev)), "sage_attn_fwd_fp4")
    return o


def _check_varlen_inputs(q, k, v, cu_seqlens_q, cu_seqlens_k):
    _check_inputs(q, k, v, cu_seqlens_q, cu_seqlens_k)
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if cu_seqlens_k.numel() != cu_seqlens_q.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    if tuple(v.shape) != tuple(k.shape) or v.dtype != q.dtype or k.dtype != q.dtype:
        raise ValueError("v must have k's shape and all inputs one dtype")


def sage_fp4_varlen_workspace_bytes(shape: SageVarlenShape) -> int:
    return int(lib.sage_fp4_varlen_workspace_bytes(_ref(shape)))


def sage_attn_fwd_fp4_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                             cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int, *,
                             is_causal: bool = False, sm_scale: Optional[float] = None,
                             out: Optional[torch.Tensor] = None,
                             workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The FP4 microscaling forward over a packed batch: q [total_q, Hq, d],
    k/v [total_k, Hkv, d], int32 cu_seqlens of B + 1 offsets. Returns o like q."""
    _check_varlen_inputs(q, k, v, cu_seqlens_q, cu_seqlens_k)
    s = varlen_shape_of(q, k, cu_seqlens_q, max_seqlen_q, max_seqlen_k)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(s.head_dim)
    dev = q.device
    o = _out_like(q, out)
    ws = _workspace_for(workspace, sage_fp4_varlen_workspace_bytes(s), dev)
    _check(lib.sage_attn_fwd_fp4_varlen(_ref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q),
                                        _ptr(cu_seqlens_k), _ptr(o), int(bool(is_causal)), float(sm_scale),
                                        _ptr(ws), ws.numel(), _stream(dev)), "sage_attn_fwd_fp4_varlen")
    return o


def sage_quant_fp4_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                          cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int, *,
                          sm_scale: Optional[float] = None) -> dict:
    """The MXFP4 stages of a packed batch, per sequence (see sage.h):
    q_codes [Hq,total_q,d/2], q_scale [Hq,total_q,d/32], k_codes and k_scale
    likewise over Hkv and total_k, k_mean [B,Hkv,d], v_codes [Hkv,d,n_pad/2]
    and v_scale [Hkv,n_pad/128,d,4] (n_pad = varlen_v_codes_stride)."""
    _check_varlen_inputs(q, k, v, cu_seqlens_q, cu_seqlens_k)
    s = varlen_shape_of(q, k, cu_seqlens_q, max_seqlen_q, max_seqlen_k)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(s.head_dim)
    B, dev, d = s.batch, q.device, s.head_dim
    npad = varlen_v_codes_stride(s.total_k, B)
    u8 = dict(dtype=torch.uint8, device=dev)
    out = {"q_codes": torch.zeros((s.heads_q, s.total_q, d // 2), **u8),
           "q_scale": torch.zeros((s.heads_q, s.total_q, d // 32), **u8),
           "k_codes": torch.zeros((s.heads_kv, s.total_k, d // 2), **u8),
           "k_scale": torch.zeros((s.heads_kv, s.total_k, d // 32), **u8),
           "k_mean": torch.zeros((B, s.heads_kv, d), dtype=torch.float32, device=dev),
           "v_codes": torch.zeros((s.heads_kv, d, npad // 2), **u8),
           "v_scale": torch.zeros((s.heads_kv, npad // 128, d, 4), **u8)}
    ws = _workspace_for(None, int(lib.sage_quant_fp4_varlen_workspace_bytes(_ref(s))), dev)
    _check(lib.sage_quant_fp4_varlen(_ref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                     float(sm_scale), _ptr(out["q_codes"]), _ptr(out["q_scale"]),
                                     _ptr(out["k_codes"]), _ptr(out["k_scale"]), _ptr(out["k_mean"]),
                                     _ptr(out["v_codes"]), _ptr(out["v_scale"]), _ptr(ws), ws.numel(),
                                     _stream(dev)), "sage_quant_fp4_varlen")
    return out


def sage_debug_qk_i32(q_codes: torch.Tensor, k_codes: torch.Tensor) -> torch.Tensor:
    """INT32 S for canonical-order codes [B,Hq,Nq,d] x [B,Hkv,Nk,d] -> [B,Hq,Nq,Nk]."""
    _check_inputs(q_codes, k_codes)
    if q_codes.dtype != torch.int8 or k_codes.dtype != torch.int8:
        raise TypeError("codes must be int8")
    if q_codes.dim() != 4 or k_codes.dim() != 4:
        raise ValueError("codes must be 4-D [B, H, N, d]")
    B, Hq, Nq, d = q_codes.shape
    _, Hkv, Nk, _ = k_codes.shape
    if k_codes.shape[0] != B or k_codes.shape[3] != d:
        raise ValueError("q_codes and k_codes differ in batch or head_dim")
    s = make_shape(B, Hq, Hkv, Nq, Nk, d)
    out = torch.empty((B, Hq, Nq, Nk), dtype=torch.int32, device=q_codes.device)
    _check(lib.sage_debug_qk_i32(_ref(s), _ptr(q_codes), _ptr(k_codes), _ptr(out), _stream(q_codes.device)),
           "sage_debug_qk_i32")
    return out


def sageattn(q, k, v, tensor_layout: str = "HND", is_causal: bool = False, sm_scale: Optional[float] = None,
             pv_dtype: str = "fp8", qk_quant_gran: str = "per_block", **kwargs):
    """Quantised attention with the scaled-dot-product-attention call shape.

    SDPA arguments this method does not implement are rejected rather than
    silently ignored (a plain monkey-patch of SDPA breaks many models when
    arguments are dropped -- heatdrop.ai review, "Caveats").
    """
    for name in ("attn_mask", "dropout_p", "enable_gqa", "scale"):
        if name in kwargs:
            val = kwargs.pop(name)
            if name == "scale":
                sm_scale = val if val is not None else sm_scale
            elif name == "dropout_p" and val:
                raise NotImplementedError("dropout is not supported")
            elif name == "attn_mask" and val is not None:
                raise NotImplementedError("explicit attention masks are not supported")
    if kwargs:
        raise TypeError(f"unexpected arguments: {sorted(kwargs)}")
    if qk_quant_gran not in QK_GRANS:
        raise ValueError(f"qk_quant_gran must be one of {sorted(QK_GRANS)}, got {qk_quant_gran!r}")
    if pv_dtype == "fp4":
        if qk_quant_gran != "per_block":
            raise ValueError("the FP4 variant has fixed MX blocks; qk_quant_gran must be per_block")
        return sage_attn_fwd_fp4(q.contiguous(), k.contiguous(), v.contiguous(), is_causal=is_causal,
                                 sm_scale=sm_scale, tensor_layout=tensor_layout)
    return sage_attn_fwd(q.contiguous(), k.contiguous(), v.contiguous(), is_causal=is_causal,
                         sm_scale=sm_scale, pv_dtype=pv_dtype, tensor_layout=tensor_layout,
                         qk_gran=qk_quant_gran)


def sageattn_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                    is_causal: bool = False, sm_scale: Optional[float] = None, pv_dtype: str = "fp8",
                    qk_quant_gran: str = "per_block"):
    """Quantised attention over a packed variable-length batch (the
    flash-attention varlen convention: tokens of all sequences concatenated,
    cu_seqlens offsets, maximum lengths)."""
    if qk_quant_gran not in QK_GRANS:
        raise ValueError(f"qk_quant_gran must be one of {sorted(QK_GRANS)}, got {qk_quant_gran!r}")
    if pv_dtype == "fp4":
        if qk_quant_gran != "per_block":
            raise ValueError("the FP4 variant has fixed MX blocks; qk_quant_gran must be per_block")
        return sage_attn_fwd_fp4_varlen(q.contiguous(), k.contiguous(), v.contiguous(), cu_seqlens_q.contiguous(),
                                        cu_seqlens_k.contiguous(), max_seqlen_q, max_seqlen_k,
                                        is_causal=is_causal, sm_scale=sm_scale)
    return sage_attn_fwd_varlen(q.contiguous(), k.contiguous(), v.contiguous(), cu_seqlens_q.contiguous(),
                                cu_seqlens_k.contiguous(), max_seqlen_q, max_seqlen_k, is_causal=is_causal,
                                sm_scale=sm_scale, pv_dtype=pv_dtype, qk_gran=qk_quant_gran)


__all__ = ["sageattn", "sageattn_varlen", "sage_attn_fwd_varlen", "sage_varlen_workspace_bytes",
           "SageVarlenShape", "varlen_shape_of", "sage_attn_fwd", "sage_attn_fwd_codes", "sage_quant_qk", "sage_quant_v",
           "sage_transpose_v", "sage_debug_qk_i32", "sage_quant_fp4", "sage_attn_fwd_fp4",
           "sage_attn_fwd_fp4_codes", "sage_fp4_workspace_bytes", "fp4_buffers", "sage_attn_fwd_fp4_varlen",
           "sage_quant_fp4_varlen", "sage_fp4_varlen_workspace_bytes", "varlen_v_codes_stride",
           "sage_block_sizes", "sage_v_codes_stride", "sage_workspace_bytes", "make_shape", "shape_of",
           "SageError", "SageShape", "QK_GRANS", "lib", "LIB_PATH"]
