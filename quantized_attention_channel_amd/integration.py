"""Framework integration of the quantised attention forward.

* ``attn_fwd_op``: the whole forward as a ``torch.library`` custom operator
  (``torch.ops.sage_mi355x.attn_fwd``) with a fake (shape-only) implementation,
  so graph capture such as ``torch.compile`` traces through it as one opaque
  node (thu-ml/SageAttention repo card, "How it works", and the heatdrop.ai
  review, "Key highlights": torch.compile support).
* ``attn_fwd_varlen_op``: the same for packed variable-length batches
  (``torch.ops.sage_mi355x.attn_fwd_varlen``; heatdrop.ai review, "Key
  highlights": variable sequence lengths within a batch), for serving code
  that keeps the tokens of all requests in one [total, heads, head_dim] tensor.
* ``patch_sdpa``: a guarded drop-in for ``torch.nn.functional.
  scaled_dot_product_attention``. The heatdrop.ai review ("Caveats") warns that
  replacing that function wholesale breaks many models, because some of their
  calls pass masks or other arguments the method does not implement. The
  guard routes only the calls the method supports (``sdpa_supported`` names
  the reason for any other call); the rest raise by default, or, when the
  caller asks for ``passthrough=True``, go to the original function unchanged.
  Routed calls always run the HIP kernels of this library.
"""
from __future__ import annotations

import math
from typing import Optional

import torch

from . import DTYPES, sageattn, sageattn_varlen

_LIB = "sage_mi355x"


@torch.library.custom_op(f"{_LIB}::attn_fwd", mutates_args=())
def attn_fwd_op(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, is_causal: bool, sm_scale: float,
                pv_dtype: str, tensor_layout: str, qk_gran: str) -> torch.Tensor:
    """Quantised attention forward (a fresh output tensor shaped like q); pv_dtype
    "fp8" or "fp16", or "fp4" for the FP4 microscaling variant."""
    return sageattn(q, k, v, tensor_layout=tensor_layout, is_causal=is_causal, sm_scale=sm_scale,
                    pv_dtype=pv_dtype, qk_quant_gran=qk_gran)


@attn_fwd_op.register_fake
def _attn_fwd_fake(q, k, v, is_causal, sm_scale, pv_dtype, tensor_layout, qk_gran):
    return torch.empty_like(q, memory_format=torch.contiguous_format)


@torch.library.custom_op(f"{_LIB}::attn_fwd_varlen", mutates_args=())
def attn_fwd_varlen_op(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                       cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int, is_causal: bool,
                       sm_scale: float, pv_dtype: str, qk_gran: str) -> torch.Tensor:
    """Quantised attention over a packed batch: q [total_q, Hq, d], k and v
    [total_k, Hkv, d], int32 cu_seqlens of B + 1 offsets; a fresh output shaped
    like q. pv_dtype "fp8", "fp16" or "fp4"."""
    return sageattn_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, is_causal=is_causal,
                           sm_scale=sm_scale, pv_dtype=pv_dtype, qk_quant_gran=qk_gran)


@attn_fwd_varlen_op.register_fake
def _attn_fwd_varlen_fake(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, is_causal, sm_scale,
                          pv_dtype, qk_gran):
    return torch.empty_like(q, memory_format=torch.contiguous_format)


def sdpa_supported(query, key, value, attn_mask=None, dropout_p=0.0, is_causal=False, scale=None,
                   enable_gqa=False) -> Optional[str]:
    """None if the method can take this scaled-dot-product-attention call,
    else the reason it cannot (structural reasons first, the device last)."""
    if attn_mask is not None:
        return "explicit attention masks are not supported"
    if dropout_p:
        return "dropout is not supported"
    if not all(isinstance(t, torch.Tensor) for t in (query, key, value)):
        return "query, key and value must be tensors"
    if query.dim() != 4 or key.dim() != 4 or value.dim() != 4:
        return "only 4-D [batch, heads, tokens, head_dim] inputs are supported"
    if query.dtype not in DTYPES or key.dtype != query.dtype or value.dtype != query.dtype:
        return "inputs must all be float16 or all be bfloat16"
    if query.shape[-1] not in (64, 128) or key.shape[-1] != query.shape[-1]:
        return "head_dim must be 64 or 128"
    if tuple(value.shape) != tuple(key.shape):
        return "value must have key's shape"
    if query.shape[0] != key.shape[0]:
        return "query and key batch sizes differ"
    hq, hkv = query.shape[1], key.shape[1]
    if hq != hkv and not (enable_gqa and hq % hkv == 0):
        return "different query and key head counts need enable_gqa and a multiple"
    if is_causal and query.shape[2] != key.shape[2]:
        return "causal masking with different query and key lengths is not supported"
    if scale is not None and not (math.isfinite(scale) and scale > 0):
        return "scale must be finite and positive"
    if torch.is_grad_enabled() and any(t.requires_grad for t in (query, key, value)):
        return "no backward pass: inputs that require grad are not supported"
    if not (query.is_cuda and key.is_cuda and value.is_cuda):
        return "inputs must be GPU tensors"
    return None


class patch_sdpa:
    """Context manager that routes supported ``F.scaled_dot_product_attention``
    calls to the quantised kernels.

    ``passthrough=False`` (default): an unsupported call raises
    ``NotImplementedError`` with the reason. ``passthrough=True``: it runs the
    original function instead. ``routed`` and ``passed`` count the calls.
    """

    def __init__(self, pv_dtype: str = "fp8", qk_quant_gran: str = "per_block", passthrough: bool = False):
        if pv_dtype not in ("fp8", "fp16", "fp4"):
            raise ValueError(f"pv_dtype must be fp8, fp16 or fp4, got {pv_dtype!r}")
        if pv_dtype == "fp4" and qk_quant_gran != "per_block":
            raise ValueError("the FP4 variant has fixed MX blocks; qk_quant_gran must be per_block")
        self.pv_dtype, self.qk_gran, self.passthrough = pv_dtype, qk_quant_gran, passthrough
        self.routed = 0
        self.passed = 0
        self._orig = None

    def _call(self, query, key, value, attn_mask=None, dropout_p=0.0, is_causal=False, scale=None,
              enable_gqa=False):
        reason = sdpa_supported(query, key, value, attn_mask, dropout_p, is_causal, scale, enable_gqa)
        if reason is not None:
            if not self.passthrough:
                raise NotImplementedError(f"scaled_dot_product_attention not routed: {reason}")
            self.passed += 1
            return self._orig(query, key, value, attn_mask=attn_mask, dropout_p=dropout_p, is_causal=is_causal,
                              scale=scale, enable_gqa=enable_gqa)
        self.routed += 1
        sm_scale = scale if scale is not None else 1.0 / math.sqrt(query.shape[-1])
        return attn_fwd_op(query, key, value, bool(is_causal), float(sm_scale), self.pv_dtype, "HND", self.qk_gran)

    def __enter__(self):
        self._orig = torch.nn.functional.scaled_dot_product_attention
        torch.nn.functional.scaled_dot_product_attention = self._call
        return self

    def __exit__(self, *exc):
        torch.nn.functional.scaled_dot_product_attention = self._orig
        return False


__all__ = ["attn_fwd_op", "attn_fwd_varlen_op", "sdpa_supported", "patch_sdpa"]
