"""Seeded synthetic Q/K/V workloads for the quantized-attention hot path.

This module only *draws* inputs. It holds none of the method's arithmetic
(no smoothing, no quantization, no softmax), so both the CPU oracle and the
HIP path can take their inputs from it without sharing any computation.

The five workloads stand in for the models the SageAttention pages measure on
(LLM prefill, image/video diffusion transformers; "SageAttention: Accurate 8-Bit
Attention for Plug-and-play Inference Acceleration", abstract): no model weights
or datasets are used. Shapes follow the pages' sequence-length regimes
(cnnetsun.cn guide, "sequence length" tips: 1K-4K, 8K-16K, 32K+).

Recipe (the same for every workload):
  1. ``torch.Generator`` on the CPU, ``manual_seed(seed)`` (seed 0 by default).
  2. Draw Q [B,Hq,N,d], K [B,Hkv,N,d], V [B,Hkv,N,d] as fp32 standard normals in
     that order, then the K channel offset o [B,Hkv,1,d], then (only when
     ``outliers > 0``) ``randperm(d)[:outliers]`` as the outlier channel set.
  3. Scale each tensor by sqrt(variance): "N(0, x)" is read as variance x.
  4. Outlier channels (one set, shared by all heads, by Q and by K) are
     multiplied by ``outlier_scale`` in Q and K.
  5. K += o (the offset is shared by all tokens of a head: a per-channel bias,
     which is what channel smoothing removes).
  6. Cast to the storage dtype (round-to-nearest-even) and, for the NHD layout,
     permute to [B,N,H,d] and make contiguous.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str            # "fp16" | "bf16"
    layout: str           # "HND" | "NHD"
    causal: bool
    pv: str               # "fp8" | "fp16"
    q_var: float = 1.0
    k_var: float = 1.0
    v_var: float = 1.0
    k_off_var: float = 4.0
    outliers: int = 0
    outlier_scale: float = 10.0
    seed: int = 0

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def attention_ops(self) -> float:
        """Counted attention operations 4*B*Hq*N^2*d, halved for causal."""
        ops = 4.0 * self.B * self.Hq * self.N * self.N * self.d
        return ops / 2 if self.causal else ops


# The five workloads. Names say what they are.
TINY = Workload("tiny_b1_h2_n256_d64_fp16", B=1, Hq=2, Hkv=2, N=256, d=64,
                dtype="fp16", layout="HND", causal=False, pv="fp16",
                k_off_var=4.0)
MID_OUTLIER = Workload("mid_b4_h32_n4096_d128_bf16_outlier", B=4, Hq=32, Hkv=32,
                       N=4096, d=128, dtype="bf16", layout="HND", causal=False,
                       pv="fp8", k_off_var=4.0, outliers=4)
GQA_CAUSAL = Workload("gqa_causal_b2_hq32_hkv8_n8192_d128_bf16_nhd", B=2, Hq=32,
                      Hkv=8, N=8192, d=128, dtype="bf16", layout="NHD",
                      causal=True, pv="fp8", k_off_var=2.0)
LONG_D64 = Workload("long_b1_h24_n16384_d64_fp16", B=1, Hq=24, Hkv=24, N=16384,
                    d=64, dtype="fp16", layout="HND", causal=False, pv="fp16",
                    q_var=1.5, k_var=1.5, v_var=1.0, k_off_var=6.0)
PEAK = Workload("peak_b1_h32_n32768_d128_fp16", B=1, Hq=32, Hkv=32, N=32768,
                d=128, dtype="fp16", layout="HND", causal=False, pv="fp8",
                k_off_var=4.0)

ALL = {w.name: w for w in (TINY, MID_OUTLIER, GQA_CAUSAL, LONG_D64, PEAK)}

TORCH_DTYPE = {"fp16": torch.float16, "bf16": torch.bfloat16}


def generate(w: Workload, device: Optional[str] = None):
    """Return (q, k, v) torch tensors in the workload's dtype and layout.

    Generation always happens on the CPU with a seeded generator, so every
    consumer sees bit-identical inputs; ``device`` only moves the result.
    """
    g = torch.Generator().manual_seed(w.seed)
    q = torch.randn((w.B, w.Hq, w.N, w.d), generator=g, dtype=torch.float32)
    k = torch.randn((w.B, w.Hkv, w.N, w.d), generator=g, dtype=torch.float32)
    v = torch.randn((w.B, w.Hkv, w.N, w.d), generator=g, dtype=torch.float32)
    off = torch.randn((w.B, w.Hkv, 1, w.d), generator=g, dtype=torch.float32)
    idx = torch.randperm(w.d, generator=g)[: w.outliers] if w.outliers else None
    q.mul_(math.sqrt(w.q_var))
    k.mul_(math.sqrt(w.k_var))
    v.mul_(math.sqrt(w.v_var))
    off.mul_(math.sqrt(w.k_off_var))
    if idx is not None:
        q[..., idx] *= w.outlier_scale
        k[..., idx] *= w.outlier_scale
    k.add_(off)
    dt = TORCH_DTYPE[w.dtype]
    q, k, v = q.to(dt), k.to(dt), v.to(dt)
    if w.layout == "NHD":
        q, k, v = (t.transpose(1, 2).contiguous() for t in (q, k, v))
    if device is not None:
        q, k, v = q.to(device), k.to(device), v.to(device)
    return q, k, v


def to_hnd(t: torch.Tensor, layout: str) -> torch.Tensor:
    """View a [B,N,H,d] tensor as [B,H,N,d] (no copy for HND inputs)."""
    return t.transpose(1, 2) if layout == "NHD" else t


def sample_rows(n: int, count: int, block: int, seed: int = 1):
    """Sorted query-row sample: ``count`` seeded random rows plus edge rows
    (0, 1, block-1, block, n-1) so the first/last tiles and a tile seam are
    always covered."""
    g = torch.Generator().manual_seed(seed)
    pick = torch.randperm(n, generator=g)[: min(count, n)].tolist()
    edges = [r for r in (0, 1, block - 1, block, n - 2, n - 1) if 0 <= r < n]
    return sorted(set(pick) | set(edges))


# ------------------------------------------------------------------ packed variable-length batches
@dataclasses.dataclass(frozen=True)
class VarlenWorkload:
    """B sequences packed along the token axis ([total, H, d] tensors).

    Recipe: the same generator, seed and variances as ``Workload``; Q, K, V are
    drawn as [total, H, d] standard normals in that order, then one K channel
    offset per (sequence, kv head) [B, Hkv, d], added to that sequence's keys
    (so each sequence has its own channel bias for its own smoothing)."""
    name: str
    lens_q: tuple
    lens_k: tuple
    Hq: int
    Hkv: int
    d: int
    dtype: str
    causal: bool
    pv: str
    k_off_var: float = 4.0
    seed: int = 0

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def B(self) -> int:
        return len(self.lens_q)

    def with_(self, **kw) -> "VarlenWorkload":
        return dataclasses.replace(self, **kw)

    def cu_seqlens(self):
        cq, ck = [0], [0]
        for a, b in zip(self.lens_q, self.lens_k):
            cq.append(cq[-1] + a)
            ck.append(ck[-1] + b)
        return cq, ck

    def attention_ops(self) -> float:
        """Counted operations 4*Hq*d per visible (query, key) pair; causal
        masking is top-left inside each sequence."""
        pairs = 0
        for nq, nk in zip(self.lens_q, self.lens_k):
            if self.causal:
                m = min(nq, nk)                    # rows i < nk see i + 1 keys, later rows all nk
                pairs += m * (m + 1) // 2 + (nq - m) * nk
            else:
                pairs += nq * nk
        return 4.0 * self.Hq * self.d * pairs


def seq_lengths(count: int, lo: int, hi: int, seed: int = 0):
    """``count`` seeded sequence lengths, log-uniform in [lo, hi] (a serving
    mix: many short requests and a few long ones)."""
    g = torch.Generator().manual_seed(seed)
    u = torch.rand(count, generator=g, dtype=torch.float64)
    return tuple(int(round(math.exp(math.log(lo) + float(x) * (math.log(hi) - math.log(lo))))) for x in u)


def generate_varlen(w: VarlenWorkload, device: Optional[str] = None):
    """Return (q, k, v, cu_seqlens_q, cu_seqlens_k): packed tensors in the
    workload's dtype and int32 offsets, generated on the CPU and moved to
    ``device``."""
    g = torch.Generator().manual_seed(w.seed)
    tq, tk = sum(w.lens_q), sum(w.lens_k)
    q = torch.randn((tq, w.Hq, w.d), generator=g, dtype=torch.float32)
    k = torch.randn((tk, w.Hkv, w.d), generator=g, dtype=torch.float32)
    v = torch.randn((tk, w.Hkv, w.d), generator=g, dtype=torch.float32)
    off = torch.randn((w.B, w.Hkv, w.d), generator=g, dtype=torch.float32) * math.sqrt(w.k_off_var)
    cq, ck = w.cu_seqlens()
    for b in range(w.B):
        k[ck[b]:ck[b + 1]] += off[b]
    dt = TORCH_DTYPE[w.dtype]
    q, k, v = q.to(dt), k.to(dt), v.to(dt)
    cu_q = torch.tensor(cq, dtype=torch.int32)
    cu_k = torch.tensor(ck, dtype=torch.int32)
    if device is not None:
        q, k, v, cu_q, cu_k = (t.to(device) for t in (q, k, v, cu_q, cu_k))
    return q, k, v, cu_q, cu_k


# An LLM-prefill serving mix: 16 requests, 256 to 16384 tokens, GQA, causal.
VARLEN_PREFILL = VarlenWorkload("varlen_prefill_16seq_hq32_hkv8_d128_bf16", lens_q=seq_lengths(16, 256, 16384),
                                lens_k=seq_lengths(16, 256, 16384), Hq=32, Hkv=8, d=128, dtype="bf16",
                                causal=True, pv="fp8")
