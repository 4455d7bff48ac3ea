"""The SageAttention forward method, step by step, on the CPU.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix, and where:
  * K is smoothed along the channel direction before it is quantised to INT8
    (jisaku.com glossary, 概要 and 主な特徴・仕組み; heatdrop.ai review, "The
    interesting bit", calls it outlier smoothing).
  * QK^T runs in INT8, PV in FP8 or FP16 (thu-ml/SageAttention repo card,
    "How it works"; heatdrop.ai review, "What it does").
  * The attention weights P are handled in FP8 (jisaku.com glossary, 概要).
  * PV uses two-level accumulation (repo card, "How it works"; heatdrop.ai,
    "The interesting bit" and "Key highlights").
  * Group-query attention, causal masking and the HND/NHD layouts are part of
    the interface (heatdrop.ai "Key highlights"; cnnetsun.cn guide, basic
    usage and performance-tuning tips).
The shape of the computation (per-channel mean over tokens, per-block INT8 with
INT32 accumulation, online FlashAttention-style softmax, P in FP8 e4m3) is the
plain reading of those passages.

Readings where the pages are silent (each also listed in the design notes):
  [R1] INT8 codes round half to even.
  [R2] scale s = fp32(a/127); codes use x * fp32(127/a) -- one correctly rounded
       multiply, never fused with the smoothing subtraction.
  [R3] codes are symmetric in [-127, 127].
  [R4] an all-zero block gets scale 0 and codes 0.
  [R5] the K mean runs over all Nk tokens of a (batch, kv-head).
  [R6] K channel sums are exact (rounded once to fp64), divided by Nk in
       fp64 and rounded once to fp32.
  [R7] quantisation blocks: BLK_Q = 128 query tokens, BLK_K = 64 key tokens,
       starting at token 0, the last block possibly short; one scale per
       (batch, head, block) over all d channels.
  [R8] only K is smoothed (Q and V are not).
  [R9] V is quantised to e4m3 per channel over all tokens: s_v = fp32(a_v/448),
       codes e4m3(fp32(V * fp32(448/a_v))).
  [R10] sm_scale and log2(e) enter through the dequantisation factor
       c = fp32(s_q * s_k * sm_scale * log2 e); scores live in the log2 domain.
  [R11] causal masking is top-left aligned (key j > query i is masked).
  [R12] P goes to e4m3 as e4m3(fp32(448 * P~)); the factor 448 cancels against
       the row sum (R16), s_v is applied in the epilogue.
  [R13] in FP16-PV mode P is rounded to the input dtype (fp16 or bf16) and
       multiplied with the unquantised V.
  [R14] the online softmax walks KV tiles of BKV keys from key 0 upward; BKV
       is part of the method's definition (P codes depend on the running max).
  [R15] two-level accumulation: level 1 sums the products of a group of keys
       (here one KV tile, R = P . V_tile; the GPU kernel's level 1 is one matrix
       instruction, 64 keys in FP8 mode), level 2 is O = alpha*O + R in a wider
       accumulator. The e4m3 products are exact and their sums fit in fp64, so
       the span of level 1 changes no value here; on the GPU it changes fp32
       rounding only.
  [R16] the row sum l accumulates the P values that enter the PV product (the
       e4m3 values of 448 * P~ in FP8 mode, the fp16/bf16-rounded P~ in FP16
       mode), so the output is normalised by the weights actually applied;
       against fp64 exact attention this is equal to or slightly better than
       summing the unquantised P~.
  [R20] per-thread quantisation (heatdrop.ai review, "The interesting bit",
       names it next to the smoothing, without a definition) is read as the
       finest grouping the GPU kernel's matrix-product lane layout gives at no
       extra cost: every query token has its own scale (BLK_Q = 1) and every
       run of 16 consecutive keys shares one (BLK_K = 16), blocks starting at
       token 0. All the per-block rules above then apply per group.
  [R21] variable-length batches (heatdrop.ai review, "Key highlights": variable
       sequence lengths within a batch) are packed along the token axis with
       cumulative offsets; every sequence is one independent attention by the
       method -- its own K channel mean, blocks from its own first token, its
       own V channel scales, causal masking top-left inside the sequence. A
       sequence with queries but no keys has zero output rows.
  [R22] the FP4 microscaling variant (SageAttention3: heatdrop.ai review, "Key
       highlights"; cnnetsun.cn guide, 序列长度优化技巧 -- named, never defined)
       is read as OCP MXFP4: E2M1 elements with one E8M0 power-of-two scale per
       32 elements along the contraction axis of each product (oracle/mxfp4.py).
       Q and the smoothed K are blocked per token and 32 channels, V per channel
       and 32 keys (from key 0 of the sequence), P~ per query row and 32 keys of
       its KV tile. K smoothing [R5, R6, R8] is kept; there is no V scale in the
       epilogue (the block scales enter the products).
  [R23] the P block scale follows the same rule as every other MX block (shared
       exponent floor(log2 max P~) - 2), and the row sum adds the P values that
       enter the PV product [R16]; the online softmax is unchanged [R14, R15].
  [R24] the softmax temperature and log2(e) scale Q before its quantisation:
       Q' = fp32(Q * c), c = fp32(sm_scale * log2 e), goes to MXFP4, and the
       product gives log2-domain scores directly: S2 = fp32(dequant(Q') .
       dequant(K)^T) (exact here in fp64, rounded once; the matrix cores sum it
       in fp32). In the INT8 method the same factor rides in the dequantisation
       [R10]; here no per-score multiply is left (the MX scales are powers of
       two and cannot carry it).
"""
from __future__ import annotations

import math

import numpy as np
import torch

from .fp8_e4m3 import E4M3_MAX, e4m3_encode, e4m3_decode, e4m3_round
from .mxfp4 import mxfp4_quantize

LOG2E = 1.4426950408889634
INT8_MAX = 127.0

BLK_Q = 128        # [R7]
BLK_K = 64         # [R7]
PER_THREAD_BLK_Q = 1     # [R20]
PER_THREAD_BLK_K = 16    # [R20]
BKV = {64: 128, 128: 128}   # [R14] KV tile per head dim


def as_hnd(x: np.ndarray, layout: str) -> np.ndarray:
    """[B,N,H,d] -> [B,H,N,d] view for NHD inputs (interface layouts: cnnetsun.cn
    guide, performance-tuning tips, HND or NHD)."""
    return np.swapaxes(x, 1, 2) if layout == "NHD" else x


# ---------------------------------------------------------------------------
# Step 1: K channel mean  (glossary 概要: smoothing along the channel direction)
# ---------------------------------------------------------------------------
def _exact_sums(x: np.ndarray) -> np.ndarray:
    """sum over axis 0 of x [N, d] (float64), each column's exact sum rounded
    once to fp64. Where every partial sum is an integer multiple of the
    column's finest unit g (the lowest set significand bit among its nonzero
    values) below g * 2^53, plain fp64 addition is exact in any order; the
    other columns are summed by math.fsum."""
    total = x.sum(axis=0)
    a = np.abs(x)
    m, e = np.frexp(a)                                     # a = m 2^e, m in [0.5, 1)
    sig = (m * 2.0 ** 53).astype(np.int64)                 # exact: m has at most 53 bits
    low = sig & -sig                                       # lowest set bit (0 for zeros)
    unit = np.where(low > 0, np.ldexp(low.astype(np.float64), e - 53), np.inf).min(axis=0)
    for c in np.nonzero(a.sum(axis=0) >= unit * 2.0 ** 53)[0]:
        total[c] = math.fsum(x[:, c])
    return total


def k_channel_mean(k: np.ndarray) -> np.ndarray:
    """mu[b,h,c] = fp32( (sum_t K[b,h,t,c]) / Nk ): the exact sum rounded to
    fp64, an fp64 division, one rounding to fp32 [R5, R6].

    ``k``: float32 array [B,Hkv,Nk,d] holding the fp16/bf16 input values.
    """
    B, H, n, d = k.shape
    x = np.asarray(k, dtype=np.float64)
    total = np.zeros((B, H, d), np.float64)
    for b in range(B):
        for h in range(H):
            total[b, h] = _exact_sums(x[b, h])
    return (total / n).astype(np.float32)


# ---------------------------------------------------------------------------
# Steps 2-3: smoothing and per-block INT8 quantisation
#            (repo card "How it works": INT8 for QK^T; glossary 概要)
# ---------------------------------------------------------------------------
def smooth_k(k: np.ndarray, mu: np.ndarray) -> np.ndarray:
    """Ks = fp32(K - mu), one fp32 subtraction per element."""
    return (np.asarray(k, dtype=np.float32) - mu[:, :, None, :].astype(np.float32)).astype(np.float32)


def quant_int8_blocks(x: np.ndarray, blk: int):
    """Per-block symmetric INT8 [R1-R4, R7].

    ``x``: float32 [B,H,N,d]. Returns (codes int8 [B,H,N,d], scales float32
    [B,H,ceil(N/blk)]). For each (b, h, block): a = max |x| over the block's
    tokens and channels, s = fp32(a/127), code = RNE(fp32(x * fp32(127/a))).
    """
    x = np.asarray(x, dtype=np.float32)
    B, H, N, d = x.shape
    nblk = -(-N // blk)
    pad = nblk * blk - N
    xp = np.concatenate([x, np.zeros((B, H, pad, d), np.float32)], axis=2) if pad else x
    xb = xp.reshape(B, H, nblk, blk, d)
    a = np.abs(xb).max(axis=(3, 4))                                   # exact
    scale = (a / np.float32(INT8_MAX)).astype(np.float32)             # fp32 divide, RN
    with np.errstate(divide="ignore"):
        inv = np.where(a > 0, np.float32(INT8_MAX) / np.where(a > 0, a, 1), 0).astype(np.float32)
    prod = (xb * inv[:, :, :, None, None]).astype(np.float32)         # fp32 multiply, RN
    codes = np.rint(prod)                                             # ties to even [R1]
    if np.abs(codes).max(initial=0) > INT8_MAX:
        raise AssertionError("INT8 code outside [-127, 127]")
    codes = codes.astype(np.int8).reshape(B, H, nblk * blk, d)[:, :, :N]
    return codes, scale


def quant_qk(q: np.ndarray, k: np.ndarray, *, blk_q: int = BLK_Q, blk_k: int = BLK_K, k_mean=None):
    """The whole Q/K quantisation stage on canonical [B,H,N,d] float32 arrays.

    Returns dict(q8, q_scale, k8, k_scale, k_mean). ``k_mean`` may be given to
    quantise K against an externally supplied mean.
    """
    mu = k_channel_mean(k) if k_mean is None else np.asarray(k_mean, np.float32)
    q8, sq = quant_int8_blocks(q, blk_q)
    k8, sk = quant_int8_blocks(smooth_k(k, mu), blk_k)
    return dict(q8=q8, q_scale=sq, k8=k8, k_scale=sk, k_mean=mu)


# ---------------------------------------------------------------------------
# V to FP8 per channel (repo card / heatdrop.ai: FP8 for the PV product) [R9]
# ---------------------------------------------------------------------------
def quant_v_fp8(v: np.ndarray):
    """Returns (codes uint8 [B,H,d,N] -- keys contiguous per channel --,
    scales float32 [B,H,d])."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).max(axis=2)                                         # [B,H,d]
    scale = (a / np.float32(E4M3_MAX)).astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(a > 0, np.float32(E4M3_MAX) / np.where(a > 0, a, 1), 0).astype(np.float32)
    prod = (v * inv[:, :, None, :]).astype(np.float32)
    codes = e4m3_encode(prod)
    return np.ascontiguousarray(np.swapaxes(codes, 2, 3)), scale


# ---------------------------------------------------------------------------
# Step 4: INT32 QK^T
# ---------------------------------------------------------------------------
def qk_int32(q8_rows: np.ndarray, k8: np.ndarray) -> np.ndarray:
    """S_int = q8 . k8^T for one head: [R,d] x [Nk,d] -> int64 [R,Nk].

    Products of int8 codes summed over d <= 256 stay below 2^23 in magnitude,
    so an fp64 matrix product (a library primitive) is exact; the result is
    returned as integers.
    """
    s = np.asarray(q8_rows, np.float64) @ np.asarray(k8, np.float64).T
    return s.astype(np.int64)


def dequant_factor(sq_rows: np.ndarray, sk_keys: np.ndarray, sm_scale: float) -> np.ndarray:
    """c[i,j] = fp32(s_q[blk(i)] * s_k[blk(j)] * sm_scale * log2 e) [R10]."""
    return (sq_rows.astype(np.float64)[:, None] * sk_keys.astype(np.float64)[None, :]
            * (float(sm_scale) * LOG2E)).astype(np.float32)


# ---------------------------------------------------------------------------
# Steps 5-9: tiled online softmax with P quantisation and two-level PV
# ---------------------------------------------------------------------------
def online_softmax_pv(s2: np.ndarray, vals: np.ndarray, *, bkv: int, p_codec, work_dtype,
                      row_sum_unquantised: bool = False):
    """FlashAttention-style online softmax over KV tiles of ``bkv`` keys [R14, R15].

    ``s2``  : [R, Nk] log2-domain scores, -inf where masked.
    ``vals``: [Nk, dv] float64 values entering the PV product (dequantised-code
              domain: V8 codes' values in FP8 mode, V itself in FP16 mode).
    ``p_codec``: maps the fp32 P~ tile to the values that enter the PV product
              (None: identity).
    ``work_dtype``: np.float32 for the method (scores, max, P~ in fp32),
              np.float64 for the unquantised reference recurrence.
    ``row_sum_unquantised``: the rejected reading of [R16] (l adds the fp32
              P~ instead of the values entering PV); only for tests that
              measure how far that reading lands from the chosen one.

    Per tile t, in ascending order:
      m_new = max(m_old, max_j s2);  alpha = exp2(m_old - m_new)  (0 on the first tile)
      P~    = exp2(s2 - m_new)
      P     = codec(P~)                                (the values entering PV)
      l     = alpha * l + sum_j P                      [R16]
      R     = P . vals_tile                            (level 1: fresh per tile)
      O     = alpha * O + R                            (level 2)
    Returns (O [R,dv] float64, l [R] float64) -- not yet normalised.
    """
    R_, nk = s2.shape
    dv = vals.shape[1]
    m = np.full(R_, -np.inf, dtype=work_dtype)
    l = np.zeros(R_, dtype=np.float64)
    o = np.zeros((R_, dv), dtype=np.float64)
    for t0 in range(0, nk, bkv):
        st = s2[:, t0:t0 + bkv].astype(work_dtype)
        m_new = np.maximum(m, st.max(axis=1))
        live = np.isfinite(m_new)                     # rows with at least one visible key so far
        m_safe = np.where(live, m_new, 0).astype(work_dtype)
        with np.errstate(invalid="ignore"):
            alpha = np.where(np.isfinite(m), np.exp2((m - m_safe).astype(work_dtype)), 0.0)
            p = np.exp2((st - m_safe[:, None]).astype(work_dtype)).astype(work_dtype)
        p = np.where(live[:, None], p, 0).astype(work_dtype)
        alpha = np.where(live, alpha, 0.0).astype(np.float64)
        pq = p.astype(np.float64) if p_codec is None else p_codec(p)
        l = alpha * l + (p.astype(np.float64) if row_sum_unquantised else pq).sum(axis=1)   # [R16]
        r = pq @ vals[t0:t0 + bkv]                    # level 1 (exact for e4m3 x e4m3)
        o = alpha[:, None] * o + r                    # level 2
        m = m_new
    return o, l


def _p_codec_fp8(p: np.ndarray) -> np.ndarray:
    """P8 value = e4m3(fp32(448 * P~)) [R12]."""
    return e4m3_round((p.astype(np.float32) * np.float32(E4M3_MAX)).astype(np.float32))


def _round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round to fp16/bf16 (RNE) and return the rounded values as float64."""
    if dtype == "fp16":
        return np.asarray(x).astype(np.float16).astype(np.float64)
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32)))
        return t.to(torch.bfloat16).to(torch.float64).numpy()
    raise ValueError(dtype)


def _p_codec_half(dtype: str):
    def codec(p):
        return _round_to(p.astype(np.float32), dtype)       # [R13]
    return codec


# Readings the method does NOT take, selectable by name so that tests can
# measure how far each one lands from the chosen reading (the parity bounds
# must tell them apart). None of them is the method.
REJECTED_READINGS = (
    "p_unrounded",           # [R12]/[R13] rejected: P enters PV unrounded (FP8 mode: 448 P~ unquantised)
    "row_sum_unquantised",   # [R16] rejected: l adds the fp32 P~ rather than the values entering PV
    "p_half_bf16",           # [R13] rejected for fp16 inputs: P rounded to bf16
    "p_half_fp16",           # [R13] rejected for bf16 inputs: P rounded to fp16
)


def sage_attention(q, k, v, *, dtype: str, is_causal: bool, sm_scale: float, pv: str,
                   layout: str = "HND", blk_q: int = BLK_Q, blk_k: int = BLK_K, bkv=None,
                   rows=None, parts=None, return_fp64: bool = False, rejected: tuple = ()):
    """Quantised attention forward, step by step.

    ``q,k,v``: float32 numpy arrays holding the fp16/bf16 input values in
    ``layout`` ([B,H,N,d] for HND, [B,N,H,d] for NHD). ``rows``: optional
    sorted query rows to compute (output row i depends only on Q's block
    containing i and on all of K and V). ``parts``: optional precomputed
    quantisation outputs (dict from ``quant_qk`` plus ``v8``/``v_scale``).
    Returns [B,Hq,R,d] in HND order, rounded to ``dtype`` (float64 array of the
    rounded values), or the unrounded fp64 result when ``return_fp64``.
    ``rejected``: names from REJECTED_READINGS to compute a rejected reading
    instead of the method (tests only; empty for the method itself).
    """
    unknown = set(rejected) - set(REJECTED_READINGS)
    if unknown:
        raise ValueError(f"unknown readings {sorted(unknown)}")
    q = as_hnd(np.asarray(q, np.float32), layout)
    k = as_hnd(np.asarray(k, np.float32), layout)
    v = as_hnd(np.asarray(v, np.float32), layout)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    bkv = BKV[d] if bkv is None else bkv
    rows = np.arange(Nq) if rows is None else np.asarray(rows)

    if parts is None:
        parts = quant_qk(q, k, blk_q=blk_q, blk_k=blk_k)
        if pv == "fp8":
            parts["v8"], parts["v_scale"] = quant_v_fp8(v)
    q8, sq, k8, sk = parts["q8"], parts["q_scale"], parts["k8"], parts["k_scale"]
    if pv == "fp8":
        vals_all = e4m3_decode(parts["v8"])                 # [B,Hkv,d,Nk]
        codec = _p_codec_fp8
        if "p_unrounded" in rejected:
            codec = lambda p: p.astype(np.float64) * E4M3_MAX          # noqa: E731
    elif pv == "fp16":
        half = dtype
        if "p_half_bf16" in rejected:
            half = "bf16"
        if "p_half_fp16" in rejected:
            half = "fp16"
        codec = _p_codec_half(half)
        if "p_unrounded" in rejected:
            codec = lambda p: p.astype(np.float64)                     # noqa: E731
    else:
        raise ValueError(pv)
    row_sum_unq = "row_sum_unquantised" in rejected

    keys = np.arange(Nk)
    out = np.empty((B, Hq, len(rows), d), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            s_int = qk_int32(q8[b, h, rows], k8[b, g])                          # step 4
            c = dequant_factor(sq[b, h, rows // blk_q], sk[b, g, keys // blk_k], sm_scale)
            s2 = (s_int.astype(np.float32) * c).astype(np.float32)              # step 5
            if is_causal:
                s2 = np.where(keys[None, :] > rows[:, None], np.float32(-np.inf), s2)
            if pv == "fp8":
                vals = np.ascontiguousarray(vals_all[b, g].T)                   # [Nk, d] code values
            else:
                vals = v[b, g].astype(np.float64)
            o, l = online_softmax_pv(s2, vals, bkv=bkv, p_codec=codec, work_dtype=np.float32,
                                     row_sum_unquantised=row_sum_unq)
            if row_sum_unq and pv == "fp8":
                l = l * E4M3_MAX                                                # P8 carries the factor 448
            if pv == "fp8":                                                     # epilogue
                o = o * parts["v_scale"][b, g].astype(np.float64)[None, :]
            out[b, h] = o / l[:, None]
    if return_fp64:
        return out
    return _round_to(out, dtype)


def sage_attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, *, dtype: str, is_causal: bool, sm_scale: float,
                          pv: str, blk_q: int = BLK_Q, blk_k: int = BLK_K, return_fp64: bool = False):
    """Packed variable-length batch [R21].

    ``q``: [total_q, Hq, d], ``k``/``v``: [total_k, Hkv, d] (float32 arrays of
    the input values); ``cu_seqlens_*``: B + 1 non-decreasing offsets. Sequence
    b is q[cu_q[b]:cu_q[b+1]] against k, v[cu_k[b]:cu_k[b+1]], run through
    ``sage_attention`` as a batch of one. Returns [total_q, Hq, d].
    """
    q, k, v = (np.asarray(x, np.float32) for x in (q, k, v))
    cq = [int(x) for x in cu_seqlens_q]
    ck = [int(x) for x in cu_seqlens_k]
    out = np.zeros((q.shape[0], q.shape[1], q.shape[2]), np.float64)
    for b in range(len(cq) - 1):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        if q1 == q0 or k1 == k0:
            continue                                    # no rows, or no keys: zero rows
        o = sage_attention(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1], dtype=dtype, is_causal=is_causal,
                           sm_scale=sm_scale, pv=pv, layout="NHD", blk_q=blk_q, blk_k=blk_k,
                           return_fp64=return_fp64)
        out[q0:q1] = o[0].transpose(1, 0, 2)
    return out


# ---------------------------------------------------------------------------
# FP4 microscaling variant (SageAttention3: heatdrop.ai review, "Key
# highlights"; cnnetsun.cn guide, 序列长度优化技巧) [R22-R24]
# ---------------------------------------------------------------------------
def fp4_score_factor(sm_scale: float) -> np.float32:
    """c = fp32(sm_scale * log2 e), applied to Q before its quantisation [R24].
    sm_scale is taken as fp32 (the type the library's interface carries it in),
    the product in fp64, rounded once to fp32."""
    return np.float32(float(np.float32(sm_scale)) * LOG2E)


def quant_qk_fp4(q: np.ndarray, k: np.ndarray, *, sm_scale: float, k_mean=None):
    """Q' = fp32(Q * c) [R24] and smoothed K to MXFP4 along the head dimension
    [R22]: one E8M0 scale per token and 32 consecutive channels. Returns
    dict(q4, q_exp, qd, k4, k_exp, kd, k_mean): codes [B,H,N,d] (one E2M1 code
    per byte), block exponents [B,H,N,d/32], dequantised values (float64)."""
    mu = k_channel_mean(k) if k_mean is None else np.asarray(k_mean, np.float32)
    qs = (np.asarray(q, np.float32) * fp4_score_factor(sm_scale)).astype(np.float32)
    q4, qe, qd = mxfp4_quantize(qs, axis=3)
    k4, ke, kd = mxfp4_quantize(smooth_k(k, mu), axis=3)
    return dict(q4=q4, q_exp=qe, qd=qd, k4=k4, k_exp=ke, kd=kd, k_mean=mu)


def quant_v_fp4(v: np.ndarray):
    """V to MXFP4 along the tokens [R22]: one E8M0 scale per channel and 32
    consecutive keys from key 0. Returns (codes [B,H,N,d], exponents
    [B,H,ceil(N/32),d], dequantised float64 [B,H,N,d])."""
    return mxfp4_quantize(np.asarray(v, np.float32), axis=2)


def _p_codec_fp4(p: np.ndarray) -> np.ndarray:
    """P~ of one KV tile to MXFP4 along the keys [R23]: per query row, blocks of
    32 consecutive keys of the tile; returns the dequantised values."""
    return mxfp4_quantize(p.astype(np.float32), axis=1)[2]


def sage_attention_fp4(q, k, v, *, dtype: str, is_causal: bool, sm_scale: float, layout: str = "HND",
                       bkv=None, rows=None, parts=None, return_fp64: bool = False):
    """The FP4 microscaling variant of the forward, step by step [R22-R24].

    K is smoothed as in the INT8 method; Q' = fp32(Q * fp32(sm_scale * log2 e))
    and K go to MXFP4 along the head dimension, S2 = fp32(dequant(Q')
    dequant(K)^T) (exact in fp64, rounded once; the matrix cores accumulate it
    in fp32); the online softmax is the method's (KV tiles of BKV keys,
    running max); P~ goes
    to MXFP4 per query row and 32 keys; the row sum adds the dequantised P
    [R16]; PV uses V in MXFP4 per channel and 32 keys, accumulated in two
    levels as before. ``parts``: optional dict from quant_qk_fp4 plus ``vd``.
    Returns [B,Hq,R,d] (HND), rounded to ``dtype`` unless ``return_fp64``.
    """
    q = as_hnd(np.asarray(q, np.float32), layout)
    k = as_hnd(np.asarray(k, np.float32), layout)
    v = as_hnd(np.asarray(v, np.float32), layout)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    bkv = BKV[d] if bkv is None else bkv
    rows = np.arange(Nq) if rows is None else np.asarray(rows)
    if parts is None:
        parts = quant_qk_fp4(q, k, sm_scale=sm_scale)
        parts["vd"] = quant_v_fp4(v)[2]
    keys = np.arange(Nk)
    out = np.empty((B, Hq, len(rows), d), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            s2 = (parts["qd"][b, h, rows] @ parts["kd"][b, g].T).astype(np.float32)   # [R24]
            if is_causal:
                s2 = np.where(keys[None, :] > rows[:, None], np.float32(-np.inf), s2)
            o, l = online_softmax_pv(s2, parts["vd"][b, g], bkv=bkv, p_codec=_p_codec_fp4,
                                     work_dtype=np.float32)
            out[b, h] = o / l[:, None]
    if return_fp64:
        return out
    return _round_to(out, dtype)
