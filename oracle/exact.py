"""fp64 reference attention without any quantisation.

``exact_attention`` is plain softmax attention (the operation SageAttention
replaces: a drop-in for scaled-dot-product attention -- cnnetsun.cn guide,
basic usage; thu-ml/SageAttention repo card, "How to use"), written from its
definition O = softmax(Q K^T * sm_scale) V with row i attending keys j <= i
under the causal flag (top-left aligned, the scaled-dot-product-attention
convention).

``online_softmax_attention`` runs the oracle's own tiled online-softmax
recurrence (``sage_ref.online_softmax_pv``) in fp64 with the identity codec;
the pins compare the two to show that the recurrence reaches the exact result.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).
"""
from __future__ import annotations

import numpy as np

from . import sage_ref


def exact_attention(q, k, v, *, is_causal: bool, sm_scale: float, rows=None):
    """fp64 softmax attention on canonical [B,H,N,d] arrays (GQA by head groups).

    Returns float64 [B,Hq,R,d] for the query rows ``rows`` (all rows if None).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    rows = np.arange(Nq) if rows is None else np.asarray(rows)
    out = np.empty((B, Hq, len(rows), v.shape[3]), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            s = q[b, h, rows] @ k[b, h // G].T * sm_scale
            if is_causal:
                s = np.where(np.arange(Nk)[None, :] > rows[:, None], -np.inf, s)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            out[b, h] = (p @ v[b, h // G]) / p.sum(axis=1, keepdims=True)
    return out


def online_softmax_attention(q, k, v, *, is_causal: bool, sm_scale: float, bkv: int, rows=None):
    """Tiled online softmax in fp64 with no quantisation at all.

    Uses the oracle's recurrence ``sage_ref.online_softmax_pv`` with the
    identity P codec and scores in the log2 domain, then O / l.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    rows = np.arange(Nq) if rows is None else np.asarray(rows)
    out = np.empty((B, Hq, len(rows), v.shape[3]), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            s2 = (q[b, h, rows] @ k[b, h // G].T) * (sm_scale * sage_ref.LOG2E)
            if is_causal:
                s2 = np.where(np.arange(Nk)[None, :] > rows[:, None], -np.inf, s2)
            o, l = sage_ref.online_softmax_pv(s2, v[b, h // G], bkv=bkv,
                                              p_codec=None, work_dtype=np.float64)
            out[b, h] = o / l[:, None]
    return out


def exact_attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, *, is_causal: bool, sm_scale: float):
    """fp64 softmax attention of every sequence of a packed batch ([total, H, d]
    arrays, B + 1 offsets); a sequence without keys has zero rows."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    out = np.zeros((q.shape[0], q.shape[1], v.shape[2]), np.float64)
    cq = [int(x) for x in cu_seqlens_q]
    ck = [int(x) for x in cu_seqlens_k]
    for b in range(len(cq) - 1):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        if q1 == q0 or k1 == k0:
            continue
        o = exact_attention(q[None, q0:q1].transpose(0, 2, 1, 3), k[None, k0:k1].transpose(0, 2, 1, 3),
                            v[None, k0:k1].transpose(0, 2, 1, 3), is_causal=is_causal, sm_scale=sm_scale)
        out[q0:q1] = o[0].transpose(1, 0, 2)
    return out
