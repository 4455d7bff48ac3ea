"""Shared helpers for the GPU parity tests (compare the HIP path with the oracle)."""
from __future__ import annotations

import sys

import numpy as np

# Tolerances of the float output (the method's stated bar):
#   against the oracle:            cosine >= 0.9999 and sum|o-r| / sum|r| <= 1e-3
#   against fp64 exact attention:  cosine >= 0.999
COS_ORACLE = 0.9999
RL1_ORACLE = 1e-3
COS_EXACT = 0.999


def cos(a, b) -> float:
    a = np.ravel(np.asarray(a, np.float64))
    b = np.ravel(np.asarray(b, np.float64))
    return float(a @ b / np.sqrt((a @ a) * (b @ b)))


def rel_l1(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.abs(a - b).sum() / np.abs(b).sum())


def worst_head_cos(a, b) -> float:
    return min(cos(a[i, j], b[i, j]) for i in range(a.shape[0]) for j in range(a.shape[1]))


def say(*args):
    """Progress line, flushed (names the case before a GPU step)."""
    print(*args, flush=True)
    sys.stdout.flush()


# ------------------------------------------------------------------ full-size parity on sampled rows
PAIR = 256    # queries per attention work-group (two 128-query groups)
GROUP = 128


def rows_per_head(n: int, heads: int, seed: int = 7):
    """Query rows to check for each of ``heads`` (batch, head) pairs: one seeded
    row from every 256-query work-group, taken from its first and its second
    128-query group on alternate work-groups (the alternation flips between
    heads), plus the edge rows 0, 1, 127, 128, n-2 and n-1. Output row i depends
    only on the quantisation block of query i and on all of K and V, so rows can
    be checked one by one."""
    g = np.random.default_rng(seed)
    edges = {r for r in (0, 1, GROUP - 1, GROUP, n - 2, n - 1) if 0 <= r < n}
    out = []
    for h in range(heads):
        rows = set(edges)
        for i, p0 in enumerate(range(0, n, PAIR)):
            lo = p0 + ((i + h) % 2) * GROUP
            if lo >= n:
                lo = p0
            hi = min(lo + GROUP, n)
            rows.add(int(g.integers(lo, hi)))
        out.append(np.array(sorted(rows)))
    return out


def oracle_rows_per_head(sage_ref, qn, kn, vn, parts, *, dtype, causal, sm_scale, pv, rows, blk_q, blk_k,
                         rejected=()):
    """The oracle's output rows ``rows[b*Hq + h]`` of every (batch, query head),
    from the quantisation stages in ``parts`` (canonical HND arrays)."""
    B, Hq = qn.shape[:2]
    G = Hq // kn.shape[1]
    out = []
    for b in range(B):
        for h in range(Hq):
            g = h // G
            sub = {"q8": parts["q8"][b:b + 1, h:h + 1], "q_scale": parts["q_scale"][b:b + 1, h:h + 1],
                   "k8": parts["k8"][b:b + 1, g:g + 1], "k_scale": parts["k_scale"][b:b + 1, g:g + 1]}
            if pv == "fp8":
                sub["v8"] = parts["v8"][b:b + 1, g:g + 1]
                sub["v_scale"] = parts["v_scale"][b:b + 1, g:g + 1]
            r = sage_ref.sage_attention(qn[b:b + 1, h:h + 1], kn[b:b + 1, g:g + 1], vn[b:b + 1, g:g + 1],
                                        dtype=dtype, is_causal=causal, sm_scale=sm_scale, pv=pv,
                                        rows=rows[b * Hq + h], parts=sub, blk_q=blk_q, blk_k=blk_k,
                                        rejected=rejected)
            out.append(r[0, 0])
    return out


def exact_rows_per_head(exact, qn, kn, vn, *, causal, sm_scale, rows):
    B, Hq = qn.shape[:2]
    G = Hq // kn.shape[1]
    out = []
    for b in range(B):
        for h in range(Hq):
            g = h // G
            e = exact.exact_attention(qn[b:b + 1, h:h + 1], kn[b:b + 1, g:g + 1], vn[b:b + 1, g:g + 1],
                                      is_causal=causal, sm_scale=sm_scale, rows=rows[b * Hq + h])
            out.append(e[0, 0])
    return out


def check_heads(got, ref, *, cos_min=COS_ORACLE, rl1_max=RL1_ORACLE):
    """Per-(batch, head) cosine and relative L1 against the oracle; returns the
    worst values (asserting each head meets the bound)."""
    worst_c, worst_r = 1.0, 0.0
    for i, (a, b) in enumerate(zip(got, ref)):
        c, r = cos(a, b), rel_l1(a, b)
        assert c >= cos_min and r <= rl1_max, f"head {i}: cos={c:.7f} rel_l1={r:.2e}"
        worst_c, worst_r = min(worst_c, c), max(worst_r, r)
    return worst_c, worst_r
