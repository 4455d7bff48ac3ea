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
