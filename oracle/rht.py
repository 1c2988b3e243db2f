"""Randomized Hadamard transform (step (1) of the PGKQ pipeline on the
EdgeLLM-Nano paper page: precondition the keys with a randomized Hadamard
transform).

Reading used here: the printed "K~ = RHK" does not type-check for K in
R^{N x d}; per key k in R^d the transform is

    k~ = H (signs * k[perm]) / sqrt(d)

with ``signs`` a Rademacher vector (the random +-1 R), ``perm`` the optional
channel order of step (0) (identity when step (0) is off), and H the d x d
Sylvester Hadamard matrix in natural order, H[i, j] = (-1)^popcount(i & j).
The 1/sqrt(d) factor makes the transform orthonormal.  The oracle multiplies by
the dense matrix on purpose (no fast transform).

With ``hadamard=False`` (the "without Hadamard" ablation of the same page) the
transform is the identity after the optional reorder: k~ = k[perm].
"""

from __future__ import annotations

import math

import numpy as np


def sylvester(d: int) -> np.ndarray:
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    H = np.ones((1, 1), dtype=np.float64)
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    return H


def forward(x, signs, perm=None, hadamard: bool = True) -> np.ndarray:
    """k~ for every row of x ([..., d]); float64."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if perm is not None:
        x = x[..., np.asarray(perm, dtype=np.int64)]
    if not hadamard:
        return x.copy()
    xs = x * np.asarray(signs, dtype=np.float64)
    H = sylvester(d)
    return (xs @ H.T) / math.sqrt(d)


def inverse(kt, signs, perm=None, hadamard: bool = True) -> np.ndarray:
    """Original-domain vector from k~ (H H^T = d I)."""
    kt = np.asarray(kt, dtype=np.float64)
    d = kt.shape[-1]
    if hadamard:
        H = sylvester(d)
        xs = (kt @ H) / math.sqrt(d)
        xp = xs * np.asarray(signs, dtype=np.float64)
    else:
        xp = kt.copy()
    if perm is None:
        return xp
    out = np.empty_like(xp)
    out[..., np.asarray(perm, dtype=np.int64)] = xp
    return out
