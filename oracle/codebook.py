"""Lloyd-Max radius codebook for the Beta prior.

Source: EdgeLLM-Nano paper page, the paragraph following "PGKQ pipeline": the
radii are quantized with the codebook obtained by Lloyd-Max for the Beta prior,
not refit on data.  The Lloyd-Max iteration (nearest-level cells, then centroid
update) is the one the ManthanQuant page describes.

Reading used here.  For a pair (x, y) of an isotropic key in d dimensions after
the randomized Hadamard transform, u = r^2 / ||k||^2 follows Beta(1, n - 1) with
n = d / 2 pairs.  The codebook is designed for rho = (r / ||k||) * sqrt(n), which
has E[rho^2] = 1:

    density  f(rho) = (2 rho (n - 1) / n) (1 - rho^2 / n)^(n - 2),  0 <= rho <= sqrt(n)
    CDF      F(rho) = 1 - (1 - rho^2 / n)^(n - 1)
    partial first moment
             int_a^b rho f(rho) drho
               = sqrt(n) (n - 1) B(3/2, n - 1) [I_{b^2/n}(3/2, n-1) - I_{a^2/n}(3/2, n-1)]

The per-head table in absolute radius units multiplies rho by
sigma_h = s_h / sqrt(n), where s_h = sqrt(mean ||k||^2) over the keys being
encoded (the pages' "calibration keys"); see ``calibrate.head_scale``.
"""

from __future__ import annotations

import math

import numpy as np
from scipy.special import beta as beta_fn
from scipy.special import betainc


def rho_cdf(rho, n: int):
    rho = np.asarray(rho, dtype=np.float64)
    u = np.clip(rho * rho / n, 0.0, 1.0)
    with np.errstate(divide="ignore"):
        return -np.expm1((n - 1) * np.log1p(-u))


def rho_quantile(p, n: int):
    p = np.asarray(p, dtype=np.float64)
    with np.errstate(divide="ignore"):
        u = -np.expm1(np.log1p(-p) / (n - 1))
    return np.sqrt(n * u)


def rho_pdf(rho, n: int):
    rho = np.asarray(rho, dtype=np.float64)
    u = np.clip(rho * rho / n, 0.0, 1.0)
    return (2.0 * rho * (n - 1) / n) * (1.0 - u) ** (n - 2)


def partial_mass(a, b, n: int):
    """P(a < rho <= b)."""
    return rho_cdf(b, n) - rho_cdf(a, n)


def partial_moment(a, b, n: int):
    """E[rho * 1{a < rho <= b}] via the regularized incomplete beta function."""
    ua = np.clip(np.asarray(a, dtype=np.float64) ** 2 / n, 0.0, 1.0)
    ub = np.clip(np.asarray(b, dtype=np.float64) ** 2 / n, 0.0, 1.0)
    c = math.sqrt(n) * (n - 1) * beta_fn(1.5, n - 1)
    return c * (betainc(1.5, n - 1, ub) - betainc(1.5, n - 1, ua))


def distortion(levels, thresholds, n: int) -> float:
    """E[(rho - Q(rho))^2] for the quantizer with the given cells and levels."""
    levels = np.asarray(levels, dtype=np.float64)
    edges = np.concatenate([[0.0], np.asarray(thresholds, dtype=np.float64), [math.sqrt(n)]])
    P = partial_mass(edges[:-1], edges[1:], n)
    M = partial_moment(edges[:-1], edges[1:], n)
    return float(1.0 - 2.0 * np.dot(levels, M) + np.dot(levels * levels, P))


def lloyd_max_beta(head_dim: int, b_main: int, tol: float = 1e-13, max_iter: int = 200000,
                   init=None, history: bool = False):
    """Lloyd-Max quantizer of rho for the Beta(1, n - 1) radius prior.

    Returns (levels, thresholds) in rho units, float64, levels ascending, with
    thresholds[j] = (levels[j] + levels[j+1]) / 2.  The iteration starts from the
    quantile midpoints F^-1((j + 1/2) / L) unless ``init`` is given, and stops
    when no level moves by more than ``tol``.  With ``history`` the distortion
    after every iteration is returned as a third value.
    """
    n = head_dim // 2
    L = 1 << b_main
    if n < 2 or L < 2:
        raise ValueError("need head_dim >= 4 and b_main >= 1")
    top = math.sqrt(n)
    if init is None:
        c = rho_quantile((np.arange(L) + 0.5) / L, n)
    else:
        c = np.array(init, dtype=np.float64)
    hist = []
    for _ in range(max_iter):
        t = 0.5 * (c[:-1] + c[1:])
        edges = np.concatenate([[0.0], t, [top]])
        P = partial_mass(edges[:-1], edges[1:], n)
        M = partial_moment(edges[:-1], edges[1:], n)
        c_new = M / P
        if history:
            hist.append(distortion(c_new, 0.5 * (c_new[:-1] + c_new[1:]), n))
        moved = float(np.max(np.abs(c_new - c)))
        c = c_new
        if moved < tol:
            break
    else:  # pragma: no cover - convergence failure is a bug
        raise RuntimeError("Lloyd-Max did not converge")
    t = 0.5 * (c[:-1] + c[1:])
    if history:
        return c, t, hist
    return c, t


def lloyd_max_empirical(samples, b_main: int, max_iter: int = 100000, history: bool = False):
    """Lloyd-Max quantizer fitted to samples of rho (the empirical refit of the
    PGKQ-KV paragraphs, PGKQ-KV': the same two conditions as for the prior,
    with the sample distribution in place of the Beta density).

    Start: the sample quantiles at (j + 1/2) / L (sorted sample at index
    floor((j + 1/2) N / L)).  Step: thresholds at the midpoints of adjacent
    levels; a sample goes to the cell #{j : t_j < rho} (the decision rule of
    the encoder); each level becomes the mean of its cell (an empty cell keeps
    its level).  Stops when no sample changes cell, i.e. at a fixed point
    where every level is exactly its cell's mean.  Returns (levels, thresholds)
    float64; with ``history`` also the mean squared error after every step.
    """
    x = np.sort(np.asarray(samples, dtype=np.float64).ravel())
    N = x.size
    L = 1 << b_main
    if N < L or L < 2:
        raise ValueError("need at least 2^b_main samples and b_main >= 1")
    c = x[((np.arange(L) + 0.5) * N / L).astype(np.int64)].copy()
    cells = None
    hist = []
    for _ in range(max_iter):
        t = 0.5 * (c[:-1] + c[1:])
        new_cells = np.sum(t[None, :] < x[:, None], axis=1)
        if cells is not None and np.array_equal(new_cells, cells):
            break
        cells = new_cells
        for j in range(L):
            members = x[cells == j]
            if members.size:
                c[j] = members.mean()
        if history:
            hist.append(float(np.mean((x - c[cells]) ** 2)))
    else:  # pragma: no cover - the assignment sequence is finite
        raise RuntimeError("empirical Lloyd-Max did not converge")
    t = 0.5 * (c[:-1] + c[1:])
    if history:
        return c, t, hist
    return c, t


def scaled_table(levels, thresholds, head_scale: float, head_dim: int):
    """Per-head table in radius units, rounded to fp32: (levels32, thresholds32).

    sigma_h = head_scale / sqrt(head_dim / 2); both arrays are rho * sigma_h
    computed in float64 and rounded once to fp32.  These fp32 values are the
    ``codebook`` input of the encoder and the decoder, and the oracle uses the
    same fp32 values.
    """
    sigma = float(head_scale) / math.sqrt(head_dim // 2)
    lv = (np.asarray(levels, dtype=np.float64) * sigma).astype(np.float32)
    th = (np.asarray(thresholds, dtype=np.float64) * sigma).astype(np.float32)
    return lv, th


def pack_table(levels32, thresholds32) -> np.ndarray:
    """The per-head codebook record: L levels then L - 1 thresholds then +inf (2L floats)."""
    lv = np.asarray(levels32, dtype=np.float32)
    th = np.asarray(thresholds32, dtype=np.float32)
    return np.concatenate([lv, th, np.array([np.inf], dtype=np.float32)])


def unpack_table(rec, b_main: int):
    L = 1 << b_main
    rec = np.asarray(rec, dtype=np.float32)
    return rec[..., :L], rec[..., L:2 * L - 1]
