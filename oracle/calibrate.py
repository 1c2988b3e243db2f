"""Calibration statistics: step (0) channel reorder and the per-head radius scale.

Source: EdgeLLM-Nano paper page, "PGKQ pipeline", step (0): optionally reorder
channels by decreasing l2 norm and group them so that one high-norm and one
low-norm channel share a group.  The pipeline starts from "calibration keys K";
this oracle takes the calibration keys to be the keys being encoded, per
(layer, kv-head), over every sequence and token.

Readings used here:
* a group is a polar pair (2i, 2i+1);
* channels are sorted by descending l2 norm with a stable sort (ties keep the
  lower channel index first), giving ranks pi_0 .. pi_{d-1};
* the reordered channel list is [pi_0, pi_{d-1}, pi_1, pi_{d-2}, ...], i.e.
  perm[2i] = pi_i and perm[2i+1] = pi_{d-1-i}, and k_reordered[c] = k[perm[c]];
* the per-head radius scale is s_h = sqrt(mean over keys of ||k||^2).
"""

from __future__ import annotations

import math

import numpy as np


def channel_sumsq(keys) -> np.ndarray:
    """Per-channel sum of squares over all leading axes; keys [..., d] -> [d] float64."""
    k = np.asarray(keys, dtype=np.float64)
    k = k.reshape(-1, k.shape[-1])
    return np.einsum("tc,tc->c", k, k)


def reorder_perm(sumsq) -> np.ndarray:
    sumsq = np.asarray(sumsq, dtype=np.float64)
    d = sumsq.shape[-1]
    # descending l2 norm is descending sum of squares; sorting the sums avoids
    # ties that a square root could create between distinct sums
    ranks = np.argsort(-sumsq, kind="stable")
    perm = np.empty(d, dtype=np.int64)
    for i in range(d // 2):
        perm[2 * i] = ranks[i]
        perm[2 * i + 1] = ranks[d - 1 - i]
    return perm


def head_scale(sumsq, n_keys: int) -> float:
    return math.sqrt(float(np.sum(np.asarray(sumsq, dtype=np.float64))) / n_keys)
