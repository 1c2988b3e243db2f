"""PGKQ key encoding: steps (1)-(4) of the PGKQ pipeline on the EdgeLLM-Nano
paper page, per key, in float64.

Steps, in the page's order:
  (1) randomized Hadamard transform of the key (``rht.forward``);
  (2) adjacent HT-domain components form pairs; each pair becomes a radius
      r_i and an angle theta_i;
  (3) the radius is quantized with the b_main-bit scalar codebook and the angle
      on a b_angle-bit uniform grid over [-pi, pi];
  (4) optionally (QJL) the residual is projected onto m = head_dim random
      directions and only the signs are kept, plus one FP16 residual norm.

Readings used here (the page leaves these steps open):
* pairs are (2i, 2i+1): x = k~[2i], y = k~[2i+1], r = hypot(x, y),
  theta = atan2(y, x);
* radius code = number of thresholds T_j strictly below r (nearest level, a
  radius equal to a threshold takes the lower code); T_j are the fp32 values of
  the per-head table;
* the angle grid is mid-rise: A = 2^b_angle equal cells of width 2 pi / A,
  code = floor((theta + pi) / (2 pi / A)) mod A, reconstruction at the cell
  centre -pi + (a + 1/2) 2 pi / A;
* the residual lives in the HT domain: eps~ = k~ - k~hat with
  k~hat = level[rc] (cos thetahat[ac], sin thetahat[ac]) per pair.  This is
  the page's eps = K - Khat seen through the orthonormal transform, and the
  projection S_h applied to eps~ has the same Gaussian law as one applied to eps;
* S_h is an m x d matrix of i.i.d. N(0, 1) entries, one per kv-head, given in
  fp32; bit_j = [ (S_h eps~)_j >= 0 ] (sign(0) = +1);
* the stored norm nu is ||eps~||_2 rounded to fp16 (nearest, ties to even),
  with values beyond the fp16 range saturated to 65504.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from . import rht

FP16_MAX = 65504.0


@dataclass(frozen=True)
class Params:
    head_dim: int
    b_main: int
    b_angle: int
    qjl_m: int
    hadamard: bool = True

    @property
    def n_pairs(self) -> int:
        return self.head_dim // 2

    @property
    def n_levels(self) -> int:
        return 1 << self.b_main

    @property
    def n_angles(self) -> int:
        return 1 << self.b_angle


def angle_centers(b_angle: int) -> np.ndarray:
    A = 1 << b_angle
    delta = 2.0 * math.pi / A
    return -math.pi + (np.arange(A) + 0.5) * delta


def angle_code(theta, b_angle: int) -> np.ndarray:
    A = 1 << b_angle
    delta = 2.0 * math.pi / A
    return np.floor((np.asarray(theta, dtype=np.float64) + math.pi) / delta).astype(np.int64) % A


def radius_code(r, thresholds32) -> np.ndarray:
    th = np.asarray(thresholds32, dtype=np.float32).astype(np.float64)
    r = np.asarray(r, dtype=np.float64)
    return np.sum(th < r[..., None], axis=-1).astype(np.int64)


def to_fp16_saturating(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        h = x.astype(np.float16)
    return np.where(np.isinf(h) & np.isfinite(x), np.float16(FP16_MAX), h).astype(np.float16)


@dataclass
class Fields:
    """Unpacked codes of N keys plus the values the decisions were taken on."""

    rc: np.ndarray        # [N, n] radius codes
    ac: np.ndarray        # [N, n] angle codes
    bits: np.ndarray      # [N, m] bool QJL sign bits (m = 0 without QJL)
    nu: np.ndarray        # [N] fp16 residual norm (zeros without QJL)
    # diagnostics
    kt: np.ndarray        # [N, d] HT-domain key
    r: np.ndarray         # [N, n]
    theta: np.ndarray     # [N, n]
    eps: np.ndarray       # [N, d] HT-domain residual (zeros without QJL)
    eps_norm: np.ndarray  # [N] float64 ||eps~||
    u: np.ndarray         # [N, m] projections S_h eps~


def reconstruct_pairs(rc, ac, levels32, b_angle: int):
    """k~hat per pair: (level[rc] cos thetahat[ac], level[rc] sin thetahat[ac])."""
    lv = np.asarray(levels32, dtype=np.float32).astype(np.float64)
    c = angle_centers(b_angle)
    rad = lv[np.asarray(rc)]
    return rad * np.cos(c[np.asarray(ac)]), rad * np.sin(c[np.asarray(ac)])


def encode_keys(K, signs, perm, levels32, thresholds32, S, params: Params) -> Fields:
    """Encode keys [N, d] of one kv-head (all keys share signs, perm, table and S)."""
    K = np.asarray(K)
    N, d = K.shape
    if d != params.head_dim:
        raise ValueError("head_dim mismatch")
    kt = rht.forward(K.astype(np.float64), signs, perm, params.hadamard)
    x = kt[:, 0::2]
    y = kt[:, 1::2]
    r = np.hypot(x, y)
    theta = np.arctan2(y, x)
    rc = radius_code(r, thresholds32)
    ac = angle_code(theta, params.b_angle)
    m = params.qjl_m
    if m > 0:
        hx, hy = reconstruct_pairs(rc, ac, levels32, params.b_angle)
        eps = np.empty_like(kt)
        eps[:, 0::2] = x - hx
        eps[:, 1::2] = y - hy
        eps_norm = np.sqrt(np.sum(eps * eps, axis=1))
        nu = to_fp16_saturating(eps_norm)
        Sd = np.asarray(S, dtype=np.float32).astype(np.float64)
        if Sd.shape != (m, d):
            raise ValueError("S must be [m, d]")
        u = eps @ Sd.T
        bits = u >= 0.0
    else:
        eps = np.zeros_like(kt)
        eps_norm = np.zeros(N)
        nu = np.zeros(N, dtype=np.float16)
        u = np.zeros((N, 0))
        bits = np.zeros((N, 0), dtype=bool)
    return Fields(rc=rc, ac=ac, bits=bits, nu=nu, kt=kt, r=r, theta=theta, eps=eps,
                  eps_norm=eps_norm, u=u)


def encode_cache(K, signs, perm, tables, S, params: Params):
    """Encode a cache K [n_seq, n_kv, T, d]; per-kv-head inputs indexed by h.

    ``tables`` is a list over kv-heads of (levels32, thresholds32); ``perm`` is
    None or [n_kv, d].  Returns a nested list fields[b][h].
    """
    K = np.asarray(K)
    n_seq, n_kv = K.shape[:2]
    out = []
    for b in range(n_seq):
        row = []
        for h in range(n_kv):
            lv, th = tables[h]
            row.append(encode_keys(K[b, h], signs[h], None if perm is None else perm[h], lv, th,
                                   None if S is None else S[h], params))
        out.append(row)
    return out
