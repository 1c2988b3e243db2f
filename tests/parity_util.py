"""Parity helpers for the GPU tests: oracle-side setup of a workload and the
decision-boundary classification of code mismatches.

Code parity rule (the stated bar: codes bit-exact except values within 1e-6
relative of a decision boundary, whose count is reported and must stay below
1e-5 of all code fields).  A mismatched field counts as a boundary case when
  radius code : |r - T_j| <= 1e-6 T_j for the threshold nearest to r;
  angle code  : theta is within 1e-6 rad of a cell edge;
  QJL bit     : |(S_h eps~)_j| <= 1e-6 ||S_h,j|| ||eps~||;
  norm (fp16) : ||eps~|| is within 1e-6 ||eps~|| of an fp16 rounding midpoint.
Sign bits and the norm of a token whose polar codes already differ are
*consequential* (they follow from a different residual), not independent.
"""

from __future__ import annotations

import math

import numpy as np

from oracle import calibrate, codebook, encode, layout
from oracle.encode import Params

REL = 1e-6


def oracle_tables(K, cfg, reorder=False):
    """Per-kv-head (levels32, thresholds32) and perm from the oracle, K [n_seq, n_kv, T, d]."""
    n_seq, n_kv, T, d = K.shape
    c, t = codebook.lloyd_max_beta(d, cfg.b_main)
    tables, perms, sums = [], [], []
    for h in range(n_kv):
        ss = calibrate.channel_sumsq(K[:, h])
        sums.append(ss)
        tables.append(codebook.scaled_table(c, t, calibrate.head_scale(ss, n_seq * T), d))
        perms.append(calibrate.reorder_perm(ss) if reorder else np.arange(d))
    return tables, np.stack(perms), np.stack(sums)


def codebook_array(tables):
    return np.stack([codebook.pack_table(lv, th) for lv, th in tables]).astype(np.float32)


def _fp16_midpoint_distance(v):
    v = np.asarray(v, dtype=np.float64)
    h = v.astype(np.float16)
    up = np.nextafter(h, np.float16(np.inf))
    dn = np.nextafter(h, np.float16(-np.inf))
    hf, uf, df = h.astype(np.float64), up.astype(np.float64), dn.astype(np.float64)
    m1 = 0.5 * (hf + uf)
    m2 = 0.5 * (hf + df)
    return np.minimum(np.abs(v - m1), np.abs(v - m2))


def classify(of: encode.Fields, got: dict, thresholds32, S, p: Params):
    """Compare GPU fields (dict from layout.unpack_stream) with oracle fields."""
    th = np.asarray(thresholds32, dtype=np.float32).astype(np.float64)
    rc_m = got["rc"] != of.rc
    ac_m = got["ac"] != of.ac
    res = {"fields": of.rc.size + of.ac.size, "mismatch": 0, "boundary": 0, "consequential": 0,
           "unexplained": 0}
    # radius
    if rc_m.any():
        r = of.r[rc_m]
        dist = np.min(np.abs(r[:, None] - th[None, :]) / th[None, :], axis=1)
        bnd = dist <= REL
        res["boundary"] += int(bnd.sum())
        res["unexplained"] += int((~bnd).sum())
    # angle: edges at -pi + k 2 pi / A
    if ac_m.any():
        A = 1 << p.b_angle
        delta = 2 * math.pi / A
        x = (of.theta[ac_m] + math.pi) / delta
        dist = np.abs(x - np.round(x)) * delta
        bnd = dist <= REL
        res["boundary"] += int(bnd.sum())
        res["unexplained"] += int((~bnd).sum())
    res["mismatch"] += int(rc_m.sum() + ac_m.sum())
    if p.qjl_m:
        polar_bad = (rc_m | ac_m).any(axis=1)
        bits_m = got["bits"] != of.bits
        nu_m = got["nu"].view(np.uint16) != of.nu.view(np.uint16)
        res["fields"] += of.bits.size + of.nu.size
        res["mismatch"] += int(bits_m.sum() + nu_m.sum())
        cons = int(bits_m[polar_bad].sum() + nu_m[polar_bad].sum())
        res["consequential"] += cons
        ok = ~polar_bad
        bm = bits_m & ok[:, None]
        if bm.any():
            Sd = np.asarray(S, dtype=np.float32).astype(np.float64)
            srow = np.linalg.norm(Sd, axis=1)
            tok, j = np.nonzero(bm)
            scale = srow[j] * of.eps_norm[tok]
            bnd = np.abs(of.u[tok, j]) <= REL * scale
            res["boundary"] += int(bnd.sum())
            res["unexplained"] += int((~bnd).sum())
        nm = nu_m & ok
        if nm.any():
            dist = _fp16_midpoint_distance(of.eps_norm[nm])
            bnd = dist <= REL * of.eps_norm[nm]
            res["boundary"] += int(bnd.sum())
            res["unexplained"] += int((~bnd).sum())
    return res


def merge_counts(acc, r):
    for k, v in r.items():
        acc[k] = acc.get(k, 0) + v
    return acc


def assert_code_parity(counts):
    assert counts["unexplained"] == 0, counts
    # below 1e-5 of all code fields (for small cases: none at all)
    assert counts["mismatch"] < max(1e-5 * counts["fields"], 1.0), counts
