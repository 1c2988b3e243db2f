"""Analytic attention logits from PGKQ codes, softmax, and the FP16-V weighted sum.

Source: EdgeLLM-Nano paper page, "PGKQ pipeline" (last sentences: the codes are
never inverted into Khat; logits are computed analytically from Q, rhat,
thetahat and, with QJL, the residual sketch) and the throughput paragraph (the
decode path consists of a Hadamard rotation of Q, polar reconstruction and a
QJL correction inside the model's attention-logit hook).  "Bit budget": V is
not compressed (FP16).

Readings used here:
* the query goes through the same transform as the keys of its kv-head:
  q~ = H (signs * q[perm]) / sqrt(d); then <q~, k~> = <q, k>;
* the logit estimates <q, k>:
      s = sum_i level[rc_i] (q~[2i] cos thetahat[ac_i] + q~[2i+1] sin thetahat[ac_i])
          + kappa * nu * sum_j (S_h q~)_j (2 bit_j - 1),     kappa = sqrt(pi/2) / m.
  The QJL term follows from E[(s.q) sign(s.e)] = sqrt(2/pi) <q, e> / ||e|| for
  s ~ N(0, I) (the QJL estimator; the page does not print it);
* attention weights p = softmax(scale * s) over every cached token (no mask),
  scale = 1/sqrt(d) unless given; out = sum_t p_t V_t with V in fp16 read as is;
* grouped-query attention: query head hq reads kv-head hq // (n_q / n_kv).
"""

from __future__ import annotations

import math

import numpy as np

from . import rht
from .encode import Params, angle_centers, reconstruct_pairs


def kappa(m: int) -> float:
    return math.sqrt(math.pi / 2.0) / m


def query_transform(q, signs, perm, params: Params) -> np.ndarray:
    return rht.forward(np.asarray(q, dtype=np.float64), signs, perm, params.hadamard)


def angle_lut(qt, b_angle: int) -> np.ndarray:
    """LUT[i, a] = q~[2i] cos thetahat_a + q~[2i+1] sin thetahat_a, [n, A]."""
    c = angle_centers(b_angle)
    return qt[0::2, None] * np.cos(c)[None, :] + qt[1::2, None] * np.sin(c)[None, :]


def qjl_term(qt, S, bits, nu, m: int) -> np.ndarray:
    """kappa * nu_t * sum_j (S q~)_j (2 bit_tj - 1) for every token t."""
    Sd = np.asarray(S, dtype=np.float32).astype(np.float64)
    sq = Sd @ qt
    sgn = 2.0 * np.asarray(bits, dtype=np.float64) - 1.0
    return kappa(m) * np.asarray(nu, dtype=np.float64) * (sgn @ sq)


def analytic_logits(q, codes, levels32, S, signs, perm, params: Params) -> np.ndarray:
    """Raw logits (estimates of <q, k_t>) of one query against one stream's codes.

    ``codes`` has rc [T, n], ac [T, n], bits [T, m], nu [T] (a dict or Fields).
    """
    rc, ac, bits, nu = _fields(codes)
    qt = query_transform(q, signs, perm, params)
    lut = angle_lut(qt, params.b_angle)
    lv = np.asarray(levels32, dtype=np.float32).astype(np.float64)
    n = params.n_pairs
    main = np.sum(lv[rc] * lut[np.arange(n)[None, :], ac], axis=1)
    if params.qjl_m:
        main = main + qjl_term(qt, S, bits, nu, params.qjl_m)
    return main


def softmax_weights(logits, scale: float) -> np.ndarray:
    z = scale * np.asarray(logits, dtype=np.float64)
    z = z - np.max(z)
    e = np.exp(z)
    return e / np.sum(e)


def attend(logits, V, scale: float) -> np.ndarray:
    p = softmax_weights(logits, scale)
    return p @ np.asarray(V, dtype=np.float64)


def partial_state(logits, V, scale: float):
    """(m, l, o) of one token block: m = max scaled logit, l = sum e^(z - m), o = sum e^(z - m) V."""
    z = scale * np.asarray(logits, dtype=np.float64)
    mx = float(np.max(z))
    e = np.exp(z - mx)
    return mx, float(np.sum(e)), e @ np.asarray(V, dtype=np.float64)


def merge_states(states) -> np.ndarray:
    """Log-sum-exp merge of block states into the normalized output."""
    M = max(s[0] for s in states)
    num = sum(math.exp(s[0] - M) * s[2] for s in states)
    den = sum(math.exp(s[0] - M) * s[1] for s in states)
    return num / den


def split_attend(logits, V, scale: float, n_splits: int) -> np.ndarray:
    T = len(logits)
    bounds = np.linspace(0, T, n_splits + 1).astype(int)
    states = [partial_state(logits[a:b], V[a:b], scale)
              for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
    return merge_states(states)


def decode_cache(q, codes, V, tables, S, signs, perm, params: Params, scale=None):
    """Decode attention for a whole cache.

    q [n_seq, n_q, d]; codes[b][h] per stream; V [n_seq, n_kv, T, d];
    tables[h] = (levels32, thresholds32).  Returns (out [n_seq, n_q, d], logits
    [n_seq, n_q, T]).
    """
    q = np.asarray(q, dtype=np.float64)
    n_seq, n_q, d = q.shape
    n_kv = len(tables)
    G = n_q // n_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    T = np.asarray(V[0][0]).shape[0]
    out = np.zeros((n_seq, n_q, d))
    lg = np.zeros((n_seq, n_q, T))
    for b in range(n_seq):
        for hq in range(n_q):
            h = hq // G
            s = analytic_logits(q[b, hq], codes[b][h], tables[h][0],
                                None if S is None else S[h], signs[h],
                                None if perm is None else perm[h], params)
            lg[b, hq] = s
            out[b, hq] = attend(s, V[b][h], scale)
    return out, lg


def fp16_attention(q, K16, V16, scale=None):
    """FP16-cache decode attention: softmax(scale q . K) V with K, V read from fp16.

    q [n_seq, n_q, d]; K16, V16 [n_seq, n_kv, T, d].  Returns (out, logits).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K16, dtype=np.float16).astype(np.float64)
    V = np.asarray(V16, dtype=np.float16).astype(np.float64)
    n_seq, n_q, d = q.shape
    n_kv = K.shape[1]
    G = n_q // n_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((n_seq, n_q, d))
    lg = np.zeros((n_seq, n_q, K.shape[2]))
    for b in range(n_seq):
        for hq in range(n_q):
            s = K[b, hq // G] @ q[b, hq]
            lg[b, hq] = s
            out[b, hq] = attend(s, V[b, hq // G], scale)
    return out, lg


def dequantize_keys(codes, levels32, S, signs, perm, params: Params) -> np.ndarray:
    """Explicit reconstruction Khat in the original key domain (for checking only:
    the decoder never builds it).  k~hat per pair from (rc, ac), plus the QJL
    residual estimate kappa * nu * S_h^T (2 bits - 1), then the inverse transform."""
    rc, ac, bits, nu = _fields(codes)
    hx, hy = reconstruct_pairs(rc, ac, levels32, params.b_angle)
    T = rc.shape[0]
    kt = np.empty((T, params.head_dim))
    kt[:, 0::2] = hx
    kt[:, 1::2] = hy
    if params.qjl_m:
        Sd = np.asarray(S, dtype=np.float32).astype(np.float64)
        sgn = 2.0 * np.asarray(bits, dtype=np.float64) - 1.0
        kt = kt + kappa(params.qjl_m) * np.asarray(nu, dtype=np.float64)[:, None] * (sgn @ Sd)
    return rht.inverse(kt, signs, perm, params.hadamard)


def _fields(codes):
    if isinstance(codes, dict):
        return codes["rc"], codes["ac"], codes["bits"], codes["nu"]
    return codes.rc, codes.ac, codes.bits, codes.nu
