"""PGKQ-KV: the value cache coded like the keys.

Source: EdgeLLM-Nano paper page, the PGKQ-KV paragraphs (PGKQ's polar
representation, Lloyd-Max codebooks and QJL projection also applied to V, with
the Hadamard rotation disabled for V; Beta-prior tables (PGKQ-KV) or an
empirical refit (PGKQ-KV')), the throughput paragraph (its KV-byte budget of
184 320 at the 128-token example = twice the K-only 92 160) and "Bit budget"
(the record size).

Test infrastructure only: imported by the tests, the smoke check and the CPU
baseline of the benchmark, never by the library.

Readings used here:
* the values of one (layer, kv-head) go through the key encoder with the
  identity transform (no sign flips, no channel reorder): pairs (v_2i, v_2i+1)
  -> radius code against the Beta-prior Lloyd-Max table scaled by
  s_h^V = sqrt(mean_t ||v_t||^2) over the values being encoded (the key-side
  reading of the head scale applied to V), mid-rise angle code, QJL bits of
  S^V_h eps with a projection S^V_h of its own, nu = fp16(||eps||);
  b_angle = b_main - 1 as for keys;
* the decoder needs sum_t p_t V-hat_t with V-hat_t the reconstruction the
  codes define: per pair level[rc] (cos thetahat[ac], sin thetahat[ac]), plus
  the QJL residual estimate kappa nu S^V^T (2 bits - 1) (the vector form of the
  logit estimator: its inner product with any q is the QJL logit term);
* p is the softmax of the PGKQ key logits (the K-side path unchanged);
* PGKQ-KV' only swaps the table (any fp32 levels / thresholds): not separate.
"""

from __future__ import annotations

import math

import numpy as np

from . import attn, calibrate, codebook, encode
from .encode import Params


def value_params(head_dim: int, b_main: int, qjl_m: int) -> Params:
    """Parameters of the value encoder: the key encoder without the transform."""
    return Params(head_dim, b_main, b_main - 1, qjl_m, False)


def value_tables(V, b_main: int):
    """Per-kv-head (levels32, thresholds32) for V [n_seq, n_kv, T, d]: the unit
    Beta-prior table scaled by s_h^V / sqrt(d/2)."""
    V = np.asarray(V, dtype=np.float64)
    n_seq, n_kv, T, d = V.shape
    c, t = codebook.lloyd_max_beta(d, b_main)
    tables = []
    for h in range(n_kv):
        Vh = V[:, h].reshape(-1, d)
        ss = calibrate.channel_sumsq(Vh)
        tables.append(codebook.scaled_table(c, t, calibrate.head_scale(ss, len(Vh)), d))
    return tables


def encode_values(V, levels32, thresholds32, S, params: Params) -> encode.Fields:
    """Codes of the values [N, d] of one kv-head."""
    d = params.head_dim
    return encode.encode_keys(V, np.ones(d), None, levels32, thresholds32, S, params)


def dequantize_values(fields, levels32, S, params: Params) -> np.ndarray:
    """V-hat [N, d]: the explicit reconstruction the codes define."""
    d = params.head_dim
    return attn.dequantize_keys(fields, levels32, S, np.ones(d), None, params)


def code_domain_output(p, fields, levels32, S, params: Params) -> np.ndarray:
    """sum_t p_t V-hat_t computed without forming V-hat: the pair reconstructions
    weighted by p, plus kappa S^T (sum_t p_t nu_t (2 bits_t - 1)) once at the
    end (the form the decoder follows).  Equal to p @ V-hat up to rounding."""
    p = np.asarray(p, dtype=np.float64)
    hx, hy = encode.reconstruct_pairs(fields.rc, fields.ac, levels32, params.b_angle)
    out = np.zeros(params.head_dim)
    out[0::2] = p @ hx
    out[1::2] = p @ hy
    if params.qjl_m:
        sgn = 2.0 * np.asarray(fields.bits, dtype=np.float64) - 1.0
        a = (p * np.asarray(fields.nu, dtype=np.float64)) @ sgn
        Sd = np.asarray(S, dtype=np.float32).astype(np.float64)
        out = out + attn.kappa(params.qjl_m) * (a @ Sd)
    return out


def decode_kv(q, k_fields, v_fields, k_tables, v_tables, S_k, S_v, signs, perm, pk: Params,
              pv: Params, scale=None):
    """PGKQ-KV decode attention for a whole cache: q [n_seq, n_q, d];
    k_fields / v_fields [b][h] per stream.  Returns (out, logits)."""
    q = np.asarray(q, dtype=np.float64)
    n_seq, n_q, d = q.shape
    n_kv = len(k_tables)
    G = n_q // n_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    T = len(k_fields[0][0].nu)
    out = np.zeros((n_seq, n_q, d))
    lg = np.zeros((n_seq, n_q, T))
    for b in range(n_seq):
        for h in range(n_kv):
            Vh = dequantize_values(v_fields[b][h], v_tables[h][0],
                                   None if S_v is None else S_v[h], pv)
            for g in range(G):
                hq = h * G + g
                s = attn.analytic_logits(q[b, hq], k_fields[b][h], k_tables[h][0],
                                         None if S_k is None else S_k[h], signs[h],
                                         None if perm is None else perm[h], pk)
                lg[b, hq] = s
                out[b, hq] = attn.softmax_weights(s, scale) @ Vh
    return out, lg
