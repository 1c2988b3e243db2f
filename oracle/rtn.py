"""Per-token asymmetric round-to-nearest (RTN) key quantization, the control of
the EdgeLLM-Nano paper page ("Comparison to simpler baselines": per-token
asymmetric RTN of K at INT3 / INT4 with an FP16 scale and zero-point per
quantized vector, V kept in FP16; 3.50 / 4.50 bits per element).

Test infrastructure only: imported by the tests, the smoke check and the CPU
baseline of the benchmark, never by the library.

Readings used here (the page gives only the bit budget):
* per key vector k (d values): lo = min k, hi = max k, both rounded to fp16
  (a -0 extreme counts as +0);
  scale = fp16((hi16 - lo16) / (2^b - 1)) (a zero range gives scale 1);
  zero-point = lo16 (an fp16 offset, so that the record holds exactly two FP16
  numbers);
* code_c = clamp(round_half_even((k_c - zp) / scale), 0, 2^b - 1), decided in
  float64 from the fp16 scale and zero-point;
* dequantized k_c = zp + scale * code_c; the logit is <q, khat> (no transform).

Record of one token (this implementation's layout; exactly d b / 8 + 4 bytes):
d b-bit codes as a bit stream (code c at bits [b c, b c + b), least significant
first, d b / 32 uint32 words), then one uint32 holding the fp16 scale (low half)
and the fp16 zero-point (high half).  A stream of capacity C stores word w of
token t at byte 4 (w C + t).
"""

from __future__ import annotations

import numpy as np


def quantize(K, bits: int):
    K = np.asarray(K, dtype=np.float64)
    # + 0.0 turns a -0 extreme into +0 (the sign of a zero extreme is otherwise
    # left to the order of the comparisons)
    lo = (K.min(axis=-1) + 0.0).astype(np.float16)
    hi = (K.max(axis=-1) + 0.0).astype(np.float16)
    qmax = (1 << bits) - 1
    rng = hi.astype(np.float64) - lo.astype(np.float64)
    scale = (rng / qmax).astype(np.float16)
    scale = np.where(scale.astype(np.float64) > 0, scale, np.float16(1.0)).astype(np.float16)
    zp = lo
    q = np.rint((K - zp.astype(np.float64)[..., None]) / scale.astype(np.float64)[..., None])
    codes = np.clip(q, 0, qmax).astype(np.int64)
    return codes, scale, zp


def dequantize(codes, scale, zp) -> np.ndarray:
    return zp.astype(np.float64)[..., None] + scale.astype(np.float64)[..., None] * codes


def logits(q, codes, scale, zp) -> np.ndarray:
    return dequantize(codes, scale, zp) @ np.asarray(q, dtype=np.float64)


def record_bytes(head_dim: int, bits: int) -> int:
    return head_dim * bits // 8 + 4


def pack_stream(codes, scale, zp, bits: int, capacity: int, token_offset: int = 0, buf=None):
    """Write N tokens' records into slots [token_offset, token_offset + N) of one
    stream buffer (uint8, capacity * record_bytes); other slots are untouched."""
    codes = np.asarray(codes, dtype=np.uint64)
    N, d = codes.shape
    nc = d * bits // 32
    if buf is None:
        buf = np.zeros(capacity * record_bytes(d, bits), dtype=np.uint8)
    words = buf.view(np.uint32).reshape(nc + 1, capacity)
    acc = np.zeros((nc + 1, N), dtype=np.uint64)  # one spare word for the carry
    for c in range(d):
        off = bits * c
        w, s = off // 32, off % 32
        v = codes[:, c] << np.uint64(s)          # at most 35 bits
        acc[w] |= v & np.uint64(0xFFFFFFFF)
        acc[w + 1] |= v >> np.uint64(32)
    sl = slice(token_offset, token_offset + N)
    words[:nc, sl] = acc[:nc].astype(np.uint32)
    sb = np.asarray(scale, dtype=np.float16).view(np.uint16).astype(np.uint32)
    zb = np.asarray(zp, dtype=np.float16).view(np.uint16).astype(np.uint32)
    words[nc, sl] = sb | (zb << np.uint32(16))
    return buf


def unpack_stream(buf, head_dim: int, bits: int, capacity: int, n_tokens: int, token_offset: int = 0):
    nc = head_dim * bits // 32
    words = np.asarray(buf, dtype=np.uint8).view(np.uint32).reshape(nc + 1, capacity)
    w64 = words[:, token_offset:token_offset + n_tokens].astype(np.uint64)
    codes = np.zeros((n_tokens, head_dim), dtype=np.int64)
    mask = np.uint64((1 << bits) - 1)
    for c in range(head_dim):
        off = bits * c
        w, s = off // 32, off % 32
        pair = w64[w] | (w64[w + 1] << np.uint64(32)) if w + 1 < nc else w64[w]
        codes[:, c] = ((pair >> np.uint64(s)) & mask).astype(np.int64)
    sz = words[nc, token_offset:token_offset + n_tokens]
    scale = (sz & 0xFFFF).astype(np.uint16).view(np.float16)
    zp = (sz >> 16).astype(np.uint16).view(np.float16)
    return codes, scale, zp


def pack_cache(K, bits: int, capacity: int):
    """Quantize and pack K [n_seq, n_kv, T, d] -> [n_seq, n_kv, capacity * record] uint8."""
    n_seq, n_kv, T, d = K.shape
    out = np.zeros((n_seq, n_kv, capacity * record_bytes(d, bits)), dtype=np.uint8)
    for b in range(n_seq):
        for h in range(n_kv):
            if T:
                codes, scale, zp = quantize(K[b, h], bits)
                pack_stream(codes, scale, zp, bits, capacity, 0, out[b, h])
    return out


def decode_cache(q, K, V, bits: int, scale_sm=None):
    """RTN decode attention: q [n_seq, n_q, d]; K, V [n_seq, n_kv, T, d].
    Returns (out, logits) in float64."""
    from .attn import attend
    q = np.asarray(q, dtype=np.float64)
    n_seq, n_q, d = q.shape
    n_kv = K.shape[1]
    G = n_q // n_kv
    sm = 1.0 / np.sqrt(d) if scale_sm is None else scale_sm
    out = np.zeros((n_seq, n_q, d))
    lg = np.zeros((n_seq, n_q, K.shape[2]))
    for b in range(n_seq):
        for h in range(n_kv):
            codes, scale, zp = quantize(K[b, h], bits)
            Khat = dequantize(codes, scale, zp)
            for g in range(G):
                s = Khat @ q[b, h * G + g]
                lg[b, h * G + g] = s
                out[b, h * G + g] = attend(s, V[b, h], sm)
    return out, lg
