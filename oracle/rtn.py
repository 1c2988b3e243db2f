"""Per-token asymmetric round-to-nearest (RTN) key quantization, the control of
the EdgeLLM-Nano paper page ("Comparison to simpler baselines": per-token
asymmetric RTN of K at INT3 / INT4 with an FP16 scale and zero-point per
quantized vector, V kept in FP16).

Readings used here (the page gives only the bit budget):
* per key vector k (d values): lo = min k, hi = max k, both rounded to fp16;
  scale = fp16((hi16 - lo16) / (2^b - 1)) (a zero range gives scale 1);
  zero-point = lo16 (an fp16 offset rather than an integer zero-point, so that
  the record is exactly two FP16 numbers);
* code_c = clamp(round_half_even((k_c - zp) / scale), 0, 2^b - 1), decided in
  float64 from the fp16 scale and zero-point;
* dequantized k_c = zp + scale * code_c; the logit is <q, khat>.
"""

from __future__ import annotations

import numpy as np


def quantize(K, bits: int):
    K = np.asarray(K, dtype=np.float64)
    lo = K.min(axis=-1).astype(np.float16)
    hi = K.max(axis=-1).astype(np.float16)
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
