"""Byte and bits-per-element accounting of the compressed key cache.

Source: EdgeLLM-Nano paper page, "Bit budget" ((b_main + b_angle)/2 bits per
element for the polar codes, 1 bit per element of QJL signs, 16/qjl_m bits per
element for the FP16 residual norm; V stays FP16; the K-only figure averages
FP16 V with the PGKQ key bits over a 512-slot context with 511 occupied slots),
the codebook paragraph after "PGKQ pipeline" (the 128-token K+V byte example),
the RTN paragraph ("Comparison to simpler baselines": FP16 scale and
zero-point per quantized vector) and the PGKQ-KV paragraphs (the same recipe
applied to V; byte budget of the throughput paragraph).

Reading used for the 511-slot figure: the capacity average
(16 + key_bpe) / 2 * 511 / 512.  The same factor reproduces the PGKQ-KV range
printed for k2v2 and k4v4.
"""

from __future__ import annotations


def key_record_bytes(head_dim: int, b_main: int, b_angle: int, qjl_m: int) -> float:
    n = head_dim // 2
    b = n * (b_main + b_angle) / 8.0
    if qjl_m:
        b += qjl_m / 8.0 + 2.0
    return b


def key_bits_per_element(head_dim: int, b_main: int, b_angle: int, qjl_m: int) -> float:
    return key_record_bytes(head_dim, b_main, b_angle, qjl_m) * 8.0 / head_dim


def polar_bits_per_element(b_main: int, b_angle: int) -> float:
    return (b_main + b_angle) / 2.0


def qjl_bits_per_element(head_dim: int, qjl_m: int) -> float:
    # m sign bits plus one FP16 norm per head vector, spread over head_dim elements
    return (qjl_m + 16.0) / head_dim


def cache_bytes(n_layers_heads: int, n_tokens: int, head_dim: int, b_main: int, b_angle: int,
                qjl_m: int, v_fp16: bool = True) -> dict:
    k = n_layers_heads * n_tokens * key_record_bytes(head_dim, b_main, b_angle, qjl_m)
    v = n_layers_heads * n_tokens * head_dim * 2 if v_fp16 else 0
    return {"k": k, "v": v, "kv": k + v}


def fp16_cache_bytes(n_layers_heads: int, n_tokens: int, head_dim: int) -> int:
    return 2 * n_layers_heads * n_tokens * head_dim * 2


def occupied_average_bpe(k_bpe: float, v_bpe: float, capacity: int = 512,
                         occupied: int = 511) -> float:
    return (k_bpe + v_bpe) / 2.0 * occupied / capacity


def rtn_bits_per_element(bits: int, head_dim: int) -> float:
    # one FP16 scale and one FP16 zero-point per quantized head vector
    return bits + 32.0 / head_dim
