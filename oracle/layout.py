"""Packed layout of one compressed key stream (one (sequence, kv-head)).

The pages fix only the byte count of a record (EdgeLLM-Nano paper page,
"Bit budget": (b_main + b_angle) / 2 bits per element for the polar codes,
1 bit per element of QJL signs, one FP16 norm per token), i.e.
K_B = n (b_main + b_angle) / 8 + [QJL] (m / 8 + 2) bytes per token-head.
The arrangement below is this implementation's own; it keeps exactly K_B bytes
per token slot:

    P = b_main + b_angle bits per pair; joint code c_i = rc_i | (ac_i << b_main)
    per token, a code stream of n P bits: c_i occupies bits [P i, P i + P) of the
      stream, least significant bit first, in NC = n P / 32 little-endian uint32
      words (stream bit q lives in word q // 32 at bit q mod 32);
    then (QJL) m / 32 sign words: sign bit j at bit j mod 32 of word j // 32;
    a stream of capacity C tokens stores word w of token t at byte 4 (w C + t)
      (word-major rows of C words), followed (QJL) by a row of C fp16 norms.

This module packs and unpacks with plain per-field loops; it shares nothing with
the library's device code.
"""

from __future__ import annotations

import numpy as np

from .encode import Params


def record_bytes(p: Params) -> int:
    n = p.n_pairs
    kb = n * (p.b_main + p.b_angle) // 8
    if p.qjl_m:
        kb += p.qjl_m // 8 + 2
    return kb


def code_words(p: Params) -> int:
    return p.n_pairs * (p.b_main + p.b_angle) // 32


def n_words(p: Params) -> int:
    return code_words(p) + p.qjl_m // 32


def check_packable(p: Params):
    if p.n_pairs % 32 or p.qjl_m % 32:
        raise ValueError("packing needs head_dim/2 and qjl_m to be multiples of 32")


def _stream_bits_to_words(bits):
    """bool [N, 32k] -> uint32 [N, k], stream bit q at bit q % 32 of word q // 32."""
    N, L = bits.shape
    b = bits.reshape(N, L // 32, 32).astype(np.uint64)
    weights = np.uint64(1) << np.arange(32, dtype=np.uint64)
    return (b * weights).sum(axis=-1).astype(np.uint32)


def _words_to_stream_bits(words, L):
    N = words.shape[0]
    w = words.astype(np.uint64)[..., None]
    b = ((w >> np.arange(32, dtype=np.uint64)) & np.uint64(1)).astype(bool)
    return b.reshape(N, -1)[:, :L]


def _codes_to_stream_bits(codes, P):
    """int [N, n] codes -> bool [N, n P]: bit k of code i at stream position P i + k."""
    N, n = codes.shape
    out = np.zeros((N, n * P), dtype=bool)
    for i in range(n):
        for k in range(P):
            out[:, P * i + k] = (codes[:, i] >> k) & 1
    return out


def _stream_bits_to_codes(bits, n, P):
    N = bits.shape[0]
    codes = np.zeros((N, n), dtype=np.int64)
    for i in range(n):
        for k in range(P):
            codes[:, i] |= bits[:, P * i + k].astype(np.int64) << k
    return codes


def pack_stream(fields, p: Params, capacity: int, token_offset: int = 0, buf=None) -> np.ndarray:
    """Write the codes of N tokens into slots [token_offset, token_offset + N)."""
    check_packable(p)
    n = p.n_pairs
    P = p.b_main + p.b_angle
    N = np.asarray(fields.rc).shape[0]
    if token_offset + N > capacity:
        raise ValueError("tokens exceed capacity")
    NC, W = code_words(p), n_words(p)
    if buf is None:
        buf = np.zeros(capacity * record_bytes(p), dtype=np.uint8)
    words = buf[: W * 4 * capacity].view(np.uint32).reshape(W, capacity)
    sl = slice(token_offset, token_offset + N)
    joint = np.asarray(fields.rc, dtype=np.int64) | (np.asarray(fields.ac, dtype=np.int64) << p.b_main)
    words[:NC, sl] = _stream_bits_to_words(_codes_to_stream_bits(joint, P)).T
    if p.qjl_m:
        words[NC:W, sl] = _stream_bits_to_words(np.asarray(fields.bits, dtype=bool)).T
        norms = buf[W * 4 * capacity:].view(np.float16)
        norms[sl] = np.asarray(fields.nu, dtype=np.float16)
    return buf


def unpack_stream(buf, p: Params, capacity: int, n_tokens: int, token_offset: int = 0):
    """Inverse of ``pack_stream``: dict(rc, ac, bits, nu) of the tokens."""
    check_packable(p)
    n = p.n_pairs
    P = p.b_main + p.b_angle
    NC, W = code_words(p), n_words(p)
    buf = np.asarray(buf, dtype=np.uint8)
    words = buf[: W * 4 * capacity].view(np.uint32).reshape(W, capacity)
    sl = slice(token_offset, token_offset + n_tokens)
    joint = _stream_bits_to_codes(_words_to_stream_bits(words[:NC, sl].T, n * P), n, P)
    rc = joint & ((1 << p.b_main) - 1)
    ac = joint >> p.b_main
    if p.qjl_m:
        bits = _words_to_stream_bits(words[NC:W, sl].T, p.qjl_m)
        nu = buf[W * 4 * capacity: capacity * record_bytes(p)].view(np.float16)[sl].copy()
    else:
        bits = np.zeros((n_tokens, 0), dtype=bool)
        nu = np.zeros(n_tokens, dtype=np.float16)
    return {"rc": rc, "ac": ac, "bits": bits, "nu": nu}


def pack_cache(fields, p: Params, capacity: int) -> np.ndarray:
    """fields[b][h] -> uint8 [n_seq, n_kv, capacity * K_B]."""
    n_seq = len(fields)
    n_kv = len(fields[0])
    out = np.zeros((n_seq, n_kv, capacity * record_bytes(p)), dtype=np.uint8)
    for b in range(n_seq):
        for h in range(n_kv):
            pack_stream(fields[b][h], p, capacity, 0, out[b, h])
    return out
