"""Shared set-up for the GPU parity tests: synthetic inputs, the oracle's side
of a case, and the device tensors handed to the library through the binding."""

from __future__ import annotations

import numpy as np
import torch

from oracle import attn, encode, layout
from oracle.encode import Params
from synth import make_inputs

from parity_util import codebook_array, oracle_tables

DEV = "cuda:0"


def params_of(cfg, hadamard=True) -> Params:
    return Params(cfg.head_dim, cfg.b_main, cfg.b_angle, cfg.qjl_m, hadamard)


def lib_params(p: Params):
    from compressed_cache_decode_pgkq_amd import PgkqParams
    return PgkqParams(p.head_dim, p.b_main, p.b_angle, p.qjl_m, 1 if p.hadamard else 0)


def to_dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def q_tensor(q, q_dtype):
    t = torch.from_numpy(np.ascontiguousarray(q))
    if q_dtype == "bf16":
        t = t.to(torch.bfloat16)   # values are already bf16-representable
    elif q_dtype == "f16":
        t = t.to(torch.float16)
    return t.to(DEV)


def k_tensor(K):
    return torch.from_numpy(np.ascontiguousarray(K)).to(DEV)


VALUE_TILE = 32


def value_capacity(T: int) -> int:
    """Smallest value-cache capacity holding T tokens (a multiple of the 32-token tile)."""
    return max(VALUE_TILE, -(-T // VALUE_TILE) * VALUE_TILE)


def tile_values(V, cap):
    """Rows V [n_seq, n_kv, T, d] -> an [n_seq, n_kv, cap, d] fp16 array whose memory is the
    32-token-tile value cache: element (t, c) at half-word
    (t/32) 32 d + ((c/16) 4 + (t%32)/8) 128 + (c%16) 8 + t%8 of its stream.
    Slots past T are zero."""
    n_seq, n_kv, T, d = V.shape
    buf = np.zeros((n_seq, n_kv, cap, d), dtype=np.float16)
    buf[:, :, :T] = V
    # t = 32 a + 8 b + e, c = 16 f + g  ->  order (a, f, b, g, e)
    x = buf.reshape(n_seq, n_kv, cap // 32, 4, 8, d // 16, 16).transpose(0, 1, 2, 5, 3, 6, 4)
    return np.ascontiguousarray(x).reshape(n_seq, n_kv, cap, d)


def untile_values(buf, T=None):
    """Inverse of tile_values: the tiled cache (array of shape [n_seq, n_kv, cap, d]) -> rows."""
    n_seq, n_kv, cap, d = buf.shape
    x = np.asarray(buf).reshape(n_seq, n_kv, cap // 32, d // 16, 4, 16, 8).transpose(0, 1, 2, 4, 6, 3, 5)
    rows = np.ascontiguousarray(x).reshape(n_seq, n_kv, cap, d)
    return rows if T is None else rows[:, :, :T]


def v_cache(V, cap):
    """Device copy of the tiled value cache of rows V."""
    return to_dev(tile_values(np.asarray(V, dtype=np.float16), cap))


class Case:
    """Oracle-side encoding of a workload plus its device copies."""

    def __init__(self, cfg, n_tokens=None, capacity=None, reorder=False, hadamard=True,
                 inputs=None):
        self.cfg = cfg
        self.p = params_of(cfg, hadamard)
        inp = inputs if inputs is not None else make_inputs(cfg)
        T = cfg.n_tokens if n_tokens is None else n_tokens
        self.T = T
        self.cap = capacity if capacity is not None else value_capacity(T)
        self.K = inp["K"][:, :, :T]
        self.V = inp["V"][:, :, :T]
        self.q = inp["q"]
        self.signs = inp["signs"]
        self.S = inp["S"] if cfg.qjl_m else None
        Kc = self.K if T > 0 else inp["K"][:, :, :1]
        self.tables, self.perm, self.sumsq = oracle_tables(Kc, cfg, reorder)
        self.perm_arg = self.perm if reorder else None
        self.cb = codebook_array(self.tables)

    # ---- oracle side
    def oracle_fields(self):
        if not hasattr(self, "_fields"):
            self._fields = encode.encode_cache(self.K, self.signs, self.perm_arg, self.tables,
                                               self.S, self.p)
        return self._fields

    def oracle_codes(self):
        rb = layout.record_bytes(self.p)
        n_seq, n_kv = self.K.shape[:2]
        out = np.zeros((n_seq, n_kv, self.cap * rb), dtype=np.uint8)
        f = self.oracle_fields()
        for b in range(n_seq):
            for h in range(n_kv):
                layout.pack_stream(f[b][h], self.p, self.cap, 0, out[b, h])
        return out

    def oracle_decode(self, q=None, scale=None):
        q = self.q if q is None else q
        return attn.decode_cache(q, self.oracle_fields(), self.V, self.tables, self.S, self.signs,
                                 self.perm_arg, self.p, scale)

    # ---- device side
    def dev_inputs(self):
        cap = self.cap
        n_seq, n_kv, _, d = self.K.shape
        return dict(
            signs=to_dev(self.signs),
            perm=to_dev(self.perm.astype(np.uint16).view(np.int16)) if self.perm_arg is not None else None,
            codebook=to_dev(self.cb),
            S=to_dev(self.S) if self.S is not None else None,
            V=v_cache(self.V, cap),
        )
