"""Shared set-up for the GPU parity tests: synthetic inputs, the oracle's side
of a case, and the device tensors handed to the library through the binding."""

from __future__ import annotations

import numpy as np
import torch

from oracle import attn, encode, layout
from oracle.encode import Params
from synth import make_inputs

from parity_util import classify, codebook_array, merge_counts, oracle_tables

DEV = "cuda:0"
OUT_TOL = 1e-3     # attention outputs, max-abs
LOGIT_TOL = 2e-3   # logits, in units of ||q|| ||k||
GUARD = 4096       # bytes of guard band on each side of an output or workspace


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


def tile_values(V, cap, spare=0.0):
    """Rows V [n_seq, n_kv, T, d] -> an [n_seq, n_kv, cap, d] fp16 array whose memory is the
    32-token-tile value cache: element (t, c) at half-word
    (t/32) 32 d + ((c/16) 4 + (t%32)/8) 128 + (c%16) 8 + t%8 of its stream.
    Slots past T hold `spare`."""
    n_seq, n_kv, T, d = V.shape
    buf = np.full((n_seq, n_kv, cap, d), spare, dtype=np.float16)
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


def v_cache(V, cap, spare=0.0):
    """Device copy of the tiled value cache of rows V (slots past the rows hold `spare`)."""
    return to_dev(tile_values(np.asarray(V, dtype=np.float16), cap, spare))


class Case:
    """Oracle-side encoding of a workload plus its device copies."""

    def __init__(self, cfg, n_tokens=None, capacity=None, reorder=False, hadamard=True,
                 inputs=None, v_spare=0.0):
        self.cfg = cfg
        self.v_spare = v_spare  # value of the cache's spare slots on the device
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
            V=v_cache(self.V, cap, self.v_spare),
        )


class Guarded:
    """A device tensor of the given shape and dtype inside a larger byte buffer
    whose GUARD bytes on either side are all-ones (NaN as fp16 / fp32): after a
    call, `check()` asserts the kernels wrote nothing outside the tensor.  The
    tensor itself starts out all-ones as well, so an element no kernel writes
    stays NaN and fails the comparison."""

    def __init__(self, shape, dtype):
        n = 1
        for s in shape:
            n *= int(s)
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        self.raw = torch.full((2 * GUARD + nbytes,), 0xFF, dtype=torch.uint8, device=DEV)
        self.nbytes = nbytes
        self.t = self.raw[GUARD:GUARD + nbytes].view(dtype).view(*shape)

    def check(self, what):
        lo = self.raw[:GUARD]
        hi = self.raw[GUARD + self.nbytes:]
        assert bool(torch.all(lo == 0xFF)) and bool(torch.all(hi == 0xFF)), \
            f"{what}: a kernel wrote outside its buffer"


def gpu_encode(case, K=None):
    import compressed_cache_decode_pgkq_amd as api
    dev = case.dev_inputs()
    Kt = k_tensor(case.K if K is None else K)
    codes = api.pgkq_encode(lib_params(case.p), Kt, dev["signs"], dev["perm"], dev["codebook"],
                            dev["S"], capacity=case.cap)
    torch.cuda.synchronize()
    return codes.cpu().numpy()


def code_counts(case, got):
    f = case.oracle_fields()
    counts = {}
    n_seq, n_kv = case.K.shape[:2]
    for b in range(n_seq):
        for h in range(n_kv):
            u = layout.unpack_stream(got[b, h], case.p, case.cap, case.T)
            merge_counts(counts, classify(f[b][h], u, case.tables[h][1],
                                          None if case.S is None else case.S[h], case.p))
    return counts


def logit_bound(case, b, hq, q=None):
    q = case.q if q is None else q
    G = q.shape[1] // case.K.shape[1]
    qn = np.linalg.norm(q[b, hq].astype(np.float64))
    kn = np.linalg.norm(case.K[b, hq // G].astype(np.float64), axis=1)
    return LOGIT_TOL * qn * kn


def check_decode(case, n_splits=0, q_override=None, q_dtype=None):
    """Decode attention and the logit hook on the oracle's own code buffer against
    the oracle; outputs, logits and workspaces sit between guard bands."""
    import compressed_cache_decode_pgkq_amd as api
    dev = case.dev_inputs()
    p = lib_params(case.p)
    q = case.q if q_override is None else q_override
    qt = q_tensor(q, q_dtype or case.cfg.q_dtype)
    codes = to_dev(case.oracle_codes())
    n_seq, n_q, d = q.shape
    n_kv = case.K.shape[1]
    out = Guarded((n_seq, n_q, d), torch.float32)
    lg = Guarded((n_seq, n_q, case.T), torch.float32)
    nb = api.pgkq_decode_workspace_bytes(p, n_seq, n_q, n_kv, case.T, n_splits)
    ws = Guarded((max(nb, 16),), torch.uint8)
    nb_l = api.pgkq_decode_workspace_bytes(p, n_seq, n_q, n_kv, case.T, 0)
    ws_l = Guarded((max(nb_l, 16),), torch.uint8)
    api.pgkq_decode_attn(p, qt, codes, dev["V"], dev["signs"], dev["perm"], dev["codebook"],
                         dev["S"], n_tokens=case.T, n_splits=n_splits, out=out.t, workspace=ws.t)
    api.pgkq_estimate_logits(p, qt, codes, n_kv, case.cap, dev["signs"], dev["perm"],
                             dev["codebook"], dev["S"], n_tokens=case.T, logits=lg.t, workspace=ws_l.t)
    torch.cuda.synchronize()
    for g, what in ((out, "out"), (lg, "logits"), (ws, "workspace"), (ws_l, "logit workspace")):
        g.check(what)
    ref, ref_lg = case.oracle_decode(q=q)
    o = out.t.cpu().numpy()
    l = lg.t.cpu().numpy()
    err = float(np.max(np.abs(o - ref))) if o.size else 0.0
    assert np.all(np.isfinite(o))
    worst = 0.0
    if case.T:
        for b in range(n_seq):
            for hq in range(n_q):
                bound = logit_bound(case, b, hq, q)
                worst = max(worst, float(np.max(np.abs(l[b, hq] - ref_lg[b, hq]) / bound)))
    print(f"decode max-abs {err:.3e}  logit err / bound {worst:.3e}")
    assert err <= OUT_TOL
    assert worst <= 1.0
    return o
