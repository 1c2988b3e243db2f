"""PyTorch-facing binding of the PGKQ C ABI: argument marshalling only.

Every function has the name of the C entry point it calls.  Tensors must live
on the GPU; device memory for outputs and workspaces is allocated with PyTorch
when the caller does not pass it, and work is enqueued on the current PyTorch
stream.  All arithmetic happens in the HIP kernels of libpgkq.so.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np
import torch

from . import _lib as L


@dataclass(frozen=True)
class PgkqParams:
    head_dim: int
    b_main: int
    b_angle: int
    qjl_m: int
    hadamard: int = 1

    def c(self) -> L.PgkqParams:
        return L.PgkqParams(self.head_dim, self.b_main, self.b_angle, self.qjl_m, self.hadamard)


_DT = {torch.float32: L.PGKQ_F32, torch.float16: L.PGKQ_F16, torch.bfloat16: L.PGKQ_BF16}


def _dtype(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("PGKQ entry points take device tensors")
    if not t.is_contiguous():
        raise ValueError("PGKQ entry points take contiguous tensors")
    return ctypes.c_void_p(t.data_ptr())


def _half(t):
    """Device pointer of an fp16 tensor (value caches, value rows, fp16 keys)."""
    if t is not None and t.dtype != torch.float16:
        raise TypeError(f"expected a float16 tensor, got {t.dtype}")
    return _ptr(t)


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _expect_shape(t, shape, what):
    """Raise before anything is launched when a tensor's shape is not the one the
    call's sizes imply (the C ABI sees pointers only, so this check lives here)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _expect_codes(codes, n_streams, capacity, record, what="codes"):
    if record == 0:
        return  # invalid parameters: the library call itself reports them
    want = int(n_streams) * int(capacity) * int(record)
    got = _nbytes(codes)
    if got != want:
        raise ValueError(f"{what}: {got} bytes, expected n_seq * n_kv * capacity * record bytes "
                         f"= {n_streams} * {capacity} * {record} = {want}")


def _code_capacity(codes, n_streams, record, what="codes"):
    """Slots per stream of an existing code buffer (its size must be a whole number of them)."""
    per = int(n_streams) * int(record)
    if per <= 0:
        return 1  # invalid parameters: the library call itself reports them
    got = _nbytes(codes)
    if got % per:
        raise ValueError(f"{what}: {got} bytes is not a whole number of "
                         f"n_seq * n_kv * record = {per}-byte slot rows")
    return got // per


def default_capacity(n_tokens: int) -> int:
    """Slots per stream used when the caller gives none: n_tokens rounded up to the
    32-token value tile (the same rule as pgkq_pack_values), so that the key codes
    and the value cache of one stream always agree."""
    return max(32, (int(n_tokens) + 31) // 32 * 32)


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _opts(n_splits: int, events):
    o = L.PgkqLaunchOpts(int(n_splits), None, None)
    if events is not None:
        o.scan_start = ctypes.c_void_p(events[0].cuda_event)
        o.scan_stop = ctypes.c_void_p(events[1].cuda_event)
    return o


def _ws(nbytes: int, device, workspace):
    if nbytes == 0:
        return workspace, 0
    if workspace is None or workspace.numel() * workspace.element_size() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def pgkq_version() -> str:
    return L.lib().pgkq_version().decode()


def pgkq_record_bytes(params: PgkqParams) -> int:
    return int(L.lib().pgkq_record_bytes(ctypes.byref(params.c())))


def pgkq_codes_bytes(params: PgkqParams, n_streams: int, capacity: int) -> int:
    return int(L.lib().pgkq_codes_bytes(ctypes.byref(params.c()), n_streams, capacity))


def pgkq_lloyd_max_beta(head_dim: int, b_main: int):
    n = 1 << b_main
    lv = (ctypes.c_double * n)()
    th = (ctypes.c_double * max(n - 1, 1))()
    L.check(L.lib().pgkq_lloyd_max_beta(head_dim, b_main, lv, th), "pgkq_lloyd_max_beta")
    return np.array(lv[:], dtype=np.float64), np.array(th[: n - 1], dtype=np.float64)


def pgkq_lloyd_max_empirical(samples, b_main: int):
    """Lloyd-Max table refit on a host sample of rho values -> (levels, thresholds)."""
    x = np.ascontiguousarray(np.asarray(samples, dtype=np.float64).ravel())
    n = 1 << b_main
    lv = (ctypes.c_double * n)()
    th = (ctypes.c_double * max(n - 1, 1))()
    L.check(L.lib().pgkq_lloyd_max_empirical(
        x.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), x.size, b_main, lv, th),
        "pgkq_lloyd_max_empirical")
    return np.array(lv[:], dtype=np.float64), np.array(th[: n - 1], dtype=np.float64)


def pgkq_calibrate(params: PgkqParams, K: torch.Tensor, reorder: bool = False, stream=None):
    """K [n_seq, n_kv, n_tokens, d] -> (sumsq [n_kv, d] f64, perm [n_kv, d] i16 bits of u16,
    codebook [n_kv, 2L] f32)."""
    n_seq, n_kv, n_tok, d = K.shape
    p = params.c()
    dev = K.device
    sumsq = torch.empty((n_kv, d), dtype=torch.float64, device=dev)
    perm = torch.empty((n_kv, d), dtype=torch.int16, device=dev)
    cb = torch.empty((n_kv, 2 << params.b_main), dtype=torch.float32, device=dev)
    nb = int(L.lib().pgkq_calibrate_workspace_bytes(ctypes.byref(p), n_seq, n_kv, n_tok))
    ws, wsb = _ws(max(nb, 256), dev, None)
    st = L.lib().pgkq_calibrate(ctypes.byref(p), _ptr(K), _dtype(K), n_seq, n_kv, n_tok,
                                1 if reorder else 0, _ptr(sumsq), _ptr(perm), _ptr(cb), _ptr(ws),
                                wsb, _stream(stream))
    L.check(st, "pgkq_calibrate")
    return sumsq, perm, cb


def pgkq_encode(params: PgkqParams, K: torch.Tensor, signs: torch.Tensor, perm, codebook,
                S, codes=None, capacity=None, token_offset: int = 0, stream=None):
    """Encode K [n_seq, n_kv, n_tokens, d] into codes [n_seq, n_kv, capacity * record] uint8.

    Without ``codes`` a zeroed buffer of ``capacity`` slots per stream is made
    (default: n_tokens rounded up to 32, as for the value cache); with ``codes``
    its size must be n_seq * n_kv * capacity * record bytes (capacity defaults to
    what the buffer holds)."""
    n_seq, n_kv, n_tok, d = K.shape
    p = params.c()
    rb = pgkq_record_bytes(params)
    if codes is None:
        cap = int(capacity) if capacity is not None else default_capacity(n_tok)
        codes = torch.zeros((n_seq, n_kv, cap * rb), dtype=torch.uint8, device=K.device)
    else:
        cap = int(capacity) if capacity is not None else _code_capacity(codes, n_seq * n_kv, rb)
        _expect_codes(codes, n_seq * n_kv, cap, rb)
    st = L.lib().pgkq_encode(ctypes.byref(p), _ptr(K), _dtype(K), n_seq, n_kv, n_tok, _ptr(signs),
                             _ptr(perm), _ptr(codebook), _ptr(S), _ptr(codes), cap,
                             int(token_offset), _stream(stream))
    L.check(st, "pgkq_encode")
    return codes


def pgkq_decode_workspace_bytes(params: PgkqParams, n_seq, n_q, n_kv, n_tokens, n_splits=0) -> int:
    o = _opts(n_splits, None)
    return int(L.lib().pgkq_decode_workspace_bytes(ctypes.byref(params.c()), n_seq, n_q, n_kv,
                                                    n_tokens, ctypes.byref(o)))


def pgkq_decode_attn(params: PgkqParams, q: torch.Tensor, codes: torch.Tensor, V: torch.Tensor,
                     signs, perm, codebook, S, n_tokens=None, softmax_scale: float = 0.0,
                     n_splits: int = 0, out=None, workspace=None, events=None, stream=None):
    """q [n_seq, n_q, d]; codes [n_seq, n_kv, cap * record]; V the fp16 value cache
    [n_seq, n_kv, cap, d] in 32-token tiles (pgkq_pack_values)."""
    n_seq, n_q, d = q.shape
    n_kv, cap = V.shape[1], V.shape[2]
    _expect_shape(V, (n_seq, n_kv, cap, d), "V")
    _expect_codes(codes, n_seq * n_kv, cap, pgkq_record_bytes(params))
    n_tok = cap if n_tokens is None else int(n_tokens)
    p = params.c()
    o = _opts(n_splits, events)
    if out is None:
        out = torch.empty((n_seq, n_q, d), dtype=torch.float32, device=q.device)
    _expect_shape(out, (n_seq, n_q, d), "out")
    nb = int(L.lib().pgkq_decode_workspace_bytes(ctypes.byref(p), n_seq, n_q, n_kv, n_tok,
                                                  ctypes.byref(o)))
    ws, wsb = _ws(nb, q.device, workspace)
    st = L.lib().pgkq_decode_attn(ctypes.byref(p), _ptr(q), _dtype(q), n_seq, n_q, n_kv, n_tok, cap,
                                  _ptr(signs), _ptr(perm), _ptr(codebook), _ptr(S), _ptr(codes),
                                  _half(V), _ptr(out), float(softmax_scale), ctypes.byref(o),
                                  _ptr(ws), wsb, _stream(stream))
    L.check(st, "pgkq_decode_attn")
    return out


def pgkq_decode_attn_noalloc(params: PgkqParams, q: torch.Tensor, codes: torch.Tensor,
                             V: torch.Tensor, signs, perm, codebook, S, out: torch.Tensor,
                             n_tokens=None, softmax_scale: float = 0.0, n_splits: int = 0,
                             stream=None):
    """pgkq_decode_attn with the library's built-in scratch as the workspace: the
    caller passes inputs and `out` [n_seq, n_q, d] fp32; nothing is allocated."""
    n_seq, n_q, d = q.shape
    n_kv, cap = V.shape[1], V.shape[2]
    _expect_shape(V, (n_seq, n_kv, cap, d), "V")
    _expect_codes(codes, n_seq * n_kv, cap, pgkq_record_bytes(params))
    _expect_shape(out, (n_seq, n_q, d), "out")
    n_tok = cap if n_tokens is None else int(n_tokens)
    o = _opts(n_splits, None)
    st = L.lib().pgkq_decode_attn_noalloc(ctypes.byref(params.c()), _ptr(q), _dtype(q), n_seq, n_q,
                                          n_kv, n_tok, cap, _ptr(signs), _ptr(perm), _ptr(codebook),
                                          _ptr(S), _ptr(codes), _half(V), _ptr(out),
                                          float(softmax_scale), ctypes.byref(o), _stream(stream))
    L.check(st, "pgkq_decode_attn_noalloc")
    return out


def pgkq_decode_step(params: PgkqParams, q: torch.Tensor, k_new: torch.Tensor,
                     v_new: torch.Tensor, codes: torch.Tensor, V: torch.Tensor, n_cached: int,
                     signs, perm, codebook, S, softmax_scale: float = 0.0, n_splits: int = 0,
                     out=None, workspace=None, events=None, stream=None):
    """Append k_new, v_new [n_seq, n_kv, d] at slot n_cached of codes / V (in place),
    then decode attention over n_cached + 1 tokens -> out [n_seq, n_q, d]."""
    n_seq, n_q, d = q.shape
    n_kv, cap = V.shape[1], V.shape[2]
    _expect_shape(V, (n_seq, n_kv, cap, d), "V")
    _expect_shape(k_new, (n_seq, n_kv, d), "k_new")
    _expect_shape(v_new, (n_seq, n_kv, d), "v_new")
    _expect_codes(codes, n_seq * n_kv, cap, pgkq_record_bytes(params))
    p = params.c()
    o = _opts(n_splits, events)
    if out is None:
        out = torch.empty((n_seq, n_q, d), dtype=torch.float32, device=q.device)
    _expect_shape(out, (n_seq, n_q, d), "out")
    nb = int(L.lib().pgkq_decode_workspace_bytes(ctypes.byref(p), n_seq, n_q, n_kv,
                                                  int(n_cached) + 1, ctypes.byref(o)))
    ws, wsb = _ws(nb, q.device, workspace)
    st = L.lib().pgkq_decode_step(ctypes.byref(p), _ptr(q), _dtype(q), _ptr(k_new), _dtype(k_new),
                                  _half(v_new), n_seq, n_q, n_kv, int(n_cached), cap, _ptr(signs),
                                  _ptr(perm), _ptr(codebook), _ptr(S), _ptr(codes), _half(V),
                                  _ptr(out), float(softmax_scale), ctypes.byref(o), _ptr(ws), wsb,
                                  _stream(stream))
    L.check(st, "pgkq_decode_step")
    return out


def pgkq_estimate_logits(params: PgkqParams, q: torch.Tensor, codes: torch.Tensor, n_kv: int,
                         capacity: int, signs, perm, codebook, S, n_tokens=None, logits=None,
                         workspace=None, stream=None):
    """Raw logits [n_seq, n_q, n_tokens] fp32 (no softmax scale)."""
    n_seq, n_q, d = q.shape
    _expect_codes(codes, n_seq * n_kv, capacity, pgkq_record_bytes(params))
    n_tok = capacity if n_tokens is None else int(n_tokens)
    p = params.c()
    if logits is None:
        logits = torch.empty((n_seq, n_q, n_tok), dtype=torch.float32, device=q.device)
    _expect_shape(logits, (n_seq, n_q, n_tok), "logits")
    nb = int(L.lib().pgkq_decode_workspace_bytes(ctypes.byref(p), n_seq, n_q, n_kv, n_tok, None))
    ws, wsb = _ws(nb, q.device, workspace)
    st = L.lib().pgkq_estimate_logits(ctypes.byref(p), _ptr(q), _dtype(q), n_seq, n_q, n_kv, n_tok,
                                      capacity, _ptr(signs), _ptr(perm), _ptr(codebook), _ptr(S),
                                      _ptr(codes), _ptr(logits), _ptr(ws), wsb, _stream(stream))
    L.check(st, "pgkq_estimate_logits")
    return logits


def pgkq_fp16_decode_workspace_bytes(head_dim, n_seq, n_q, n_kv, n_tokens, n_splits=0) -> int:
    o = _opts(n_splits, None)
    return int(L.lib().pgkq_fp16_decode_workspace_bytes(head_dim, n_seq, n_q, n_kv, n_tokens,
                                                         ctypes.byref(o)))


def pgkq_calibrate_workspace_bytes(params: PgkqParams, n_seq, n_kv, n_tokens) -> int:
    return int(L.lib().pgkq_calibrate_workspace_bytes(ctypes.byref(params.c()), n_seq, n_kv,
                                                       n_tokens))


def pgkq_status_string(status: int) -> str:
    return L.status_string(status)


def pgkq_pack_values(rows: torch.Tensor, capacity=None, cache=None, slot_offset: int = 0,
                     stream=None):
    """fp16 value rows [n_seq, n_kv, T, d] -> the value cache [n_seq, n_kv, capacity, d] in
    32-token tiles (slots [slot_offset, slot_offset + T) written; capacity defaults to T
    rounded up to 32)."""
    n_seq, n_kv, T, d = rows.shape
    if cache is None:
        cap = int(capacity) if capacity is not None else default_capacity(T)
        cache = torch.zeros((n_seq, n_kv, cap, d), dtype=torch.float16, device=rows.device)
    cap = cache.shape[2]
    _expect_shape(cache, (n_seq, n_kv, cap, d), "cache")
    rows = rows.contiguous()
    st = L.lib().pgkq_pack_values(_half(rows), n_seq * n_kv, T, d, _half(cache), cap, int(slot_offset),
                                  _stream(stream))
    L.check(st, "pgkq_pack_values")
    return cache


def pgkq_unpack_values(cache: torch.Tensor, n_tokens=None, slot_offset: int = 0, stream=None):
    """Slots [slot_offset, slot_offset + n_tokens) of a tiled value cache -> rows
    [n_seq, n_kv, n_tokens, d] fp16."""
    n_seq, n_kv, cap, d = cache.shape
    T = cap - int(slot_offset) if n_tokens is None else int(n_tokens)
    rows = torch.empty((n_seq, n_kv, T, d), dtype=torch.float16, device=cache.device)
    st = L.lib().pgkq_unpack_values(_half(cache), n_seq * n_kv, cap, d, int(slot_offset), T,
                                    _ptr(rows), _stream(stream))
    L.check(st, "pgkq_unpack_values")
    return rows


def pgkq_fp16_decode_attn(q: torch.Tensor, K16: torch.Tensor, V16: torch.Tensor, n_tokens=None,
                          softmax_scale: float = 0.0, n_splits: int = 0, out=None, workspace=None,
                          events=None, stream=None):
    """K16 [n_seq, n_kv, cap, d] fp16 rows; V16 the tiled value cache of the same shape."""
    n_seq, n_q, d = q.shape
    n_kv, cap = K16.shape[1], K16.shape[2]
    _expect_shape(K16, (n_seq, n_kv, cap, d), "K16")
    _expect_shape(V16, (n_seq, n_kv, cap, d), "V16")
    n_tok = cap if n_tokens is None else int(n_tokens)
    o = _opts(n_splits, events)
    if out is None:
        out = torch.empty((n_seq, n_q, d), dtype=torch.float32, device=q.device)
    nb = int(L.lib().pgkq_fp16_decode_workspace_bytes(d, n_seq, n_q, n_kv, n_tok, ctypes.byref(o)))
    ws, wsb = _ws(nb, q.device, workspace)
    st = L.lib().pgkq_fp16_decode_attn(_ptr(q), _dtype(q), n_seq, n_q, n_kv, n_tok, cap, d,
                                       _half(K16), _half(V16), _ptr(out), float(softmax_scale),
                                       ctypes.byref(o), _ptr(ws) if ws is not None else None, wsb,
                                       _stream(stream))
    L.check(st, "pgkq_fp16_decode_attn")
    return out


# ---------------------------------------------------------------- PGKQ-KV


def pgkq_kv_decode_workspace_bytes(pk: PgkqParams, pv: PgkqParams, n_seq, n_q, n_kv, n_tokens,
                                   n_splits=0) -> int:
    o = _opts(n_splits, None)
    return int(L.lib().pgkq_kv_decode_workspace_bytes(ctypes.byref(pk.c()), ctypes.byref(pv.c()),
                                                       n_seq, n_q, n_kv, n_tokens, ctypes.byref(o)))


def pgkq_kv_decode_attn(pk: PgkqParams, pv: PgkqParams, q: torch.Tensor, codes_k: torch.Tensor,
                        codes_v: torch.Tensor, n_kv: int, capacity: int, signs, perm, codebook_k,
                        S_k, codebook_v, S_v, n_tokens=None, softmax_scale: float = 0.0,
                        n_splits: int = 0, out=None, workspace=None, events=None, stream=None):
    """Decode attention over key codes and value codes [n_seq, n_kv, capacity * record]."""
    n_seq, n_q, d = q.shape
    _expect_codes(codes_k, n_seq * n_kv, capacity, pgkq_record_bytes(pk), "codes_k")
    _expect_codes(codes_v, n_seq * n_kv, capacity, pgkq_record_bytes(pv), "codes_v")
    n_tok = capacity if n_tokens is None else int(n_tokens)
    o = _opts(n_splits, events)
    if out is None:
        out = torch.empty((n_seq, n_q, d), dtype=torch.float32, device=q.device)
    _expect_shape(out, (n_seq, n_q, d), "out")
    ck, cv = pk.c(), pv.c()
    nb = int(L.lib().pgkq_kv_decode_workspace_bytes(ctypes.byref(ck), ctypes.byref(cv), n_seq, n_q,
                                                     n_kv, n_tok, ctypes.byref(o)))
    ws, wsb = _ws(nb, q.device, workspace)
    st = L.lib().pgkq_kv_decode_attn(ctypes.byref(ck), ctypes.byref(cv), _ptr(q), _dtype(q), n_seq,
                                     n_q, n_kv, n_tok, capacity, _ptr(signs), _ptr(perm),
                                     _ptr(codebook_k), _ptr(S_k), _ptr(codes_k), _ptr(codebook_v),
                                     _ptr(S_v), _ptr(codes_v), _ptr(out), float(softmax_scale),
                                     ctypes.byref(o), _ptr(ws), wsb, _stream(stream))
    L.check(st, "pgkq_kv_decode_attn")
    return out


# ---------------------------------------------------------------- RTN control


def pgkq_rtn_record_bytes(head_dim: int, bits: int) -> int:
    return int(L.lib().pgkq_rtn_record_bytes(head_dim, bits))


def pgkq_rtn_encode(K: torch.Tensor, bits: int, codes=None, capacity=None, token_offset: int = 0,
                    stream=None):
    """K [n_seq, n_kv, n_tokens, d] (fp32 / fp16) -> codes [n_seq, n_kv, capacity * record] uint8."""
    n_seq, n_kv, n_tok, d = K.shape
    rb = pgkq_rtn_record_bytes(d, bits)
    if codes is None:
        cap = int(capacity) if capacity is not None else default_capacity(n_tok)
        codes = torch.zeros((n_seq, n_kv, cap * rb), dtype=torch.uint8, device=K.device)
    else:
        cap = int(capacity) if capacity is not None else _code_capacity(codes, n_seq * n_kv, rb)
        _expect_codes(codes, n_seq * n_kv, cap, rb)
    st = L.lib().pgkq_rtn_encode(d, bits, _ptr(K), _dtype(K), n_seq, n_kv, n_tok, _ptr(codes), cap,
                                 int(token_offset), _stream(stream))
    L.check(st, "pgkq_rtn_encode")
    return codes


def pgkq_rtn_decode_workspace_bytes(head_dim, n_seq, n_q, n_kv, n_tokens, n_splits=0) -> int:
    o = _opts(n_splits, None)
    return int(L.lib().pgkq_rtn_decode_workspace_bytes(head_dim, n_seq, n_q, n_kv, n_tokens,
                                                        ctypes.byref(o)))


def pgkq_rtn_decode_attn(q: torch.Tensor, codes: torch.Tensor, V: torch.Tensor, bits: int,
                         n_tokens=None, softmax_scale: float = 0.0, n_splits: int = 0, out=None,
                         workspace=None, events=None, stream=None):
    """q [n_seq, n_q, d]; codes [n_seq, n_kv, cap * record]; V the tiled fp16 value cache
    [n_seq, n_kv, cap, d]."""
    n_seq, n_q, d = q.shape
    n_kv, cap = V.shape[1], V.shape[2]
    _expect_shape(V, (n_seq, n_kv, cap, d), "V")
    _expect_codes(codes, n_seq * n_kv, cap, pgkq_rtn_record_bytes(d, bits))
    n_tok = cap if n_tokens is None else int(n_tokens)
    o = _opts(n_splits, events)
    if out is None:
        out = torch.empty((n_seq, n_q, d), dtype=torch.float32, device=q.device)
    _expect_shape(out, (n_seq, n_q, d), "out")
    nb = int(L.lib().pgkq_rtn_decode_workspace_bytes(d, n_seq, n_q, n_kv, n_tok, ctypes.byref(o)))
    ws, wsb = _ws(nb, q.device, workspace)
    st = L.lib().pgkq_rtn_decode_attn(d, bits, _ptr(q), _dtype(q), n_seq, n_q, n_kv, n_tok, cap,
                                      _ptr(codes), _half(V), _ptr(out), float(softmax_scale),
                                      ctypes.byref(o), _ptr(ws), wsb, _stream(stream))
    L.check(st, "pgkq_rtn_decode_attn")
    return out


def pgkq_rtn_logits(q: torch.Tensor, codes: torch.Tensor, n_kv: int, capacity: int, bits: int,
                    n_tokens=None, logits=None, workspace=None, stream=None):
    """Raw RTN logits [n_seq, n_q, n_tokens] fp32."""
    n_seq, n_q, d = q.shape
    _expect_codes(codes, n_seq * n_kv, capacity, pgkq_rtn_record_bytes(d, bits))
    n_tok = capacity if n_tokens is None else int(n_tokens)
    if logits is None:
        logits = torch.empty((n_seq, n_q, n_tok), dtype=torch.float32, device=q.device)
    _expect_shape(logits, (n_seq, n_q, n_tok), "logits")
    nb = int(L.lib().pgkq_rtn_decode_workspace_bytes(d, n_seq, n_q, n_kv, n_tok, None))
    ws, wsb = _ws(nb, q.device, workspace)
    st = L.lib().pgkq_rtn_logits(d, bits, _ptr(q), _dtype(q), n_seq, n_q, n_kv, n_tok, capacity,
                                 _ptr(codes), _ptr(logits), _ptr(ws), wsb, _stream(stream))
    L.check(st, "pgkq_rtn_logits")
    return logits


def pgkq_stream_read(src: torch.Tensor, xor_out=None, stream=None):
    """Read probe: reads every byte of `src` the way the decode scans read the
    cache and XORs its 32-bit words into `xor_out` (a one-element int32 device
    tensor, zero-filled here when not given).  Returns `xor_out`."""
    if xor_out is None:
        xor_out = torch.zeros(1, dtype=torch.int32, device=src.device)
    if _nbytes(xor_out) < 4:
        raise ValueError("xor_out: needs one 32-bit word")
    st = L.lib().pgkq_stream_read(_ptr(src), _nbytes(src), _ptr(xor_out), _stream(stream))
    L.check(st, "pgkq_stream_read")
    return xor_out
