"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes records and workspaces, builds the codebook on the host,
and rejects every invalid argument before touching the device."""

import ctypes
import os
import re

import numpy as np
import pytest

from compressed_cache_decode_pgkq_amd import _lib as L
from compressed_cache_decode_pgkq_amd import api
from oracle import codebook

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pgkq.h")

A = 0x100000  # a 16-byte aligned stand-in pointer, never dereferenced (validation fails first)
MIS = A + 8


def _vp(x):
    return ctypes.c_void_p(x)


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pgkq_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 12
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.SIGNATURES), "binding and header disagree"


def test_status_strings_and_version():
    lib = L.lib()
    for s in range(7):
        assert lib.pgkq_status_string(s)
    assert b"gfx950" in lib.pgkq_version()


@pytest.mark.parametrize("prm,rb", [((64, 3, 2, 64), 30), ((64, 4, 3, 0), 28), ((128, 3, 2, 128), 58),
                                    ((128, 4, 3, 128), 74), ((64, 2, 1, 64), 22), ((128, 3, 2, 0), 40)])
def test_record_bytes(prm, rb):
    p = api.PgkqParams(*prm)
    assert api.pgkq_record_bytes(p) == rb
    assert api.pgkq_codes_bytes(p, 24, 128) == 24 * 128 * rb
    # the printed 128-token example: 92 160 bytes of keys for 24 heads
    if prm == (64, 3, 2, 64):
        assert api.pgkq_codes_bytes(p, 24, 128) == 92160


@pytest.mark.parametrize("prm", [(96, 3, 2, 0), (64, 3, 3, 0), (64, 5, 4, 0), (64, 1, 0, 0),
                                 (64, 3, 2, 32), (64, 3, 2, 64, 2)])
def test_invalid_params_have_no_record(prm):
    assert api.pgkq_record_bytes(api.PgkqParams(*prm)) == 0


@pytest.mark.parametrize("d,b", [(64, 2), (64, 3), (64, 4), (128, 3), (128, 4), (16, 2)])
def test_host_lloyd_max_matches_oracle(d, b):
    lv, th = api.pgkq_lloyd_max_beta(d, b)
    c, t = codebook.lloyd_max_beta(d, b)
    np.testing.assert_allclose(lv, c, rtol=0, atol=1e-11)
    np.testing.assert_allclose(th, t, rtol=0, atol=1e-11)


def test_host_lloyd_max_rejects():
    lv = (ctypes.c_double * 16)()
    th = (ctypes.c_double * 16)()
    lib = L.lib()
    assert lib.pgkq_lloyd_max_beta(64, 3, None, th) == L.PGKQ_ERR_NULL
    assert lib.pgkq_lloyd_max_beta(3, 3, lv, th) == L.PGKQ_ERR_UNSUPPORTED
    assert lib.pgkq_lloyd_max_beta(64, 0, lv, th) == L.PGKQ_ERR_UNSUPPORTED


def _refit_samples(kind):
    rng = np.random.default_rng(5)
    if kind == "halfnormal":
        return np.abs(rng.standard_normal(20000)) * 1.7
    if kind == "prior":
        return codebook.rho_quantile(rng.random(30000), 64)
    if kind == "ties":   # heavy duplicates, some cells may empty
        return rng.integers(0, 12, size=3000).astype(np.float64) * 0.25
    return rng.standard_normal(16) + 3.0   # exactly 2^b samples at b = 4


@pytest.mark.parametrize("kind,b", [("halfnormal", 2), ("halfnormal", 3), ("prior", 4),
                                    ("ties", 3), ("minimal", 4)])
def test_host_empirical_lloyd_max_matches_oracle(kind, b):
    x = _refit_samples(kind)
    lv, th = api.pgkq_lloyd_max_empirical(x, b)
    c, t = codebook.lloyd_max_empirical(x, b)
    np.testing.assert_allclose(lv, c, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(th, t, rtol=1e-12, atol=1e-14)


def test_host_empirical_lloyd_max_rejects():
    lv = (ctypes.c_double * 16)()
    th = (ctypes.c_double * 16)()
    lib = L.lib()
    x = np.abs(np.random.default_rng(0).standard_normal(64))
    xp = x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    assert lib.pgkq_lloyd_max_empirical(None, 64, 3, lv, th) == L.PGKQ_ERR_NULL
    assert lib.pgkq_lloyd_max_empirical(xp, 64, 3, None, th) == L.PGKQ_ERR_NULL
    assert lib.pgkq_lloyd_max_empirical(xp, 7, 3, lv, th) == L.PGKQ_ERR_SHAPE
    assert lib.pgkq_lloyd_max_empirical(xp, 64, 0, lv, th) == L.PGKQ_ERR_UNSUPPORTED
    assert lib.pgkq_lloyd_max_empirical(xp, 64, 9, lv, th) == L.PGKQ_ERR_UNSUPPORTED
    y = x.copy()
    y[5] = np.nan
    assert lib.pgkq_lloyd_max_empirical(y.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), 64, 3,
                                        lv, th) == L.PGKQ_ERR_UNSUPPORTED


def _params(*prm):
    return ctypes.byref(L.PgkqParams(*prm))


def _encode(p=(64, 3, 2, 64, 1), K=A, kd=L.PGKQ_F32, n_seq=1, n_kv=2, n_tok=16, signs=A, perm=None,
            cb=A, S=A, codes=A, cap=16, off=0):
    return L.lib().pgkq_encode(_params(*p) if p else None, _vp(K) if K else None, kd, n_seq, n_kv,
                               n_tok, _vp(signs) if signs else None, _vp(perm) if perm else None,
                               _vp(cb) if cb else None, _vp(S) if S else None,
                               _vp(codes) if codes else None, cap, off, None)


def test_encode_validation():
    assert _encode(p=None) == L.PGKQ_ERR_NULL
    assert _encode(K=0) == L.PGKQ_ERR_NULL
    assert _encode(S=0) == L.PGKQ_ERR_NULL            # QJL needs S
    assert _encode(codes=0) == L.PGKQ_ERR_NULL
    assert _encode(p=(96, 3, 2, 0, 1)) == L.PGKQ_ERR_UNSUPPORTED
    assert _encode(p=(64, 3, 1, 64, 1)) == L.PGKQ_ERR_UNSUPPORTED
    assert _encode(kd=L.PGKQ_BF16) == L.PGKQ_ERR_UNSUPPORTED
    assert _encode(kd=7) == L.PGKQ_ERR_UNSUPPORTED
    assert _encode(n_seq=0) == L.PGKQ_ERR_SHAPE
    assert _encode(n_kv=70000) == L.PGKQ_ERR_SHAPE
    assert _encode(n_tok=17) == L.PGKQ_ERR_SHAPE      # beyond capacity
    assert _encode(off=1) == L.PGKQ_ERR_SHAPE
    assert _encode(n_tok=-1) == L.PGKQ_ERR_SHAPE
    assert _encode(cap=15, n_tok=8) == L.PGKQ_ERR_SHAPE  # odd capacity with QJL
    # a stream beyond the 32-bit range of the buffer stores (d64 b3 + QJL: 30 B a token)
    assert _encode(cap=1 << 28, n_tok=0) == L.PGKQ_ERR_SHAPE
    assert _encode(cap=1 << 27, n_tok=0) == L.PGKQ_OK
    assert _encode(K=MIS) == L.PGKQ_ERR_ALIGN
    assert _encode(codes=MIS) == L.PGKQ_ERR_ALIGN
    assert _encode(perm=MIS) == L.PGKQ_ERR_ALIGN
    # zero tokens: valid no-op, nothing enqueued
    assert _encode(n_tok=0) == L.PGKQ_OK
    # no QJL: S may be NULL
    assert _encode(p=(64, 4, 3, 0, 1), S=0, n_tok=0) == L.PGKQ_OK


def _decode(p=(128, 3, 2, 128, 1), q=A, qd=L.PGKQ_BF16, n_seq=2, n_q=8, n_kv=2, n_tok=100, cap=128,
            signs=A, perm=None, cb=A, S=A, codes=A, V=A, out=A, ws=A, wsb=1 << 30, n_splits=0):
    o = L.PgkqLaunchOpts(n_splits, None, None)
    return L.lib().pgkq_decode_attn(_params(*p), _vp(q) if q else None, qd, n_seq, n_q, n_kv, n_tok,
                                    cap, _vp(signs), _vp(perm) if perm else None, _vp(cb),
                                    _vp(S) if S else None, _vp(codes) if codes else None,
                                    _vp(V) if V else None, _vp(out) if out else None, 0.0,
                                    ctypes.byref(o), _vp(ws) if ws else None, wsb, None)


def test_decode_validation():
    assert _decode(q=0) == L.PGKQ_ERR_NULL
    assert _decode(V=0) == L.PGKQ_ERR_NULL
    assert _decode(out=0) == L.PGKQ_ERR_NULL
    assert _decode(ws=0) == L.PGKQ_ERR_NULL
    assert _decode(S=0) == L.PGKQ_ERR_NULL
    assert _decode(n_q=6) == L.PGKQ_ERR_UNSUPPORTED   # group of 3
    assert _decode(n_q=7) == L.PGKQ_ERR_SHAPE         # not a multiple of n_kv
    assert _decode(n_q=32) == L.PGKQ_ERR_UNSUPPORTED  # group of 16
    assert _decode(n_tok=129) == L.PGKQ_ERR_SHAPE
    assert _decode(cap=127, n_tok=100) == L.PGKQ_ERR_SHAPE
    assert _decode(qd=9) == L.PGKQ_ERR_UNSUPPORTED
    assert _decode(V=MIS) == L.PGKQ_ERR_ALIGN
    assert _decode(out=MIS) == L.PGKQ_ERR_ALIGN
    assert _decode(wsb=16) == L.PGKQ_ERR_WORKSPACE
    p = api.PgkqParams(128, 3, 2, 128)
    need = api.pgkq_decode_workspace_bytes(p, 2, 8, 2, 100)
    assert need > 0
    assert _decode(wsb=need - 1) == L.PGKQ_ERR_WORKSPACE


def test_logits_and_fp16_validation():
    lib = L.lib()
    st = lib.pgkq_estimate_logits(_params(64, 3, 2, 64, 1), _vp(A), L.PGKQ_F32, 1, 4, 4, 10, 16,
                                  _vp(A), None, _vp(A), _vp(A), _vp(A), None, _vp(A), 1 << 20, None)
    assert st == L.PGKQ_ERR_NULL
    o = L.PgkqLaunchOpts(0, None, None)
    st = lib.pgkq_fp16_decode_attn(_vp(A), L.PGKQ_F32, 1, 4, 4, 10, 16, 96, _vp(A), _vp(A), _vp(A),
                                   0.0, ctypes.byref(o), _vp(A), 1 << 20, None)
    assert st == L.PGKQ_ERR_UNSUPPORTED
    st = lib.pgkq_fp16_decode_attn(_vp(A), L.PGKQ_F32, 1, 4, 4, 10, 16, 64, None, _vp(A), _vp(A),
                                   0.0, ctypes.byref(o), _vp(A), 1 << 20, None)
    assert st == L.PGKQ_ERR_NULL
    st = lib.pgkq_fp16_decode_attn(_vp(A), L.PGKQ_F32, 1, 12, 4, 10, 16, 64, _vp(A), _vp(A), _vp(A),
                                   0.0, ctypes.byref(o), _vp(A), 1 << 20, None)
    assert st == L.PGKQ_ERR_UNSUPPORTED
    need = lib.pgkq_fp16_decode_workspace_bytes(128, 16, 32, 8, 32768, ctypes.byref(o))
    st = lib.pgkq_fp16_decode_attn(_vp(A), L.PGKQ_F32, 16, 32, 8, 32768, 32768, 128, _vp(A), _vp(A),
                                   _vp(A), 0.0, ctypes.byref(o), _vp(A), need - 1, None)
    assert need > 0 and st == L.PGKQ_ERR_WORKSPACE


def test_calibrate_validation():
    lib = L.lib()
    p = _params(128, 3, 2, 128, 1)
    need = lib.pgkq_calibrate_workspace_bytes(p, 16, 8, 32768)
    assert need >= 8 * 128 * 8
    args = dict(K=A, kd=L.PGKQ_F16, n_seq=16, n_kv=8, n_tok=32768, reorder=1, ss=A, perm=A, cb=A,
                ws=A, wsb=need)

    def call(**kw):
        a = dict(args, **kw)
        return lib.pgkq_calibrate(p, _vp(a["K"]) if a["K"] else None, a["kd"], a["n_seq"], a["n_kv"],
                                  a["n_tok"], a["reorder"], _vp(a["ss"]),
                                  _vp(a["perm"]) if a["perm"] else None, _vp(a["cb"]), _vp(a["ws"]),
                                  a["wsb"], None)

    assert call(K=0) == L.PGKQ_ERR_NULL
    assert call(perm=0) == L.PGKQ_ERR_NULL
    assert call(n_tok=0) == L.PGKQ_ERR_SHAPE
    assert call(wsb=need - 1) == L.PGKQ_ERR_WORKSPACE
    assert call(K=MIS) == L.PGKQ_ERR_ALIGN
    assert call(kd=L.PGKQ_BF16) == L.PGKQ_ERR_UNSUPPORTED


def test_workspace_sizes_grow_with_splits():
    p = api.PgkqParams(128, 4, 3, 128)
    w1 = api.pgkq_decode_workspace_bytes(p, 1, 32, 8, 131072, n_splits=1)
    w256 = api.pgkq_decode_workspace_bytes(p, 1, 32, 8, 131072, n_splits=256)
    # 256 partitions are one per wavefront: 64 workgroups, whose wavefronts are
    # merged in the workgroup, so 64 partial states per query head
    assert w256 - w1 >= 32 * 64 * (128 + 4) * 4 - 256


def test_buffer_range_limit_is_rejected():
    # one stream's value rows beyond 4 GiB (32-bit buffer offsets): capacity * 128 * 2
    assert _decode(cap=1 << 24, n_tok=100) == L.PGKQ_ERR_SHAPE
    o = L.PgkqLaunchOpts(0, None, None)
    st = L.lib().pgkq_fp16_decode_attn(_vp(A), L.PGKQ_F32, 1, 4, 4, 10, 1 << 24, 128, _vp(A),
                                       _vp(A), _vp(A), 0.0, ctypes.byref(o), _vp(A), 1 << 30, None)
    assert st == L.PGKQ_ERR_SHAPE


@pytest.mark.parametrize("d,bits,rb", [(64, 3, 28), (64, 4, 36), (128, 3, 52), (128, 4, 68)])
def test_rtn_record_bytes(d, bits, rb):
    assert api.pgkq_rtn_record_bytes(d, bits) == rb


@pytest.mark.parametrize("d,bits", [(64, 2), (64, 8), (96, 4), (128, 5)])
def test_rtn_unsupported_has_no_record(d, bits):
    assert api.pgkq_rtn_record_bytes(d, bits) == 0


def _rtn_encode(d=64, bits=3, K=A, kd=L.PGKQ_F16, n_seq=2, n_kv=3, n_tok=16, codes=A, cap=16, off=0):
    return L.lib().pgkq_rtn_encode(d, bits, _vp(K) if K else None, kd, n_seq, n_kv, n_tok,
                                   _vp(codes) if codes else None, cap, off, None)


def test_rtn_encode_validation():
    assert _rtn_encode(K=0) == L.PGKQ_ERR_NULL
    assert _rtn_encode(codes=0) == L.PGKQ_ERR_NULL
    assert _rtn_encode(bits=2) == L.PGKQ_ERR_UNSUPPORTED
    assert _rtn_encode(d=96) == L.PGKQ_ERR_UNSUPPORTED
    assert _rtn_encode(kd=L.PGKQ_BF16) == L.PGKQ_ERR_UNSUPPORTED
    assert _rtn_encode(n_seq=0) == L.PGKQ_ERR_SHAPE
    assert _rtn_encode(n_tok=17) == L.PGKQ_ERR_SHAPE
    assert _rtn_encode(off=1) == L.PGKQ_ERR_SHAPE
    assert _rtn_encode(cap=0, n_tok=0) == L.PGKQ_ERR_SHAPE
    assert _rtn_encode(K=MIS) == L.PGKQ_ERR_ALIGN
    assert _rtn_encode(codes=MIS) == L.PGKQ_ERR_ALIGN
    assert _rtn_encode(n_tok=0) == L.PGKQ_OK


def _rtn_decode(d=128, bits=4, q=A, qd=L.PGKQ_BF16, n_seq=2, n_q=8, n_kv=2, n_tok=100, cap=128,
                codes=A, V=A, out=A, ws=A, wsb=1 << 30, n_splits=0):
    o = L.PgkqLaunchOpts(n_splits, None, None)
    return L.lib().pgkq_rtn_decode_attn(d, bits, _vp(q) if q else None, qd, n_seq, n_q, n_kv, n_tok,
                                        cap, _vp(codes) if codes else None, _vp(V) if V else None,
                                        _vp(out) if out else None, 0.0, ctypes.byref(o),
                                        _vp(ws) if ws else None, wsb, None)


def test_rtn_decode_validation():
    assert _rtn_decode(q=0) == L.PGKQ_ERR_NULL
    assert _rtn_decode(codes=0) == L.PGKQ_ERR_NULL
    assert _rtn_decode(V=0) == L.PGKQ_ERR_NULL
    assert _rtn_decode(out=0) == L.PGKQ_ERR_NULL
    assert _rtn_decode(ws=0) == L.PGKQ_ERR_NULL
    assert _rtn_decode(bits=5) == L.PGKQ_ERR_UNSUPPORTED
    assert _rtn_decode(n_q=6) == L.PGKQ_ERR_UNSUPPORTED
    assert _rtn_decode(n_q=7) == L.PGKQ_ERR_SHAPE
    assert _rtn_decode(n_tok=129) == L.PGKQ_ERR_SHAPE
    assert _rtn_decode(cap=1 << 24) == L.PGKQ_ERR_SHAPE
    assert _rtn_decode(qd=9) == L.PGKQ_ERR_UNSUPPORTED
    assert _rtn_decode(V=MIS) == L.PGKQ_ERR_ALIGN
    assert _rtn_decode(codes=MIS) == L.PGKQ_ERR_ALIGN
    need = api.pgkq_rtn_decode_workspace_bytes(128, 2, 8, 2, 100)
    assert need > 0
    assert _rtn_decode(wsb=need - 1) == L.PGKQ_ERR_WORKSPACE
    st = L.lib().pgkq_rtn_logits(64, 3, _vp(A), L.PGKQ_F32, 1, 4, 4, 10, 16, _vp(A), None, _vp(A),
                                 1 << 20, None)
    assert st == L.PGKQ_ERR_NULL
    # more splits need more workspace
    w1 = api.pgkq_rtn_decode_workspace_bytes(128, 1, 32, 8, 131072, n_splits=1)
    w256 = api.pgkq_rtn_decode_workspace_bytes(128, 1, 32, 8, 131072, n_splits=256)
    assert w256 - w1 >= 32 * 64 * (128 + 4) * 4 - 256


def test_decode_step_validation():
    lib = L.lib()
    o = L.PgkqLaunchOpts(0, None, None)

    def call(k=A, kd=L.PGKQ_F16, v=A, n_cached=99, cap=128, codes=A, V=A, out=A, wsb=1 << 30):
        return lib.pgkq_decode_step(_params(128, 3, 2, 128, 1), _vp(A), L.PGKQ_BF16,
                                    _vp(k) if k else None, kd, _vp(v) if v else None, 2, 8, 2,
                                    n_cached, cap, _vp(A), None, _vp(A), _vp(A),
                                    _vp(codes) if codes else None, _vp(V) if V else None,
                                    _vp(out) if out else None, 0.0, ctypes.byref(o), _vp(A), wsb,
                                    None)

    assert call(k=0) == L.PGKQ_ERR_NULL
    assert call(v=0) == L.PGKQ_ERR_NULL
    assert call(codes=0) == L.PGKQ_ERR_NULL
    assert call(V=0) == L.PGKQ_ERR_NULL
    assert call(out=0) == L.PGKQ_ERR_NULL
    assert call(kd=L.PGKQ_BF16) == L.PGKQ_ERR_UNSUPPORTED
    assert call(n_cached=128) == L.PGKQ_ERR_SHAPE     # no free slot
    assert call(n_cached=-1) == L.PGKQ_ERR_SHAPE
    assert call(k=MIS) == L.PGKQ_ERR_ALIGN
    assert call(v=MIS) == L.PGKQ_ERR_ALIGN
    assert call(wsb=16) == L.PGKQ_ERR_WORKSPACE


def test_value_cache_capacity_must_be_a_tile_multiple():
    """fp16 value caches come in 32-token tiles: every entry point that reads one
    rejects a capacity that is not a multiple of 32 (even ones included)."""
    assert _decode(cap=144, n_tok=100) == L.PGKQ_ERR_SHAPE
    assert _rtn_decode(cap=144) == L.PGKQ_ERR_SHAPE
    o = L.PgkqLaunchOpts(0, None, None)
    st = L.lib().pgkq_fp16_decode_attn(_vp(A), L.PGKQ_F32, 1, 4, 4, 10, 48, 64, _vp(A), _vp(A),
                                       _vp(A), 0.0, ctypes.byref(o), _vp(A), 1 << 20, None)
    assert st == L.PGKQ_ERR_SHAPE
    st = L.lib().pgkq_decode_step(_params(128, 3, 2, 128, 1), _vp(A), L.PGKQ_BF16, _vp(A), L.PGKQ_F16,
                                  _vp(A), 2, 8, 2, 99, 144, _vp(A), None, _vp(A), _vp(A), _vp(A),
                                  _vp(A), _vp(A), 0.0, ctypes.byref(o), _vp(A), 1 << 30, None)
    assert st == L.PGKQ_ERR_SHAPE


def test_decode_step_grid_rows_limit():
    """The preparation launch of a step holds n_q + n_kv grid rows: at most
    65535.  With 8 query heads per kv-head n_kv = 7282 gives 65538 rows and
    is rejected before anything is enqueued (n_q = 58256 alone is within the
    limit of a plain decode)."""
    o = L.PgkqLaunchOpts(0, None, None)

    def call(n_kv):
        return L.lib().pgkq_decode_step(_params(128, 3, 2, 128, 1), _vp(A), L.PGKQ_BF16, _vp(A),
                                        L.PGKQ_F16, _vp(A), 1, 8 * n_kv, n_kv, 99, 128, _vp(A), None,
                                        _vp(A), _vp(A), _vp(A), _vp(A), _vp(A), 0.0, ctypes.byref(o),
                                        _vp(A), 1 << 40, None)

    assert call(7282) == L.PGKQ_ERR_SHAPE


def test_pack_values_validation():
    lib = L.lib()

    def pack(rows=A, n_streams=4, T=50, d=128, cache=A, cap=64, off=0):
        return lib.pgkq_pack_values(_vp(rows) if rows else None, n_streams, T, d,
                                    _vp(cache) if cache else None, cap, off, None)

    def unpack(cache=A, n_streams=4, cap=64, d=128, off=0, T=50, rows=A):
        return lib.pgkq_unpack_values(_vp(cache) if cache else None, n_streams, cap, d, off, T,
                                      _vp(rows) if rows else None, None)

    for f in (pack, unpack):
        assert f(d=8) == L.PGKQ_ERR_UNSUPPORTED
        assert f(d=72) == L.PGKQ_ERR_UNSUPPORTED
        assert f(d=2048) == L.PGKQ_ERR_UNSUPPORTED
        assert f(cap=48) == L.PGKQ_ERR_SHAPE
        assert f(off=20) == L.PGKQ_ERR_SHAPE          # 20 + 50 > 64
        assert f(T=-1) == L.PGKQ_ERR_SHAPE
        assert f(n_streams=-1) == L.PGKQ_ERR_SHAPE
        assert f(cap=1 << 24) == L.PGKQ_ERR_SHAPE     # stream beyond the 32-bit buffer range
        assert f(rows=0) == L.PGKQ_ERR_NULL
        assert f(cache=0) == L.PGKQ_ERR_NULL
        assert f(T=0, rows=0, cache=0) == L.PGKQ_OK    # empty: nothing to move
        assert f(n_streams=0, rows=0, cache=0) == L.PGKQ_OK
        assert f(cache=MIS) == L.PGKQ_ERR_ALIGN       # the tiled side moves 16-byte pieces
        assert f(rows=A + 1) == L.PGKQ_ERR_ALIGN      # fp16 rows: 2-byte aligned


# ------------------------------------------------------------------ binding size checks
# The C ABI sees pointers only, so the binding checks that a code buffer and a
# value cache agree with the sizes the call implies, before anything is launched
# (CPU tensors here: a passing check would only fail later, at the device-pointer
# step, with a different message).

def test_binding_rejects_mismatched_code_and_value_buffers():
    import torch
    p = api.PgkqParams(64, 3, 2, 64)
    rb = api.pgkq_record_bytes(p)
    n_seq, n_kv, n_q, d, cap = 2, 3, 6, 64, 64
    q = torch.zeros((n_seq, n_q, d))
    V = torch.zeros((n_seq, n_kv, cap, d), dtype=torch.float16)
    good = torch.zeros((n_seq, n_kv, cap * rb), dtype=torch.uint8)
    short = torch.zeros((n_seq, n_kv, (cap - 32) * rb), dtype=torch.uint8)
    with pytest.raises(ValueError, match="codes: .* bytes"):
        api.pgkq_decode_attn(p, q, short, V, None, None, None, None)
    with pytest.raises(ValueError, match="V: shape"):
        api.pgkq_decode_attn(p, q, good, V[:, :, :, :32].contiguous(), None, None, None, None)
    with pytest.raises(ValueError, match="codes: .* bytes"):
        api.pgkq_estimate_logits(p, q, short, n_kv, cap, None, None, None, None)
    with pytest.raises(ValueError, match="k_new: shape"):
        api.pgkq_decode_step(p, q, torch.zeros((n_seq, n_kv + 1, d)), torch.zeros((n_seq, n_kv, d)),
                             good, V, 0, None, None, None, None)
    with pytest.raises(ValueError, match="codes: .* bytes"):
        api.pgkq_decode_step(p, q, torch.zeros((n_seq, n_kv, d)),
                             torch.zeros((n_seq, n_kv, d), dtype=torch.float16), short, V, 0,
                             None, None, None, None)
    K = torch.zeros((n_seq, n_kv, 40, d))
    with pytest.raises(ValueError, match="codes: .* bytes"):
        api.pgkq_encode(p, K, None, None, None, None, codes=short, capacity=cap)
    with pytest.raises(ValueError, match="whole number"):
        api.pgkq_encode(p, K, None, None, None, None, codes=good[:, :, :-1].contiguous())
    pv = api.PgkqParams(64, 3, 2, 64, 0)
    with pytest.raises(ValueError, match="codes_v: .* bytes"):
        api.pgkq_kv_decode_attn(p, pv, q, good, short, n_kv, cap, None, None, None, None, None, None)
    rtn_rb = api.pgkq_rtn_record_bytes(d, 4)
    with pytest.raises(ValueError, match="codes: .* bytes"):
        api.pgkq_rtn_decode_attn(q, torch.zeros((n_seq, n_kv, cap * rtn_rb - 4), dtype=torch.uint8),
                                 V, 4)
    with pytest.raises(ValueError, match="K16: shape"):
        api.pgkq_fp16_decode_attn(q, torch.zeros((n_seq, n_kv, cap, 32), dtype=torch.float16), V)


def test_binding_default_capacity_matches_the_value_cache():
    # the key-code default and the value-cache default agree for ragged lengths
    for T in (1, 31, 32, 33, 100, 512):
        assert api.default_capacity(T) % 32 == 0
        assert api.default_capacity(T) >= T
        assert api.default_capacity(T) - T < 32 or T < 32


# ------------------------------------------------------------------ decode without allocation

def _decode_noalloc(p=(128, 3, 2, 128, 1), q=A, n_seq=2, n_q=8, n_kv=2, n_tok=100, cap=128,
                    signs=A, cb=A, S=A, codes=A, V=A, out=A, n_splits=0):
    o = L.PgkqLaunchOpts(n_splits, None, None)
    return L.lib().pgkq_decode_attn_noalloc(_params(*p), _vp(q) if q else None, L.PGKQ_BF16, n_seq,
                                            n_q, n_kv, n_tok, cap, _vp(signs), None, _vp(cb),
                                            _vp(S) if S else None, _vp(codes) if codes else None,
                                            _vp(V) if V else None, _vp(out) if out else None, 0.0,
                                            ctypes.byref(o), None)


def test_decode_noalloc_validation_before_any_device_call():
    assert _decode_noalloc(q=0) == L.PGKQ_ERR_NULL
    assert _decode_noalloc(out=0) == L.PGKQ_ERR_NULL
    assert _decode_noalloc(V=0) == L.PGKQ_ERR_NULL
    assert _decode_noalloc(n_q=6) == L.PGKQ_ERR_UNSUPPORTED
    assert _decode_noalloc(n_tok=129) == L.PGKQ_ERR_SHAPE
    assert _decode_noalloc(out=MIS) == L.PGKQ_ERR_ALIGN
    # a call whose workspace would exceed the built-in scratch is refused
    p = api.PgkqParams(128, 3, 2, 128)
    need = api.pgkq_decode_workspace_bytes(p, 64, 32, 8, 32768, 16)
    assert need > L.PGKQ_NOALLOC_SCRATCH_BYTES
    assert _decode_noalloc(n_seq=64, n_q=32, n_kv=8, n_tok=32768, cap=32768,
                           n_splits=16) == L.PGKQ_ERR_WORKSPACE
    # the benchmark's 32k-token cache fits
    assert api.pgkq_decode_workspace_bytes(p, 16, 32, 8, 32768, 8) <= L.PGKQ_NOALLOC_SCRATCH_BYTES


def test_noalloc_scratch_size_matches_the_header():
    src = open(HEADER).read()
    m = re.search(r"#define PGKQ_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == L.PGKQ_NOALLOC_SCRATCH_BYTES


def test_stream_read_validation():
    lib = L.lib()
    assert lib.pgkq_stream_read(None, 0, None, None) == L.PGKQ_OK        # empty read: no-op
    assert lib.pgkq_stream_read(None, 16, _vp(A), None) == L.PGKQ_ERR_NULL
    assert lib.pgkq_stream_read(_vp(A), 16, None, None) == L.PGKQ_ERR_NULL
    assert lib.pgkq_stream_read(_vp(A), 24, _vp(A), None) == L.PGKQ_ERR_SHAPE   # not 16-byte rows
    assert lib.pgkq_stream_read(_vp(A), (1 << 39) + 16, _vp(A), None) == L.PGKQ_ERR_SHAPE
    assert lib.pgkq_stream_read(_vp(MIS), 16, _vp(A), None) == L.PGKQ_ERR_ALIGN
    assert lib.pgkq_stream_read(_vp(A), 16, _vp(A + 2), None) == L.PGKQ_ERR_ALIGN


@pytest.mark.parametrize("n_seq,n_kv", [(1, 1), (1, 8), (16, 8), (64, 24), (200, 8)])
def test_workspace_planning_sweep(n_seq, n_kv):
    """Workspace sizes over token counts from 1 to 2^31 and requested split
    counts from automatic to 4096: never zero for a valid shape, never smaller
    than the query preparation plus one partial state per split actually used,
    and monotone in the requested split count beyond the automatic plan."""
    p = api.PgkqParams(128, 3, 2, 128)
    n_q = 4 * n_kv
    prep = n_seq * n_q * ((128 + 64 * 4 + 128 + 3) // 4 * 4) * 4
    for T in (1, 63, 64, 65, 511, 4096, 32768, 131072, 1 << 31):
        for ns in (0, 1, 2, 7, 8, 64, 256, 4096):
            w = api.pgkq_decode_workspace_bytes(p, n_seq, n_q, n_kv, T, n_splits=ns)
            assert w >= prep, (T, ns, w)
            if ns == 1 and T <= 1 << 18:
                assert w < prep + 256, (T, w)   # one split: no partial states
            if ns == 1 and T > 1 << 18:
                # a split holds at most 2^18 tokens: the request is raised
                n = -(-T // (1 << 18))
                assert w >= prep + n_seq * n_q * n * (128 + 4) * 4, (T, w)
            wk = api.pgkq_kv_decode_workspace_bytes(p, api.PgkqParams(128, 3, 2, 128, 0),
                                                    n_seq, n_q, n_kv, T, n_splits=ns)
            assert wk >= prep, (T, ns, wk)
            wf = api.pgkq_fp16_decode_workspace_bytes(128, n_seq, n_q, n_kv, T, n_splits=ns)
            wr = api.pgkq_rtn_decode_workspace_bytes(128, n_seq, n_q, n_kv, T, n_splits=ns)
            assert wf >= 0 and wr > 0


def test_host_check_build_launches_only_valid_calls():
    """Against the host-check build of the ABI layer (a stand-in device layer
    that validates each argument block and counts the calls, launching
    nothing): invalid calls reach no device call, and valid decode, encode and
    logits calls over a range of shapes hand the device layer consistent plans.
    The product library has no stand-in, so this test needs the host-check
    build (tests/test_host_sanitized.py runs it there)."""
    lib = L.lib()
    if not hasattr(lib, "pgkq_hostcheck_calls"):
        pytest.skip("needs the host-check build of the ABI layer")
    calls = lib.pgkq_hostcheck_calls
    calls.restype = ctypes.c_int
    c0 = calls()
    assert _decode(q=0) == L.PGKQ_ERR_NULL
    assert _decode(n_q=6) == L.PGKQ_ERR_UNSUPPORTED
    assert _decode(wsb=16) == L.PGKQ_ERR_WORKSPACE
    assert _encode(n_tok=17) == L.PGKQ_ERR_SHAPE
    assert _encode(K=MIS) == L.PGKQ_ERR_ALIGN
    assert calls() == c0
    for n_seq, n_kv, grp, T, ns in [(1, 8, 4, 131072, 0), (16, 8, 4, 32768, 8), (2, 2, 1, 100, 0),
                                    (2, 2, 1, 100, 1), (3, 1, 8, 5000, 7), (1, 4, 2, 64, 4096)]:
        cap = (T + 31) // 32 * 32
        n_q = grp * n_kv
        p = api.PgkqParams(128, 3, 2, 128)
        need = api.pgkq_decode_workspace_bytes(p, n_seq, n_q, n_kv, T, n_splits=ns)
        c1 = calls()
        assert _decode(n_seq=n_seq, n_q=n_q, n_kv=n_kv, n_tok=T, cap=cap, wsb=need,
                       n_splits=ns) == L.PGKQ_OK
        assert calls() > c1
    assert _encode(n_tok=16) == L.PGKQ_OK
    # the logit hook at a code stream of 58 040 098 74-byte records (4.0 GiB):
    # accepted, while decode attention needs the value rows to fit as well
    cap = 0xFFFFFFF0 // 74 // 2 * 2
    c1 = calls()
    st = lib.pgkq_estimate_logits(_params(128, 4, 3, 128, 1), _vp(A), L.PGKQ_F32, 1, 4, 1, cap, cap,
                                  _vp(A), None, _vp(A), _vp(A), _vp(A), _vp(A), _vp(A), 1 << 30, None)
    assert st == L.PGKQ_OK and calls() > c1
    cap32 = cap // 32 * 32   # a whole number of value tiles: rejected for the value range only
    assert _decode(p=(128, 4, 3, 128, 1), n_seq=1, n_q=4, n_kv=1, n_tok=cap32, cap=cap32,
                   wsb=1 << 30) == L.PGKQ_ERR_SHAPE


def test_split_count_beyond_the_grid_is_rejected():
    # 16 777 184 tokens at one partition per 256 tokens: 65 536 splits, one more
    # than a grid dimension holds
    cap = (1 << 24) - 32
    p = api.PgkqParams(64, 3, 2, 64)
    assert _decode(p=(64, 3, 2, 64, 1), n_seq=1, n_q=2, n_kv=2, n_tok=cap, cap=cap,
                   n_splits=1 << 20) == L.PGKQ_ERR_SHAPE
    assert api.pgkq_decode_workspace_bytes(p, 1, 2, 2, cap, n_splits=1 << 20) > 0
