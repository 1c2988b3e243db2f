"""ctypes declarations of the PGKQ C ABI (include/pgkq.h).

Loads ``libpgkq.so`` from this package directory.  There is no fallback: if
the library has not been built the import of any entry point raises.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# PGKQ_LIB names another build of the same ABI (the sanitized host-only build
# of the validation layer that the CPU tests load); unset, the in-tree library.
LIB_PATH = os.environ.get("PGKQ_LIB") or os.path.join(_HERE, "libpgkq.so")

PGKQ_OK = 0
PGKQ_ERR_NULL = 1
PGKQ_ERR_SHAPE = 2
PGKQ_ERR_UNSUPPORTED = 3
PGKQ_ERR_ALIGN = 4
PGKQ_ERR_WORKSPACE = 5
PGKQ_ERR_HIP = 6

PGKQ_NOALLOC_SCRATCH_BYTES = 8 << 20

PGKQ_F32 = 0
PGKQ_F16 = 1
PGKQ_BF16 = 2


class PgkqParams(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("b_main", ctypes.c_int32),
                ("b_angle", ctypes.c_int32), ("qjl_m", ctypes.c_int32),
                ("hadamard", ctypes.c_int32)]


class PgkqLaunchOpts(ctypes.Structure):
    _fields_ = [("n_splits", ctypes.c_int32), ("scan_start", ctypes.c_void_p),
                ("scan_stop", ctypes.c_void_p)]


class PgkqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None

_P = ctypes.POINTER(PgkqParams)
_O = ctypes.POINTER(PgkqLaunchOpts)
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_f32 = ctypes.c_float

SIGNATURES = {
    "pgkq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pgkq_version": (ctypes.c_char_p, []),
    "pgkq_record_bytes": (_sz, [_P]),
    "pgkq_codes_bytes": (_sz, [_P, _i64, _i64]),
    "pgkq_lloyd_max_beta": (ctypes.c_int, [_i32, _i32, ctypes.POINTER(ctypes.c_double),
                                           ctypes.POINTER(ctypes.c_double)]),
    "pgkq_lloyd_max_empirical": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double), _i64, _i32,
                                                ctypes.POINTER(ctypes.c_double),
                                                ctypes.POINTER(ctypes.c_double)]),
    "pgkq_pack_values": (ctypes.c_int, [_vp, _i64, _i64, _i32, _vp, _i64, _i64, _vp]),
    "pgkq_unpack_values": (ctypes.c_int, [_vp, _i64, _i64, _i32, _i64, _i64, _vp, _vp]),
    "pgkq_calibrate_workspace_bytes": (_sz, [_P, _i64, _i64, _i64]),
    "pgkq_calibrate": (ctypes.c_int, [_P, _vp, ctypes.c_int, _i64, _i64, _i64, _i32, _vp, _vp, _vp,
                                      _vp, _sz, _vp]),
    "pgkq_encode": (ctypes.c_int, [_P, _vp, ctypes.c_int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp,
                                   _i64, _i64, _vp]),
    "pgkq_decode_workspace_bytes": (_sz, [_P, _i64, _i64, _i64, _i64, _O]),
    "pgkq_decode_attn": (ctypes.c_int, [_P, _vp, ctypes.c_int, _i64, _i64, _i64, _i64, _i64, _vp,
                                        _vp, _vp, _vp, _vp, _vp, _vp, _f32, _O, _vp, _sz, _vp]),
    "pgkq_decode_attn_noalloc": (ctypes.c_int, [_P, _vp, ctypes.c_int, _i64, _i64, _i64, _i64, _i64,
                                                _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _O, _vp]),
    "pgkq_decode_step": (ctypes.c_int, [_P, _vp, ctypes.c_int, _vp, ctypes.c_int, _vp, _i64, _i64,
                                        _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _O,
                                        _vp, _sz, _vp]),
    "pgkq_estimate_logits": (ctypes.c_int, [_P, _vp, ctypes.c_int, _i64, _i64, _i64, _i64, _i64,
                                            _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "pgkq_fp16_decode_workspace_bytes": (_sz, [_i32, _i64, _i64, _i64, _i64, _O]),
    "pgkq_fp16_decode_attn": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _i64, _i64, _i32,
                                             _vp, _vp, _vp, _f32, _O, _vp, _sz, _vp]),
    "pgkq_kv_decode_workspace_bytes": (_sz, [_P, _P, _i64, _i64, _i64, _i64, _O]),
    "pgkq_kv_decode_attn": (ctypes.c_int, [_P, _P, _vp, ctypes.c_int, _i64, _i64, _i64, _i64, _i64,
                                           _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _O,
                                           _vp, _sz, _vp]),
    "pgkq_rtn_record_bytes": (_sz, [_i32, _i32]),
    "pgkq_rtn_encode": (ctypes.c_int, [_i32, _i32, _vp, ctypes.c_int, _i64, _i64, _i64, _vp, _i64,
                                       _i64, _vp]),
    "pgkq_rtn_decode_workspace_bytes": (_sz, [_i32, _i64, _i64, _i64, _i64, _O]),
    "pgkq_rtn_decode_attn": (ctypes.c_int, [_i32, _i32, _vp, ctypes.c_int, _i64, _i64, _i64, _i64,
                                            _i64, _vp, _vp, _vp, _f32, _O, _vp, _sz, _vp]),
    "pgkq_rtn_logits": (ctypes.c_int, [_i32, _i32, _vp, ctypes.c_int, _i64, _i64, _i64, _i64, _i64,
                                       _vp, _vp, _vp, _sz, _vp]),
    "pgkq_stream_read": (ctypes.c_int, [_vp, ctypes.c_uint64, _vp, _vp]),
}


def lib():
    """The loaded library (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"PGKQ HIP library not built: {LIB_PATH} is missing "
                "(run python -m compressed_cache_decode_pgkq_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    try:
        return lib().pgkq_status_string(int(status)).decode()
    except ImportError:
        return f"status {status}"


def check(status: int, where: str):
    if status != PGKQ_OK:
        raise PgkqError(status, where)
