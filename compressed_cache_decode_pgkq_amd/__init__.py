"""PGKQ compressed-key cache for AMD Instinct MI355X (gfx950).

Encode (randomized Hadamard transform, polar codes, QJL residual sketch) and
analytic decode attention over the codes, as hand-written HIP kernels behind
the C ABI of ``include/pgkq.h`` (``libpgkq.so``).  This package holds the build
script and a thin PyTorch/ctypes binding whose functions carry the names of the
C entry points.
"""

from .api import (  # noqa: F401
    PgkqParams,
    pgkq_calibrate,
    pgkq_calibrate_workspace_bytes,
    pgkq_codes_bytes,
    pgkq_decode_attn,
    pgkq_decode_attn_noalloc,
    pgkq_decode_step,
    pgkq_decode_workspace_bytes,
    pgkq_encode,
    pgkq_estimate_logits,
    pgkq_fp16_decode_attn,
    pgkq_fp16_decode_workspace_bytes,
    pgkq_kv_decode_attn,
    pgkq_kv_decode_workspace_bytes,
    pgkq_lloyd_max_beta,
    pgkq_lloyd_max_empirical,
    pgkq_pack_values,
    pgkq_record_bytes,
    pgkq_rtn_decode_attn,
    pgkq_rtn_decode_workspace_bytes,
    pgkq_rtn_encode,
    pgkq_rtn_logits,
    pgkq_rtn_record_bytes,
    pgkq_status_string,
    pgkq_stream_read,
    pgkq_unpack_values,
    pgkq_version,
)
from ._lib import PgkqError  # noqa: F401
