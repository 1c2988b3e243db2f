"""CPU oracle for PGKQ (polar-guided key-cache quantization) encode and
analytic decode attention.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 NumPy/SciPy
statement of what the PGKQ path computes, written from the EdgeLLM-Nano paper
page (signal-papers read view of arXiv 2610.14475, paragraphs "PGKQ pipeline",
the Lloyd-Max codebook paragraph after it, and "Bit budget").  Only the test
suite, the smoke check of ``__graft_entry__`` and the CPU-baseline leg of
``bench.py`` may import it.  It shares no code with the HIP library and never
imports it; the HIP library never imports this.

Modules
-------
codebook    Lloyd-Max radius codebook for the Beta prior, and its per-head scaling
rht         randomized Hadamard transform with a dense Sylvester matrix
calibrate   per-channel statistics, channel reorder (step 0), head scale
encode      per-key codes: radius code, angle code, QJL sign bits, residual norm
layout      bit-plane packing of the codes (and unpacking)
attn        analytic logits, softmax and FP16-V weighted sum, split/merge,
            the FP16-cache comparator and an explicit dequantizer
accounting  byte and bits-per-element accounting of the compressed cache
rtn         per-token asymmetric round-to-nearest key quantization (control):
            quantizer, record layout and decode attention
kv          PGKQ-KV: values coded by the key encoder without the transform,
            their reconstruction and decode attention

Parity pins live in ``tests/test_oracle_pins.py``.  Parity unpinned: the
absolute codebook values and the code values for any given input (the pages
print neither a codebook table nor a worked example); they are fixed only by the
readings stated in each module plus the invariants the tests check.
"""

from . import accounting, attn, calibrate, codebook, encode, kv, layout, rht, rtn  # noqa: F401
from .encode import Params  # noqa: F401
