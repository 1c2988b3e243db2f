"""Seeded synthetic inputs for the PGKQ encode/decode path.

This package holds only input generation (random draws and dtype rounding of
those draws).  It contains none of the method's arithmetic, so both the HIP
path and the CPU oracle may take their inputs from it without sharing code.
"""

from .inputs import (  # noqa: F401
    CONFIGS,
    WorkloadConfig,
    bf16_round,
    make_inputs,
    stream_keys,
    stream_values,
)
