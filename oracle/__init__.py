"""fp64 CPU oracle for masked bidirectional attention.

Test infrastructure only: imported by the tests, the smoke check and the
CPU-baseline leg of the bench, never by the library.  See ``mzref``.
"""
from .mzref import (  # noqa: F401
    attend,
    decode,
    decode_bf16,
    decode_fp16,
    decode_fp32,
    live_set_fwd,
    mzref_decode,
    mzref_decode_append,
    rms_norm,
    rope_cos_sin,
    round_bf16,
    mzref_fwd,
    parity_stats,
    rope_interleaved,
    rope_inv_freq,
    segment_positions,
    within_tolerance,
)
