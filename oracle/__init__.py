"""fp64 CPU oracle for the attention forward.

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the product path.
"""

from .attention import (  # noqa: F401
    backward,
    backward_dkdv_rows,
    backward_dq_rows,
    decode,
    decode_split,
    kv_head,
    prefill,
    prefill_lse,
    prefill_lse_rows,
    prefill_rows,
)
