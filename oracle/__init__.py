"""fp64 CPU oracle for the WKV-7 recurrence.

Test infrastructure only: imported by tests/, by the package smoke check and
by the benchmark's CPU-baseline leg, never by the product path.
"""
from .wkv7_oracle import (  # noqa: F401
    as_f64, decay_from_logneglog, wkv7_forward, wkv7_brute, wkv7_unrolled, wkv7_chunked,
)
