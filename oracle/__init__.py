"""CPU reference (oracle) for single-precision GEMM.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the package smoke check
and the benchmark's CPU-baseline leg, never by the HIP library's code path.
"""

from .oracle import (  # noqa: F401
    OracleResult,
    load,
    normalised_error,
    oracle_sgemm,
    oracle_threads,
)
