"""CPU oracle for row-major SGEMM (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package; the GPU library never does.
"""
from .oracle import (  # noqa: F401
    Oracle,
    build_oracle,
    compile_oracle,
    default_oracle,
    oracle_threads,
    sgemm_rm_ref,
    sgemm_rm_ref_entries,
)
