"""CPU fp64 oracle for paged-KV attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by
the CPU-baseline leg of the benchmark.  The HIP library never imports,
links or calls anything here, and this package imports nothing from it.
"""
from .oracle import (  # noqa: F401
    build,
    lib_path,
    num_threads,
    set_num_threads,
    store_kv,
    gather_kv,
    prefill,
    decode,
    F32,
    BF16,
)
