"""Attention over a block-paged KV cache on AMD Instinct MI355X (gfx950).

The product is libpa.so, a C-ABI library of hand-written HIP kernels
(include/pa.h).  This package is its thin Python binding: the functions
below carry the same names as the C entry points and only marshal torch
tensors (device pointers, sizes, the current stream).
"""
from ._lib import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    PA_BF16,
    PA_F32,
    PaError,
    PaPool,
    load,
    pa_decode,
    pa_decode_order,
    pa_decode_workspace_bytes,
    pa_gather_kv,
    pa_prefill_varlen,
    pa_prefill_workspace_bytes,
    pa_store_kv,
    pool_desc,
    validate_decode_metadata,
    validate_prefill_metadata,
)
