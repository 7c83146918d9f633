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
    PA_F16,
    PA_F32,
    PA_INT8,
    PaError,
    PaPool,
    load,
    pa_copy_blocks,
    pa_decode,
    pa_decode_static,
    pa_decode_int8,
    pa_decode_int8_workspace_bytes,
    pa_decode_order,
    pa_decode_workspace_bytes,
    pa_gather_kv,
    pa_prefill_varlen,
    pa_prefill_varlen_int8,
    pa_prefill_workspace_bytes,
    pa_store_kv,
    pa_store_kv_int8,
    pool_desc,
    pool_desc_int8,
    validate_decode_metadata,
    validate_prefill_metadata,
)
