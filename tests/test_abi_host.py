"""The C-ABI library on the CPU: it loads, exports every symbol include/pa.h
declares, and its pure-host paths (argument checks that return before any
launch, workspace sizing, metadata validators) behave as documented.  No
kernel is launched here."""
import ctypes
import os
import re

import numpy as np
import pytest

import paged_kv_attention_mapping_amd as pa
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "pa.h")).read()
    return set(re.findall(r"^\S.*?\b(pa_[a-z_]+)\s*\(", text, flags=re.M))


def test_header_declares_what_the_binding_expects():
    assert _declared_symbols() == set(pa.EXPORTS)


def test_library_loads_and_exports_every_symbol():
    lib = pa.load()
    for name in _declared_symbols():
        assert hasattr(lib, name), name
    assert lib.pa_abi_version() == 2
    assert lib.pa_status_string(0) == b"ok"
    assert b"workspace" in lib.pa_status_string(5)


def _pool(nb=4, bs=16, hkv=2, d=32, dtype=pa.PA_F32):
    return pa.PaPool(nb, bs, hkv, d, dtype)


def test_host_argument_errors_return_before_launch():
    lib = pa.load()
    pool = _pool()
    # null pool
    assert lib.pa_store_kv(None, 64, None, 64, None, 1, None, None, None, None) == 1
    # bad dtype
    bad = _pool(dtype=7)
    assert lib.pa_store_kv(None, 64, None, 64, None, 1, None, None, ctypes.byref(bad), None) == 3
    # null data with tokens
    assert lib.pa_store_kv(None, 64, None, 64, None, 1, None, None, ctypes.byref(pool), None) == 1
    # zero tokens is a no-op
    assert lib.pa_store_kv(None, 64, None, 64, None, 0, None, None, ctypes.byref(pool), None) == 0
    # block size must be a power of two
    odd = _pool(bs=12)
    assert lib.pa_store_kv(None, 64, None, 64, None, 0, None, None, ctypes.byref(odd), None) == 4
    # group size 3 is not built; head_dim 48 is not built
    args = [None, 96, 6, None, None, None, None, None, None, None, 1, 1, 1, 1, 1, 0.1, None, None, 0, None]
    args[5] = ctypes.byref(_pool(hkv=2))
    assert lib.pa_prefill_varlen(*args) == 4
    args[2], args[5] = 4, ctypes.byref(_pool(d=48))
    assert lib.pa_prefill_varlen(*args) == 4
    args[2], args[5] = 3, ctypes.byref(_pool(hkv=2))
    assert lib.pa_prefill_varlen(*args) == 2      # 3 % 2 != 0
    # decode: zero sequences is a no-op, nulls are rejected
    assert lib.pa_decode(None, 64, 4, None, None, ctypes.byref(pool), None, None, 1, 0, 0, 0.1,
                         None, None, None, 0, None) == 0
    assert lib.pa_decode(None, 64, 4, None, None, ctypes.byref(pool), None, None, 1, 3, 10, 0.1,
                         None, None, None, 0, None) == 1
    # decode order: no-op, nulls, negative and too many rows
    assert lib.pa_decode_order(None, 0, None, None) == 0
    assert lib.pa_decode_order(None, 5, None, None) == 1
    assert lib.pa_decode_order(None, -1, None, None) == 2
    dummy = ctypes.c_void_p(16)  # never dereferenced: the size check comes first
    assert lib.pa_decode_order(dummy, 2049, dummy, None) == 4
    # the softmax scale must be finite and positive (checked before any pointer)
    for scale in (0.0, -0.1, float("inf"), float("nan")):
        assert lib.pa_decode(None, 64, 4, None, None, ctypes.byref(pool), None, None, 1, 3, 10, scale,
                             None, None, None, 0, None) == 2
        args = [None, 64, 4, None, None, ctypes.byref(pool), None, None, None, None, 1, 1, 1, 1, 1, scale,
                None, None, 0, None]
        assert lib.pa_prefill_varlen(*args) == 2


def test_workspace_sizes_follow_the_split_plan():
    lib = pa.load()
    c5b = pa.PaPool(131088, 16, 8, 128, pa.PA_BF16)
    n = lib.pa_decode_workspace_bytes(64, 16, 32768, ctypes.byref(c5b))
    assert n > 0 and n % (130 * 4) == 0
    # one short sequence needs no partials only if a single split covers it
    small = pa.PaPool(4, 16, 2, 32, pa.PA_F32)
    assert lib.pa_decode_workspace_bytes(0, 4, 10, ctypes.byref(small)) == 0


def test_validators_accept_generated_metadata():
    for case in (W.c2_varlen(32, with_values=False), W.c3_prefix(with_values=False),
                 W.c5a_mixed(with_values=False)):
        pool = pa.PaPool(case.num_blocks, case.block_size, case.num_kv_heads, case.head_dim, pa.PA_BF16)
        pa.validate_prefill_metadata(case.cu_seqlens_q, case.cu_seqlens_k, case.q_offsets,
                                     case.block_table, case.max_seqlen_q, case.max_seqlen_k, pool,
                                     np.concatenate([case.slot_cached, case.slot_new]))
    dec = W.c4_decode_layout()
    pool = pa.PaPool(dec.num_blocks, dec.block_size, dec.num_kv_heads, dec.head_dim, pa.PA_BF16)
    pa.validate_decode_metadata(dec.context_lens, dec.block_table, dec.max_context_len, pool, dec.slot_new,
                                row_order=np.argsort(-dec.context_lens, kind="stable"))


def test_validators_reject_bad_metadata():
    case = W.c3_prefix(with_values=False)
    pool = pa.PaPool(case.num_blocks, case.block_size, case.num_kv_heads, case.head_dim, pa.PA_BF16)
    bt = case.block_table.copy()
    bt[1, 0] = case.num_blocks  # out of range
    with pytest.raises(pa.PaError, match="out of range"):
        pa.validate_prefill_metadata(case.cu_seqlens_q, case.cu_seqlens_k, case.q_offsets, bt,
                                     case.max_seqlen_q, case.max_seqlen_k, pool)
    with pytest.raises(pa.PaError, match="q_offset"):
        pa.validate_prefill_metadata(case.cu_seqlens_q, case.cu_seqlens_k, [255, 256], case.block_table,
                                     case.max_seqlen_q, case.max_seqlen_k, pool)
    dup = np.concatenate([case.slot_new, case.slot_new[:1]])
    with pytest.raises(pa.PaError, match="twice"):
        pa.validate_prefill_metadata(case.cu_seqlens_q, case.cu_seqlens_k, case.q_offsets,
                                     case.block_table, case.max_seqlen_q, case.max_seqlen_k, pool, dup)
    dec = W.c4_decode_layout()
    pool = pa.PaPool(dec.num_blocks, dec.block_size, dec.num_kv_heads, dec.head_dim, pa.PA_BF16)
    with pytest.raises(pa.PaError, match="context_lens"):
        pa.validate_decode_metadata(dec.context_lens, dec.block_table, 1000, pool)
    order = np.arange(len(dec.context_lens))
    order[3] = order[4]  # a repeated row (and a missing one)
    with pytest.raises(pa.PaError, match="row_order"):
        pa.validate_decode_metadata(dec.context_lens, dec.block_table, dec.max_context_len, pool,
                                    row_order=order)
