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
    return set(re.findall(r"^\S.*?\b(pa_[a-z0-9_]+)\s*\(", text, flags=re.M))


def test_header_declares_what_the_binding_expects():
    assert _declared_symbols() == set(pa.EXPORTS)


def test_library_loads_and_exports_every_symbol():
    lib = pa.load()
    for name in _declared_symbols():
        assert hasattr(lib, name), name
    assert lib.pa_abi_version() == 6
    assert lib.pa_status_string(0) == b"ok"
    assert b"workspace" in lib.pa_status_string(5)


def test_library_exports_exactly_the_header():
    """The dynamic symbol table of libpa.so defines the C entry points that
    include/pa.h declares and no other symbol (no helper, no C++ name)."""
    import subprocess
    res = subprocess.run(["nm", "-D", "--defined-only", pa.LIB_PATH], capture_output=True, text=True,
                         check=True)
    exported = set()
    for line in res.stdout.splitlines():
        parts = line.split()
        if len(parts) == 3 and parts[1] in "TtDdBbRrVvWwiu" and not parts[2].startswith("PA_"):
            exported.add(parts[2])
    assert exported == _declared_symbols(), sorted(exported ^ _declared_symbols())


def _pool(nb=4, bs=16, hkv=2, d=32, dtype=pa.PA_F32):
    return pa.PaPool(nb, bs, hkv, d, dtype)


def test_int8_store_host_errors():
    """pa_store_kv_int8 takes PA_INT8 pools only (and the bf16/fp32 calls
    refuse them), bf16, fp16 or fp32 sources, head_dim a power of two from 8 to 256
    (the lanes of a head vector reduce its max |x| as one group)."""
    lib = pa.load()
    i8 = _pool(d=128, dtype=pa.PA_INT8)
    dummy = ctypes.c_void_p(4096)
    args = [dummy, 256, dummy, 256, pa.PA_BF16, dummy, 3, dummy, dummy, dummy, dummy, ctypes.byref(i8), None]
    a = list(args); a[11] = ctypes.byref(_pool(d=128, dtype=pa.PA_BF16))
    assert lib.pa_store_kv_int8(*a) == 3                       # pool not INT8
    a = list(args); a[4] = pa.PA_INT8
    assert lib.pa_store_kv_int8(*a) == 3                       # source must be bf16 / fp16 / fp32
    for d in (36, 24, 40, 48, 96, 4, 512):
        a = list(args); a[11] = ctypes.byref(_pool(d=d, dtype=pa.PA_INT8))
        assert lib.pa_store_kv_int8(*a) == 4, d                # head_dim not a power of two in 8..256
    a = list(args); a[6] = 0
    assert lib.pa_store_kv_int8(*a) == 0                       # no tokens: no-op
    a = list(args); a[9] = None
    assert lib.pa_store_kv_int8(*a) == 1                       # scale pool missing
    a = list(args); a[1] = 100
    assert lib.pa_store_kv_int8(*a) == 2                       # row stride < Hkv * D
    a = list(args); a[8] = ctypes.c_void_p(4100)
    assert lib.pa_store_kv_int8(*a) == 4                       # code pool not 8-byte aligned
    assert lib.pa_store_kv(dummy, 256, dummy, 256, dummy, 1, dummy, dummy, ctypes.byref(i8), None) == 3


def test_int8_decode_host_errors_and_workspace():
    """pa_decode_int8 takes PA_INT8 pools, q of bf16 / fp16 / fp32, query
    groups of 1, 2, 4 or 8; its workspace follows the same split plan as
    pa_decode."""
    lib = pa.load()
    dummy = ctypes.c_void_p(4096)
    i8 = _pool(nb=64, bs=16, hkv=8, d=128, dtype=pa.PA_INT8)
    def call(pool, hq=16, qd=pa.PA_BF16, n=4, scale=0.1, ws=None, wsb=0, max_ctx=100):
        return lib.pa_decode_int8(dummy, hq * 128, hq, qd, dummy, dummy, dummy, dummy, ctypes.byref(pool),
                                  dummy, dummy, 8, n, max_ctx, scale, None, dummy, ws, wsb, None)
    assert call(_pool(nb=64, bs=16, hkv=8, d=128, dtype=pa.PA_BF16)) == 3   # pool not INT8
    assert call(i8, qd=pa.PA_INT8) == 3                                      # q must be bf16 / fp32
    assert call(i8, hq=128) == 4                                             # group 16 is not built
    assert call(i8, hq=12) == 2                                              # not a multiple of Hkv
    assert call(i8, scale=0.0) == 2
    assert call(i8, n=0) == 0
    assert lib.pa_decode(dummy, 16 * 128, 16, dummy, dummy, ctypes.byref(i8), dummy, dummy, 8, 4, 100, 0.1,
                         None, dummy, None, 0, None) == 3                    # bf16 decode refuses INT8 pools
    # one long row splits: a workspace is required and sized like pa_decode's fp32 partials
    need = lib.pa_decode_int8_workspace_bytes(1, 16, 1 << 16, ctypes.byref(i8))
    assert need > 0 and need % (16 * (128 + 2) * 4) == 0
    assert call(i8, n=1, max_ctx=1 << 16) == 5                             # split plan, no workspace given
    assert lib.pa_decode_int8_workspace_bytes(256, 16, 2048, ctypes.byref(i8)) == 0


def test_int8_prefill_host_errors():
    lib = pa.load()
    dummy = ctypes.c_void_p(4096)
    i8 = _pool(nb=64, bs=16, hkv=8, d=128, dtype=pa.PA_INT8)
    def call(pool, hq=16, qd=pa.PA_BF16, n=2, tq=10, scale=0.1):
        return lib.pa_prefill_varlen_int8(dummy, hq * 128, hq, qd, dummy, dummy, dummy, dummy, ctypes.byref(pool),
                                          dummy, dummy, dummy, dummy, 8, n, tq, 5, 5, scale, dummy, None, 0, None)
    assert call(_pool(nb=64, bs=16, hkv=8, d=128, dtype=pa.PA_BF16)) == 3
    assert call(i8, qd=7) == 3
    assert call(i8, hq=128) == 4
    assert call(i8, scale=-1.0) == 2
    assert call(i8, n=0) == 0 and call(i8, tq=0) == 0
    assert lib.pa_prefill_varlen(dummy, 16 * 128, 16, dummy, dummy, ctypes.byref(i8), dummy, dummy, dummy, dummy,
                                 8, 2, 10, 5, 5, 0.1, dummy, None, 0, None) == 3


def test_f16_pools_and_queries_pass_the_dtype_checks():
    """PA_F16 pools and fp16 INT8 sources / queries get past the element-type
    check and stop at the next one (a null pointer), before any launch."""
    lib = pa.load()
    f16 = _pool(nb=8, bs=16, hkv=2, d=64, dtype=pa.PA_F16)
    assert lib.pa_store_kv(None, 128, None, 128, None, 1, None, None, ctypes.byref(f16), None) == 1
    assert lib.pa_gather_kv(None, None, ctypes.byref(f16), None, None, 1, 1, 1, None, None, None) == 1
    assert lib.pa_decode(None, 128, 2, None, None, ctypes.byref(f16), None, None, 1, 1, 1, 0.1, None, None,
                         None, 0, None) == 1
    assert lib.pa_decode_workspace_bytes(64, 16, 32768, ctypes.byref(_pool(nb=1, hkv=8, d=128,
                                                                           dtype=pa.PA_F16))) > 0
    i8 = _pool(d=128, dtype=pa.PA_INT8)
    dummy = ctypes.c_void_p(4096)
    assert lib.pa_store_kv_int8(dummy, 256, dummy, 256, pa.PA_F16, dummy, 3, dummy, dummy, None, dummy,
                                ctypes.byref(i8), None) == 1
    assert lib.pa_decode_int8(None, 256, 4, pa.PA_F16, None, None, None, None, ctypes.byref(i8), None, None, 1,
                              1, 1, 0.1, None, None, None, 0, None) == 1
    assert lib.pa_decode_int8(None, 256, 4, 9, None, None, None, None, ctypes.byref(i8), None, None, 1,
                              1, 1, 0.1, None, None, None, 0, None) == 3


def test_copy_blocks_host_errors():
    lib = pa.load()
    dummy = ctypes.c_void_p(4096)
    bf = _pool(dtype=pa.PA_BF16)
    i8 = _pool(dtype=pa.PA_INT8)
    assert lib.pa_copy_blocks(dummy, dummy, None, None, None, dummy, dummy, dummy, 1, None) == 1
    assert lib.pa_copy_blocks(dummy, dummy, None, None, ctypes.byref(_pool(dtype=9)), dummy, dummy, dummy, 1,
                              None) == 3
    assert lib.pa_copy_blocks(dummy, dummy, None, None, ctypes.byref(bf), dummy, dummy, dummy, -1, None) == 2
    assert lib.pa_copy_blocks(None, None, None, None, ctypes.byref(bf), None, None, None, 0, None) == 0
    assert lib.pa_copy_blocks(dummy, dummy, None, None, ctypes.byref(i8), dummy, dummy, dummy, 1, None) == 1
    assert lib.pa_copy_blocks(dummy, None, None, None, ctypes.byref(bf), dummy, dummy, dummy, 1, None) == 1


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
    # at most 65536 KV heads, and fewer than 2^31 (slot, head) rows per block
    for hkv, bs in ((65537, 1), (32768, 65536), (65536, 32768)):
        big = _pool(hkv=hkv, bs=bs)
        assert lib.pa_store_kv(None, 64, None, 64, None, 0, None, None, ctypes.byref(big), None) == 4, (hkv, bs)
        assert lib.pa_decode(None, 64, hkv, None, None, ctypes.byref(big), None, None, 1, 3, 10, 0.1,
                             None, None, None, 0, None) == 4, (hkv, bs)
    ok = _pool(hkv=65536, bs=16384)  # 2^30 rows per block: allowed
    assert lib.pa_store_kv(None, 64, None, 64, None, 0, None, None, ctypes.byref(ok), None) == 0
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


def test_split_plan_follows_the_documented_rule():
    """The decode workspace reveals the planned split slots per row: enough
    (row, KV head, split) workgroups for two rounds of resident workgroups
    (1024 at 8 waves), at least 16 rounds of keys (1024 at bf16, head_dim
    128) per split at max_context_len, none longer than the staged block ids
    allow.  Pure host arithmetic: nothing is launched."""
    lib = pa.load()

    def ws(rows, hq, max_ctx, **pool):
        p = _pool(**pool)
        return lib.pa_decode_workspace_bytes(rows, hq, max_ctx, ctypes.byref(p))

    per_split = 16 * (128 + 2) * 4                     # one row's partials for 16 query heads
    bf = dict(nb=64, bs=16, hkv=8, d=128, dtype=pa.PA_BF16)
    assert ws(256, 16, 2048, **bf) == 0                # 2048 units already fill the GPU: no split
    assert ws(64, 16, 32768, **bf) == 64 * 2 * per_split      # 512 units -> 2 splits
    assert ws(1, 16, 20000, **bf) == 1 * 20 * per_split       # min(128, ceil(20000 / 1024)) = 20
    assert ws(8, 16, 512, **bf) == 0                   # 512 keys < 16 rounds: one split
    assert ws(32, 16, 4096, **bf) == 32 * 4 * per_split       # min(4, 4) = 4
    # block size 1: a split may span at most 4095 block ids (4032 keys in whole rounds)
    one = dict(nb=1 << 20, bs=1, hkv=8, d=128, dtype=pa.PA_BF16)
    assert ws(256, 16, 1 << 20, **one) == 256 * (-(-(1 << 20) // 4032)) * per_split
