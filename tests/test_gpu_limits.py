"""Limits of the supported shapes on the GPU, against the fp64 oracle: the
largest block size (65536 tokens per block, contexts across block
boundaries), the widest head with the largest group (d 256, 8 query heads per
KV head), a decode batch of 4096 rows (more than a row order covers),
empty batches, and broken metadata kept inside the buffers."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_mapping_amd as pa
import workloads as W
from helpers import host_pools_with_prefix, max_abs_err, say, to_dev, to_host_bits, tol

pytestmark = pytest.mark.gpu


def _decode(case, row_order=True):
    kp, vp = case.empty_pools()
    oracle.store_kv(case.k_hist, case.v_hist, case.slot_hist, kp, vp)
    kd, vd = to_dev(kp), to_dev(vp)
    pa.pa_store_kv(to_dev(case.k_new), to_dev(case.v_new), to_dev(case.slot_new), kd, vd)
    oracle.store_kv(case.k_new, case.v_new, case.slot_new, kp, vp)
    ctx = to_dev(case.context_lens)
    order = pa.pa_decode_order(ctx) if row_order else None
    out = pa.pa_decode(to_dev(case.q), kd, vd, ctx, to_dev(case.block_table), case.max_context_len, case.scale,
                       row_order=order)
    torch.cuda.synchronize()
    return out, kp, vp


def test_block_size_65536_decode_and_prefill():
    """Blocks of 65536 tokens: rows of 70000 and 65536 keys (across and at a
    block boundary) decode; a 96-token chunk after a 69904-token prefix
    prefills on the matrix cores (every row)."""
    bs = 65536
    dec = W.make_decode("bs64k", 9400, [70000, 65536, 3], 4, 2, 128, bs, "bf16", num_spare=1)
    say("[limits] decode, block size 65536")
    out, kp, vp = _decode(dec)
    ref = oracle.decode(dec.q, kp, vp, dec.context_lens, dec.block_table, dec.scale)
    err = max_abs_err(out, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol("bf16")

    pf = W.make_prefill("bs64k_pf", 9401, [96], [69904], 4, 2, 128, bs, "bf16", num_spare=1)
    say("[limits] prefill, block size 65536, 96 rows after 69904 cached keys")
    kp, vp = host_pools_with_prefix(pf)
    kd, vd = to_dev(kp), to_dev(vp)
    pa.pa_store_kv(to_dev(pf.k_new), to_dev(pf.v_new), to_dev(pf.slot_new), kd, vd)
    oracle.store_kv(pf.k_new, pf.v_new, pf.slot_new, kp, vp)
    offs = np.asarray(pf.q_offsets, np.int32)
    got = pa.pa_prefill_varlen(to_dev(pf.q), kd, vd, to_dev(pf.cu_seqlens_q), to_dev(pf.cu_seqlens_k), to_dev(offs),
                               to_dev(pf.block_table), pf.max_seqlen_q, pf.max_seqlen_k, pf.scale)
    torch.cuda.synchronize()
    ref = oracle.prefill(pf.q, kp, vp, pf.cu_seqlens_q, pf.cu_seqlens_k, offs, pf.block_table, pf.scale)
    err = max_abs_err(got, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol("bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_head_dim_256_group_8(dtype):
    """The widest head with the largest group: decode (4-wave workgroups) and
    prefill (the row-per-token path) with 16 query heads on 2 KV heads."""
    dec = W.make_decode("d256g8", 9410, [0, 1, 333, 2000, 4100], 16, 2, 256, 16, dtype)
    say(f"[limits] decode d=256 group 8 {dtype}")
    out, kp, vp = _decode(dec)
    ref = oracle.decode(dec.q, kp, vp, dec.context_lens, dec.block_table, dec.scale)
    assert max_abs_err(out, ref) <= tol(dtype)

    pf = W.make_prefill("d256g8_pf", 9411, [70, 1, 129], [0, 40, 300], 16, 2, 256, 16, dtype)
    say(f"[limits] prefill d=256 group 8 {dtype}")
    kp, vp = host_pools_with_prefix(pf)
    kd, vd = to_dev(kp), to_dev(vp)
    pa.pa_store_kv(to_dev(pf.k_new), to_dev(pf.v_new), to_dev(pf.slot_new), kd, vd)
    oracle.store_kv(pf.k_new, pf.v_new, pf.slot_new, kp, vp)
    offs = np.asarray(pf.q_offsets, np.int32)
    got = pa.pa_prefill_varlen(to_dev(pf.q), kd, vd, to_dev(pf.cu_seqlens_q), to_dev(pf.cu_seqlens_k), to_dev(offs),
                               to_dev(pf.block_table), pf.max_seqlen_q, pf.max_seqlen_k, pf.scale)
    torch.cuda.synchronize()
    ref = oracle.prefill(pf.q, kp, vp, pf.cu_seqlens_q, pf.cu_seqlens_k, offs, pf.block_table, pf.scale)
    assert max_abs_err(got, ref) <= tol(dtype)


def test_decode_4096_rows_without_row_order():
    """More rows than pa_decode_order ranks (it takes at most 2048): the rows
    run in index order; padding rows (context 0) return zeros."""
    rng = np.random.default_rng(9420)
    ctx = rng.integers(0, 300, size=4096).astype(np.int32)
    dec = W.make_decode("rows4096", 9420, ctx, 16, 8, 64, 32, "bf16")
    say("[limits] decode 4096 rows")
    out, kp, vp = _decode(dec, row_order=False)
    ref = oracle.decode(dec.q, kp, vp, dec.context_lens, dec.block_table, dec.scale)
    assert max_abs_err(out, ref) <= tol("bf16")
    zero = np.nonzero(ctx == 0)[0]
    assert (to_host_bits(out)[zero] == 0).all()


def test_empty_batches_are_no_ops():
    """No sequences, or no query tokens: every call returns without a launch
    and leaves its output untouched."""
    kd = torch.zeros((4, 16, 8, 128), dtype=torch.bfloat16, device="cuda")
    vd = torch.zeros_like(kd)
    empty_rows = torch.empty((0, 8, 128), dtype=torch.bfloat16, device="cuda")
    pa.pa_store_kv(empty_rows, empty_rows, torch.empty(0, dtype=torch.int32, device="cuda"), kd, vd)
    q0 = torch.empty((0, 16, 128), dtype=torch.bfloat16, device="cuda")
    i32 = lambda *v: torch.tensor(v, dtype=torch.int32, device="cuda")  # noqa: E731
    out = pa.pa_decode(q0, kd, vd, torch.empty(0, dtype=torch.int32, device="cuda"),
                       torch.empty((0, 1), dtype=torch.int32, device="cuda"), 0, 0.1)
    assert out.shape == (0, 16, 128)
    sentinel = torch.full((0, 16, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    pa.pa_prefill_varlen(q0, kd, vd, i32(0, 0), i32(0, 5), i32(5), i32(0).view(1, 1), 0, 5, 0.1, out=sentinel)
    torch.cuda.synchronize()


def test_broken_metadata_stays_inside_the_buffers():
    """Broken preconditions give wrong numbers, never accesses outside the
    buffers: cu_seqlens_q past total_q (MFMA prefill), row_order entries
    outside [0, num_seqs) (decode), cu_seqlens_k that skip rows (gather).
    Each output is a prefix of a larger tensor whose tail must keep its
    canary bits."""
    case = W.make_prefill("broken", 9430, [50, 50], [0, 7], 16, 8, 128, 16, "bf16")
    kp, vp = host_pools_with_prefix(case)
    kd, vd = to_dev(kp), to_dev(vp)
    pa.pa_store_kv(to_dev(case.k_new), to_dev(case.v_new), to_dev(case.slot_new), kd, vd)
    canary = -4096.0                                             # exact in bf16
    big = torch.full((case.total_q + 64, 16, 128), canary, dtype=torch.bfloat16, device="cuda")
    cu_q = np.array([0, 50, 10 ** 6], np.int32)                  # claims rows far past total_q = 100
    pa.pa_prefill_varlen(to_dev(case.q), kd, vd, to_dev(cu_q), to_dev(case.cu_seqlens_k),
                         to_dev(np.asarray(case.q_offsets, np.int32)), to_dev(case.block_table), 64,
                         case.max_seqlen_k, case.scale, out=big[:case.total_q])
    dec = W.make_decode("broken_dec", 9431, [5, 40, 300, 17, 0, 64, 1, 90], 16, 8, 128, 16, "bf16")
    dk, dv = dec.empty_pools()
    oracle.store_kv(dec.k_hist, dec.v_hist, dec.slot_hist, dk, dv)
    oracle.store_kv(dec.k_new, dec.v_new, dec.slot_new, dk, dv)
    dbig = torch.full((dec.num_seqs + 16, 16, 128), canary, dtype=torch.bfloat16, device="cuda")
    order = np.array([3, 99, -3, 0, 7, 2 ** 31 - 1, 1, 5], np.int32)
    pa.pa_decode(to_dev(dec.q), to_dev(dk), to_dev(dv), to_dev(dec.context_lens), to_dev(dec.block_table),
                 dec.max_context_len, dec.scale, out=dbig[:dec.num_seqs], row_order=to_dev(order))
    gbig = torch.full((40 + 16, 8, 128), canary, dtype=torch.bfloat16, device="cuda")
    vbig = gbig.clone()
    cu_k = np.array([5, 30, 12], np.int32)                       # rows 0..4 before the first sequence
    lib = pa.load()
    import ctypes
    pool = pa.pool_desc(kd)
    bt = to_dev(case.block_table)
    cu_k_d = to_dev(cu_k)
    code = lib.pa_gather_kv(kd.data_ptr(), vd.data_ptr(), ctypes.byref(pool), cu_k_d.data_ptr(), bt.data_ptr(),
                            bt.shape[1], 2, 40, gbig.data_ptr(), vbig.data_ptr(),
                            torch.cuda.current_stream().cuda_stream)
    assert code == 0
    torch.cuda.synchronize()
    assert (big[case.total_q:].float() == canary).all(), "prefill wrote past total_q"
    assert (dbig[dec.num_seqs:].float() == canary).all(), "decode wrote past num_seqs"
    assert (gbig[40:].float() == canary).all() and (vbig[40:].float() == canary).all(), "gather wrote past total_k"
    assert (gbig[:5].float() == canary).all(), "gather wrote rows no sequence owns"
    # rows the order still names exactly are right
    ref = oracle.decode(dec.q, dk, dv, dec.context_lens, dec.block_table, dec.scale, seqs=np.array([0, 3], np.int32))
    assert max_abs_err(dbig[torch.tensor([0, 3], device="cuda")], ref) <= tol("bf16")
