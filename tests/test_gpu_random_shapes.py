"""Seeded random shapes through the prefill and the decode against the fp64
oracle.  Head dim, query group, KV heads, block size, element type, ragged
lengths and cached prefixes are drawn together, so combinations that the
targeted tests do not name (head_dim 256 with a group of 8 and blocks of 4 in
a launch of many sequences, fp16 with blocks of 1, ...) still meet the
oracle.  Sizes are capped so the oracle finishes each case in a second or
two."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_mapping_amd as pa
import workloads as W
from helpers import host_pools_with_prefix, max_abs_err, say, to_dev, tol

pytestmark = pytest.mark.gpu

PREFILL_CASES = 16
DECODE_CASES = 12


def _heads(rng):
    group = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    while group * hkv > 16:  # keep the oracle's work small
        hkv //= 2
    return group * max(hkv, 1), max(hkv, 1)


@pytest.mark.parametrize("i", range(PREFILL_CASES))
def test_random_prefill_shapes(i):
    rng = np.random.default_rng(9900 + i)
    d = int(rng.choice([32, 64, 128, 256]))
    hq, hkv = _heads(rng)
    bs = int(rng.choice([1, 2, 4, 16, 32, 256]))
    dtype = str(rng.choice(["bf16", "f16", "f32"]))
    n = int(rng.integers(1, 13))
    q_lens = rng.integers(0, 201, size=n).tolist()
    q_offs = rng.integers(0, 301, size=n).tolist()
    if rng.random() < 0.25:  # every sequence the same new-token count (the grouped tile order)
        q_lens = [int(q_lens[0]) or 1] * n
    case = W.make_prefill("rand", 9900 + i, q_lens, q_offs, hq, hkv, d, bs, dtype)
    say(f"[random prefill {i}] {dtype} d={d} {hq}/{hkv} bs={bs} q={q_lens} off={q_offs}")
    kp, vp = host_pools_with_prefix(case)
    kd, vd = to_dev(kp), to_dev(vp)
    pa.pa_store_kv(to_dev(case.k_new), to_dev(case.v_new), to_dev(case.slot_new), kd, vd)
    oracle.store_kv(case.k_new, case.v_new, case.slot_new, kp, vp)
    out = pa.pa_prefill_varlen(to_dev(case.q), kd, vd, to_dev(case.cu_seqlens_q), to_dev(case.cu_seqlens_k),
                               to_dev(np.asarray(case.q_offsets, np.int32)), to_dev(case.block_table),
                               case.max_seqlen_q, case.max_seqlen_k, case.scale)
    torch.cuda.synchronize()
    ref = oracle.prefill(case.q, kp, vp, case.cu_seqlens_q, case.cu_seqlens_k, case.q_offsets, case.block_table,
                         case.scale)
    err = max_abs_err(out, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol(dtype)


@pytest.mark.parametrize("i", range(DECODE_CASES))
def test_random_decode_shapes(i):
    rng = np.random.default_rng(9950 + i)
    d = int(rng.choice([32, 64, 128, 256]))
    hq, hkv = _heads(rng)
    bs = int(rng.choice([1, 2, 4, 16, 32, 256]))
    dtype = str(rng.choice(["bf16", "f16", "f32"]))
    n = int(rng.integers(1, 40))
    ctx = rng.integers(1, 3001, size=n).tolist()
    case = W.make_decode("rand", 9950 + i, ctx, hq, hkv, d, bs, dtype)
    say(f"[random decode {i}] {dtype} d={d} {hq}/{hkv} bs={bs} rows={n} max ctx={max(ctx)}")
    kp, vp = case.empty_pools()
    oracle.store_kv(case.k_hist, case.v_hist, case.slot_hist, kp, vp)
    kd, vd = to_dev(kp), to_dev(vp)
    pa.pa_store_kv(to_dev(case.k_new), to_dev(case.v_new), to_dev(case.slot_new), kd, vd)
    oracle.store_kv(case.k_new, case.v_new, case.slot_new, kp, vp)
    ctx_d = to_dev(case.context_lens)
    order = pa.pa_decode_order(ctx_d) if rng.random() < 0.5 else None
    out = pa.pa_decode(to_dev(case.q), kd, vd, ctx_d, to_dev(case.block_table), case.max_context_len, case.scale,
                       row_order=order)
    torch.cuda.synchronize()
    ref = oracle.decode(case.q, kp, vp, case.context_lens, case.block_table, case.scale)
    err = max_abs_err(out, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol(dtype)


INT8_CASES = 10


@pytest.mark.parametrize("i", range(INT8_CASES))
def test_random_int8_shapes(i):
    """INT8 pools: the quantizing store (bit for bit against the oracle), then
    a prefill and a decode over the same pools."""
    from oracle import int8 as Q
    from test_gpu_int8 import assert_pools_equal, dev_pools, int8_pools
    rng = np.random.default_rng(9990 + i)
    d = int(rng.choice([32, 64, 128, 256]))
    hq, hkv = _heads(rng)
    bs = int(rng.choice([1, 4, 16, 256]))
    dtype = str(rng.choice(["bf16", "f16", "f32"]))
    n = int(rng.integers(1, 9))
    q_lens = rng.integers(1, 151, size=n).tolist()
    q_offs = rng.integers(0, 301, size=n).tolist()
    case = W.make_prefill("rand_i8", 9990 + i, q_lens, q_offs, hq, hkv, d, bs, dtype)
    say(f"[random int8 {i}] {dtype} d={d} {hq}/{hkv} bs={bs} q={q_lens} off={q_offs}")
    host = int8_pools(case.num_blocks, case.block_size, hkv, d)
    dev = dev_pools(*host)
    for k, v, s in ((case.k_cached, case.v_cached, case.slot_cached), (case.k_new, case.v_new, case.slot_new)):
        if len(s):
            pa.pa_store_kv_int8(to_dev(k), to_dev(v), to_dev(s), *dev)
            Q.store_kv(k, v, s, *host)
    torch.cuda.synchronize()
    assert_pools_equal(dev, host)
    offs = np.asarray(case.q_offsets, np.int32)
    out = pa.pa_prefill_varlen_int8(to_dev(case.q), *dev, to_dev(case.cu_seqlens_q), to_dev(case.cu_seqlens_k),
                                    to_dev(offs), to_dev(case.block_table), case.max_seqlen_q, case.max_seqlen_k,
                                    case.scale)
    torch.cuda.synchronize()
    ref = Q.prefill(case.q, *host, case.cu_seqlens_q, case.cu_seqlens_k, offs, case.block_table, case.scale)
    err = max_abs_err(out, ref)
    say(f"  prefill max-abs {err:.3e}")
    assert err <= tol(dtype)
    # decode: the last query row of each sequence against its whole context
    last = (np.asarray(case.cu_seqlens_q[1:]) - 1).astype(np.int64)
    ctx = (np.asarray(case.cu_seqlens_k[1:]) - np.asarray(case.cu_seqlens_k[:-1])).astype(np.int32)
    qd = case.q[last]
    outd = pa.pa_decode_int8(to_dev(qd), *dev, to_dev(ctx), to_dev(case.block_table), int(ctx.max()), case.scale)
    torch.cuda.synchronize()
    refd = Q.decode(qd, *host, ctx, case.block_table, case.scale)
    errd = max_abs_err(outd, refd)
    say(f"  decode max-abs {errd:.3e}")
    assert errd <= tol(dtype)
