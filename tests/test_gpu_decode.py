"""pa_decode on the GPU against the fp64 oracle: C1's decode steps, C4 (256
sequences x U[100,2048], one layer pool in full plus a second layer), C5b
(64 x 32768, every row) and edge cases."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_mapping_amd as pa
import workloads as W
from helpers import as_f64, max_abs_err, say, to_dev, to_host_bits, tol

pytestmark = pytest.mark.gpu


def host_decode_pools(case):
    kp, vp = case.empty_pools()
    oracle.store_kv(case.k_hist, case.v_hist, case.slot_hist, kp, vp)
    return kp, vp


def run_decode_host_case(case):
    kp, vp = host_decode_pools(case)
    kd, vd = to_dev(kp), to_dev(vp)
    pa.pa_store_kv(to_dev(case.k_new), to_dev(case.v_new), to_dev(case.slot_new), kd, vd)
    oracle.store_kv(case.k_new, case.v_new, case.slot_new, kp, vp)
    out = pa.pa_decode(to_dev(case.q), kd, vd, to_dev(case.context_lens), to_dev(case.block_table),
                       case.max_context_len, case.scale)
    torch.cuda.synchronize()
    assert to_host_bits(kd).tobytes() == kp.tobytes()
    ref = oracle.decode(case.q, kp, vp, case.context_lens, case.block_table, case.scale)
    return out, ref


def test_c1_prefill_then_four_decode_steps():
    pre, steps = W.c1_tiny()
    say("[decode] c1: prefill + 4 decode steps")
    kp, vp = pre.empty_pools()
    kd, vd = to_dev(kp), to_dev(vp)
    pa.pa_store_kv(to_dev(pre.k_new), to_dev(pre.v_new), to_dev(pre.slot_new), kd, vd)
    oracle.store_kv(pre.k_new, pre.v_new, pre.slot_new, kp, vp)
    out = pa.pa_prefill_varlen(to_dev(pre.q), kd, vd, to_dev(pre.cu_seqlens_q), to_dev(pre.cu_seqlens_k),
                               to_dev(np.zeros(3, np.int32)), to_dev(pre.block_table), 40, 40, pre.scale)
    ref = oracle.prefill(pre.q, kp, vp, pre.cu_seqlens_q, pre.cu_seqlens_k, [0, 0, 0], pre.block_table,
                         pre.scale)
    assert max_abs_err(out, ref) <= tol("f32")
    for t, st in enumerate(steps):
        pa.pa_store_kv(to_dev(st["k_new"]), to_dev(st["v_new"]), to_dev(st["slot_new"]), kd, vd)
        oracle.store_kv(st["k_new"], st["v_new"], st["slot_new"], kp, vp)
        o = pa.pa_decode(to_dev(st["q"]), kd, vd, to_dev(st["context_lens"]), to_dev(pre.block_table),
                         int(st["context_lens"].max()), pre.scale)
        torch.cuda.synchronize()
        assert to_host_bits(kd).tobytes() == kp.tobytes()
        r = oracle.decode(st["q"], kp, vp, st["context_lens"], pre.block_table, pre.scale)
        err = max_abs_err(o, r)
        say(f"  step {t}: max-abs {err:.2e}")
        assert err <= tol("f32")


def _device_layer(layout, layer, poison=True):
    """Fill one layer's pools and queries on the device from seeded torch
    generators; NaN-poison every slot no sequence uses."""
    nb, bs, hkv, d = layout.num_blocks, layout.block_size, layout.num_kv_heads, layout.head_dim
    kd = W.device_normal((nb, bs, hkv, d), 4100 + 2 * layer)
    vd = W.device_normal((nb, bs, hkv, d), 4101 + 2 * layer)
    q = W.device_normal((layout.num_seqs, layout.num_q_heads, d), 9000 + layer)
    if poison:
        used = np.zeros(nb * bs, bool)
        for s, n in enumerate(layout.context_lens.tolist()):
            nblk = -(-n // bs)
            blocks = layout.block_table[s, :nblk].astype(np.int64)
            slots = (blocks[:, None] * bs + np.arange(bs)[None, :]).reshape(-1)[:n]
            used[slots] = True
        idx = torch.as_tensor(np.nonzero(~used)[0], device="cuda")
        nan = torch.tensor(float("nan"), dtype=kd.dtype, device="cuda")
        kd.view(nb * bs, -1)[idx] = nan
        vd.view(nb * bs, -1)[idx] = nan
    return q, kd, vd


def test_c4_batch_decode_full_layer():
    lay = W.c4_decode_layout()
    say(f"[decode] c4 layer 0: {lay.num_seqs} seqs, max ctx {lay.max_context_len}")
    q, kd, vd = _device_layer(lay, 0)
    out = pa.pa_decode(q, kd, vd, to_dev(lay.context_lens), to_dev(lay.block_table), lay.max_context_len,
                       lay.scale)
    torch.cuda.synchronize()
    kp, vp, qh = to_host_bits(kd), to_host_bits(vd), to_host_bits(q)
    ref = oracle.decode(qh, kp, vp, lay.context_lens, lay.block_table, lay.scale)
    err = max_abs_err(out, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol("bf16")


def test_c4_second_layer_pool_every_row():
    lay = W.c4_decode_layout()
    say("[decode] c4 layer 27, every row")
    q, kd, vd = _device_layer(lay, 27)
    out = pa.pa_decode(q, kd, vd, to_dev(lay.context_lens), to_dev(lay.block_table), lay.max_context_len,
                       lay.scale)
    torch.cuda.synchronize()
    ref = oracle.decode(to_host_bits(q), to_host_bits(kd), to_host_bits(vd), lay.context_lens,
                        lay.block_table, lay.scale)
    err = max_abs_err(out, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol("bf16")


def test_c5b_long_context_every_row():
    lay = W.c5b_decode_layout()
    say("[decode] c5b 64 x 32768, every row")
    q, kd, vd = _device_layer(lay, 0)
    out = pa.pa_decode(q, kd, vd, to_dev(lay.context_lens), to_dev(lay.block_table), lay.max_context_len,
                       lay.scale)
    torch.cuda.synchronize()
    ref = oracle.decode(to_host_bits(q), to_host_bits(kd), to_host_bits(vd), lay.context_lens,
                        lay.block_table, lay.scale)
    err = max_abs_err(out, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol("bf16")
    again = pa.pa_decode(q, kd, vd, to_dev(lay.context_lens), to_dev(lay.block_table), lay.max_context_len,
                         lay.scale)
    torch.cuda.synchronize()
    assert to_host_bits(again).tobytes() == to_host_bits(out).tobytes(), "not run-to-run deterministic"


@pytest.mark.parametrize("dtype,d,hq,hkv,bs", [
    ("bf16", 128, 16, 8, 16), ("bf16", 128, 16, 8, 256), ("f32", 32, 4, 2, 16), ("bf16", 64, 8, 1, 1),
    ("f32", 256, 8, 4, 32), ("bf16", 32, 16, 2, 64), ("f32", 128, 4, 4, 16),
])
def test_ragged_contexts_and_padding_rows(dtype, d, hq, hkv, bs):
    """Contexts of 0 (a padding row), 1, exact block multiples and ragged
    lengths up to several splits."""
    ctx = [0, 1, bs, 2 * bs + 1, 1023, 1024, 1025, 3000, 17, 0, 5000]
    case = W.make_decode("ragged", 300 + d, ctx, hq, hkv, d, bs, dtype)
    say(f"[decode] ragged {dtype} d={d} {hq}/{hkv} bs={bs}")
    out, ref = run_decode_host_case(case)
    assert max_abs_err(out, ref) <= tol(dtype)
    g = as_f64(out)
    assert (g[0] == 0).all() and (g[9] == 0).all()


def test_batch_one_long_context_many_splits():
    case = W.make_decode("b1", 31, [20000], 16, 8, 128, 16, "bf16")
    say("[decode] batch 1 x 20000")
    out, ref = run_decode_host_case(case)
    assert max_abs_err(out, ref) <= tol("bf16")


@pytest.mark.parametrize("num_rows", [600, 601, 1100])
def test_many_rows_with_ties_and_padding(num_rows):
    """More (row, KV head) work items than run at once, lengths from a small
    set (most rows tie) and every 7th row a padding row (context 0): the
    longest-first order is the stable argsort of -context_lens, and decoding
    with it gives the oracle's result, bit-identical to the given order."""
    rng = np.random.default_rng(4100 + num_rows)
    ctx = rng.choice([1, 16, 33, 64, 100, 255, 256, 300], size=num_rows)
    ctx[::7] = 0
    case = W.make_decode("ties", 4200 + num_rows, [int(c) for c in ctx], 16, 8, 64, 16, "bf16")
    say(f"[decode] {num_rows} rows with ties and padding")
    out, ref = run_decode_host_case(case)
    assert max_abs_err(out, ref) <= tol("bf16")
    g = as_f64(out)
    assert (g[::7] == 0).all()
    cl = to_dev(case.context_lens)
    order = pa.pa_decode_order(cl)
    torch.cuda.synchronize()
    assert np.array_equal(order.cpu().numpy(), np.argsort(-case.context_lens, kind="stable"))
    kp, vp = host_decode_pools(case)
    oracle.store_kv(case.k_new, case.v_new, case.slot_new, kp, vp)
    ordered = pa.pa_decode(to_dev(case.q), to_dev(kp), to_dev(vp), cl, to_dev(case.block_table),
                           case.max_context_len, case.scale, row_order=order)
    torch.cuda.synchronize()
    assert to_host_bits(ordered).tobytes() == to_host_bits(out).tobytes()


def test_c4_row_order_changes_nothing():
    """C4 decoded in longest-first order equals the given order bit for bit."""
    lay = W.c4_decode_layout()
    say("[decode] C4 with and without row order")
    kd = W.device_normal((lay.num_blocks, lay.block_size, lay.num_kv_heads, lay.head_dim), 7)
    vd = W.device_normal((lay.num_blocks, lay.block_size, lay.num_kv_heads, lay.head_dim), 8)
    q = W.device_normal((lay.num_seqs, lay.num_q_heads, lay.head_dim), 9)
    cl, bt = to_dev(lay.context_lens), to_dev(lay.block_table)
    base = pa.pa_decode(q, kd, vd, cl, bt, lay.max_context_len, lay.scale)
    order = pa.pa_decode_order(cl)
    ordered = pa.pa_decode(q, kd, vd, cl, bt, lay.max_context_len, lay.scale, row_order=order)
    torch.cuda.synchronize()
    assert np.array_equal(order.cpu().numpy(), np.argsort(-lay.context_lens, kind="stable"))
    assert to_host_bits(ordered).tobytes() == to_host_bits(base).tobytes()


@pytest.mark.parametrize("pad", [-1, 2**31 - 1])
def test_table_padding_is_never_read(pad):
    """Decode reads no block-table entry past a row's last needed block:
    padding with -1 or a huge id changes no output bit."""
    case = W.make_decode("pad", 7400, [1, 17, 300, 1000, 40], 16, 8, 128, 16, "bf16")
    say(f"[decode] table padding {pad}")
    out, ref = run_decode_host_case(case)
    assert max_abs_err(out, ref) <= tol("bf16")
    kp, vp = host_decode_pools(case)
    oracle.store_kv(case.k_new, case.v_new, case.slot_new, kp, vp)
    bt = case.block_table.copy()
    for s, c in enumerate(case.context_lens):
        bt[s, max(1, -(-int(c) // case.block_size)):] = pad
    again = pa.pa_decode(to_dev(case.q), to_dev(kp), to_dev(vp), to_dev(case.context_lens), to_dev(bt),
                         case.max_context_len, case.scale)
    torch.cuda.synchronize()
    assert to_host_bits(again).tobytes() == to_host_bits(out).tobytes()
