"""fp16 (IEEE binary16) on the GPU against the fp64 oracle: the store and the
gather bit for bit, decode and prefill element by element within the fp16
tolerance, the fork's microbenchmark decode shape, and INT8 pools quantized
from fp16 rows and read by fp16 queries."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_mapping_amd as pa
import workloads as W
from oracle import blocks as B
from oracle import int8 as Q
from helpers import as_f64, host_pools_with_prefix, max_abs_err, say, to_dev, to_host_bits, tol

pytestmark = pytest.mark.gpu

F16 = "f16"


def _store_both(case, kp, vp, kd, vd):
    pa.pa_store_kv(to_dev(case.k_new), to_dev(case.v_new), to_dev(case.slot_new), kd, vd)
    oracle.store_kv(case.k_new, case.v_new, case.slot_new, kp, vp)


# ---------------------------------------------------------------- store / gather

@pytest.mark.parametrize("d,bs,hkv", [(128, 256, 8), (64, 16, 2), (32, 1, 1), (256, 4, 4), (128, 16, 8)])
def test_store_and_gather_bit_exact(d, bs, hkv):
    case = W.make_prefill("f16_store", 70 + d + bs, [1, 67, 0, 130, 5], [0, 13, 9, 0, 250], hkv, hkv, d, bs, F16)
    say(f"[f16 store/gather] d={d} bs={bs} hkv={hkv} T={len(case.slot_new)}")
    kp, vp = host_pools_with_prefix(case)
    kd, vd = to_dev(kp), to_dev(vp)
    _store_both(case, kp, vp, kd, vd)
    torch.cuda.synchronize()
    assert to_host_bits(kd).view(np.uint16).tobytes() == kp.view(np.uint16).tobytes()
    assert to_host_bits(vd).view(np.uint16).tobytes() == vp.view(np.uint16).tobytes()
    total = int(case.cu_seqlens_k[-1])
    ko, vo = pa.pa_gather_kv(kd, vd, to_dev(case.cu_seqlens_k), to_dev(case.block_table), total)
    kr, vr = oracle.gather_kv(kp, vp, case.cu_seqlens_k, case.block_table)
    torch.cuda.synchronize()
    assert to_host_bits(ko).tobytes() == kr.tobytes()
    assert to_host_bits(vo).tobytes() == vr.tobytes()


def test_store_strided_rows_and_padding_slots():
    """Rows taken from a wider [T, 2*Hkv*D] buffer (not a multiple of 16 bytes
    apart: the element path) and slot -1 padding tokens."""
    rng = np.random.default_rng(77)
    nb, bs, hkv, d = 6, 16, 2, 32
    kp = W.poisoned_pool(nb, bs, hkv, d, F16)
    vp = kp.copy()
    wide_k = W.normal(rng, (9, hkv * d + 3), F16)
    wide_v = W.normal(rng, (9, hkv * d + 3), F16)
    slots = np.array([5, -1, 17, 90, -1, 0, 33, 64, 95], np.int32)
    kd, vd = to_dev(kp), to_dev(vp)
    k_t = to_dev(wide_k)[:, :hkv * d].view(9, hkv, d)
    v_t = to_dev(wide_v)[:, :hkv * d].view(9, hkv, d)
    pa.pa_store_kv(k_t, v_t, to_dev(slots), kd, vd)
    oracle.store_kv(np.ascontiguousarray(wide_k[:, :hkv * d]).reshape(9, hkv, d),
                    np.ascontiguousarray(wide_v[:, :hkv * d]).reshape(9, hkv, d), slots, kp, vp)
    torch.cuda.synchronize()
    assert to_host_bits(kd).tobytes() == kp.tobytes()
    assert to_host_bits(vd).tobytes() == vp.tobytes()


def test_copy_blocks_bit_exact():
    rng = np.random.default_rng(78)
    nb, bs, hkv, d = 10, 16, 8, 128
    host = [W.normal(rng, (nb, bs, hkv, d), F16) for _ in range(2)]
    dev = [to_dev(h) for h in host]
    src = np.array([3, 7, 1], np.int32)
    dst = np.array([0, 5, 9], np.int32)
    n = np.array([16, 1, 9], np.int32)
    pa.pa_copy_blocks(to_dev(src), to_dev(dst), to_dev(n), *dev)
    B.copy_blocks(host, src, dst, n)
    torch.cuda.synchronize()
    for dv, h in zip(dev, host):
        assert to_host_bits(dv).tobytes() == h.tobytes()


# ---------------------------------------------------------------- decode

def _decode_host_case(case):
    kp, vp = case.empty_pools()
    oracle.store_kv(case.k_hist, case.v_hist, case.slot_hist, kp, vp)
    kd, vd = to_dev(kp), to_dev(vp)
    _store_both(case, kp, vp, kd, vd)
    out = pa.pa_decode(to_dev(case.q), kd, vd, to_dev(case.context_lens), to_dev(case.block_table),
                       case.max_context_len, case.scale)
    torch.cuda.synchronize()
    assert to_host_bits(kd).tobytes() == kp.tobytes()
    ref = oracle.decode(case.q, kp, vp, case.context_lens, case.block_table, case.scale)
    return out, ref


@pytest.mark.parametrize("d,hq,hkv,bs", [
    (128, 16, 8, 16), (128, 16, 8, 256), (64, 8, 1, 32), (256, 8, 2, 16), (32, 16, 4, 1), (128, 32, 4, 64),
])
def test_decode_ragged_contexts(d, hq, hkv, bs):
    ctx = [0, 1, bs, 2 * bs + 1, 1023, 1024, 1025, 3000, 17, 0, 5000]
    case = W.make_decode("f16_dec", 800 + d + hq + bs, ctx, hq, hkv, d, bs, F16)
    say(f"[f16 decode] d={d} {hq}/{hkv} bs={bs}")
    out, ref = _decode_host_case(case)
    err = max_abs_err(out, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol(F16)
    g = as_f64(out)
    assert (g[0] == 0).all() and (g[9] == 0).all()


@pytest.mark.parametrize("bs", [16, 256])
def test_decode_fork_microbenchmark_shape(bs):
    case = W.fork_microbench_decode(block_size=bs)
    say(f"[f16 decode] fork microbenchmark 8 x 512, bs={bs}")
    out, ref = _decode_host_case(case)
    err = max_abs_err(out, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol(F16)


def test_decode_one_long_row_many_splits():
    case = W.make_decode("f16_b1", 831, [20000], 16, 8, 128, 16, F16)
    say("[f16 decode] batch 1 x 20000")
    out, ref = _decode_host_case(case)
    assert max_abs_err(out, ref) <= tol(F16)


def test_decode_c4_layer_every_row():
    """The 256 x U[100, 2048] decode layer in fp16, values drawn on the device."""
    lay = W.c4_decode_layout(dtype=F16)
    nb, bs, hkv, d = lay.num_blocks, lay.block_size, lay.num_kv_heads, lay.head_dim
    say(f"[f16 decode] c4 layer: {lay.num_seqs} seqs, every row")
    kd = W.device_normal((nb, bs, hkv, d), 4300, dtype=F16)
    vd = W.device_normal((nb, bs, hkv, d), 4301, dtype=F16)
    q = W.device_normal((lay.num_seqs, lay.num_q_heads, d), 9300, dtype=F16)
    out = pa.pa_decode(q, kd, vd, to_dev(lay.context_lens), to_dev(lay.block_table), lay.max_context_len,
                       lay.scale)
    torch.cuda.synchronize()
    ref = oracle.decode(to_host_bits(q), to_host_bits(kd), to_host_bits(vd), lay.context_lens, lay.block_table,
                        lay.scale)
    err = max_abs_err(out, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol(F16)


# ---------------------------------------------------------------- prefill

def _prefill(case, rows=None):
    kp, vp = host_pools_with_prefix(case)
    kd, vd = to_dev(kp), to_dev(vp)
    _store_both(case, kp, vp, kd, vd)
    offs = np.asarray(case.q_offsets, np.int32)
    out = pa.pa_prefill_varlen(to_dev(case.q), kd, vd, to_dev(case.cu_seqlens_q), to_dev(case.cu_seqlens_k),
                               to_dev(offs), to_dev(case.block_table), case.max_seqlen_q, case.max_seqlen_k,
                               case.scale)
    torch.cuda.synchronize()
    ref = oracle.prefill(case.q, kp, vp, case.cu_seqlens_q, case.cu_seqlens_k, offs, case.block_table,
                         case.scale, rows=rows)
    got = out if rows is None else out[torch.as_tensor(rows, device="cuda").long()]
    return got, ref


@pytest.mark.parametrize("d,hq,hkv,bs", [
    (128, 16, 8, 16), (64, 8, 1, 32), (128, 4, 4, 1), (32, 4, 2, 16), (256, 4, 2, 16), (128, 32, 4, 64),
    (128, 16, 8, 256), (64, 16, 4, 8),
])
def test_prefill_ragged_shapes_and_offsets(d, hq, hkv, bs):
    case = W.make_prefill("f16_pf", 850 + d + hq + bs, [1, 67, 0, 130, 5, 200], [0, 13, 9, 0, 250, 61], hq, hkv,
                          d, bs, F16)
    say(f"[f16 prefill] ragged d={d} {hq}/{hkv} bs={bs}")
    got, ref = _prefill(case)
    err = max_abs_err(got, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol(F16)


@pytest.mark.parametrize("make", ["c2_8x128", "c3_prefix"])
def test_prefill_configurations(make):
    case = W.c2_varlen(128, dtype=F16) if make == "c2_8x128" else W.c3_prefix(dtype=F16)
    say(f"[f16 prefill] {case.name}")
    got, ref = _prefill(case)
    assert max_abs_err(got, ref) <= tol(F16)


def test_prefill_c5a_long_every_row():
    case = W.c5a_long(dtype=F16)
    say("[f16 prefill] c5a 1x4096, every row")
    got, ref = _prefill(case)
    err = max_abs_err(got, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol(F16)


def test_prefill_c5a_mixed_every_row():
    case = W.c5a_mixed(dtype=F16)
    say(f"[f16 prefill] c5a mixed {case.num_seqs} seqs, every row")
    got, ref = _prefill(case)
    err = max_abs_err(got, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol(F16)


def test_prefill_single_visible_key_rows_return_v_and_determinism():
    """Row 0 of a fresh prompt sees key 0 only: its output is V[0] bit for bit
    (P = 1 and l = 1 are exact in fp16); a second launch repeats every bit."""
    case = W.make_prefill("f16_one", 890, [1, 64, 129], [0, 0, 0], 16, 8, 128, 16, F16)
    say("[f16 prefill] single-key rows + determinism")
    kp, vp = host_pools_with_prefix(case)
    kd, vd = to_dev(kp), to_dev(vp)
    _store_both(case, kp, vp, kd, vd)
    args = (to_dev(case.cu_seqlens_q), to_dev(case.cu_seqlens_k), to_dev(np.zeros(3, np.int32)),
            to_dev(case.block_table), case.max_seqlen_q, case.max_seqlen_k, case.scale)
    out = pa.pa_prefill_varlen(to_dev(case.q), kd, vd, *args)
    again = pa.pa_prefill_varlen(to_dev(case.q), kd, vd, *args)
    torch.cuda.synchronize()
    for s in range(3):
        r = int(case.cu_seqlens_q[s])
        assert (to_host_bits(out[r]) == np.repeat(case.v_new[r], 2, axis=0)).all()
    assert to_host_bits(again).tobytes() == to_host_bits(out).tobytes()


@pytest.mark.parametrize("direction", ["rising", "falling"])
def test_prefill_steep_score_ramp(direction):
    """Scores along a ramp of about 200 log2 units over 1024 keys: rising
    scores keep pushing the probabilities past the fp16 bound (2^14 per lane
    and block), so the rescale path runs again and again; falling scores make
    later keys underflow against the first block."""
    case = W.make_prefill("f16_ramp", 7150, [1024], [0], 16, 8, 128, 16, F16)
    rng = np.random.default_rng(7151)
    u = rng.standard_normal(128)
    u /= np.linalg.norm(u)
    ramp = 40.0 * np.arange(1024) / 1024.0
    if direction == "falling":
        ramp = ramp[::-1].copy()
    case.q = np.broadcast_to(40.0 * u, (1024, 16, 128)).astype(np.float16)
    case.k_new = np.broadcast_to(ramp[:, None, None] * u[None, None, :], (1024, 8, 128)).astype(np.float16)
    say(f"[f16 prefill] steep {direction} score ramp")
    got, ref = _prefill(case)
    err = max_abs_err(got, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol(F16)


# ---------------------------------------------------------------- INT8 pools, fp16 rows and queries

def _int8_pools(nb, bs, hkv, d):
    kq = np.full((nb, bs, hkv, d), -128, np.int8)
    ks = np.full((nb, bs, hkv), np.float16(np.nan), np.float16)
    return [kq, kq.copy(), ks, ks.copy()]


def _assert_same(dev, host):
    for dv, h in zip(dev, host):
        assert dv.cpu().numpy().view(np.uint8).tobytes() == h.view(np.uint8).tobytes()


def test_int8_store_from_fp16_rows_bit_exact():
    """fp16 sources quantize to the oracle's codes and scale bits, including
    rows at the quantizer's edges (zero, exact halves, subnormal fp16)."""
    rng = np.random.default_rng(91)
    nb, bs, hkv, d = 8, 16, 2, 128
    t = 40
    k = W.normal(rng, (t, hkv, d), F16)
    v = W.normal(rng, (t, hkv, d), F16)
    k[0] = 0
    k[1, 0, :8] = np.array([127, 2.5, -2.5, 0.5, -0.5, 1.5, -1.5, 126.5], np.float16)
    k[1, 0, 8:] = 0
    k[2, 1, :] = np.float16(2.0 ** -24)
    v[3, 0, :] = np.float16(65504.0)
    v[3, 0, 1] = np.float16(-65504.0)
    slots = np.random.default_rng(92).permutation(nb * bs)[:t].astype(np.int32)
    slots[5] = -1
    host = _int8_pools(nb, bs, hkv, d)
    dev = [torch.from_numpy(h.copy()).cuda() for h in host]
    pa.pa_store_kv_int8(to_dev(k), to_dev(v), to_dev(slots), *dev)
    Q.store_kv(k, v, slots, *host)
    torch.cuda.synchronize()
    _assert_same(dev, host)


def _int8_case_pools(case):
    host = _int8_pools(case.num_blocks, case.block_size, case.num_kv_heads, case.head_dim)
    dev = [torch.from_numpy(h.copy()).cuda() for h in host]
    return host, dev


@pytest.mark.parametrize("d,hq,hkv,bs,ctx", [
    (128, 16, 8, 16, [512] * 8),                       # the fork's microbenchmark shape
    (128, 16, 8, 256, [1, 2, 100, 255, 256, 257, 1000, 2048]),
    (64, 8, 8, 32, [3, 64, 129, 700]),
    (256, 8, 2, 16, [40, 300, 17, 0]),
    (128, 32, 4, 16, [1, 500, 1500, 0, 64]),           # group 8
])
def test_int8_decode_fp16_queries(d, hq, hkv, bs, ctx):
    case = W.make_decode("i8_f16", 870 + d + bs, ctx, hq, hkv, d, bs, F16)
    say(f"[f16 int8 decode] d={d} {hq}/{hkv} bs={bs} ctx={ctx[:4]}")
    host, dev = _int8_case_pools(case)
    for k, v, s in ((case.k_hist, case.v_hist, case.slot_hist), (case.k_new, case.v_new, case.slot_new)):
        if len(s):
            pa.pa_store_kv_int8(to_dev(k), to_dev(v), to_dev(s), *dev)
            Q.store_kv(k, v, s, *host)
    out = pa.pa_decode_int8(to_dev(case.q), *dev, to_dev(case.context_lens), to_dev(case.block_table),
                            case.max_context_len, case.scale)
    torch.cuda.synchronize()
    _assert_same(dev, host)
    ref = Q.decode(case.q, *host, case.context_lens, case.block_table, case.scale)
    err = max_abs_err(out, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol(F16)


INT8_F16_PREFILL = {  # name: (q_lens, q_offsets, hq, hkv, d, bs); even hkv and d 64/128 run the MFMA path
    "ragged_16_8_d128_bs16": ([1, 67, 0, 130, 5], [0, 13, 9, 0, 250], 16, 8, 128, 16),
    "ragged_8_2_d64_bs8": ([33, 4, 90, 200], [7, 0, 100, 31], 8, 2, 64, 8),
    "group4_16_4_d128_bs32": ([128, 77], [0, 300], 16, 4, 128, 32),
    "odd_hkv_rows_path_6_3_d128": ([40, 9], [5, 0], 6, 3, 128, 16),
    "d256_rows_path": ([20, 3], [0, 11], 4, 2, 256, 16),
    "group8_16_2_d128_bs16": ([90, 1, 200], [0, 33, 150], 16, 2, 128, 16),
}


@pytest.mark.parametrize("name", list(INT8_F16_PREFILL))
def test_int8_prefill_fp16_queries(name):
    q_lens, q_offs, hq, hkv, d, bs = INT8_F16_PREFILL[name]
    case = W.make_prefill("i8_f16_pf", 880 + d + hq + bs, q_lens, q_offs, hq, hkv, d, bs, F16)
    say(f"[f16 int8 prefill] {name}")
    host, dev = _int8_case_pools(case)
    for k, v, s in ((case.k_cached, case.v_cached, case.slot_cached), (case.k_new, case.v_new, case.slot_new)):
        if len(s):
            pa.pa_store_kv_int8(to_dev(k), to_dev(v), to_dev(s), *dev)
            Q.store_kv(k, v, s, *host)
    offs = np.asarray(case.q_offsets, np.int32)
    out = pa.pa_prefill_varlen_int8(to_dev(case.q), *dev, to_dev(case.cu_seqlens_q), to_dev(case.cu_seqlens_k),
                                    to_dev(offs), to_dev(case.block_table), case.max_seqlen_q, case.max_seqlen_k,
                                    case.scale)
    torch.cuda.synchronize()
    ref = Q.prefill(case.q, *host, case.cu_seqlens_q, case.cu_seqlens_k, offs, case.block_table, case.scale)
    err = max_abs_err(out, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol(F16)


def test_int8_prefill_fp16_queries_c5a_every_row():
    """1 x 4096 causal over INT8 pools quantized from fp16 rows, fp16 queries
    (the fp16 matrix-core path), every row."""
    case = W.c5a_long(dtype=F16)
    say("[f16 int8 prefill] c5a 1x4096, every row")
    host, dev = _int8_case_pools(case)
    pa.pa_store_kv_int8(to_dev(case.k_new), to_dev(case.v_new), to_dev(case.slot_new), *dev)
    Q.store_kv(case.k_new, case.v_new, case.slot_new, *host)
    offs = np.asarray(case.q_offsets, np.int32)
    out = pa.pa_prefill_varlen_int8(to_dev(case.q), *dev, to_dev(case.cu_seqlens_q), to_dev(case.cu_seqlens_k),
                                    to_dev(offs), to_dev(case.block_table), case.max_seqlen_q, case.max_seqlen_k,
                                    case.scale)
    torch.cuda.synchronize()
    ref = Q.prefill(case.q, *host, case.cu_seqlens_q, case.cu_seqlens_k, offs, case.block_table, case.scale)
    err = max_abs_err(out, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol(F16)


def test_int8_prefill_fp16_saturates_at_the_largest_fp16():
    """Rows holding +-65504: 127 times the fp16 scale (516) passes 65504, so the
    fp16 matrix-core path saturates the dequantized values instead of making
    them infinite; every output stays finite."""
    case = W.make_prefill("i8_f16_sat", 881, [40], [0], 16, 8, 128, 16, F16)
    case.k_new[3, :, 0] = np.float16(65504.0)
    case.v_new[5, :, 1] = np.float16(-65504.0)
    case.q[:] = (case.q.astype(np.float32) * 1e-4).astype(np.float16)
    host, dev = _int8_case_pools(case)
    pa.pa_store_kv_int8(to_dev(case.k_new), to_dev(case.v_new), to_dev(case.slot_new), *dev)
    offs = np.asarray(case.q_offsets, np.int32)
    out = pa.pa_prefill_varlen_int8(to_dev(case.q), *dev, to_dev(case.cu_seqlens_q), to_dev(case.cu_seqlens_k),
                                    to_dev(offs), to_dev(case.block_table), case.max_seqlen_q, case.max_seqlen_k,
                                    case.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
