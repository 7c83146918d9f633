"""INT8 KV cache on the GPU: the quantizing store bit-exact against the
oracle (codes and fp16 scale bits), on poisoned pools."""
import numpy as np
import pytest
import torch

import paged_kv_attention_mapping_amd as pa
import workloads as W
from oracle import int8 as Q
from helpers import say, to_dev

pytestmark = pytest.mark.gpu

POISON_CODE = -128          # never produced by the quantizer
POISON_SCALE = np.float16(np.nan)


def int8_pools(nb, bs, hkv, d):
    kq = np.full((nb, bs, hkv, d), POISON_CODE, np.int8)
    ks = np.full((nb, bs, hkv), POISON_SCALE, np.float16)
    return kq, kq.copy(), ks, ks.copy()


def dev_pools(kq, vq, ks, vs):
    return (torch.from_numpy(kq).cuda(), torch.from_numpy(vq).cuda(), torch.from_numpy(ks).cuda(),
            torch.from_numpy(vs).cuda())


def assert_pools_equal(dev, host):
    for d, h in zip(dev, host):
        got = d.cpu().numpy()
        assert got.dtype == h.dtype
        assert got.view(np.uint8).tobytes() == h.view(np.uint8).tobytes()


STORE_CASES = {
    "c1_prefill_f32_d32": lambda: W.c1_tiny()[0],
    "c2_8x32": lambda: W.c2_varlen(32),
    "c3_prefix": W.c3_prefix,
    "c5a_4096": W.c5a_long,
    "c5a_mixed": W.c5a_mixed,
}


@pytest.mark.parametrize("name", list(STORE_CASES))
def test_store_int8_bit_exact_on_poisoned_pools(name):
    case = STORE_CASES[name]()
    nb, bs, hkv, d = case.empty_pools()[0].shape
    say(f"[int8 store] {name} T={len(case.slot_new)} d={d} src={case.dtype}")
    host = int8_pools(nb, bs, hkv, d)
    dev = dev_pools(*host)
    pa.pa_store_kv_int8(to_dev(case.k_new), to_dev(case.v_new), to_dev(case.slot_new), *dev)
    Q.store_kv(case.k_new, case.v_new, case.slot_new, *host)
    torch.cuda.synchronize()
    assert_pools_equal(dev, host)


def _special_rows(d):
    """Head vectors at the quantizer's edges, all exactly representable in bf16."""
    rows = []
    rows.append(np.zeros(d))                                            # all zero: fp16 scale 0
    r = np.zeros(d); r[:8] = [127, 2.5, -2.5, 0.5, -0.5, 1.5, -1.5, 126.5]; rows.append(r)  # exact halves
    r = np.full(d, 1e-10); rows.append(r)                              # scale floor 1e-8
    r = np.linspace(-3e5, 2e5, d); rows.append(r)                      # large, negative max
    r = np.zeros(d); r[0] = -1.0; r[1] = 1.0 / 254; r[2] = -1.0 / 254; rows.append(r)  # near half codes
    r = np.full(d, 7.0); rows.append(r)                                 # all equal: every code 127
    r = np.zeros(d); r[d - 1] = 3.0e-39; rows.append(r)                # subnormal input
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("src", ["bf16", "f32"])
def test_store_int8_edge_values(src):
    d, hkv, bs, nb = 128, 2, 16, 4
    base = _special_rows(d)
    t = len(base)
    k = np.stack([base, -base[::-1]], axis=1)                          # [T, 2, d]
    v = np.stack([base[::-1] * 0.5, base], axis=1)
    if src == "bf16":
        k, v = W.f32_to_bf16_bits(k), W.f32_to_bf16_bits(v)
    rng = np.random.default_rng(7)
    slots = rng.permutation(nb * bs)[:t].astype(np.int32)
    host = int8_pools(nb, bs, hkv, d)
    dev = dev_pools(*host)
    say(f"[int8 store] edge values src={src}")
    pa.pa_store_kv_int8(to_dev(k), to_dev(v), to_dev(slots), *dev)
    Q.store_kv(k, v, slots, *host)
    torch.cuda.synchronize()
    assert_pools_equal(dev, host)


def test_store_int8_padding_slots_and_strided_unaligned_rows():
    """Slot -1 rows are skipped; fp32 rows one element apart from 16-byte
    alignment take the per-element load path; bf16 rows with a wider stride."""
    rng = np.random.default_rng(8)
    nb, bs, hkv, d, t = 8, 4, 4, 64, 19
    slots = rng.permutation(nb * bs)[:t].astype(np.int32)
    slots[[2, 7, 11]] = -1
    for src, extra in (("f32", 1), ("bf16", 8)):
        big = W.normal(rng, (t, hkv * d + extra), src)
        kt = to_dev(big)
        k = kt.as_strided((t, hkv, d), (hkv * d + extra, d, 1))
        vt = to_dev(W.normal(rng, (t, hkv * d + extra), src))
        v = vt.as_strided((t, hkv, d), (hkv * d + extra, d, 1))
        host = int8_pools(nb, bs, hkv, d)
        dev = dev_pools(*host)
        say(f"[int8 store] strided src={src} extra={extra}")
        pa.pa_store_kv_int8(k, v, to_dev(slots), *dev)
        kh = np.ascontiguousarray(big[:, : hkv * d]).reshape(t, hkv, d)
        vh_bits = vt.cpu()
        vh = (vh_bits.view(torch.int16).numpy().view(np.uint16) if src == "bf16" else vh_bits.numpy())
        vh = np.ascontiguousarray(vh[:, : hkv * d]).reshape(t, hkv, d)
        Q.store_kv(kh, vh, slots, *host)
        torch.cuda.synchronize()
        assert_pools_equal(dev, host)


# ---------------------------------------------------------------- decode

from helpers import max_abs_err, tol  # noqa: E402


def _store_case_int8(case):
    """Host and device INT8 pools holding the case's history and new token,
    both quantized (device by pa_store_kv_int8, host by the oracle)."""
    host = int8_pools(case.num_blocks, case.block_size, case.num_kv_heads, case.head_dim)
    dev = dev_pools(*host)
    for k, v, s in ((case.k_hist, case.v_hist, case.slot_hist), (case.k_new, case.v_new, case.slot_new)):
        if len(s):
            pa.pa_store_kv_int8(to_dev(k), to_dev(v), to_dev(s), *dev)
            Q.store_kv(k, v, s, *host)
    torch.cuda.synchronize()
    assert_pools_equal(dev, host)
    return host, dev


DECODE_SHAPES = [  # (dtype, d, hq, hkv, bs, context lengths)
    ("bf16", 128, 16, 8, 16, [511] * 8),                       # the pages' microbenchmark shape
    ("bf16", 128, 16, 8, 256, [1, 2, 100, 255, 256, 257, 1000, 2048]),
    ("f32", 32, 4, 2, 16, [9, 21, 44]),                         # C1's shape, fp32
    ("bf16", 64, 8, 8, 32, [3, 64, 129, 700]),                  # group 1
    ("bf16", 256, 8, 2, 16, [40, 300, 17]),                     # group 4, head_dim 256
    ("f32", 128, 8, 4, 64, [0, 5, 333]),                        # a padding row (context 0)
    ("bf16", 128, 16, 2, 16, [1, 300, 2048, 0, 77]),            # group 8: two virtual heads per pool head
    ("f32", 64, 32, 4, 32, [3, 64, 129, 700]),                  # group 8, head_dim 64
]


@pytest.mark.parametrize("dtype,d,hq,hkv,bs,ctx", DECODE_SHAPES)
def test_decode_int8_against_oracle(dtype, d, hq, hkv, bs, ctx):
    case = W.make_decode("i8", 600 + d + hq + bs, ctx, hq, hkv, d, bs, dtype)
    say(f"[int8 decode] {dtype} d={d} {hq}/{hkv} bs={bs} ctx={ctx}")
    host, dev = _store_case_int8(case)
    out = pa.pa_decode_int8(to_dev(case.q), *dev, to_dev(case.context_lens), to_dev(case.block_table),
                            case.max_context_len, case.scale)
    torch.cuda.synchronize()
    ref = Q.decode(case.q, *host, case.context_lens, case.block_table, case.scale)
    err = max_abs_err(out, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol(dtype)


@pytest.mark.parametrize("vscale", [1e-4, 30.0])
def test_decode_int8_v_rows_far_from_unit_size(vscale):
    """V rows scaled by 1e-4 (fp16 scales near 3e-6) and by 30: the fp16
    weights of the V code pairs stay accurate relative to the output's own
    size (bf16 queries, the fp16-pair V path)."""
    case = W.make_decode("i8_vmag", 640, [1, 300, 2048, 77, 1000], 16, 8, 128, 16, "bf16")
    scale = lambda bits: W.f32_to_bf16_bits(W.bf16_bits_to_f32(bits) * np.float32(vscale))  # noqa: E731
    case.v_hist, case.v_new = scale(case.v_hist), scale(case.v_new)
    say(f"[int8 decode] V rows x {vscale}")
    host, dev = _store_case_int8(case)
    out = pa.pa_decode_int8(to_dev(case.q), *dev, to_dev(case.context_lens), to_dev(case.block_table),
                            case.max_context_len, case.scale)
    torch.cuda.synchronize()
    ref = Q.decode(case.q, *host, case.context_lens, case.block_table, case.scale)
    rel = max_abs_err(out, ref) / float(np.abs(ref).max())
    say(f"  max-abs / max |ref| {rel:.3e}")
    assert rel <= 1e-2


def test_decode_int8_one_long_row_many_splits_and_row_order():
    """One 30000-token row (split across many workgroups and merged), plus a
    short one; the longest-first row order gives bit-identical results."""
    case = W.make_decode("i8_long", 77, [30000, 7], 16, 8, 128, 16, "bf16")
    say("[int8 decode] 30000 + 7 tokens, splits")
    host, dev = _store_case_int8(case)
    ctx, bt = to_dev(case.context_lens), to_dev(case.block_table)
    out = pa.pa_decode_int8(to_dev(case.q), *dev, ctx, bt, case.max_context_len, case.scale)
    out2 = pa.pa_decode_int8(to_dev(case.q), *dev, ctx, bt, case.max_context_len, case.scale,
                             row_order=pa.pa_decode_order(ctx))
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    ref = Q.decode(case.q, *host, case.context_lens, case.block_table, case.scale)
    assert max_abs_err(out, ref) <= tol("bf16")


def _device_int8_layer(lay, layer):
    """A decode layer's INT8 pools built on the device: bf16 K/V drawn from
    seeded generators, quantized by pa_store_kv_int8 over every slot; slots
    no sequence uses get poisoned codes and NaN scales."""
    nb, bs, hkv, d = lay.num_blocks, lay.block_size, lay.num_kv_heads, lay.head_dim
    kq = torch.empty((nb, bs, hkv, d), dtype=torch.int8, device="cuda")
    vq = torch.empty_like(kq)
    ks = torch.empty((nb, bs, hkv), dtype=torch.float16, device="cuda")
    vs = torch.empty_like(ks)
    chunk = 1 << 16  # slots quantized per call, bounding the bf16 staging
    for c0 in range(0, nb * bs, chunk):
        n = min(chunk, nb * bs - c0)
        k = W.device_normal((n, hkv, d), 7000 + 2 * layer + c0)
        v = W.device_normal((n, hkv, d), 7001 + 2 * layer + c0)
        pa.pa_store_kv_int8(k, v, torch.arange(c0, c0 + n, dtype=torch.int32, device="cuda"), kq, vq, ks, vs)
    used = np.zeros(nb * bs, bool)
    for s, n in enumerate(lay.context_lens.tolist()):
        nblk = -(-n // bs)
        blocks = lay.block_table[s, :nblk].astype(np.int64)
        used[(blocks[:, None] * bs + np.arange(bs)[None, :]).reshape(-1)[:n]] = True
    idx = torch.as_tensor(np.nonzero(~used)[0], device="cuda")
    kq.view(nb * bs, -1)[idx] = POISON_CODE
    vq.view(nb * bs, -1)[idx] = POISON_CODE
    ks.view(nb * bs, -1)[idx] = float("nan")
    vs.view(nb * bs, -1)[idx] = float("nan")
    q = W.device_normal((lay.num_seqs, lay.num_q_heads, d), 9500 + layer)
    return q, (kq, vq, ks, vs)


def _compact_host(lay, dev, seqs):
    """Host copies of just the blocks the given sequences use, with a
    compacted block table (ids 0..n-1), for the oracle."""
    bs = lay.block_size
    rows = []
    for s in seqs:
        nblk = -(-int(lay.context_lens[s]) // bs)
        rows.append(lay.block_table[s, :nblk].astype(np.int64))
    ids = np.concatenate(rows)
    sel = torch.as_tensor(ids, device="cuda")
    host = tuple(t[sel].cpu().numpy() for t in dev)
    width = max(len(r) for r in rows)
    table = np.zeros((len(seqs), width), np.int32)
    o = 0
    for i, r in enumerate(rows):
        table[i, :len(r)] = np.arange(o, o + len(r))
        o += len(r)
    return host, table


def _int8_decode_every_row(lay, out, q, dev, chunk):
    """Max-abs error of every row of an INT8 decode layer against the oracle,
    taken over chunks of sequences (their blocks copied to the host and
    dequantized one chunk at a time)."""
    err = 0.0
    for c0 in range(0, lay.num_seqs, chunk):
        seqs = list(range(c0, min(c0 + chunk, lay.num_seqs)))
        host, table = _compact_host(lay, dev, seqs)
        sel = torch.as_tensor(seqs, device="cuda")
        qh = q[sel].view(torch.int16).cpu().numpy().view(np.uint16)
        ref = Q.decode(qh, *host, lay.context_lens[seqs], table, lay.scale)
        err = max(err, max_abs_err(out[sel], ref))
    return err


def test_decode_int8_c4_layer_every_row():
    lay = W.c4_decode_layout()
    say(f"[int8 decode] c4 layer: {lay.num_seqs} seqs, every row")
    q, dev = _device_int8_layer(lay, 0)
    ctx = to_dev(lay.context_lens)
    out = pa.pa_decode_int8(q, *dev, ctx, to_dev(lay.block_table), lay.max_context_len, lay.scale,
                            row_order=pa.pa_decode_order(ctx))
    torch.cuda.synchronize()
    err = _int8_decode_every_row(lay, out, q, dev, 256)
    say(f"  max-abs {err:.3e}")
    assert err <= tol("bf16")


def test_decode_int8_c5b_every_row():
    lay = W.c5b_decode_layout()
    say("[int8 decode] c5b 64 x 32768, every row")
    q, dev = _device_int8_layer(lay, 0)
    out = pa.pa_decode_int8(q, *dev, to_dev(lay.context_lens), to_dev(lay.block_table), lay.max_context_len,
                            lay.scale)
    torch.cuda.synchronize()
    err = _int8_decode_every_row(lay, out, q, dev, 8)
    say(f"  max-abs {err:.3e}")
    assert err <= tol("bf16")


# ---------------------------------------------------------------- prefill

PREFILL_CASES = {
    "c2_8x32": lambda: W.c2_varlen(32),
    "c2_8x128": lambda: W.c2_varlen(128),
    "c3_prefix": W.c3_prefix,
    "c1_prefill_f32_d32": lambda: W.c1_tiny()[0],
    "ragged_g4_d64_bs8": lambda: W.make_prefill("i8_ragged", 901, [1, 67, 0, 130, 5], [0, 13, 9, 0, 250], 8, 2, 64,
                                                8, "bf16"),
    "ragged_g1_d256_f32": lambda: W.make_prefill("i8_ragged2", 902, [33, 4, 90], [7, 0, 100], 4, 4, 256, 16,
                                                 "f32"),
    "ragged_g8_d128": lambda: W.make_prefill("i8_ragged3", 903, [50, 1, 130], [0, 20, 300], 16, 2, 128, 16,
                                             "bf16"),
}


@pytest.mark.parametrize("name", list(PREFILL_CASES))
def test_prefill_int8_against_oracle(name):
    case = PREFILL_CASES[name]()
    nb, bs, hkv, d = case.empty_pools()[0].shape
    say(f"[int8 prefill] {name}")
    host = int8_pools(nb, bs, hkv, d)
    dev = dev_pools(*host)
    for k, v, s in ((case.k_cached, case.v_cached, case.slot_cached), (case.k_new, case.v_new, case.slot_new)):
        if len(s):
            pa.pa_store_kv_int8(to_dev(k), to_dev(v), to_dev(s), *dev)
            Q.store_kv(k, v, s, *host)
    offs = np.asarray(case.q_offsets, np.int32)
    out = pa.pa_prefill_varlen_int8(to_dev(case.q), *dev, to_dev(case.cu_seqlens_q), to_dev(case.cu_seqlens_k),
                                    to_dev(offs), to_dev(case.block_table), case.max_seqlen_q, case.max_seqlen_k,
                                    case.scale)
    torch.cuda.synchronize()
    assert_pools_equal(dev, host)
    ref = Q.prefill(case.q, *host, case.cu_seqlens_q, case.cu_seqlens_k, offs, case.block_table, case.scale)
    err = max_abs_err(out, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol(case.dtype)


def test_prefill_int8_suffix_equals_rows_of_full_prefill():
    """C3's 44-token suffixes over their cached 256-token blocks equal (to
    the bf16 tolerance: the two launches split the rows' keys differently)
    rows 256..299 of a full 300-token INT8 prefill over the same pools, and
    both match the oracle."""
    case = W.c3_prefix()
    nb, bs, hkv, d = case.empty_pools()[0].shape
    host = int8_pools(nb, bs, hkv, d)
    dev = dev_pools(*host)
    for k, v, s in ((case.k_cached, case.v_cached, case.slot_cached), (case.k_new, case.v_new, case.slot_new)):
        pa.pa_store_kv_int8(to_dev(k), to_dev(v), to_dev(s), *dev)
        Q.store_kv(k, v, s, *host)
    offs = np.asarray(case.q_offsets, np.int32)
    suffix = pa.pa_prefill_varlen_int8(to_dev(case.q), *dev, to_dev(case.cu_seqlens_q), to_dev(case.cu_seqlens_k),
                                       to_dev(offs), to_dev(case.block_table), 44, 300, case.scale)
    rng = np.random.default_rng(3)
    q_full = W.normal(rng, (600, case.num_q_heads, d), "bf16")
    q_full[256:300] = case.q[:44]
    q_full[556:600] = case.q[44:]
    full = pa.pa_prefill_varlen_int8(to_dev(q_full), *dev, to_dev(np.array([0, 300, 600], np.int32)),
                                     to_dev(case.cu_seqlens_k), to_dev(np.zeros(2, np.int32)),
                                     to_dev(case.block_table), 300, 300, case.scale)
    torch.cuda.synchronize()
    rows = torch.as_tensor(np.r_[256:300, 556:600], device="cuda")
    ref = Q.prefill(case.q, *host, case.cu_seqlens_q, case.cu_seqlens_k, offs, case.block_table, case.scale)
    assert max_abs_err(suffix, ref) <= tol("bf16")
    assert max_abs_err(full[rows], ref) <= tol("bf16")


def test_prefill_int8_c5a_mixed_every_row():
    """C5a-ii (8192 tokens over ~13 sequences, a resumed chunk first), INT8
    pools, every row."""
    case = W.c5a_mixed()
    nb, bs, hkv, d = case.empty_pools()[0].shape
    say(f"[int8 prefill] c5a mixed {case.total_q} tokens")
    host = int8_pools(nb, bs, hkv, d)
    dev = dev_pools(*host)
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
    assert err <= tol("bf16")


def test_prefill_int8_c5a_4096_every_row():
    """C5a-i (1 x 4096, block 16) over INT8 pools on the query-tiled MFMA path."""
    case = W.c5a_long()
    nb, bs, hkv, d = case.empty_pools()[0].shape
    say("[int8 prefill] c5a 1x4096, every row")
    host = int8_pools(nb, bs, hkv, d)
    dev = dev_pools(*host)
    pa.pa_store_kv_int8(to_dev(case.k_new), to_dev(case.v_new), to_dev(case.slot_new), *dev)
    Q.store_kv(case.k_new, case.v_new, case.slot_new, *host)
    offs = np.zeros(1, np.int32)
    out = pa.pa_prefill_varlen_int8(to_dev(case.q), *dev, to_dev(case.cu_seqlens_q), to_dev(case.cu_seqlens_k),
                                    to_dev(offs), to_dev(case.block_table), 4096, 4096, case.scale)
    torch.cuda.synchronize()
    ref = Q.prefill(case.q, *host, case.cu_seqlens_q, case.cu_seqlens_k, offs, case.block_table, case.scale)
    err = max_abs_err(out, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol("bf16")


@pytest.mark.parametrize("qdtype,d,hq,hkv", [("bf16", 128, 16, 8), ("f16", 128, 16, 8), ("bf16", 64, 8, 2),
                                             ("f16", 128, 32, 4)])
def test_prefill_int8_many_short_sequences(qdtype, d, hq, hkv):
    """80 sequences of 1..200 new tokens after 0..300 cached ones over INT8
    pools: more workgroups than CUs, which selects the 4-wave layout (64-key
    steps, two scale-fetching waves)."""
    rng = np.random.default_rng(9500 + d + hq)
    q_lens = rng.integers(1, 200, size=80, endpoint=True).tolist()
    q_offs = rng.integers(0, 300, size=80, endpoint=True).tolist()
    case = W.make_prefill("i8_many", 9500 + d + hq, q_lens, q_offs, hq, hkv, d, 16, qdtype)
    say(f"[int8 prefill] 80 short sequences, {qdtype} queries, d={d} {hq}/{hkv}")
    nb, bs, _, _ = case.empty_pools()[0].shape
    host = int8_pools(nb, bs, hkv, d)
    dev = dev_pools(*host)
    for k, v, sl in ((case.k_cached, case.v_cached, case.slot_cached), (case.k_new, case.v_new, case.slot_new)):
        if len(sl):
            pa.pa_store_kv_int8(to_dev(k), to_dev(v), to_dev(sl), *dev)
            Q.store_kv(k, v, sl, *host)
    offs = np.asarray(case.q_offsets, np.int32)
    out = pa.pa_prefill_varlen_int8(to_dev(case.q), *dev, to_dev(case.cu_seqlens_q), to_dev(case.cu_seqlens_k),
                                    to_dev(offs), to_dev(case.block_table), case.max_seqlen_q, case.max_seqlen_k,
                                    case.scale)
    torch.cuda.synchronize()
    ref = Q.prefill(case.q, *host, case.cu_seqlens_q, case.cu_seqlens_k, offs, case.block_table, case.scale)
    err = max_abs_err(out, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol(qdtype)
