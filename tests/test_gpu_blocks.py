"""pa_copy_blocks on the GPU: bit-exact against the reference copy, and the
block-table fork it serves (a child copies its parent's partial last block,
then both decode) through the bf16 and INT8 decode kernels."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_mapping_amd as pa
import workloads as W
from oracle import blocks as B
from oracle import int8 as Q
from helpers import max_abs_err, say, to_dev, to_host_bits, tol

pytestmark = pytest.mark.gpu

LAYOUTS = [  # (dtype, nb, bs, hkv, d): the last two take the 2-byte path (blocks not 16-byte multiples)
    ("bf16", 12, 256, 8, 128),
    ("f32", 9, 16, 2, 32),
    ("int8", 10, 16, 8, 128),
    ("bf16", 7, 1, 1, 4),
    ("int8", 6, 2, 1, 8),
]


def _pairs(rng, nb, bs):
    perm = rng.permutation(nb)
    k = nb // 2
    src, dst = perm[:k].astype(np.int32), perm[k:2 * k].astype(np.int32)
    n = rng.integers(0, bs + 1, size=k).astype(np.int32)
    n[0] = bs
    src = np.concatenate([src, [nb + 3, 0]]).astype(np.int32)     # an id outside the pool
    dst = np.concatenate([dst, [0, -2]]).astype(np.int32)          # a negative id
    n = np.concatenate([n, [1, 1]]).astype(np.int32)
    return src, dst, n


@pytest.mark.parametrize("dtype,nb,bs,hkv,d", LAYOUTS)
def test_copy_blocks_bit_exact(dtype, nb, bs, hkv, d):
    rng = np.random.default_rng(nb * 100 + bs + d)
    say(f"[copy_blocks] {dtype} nb={nb} bs={bs} hkv={hkv} d={d}")
    if dtype == "int8":
        host = [rng.integers(-127, 128, size=(nb, bs, hkv, d)).astype(np.int8) for _ in range(2)]
        host += [rng.standard_normal((nb, bs, hkv)).astype(np.float16) for _ in range(2)]
        dev = [torch.from_numpy(h.copy()).cuda() for h in host]
    else:
        host = [W.normal(rng, (nb, bs, hkv, d), dtype) for _ in range(2)]
        dev = [to_dev(h) for h in host]
    src, dst, n = _pairs(rng, nb, bs)
    pa.pa_copy_blocks(to_dev(src), to_dev(dst), to_dev(n), *dev)
    B.copy_blocks(host, src, dst, n)
    torch.cuda.synchronize()
    for dv, h in zip(dev, host):
        got = dv.cpu().numpy() if dtype == "int8" else to_host_bits(dv)
        assert got.view(np.uint8).tobytes() == h.view(np.uint8).tobytes()


def _fork_case(rng, dtype):
    nb, bs, hkv, d, hq = 8, 16, 8, 128, 16
    parent = np.array([[6, 1, 4]], np.int32)
    child = np.array([[6, 1, 2]], np.int32)
    slots = np.array([parent[0, j // bs] * bs + j % bs for j in range(37)], np.int32)
    toks = (W.normal(rng, (37, hkv, d), "bf16"), W.normal(rng, (37, hkv, d), "bf16"))
    q = W.normal(rng, (1, hq, d), "bf16")
    return nb, bs, hkv, d, hq, parent, child, slots, toks, q


def test_fork_then_diverge_bf16_decode():
    rng = np.random.default_rng(21)
    nb, bs, hkv, d, hq, parent, child, slots, (kt, vt), q = _fork_case(rng, "bf16")
    say("[copy_blocks] fork of a partial last block, bf16 decode")
    kp, vp = W.poisoned_pool(nb, bs, hkv, d, "bf16"), W.poisoned_pool(nb, bs, hkv, d, "bf16")
    kd, vd = to_dev(kp), to_dev(vp)
    pa.pa_store_kv(to_dev(kt), to_dev(vt), to_dev(slots), kd, vd)
    oracle.store_kv(kt, vt, slots, kp, vp)
    pa.pa_copy_blocks(to_dev(np.array([4], np.int32)), to_dev(np.array([2], np.int32)),
                      to_dev(np.array([5], np.int32)), kd, vd)
    B.copy_blocks([kp, vp], [4], [2], [5])
    qd, ctx = to_dev(q), to_dev(np.array([37], np.int32))
    o_par = pa.pa_decode(qd, kd, vd, ctx, to_dev(parent), 37, 0.1)
    o_chi = pa.pa_decode(qd, kd, vd, ctx, to_dev(child), 37, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(o_par, o_chi)
    new = [(W.normal(rng, (1, hkv, d), "bf16"), W.normal(rng, (1, hkv, d), "bf16")) for _ in range(2)]
    for (k1, v1), slot in zip(new, (4 * bs + 5, 2 * bs + 5)):
        pa.pa_store_kv(to_dev(k1), to_dev(v1), to_dev(np.array([slot], np.int32)), kd, vd)
        oracle.store_kv(k1, v1, [slot], kp, vp)
    ctx2 = to_dev(np.array([38], np.int32))
    for table in (parent, child):
        out = pa.pa_decode(qd, kd, vd, ctx2, to_dev(table), 38, 0.1)
        torch.cuda.synchronize()
        ref = oracle.decode(q, kp, vp, [38], table, 0.1)
        assert max_abs_err(out, ref) <= tol("bf16")


def test_fork_int8_codes_and_scales():
    rng = np.random.default_rng(22)
    nb, bs, hkv, d, hq, parent, child, slots, (kt, vt), q = _fork_case(rng, "int8")
    say("[copy_blocks] fork, INT8 pools")
    kq = torch.zeros((nb, bs, hkv, d), dtype=torch.int8, device="cuda"); vq = torch.zeros_like(kq)
    ks = torch.zeros((nb, bs, hkv), dtype=torch.float16, device="cuda"); vs = torch.zeros_like(ks)
    pa.pa_store_kv_int8(to_dev(kt), to_dev(vt), to_dev(slots), kq, vq, ks, vs)
    pa.pa_copy_blocks(to_dev(np.array([4], np.int32)), to_dev(np.array([2], np.int32)),
                      to_dev(np.array([5], np.int32)), kq, vq, ks, vs)
    qd, ctx = to_dev(q), to_dev(np.array([37], np.int32))
    o_par = pa.pa_decode_int8(qd, kq, vq, ks, vs, ctx, to_dev(parent), 37, 0.1)
    o_chi = pa.pa_decode_int8(qd, kq, vq, ks, vs, ctx, to_dev(child), 37, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(o_par, o_chi)
    host = tuple(t.cpu().numpy() for t in (kq, vq, ks, vs))
    ref = Q.decode(q, *host, [37], child, 0.1)
    assert max_abs_err(o_chi, ref) <= tol("bf16")


def test_fork_all_c4_partial_last_blocks_timed():
    """Every C4 sequence forks its partial last block (bs 256) into a spare
    block of the same pool; the copies are checked by sampling and timed."""
    lay = W.c4_decode_layout()
    nb, bs, hkv, d = lay.num_blocks, lay.block_size, lay.num_kv_heads, lay.head_dim
    extra = lay.num_seqs
    kd = W.device_normal((nb + extra, bs, hkv, d), 31)
    vd = W.device_normal((nb + extra, bs, hkv, d), 32)
    ctx = lay.context_lens.astype(np.int64)
    last = np.array([lay.block_table[s, (ctx[s] - 1) // bs] for s in range(lay.num_seqs)], np.int32)
    n = (((ctx - 1) % bs) + 1).astype(np.int32)
    dst = np.arange(nb, nb + extra, dtype=np.int32)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    src_d, dst_d, n_d = to_dev(last), to_dev(dst), to_dev(n)
    pa.pa_copy_blocks(src_d, dst_d, n_d, kd, vd)
    torch.cuda.synchronize()
    a.record()
    for _ in range(10):
        pa.pa_copy_blocks(src_d, dst_d, n_d, kd, vd)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 100
    moved = int(n.sum()) * hkv * d * 2 * 2 * 2   # K and V, read and write
    say(f"  {lay.num_seqs} forks, {int(n.sum())} tokens: {us:.1f} us, {moved / us / 1e3:.0f} GB/s")
    for s in (0, 17, 255):
        k_src = kd[last[s], : n[s]]
        assert torch.equal(kd[dst[s], : n[s]], k_src) and torch.equal(vd[dst[s], : n[s]], vd[last[s], : n[s]])
