"""Pins of the INT8 KV-cache oracle (CPU only).

Every test checks the oracle against something other than its own formula:
values and properties the pages state ("LLM inference interview notes
(nano-vllm fork)", Q3 parts 1, 2 and 4, and the follow-up on all-zero
vectors), brute force over every candidate code or fp16 value, and closed
forms of attention.
"""
import numpy as np
import pytest

import oracle
from oracle import int8 as Q
import workloads as W


def _rand_vectors(seed, n, d, spread=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d)).astype(np.float32)
    if spread:  # magnitudes over many binades, as model activations have
        x *= np.exp2(rng.integers(-12, 12, size=(n, 1))).astype(np.float32)
    return x


def test_largest_element_maps_to_127_and_no_code_is_minus_128():
    """Part 1: dividing by max/127 sends the largest |x| to +-127 exactly;
    127.5 truncates to 127, so the range never overflows (no clamp)."""
    x = _rand_vectors(1, 4000, 128)
    codes, _, _ = Q.quantize(x)
    i = np.argmax(np.abs(x), axis=1)
    top = codes[np.arange(len(x)), i].astype(np.int32)
    assert np.array_equal(np.abs(top), np.full(len(x), 127))
    assert np.array_equal(np.sign(top), np.sign(x[np.arange(len(x)), i]).astype(np.int32))
    assert codes.min() >= -127 and codes.max() <= 127


def test_round_half_away_from_zero_on_exact_halves():
    """Part 1: x/scale + 0.5 (or - 0.5 below zero), truncated: exact halves go
    away from zero, unlike round-half-to-even."""
    x = np.array([[127.0, 2.5, -2.5, 0.5, -0.5, 1.5, -1.5, 126.5, -0.0, 0.49999997]], np.float32)
    codes, scale, s16 = Q.quantize(x)
    assert scale[0] == np.float32(1.0) and s16[0] == np.float16(1.0)
    # The last value is the float just below 0.5: adding 0.5 in fp32 gives
    # 1 - 2^-25, which rounds to 1.0, so the pages' "+0.5 then truncate"
    # yields 1 where exact half-away rounding would give 0.  Both sides take
    # this decision in fp32.
    assert codes[0].tolist() == [127, 3, -3, 1, -1, 2, -2, 127, 0, 1]
    # half-to-even would differ on 2.5, -2.5, 0.5, -0.5, 126.5
    assert np.round(x[0, 1:5]).tolist() == [2.0, -2.0, 0.0, -0.0]


def test_each_code_is_the_nearest_integer_ties_away_brute_force():
    """Every code is, among all 255 candidates, the integer nearest to
    x/scale (fp32), ties going away from zero (random data stays clear of
    the half-ulp band below a half-point where the fp32 "+0.5" rounds up)."""
    x = _rand_vectors(2, 300, 64)
    codes, scale, _ = Q.quantize(x)
    qf = (x / scale[:, None]).astype(np.float32).astype(np.float64)
    cand = np.arange(-127, 128, dtype=np.float64)
    dist = np.abs(qf[..., None] - cand)                      # [n, d, 255]
    best = dist.min(axis=-1, keepdims=True)
    tie_ok = np.where(dist == best, np.abs(cand), -1.0)      # among the nearest, the largest |n|
    pick = cand[np.argmax(tie_ok, axis=-1)]
    assert np.array_equal(codes.astype(np.float64), pick)


def _all_finite_fp16():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    ok = np.isfinite(vals)
    return bits[ok], vals[ok]


def test_stored_scale_is_nearest_fp16_ties_to_even_brute_force():
    """The scale is stored as the fp16 nearest to the fp32 scale, ties to the
    even significand (checked against every finite fp16 value)."""
    bits, vals = _all_finite_fp16()
    x = _rand_vectors(3, 400, 32)
    _, scale, s16 = Q.quantize(x)
    for s, h in zip(scale.astype(np.float64), s16):
        d = np.abs(vals - s)
        m = d.min()
        cands = bits[d == m]
        if len(cands) > 1:
            cands = cands[(cands & 1) == 0]
        got = np.float16(h).view(np.uint16)
        assert got in cands


def test_all_zero_vector_scale_underflows_fp16_and_decodes_to_zero():
    """Follow-up on all-zero vectors: the 1e-8 floor avoids a zero division,
    but 1e-8 is below fp16's smallest subnormal, so the stored scale is 0;
    codes are 0 and so is every dequantized value."""
    x = np.zeros((3, 128), np.float32)
    codes, scale, s16 = Q.quantize(x)
    assert np.all(scale == np.float32(1.0e-8))
    assert np.all(s16.view(np.uint16) == 0)
    assert not np.any(codes)
    assert not np.any(Q.dequantize(codes, s16))
    # a tiny but nonzero vector also takes the floor and keeps its codes
    t = np.full((1, 4), 1.0e-10, np.float32)
    c2, sc2, _ = Q.quantize(t)
    assert sc2[0] == np.float32(1.0e-8) and c2[0].tolist() == [0, 0, 0, 0]


def test_recovered_values_within_half_a_step():
    """Part 4 (operator level): a recovered value is off by at most about
    half a quantization step.  With the fp32 scale s used to quantize and
    its fp16 rounding s16 used to dequantize: |code*s16 - x| <= s/2 + 127|s16 - s|."""
    x = _rand_vectors(4, 2000, 128, spread=False)
    codes, scale, s16 = Q.quantize(x)
    rec = Q.dequantize(codes, s16).astype(np.float64)
    s = scale.astype(np.float64)[:, None]
    bound = s / 2 + 127 * np.abs(s16.astype(np.float64)[:, None] - s) + 1e-12
    assert np.all(np.abs(rec - x) <= bound)
    assert np.max(np.abs(rec - x) / s) <= 0.5 + 127 * 2.0 ** -11


def test_bytes_per_token_head_is_130_of_256():
    """Part 1, storage: at head_dim 128 a (token, KV head) takes 128 int8
    bytes plus a 2-byte fp16 scale, 130 B against 256 B in bf16 (50.78%)."""
    nb, bs, hkv, d = 4, 16, 8, 128
    kq = np.zeros((nb, bs, hkv, d), np.int8)
    ks = np.zeros((nb, bs, hkv), np.float16)
    per = (kq.nbytes + ks.nbytes) / (nb * bs * hkv)
    assert per == 130.0 and round(per / (d * 2), 4) == 0.5078


def test_store_skips_minus_one_and_round_trips():
    """Store then read back by slot equals quantizing the input; slot -1
    leaves the pools' poisoned bits untouched."""
    rng = np.random.default_rng(5)
    nb, bs, hkv, d = 6, 4, 2, 32
    k = W.normal(rng, (7, hkv, d), "bf16")
    v = W.normal(rng, (7, hkv, d), "bf16")
    slots = np.array([3, -1, 0, 17, -1, 22, 8], np.int32)
    kq = np.full((nb, bs, hkv, d), -128, np.int8)
    vq = kq.copy()
    ks = np.full((nb, bs, hkv), np.nan, np.float16)
    vs = ks.copy()
    Q.store_kv(k, v, slots, kq, vq, ks, vs)
    kc, _, k16 = Q.quantize(k)
    vc, _, v16 = Q.quantize(v)
    flat_kq, flat_ks = kq.reshape(-1, hkv, d), ks.reshape(-1, hkv)
    flat_vq, flat_vs = vq.reshape(-1, hkv, d), vs.reshape(-1, hkv)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        assert np.array_equal(flat_kq[s], kc[t]) and np.array_equal(flat_vq[s], vc[t])
        assert np.array_equal(flat_ks[s].view(np.uint16), k16[t].view(np.uint16))
        assert np.array_equal(flat_vs[s].view(np.uint16), v16[t].view(np.uint16))
    used = set(int(s) for s in slots if s >= 0)
    for s in range(nb * bs):
        if s not in used:
            assert np.all(flat_kq[s] == -128) and np.all(np.isnan(flat_ks[s]))


def test_single_visible_key_returns_dequantized_v():
    """Row 0 of a fresh prompt sees only key 0: its output is key 0's
    dequantized V exactly."""
    case = W.make_prefill("i8_first_row", 11, [5, 9], [0, 0], 4, 2, 32, 4, "bf16")
    nb, bs, hkv, d = case.empty_pools()[0].shape
    kq = np.zeros((nb, bs, hkv, d), np.int8); vq = kq.copy()
    ks = np.zeros((nb, bs, hkv), np.float16); vs = ks.copy()
    Q.store_kv(case.k_new, case.v_new, case.slot_new, kq, vq, ks, vs)
    out = Q.prefill(case.q, kq, vq, ks, vs, case.cu_seqlens_q, case.cu_seqlens_k, [0, 0], case.block_table,
                    case.scale)
    _, vf = Q.dequantize_pools(kq, vq, ks, vs)
    for s, start in enumerate(case.cu_seqlens_q[:-1]):
        blk = case.block_table[s][0]
        for h in range(4):
            assert np.array_equal(out[start, h], vf[blk, 0, h // 2].astype(np.float64))


def test_uniform_keys_average_dequantized_values():
    """If every visible key is the same vector, attention is the plain mean
    of the visible dequantized values."""
    rng = np.random.default_rng(12)
    nb, bs, hkv, d, ctx = 8, 4, 1, 16, 13
    kq = np.zeros((nb, bs, hkv, d), np.int8); vq = kq.copy()
    ks = np.zeros((nb, bs, hkv), np.float16); vs = ks.copy()
    table = np.array([[5, 2, 7, 0]], np.int32)
    slots = np.array([table[0, j // bs] * bs + j % bs for j in range(ctx)], np.int32)
    k = np.repeat(W.normal(rng, (1, hkv, d), "bf16"), ctx, axis=0)
    v = W.normal(rng, (ctx, hkv, d), "bf16")
    Q.store_kv(k, v, slots, kq, vq, ks, vs)
    q = W.normal(rng, (1, 2, d), "bf16")
    out = Q.decode(q, kq, vq, ks, vs, [ctx], table, 0.25)
    vc, _, v16 = Q.quantize(v)
    mean = Q.dequantize(vc, v16).astype(np.float64).mean(axis=0)[0]
    assert np.allclose(out[0, 0], mean, atol=1e-12) and np.allclose(out[0, 1], mean, atol=1e-12)


def test_attention_accuracy_matches_the_pages_microbenchmark():
    """Part 4 (attention level): on synthetic data at the microbenchmark's
    shape (batch 8, 16 query / 8 KV heads, head_dim 128, context 511) the
    pages report mean / max absolute error 0.00052 / 0.0027 and cosine
    similarity 0.999958 against the float kernel.  The oracle's INT8 decode
    against its bf16 decode on N(0,1) data lands in the same range."""
    rng = np.random.default_rng(13)
    b, hq, hkv, d, ctx, bs = 8, 16, 8, 128, 511, 16
    nbps = (ctx + bs - 1) // bs
    nb = b * nbps
    perm = rng.permutation(nb).astype(np.int32)
    table = perm.reshape(b, nbps)
    k = W.normal(rng, (b * ctx, hkv, d), "bf16")
    v = W.normal(rng, (b * ctx, hkv, d), "bf16")
    slots = np.concatenate([[table[s, j // bs] * bs + j % bs for j in range(ctx)] for s in range(b)]).astype(np.int32)
    kp = W.poisoned_pool(nb, bs, hkv, d, "bf16"); vp = W.poisoned_pool(nb, bs, hkv, d, "bf16")
    oracle.store_kv(k, v, slots, kp, vp)
    kq = np.zeros((nb, bs, hkv, d), np.int8); vq = kq.copy()
    ks = np.zeros((nb, bs, hkv), np.float16); vs = ks.copy()
    Q.store_kv(k, v, slots, kq, vq, ks, vs)
    q = W.normal(rng, (b, hq, d), "bf16")
    ctxs = np.full(b, ctx, np.int32)
    ref = oracle.decode(q, kp, vp, ctxs, table, d ** -0.5)
    got = Q.decode(q, kq, vq, ks, vs, ctxs, table, d ** -0.5)
    err = np.abs(got - ref)
    cos = np.sum(got * ref) / np.sqrt(np.sum(got * got) * np.sum(ref * ref))
    assert 1e-4 < err.mean() < 2e-3 and err.max() < 1e-2
    assert cos > 0.9999
