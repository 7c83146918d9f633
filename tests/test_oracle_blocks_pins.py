"""Pins of the block copy-on-write reference (CPU only): bit-exact copies of
the valid slots and nothing else, and the fork semantics the pages describe
checked through attention: a child that forks a parent's partial last block
attends exactly like the parent until the two append different tokens, and
afterwards each sees only its own."""
import numpy as np

import oracle
from oracle import blocks as B
import workloads as W


def test_copies_valid_slots_bitwise_and_nothing_else():
    rng = np.random.default_rng(1)
    nb, bs, hkv, d = 8, 16, 2, 32
    k = W.poisoned_pool(nb, bs, hkv, d, "bf16")
    k[:] = W.normal(rng, k.shape, "bf16")
    before = k.copy()
    B.copy_blocks([k], [3, 5, 6], [1, 0, 7], [5, 16, 0])
    assert np.array_equal(k[1, :5], before[3, :5]) and np.array_equal(k[1, 5:], before[1, 5:])
    assert np.array_equal(k[0], before[5])                    # a full block
    assert np.array_equal(k[7], before[7])                    # zero valid slots: untouched
    for b in (2, 3, 4, 5, 6):
        assert np.array_equal(k[b], before[b])                # sources and bystanders unchanged


def test_out_of_range_pairs_are_skipped():
    k = np.arange(4 * 4 * 2, dtype=np.float32).reshape(4, 4, 2)
    before = k.copy()
    B.copy_blocks([k], [9, 1, 0], [0, -1, 2], [2, 2, 5])
    assert np.array_equal(k, before)


def test_fork_of_a_partial_last_block_attends_like_the_parent():
    """Parent sequence of 37 tokens in 16-token blocks: 2 full blocks and a
    last block holding 5 tokens.  The child shares the full blocks and gets a
    copy of the last one.  Before any append both decode the same query to
    the same output; after each appends its own token, each output equals a
    fresh computation over its own tokens only."""
    rng = np.random.default_rng(2)
    nb, bs, hkv, d, hq = 8, 16, 2, 32, 4
    k = W.poisoned_pool(nb, bs, hkv, d, "bf16"); v = W.poisoned_pool(nb, bs, hkv, d, "bf16")
    parent = np.array([[6, 1, 4]], np.int32)
    slots = np.array([parent[0, j // bs] * bs + j % bs for j in range(37)], np.int32)
    kt, vt = W.normal(rng, (37, hkv, d), "bf16"), W.normal(rng, (37, hkv, d), "bf16")
    oracle.store_kv(kt, vt, slots, k, v)
    child = parent.copy(); child[0, 2] = 2
    B.copy_blocks([k, v], [4], [2], [37 - 2 * bs])
    q = W.normal(rng, (1, hq, d), "bf16")
    o_par = oracle.decode(q, k, v, [37], parent, 0.2)
    o_chi = oracle.decode(q, k, v, [37], child, 0.2)
    assert np.array_equal(o_par, o_chi)
    # each appends a different token at position 37 (slot 5 of its own last block)
    kp_, vp_ = W.normal(rng, (1, hkv, d), "bf16"), W.normal(rng, (1, hkv, d), "bf16")
    kc_, vc_ = W.normal(rng, (1, hkv, d), "bf16"), W.normal(rng, (1, hkv, d), "bf16")
    oracle.store_kv(kp_, vp_, [4 * bs + 5], k, v)
    oracle.store_kv(kc_, vc_, [2 * bs + 5], k, v)
    o_par2 = oracle.decode(q, k, v, [38], parent, 0.2)
    o_chi2 = oracle.decode(q, k, v, [38], child, 0.2)
    # fresh pools holding each sequence's own 38 tokens contiguously
    for toks_k, toks_v, out in ((np.concatenate([kt, kp_]), np.concatenate([vt, vp_]), o_par2),
                                (np.concatenate([kt, kc_]), np.concatenate([vt, vc_]), o_chi2)):
        k2 = W.poisoned_pool(3, bs, hkv, d, "bf16"); v2 = W.poisoned_pool(3, bs, hkv, d, "bf16")
        oracle.store_kv(toks_k, toks_v, np.arange(38, dtype=np.int32), k2, v2)
        ref = oracle.decode(q, k2, v2, [38], np.array([[0, 1, 2]], np.int32), 0.2)
        assert np.array_equal(out, ref)
    assert not np.array_equal(o_par2, o_chi2)
