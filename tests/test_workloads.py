"""The seeded generator: determinism and the structural facts the kernels rely on."""
import numpy as np
import pytest

import workloads as W


def _check_layout(table, lens, block_size, num_blocks, spare):
    need = [max(1, -(-int(n) // block_size)) for n in lens]
    used = np.concatenate([table[s, :n] for s, n in enumerate(need)])
    assert len(np.unique(used)) == len(used), "a physical block is dealt twice"
    assert used.min() >= 0 and used.max() < num_blocks
    assert not set(used.tolist()) & set(np.asarray(spare).tolist())
    for s, n in enumerate(need):
        assert set(table[s, n:].tolist()) <= set(np.asarray(spare).tolist())


@pytest.mark.parametrize("make", [lambda: W.c2_varlen(32), lambda: W.c2_varlen(256), W.c3_prefix,
                                  W.c5a_mixed])
def test_prefill_cases_are_deterministic_and_consistent(make):
    a, b = make(), make()
    assert a.q.tobytes() == b.q.tobytes() and a.k_new.tobytes() == b.k_new.tobytes()
    assert (a.block_table == b.block_table).all()
    assert all(qo + ql == kl for qo, ql, kl in zip(a.q_offsets, a.q_lens, a.k_lens))
    _check_layout(a.block_table, a.k_lens, a.block_size, a.num_blocks, a.spare_blocks)
    slots = np.concatenate([a.slot_cached, a.slot_new])
    assert len(np.unique(slots)) == len(slots)
    assert slots.min() >= 0 and slots.max() < a.num_blocks * a.block_size


def test_config_sizes():
    pre, dec = W.c1_tiny()
    assert pre.q_lens == [5, 17, 40] and pre.causal_pairs == 988 and pre.num_blocks == 16
    assert [d["context_lens"].tolist() for d in dec][-1] == [9, 21, 44]
    for n, pairs in ((32, 4224), (128, 66048), (256, 263168)):
        c = W.c2_varlen(n, with_values=False)
        assert c.causal_pairs == 8 * n * (n + 1) // 2 and c.total_q == 8 * n
        assert c.causal_pairs == pairs
    c3 = W.c3_prefix(with_values=False)
    assert c3.causal_pairs == 24508 and c3.k_lens == [300, 300]
    c5 = W.c5a_long(with_values=False)
    assert c5.causal_pairs == 8390656 and c5.num_blocks == 256 + 16
    mixed = W.c5a_mixed(with_values=False)
    assert mixed.total_q == 8192 and mixed.q_offsets[0] > 0 and all(o == 0 for o in mixed.q_offsets[1:])
    assert all(100 <= ql + qo <= 1024 for ql, qo in zip(mixed.q_lens[:-1], mixed.q_offsets[:-1]))


def test_decode_layouts():
    c4 = W.c4_decode_layout()
    assert c4.num_seqs == 256 and c4.context_lens.min() >= 100 and c4.context_lens.max() <= 2048
    _check_layout(c4.block_table, c4.context_lens, 256, c4.num_blocks, c4.spare_blocks)
    assert len(np.unique(c4.slot_new)) == 256
    c5b = W.c5b_decode_layout()
    assert c5b.block_table.shape == (64, 2048) and c5b.num_blocks == 131072 + 16
    assert c5b.kv_bytes() == 64 * 32768 * 8 * 128 * 2 * 2
    _check_layout(c5b.block_table, c5b.context_lens, 16, c5b.num_blocks, c5b.spare_blocks)


def test_c1_decode_slots_follow_prefill():
    pre, dec = W.c1_tiny()
    seen = set(pre.slot_new.tolist())
    for step in dec:
        for s in step["slot_new"].tolist():
            assert s not in seen
            seen.add(s)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5], np.float32)
    b = W.f32_to_bf16_bits(x)
    assert b[0] == 0x3F80
    assert b[1] == 0x3F80          # halfway, ties to even (down)
    assert b[2] == 0x3F82          # halfway, ties to even (up)
    assert W.bf16_bits_to_f32(b)[3] == -2.5
    import torch
    t = torch.from_numpy(np.random.default_rng(0).standard_normal(4096, dtype=np.float32))
    ref = t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (W.f32_to_bf16_bits(t.numpy()) == ref).all()
