"""Pins for the CPU fp64 oracle: each test checks the oracle against something
other than itself -- a worked example printed on the pages, a textbook or
library routine, a closed form, or an invariant the pages fix.

Runs on the CPU only.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _case_pools(case):
    """Host pools holding the cached prefix and the new tokens (oracle store)."""
    kp, vp = case.empty_pools()
    if len(case.slot_cached):
        oracle.store_kv(case.k_cached, case.v_cached, case.slot_cached, kp, vp)
    oracle.store_kv(case.k_new, case.v_new, case.slot_new, kp, vp)
    return kp, vp


def _as_f64(a):
    if a.dtype == np.uint16:
        return W.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def _sdpa_causal(q, k, v, group, scale, mask=None):
    """torch CPU float64 SDPA; q [N,Hq,D], k/v [S,Hkv,D]; GQA by repeating kv heads."""
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).repeat_interleave(group, dim=1).permute(1, 0, 2)[None].contiguous()
    vt = torch.from_numpy(v).repeat_interleave(group, dim=1).permute(1, 0, 2)[None].contiguous()
    if mask is None:
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    else:
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


# ---------------------------------------------------------------- store / gather

def test_gather_worked_example_left_pad():
    """mini-infer 03, section 2.4: req_b (3 tokens) left-padded to 6 gives three
    zero rows, then [20,30],[21,31],[22,32]."""
    g = json.load(open(os.path.join(GOLDEN, "gather_left_pad.json")))
    hkv, d, bs = g["num_kv_heads"], g["head_dim"], 2
    req_b = np.array(g["req_b_k_rows"], dtype=np.float32).reshape(-1, hkv, d)
    req_a = np.arange(6 * hkv * d, dtype=np.float32).reshape(6, hkv, d) + 100
    # pool of 8 blocks of 2 slots; req_a owns 3 blocks, req_b owns 2, shuffled ids
    table = np.array([[5, 0, 7], [2, 6, 6]], dtype=np.int32)
    slots_a = [table[0][j // bs] * bs + j % bs for j in range(6)]
    slots_b = [table[1][j // bs] * bs + j % bs for j in range(3)]
    kp = np.full((8, bs, hkv, d), np.nan, np.float32)
    vp = kp.copy()
    oracle.store_kv(req_a, req_a, slots_a, kp, vp)
    oracle.store_kv(req_b, req_b, slots_b, kp, vp)
    k_out, _ = oracle.gather_kv(kp, vp, [0, 6, 9], table)
    b_rows = k_out[6:9].reshape(3, d)
    padded = np.zeros((g["max_seq_len"], d), np.float32)
    padded[g["max_seq_len"] - g["req_b_len"]:] = b_rows
    np.testing.assert_array_equal(padded, np.array(g["expected_left_padded_req_b"], np.float32))
    np.testing.assert_array_equal(k_out[:6], req_a)


@settings(max_examples=40, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), bs=st.sampled_from([1, 2, 4, 16]),
       hkv=st.integers(1, 3), d=st.sampled_from([1, 4, 8]), dtype=st.sampled_from(["f32", "bf16", "f16"]),
       lens=st.lists(st.integers(1, 40), min_size=1, max_size=4))
def test_store_gather_roundtrip_bitwise(seed, bs, hkv, d, dtype, lens):
    """Store then gather returns the exact bits; untouched slots keep their bits."""
    case = W.make_prefill("rt", seed, lens, [0] * len(lens), hkv, hkv, d, bs, dtype, num_spare=2)
    kp, vp = _case_pools(case)
    k_out, v_out = oracle.gather_kv(kp, vp, case.cu_seqlens_k, case.block_table)
    assert k_out.tobytes() == case.k_new.tobytes()
    assert v_out.tobytes() == case.v_new.tobytes()
    used = np.zeros(case.num_blocks * bs, bool)
    used[case.slot_new] = True
    kflat = kp.reshape(case.num_blocks * bs, -1).view(np.uint8)
    pristine = case.empty_pools()[0].reshape(case.num_blocks * bs, -1).view(np.uint8)
    assert (kflat[~used] == pristine[~used]).all()


def test_store_skips_minus_one_slots():
    """Slot -1 marks a padding token and is skipped (nano-vllm Step 4 store kernel)."""
    kp = np.zeros((2, 4, 1, 2), np.float32)
    vp = kp.copy()
    k = np.ones((3, 1, 2), np.float32) * np.array([1, 2, 3], np.float32)[:, None, None]
    oracle.store_kv(k, k, [5, -1, 0], kp, vp)
    flat = kp.reshape(8, 2)
    assert (flat[5] == 1).all() and (flat[0] == 3).all()
    assert (flat[[1, 2, 3, 4, 6, 7]] == 0).all()


def test_store_rejects_out_of_range_slot():
    kp = np.zeros((2, 4, 1, 2), np.float32)
    with pytest.raises(RuntimeError):
        oracle.store_kv(np.ones((1, 1, 2), np.float32), np.ones((1, 1, 2), np.float32), [8], kp, kp.copy())


# ---------------------------------------------------------------- attention

@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("hq,hkv", [(4, 2), (4, 4), (8, 2), (3, 1)])
def test_identity_table_equals_textbook_causal_sdpa(dtype, hq, hkv):
    """With q_offsets 0 the paged result is dense causal attention
    (torch CPU float64 scaled_dot_product_attention, is_causal=True)."""
    lens = [1, 7, 33]
    d, bs = 16, 4
    case = W.make_prefill("dense", 11 + hq, lens, [0, 0, 0], hq, hkv, d, bs, dtype)
    kp, vp = _case_pools(case)
    out = oracle.prefill(case.q, kp, vp, case.cu_seqlens_q, case.cu_seqlens_k, case.q_offsets,
                         case.block_table, case.scale)
    cu = case.cu_seqlens_q
    for s in range(len(lens)):
        sl = slice(cu[s], cu[s + 1])
        ref = _sdpa_causal(_as_f64(case.q[sl]), _as_f64(case.k_new[sl]), _as_f64(case.v_new[sl]),
                           hq // hkv, case.scale)
        np.testing.assert_allclose(out[sl], ref, rtol=0, atol=1e-12)


def test_prefix_rows_match_bottom_right_tril_mask():
    """'推理系统' notes, KV-cache demo: with T new tokens over S keys the mask is
    ones(T, S).tril(S - T).  Paged prefill with a cached prefix equals SDPA
    under that mask on the gathered keys."""
    case = W.make_prefill("tril", 5, [9, 4], [13, 30], 4, 2, 8, 4, "f32")
    kp, vp = _case_pools(case)
    out = oracle.prefill(case.q, kp, vp, case.cu_seqlens_q, case.cu_seqlens_k, case.q_offsets,
                         case.block_table, case.scale)
    k_all, v_all = oracle.gather_kv(kp, vp, case.cu_seqlens_k, case.block_table)
    cq, ck = case.cu_seqlens_q, case.cu_seqlens_k
    for s in range(2):
        T, S = case.q_lens[s], case.k_lens[s]
        mask = torch.ones(T, S, dtype=torch.bool).tril(S - T)
        ref = _sdpa_causal(_as_f64(case.q[cq[s]:cq[s + 1]]), _as_f64(k_all[ck[s]:ck[s + 1]]),
                           _as_f64(v_all[ck[s]:ck[s + 1]]), 2, case.scale, mask=mask)
        np.testing.assert_allclose(out[cq[s]:cq[s + 1]], ref, rtol=0, atol=1e-12)


def test_suffix_prefill_equals_rows_of_full_prefill():
    """A 300-token prompt with 256 tokens cached prefills only 44 (fork Q&A,
    Q1); those 44 rows equal rows 256..299 of a full prefill (causality:
    earlier positions do not change)."""
    full = W.make_prefill("full", 77, [300, 300], [0, 0], 4, 2, 16, 16, "bf16")
    kp, vp = _case_pools(full)
    o_full = oracle.prefill(full.q, kp, vp, full.cu_seqlens_q, full.cu_seqlens_k, [0, 0],
                            full.block_table, full.scale)
    rows = np.concatenate([np.arange(256, 300), np.arange(556, 600)])
    q_suffix = full.q[rows]
    o_suf = oracle.prefill(q_suffix, kp, vp, [0, 44, 88], full.cu_seqlens_k, [256, 256],
                           full.block_table, full.scale)
    assert o_suf.tobytes() == o_full[rows].tobytes()


def test_decode_equals_last_row_of_prefill():
    full = W.make_prefill("full", 78, [37, 5, 64], [0, 0, 0], 4, 2, 8, 16, "f32")
    kp, vp = _case_pools(full)
    o_full = oracle.prefill(full.q, kp, vp, full.cu_seqlens_q, full.cu_seqlens_k, [0, 0, 0],
                            full.block_table, full.scale)
    last = full.cu_seqlens_q[1:] - 1
    o_dec = oracle.decode(full.q[last], kp, vp, full.k_lens, full.block_table, full.scale)
    assert o_dec.tobytes() == o_full[last].tobytes()


def test_row_subset_equals_rows_of_the_full_prefill():
    """The oracle's rows= path (rows in any order, repeated, from several
    sequences, with cached prefixes and a zero-length sequence) returns, bit
    for bit, the same rows of the full output; its pair count is theirs."""
    case = W.make_prefill("subset", 81, [37, 0, 5, 64, 1], [0, 9, 20, 3, 70], 4, 2, 16, 8, "bf16")
    kp, vp = _case_pools(case)
    full, full_pairs = oracle.prefill(case.q, kp, vp, case.cu_seqlens_q, case.cu_seqlens_k, case.q_offsets,
                                      case.block_table, case.scale, return_pairs=True)
    assert full_pairs == case.causal_pairs
    rows = np.array([106, 0, 41, 36, 41, 37, 42, 105, 5], np.int32)
    sub, pairs = oracle.prefill(case.q, kp, vp, case.cu_seqlens_q, case.cu_seqlens_k, case.q_offsets,
                                case.block_table, case.scale, rows=rows, return_pairs=True)
    assert sub.tobytes() == full[rows].tobytes()
    cu = np.asarray(case.cu_seqlens_q)
    seq_of = np.searchsorted(cu, rows, side="right") - 1
    visible = [min(case.q_offsets[s] + r - cu[s], case.k_lens[s] - 1) + 1 for r, s in zip(rows, seq_of)]
    assert pairs == sum(visible)


def test_sequence_subset_equals_rows_of_the_full_decode():
    """The oracle's seqs= path returns, bit for bit, the same rows of the full
    decode output (a padding row of context 0 included)."""
    case = W.make_decode("subset", 82, [9, 0, 33, 1, 200, 17], 4, 2, 16, 8, "f32")
    kp, vp = case.empty_pools()
    oracle.store_kv(case.k_hist, case.v_hist, case.slot_hist, kp, vp)
    oracle.store_kv(case.k_new, case.v_new, case.slot_new, kp, vp)
    full = oracle.decode(case.q, kp, vp, case.context_lens, case.block_table, case.scale)
    seqs = np.array([4, 1, 0, 4, 5, 2], np.int32)
    sub, pairs = oracle.decode(case.q, kp, vp, case.context_lens, case.block_table, case.scale, seqs=seqs,
                               return_pairs=True)
    assert sub.tobytes() == full[seqs].tobytes()
    assert pairs == int(np.asarray(case.context_lens)[seqs].sum())
    assert (sub[1] == 0).all()


def test_block_permutation_invariance():
    """Only the block table says where a block lives: relabelling physical
    blocks (and the table with them) gives bit-identical results."""
    case = W.make_prefill("perm", 99, [40, 17, 5], [3, 0, 11], 4, 2, 8, 4, "bf16")
    kp, vp = _case_pools(case)
    o1 = oracle.prefill(case.q, kp, vp, case.cu_seqlens_q, case.cu_seqlens_k, case.q_offsets,
                        case.block_table, case.scale)
    rng = np.random.default_rng(3)
    perm = rng.permutation(case.num_blocks)        # new id of old block b is perm[b]
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm], vp2[perm] = kp, vp
    table2 = perm[case.block_table].astype(np.int32)
    o2 = oracle.prefill(case.q, kp2, vp2, case.cu_seqlens_q, case.cu_seqlens_k, case.q_offsets,
                        table2, case.scale)
    assert o1.tobytes() == o2.tobytes()


@pytest.mark.parametrize("n", [1, 2, 5, 40, 257])
def test_pair_count_fresh_prompt(n):
    """vLLM/SGLang labs, section 2: N(N+1)/2 valid causal pairs."""
    case = W.make_prefill("pairs", n, [n], [0], 2, 1, 4, 16, "f32")
    kp, vp = _case_pools(case)
    _, pairs = oracle.prefill(case.q, kp, vp, case.cu_seqlens_q, case.cu_seqlens_k, [0],
                              case.block_table, case.scale, return_pairs=True)
    assert pairs == n * (n + 1) // 2


def test_pair_count_with_prefix():
    case = W.make_prefill("pairs", 8, [44, 7], [256, 3], 2, 1, 4, 16, "f32")
    kp, vp = _case_pools(case)
    _, pairs = oracle.prefill(case.q, kp, vp, case.cu_seqlens_q, case.cu_seqlens_k, case.q_offsets,
                              case.block_table, case.scale, return_pairs=True)
    assert pairs == 44 * 256 + 44 * 45 // 2 + 7 * 3 + 7 * 8 // 2 == case.causal_pairs


def test_single_visible_key_returns_v_exactly():
    """Row 0 of a fresh prompt sees only key 0: its output is V[0] exactly."""
    case = W.make_prefill("one", 5, [6, 1, 19], [0, 0, 0], 4, 2, 32, 16, "bf16")
    kp, vp = _case_pools(case)
    out = oracle.prefill(case.q, kp, vp, case.cu_seqlens_q, case.cu_seqlens_k, [0, 0, 0],
                         case.block_table, case.scale)
    for s in range(3):
        r = case.cu_seqlens_q[s]
        np.testing.assert_array_equal(out[r], np.repeat(_as_f64(case.v_new[r]), 2, axis=0))


def test_two_key_closed_form_pins_scale_and_exp():
    """d=1, q=1, k0=0, k1=ln(3)/scale: weights 1/4, 3/4, so O = v0/4 + 3 v1/4."""
    scale = 0.5
    kp = np.zeros((1, 4, 1, 1), np.float64).astype(np.float32)
    vp = np.zeros_like(kp)
    k = np.array([[[0.0]], [[math.log(3.0) / scale]]], np.float32)
    v = np.array([[[2.0]], [[-6.0]]], np.float32)
    oracle.store_kv(k, v, [0, 1], kp, vp)
    q = np.ones((2, 1, 1), np.float32)
    out = oracle.prefill(q, kp, vp, [0, 2], [0, 2], [0], [[0]], scale)
    k1 = float(k[1, 0, 0])  # the fp32-stored key
    w1 = math.exp(scale * k1) / (1.0 + math.exp(scale * k1))
    assert out[0, 0, 0] == 2.0
    assert abs(out[1, 0, 0] - (2.0 * (1 - w1) - 6.0 * w1)) < 1e-15
    assert abs(out[1, 0, 0] - (-4.0)) < 1e-6


def test_uniform_keys_give_mean_of_values():
    """If every visible key is the same vector, all weights are equal and the
    output is the plain mean of the visible V rows."""
    case = W.make_prefill("uni", 6, [23], [0], 2, 1, 8, 4, "f32")
    case.k_new[:] = case.k_new[0]
    kp, vp = _case_pools(case)
    out = oracle.prefill(case.q, kp, vp, case.cu_seqlens_q, case.cu_seqlens_k, [0],
                         case.block_table, case.scale)
    v = _as_f64(case.v_new)
    for i in range(23):
        np.testing.assert_allclose(out[i], np.repeat(v[:i + 1].mean(axis=0), 2, axis=0), atol=1e-12)


def test_gqa_head_mapping_contiguous_groups():
    """Query head h reads KV head h // (Hq/Hkv): give each KV head a constant V."""
    hq, hkv = 8, 2
    case = W.make_prefill("gqa", 7, [9], [0], hq, hkv, 4, 4, "f32")
    case.v_new[:, 0, :] = 1.0
    case.v_new[:, 1, :] = 2.0
    kp, vp = _case_pools(case)
    out = oracle.prefill(case.q, kp, vp, case.cu_seqlens_q, case.cu_seqlens_k, [0],
                         case.block_table, case.scale)
    for h in range(hq):
        np.testing.assert_allclose(out[:, h, :], 1.0 + (h // (hq // hkv)), atol=1e-12)


@settings(max_examples=25, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), lens=st.lists(st.integers(1, 30), min_size=1, max_size=3),
       offs=st.lists(st.integers(0, 20), min_size=3, max_size=3), bs=st.sampled_from([1, 2, 16]),
       d=st.sampled_from([4, 32]))
def test_random_tiny_against_masked_sdpa_and_convexity(seed, lens, offs, bs, d):
    """Brute force on tiny random shapes: bottom-right masked SDPA on the
    gathered keys, and each output coordinate within [min V, max V]."""
    offs = offs[:len(lens)]
    case = W.make_prefill("rnd", seed, lens, offs, 4, 2, d, bs, "bf16")
    kp, vp = _case_pools(case)
    out = oracle.prefill(case.q, kp, vp, case.cu_seqlens_q, case.cu_seqlens_k, case.q_offsets,
                         case.block_table, case.scale)
    k_all, v_all = oracle.gather_kv(kp, vp, case.cu_seqlens_k, case.block_table)
    cq, ck = case.cu_seqlens_q, case.cu_seqlens_k
    for s in range(len(lens)):
        T, S = case.q_lens[s], case.k_lens[s]
        mask = torch.ones(T, S, dtype=torch.bool).tril(S - T)
        vs = _as_f64(v_all[ck[s]:ck[s + 1]])
        ref = _sdpa_causal(_as_f64(case.q[cq[s]:cq[s + 1]]), _as_f64(k_all[ck[s]:ck[s + 1]]), vs, 2,
                           case.scale, mask=mask)
        np.testing.assert_allclose(out[cq[s]:cq[s + 1]], ref, rtol=0, atol=1e-10)
        lo = np.repeat(vs.min(axis=0), 2, axis=0)
        hi = np.repeat(vs.max(axis=0), 2, axis=0)
        assert (out[cq[s]:cq[s + 1]] >= lo - 1e-12).all() and (out[cq[s]:cq[s + 1]] <= hi + 1e-12).all()


def test_poisoned_unused_slots_do_not_leak():
    """The pool is uninitialised memory (torch.empty in allocate_kv_cache);
    NaN in every slot no sequence uses must not reach the output."""
    case = W.make_prefill("nan", 12, [5, 30], [2, 0], 4, 2, 8, 16, "bf16")
    kp, vp = _case_pools(case)
    out = oracle.prefill(case.q, kp, vp, case.cu_seqlens_q, case.cu_seqlens_k, case.q_offsets,
                         case.block_table, case.scale)
    assert np.isfinite(out).all()
    assert np.isnan(W.bf16_bits_to_f32(kp)).any()


def test_decode_zero_context_is_zero():
    """A padding row of a captured decode batch has context length 0: its
    output is defined as zero."""
    case = W.make_decode("pad", 1, [5, 0, 3], 2, 1, 4, 4, "f32")
    kp, vp = case.empty_pools()
    oracle.store_kv(case.k_hist, case.v_hist, case.slot_hist, kp, vp)
    oracle.store_kv(case.k_new, case.v_new, case.slot_new, kp, vp)
    out = oracle.decode(case.q, kp, vp, case.context_lens, case.block_table, case.scale)
    assert (out[1] == 0).all() and np.isfinite(out).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_decode_equals_unmasked_sdpa_over_context(dtype):
    """A decode query sits at the last position, so it sees every key of its
    context (nano-vllm Step 5, prepare_decode: context length = len(seq)):
    plain unmasked SDPA of one query over the gathered context."""
    case = W.make_decode("dec", 21, [1, 16, 17, 50], 4, 2, 8, 16, dtype)
    kp, vp = case.empty_pools()
    oracle.store_kv(case.k_hist, case.v_hist, case.slot_hist, kp, vp)
    oracle.store_kv(case.k_new, case.v_new, case.slot_new, kp, vp)
    out = oracle.decode(case.q, kp, vp, case.context_lens, case.block_table, case.scale)
    cu = np.concatenate([[0], np.cumsum(case.context_lens)]).astype(np.int32)
    k_all, v_all = oracle.gather_kv(kp, vp, cu, case.block_table)
    for s in range(case.num_seqs):
        n = int(case.context_lens[s])
        mask = torch.ones(1, n, dtype=torch.bool)
        ref = _sdpa_causal(_as_f64(case.q[s:s + 1]), _as_f64(k_all[cu[s]:cu[s + 1]]),
                           _as_f64(v_all[cu[s]:cu[s + 1]]), 2, case.scale, mask=mask)
        np.testing.assert_allclose(out[s:s + 1], ref, rtol=0, atol=1e-12)
