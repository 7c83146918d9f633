"""pa_prefill_varlen on the GPU against the fp64 oracle, element by element
(max-abs 2e-2 for bf16, 1e-5 for fp32), on the configurations and edge cases."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_mapping_amd as pa
import workloads as W
from helpers import host_pools_with_prefix, max_abs_err, say, to_dev, to_host_bits, tol

pytestmark = pytest.mark.gpu


def run_prefill(case, rows=None):
    """Store the new tokens on the GPU, prefill, and return (gpu_out, oracle_out, host pools)."""
    kp, vp = host_pools_with_prefix(case)
    kd, vd = to_dev(kp), to_dev(vp)
    pa.pa_store_kv(to_dev(case.k_new), to_dev(case.v_new), to_dev(case.slot_new), kd, vd)
    oracle.store_kv(case.k_new, case.v_new, case.slot_new, kp, vp)
    out = pa.pa_prefill_varlen(to_dev(case.q), kd, vd, to_dev(case.cu_seqlens_q), to_dev(case.cu_seqlens_k),
                               to_dev(np.asarray(case.q_offsets, np.int32)), to_dev(case.block_table),
                               case.max_seqlen_q, case.max_seqlen_k, case.scale)
    torch.cuda.synchronize()
    ref = oracle.prefill(case.q, kp, vp, case.cu_seqlens_q, case.cu_seqlens_k, case.q_offsets,
                         case.block_table, case.scale, rows=rows)
    got = out if rows is None else out[torch.as_tensor(np.asarray(rows), device=out.device).long()]
    return got, ref, (kp, vp, kd, vd, out)


def test_c1_tiny_fp32():
    pre, _ = W.c1_tiny()
    say("[prefill] c1 fp32")
    got, ref, _ = run_prefill(pre)
    err = max_abs_err(got, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol("f32")


@pytest.mark.parametrize("n", [32, 128, 256])
def test_c2_varlen_bf16(n):
    case = W.c2_varlen(n)
    say(f"[prefill] c2 8x{n}")
    got, ref, _ = run_prefill(case)
    err = max_abs_err(got, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol("bf16")


def test_c3_prefix_suffix_and_full_rows():
    """C3: the 44-token suffix over a cached 256-token block; also equal (within
    tolerance) to rows 256..299 of a full 300-token prefill on the GPU."""
    case = W.c3_prefix()
    say("[prefill] c3 prefix")
    got, ref, (kp, vp, kd, vd, out) = run_prefill(case)
    err = max_abs_err(got, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol("bf16")
    # full prefill of the same 300 tokens (queries of the cached part drawn fresh)
    rng = np.random.default_rng(1)
    q_full = W.normal(rng, (600, 16, 128), "bf16")
    q_full[256:300] = case.q[:44]
    q_full[556:600] = case.q[44:]
    full = pa.pa_prefill_varlen(to_dev(q_full), kd, vd, to_dev(np.array([0, 300, 600], np.int32)),
                                to_dev(case.cu_seqlens_k), to_dev(np.zeros(2, np.int32)),
                                to_dev(case.block_table), 300, 300, case.scale)
    torch.cuda.synchronize()
    rows = np.r_[256:300, 556:600]
    assert max_abs_err(full[torch.as_tensor(rows, device="cuda")], ref) <= tol("bf16")


def test_c5a_long_4096_every_row():
    """C5a-i: all 4096 rows x 16 heads of the long prompt against the oracle
    (every one of the N(N+1)/2 causal pairs contributes to some row)."""
    case = W.c5a_long()
    say("[prefill] c5a 1x4096, every row")
    got, ref, _ = run_prefill(case)
    err = max_abs_err(got, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol("bf16")


def test_c5a_mixed_chunked_every_row():
    """C5a-ii: all 8192 packed rows of the chunked batch against the oracle."""
    case = W.c5a_mixed()
    say(f"[prefill] c5a mixed {case.num_seqs} seqs, every row")
    got, ref, _ = run_prefill(case)
    err = max_abs_err(got, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol("bf16")


@pytest.mark.parametrize("dtype,d,hq,hkv,bs", [
    ("bf16", 128, 16, 8, 16), ("bf16", 64, 8, 1, 32), ("bf16", 128, 4, 4, 1), ("bf16", 32, 4, 2, 16),
    ("bf16", 256, 4, 2, 16), ("f32", 128, 8, 2, 16), ("f32", 64, 8, 8, 4), ("bf16", 128, 32, 4, 64),
    ("bf16", 128, 8, 8, 16), ("bf16", 128, 16, 8, 4), ("bf16", 64, 16, 4, 8), ("bf16", 128, 16, 8, 256),
    ("bf16", 64, 4, 1, 2048),
])
def test_ragged_shapes_and_offsets(dtype, d, hq, hkv, bs):
    """Ragged lengths spanning several tiles plus tails, arbitrary cached
    prefixes (not block aligned), a zero-length sequence in the middle."""
    q_lens = [1, 67, 0, 130, 5, 200]
    q_offs = [0, 13, 9, 0, 250, 61]
    case = W.make_prefill("ragged", 100 + d + hq, q_lens, q_offs, hq, hkv, d, bs, dtype)
    say(f"[prefill] ragged {dtype} d={d} {hq}/{hkv} bs={bs}")
    got, ref, _ = run_prefill(case)
    assert max_abs_err(got, ref) <= tol(dtype)


@pytest.mark.parametrize("dtype,hq,hkv,bs,q_lens,q_offs", [
    ("bf16", 8, 8, 4, [700, 33, 1, 0, 257], [0, 100, 7, 3, 1000]),   # group 1, smallest MFMA block
    ("bf16", 16, 4, 256, [1500, 64], [37, 0]),                        # group 4, block 256
    ("f16", 8, 4, 16, [2048], [0]),                                   # group 2: a long prompt, every row
    ("bf16", 16, 2, 32, [300, 5, 129], [0, 600, 31]),                 # group 8
])
def test_head_dim_256_on_the_matrix_cores(dtype, hq, hkv, bs, q_lens, q_offs):
    """head_dim 256 prefill (4-wave layout, operands read per 32-key block):
    many key steps, ragged tails, cached prefixes, every row against the
    oracle."""
    case = W.make_prefill("d256", 9700 + hq + bs, q_lens, q_offs, hq, hkv, 256, bs, dtype)
    say(f"[prefill] d=256 {dtype} {hq}/{hkv} bs={bs} q={q_lens}")
    got, ref, _ = run_prefill(case)
    err = max_abs_err(got, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol(dtype)


def test_single_visible_key_rows_return_v():
    """Row 0 of a fresh prompt sees key 0 only: the output is V[0] (to bf16 rounding)."""
    case = W.make_prefill("one", 8, [1, 64, 129], [0, 0, 0], 16, 8, 128, 16, "bf16")
    say("[prefill] single-key rows")
    got, ref, _ = run_prefill(case)
    for s in range(3):
        r = int(case.cu_seqlens_q[s])
        g = to_host_bits(got[r])
        v = np.repeat(case.v_new[r], 2, axis=0)
        assert (g == v).all()


def test_block_permutation_invariance_and_determinism():
    case = W.make_prefill("perm", 9, [300, 77], [20, 0], 16, 8, 128, 16, "bf16")
    say("[prefill] permutation + determinism")
    got, ref, (kp, vp, kd, vd, out) = run_prefill(case)
    q = to_dev(case.q)
    args = (to_dev(case.cu_seqlens_q), to_dev(case.cu_seqlens_k), to_dev(np.asarray(case.q_offsets, np.int32)))
    again = pa.pa_prefill_varlen(q, kd, vd, *args, to_dev(case.block_table), case.max_seqlen_q,
                                 case.max_seqlen_k, case.scale)
    perm = np.random.default_rng(2).permutation(case.num_blocks)
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm], vp2[perm] = kp, vp
    perm_out = pa.pa_prefill_varlen(q, to_dev(kp2), to_dev(vp2), *args,
                                    to_dev(perm[case.block_table].astype(np.int32)), case.max_seqlen_q,
                                    case.max_seqlen_k, case.scale)
    torch.cuda.synchronize()
    assert to_host_bits(again).tobytes() == to_host_bits(out).tobytes()
    assert max_abs_err(perm_out, ref) <= tol("bf16")


@pytest.mark.parametrize("direction", ["rising", "falling"])
def test_steep_score_ramp(direction):
    """Every key's score is a ramp along the sequence spanning about 200 in
    log2 units over 1024 keys (q = 40u, k_j = 40 (j/1024) u for a unit vector
    u, or the ramp reversed): rising scores keep moving the softmax's running
    reference past its bound, so its rescale path runs over and over; falling
    scores make every later key underflow against the first block."""
    case = W.make_prefill("ramp", 7100, [1024], [0], 16, 8, 128, 16, "bf16")
    rng = np.random.default_rng(7101)
    u = rng.standard_normal(128)
    u /= np.linalg.norm(u)
    ramp = 40.0 * np.arange(1024) / 1024.0
    if direction == "falling":
        ramp = ramp[::-1].copy()
    case.q = W.f32_to_bf16_bits(np.broadcast_to(40.0 * u, (1024, 16, 128)).astype(np.float32))
    case.k_new = W.f32_to_bf16_bits(
        np.broadcast_to(ramp[:, None, None] * u[None, None, :], (1024, 8, 128)).astype(np.float32))
    say(f"[prefill] steep {direction} score ramp")
    got, ref, _ = run_prefill(case)
    err = max_abs_err(got, ref)
    say(f"  max-abs {err:.3e}")
    assert np.isfinite(got.float().cpu().numpy()).all()
    assert err <= tol("bf16")


def test_shared_prefix_blocks():
    """Two sequences whose block tables point at the same physical blocks for
    a 256-token cached prefix (read-only sharing, as reference-counted prefix
    blocks are): each attends to the shared keys exactly as to its own.  The
    second sequence's original prefix blocks stay NaN-poisoned and unused."""
    case = W.make_prefill("shared", 7200, [40, 70], [256, 256], 16, 8, 128, 16, "bf16")
    shared = 256 // 16
    case.block_table[1, :shared] = case.block_table[0, :shared]
    case.slot_cached = case.slot_cached[:256]
    case.k_cached, case.v_cached = case.k_cached[:256], case.v_cached[:256]
    say("[prefill] shared prefix blocks")
    got, ref, _ = run_prefill(case)
    assert max_abs_err(got, ref) <= tol("bf16")


@pytest.mark.parametrize("pad", [-1, 2**31 - 1])
def test_table_padding_is_never_read(pad):
    """Entries of a block-table row past the sequence's last needed block
    are never read: padding them with -1 or a huge id changes no output bit."""
    case = W.make_prefill("pad", 7300, [5, 70, 300, 17], [0, 30, 0, 200], 16, 8, 128, 16, "bf16")
    say(f"[prefill] table padding {pad}")
    base, ref, (kp, vp, kd, vd, _) = run_prefill(case)
    assert max_abs_err(base, ref) <= tol("bf16")
    bt = case.block_table.copy()
    for s, k in enumerate(case.k_lens):
        bt[s, -(-k // case.block_size):] = pad
    again = pa.pa_prefill_varlen(to_dev(case.q), kd, vd, to_dev(case.cu_seqlens_q), to_dev(case.cu_seqlens_k),
                                 to_dev(np.asarray(case.q_offsets, np.int32)), to_dev(bt), case.max_seqlen_q,
                                 case.max_seqlen_k, case.scale)
    torch.cuda.synchronize()
    assert to_host_bits(again).tobytes() == to_host_bits(base).tobytes()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_mixed_decode_rows_and_chunks_in_one_launch(dtype):
    """A mixed batch in one pa_prefill_varlen launch: 24 decode rows (one new
    token after contexts of up to 2000 keys) beside 2 prefill chunks, as a
    decode-first scheduler packs them (fork Q&A, Q2: shared token budget)."""
    rng = np.random.default_rng(7500)
    ctx = rng.integers(1, 2000, size=24)
    q_lens = [1] * 24 + [300, 77]
    q_offs = [int(c) for c in ctx] + [0, 512]
    case = W.make_prefill("mixed", 7500, q_lens, q_offs, 16, 8, 128, 16, dtype)
    say(f"[prefill] mixed batch: 24 decode rows + 2 chunks, {dtype}")
    got, ref, _ = run_prefill(case)
    err = max_abs_err(got, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol(dtype)


@pytest.mark.parametrize("dtype,d,hq,hkv,bs", [
    ("bf16", 128, 16, 8, 16), ("bf16", 64, 8, 1, 32), ("bf16", 128, 4, 4, 16), ("bf16", 64, 16, 4, 8),
    ("f16", 128, 16, 8, 256), ("f16", 64, 8, 2, 16), ("bf16", 128, 32, 4, 16),
])
def test_many_short_sequences_two_workgroups_per_cu(dtype, d, hq, hkv, bs):
    """80 sequences of 1..200 new tokens after 0..300 cached ones: the launch
    has more workgroups than CUs, which selects the 4-wave layout (two
    workgroups per CU, 64-key steps, no key-half merge)."""
    rng = np.random.default_rng(7600 + d + hq + hkv)
    q_lens = rng.integers(1, 200, size=80, endpoint=True).tolist()
    q_offs = rng.integers(0, 300, size=80, endpoint=True).tolist()
    case = W.make_prefill("many", 7600 + d + hq, q_lens, q_offs, hq, hkv, d, bs, dtype)
    nh = min(hq // hkv, 4)
    pairs = (-(-case.max_seqlen_q // (32 * (4 // nh))) + 1) // 2
    assert 80 * pairs * (hq // hkv // nh) * hkv > 256, "the case must exceed one workgroup per CU"
    say(f"[prefill] 80 short sequences {dtype} d={d} {hq}/{hkv} bs={bs}")
    got, ref, _ = run_prefill(case)
    err = max_abs_err(got, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol(dtype)


@pytest.mark.parametrize("n,length,hq,hkv", [(67, 96, 16, 8), (64, 128, 16, 8), (9, 300, 8, 2)])
def test_equal_length_sequences_in_groups(n, length, hq, hkv):
    """Equal new-token counts (total_q = n * max_seqlen_q) deal single tiles
    sequence group by sequence group (4 at a time, the last group short when
    4 does not divide n), cached prefixes of different lengths included."""
    rng = np.random.default_rng(7700 + n)
    q_offs = rng.integers(0, 200, size=n, endpoint=True).tolist()
    case = W.make_prefill("equal", 7700 + n, [length] * n, q_offs, hq, hkv, 128, 16, "bf16")
    say(f"[prefill] {n} x {length} equal-length sequences, {hq}/{hkv}")
    got, ref, _ = run_prefill(case)
    err = max_abs_err(got, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol("bf16")


@pytest.mark.parametrize("q_lens,q_offs,units", [
    ([1024, 1000], [0, 37], "single tiles that exactly fill the CUs (256 workgroups, 8-wave)"),
    ([1000, 1024, 990, 1017], [0, 24, 3, 100], "tile pairs of several sequences (256 workgroups, 8-wave)"),
    ([700, 64, 1024, 5, 300, 999], [0, 900, 0, 17, 0, 1], "single tiles longest first (4-wave)"),
])
def test_work_units_across_sequences(q_lens, q_offs, units):
    """Each work-unit choice of the launch (pairs of query tiles, single tiles
    fitting the CUs, single tiles dispatched longest first) over several
    sequences with cached prefixes: every row against the oracle."""
    case = W.make_prefill("units", 9500 + len(q_lens), q_lens, q_offs, 16, 8, 128, 16, "bf16")
    say(f"[prefill] {units}: {case.total_q} rows")
    got, ref, _ = run_prefill(case)
    err = max_abs_err(got, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= tol("bf16")
