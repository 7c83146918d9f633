"""Seeded synthetic inputs for paged-KV attention at Qwen3-0.6B attention shapes.

This module is shared by the tests, the benchmark and the smoke check.  It
holds none of the attention arithmetic: it draws lengths, deals physical
blocks, lays out slot mappings the way an engine's host-side metadata
builder does (nano-vllm deep dive, Step 5, prepare_prefill / prepare_decode),
and draws N(0,1) values.  Everything is a pure function of the seed.

Data conventions
  * bf16 tensors travel as uint16 bit patterns (numpy has no bf16); values are
    drawn in fp32 and rounded to nearest-even to bf16.  fp16 tensors are numpy
    float16 (the same fp32 draw, rounded to nearest-even by numpy's cast).
  * Pools are [num_blocks, block_size, num_kv_heads, head_dim]; every slot no
    sequence uses is filled with a quiet-NaN pattern ("poisoned").
  * block_table rows are padded past a sequence's last block with the id of a
    spare, poisoned block, so a kernel that read past the valid entries would
    return NaN instead of faulting.

Workloads (C1..C5) follow the configuration list the benchmark reports on.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

NAN_BF16 = np.uint16(0x7FC0)
NAN_F16 = np.uint16(0x7E00)
NAN_F32_BITS = np.uint32(0x7FC00000)

# Qwen3-0.6B attention shapes: 28 layers, 16 query heads, 8 KV heads, head_dim 128.
QWEN3_LAYERS = 28
QWEN3_HQ = 16
QWEN3_HKV = 8
QWEN3_D = 128


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest-even), returning uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + bias) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = NAN_BF16
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def np_dtype(dtype: str):
    return {"bf16": np.uint16, "f16": np.float16, "f32": np.float32}[dtype]


def elem_bytes(dtype: str) -> int:
    return 4 if dtype == "f32" else 2


def normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x.astype(np.float16) if dtype == "f16" else x


def poisoned_pool(num_blocks: int, block_size: int, hkv: int, d: int, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return np.full((num_blocks, block_size, hkv, d), NAN_BF16, dtype=np.uint16)
    if dtype == "f16":
        return np.full((num_blocks, block_size, hkv, d), NAN_F16, dtype=np.uint16).view(np.float16)
    return np.full((num_blocks, block_size, hkv, d), NAN_F32_BITS, dtype=np.uint32).view(np.float32)


def _deal_blocks(rng, lens, block_size, num_spare):
    """Shuffle physical ids and hand them to sequences in order.

    Returns (block_table int32 [B, W], num_blocks, spare_ids).  W is the most
    blocks any sequence needs (at least 1)."""
    need = [max(1, -(-int(n) // block_size)) for n in lens]
    num_blocks = sum(need) + num_spare
    perm = rng.permutation(num_blocks).astype(np.int32)
    width = max(need) if need else 1
    spare = perm[sum(need):]
    pad = int(spare[0]) if len(spare) else int(perm[0])
    table = np.full((len(lens), width), pad, dtype=np.int32)
    pos = 0
    for s, n in enumerate(need):
        table[s, :n] = perm[pos:pos + n]
        pos += n
    return table, num_blocks, spare


def slots_for(table_row: np.ndarray, positions, block_size: int) -> np.ndarray:
    """Flat cache slots of logical positions of one sequence (the engine's
    slot_mapping: physical block id * block_size + offset in block)."""
    positions = np.asarray(positions, dtype=np.int64)
    return (table_row[positions // block_size].astype(np.int64) * block_size
            + positions % block_size).astype(np.int32)


@dataclass
class PrefillCase:
    """One packed varlen prefill batch over a paged cache."""
    name: str
    seed: int
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    q_lens: list
    k_lens: list
    q_offsets: list
    block_table: np.ndarray
    slot_new: np.ndarray          # int32 [total_q]: slots of the new tokens
    slot_cached: np.ndarray       # int32 [total_cached]: slots of the cached prefix
    q: np.ndarray | None = None   # [total_q, Hq, D]
    k_new: np.ndarray | None = None
    v_new: np.ndarray | None = None
    k_cached: np.ndarray | None = None
    v_cached: np.ndarray | None = None
    spare_blocks: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))

    @property
    def num_seqs(self):
        return len(self.q_lens)

    @property
    def cu_seqlens_q(self):
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    @property
    def cu_seqlens_k(self):
        return np.concatenate([[0], np.cumsum(self.k_lens)]).astype(np.int32)

    @property
    def total_q(self):
        return int(sum(self.q_lens))

    @property
    def max_seqlen_q(self):
        return int(max(self.q_lens)) if self.q_lens else 0

    @property
    def max_seqlen_k(self):
        return int(max(self.k_lens)) if self.k_lens else 0

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def causal_pairs(self):
        """Visible (query, key) pairs: q_len*q_off + q_len(q_len+1)/2 per sequence."""
        return int(sum(ql * qo + ql * (ql + 1) // 2 for ql, qo in zip(self.q_lens, self.q_offsets)))

    def empty_pools(self):
        k = poisoned_pool(self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim, self.dtype)
        return k, k.copy()


@dataclass
class DecodeCase:
    """One query token per sequence over its paged context (new token included)."""
    name: str
    seed: int
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    context_lens: np.ndarray      # int32 [B], counts the new token
    block_table: np.ndarray
    slot_new: np.ndarray          # int32 [B]: slot of position ctx-1
    slot_hist: np.ndarray         # int32 [sum(ctx-1)]: slots of earlier positions
    q: np.ndarray | None = None
    k_new: np.ndarray | None = None
    v_new: np.ndarray | None = None
    k_hist: np.ndarray | None = None
    v_hist: np.ndarray | None = None
    spare_blocks: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))

    @property
    def num_seqs(self):
        return len(self.context_lens)

    @property
    def max_context_len(self):
        return int(self.context_lens.max()) if len(self.context_lens) else 0

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.head_dim)

    def kv_bytes(self):
        """Bytes of K and V one decode pass must read: each visible row once per KV head."""
        eb = elem_bytes(self.dtype)
        return int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads * self.head_dim * eb * 2

    def empty_pools(self):
        k = poisoned_pool(self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim, self.dtype)
        return k, k.copy()


def make_prefill(name, seed, q_lens, q_offsets, hq, hkv, d, block_size, dtype, num_spare=2,
                 with_values=True) -> PrefillCase:
    """A packed batch: sequence s has q_offsets[s] cached tokens and q_lens[s] new ones."""
    rng = np.random.default_rng(seed)
    q_lens = [int(x) for x in q_lens]
    q_offsets = [int(x) for x in q_offsets]
    k_lens = [a + b for a, b in zip(q_lens, q_offsets)]
    table, nb, spare = _deal_blocks(rng, k_lens, block_size, num_spare)
    slot_new, slot_cached = [], []
    for s in range(len(q_lens)):
        slot_cached.append(slots_for(table[s], range(q_offsets[s]), block_size))
        slot_new.append(slots_for(table[s], range(q_offsets[s], k_lens[s]), block_size))
    case = PrefillCase(name, seed, dtype, hq, hkv, d, block_size, nb, q_lens, k_lens, q_offsets, table,
                       np.concatenate(slot_new).astype(np.int32) if slot_new else np.zeros(0, np.int32),
                       np.concatenate(slot_cached).astype(np.int32) if slot_cached else np.zeros(0, np.int32),
                       spare_blocks=spare)
    if with_values:
        tq, tc = case.total_q, len(case.slot_cached)
        case.q = normal(rng, (tq, hq, d), dtype)
        case.k_new = normal(rng, (tq, hkv, d), dtype)
        case.v_new = normal(rng, (tq, hkv, d), dtype)
        case.k_cached = normal(rng, (tc, hkv, d), dtype)
        case.v_cached = normal(rng, (tc, hkv, d), dtype)
    return case


def make_decode(name, seed, context_lens, hq, hkv, d, block_size, dtype, num_spare=2,
                with_values=True) -> DecodeCase:
    rng = np.random.default_rng(seed)
    ctx = np.asarray(context_lens, dtype=np.int32)
    table, nb, spare = _deal_blocks(rng, ctx.tolist(), block_size, num_spare)
    slot_new = np.zeros(len(ctx), np.int32)
    hist = []
    for s, n in enumerate(ctx.tolist()):
        if n > 0:
            slot_new[s] = slots_for(table[s], [n - 1], block_size)[0]
            hist.append(slots_for(table[s], range(n - 1), block_size))
        else:
            slot_new[s] = -1  # a padding row: nothing to store, nothing to attend
    case = DecodeCase(name, seed, dtype, hq, hkv, d, block_size, nb, ctx, table, slot_new,
                      np.concatenate(hist).astype(np.int32) if hist else np.zeros(0, np.int32),
                      spare_blocks=spare)
    if with_values:
        b, th = len(ctx), len(case.slot_hist)
        case.q = normal(rng, (b, hq, d), dtype)
        case.k_new = normal(rng, (b, hkv, d), dtype)
        case.v_new = normal(rng, (b, hkv, d), dtype)
        case.k_hist = normal(rng, (th, hkv, d), dtype)
        case.v_hist = normal(rng, (th, hkv, d), dtype)
    return case


# --------------------------------------------------------------------------
# The five configurations.
# --------------------------------------------------------------------------

def c1_tiny(seed=1001):
    """3 sequences, prompts {5,17,40}, 4 q / 2 kv heads, d=32, fp32, block 16,
    a 16-block pool dealt from a seeded permutation; causal prefill, then 4
    decode steps per sequence (contexts end at 9, 21, 44).

    Returns (prefill_case, decode_steps) where every decode step is a dict with
    q [3,4,32], k_new / v_new [3,2,32], slot_new [3], context_lens [3]."""
    rng = np.random.default_rng(seed)
    prompts = [5, 17, 40]
    steps = 4
    bs, hq, hkv, d, nb = 16, 4, 2, 32, 16
    need = [-(-(n + steps) // bs) for n in prompts]
    perm = rng.permutation(nb).astype(np.int32)
    spare = perm[sum(need):]
    table = np.full((3, max(need)), spare[0], dtype=np.int32)
    pos = 0
    for s, n in enumerate(need):
        table[s, :n] = perm[pos:pos + n]
        pos += n
    slot_new = np.concatenate([slots_for(table[s], range(n), bs) for s, n in enumerate(prompts)])
    pre = PrefillCase("c1_prefill", seed, "f32", hq, hkv, d, bs, nb, prompts, list(prompts), [0, 0, 0],
                      table, slot_new.astype(np.int32), np.zeros(0, np.int32), spare_blocks=spare)
    tq = sum(prompts)
    pre.q = normal(rng, (tq, hq, d), "f32")
    pre.k_new = normal(rng, (tq, hkv, d), "f32")
    pre.v_new = normal(rng, (tq, hkv, d), "f32")
    pre.k_cached = np.zeros((0, hkv, d), np.float32)
    pre.v_cached = np.zeros((0, hkv, d), np.float32)
    dec = []
    for t in range(steps):
        lens = np.array([n + t for n in prompts], dtype=np.int32)  # tokens before this step
        dec.append(dict(
            q=normal(rng, (3, hq, d), "f32"),
            k_new=normal(rng, (3, hkv, d), "f32"),
            v_new=normal(rng, (3, hkv, d), "f32"),
            slot_new=np.array([slots_for(table[s], [lens[s]], bs)[0] for s in range(3)], np.int32),
            context_lens=(lens + 1).astype(np.int32),
        ))
    return pre, dec


def c2_varlen(n, seed=None, with_values=True, dtype="bf16"):
    """8 sequences x n tokens (n in {32,128,256}), fresh prompts, 16/8 heads,
    d=128, bf16, block 256; 16-block pool (8 used, 8 spare), shuffled."""
    seed = {32: 2032, 128: 2128, 256: 2256}.get(n, 2000 + n) if seed is None else seed
    return make_prefill(f"c2_varlen_8x{n}", seed, [n] * 8, [0] * 8, QWEN3_HQ, QWEN3_HKV, QWEN3_D,
                        256, dtype, num_spare=8, with_values=with_values)


def c3_prefix(seed=3300, with_values=True, dtype="bf16"):
    """2 sequences of 300 tokens whose first 256 tokens sit in one cached block
    each; only the 44-token suffix is prefilled (q_offsets = 256)."""
    return make_prefill("c3_prefix_2x(256+44)", seed, [44, 44], [256, 256], QWEN3_HQ, QWEN3_HKV,
                        QWEN3_D, 256, dtype, num_spare=4, with_values=with_values)


def c4_decode_layout(seed=4000, dtype="bf16"):
    """256 sequences, context lengths uniform in [100, 2048], block 256; the
    block table and lengths are shared by all 28 layers.  Values are drawn per
    layer (seed 4100 + layer) by the caller, on the device for timing."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(100, 2048, size=256, endpoint=True).astype(np.int32)
    return make_decode("c4_decode_256xU[100,2048]", seed, ctx, QWEN3_HQ, QWEN3_HKV, QWEN3_D, 256,
                       dtype, num_spare=2, with_values=False)


def c5a_long(seed=5096, with_values=True, dtype="bf16"):
    """1 sequence x 4096-token causal prefill, block 16, 16 spare blocks."""
    return make_prefill("c5a_prefill_1x4096", seed, [4096], [0], QWEN3_HQ, QWEN3_HKV, QWEN3_D, 16,
                        dtype, num_spare=16, with_values=with_values)


def c5a_mixed(seed=5192, budget=8192, with_values=True, dtype="bf16"):
    """Chunked-prefill batch under an 8192-token budget: prompt lengths uniform
    in [100, 1024]; sequence 0 resumes with a cached prefix uniform in
    [1, L0-1]; fresh prompts follow; the last one is cut so the new tokens
    sum to the budget exactly.  Block 16, ~5% spare blocks."""
    rng = np.random.default_rng(seed)
    q_lens, q_offs = [], []
    L0 = int(rng.integers(100, 1024, endpoint=True))
    c0 = int(rng.integers(1, L0 - 1, endpoint=True))
    q_lens.append(L0 - c0)
    q_offs.append(c0)
    while sum(q_lens) < budget:
        L = int(rng.integers(100, 1024, endpoint=True))
        q_lens.append(min(L, budget - sum(q_lens)))
        q_offs.append(0)
    k_total_blocks = sum(-(-(a + b) // 16) for a, b in zip(q_lens, q_offs))
    return make_prefill("c5a_mixed_chunked_8192", seed + 1, q_lens, q_offs, QWEN3_HQ, QWEN3_HKV,
                        QWEN3_D, 16, dtype, num_spare=max(1, k_total_blocks // 20),
                        with_values=with_values)


def c5b_decode_layout(seed=5327, dtype="bf16"):
    """64 sequences x 32768-token contexts, block 16 (131072 blocks + spare)."""
    ctx = np.full(64, 32768, dtype=np.int32)
    return make_decode("c5b_decode_64x32768", seed, ctx, QWEN3_HQ, QWEN3_HKV, QWEN3_D, 16, dtype,
                       num_spare=16, with_values=False)


def fork_microbench_decode(seed=8512, dtype="f16", block_size=256, with_values=True):
    """The fork's fused-dequantization microbenchmark shape (LLM inference
    interview notes (nano-vllm fork), Q3, INT8-versus-FP16 latency table):
    batch 8, 16 query / 8 KV heads, head_dim 128, fp16.  Its cache-byte
    column counts 512 tokens per sequence, so the 511 cached tokens plus the
    token being decoded give 512 visible keys per row."""
    return make_decode("fork_microbench_decode_8x512", seed, [512] * 8, QWEN3_HQ, QWEN3_HKV, QWEN3_D,
                       block_size, dtype, num_spare=2, with_values=with_values)


# --------------------------------------------------------------------------
# Device-side value fill for the large configurations (values do not affect
# timing; the same seed reproduces the same bits).
# --------------------------------------------------------------------------

def device_normal(shape, seed, device="cuda", dtype="bf16"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    return t.to(torch.float16) if dtype == "f16" else t
