"""INT8 KV cache reference: quantize on store, dequantize for attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the HIP library.

What it follows: "LLM inference interview notes (nano-vllm fork)", Q3
("how are quantization and dequantization done"), part 1 (quantize on
write, inside the store kernel) and part 2 (fused dequantization on read).

  * grain: one scale per (token, KV head), over the head_dim values of that
    head vector;
  * scale = max(max_i |x_i| / 127, 1e-8), computed in fp32 and stored as
    fp16 (round to nearest even);
  * code_i = x_i / scale (fp32, with the fp32 scale), then rounded half away
    from zero: add +0.5 to non-negative values and -0.5 to negative ones, then
    truncate toward zero to int8.  The largest |x_i| lands on +-127 exactly
    (127.5 truncates to 127), so no clamp is needed;
  * dequantized value = float(code) * float(stored fp16 scale).

The quantizer takes its integer decisions in fp32, the precision of the
pages' kernel; the dequantized values are exact in fp32 (an int8 times an
fp16 needs 18 significant bits), so attention over them is the plain fp64
attention of the bf16 oracle applied to fp32 pools.

Pools: data [num_blocks, block_size, kv_heads, head_dim] int8, scales
[num_blocks, block_size, kv_heads] float16; both indexed by the same slot.
"""
from __future__ import annotations

import numpy as np

from . import oracle as _o

_HALF = np.float32(0.5)
_QMAX = np.float32(127.0)
_FLOOR = np.float32(1.0e-8)


def widen(x: np.ndarray) -> np.ndarray:
    """Exact fp32 view of stored model values (bf16 bit patterns, fp16 or fp32)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32)
    if x.dtype == np.float16:
        return x.astype(np.float32)
    assert x.dtype == np.float32
    return x


def quantize(x: np.ndarray):
    """Quantize head vectors x[..., head_dim] (bf16 bits, fp16 or fp32).

    Returns (codes int8 [..., head_dim], scale float32 [...], stored scale
    float16 [...]).
    """
    xf = widen(x)
    amax = np.max(np.abs(xf), axis=-1)                                  # fp32, exact
    scale = np.maximum((amax / _QMAX).astype(np.float32), _FLOOR)      # fp32 division, floor 1e-8
    qf = (xf / scale[..., None]).astype(np.float32)                    # fp32 division
    r = np.where(qf >= 0, qf + _HALF, qf - _HALF).astype(np.float32)   # half away from zero ...
    codes = np.trunc(r).astype(np.int8)                                # ... then toward zero
    return codes, scale, scale.astype(np.float16)


def dequantize(codes: np.ndarray, scale16: np.ndarray) -> np.ndarray:
    """float(code) * float(scale) per element; exact in fp32."""
    return codes.astype(np.float32) * scale16.astype(np.float32)[..., None]


def store_kv(k, v, slot_mapping, kq_pool, vq_pool, ks_pool, vs_pool) -> None:
    """Quantize k/v [T, Hkv, D] per (token, head) into the int8 pools and
    their fp16 scale pools, at flat slot slot_mapping[t]; slot -1 is skipped
    (nano-vllm deep dive, Step 4, "Triton Kernel: write KV Cache")."""
    nb, bs, hkv, d = kq_pool.shape
    assert vq_pool.shape == kq_pool.shape and ks_pool.shape == vs_pool.shape == (nb, bs, hkv)
    assert kq_pool.dtype == vq_pool.dtype == np.int8 and ks_pool.dtype == vs_pool.dtype == np.float16
    slots = np.asarray(slot_mapping, dtype=np.int64)
    k = np.asarray(k).reshape(len(slots), hkv, d)
    v = np.asarray(v).reshape(len(slots), hkv, d)
    kc, _, ks = quantize(k)
    vc, _, vs = quantize(v)
    kq = kq_pool.reshape(nb * bs, hkv, d)
    vq = vq_pool.reshape(nb * bs, hkv, d)
    ksf = ks_pool.reshape(nb * bs, hkv)
    vsf = vs_pool.reshape(nb * bs, hkv)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        assert s < nb * bs
        kq[s] = kc[t]
        vq[s] = vc[t]
        ksf[s] = ks[t]
        vsf[s] = vs[t]


def dequantize_pools(kq_pool, vq_pool, ks_pool, vs_pool):
    """fp32 [NB, bs, Hkv, D] pools holding the dequantized values."""
    return dequantize(kq_pool, ks_pool), dequantize(vq_pool, vs_pool)


def prefill(q, kq_pool, vq_pool, ks_pool, vs_pool, cu_seqlens_q, cu_seqlens_k, q_offsets, block_table, scale,
            rows=None):
    """fp64 causal attention of q (bf16 bits, fp16 or fp32) over the dequantized pools."""
    kf, vf = dequantize_pools(kq_pool, vq_pool, ks_pool, vs_pool)
    return _o.prefill(widen(q), kf, vf, cu_seqlens_q, cu_seqlens_k, q_offsets, block_table, scale, rows=rows)


def decode(q, kq_pool, vq_pool, ks_pool, vs_pool, context_lens, block_table, scale, seqs=None):
    """fp64 decode attention of q (bf16 bits, fp16 or fp32) over the dequantized pools."""
    kf, vf = dequantize_pools(kq_pool, vq_pool, ks_pool, vs_pool)
    return _o.decode(widen(q), kf, vf, context_lens, block_table, scale, seqs=seqs)
