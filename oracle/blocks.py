"""Copy-on-write of a shared, mutable last block: reference.

TEST INFRASTRUCTURE ONLY: imported by the tests, never by the HIP library.

What it follows: "vLLM/SGLang interview source labs", section 4 (does vLLM
beam search fork KV blocks), the follow-up on a native block-table fork:
parent and child share block ids; when an append would land in a shared and
still mutable last block, the child gets a new block, the valid KV is copied
into it, and from then on each writes its own.  Full, immutable blocks are
never copied.  Also the "推理系统" notes, PagedAttention: shared blocks are
copied on write, as in fork.

copy_blocks: for each pair i, slots 0 .. num_valid[i]-1 of block src[i]
(every KV head, K and V, and for INT8 pools the scales too) go to the same
slots of block dst[i]; nothing else changes.
"""
from __future__ import annotations

import numpy as np


def copy_blocks(pools, src_blocks, dst_blocks, num_valid) -> None:
    """pools: arrays shaped [num_blocks, block_size, ...] (K, V, and the INT8
    scale pools if any), modified in place."""
    src = np.asarray(src_blocks, np.int64)
    dst = np.asarray(dst_blocks, np.int64)
    n = np.asarray(num_valid, np.int64)
    assert src.shape == dst.shape == n.shape
    for p in pools:
        nb, bs = p.shape[:2]
        for s, d, k in zip(src, dst, n):
            if not (0 <= s < nb and 0 <= d < nb and 0 <= k <= bs):
                continue
            p[d, :k] = p[s, :k]
