"""ctypes binding of libpa.so (C ABI in include/pa.h).

Argument marshalling only: tensors hand over data_ptr(), shapes and the
current HIP stream; every step of the computation runs in the HIP kernels.
There is no CPU fallback: if the library is missing or a call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpa.so")

PA_F32 = 0
PA_BF16 = 1
PA_INT8 = 2
PA_F16 = 3

_STATUS = {
    0: "PA_OK", 1: "PA_ERR_NULL_ARG", 2: "PA_ERR_BAD_SHAPE", 3: "PA_ERR_BAD_DTYPE",
    4: "PA_ERR_UNSUPPORTED", 5: "PA_ERR_WORKSPACE", 6: "PA_ERR_HIP", 7: "PA_ERR_BAD_METADATA",
}

# Every symbol include/pa.h declares.
EXPORTS = (
    "pa_store_kv", "pa_store_kv_int8", "pa_prefill_varlen", "pa_decode", "pa_decode_static", "pa_decode_int8",
    "pa_decode_int8_workspace_bytes", "pa_prefill_varlen_int8", "pa_prefill_int8_workspace_bytes",
    "pa_decode_order", "pa_copy_blocks",
    "pa_prefill_workspace_bytes",
    "pa_decode_workspace_bytes", "pa_gather_kv", "pa_validate_prefill_metadata",
    "pa_validate_decode_metadata", "pa_status_string", "pa_abi_version",
)


class PaPool(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int64), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class PaError(RuntimeError):
    def __init__(self, fn, code, why=""):
        self.code = code
        msg = f"{fn} failed: {_STATUS.get(code, code)}"
        super().__init__(msg + (f" ({why})" if why else ""))


_lib = None


def load() -> ctypes.CDLL:
    """Load libpa.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m paged_kv_attention_mapping_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    p, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    pool = ctypes.POINTER(PaPool)
    lib.pa_store_kv.argtypes = [p, i64, p, i64, p, i32, p, p, pool, p]
    lib.pa_store_kv_int8.argtypes = [p, i64, p, i64, i32, p, i32, p, p, p, p, pool, p]
    lib.pa_copy_blocks.argtypes = [p, p, p, p, pool, p, p, p, i32, p]
    lib.pa_prefill_varlen.argtypes = [p, i64, i32, p, p, pool, p, p, p, p, i32, i32, i32, i32, i32, f32,
                                      p, p, sz, p]
    lib.pa_decode.argtypes = [p, i64, i32, p, p, pool, p, p, i32, i32, i32, f32, p, p, p, sz, p]
    lib.pa_decode_static.argtypes = [p, i64, i32, p, p, pool, p, p, i32, i32, i32, f32, p, p, p]
    lib.pa_decode_int8.argtypes = [p, i64, i32, i32, p, p, p, p, pool, p, p, i32, i32, i32, f32, p, p, p, sz, p]
    lib.pa_decode_int8_workspace_bytes.argtypes = [i32, i32, i32, pool]
    lib.pa_decode_int8_workspace_bytes.restype = sz
    lib.pa_prefill_varlen_int8.argtypes = [p, i64, i32, i32, p, p, p, p, pool, p, p, p, p, i32, i32, i32, i32,
                                           i32, f32, p, p, sz, p]
    lib.pa_prefill_int8_workspace_bytes.argtypes = [i32, i32, i32, i32, pool]
    lib.pa_prefill_int8_workspace_bytes.restype = sz
    lib.pa_decode_order.argtypes = [p, i32, p, p]
    lib.pa_prefill_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, pool]
    lib.pa_prefill_workspace_bytes.restype = sz
    lib.pa_decode_workspace_bytes.argtypes = [i32, i32, i32, pool]
    lib.pa_decode_workspace_bytes.restype = sz
    lib.pa_gather_kv.argtypes = [p, p, pool, p, p, i32, i32, i32, p, p, p]
    lib.pa_validate_prefill_metadata.argtypes = [p, p, p, p, i32, i32, i32, i32, p, i32, pool, p, sz]
    lib.pa_validate_decode_metadata.argtypes = [p, p, i32, i32, i32, p, p, pool, p, sz]
    lib.pa_status_string.argtypes = [i32]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_abi_version.restype = ctypes.c_int
    for fn in ("pa_store_kv", "pa_store_kv_int8", "pa_prefill_varlen", "pa_prefill_varlen_int8", "pa_decode",
               "pa_decode_static", "pa_decode_int8", "pa_decode_order", "pa_copy_blocks", "pa_gather_kv",
               "pa_validate_prefill_metadata", "pa_validate_decode_metadata"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


# ---------------------------------------------------------------- marshalling

def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype == torch.float16:
        return PA_F16
    raise TypeError(f"unsupported dtype {t.dtype} (float32, bfloat16 or float16)")


def pool_desc(k_pool: torch.Tensor) -> PaPool:
    if k_pool.dim() != 4 or not k_pool.is_contiguous():
        raise ValueError("pools must be contiguous [num_blocks, block_size, num_kv_heads, head_dim]")
    nb, bs, hkv, d = k_pool.shape
    return PaPool(nb, bs, hkv, d, _dtype_code(k_pool))


def pool_desc_int8(k_pool: torch.Tensor, k_scale: torch.Tensor) -> PaPool:
    """Descriptor of an INT8 layer: int8 codes [NB, bs, Hkv, D] and float16
    scales [NB, bs, Hkv], both contiguous."""
    if k_pool.dim() != 4 or not k_pool.is_contiguous() or k_pool.dtype != torch.int8:
        raise ValueError("INT8 pools must be contiguous int8 [num_blocks, block_size, num_kv_heads, head_dim]")
    nb, bs, hkv, d = k_pool.shape
    if k_scale.shape != (nb, bs, hkv) or k_scale.dtype != torch.float16 or not k_scale.is_contiguous():
        raise ValueError("INT8 scales must be contiguous float16 [num_blocks, block_size, num_kv_heads]")
    return PaPool(nb, bs, hkv, d, PA_INT8)


def _dev(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")


def _i32(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.int32 or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name} must be a contiguous int32 GPU tensor")
    return t


def _row_stride(t: torch.Tensor, row_elems: int, name: str) -> int:
    """Row stride (elements) of a [rows, heads, dim] tensor whose rows may be strided."""
    if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise ValueError(f"{name} must be [rows, heads, head_dim] with contiguous rows")
    return t.stride(0) if t.shape[0] > 1 else row_elems


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check(fn: str, code: int):
    if code != 0:
        raise PaError(fn, code)


def _ptr(t):
    return None if t is None else t.data_ptr()


# ---------------------------------------------------------------- the calls

def pa_store_kv(k, v, slot_mapping, k_pool, v_pool):
    """Scatter k/v [T, Hkv, D] rows into the pools at slot_mapping (int32, -1 = skip)."""
    lib = load()
    _dev(k, v, k_pool, v_pool)
    pool = pool_desc(k_pool)
    if v_pool.shape != k_pool.shape or v_pool.dtype != k_pool.dtype or not v_pool.is_contiguous():
        raise ValueError("v_pool must match k_pool")
    if k.dtype != k_pool.dtype or v.dtype != k_pool.dtype:
        raise TypeError("k/v dtype must match the pools")
    row = pool.num_kv_heads * pool.head_dim
    slot_mapping = _i32(slot_mapping, "slot_mapping")
    n = slot_mapping.numel()
    if k.shape[0] != n or v.shape[0] != n:
        raise ValueError("k, v and slot_mapping must have the same number of tokens")
    _check("pa_store_kv", lib.pa_store_kv(
        _ptr(k), _row_stride(k, row, "k"), _ptr(v), _row_stride(v, row, "v"), _ptr(slot_mapping), n,
        _ptr(k_pool), _ptr(v_pool), ctypes.byref(pool), _stream()))


def pa_prefill_workspace_bytes(num_seqs, total_q, num_q_heads, max_seqlen_q, max_seqlen_k, k_pool):
    pool = pool_desc(k_pool)
    return int(load().pa_prefill_workspace_bytes(num_seqs, total_q, num_q_heads, max_seqlen_q,
                                                 max_seqlen_k, ctypes.byref(pool)))


def pa_decode_workspace_bytes(num_seqs, num_q_heads, max_context_len, k_pool):
    pool = pool_desc(k_pool)
    return int(load().pa_decode_workspace_bytes(num_seqs, num_q_heads, max_context_len, ctypes.byref(pool)))


def _workspace(nbytes, workspace, device):
    if nbytes == 0:
        return workspace, (workspace.numel() * workspace.element_size() if workspace is not None else 0)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def pa_prefill_varlen(q, k_pool, v_pool, cu_seqlens_q, cu_seqlens_k, q_offsets, block_table,
                      max_seqlen_q, max_seqlen_k, softmax_scale, out=None, workspace=None):
    """Causal varlen prefill over the paged cache; returns out [total_q, Hq, D]."""
    lib = load()
    _dev(q, k_pool, v_pool)
    pool = pool_desc(k_pool)
    total_q, hq, d = q.shape
    if d != pool.head_dim or q.dtype != k_pool.dtype:
        raise ValueError("q must match the pools' head_dim and dtype")
    cu_seqlens_q, cu_seqlens_k = _i32(cu_seqlens_q, "cu_seqlens_q"), _i32(cu_seqlens_k, "cu_seqlens_k")
    q_offsets, block_table = _i32(q_offsets, "q_offsets"), _i32(block_table, "block_table")
    num_seqs = cu_seqlens_q.numel() - 1
    if out is None:
        out = torch.empty((total_q, hq, d), dtype=q.dtype, device=q.device)
    elif not out.is_contiguous() or out.shape != (total_q, hq, d) or out.dtype != q.dtype:
        raise ValueError("out must be contiguous [total_q, Hq, D] of q's dtype")
    nbytes = pa_prefill_workspace_bytes(num_seqs, total_q, hq, max_seqlen_q, max_seqlen_k, k_pool)
    workspace, wbytes = _workspace(nbytes, workspace, q.device)
    _check("pa_prefill_varlen", lib.pa_prefill_varlen(
        _ptr(q), _row_stride(q, hq * d, "q"), hq, _ptr(k_pool), _ptr(v_pool), ctypes.byref(pool),
        _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(q_offsets), _ptr(block_table),
        block_table.shape[1], num_seqs, total_q, int(max_seqlen_q), int(max_seqlen_k),
        float(softmax_scale), _ptr(out), _ptr(workspace), wbytes, _stream()))
    return out


def pa_store_kv_int8(k, v, slot_mapping, k_pool, v_pool, k_scale, v_scale):
    """Quantize k/v [T, Hkv, D] (bf16, fp16 or fp32) per (token, KV head) into the
    INT8 code pools and fp16 scale pools at slot_mapping (int32, -1 = skip)."""
    lib = load()
    _dev(k, v, k_pool, v_pool, k_scale, v_scale)
    pool = pool_desc_int8(k_pool, k_scale)
    if v_pool.shape != k_pool.shape or v_pool.dtype != torch.int8 or not v_pool.is_contiguous():
        raise ValueError("v_pool must match k_pool")
    if v_scale.shape != k_scale.shape or v_scale.dtype != torch.float16 or not v_scale.is_contiguous():
        raise ValueError("v_scale must match k_scale")
    if k.dtype != v.dtype:
        raise TypeError("k and v must have the same dtype")
    row = pool.num_kv_heads * pool.head_dim
    slot_mapping = _i32(slot_mapping, "slot_mapping")
    n = slot_mapping.numel()
    if k.shape[0] != n or v.shape[0] != n:
        raise ValueError("k, v and slot_mapping must have the same number of tokens")
    _check("pa_store_kv_int8", lib.pa_store_kv_int8(
        _ptr(k), _row_stride(k, row, "k"), _ptr(v), _row_stride(v, row, "v"), _dtype_code(k),
        _ptr(slot_mapping), n, _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
        ctypes.byref(pool), _stream()))


def pa_copy_blocks(src_blocks, dst_blocks, num_valid, k_pool, v_pool, k_scale=None, v_scale=None):
    """Copy slots 0..num_valid[i]-1 of block src_blocks[i] to block dst_blocks[i]
    (int32 device tensors) in the K/V pools (and the INT8 scale pools)."""
    lib = load()
    _dev(k_pool, v_pool)
    pool = pool_desc_int8(k_pool, k_scale) if k_pool.dtype == torch.int8 else pool_desc(k_pool)
    if v_pool.shape != k_pool.shape or v_pool.dtype != k_pool.dtype or not v_pool.is_contiguous():
        raise ValueError("v_pool must match k_pool")
    src, dst, nv = _i32(src_blocks, "src_blocks"), _i32(dst_blocks, "dst_blocks"), _i32(num_valid, "num_valid")
    n = src.numel()
    if dst.numel() != n or nv.numel() != n:
        raise ValueError("src_blocks, dst_blocks and num_valid must have one entry per pair")
    _check("pa_copy_blocks", lib.pa_copy_blocks(_ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
                                                ctypes.byref(pool), _ptr(src), _ptr(dst), _ptr(nv), n, _stream()))


def pa_decode(q, k_pool, v_pool, context_lens, block_table, max_context_len, softmax_scale,
              out=None, workspace=None, row_order=None):
    """One query per sequence over its paged context; returns out [B, Hq, D].
    row_order: optional int32 device permutation of the rows (pa_decode_order)."""
    lib = load()
    _dev(q, k_pool, v_pool)
    pool = pool_desc(k_pool)
    b, hq, d = q.shape
    if d != pool.head_dim or q.dtype != k_pool.dtype:
        raise ValueError("q must match the pools' head_dim and dtype")
    context_lens, block_table = _i32(context_lens, "context_lens"), _i32(block_table, "block_table")
    if row_order is not None:
        row_order = _i32(row_order, "row_order")
        if row_order.numel() != b:
            raise ValueError("row_order must hold one entry per sequence")
    if out is None:
        out = torch.empty((b, hq, d), dtype=q.dtype, device=q.device)
    elif not out.is_contiguous() or out.shape != (b, hq, d) or out.dtype != q.dtype:
        raise ValueError("out must be contiguous [B, Hq, D] of q's dtype")
    nbytes = pa_decode_workspace_bytes(b, hq, max_context_len, k_pool)
    workspace, wbytes = _workspace(nbytes, workspace, q.device)
    _check("pa_decode", lib.pa_decode(
        _ptr(q), _row_stride(q, hq * d, "q"), hq, _ptr(k_pool), _ptr(v_pool), ctypes.byref(pool),
        _ptr(context_lens), _ptr(block_table), block_table.shape[1], b, int(max_context_len),
        float(softmax_scale), _ptr(row_order), _ptr(out), _ptr(workspace), wbytes, _stream()))
    return out


def pa_decode_static(q, k_pool, v_pool, context_lens, block_table, max_context_len, softmax_scale,
                     out=None, row_order=None):
    """pa_decode with its split partials in the library's per-GPU scratch
    array instead of a workspace (no allocation by the call)."""
    lib = load()
    _dev(q, k_pool, v_pool)
    pool = pool_desc(k_pool)
    b, hq, d = q.shape
    if d != pool.head_dim or q.dtype != k_pool.dtype:
        raise ValueError("q must match the pools' head_dim and dtype")
    context_lens, block_table = _i32(context_lens, "context_lens"), _i32(block_table, "block_table")
    if row_order is not None:
        row_order = _i32(row_order, "row_order")
        if row_order.numel() != b:
            raise ValueError("row_order must hold one entry per sequence")
    if out is None:
        out = torch.empty((b, hq, d), dtype=q.dtype, device=q.device)
    elif not out.is_contiguous() or out.shape != (b, hq, d) or out.dtype != q.dtype:
        raise ValueError("out must be contiguous [B, Hq, D] of q's dtype")
    _check("pa_decode_static", lib.pa_decode_static(
        _ptr(q), _row_stride(q, hq * d, "q"), hq, _ptr(k_pool), _ptr(v_pool), ctypes.byref(pool),
        _ptr(context_lens), _ptr(block_table), block_table.shape[1], b, int(max_context_len),
        float(softmax_scale), _ptr(row_order), _ptr(out), _stream()))
    return out


def pa_decode_int8_workspace_bytes(num_seqs, num_q_heads, max_context_len, k_pool, k_scale) -> int:
    pool = pool_desc_int8(k_pool, k_scale)
    return int(load().pa_decode_int8_workspace_bytes(num_seqs, num_q_heads, int(max_context_len),
                                                     ctypes.byref(pool)))


def pa_decode_int8(q, k_pool, v_pool, k_scale, v_scale, context_lens, block_table, max_context_len,
                   softmax_scale, out=None, workspace=None, row_order=None):
    """pa_decode over INT8 pools (int8 codes, fp16 scales); q/out bf16, fp16 or fp32."""
    lib = load()
    _dev(q, k_pool, v_pool, k_scale, v_scale)
    pool = pool_desc_int8(k_pool, k_scale)
    if v_pool.shape != k_pool.shape or v_pool.dtype != torch.int8 or not v_pool.is_contiguous():
        raise ValueError("v_pool must match k_pool")
    if v_scale.shape != k_scale.shape or v_scale.dtype != torch.float16 or not v_scale.is_contiguous():
        raise ValueError("v_scale must match k_scale")
    b, hq, d = q.shape
    if d != pool.head_dim:
        raise ValueError("q must match the pools' head_dim")
    context_lens, block_table = _i32(context_lens, "context_lens"), _i32(block_table, "block_table")
    if row_order is not None:
        row_order = _i32(row_order, "row_order")
        if row_order.numel() != b:
            raise ValueError("row_order must hold one entry per sequence")
    if out is None:
        out = torch.empty((b, hq, d), dtype=q.dtype, device=q.device)
    elif not out.is_contiguous() or out.shape != (b, hq, d) or out.dtype != q.dtype:
        raise ValueError("out must be contiguous [B, Hq, D] of q's dtype")
    nbytes = pa_decode_int8_workspace_bytes(b, hq, max_context_len, k_pool, k_scale)
    workspace, wbytes = _workspace(nbytes, workspace, q.device)
    _check("pa_decode_int8", lib.pa_decode_int8(
        _ptr(q), _row_stride(q, hq * d, "q"), hq, _dtype_code(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale),
        _ptr(v_scale), ctypes.byref(pool), _ptr(context_lens), _ptr(block_table), block_table.shape[1], b,
        int(max_context_len), float(softmax_scale), _ptr(row_order), _ptr(out), _ptr(workspace), wbytes,
        _stream()))
    return out


def pa_prefill_varlen_int8(q, k_pool, v_pool, k_scale, v_scale, cu_seqlens_q, cu_seqlens_k, q_offsets,
                           block_table, max_seqlen_q, max_seqlen_k, softmax_scale, out=None, workspace=None):
    """pa_prefill_varlen over INT8 pools (int8 codes, fp16 scales); q/out bf16, fp16 or fp32."""
    lib = load()
    _dev(q, k_pool, v_pool, k_scale, v_scale)
    pool = pool_desc_int8(k_pool, k_scale)
    if v_pool.shape != k_pool.shape or v_pool.dtype != torch.int8 or not v_pool.is_contiguous():
        raise ValueError("v_pool must match k_pool")
    if v_scale.shape != k_scale.shape or v_scale.dtype != torch.float16 or not v_scale.is_contiguous():
        raise ValueError("v_scale must match k_scale")
    total_q, hq, d = q.shape
    if d != pool.head_dim:
        raise ValueError("q must match the pools' head_dim")
    cu_q, cu_k = _i32(cu_seqlens_q, "cu_seqlens_q"), _i32(cu_seqlens_k, "cu_seqlens_k")
    q_offsets, block_table = _i32(q_offsets, "q_offsets"), _i32(block_table, "block_table")
    num_seqs = cu_q.numel() - 1
    if out is None:
        out = torch.empty((total_q, hq, d), dtype=q.dtype, device=q.device)
    elif not out.is_contiguous() or out.shape != (total_q, hq, d) or out.dtype != q.dtype:
        raise ValueError("out must be contiguous [total_q, Hq, D] of q's dtype")
    nbytes = int(lib.pa_prefill_int8_workspace_bytes(num_seqs, total_q, hq, int(max_seqlen_k), ctypes.byref(pool)))
    workspace, wbytes = _workspace(nbytes, workspace, q.device)
    _check("pa_prefill_varlen_int8", lib.pa_prefill_varlen_int8(
        _ptr(q), _row_stride(q, hq * d, "q"), hq, _dtype_code(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale),
        _ptr(v_scale), ctypes.byref(pool), _ptr(cu_q), _ptr(cu_k), _ptr(q_offsets), _ptr(block_table),
        block_table.shape[1], num_seqs, total_q, int(max_seqlen_q), int(max_seqlen_k), float(softmax_scale),
        _ptr(out), _ptr(workspace), wbytes, _stream()))
    return out


def pa_decode_order(context_lens, row_order=None):
    """Rows by decreasing context length (ties by index), as an int32 device
    tensor for pa_decode's row_order; one call serves every layer of a step."""
    lib = load()
    context_lens = _i32(context_lens, "context_lens")
    n = context_lens.numel()
    if row_order is None:
        row_order = torch.empty(n, dtype=torch.int32, device=context_lens.device)
    elif row_order.dtype != torch.int32 or not row_order.is_contiguous() or row_order.numel() != n:
        raise ValueError("row_order must be a contiguous int32 tensor of num_seqs entries")
    _check("pa_decode_order", lib.pa_decode_order(_ptr(context_lens), n, _ptr(row_order), _stream()))
    return row_order


def pa_gather_kv(k_pool, v_pool, cu_seqlens_k, block_table, total_k):
    """Test helper: packed [total_k, Hkv, D] copies of every sequence's K and V."""
    lib = load()
    _dev(k_pool, v_pool)
    pool = pool_desc(k_pool)
    cu_seqlens_k, block_table = _i32(cu_seqlens_k, "cu_seqlens_k"), _i32(block_table, "block_table")
    shape = (total_k, pool.num_kv_heads, pool.head_dim)
    k_out = torch.empty(shape, dtype=k_pool.dtype, device=k_pool.device)
    v_out = torch.empty(shape, dtype=k_pool.dtype, device=k_pool.device)
    _check("pa_gather_kv", lib.pa_gather_kv(
        _ptr(k_pool), _ptr(v_pool), ctypes.byref(pool), _ptr(cu_seqlens_k), _ptr(block_table),
        block_table.shape[1], cu_seqlens_k.numel() - 1, total_k, _ptr(k_out), _ptr(v_out), _stream()))
    return k_out, v_out


# ---------------------------------------------------------------- host validators

def _host_i32(a):
    import numpy as np
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def validate_prefill_metadata(cu_seqlens_q, cu_seqlens_k, q_offsets, block_table, max_seqlen_q,
                              max_seqlen_k, pool: PaPool, slot_mapping=None):
    """Check HOST copies of prefill metadata; raises PaError with the reason."""
    lib = load()
    cq, ck, qo, bt, sm = (_host_i32(x) for x in (cu_seqlens_q, cu_seqlens_k, q_offsets, block_table,
                                                  slot_mapping))
    why = ctypes.create_string_buffer(256)
    vp = ctypes.c_void_p
    code = lib.pa_validate_prefill_metadata(
        cq.ctypes.data_as(vp), ck.ctypes.data_as(vp), qo.ctypes.data_as(vp), bt.ctypes.data_as(vp),
        bt.shape[1], len(cq) - 1, max_seqlen_q, max_seqlen_k,
        None if sm is None else sm.ctypes.data_as(vp), 0 if sm is None else len(sm),
        ctypes.byref(pool), why, 256)
    if code != 0:
        raise PaError("pa_validate_prefill_metadata", code, why.value.decode())


def validate_decode_metadata(context_lens, block_table, max_context_len, pool: PaPool, slot_mapping=None,
                             row_order=None):
    lib = load()
    cl, bt, sm, ro = (_host_i32(x) for x in (context_lens, block_table, slot_mapping, row_order))
    why = ctypes.create_string_buffer(256)
    vp = ctypes.c_void_p
    code = lib.pa_validate_decode_metadata(
        cl.ctypes.data_as(vp), bt.ctypes.data_as(vp), bt.shape[1], len(cl), max_context_len,
        None if sm is None else sm.ctypes.data_as(vp), None if ro is None else ro.ctypes.data_as(vp),
        ctypes.byref(pool), why, 256)
    if code != 0:
        raise PaError("pa_validate_decode_metadata", code, why.value.decode())
