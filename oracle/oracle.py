"""ctypes wrapper over pa_oracle.c (fp64 CPU reference).

TEST INFRASTRUCTURE ONLY.  Arrays are numpy; bf16 data travels as uint16 bit
patterns, fp16 as float16, fp32 as float32.  Every function checks the C return code and
raises on failure.  The C source says which page and section each step
follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F32 = 0
BF16 = 1
F16 = 3

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_ERRORS = {1: "null argument", 2: "bad shape", 3: "bad element type", 4: "index out of range"}


def lib_path() -> str:
    return _LIB


def build(force: bool = False) -> str:
    """Compile pa_oracle.c with gcc (fp64, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
             "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        p, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = ctypes.c_int
        lib.oracle_store_kv.argtypes = [p, i64, p, i64, p, i32, p, p, i64, i32, i32, i32, i32]
        lib.oracle_gather_kv.argtypes = [p, p, i64, i32, i32, i32, i32, p, p, i32, i32, p, p]
        lib.oracle_prefill.argtypes = [p, i64, i32, i32, p, p, i64, i32, i32, i32,
                                       p, p, p, p, i32, i32, f64, p, i32, p, p]
        lib.oracle_decode.argtypes = [p, i64, i32, i32, p, p, i64, i32, i32, i32,
                                      p, p, i32, i32, f64, p, i32, p, p]
        for fn in (lib.oracle_store_kv, lib.oracle_gather_kv, lib.oracle_prefill, lib.oracle_decode):
            fn.restype = ctypes.c_int
        _lib = lib
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"oracle {what}: {_ERRORS.get(rc, rc)}")


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float16:
        return F16
    raise TypeError(f"oracle takes float32, float16 or uint16 (bf16 bits), got {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> int:
    """Host threads of the attention loops from now on (timing only); returns the number in effect."""
    return int(_load().oracle_set_num_threads(int(n)))


def store_kv(k, v, slot_mapping, k_pool, v_pool) -> None:
    """In-place scatter of k/v [T, Hkv, D] rows into pools [NB, bs, Hkv, D]."""
    lib = _load()
    assert k_pool.flags.c_contiguous and v_pool.flags.c_contiguous
    nb, bs, hkv, d = k_pool.shape
    k = np.ascontiguousarray(k).reshape(-1, hkv * d)
    v = np.ascontiguousarray(v).reshape(-1, hkv * d)
    slots = _i32(slot_mapping)
    assert k.dtype == v.dtype == k_pool.dtype == v_pool.dtype
    _check(lib.oracle_store_kv(_ptr(k), hkv * d, _ptr(v), hkv * d, _ptr(slots), len(slots),
                               _ptr(k_pool), _ptr(v_pool), nb, bs, hkv, d, _dtype_code(k_pool)),
           "store_kv")


def gather_kv(k_pool, v_pool, cu_seqlens_k, block_table):
    """Packed [total_k, Hkv, D] copies of every sequence's keys/values."""
    lib = _load()
    nb, bs, hkv, d = k_pool.shape
    cu = _i32(cu_seqlens_k)
    bt = _i32(block_table)
    total = int(cu[-1])
    k_out = np.zeros((total, hkv, d), dtype=k_pool.dtype)
    v_out = np.zeros((total, hkv, d), dtype=k_pool.dtype)
    _check(lib.oracle_gather_kv(_ptr(k_pool), _ptr(v_pool), nb, bs, hkv, d, _dtype_code(k_pool),
                                _ptr(cu), _ptr(bt), bt.shape[1], len(cu) - 1,
                                _ptr(k_out), _ptr(v_out)), "gather_kv")
    return k_out, v_out


def prefill(q, k_pool, v_pool, cu_seqlens_q, cu_seqlens_k, q_offsets, block_table, scale,
            rows=None, return_pairs=False):
    """fp64 [len(rows) or total_q, Hq, D] causal attention over the paged cache."""
    lib = _load()
    q = np.ascontiguousarray(q)
    total_q, hq, d = q.shape
    nb, bs, hkv, d2 = k_pool.shape
    assert d == d2 and q.dtype == k_pool.dtype == v_pool.dtype
    cq, ck, qo, bt = _i32(cu_seqlens_q), _i32(cu_seqlens_k), _i32(q_offsets), _i32(block_table)
    r = None if rows is None else _i32(rows)
    n = total_q if r is None else len(r)
    out = np.zeros((n, hq, d), dtype=np.float64)
    pairs = ctypes.c_int64(0)
    _check(lib.oracle_prefill(_ptr(q), hq * d, hq, _dtype_code(q), _ptr(k_pool), _ptr(v_pool),
                              nb, bs, hkv, d, _ptr(cq), _ptr(ck), _ptr(qo), _ptr(bt), bt.shape[1],
                              len(cq) - 1, float(scale), _ptr(r), n, _ptr(out), ctypes.byref(pairs)),
           "prefill")
    return (out, int(pairs.value)) if return_pairs else out


def decode(q, k_pool, v_pool, context_lens, block_table, scale, seqs=None, return_pairs=False):
    """fp64 [len(seqs) or B, Hq, D]: one query per sequence over its paged context."""
    lib = _load()
    q = np.ascontiguousarray(q)
    b, hq, d = q.shape
    nb, bs, hkv, d2 = k_pool.shape
    assert d == d2 and q.dtype == k_pool.dtype == v_pool.dtype
    cl, bt = _i32(context_lens), _i32(block_table)
    sl = None if seqs is None else _i32(seqs)
    n = b if sl is None else len(sl)
    out = np.zeros((n, hq, d), dtype=np.float64)
    pairs = ctypes.c_int64(0)
    _check(lib.oracle_decode(_ptr(q), hq * d, hq, _dtype_code(q), _ptr(k_pool), _ptr(v_pool),
                             nb, bs, hkv, d, _ptr(cl), _ptr(bt), bt.shape[1], b, float(scale),
                             _ptr(sl), n, _ptr(out), ctypes.byref(pairs)), "decode")
    return (out, int(pairs.value)) if return_pairs else out
