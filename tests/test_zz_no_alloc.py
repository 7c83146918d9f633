"""pa_decode_static -- pa_decode with its split partials in the library's
per-GPU scratch array instead of a caller workspace -- called through the C
ABI: bit-identical to pa_decode on two calls in a row (the second smaller,
so it reads what the first left in the array only where it wrote it again),
both within tolerance of the oracle; requests past the array are refused
before any device call."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_mapping_amd as pa
import workloads as W
from helpers import max_abs_err, say, to_dev, to_host_bits, tol

LIMIT = 16 << 20  # bytes of the scratch array


def test_too_large_a_request_is_refused_before_any_device_call():
    """Partials beyond the array: PA_ERR_WORKSPACE, returned by the host
    checks (no GPU needed; dummy device pointers are never touched)."""
    lib = pa.load()
    pool = pa.PaPool(1 << 24, 16, 8, 128, pa.PA_BF16)
    dummy = ctypes.c_void_p(4096)
    rows, ctx = 2048, 1 << 20
    need = lib.pa_decode_workspace_bytes(rows, 16, ctx, ctypes.byref(pool))
    assert need > LIMIT
    code = lib.pa_decode_static(dummy, 16 * 128, 16, dummy, dummy, ctypes.byref(pool), dummy, dummy, ctx // 16,
                                rows, ctx, 0.08, None, dummy, None)
    assert code == 5  # PA_ERR_WORKSPACE


@pytest.mark.gpu
def test_static_decode_matches_pa_decode_twice():
    say("[no-alloc] pa_decode_static vs pa_decode, two calls")
    runs = [W.make_decode("static_a", 9801, [20000, 7, 9000, 1, 0, 12345], 16, 8, 128, 16, "bf16"),
            W.make_decode("static_b", 9802, [5000, 300], 16, 8, 128, 16, "bf16")]
    for case in runs:
        kp, vp = case.empty_pools()
        oracle.store_kv(case.k_hist, case.v_hist, case.slot_hist, kp, vp)
        oracle.store_kv(case.k_new, case.v_new, case.slot_new, kp, vp)
        kd, vd = to_dev(kp), to_dev(vp)
        lib = pa.load()
        pool = pa.pool_desc(kd)
        need = lib.pa_decode_workspace_bytes(case.num_seqs, case.num_q_heads, case.max_context_len,
                                             ctypes.byref(pool))
        assert 0 < need <= LIMIT, need  # the split path, within the array
        q, ctx, bt = to_dev(case.q), to_dev(case.context_lens), to_dev(case.block_table)
        ref_out = pa.pa_decode(q, kd, vd, ctx, bt, case.max_context_len, case.scale)
        out = torch.full_like(ref_out, float("nan"))
        code = lib.pa_decode_static(q.data_ptr(), case.num_q_heads * case.head_dim, case.num_q_heads,
                                    kd.data_ptr(), vd.data_ptr(), ctypes.byref(pool), ctx.data_ptr(), bt.data_ptr(),
                                    bt.shape[1], case.num_seqs, case.max_context_len, case.scale, None,
                                    out.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert code == 0, code
        torch.cuda.synchronize()
        assert to_host_bits(out).tobytes() == to_host_bits(ref_out).tobytes()
        ref = oracle.decode(case.q, kp, vp, case.context_lens, case.block_table, case.scale)
        err = max_abs_err(out, ref)
        say(f"  {case.name}: {case.num_seqs} rows, partials {need} B, max-abs {err:.3e}")
        assert err <= tol("bf16")
