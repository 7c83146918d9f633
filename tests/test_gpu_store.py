"""pa_store_kv and pa_gather_kv on the GPU: bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_mapping_amd as pa
import workloads as W
from helpers import host_pools_with_prefix, say, to_dev, to_host_bits

pytestmark = pytest.mark.gpu

CASES = {
    "c1_prefill": lambda: W.c1_tiny()[0],
    "c2_8x32": lambda: W.c2_varlen(32),
    "c2_8x256": lambda: W.c2_varlen(256),
    "c3_prefix": W.c3_prefix,
    "c5a_4096": W.c5a_long,
    "c5a_mixed": W.c5a_mixed,
}


@pytest.mark.parametrize("name", list(CASES))
def test_store_bit_exact_on_poisoned_pools(name):
    case = CASES[name]()
    say(f"[store] {name} T={case.total_q}")
    kp, vp = host_pools_with_prefix(case)
    kd, vd = to_dev(kp), to_dev(vp)
    pa.pa_store_kv(to_dev(case.k_new), to_dev(case.v_new), to_dev(case.slot_new), kd, vd)
    oracle.store_kv(case.k_new, case.v_new, case.slot_new, kp, vp)
    torch.cuda.synchronize()
    assert to_host_bits(kd).tobytes() == kp.tobytes()
    assert to_host_bits(vd).tobytes() == vp.tobytes()


@pytest.mark.parametrize("name", ["c2_8x32", "c3_prefix", "c5a_mixed"])
def test_gather_bit_exact(name):
    case = CASES[name]()
    say(f"[gather] {name}")
    kp, vp = host_pools_with_prefix(case)
    oracle.store_kv(case.k_new, case.v_new, case.slot_new, kp, vp)
    ko, vo = pa.pa_gather_kv(to_dev(kp), to_dev(vp), to_dev(case.cu_seqlens_k),
                             to_dev(case.block_table), int(case.cu_seqlens_k[-1]))
    kr, vr = oracle.gather_kv(kp, vp, case.cu_seqlens_k, case.block_table)
    assert to_host_bits(ko).tobytes() == kr.tobytes()
    assert to_host_bits(vo).tobytes() == vr.tobytes()


def test_store_skips_padding_slots_and_takes_strided_rows():
    """Slots of -1 (captured-batch padding) are skipped; k/v may be strided
    views of a fused [T, (Hq + 2 Hkv) * D] projection output."""
    rng = np.random.default_rng(5)
    case = W.make_prefill("strided", 17, [7, 33], [0, 0], 4, 2, 64, 16, "bf16")
    slots = case.slot_new.copy()
    slots[[0, 9, 20]] = -1
    kp, vp = case.empty_pools()
    T, hkv, d = case.k_new.shape
    fused = W.normal(rng, (T, (4 + 2 * hkv) * d), "bf16")
    fused[:, 4 * d:(4 + hkv) * d] = case.k_new.reshape(T, -1)
    fused[:, (4 + hkv) * d:] = case.v_new.reshape(T, -1)
    fd = to_dev(fused)
    k_view = fd[:, 4 * d:(4 + hkv) * d].view(T, hkv, d)
    v_view = fd[:, (4 + hkv) * d:].view(T, hkv, d)
    kd, vd = to_dev(kp), to_dev(vp)
    say("[store] strided + padding")
    pa.pa_store_kv(k_view, v_view, to_dev(slots), kd, vd)
    oracle.store_kv(case.k_new, case.v_new, slots, kp, vp)
    torch.cuda.synchronize()
    assert to_host_bits(kd).tobytes() == kp.tobytes()
    assert to_host_bits(vd).tobytes() == vp.tobytes()


@pytest.mark.parametrize("dtype,d,bs", [("f32", 32, 1), ("bf16", 128, 256), ("f32", 256, 4),
                                        ("bf16", 32, 2)])
def test_store_shapes(dtype, d, bs):
    case = W.make_prefill("shape", 23 + d, [1, 45, 3], [0, 0, 0], 2, 2, d, bs, dtype)
    say(f"[store] {dtype} d={d} bs={bs}")
    kp, vp = case.empty_pools()
    kd, vd = to_dev(kp), to_dev(vp)
    pa.pa_store_kv(to_dev(case.k_new), to_dev(case.v_new), to_dev(case.slot_new), kd, vd)
    oracle.store_kv(case.k_new, case.v_new, case.slot_new, kp, vp)
    torch.cuda.synchronize()
    assert to_host_bits(kd).tobytes() == kp.tobytes()
    assert to_host_bits(vd).tobytes() == vp.tobytes()
