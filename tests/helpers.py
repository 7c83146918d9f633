"""Shared plumbing for the GPU tests: numpy <-> torch bit-exact transfers,
host/device pool construction, error measures.  No attention arithmetic."""
import numpy as np
import torch

import oracle
import workloads as W

BF16_TOL = 2e-2   # max-abs, bf16 attention outputs
F32_TOL = 1e-5    # max-abs, fp32 attention outputs
# max-abs, fp16 attention outputs: half an fp16 ulp of outputs below 8 in
# magnitude (2^-9) plus the fp16 rounding of the probabilities on the matrix
# cores (relative 2^-12 each, in numerator and denominator, on |v| < 5).
F16_TOL = 5e-3


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(a) -> np.ndarray:
    if isinstance(a, torch.Tensor):
        a = to_host_bits(a)
    if a.dtype == np.uint16:
        return W.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def tol(dtype: str) -> float:
    return {"bf16": BF16_TOL, "f16": F16_TOL}.get(dtype, F32_TOL)


def max_abs_err(gpu_out, ref: np.ndarray) -> float:
    g = as_f64(gpu_out)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all(), "non-finite values in the GPU output"
    return float(np.abs(g - ref).max()) if g.size else 0.0


def host_pools_with_prefix(case):
    kp, vp = case.empty_pools()
    if len(case.slot_cached):
        oracle.store_kv(case.k_cached, case.v_cached, case.slot_cached, kp, vp)
    return kp, vp


def say(*a):
    print(*a, flush=True)
