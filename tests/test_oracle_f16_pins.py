"""Pins for the oracle's IEEE binary16 (fp16) element type.

fp16 is the element type of the fork's fused-dequantization microbenchmark
("LLM inference interview notes (nano-vllm fork)", Q3, the INT8-versus-FP16
latency table).  The oracle widens fp16 bit patterns itself, in C; these tests
check that widening against numpy's own float16 -> float64 conversion over
every finite pattern, through each operand the attention reads (Q, K, V).
The textbook-SDPA, store/gather and decode pins of the other oracle test file
run at fp16 as well.

Runs on the CPU only.
"""
import numpy as np
import pytest

import oracle


def _finite_f16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16)
    return x[np.isfinite(x)]


def test_every_finite_pattern_is_widened_exactly_in_v():
    """One visible key: the output is V exactly, so it must equal numpy's
    float16 -> float64 value for all 63488 finite patterns."""
    x = _finite_f16()
    n = x.size
    assert n == 63488
    vp = x.reshape(n, 1, 1, 1).copy()
    kp = np.zeros_like(vp)
    q = np.zeros((n, 1, 1), np.float16)
    table = np.arange(n, dtype=np.int32)[:, None]
    out = oracle.decode(q, kp, vp, np.ones(n, np.int32), table, 1.0)
    np.testing.assert_array_equal(out[:, 0, 0], x.astype(np.float64))


@pytest.mark.parametrize("role", ["k", "q"])
def test_every_finite_pattern_is_widened_exactly_in_scores(role):
    """Two keys with V = (0, 1): the output is the logistic function of the
    score difference s * q * (k1 - k0) with k0 = 0.  Put the pattern under test
    in k1 (q = 1) or in q (k1 = 1); a mis-decoded pattern -- a wrong sign, a
    subnormal off by a power of two -- moves the result by far more than the
    fp64 rounding of the softmax."""
    x = _finite_f16()
    n = x.size
    scale = 1.0e-4                      # keeps s * 65504 within a few units
    kp = np.zeros((n, 2, 1, 1), np.float16)
    vp = np.zeros_like(kp)
    vp[:, 1, 0, 0] = 1.0
    if role == "k":
        kp[:, 1, 0, 0] = x
        q = np.ones((n, 1, 1), np.float16)
    else:
        kp[:, 1, 0, 0] = 1.0
        q = x.reshape(n, 1, 1).copy()
    table = np.arange(n, dtype=np.int32)[:, None]
    out = oracle.decode(q, kp, vp, np.full(n, 2, np.int32), table, scale)[:, 0, 0]
    y = scale * x.astype(np.float64)
    ref = 1.0 / (1.0 + np.exp(-y))
    assert np.abs(out - ref).max() < 1e-15
    # the smallest subnormal moves the output off 1/2 by about y/4
    tiny = np.abs(x.astype(np.float64)) == 2.0 ** -24
    assert (np.abs(out[tiny] - 0.5) > 1e-12).all()


def test_nan_patterns_widen_to_nan():
    """Exponent 31 with a nonzero fraction is NaN; a NaN value under a
    visible key poisons the output (the pools' fill value relies on it)."""
    nan = np.array([0x7E00, 0x7C01, 0xFE00], np.uint16).view(np.float16)
    vp = nan.reshape(3, 1, 1, 1).copy()
    kp = np.zeros_like(vp)
    out = oracle.decode(np.zeros((3, 1, 1), np.float16), kp, vp, np.ones(3, np.int32),
                        np.arange(3, dtype=np.int32)[:, None], 1.0)
    assert np.isnan(out).all()
