"""Pins of the oracle's static (per-tensor) and asymmetric (zero-point)
quantization.

Static ("kernels: fused silu_and_mul + dynamic per-token FP8 quantization",
Purpose: silu_and_mul_quant takes one pre-calibrated scale): with a row's
own dynamic scale it must give that row's dynamic codes (the already-pinned
quantizer); with power-of-two scales the quotient is exact and numpy's rint
decides; beyond +-127.5 scales it saturates.  FP8 static equals torch's
e4m3fn conversion of the binary32 quotient.

Asymmetric ("Skill: Write an INT8 Quantized Kernel", Inputs: a nonzero zero
point): worked rows, the exact code of zero, the reconstruction bound, and
the GEMM against Python integers and the column-sum identity.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle


def test_static_with_the_dynamic_scale_reproduces_dynamic_codes():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((40, 333)) * np.exp2(rng.integers(-10, 10, (40, 1)))).astype(np.float32)
    q_dyn, s_dyn = oracle.quant_per_token(x)
    for i in range(x.shape[0]):
        assert np.array_equal(oracle.quant_static(x[i], s_dyn[i]), q_dyn[i])


def test_static_power_of_two_scale_and_saturation():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(10000) * 100).astype(np.float32)
    for e in (-3, 0, 2):
        s = np.float32(2.0 ** e)
        want = np.clip(np.rint(x.astype(np.float64) / float(s)), -127, 127).astype(np.int8)
        assert np.array_equal(oracle.quant_static(x, s), want)
    assert np.array_equal(oracle.quant_static(np.array([127.4, 127.5, 128.0, -1e30, 1e30], np.float32), 1.0),
                          np.array([127, 127, 127, -127, 127], np.int8))
    # ties to even at half-integer quotients
    assert np.array_equal(oracle.quant_static(np.array([0.5, 1.5, 2.5, -0.5, -2.5], np.float32), 1.0),
                          np.array([0, 2, 2, 0, -2], np.int8))


def test_static_fp8_is_the_conversion_of_the_quotient():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(50000) * 40).astype(np.float32)
    s = np.float32(0.37)
    ratio = torch.from_numpy((x / s).astype(np.float32)).clamp(-448, 448)
    want = ratio.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.quant_static_fp8(x, s), want)


def test_asym_worked_rows():
    q, s, z = oracle.quant_per_token_asym(np.array([[0.0, 255.0, 100.0, 100.5]], np.float32))
    assert s[0] == np.float32(1.0) and z[0] == -128
    assert np.array_equal(q[0], np.array([-128, 127, -28, -28], np.int8))  # 100.5 ties to 100
    q, s, z = oracle.quant_per_token_asym(np.array([[-4.0, 0.0, 1.0]], np.float32))
    assert s[0] == np.float32(np.float32(5.0) / np.float32(255.0))
    lo_code = int(np.rint(np.float32(-4.0) / s[0])) + int(z[0])
    assert q[0, 0] == max(-128, lo_code) and q[0, 1] == z[0]
    q, s, z = oracle.quant_per_token_asym(np.zeros((1, 8), np.float32))   # all zero: guard
    assert s[0] == np.float32(np.float32(1e-12) / np.float32(255.0)) and np.all(q == z[0])


def test_asym_zero_is_exact_and_reconstruction_bound():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((60, 500)).astype(np.float32) + rng.uniform(-2, 2, (60, 1)).astype(np.float32)
    x[:, 7] = 0.0
    q, s, z = oracle.quant_per_token_asym(x)
    assert np.array_equal(q[:, 7].astype(np.int32), z)
    rec = (q.astype(np.float64) - z[:, None]) * s.astype(np.float64)[:, None]
    assert np.all(np.abs(rec - x) <= 0.5 * s.astype(np.float64)[:, None] * (1 + 1e-5))
    assert q.min() >= -128 and q.max() <= 127


def test_asym_is_the_symmetric_range_shifted_for_nonnegative_rows():
    # a row with min 0: lo = 0, so zp = -128 and code + 128 = rint(x / s)
    x = np.linspace(0.0, 3.0, 97, dtype=np.float32)[None, :]
    q, s, z = oracle.quant_per_token_asym(x)
    assert z[0] == -128
    assert np.array_equal(q[0].astype(np.int32) + 128, np.rint(x[0] / s[0]).astype(np.int32))


def test_asym_gemm_brute_force_and_column_sum_identity():
    rng = np.random.default_rng(5)
    m, n, k = 3, 4, 9
    a = rng.integers(-128, 128, (m, k), dtype=np.int8)
    zp = rng.integers(-128, 128, m).astype(np.int32)
    b = rng.integers(-127, 128, (k, n), dtype=np.int8)
    got = oracle.gemm_asym(a, zp, b)
    for i in range(m):
        for j in range(n):
            assert got[i, j] == sum((int(a[i, t]) - int(zp[i])) * int(b[t, j]) for t in range(k))
    assert np.array_equal(oracle.gemm_asym(a, zp, np.ascontiguousarray(b.T), oracle.B_NK), got)
    rng2 = np.random.default_rng(6)
    a = rng2.integers(-128, 128, (50, 256), dtype=np.int8)
    zp = rng2.integers(-128, 128, 50).astype(np.int32)
    b = rng2.integers(-127, 128, (256, 70), dtype=np.int8)
    ident = oracle.gemm_i32(a, b).astype(np.int64) - zp[:, None].astype(np.int64) * b.astype(np.int64).sum(0)[None, :]
    assert np.array_equal(oracle.gemm_asym(a, zp, b).astype(np.int64), ident)
