"""Pins of the oracle's per-group weight scales ("KV-cache kernels", 02 Scales
and dequantization and 03 Where scales come from: one weight scale per group
of 64-128 channels), with the groups along the reduction dimension k:

  acc[i, j] = sum_g scale_b[g, j] * sum_{t in group g} a[i, t] * B(t, j).

Each check compares the oracle with something other than its own formula:
Python integer and Fraction brute force, the per-channel GEMM it reduces to
when there is one group, one-hot group scales, linearity, a closed form.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import oracle


def _brute(a, b_kn, sb, group):
    m, k = a.shape
    n = b_kn.shape[1]
    out = np.empty((m, n), dtype=object)
    for i in range(m):
        for j in range(n):
            total = Fraction(0)
            for g in range(sb.shape[0]):
                part = sum(int(a[i, t]) * int(b_kn[t, j]) for t in range(g * group, min((g + 1) * group, k)))
                total += part * Fraction(float(sb[g, j]))
            out[i, j] = total
    return out


def _operands(rng, m, n, k, group):
    a = rng.integers(-127, 128, (m, k), dtype=np.int8)
    b = rng.integers(-127, 128, (k, n), dtype=np.int8)
    sb = rng.uniform(1e-4, 1e-1, ((k + group - 1) // group, n)).astype(np.float32)
    return a, b, sb


@pytest.mark.parametrize("m,n,k,group", [(1, 1, 1, 1), (3, 4, 10, 4), (2, 5, 17, 8), (4, 3, 64, 64),
                                         (2, 3, 130, 64)])
def test_grouped_against_fraction_brute_force(m, n, k, group):
    rng = np.random.default_rng(m * 1000 + k)
    a, b, sb = _operands(rng, m, n, k, group)
    want = _brute(a, b, sb, group)
    for layout, bb in ((oracle.B_KN, b), (oracle.B_NK, np.ascontiguousarray(b.T))):
        got = oracle.gemm_i8_grouped(a, bb, sb, group, layout)
        for i in range(m):
            for j in range(n):
                # binary64 sum of exact products: within n_groups ulps of the exact value
                assert abs(Fraction(got[i, j]) - want[i, j]) <= sb.shape[0] * 2 ** -52 * abs(want[i, j]) + 1e-300


def test_one_group_is_the_per_channel_gemm():
    rng = np.random.default_rng(7)
    m, n, k = 9, 11, 192
    a, b, _ = _operands(rng, m, n, k, k)
    s = rng.uniform(1e-3, 1e-2, n).astype(np.float32)
    got = oracle.gemm_i8_grouped(a, b, s[None, :], k)
    c = oracle.gemm_i32(a, b)
    assert np.array_equal(got, c.astype(np.float64) * s.astype(np.float64)[None, :])


def test_one_hot_group_scales_select_that_group():
    rng = np.random.default_rng(8)
    m, n, k, group = 5, 6, 256, 64
    a, b, _ = _operands(rng, m, n, k, group)
    for g in range(k // group):
        sb = np.zeros((k // group, n), np.float32)
        sb[g] = 1.0
        got = oracle.gemm_i8_grouped(a, b, sb, group)
        part = oracle.gemm_i32(np.ascontiguousarray(a[:, g * group:(g + 1) * group]),
                               np.ascontiguousarray(b[g * group:(g + 1) * group]))
        assert np.array_equal(got, part.astype(np.float64))


def test_linear_in_the_scales_and_power_of_two_exact():
    rng = np.random.default_rng(9)
    m, n, k, group = 4, 7, 384, 128
    a, b, sb = _operands(rng, m, n, k, group)
    base = oracle.gemm_i8_grouped(a, b, sb, group)
    assert np.array_equal(oracle.gemm_i8_grouped(a, b, sb * np.float32(8.0), group), base * 8.0)
    # the sum of two scale sets gives the sum of the results (up to binary64 rounding)
    sb2 = rng.uniform(1e-4, 1e-1, sb.shape).astype(np.float32)
    both = oracle.gemm_i8_grouped(a, b, (sb.astype(np.float64) + sb2).astype(np.float32), group)
    assert np.allclose(both, base + oracle.gemm_i8_grouped(a, b, sb2, group), rtol=1e-6, atol=0)


def test_closed_form_constant_operands():
    # a = 127, b = -127 everywhere, scale of group g = 2^-g: acc = -127^2 * G * sum_g 2^-g
    m, n, k, group = 2, 3, 512, 64
    a = np.full((m, k), 127, np.int8)
    b = np.full((k, n), -127, np.int8)
    sb = np.array([[2.0 ** -g] * n for g in range(k // group)], np.float32)
    got = oracle.gemm_i8_grouped(a, b, sb, group)
    want = -127 * 127 * group * sum(2.0 ** -g for g in range(k // group))
    assert np.all(got == want)


def test_dequant_grouped_is_the_product():
    acc = np.array([[1.5, -2.25], [0.0, 3.0]])
    sa = np.array([0.5, 2.0], np.float32)
    assert np.array_equal(oracle.dequant_grouped(acc, sa, 4.0), np.array([[3.0, -4.5], [0.0, 24.0]]))


def test_bad_scale_shape_is_refused():
    with pytest.raises(ValueError):
        oracle.gemm_i8_grouped(np.zeros((2, 128), np.int8), np.zeros((128, 4), np.int8),
                               np.zeros((3, 4), np.float32), 64)
