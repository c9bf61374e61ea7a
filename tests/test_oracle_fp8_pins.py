"""Pins of the oracle's FP8 path against what the definitions fix.

The FP8 path is "kernels: fused silu_and_mul + dynamic per-token FP8
quantization" (Purpose, Algorithm): scale = max(absmax, 1e-12) / fp8_max,
optionally clamped by scale_ub, codes in float8_e4m3fn (fp8_max = 448), and
the GEMM those codes feed.  None of these checks compares the oracle with its
own formula: the code values come from an exact-rational reading of the
format, the rounding from torch's float8_e4m3fn conversion, the GEMM from
Python fractions.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def _code_value(c: int):
    """The value of an e4m3fn code from the format's definition (exact)."""
    sign = -1 if c & 0x80 else 1
    e = (c >> 3) & 0xF
    m = c & 7
    if e == 0xF and m == 7:
        return None  # NaN
    if e == 0:
        return sign * Fraction(m, 8) * Fraction(1, 2 ** 6)
    return sign * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def _torch_e4m3fn(x: np.ndarray) -> np.ndarray:
    """torch's round-to-nearest-even conversion, of values clamped to the
    finite range first (the saturation the page's conversion applies)."""
    t = torch.from_numpy(np.clip(x, -448.0, 448.0).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_of_every_code():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.fp8_decode(codes)
    for c in range(256):
        want = _code_value(c)
        if want is None:
            assert np.isnan(got[c]), c
        else:
            assert Fraction(got[c]) == want, (c, got[c], want)
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0 and got[0x08] == 2.0 ** -6


def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oracle.fp8_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.fp8_encode(vals), codes)


def test_encode_matches_torch_over_whole_binades():
    # every binary32 value of 23 binades around the format's range (its
    # subnormals, normals and the saturation edge), both signs
    rng = np.random.default_rng(0)
    for e in range(-14, 10):
        mant = np.arange(1 << 23, dtype=np.uint32)
        bits = ((e + 127) << 23) | mant
        x = bits.view(np.float32)
        if e % 3:
            x = rng.choice(x, 1 << 18, replace=False)  # a sample of most binades
        for sgn in (1.0, -1.0):
            xs = (sgn * x).astype(np.float32)
            got = oracle.fp8_encode(xs)
            want = _torch_e4m3fn(xs)
            bad = np.nonzero(got != want)[0]
            assert bad.size == 0, (e, sgn, xs[bad[:3]], got[bad[:3]], want[bad[:3]])


def test_encode_matches_torch_on_random_values():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(1 << 20) * np.exp2(rng.integers(-16, 12, 1 << 20))).astype(np.float32)
    assert np.array_equal(oracle.fp8_encode(x), _torch_e4m3fn(x))


def test_ties_go_to_the_even_code():
    # the exact midpoint between consecutive finite codes rounds to the code
    # with an even mantissa (or exponent step), one binary32 ulp either side
    # to the nearer code
    for c in range(0x00, 0x7E):
        lo, hi = _code_value(c), _code_value(c + 1)
        mid = (lo + hi) / 2
        x = np.float32(float(mid))
        assert Fraction(float(x)) == mid  # the midpoint is a binary32 value
        even = c if c % 2 == 0 else c + 1
        assert oracle.fp8_encode(np.array([x]))[0] == even, (c, float(mid))
        below = np.nextafter(x, np.float32(0))
        above = np.nextafter(x, np.float32(1e9))
        assert oracle.fp8_encode(np.array([below]))[0] == c
        assert oracle.fp8_encode(np.array([above]))[0] == c + 1


def test_saturation_and_signed_zero():
    x = np.array([448.0, 463.99, 464.0, 480.0, 1e30, 3.4e38, -448.0, -1e30, 0.0, -0.0,
                  2.0 ** -10, -(2.0 ** -10), 2.0 ** -11], np.float32)
    want = np.array([0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x00, 0x80,
                     0x00, 0x80, 0x00], np.uint8)
    assert np.array_equal(oracle.fp8_encode(x), want)


def _rows(rng, m, k):
    x = rng.standard_normal((m, k)).astype(np.float32)
    x *= np.exp2(rng.integers(-20, 20, (m, 1))).astype(np.float32)
    return x


def test_quant_worked_row_with_unit_scale():
    # amax = 448 gives scale exactly 1, so the codes are the plain conversion
    x = np.array([[448.0, -1.0, 3.3, 0.01, -2.5, 2.0 ** -10, 100.0]], np.float32)
    q, s = oracle.quant_per_token_fp8(x)
    assert s[0] == np.float32(1.0)
    assert np.array_equal(q[0], _torch_e4m3fn(x[0]))


def test_quant_scales_are_the_ieee_quotient_and_codes_the_conversion():
    rng = np.random.default_rng(2)
    x = _rows(rng, 64, 300)
    q, s = oracle.quant_per_token_fp8(x)
    amax = np.abs(x).max(axis=1)
    s_ref = (np.maximum(amax, np.float32(1e-12)) / np.float32(448.0)).astype(np.float32)
    assert np.array_equal(s, s_ref)
    ratio = (x / s_ref[:, None]).astype(np.float32)
    assert np.array_equal(q, _torch_e4m3fn(ratio))


def test_quant_row_max_is_plus_minus_448_and_symmetry():
    rng = np.random.default_rng(3)
    x = _rows(rng, 50, 77)
    q, s = oracle.quant_per_token_fp8(x)
    q2, s2 = oracle.quant_per_token_fp8(-x)
    assert np.array_equal(s, s2)
    assert np.array_equal(q ^ 0x80, q2)  # only the sign bit differs
    for i in range(x.shape[0]):
        at = np.abs(x[i]) == np.abs(x[i]).max()
        assert np.all(q[i][at] == np.where(x[i][at] > 0, 0x7E, 0xFE))


def test_quant_power_of_two_covariance():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((20, 64)).astype(np.float32)
    q1, s1 = oracle.quant_per_token_fp8(x)
    for e in (-15, -4, 3, 25):
        qe, se = oracle.quant_per_token_fp8(np.ldexp(x, e).astype(np.float32))
        assert np.array_equal(qe, q1)
        assert np.array_equal(se, np.ldexp(s1, e).astype(np.float32))


def test_quant_scale_upper_bound_clamps_and_saturates():
    # scale_ub below the natural scale: the scale is scale_ub and values beyond
    # 448 * scale_ub saturate at +-448; above it, nothing changes
    x = np.array([[1000.0, -500.0, 10.0, 0.5], [1.0, -0.25, 0.125, 0.0]], np.float32)
    q0, s0 = oracle.quant_per_token_fp8(x)
    q1, s1 = oracle.quant_per_token_fp8(x, scale_ub=1.0)
    assert s1[0] == np.float32(1.0) and s1[1] == s0[1]
    assert np.array_equal(q1[1], q0[1])
    assert np.array_equal(q1[0], np.array([0x7E, 0xFE, 0x52, 0x30], np.uint8))
    assert _code_value(0x52) == 10 and _code_value(0x30) == Fraction(1, 2)


def test_quant_zero_row_uses_the_guard():
    q, s = oracle.quant_per_token_fp8(np.zeros((1, 16), np.float32))
    assert s[0] == np.float32(np.float32(1e-12) / np.float32(448.0))
    assert np.all(q == 0)


def test_fp8_gemm_brute_force_and_layouts():
    rng = np.random.default_rng(5)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    for m, n, k in ((1, 1, 1), (3, 5, 7), (4, 6, 33)):
        a = rng.choice(finite, (m, k))
        b = rng.choice(finite, (k, n))
        got = oracle.gemm_fp8(a, b)
        got_nk = oracle.gemm_fp8(a, np.ascontiguousarray(b.T), oracle.B_NK)
        for i in range(m):
            for j in range(n):
                want = sum(_code_value(int(a[i, t])) * _code_value(int(b[t, j])) for t in range(k))
                assert Fraction(got[i, j]) == want
                assert got_nk[i, j] == got[i, j]


def test_fp8_gemm_closed_forms():
    k = 4096
    one = np.full((2, k), 0x38, np.uint8)      # 1.0
    big = np.full((k, 3), 0x7E, np.uint8)      # 448
    neg = np.full((k, 3), 0xFE, np.uint8)      # -448
    assert np.all(oracle.gemm_fp8(one, big) == 448.0 * k)
    assert np.all(oracle.gemm_fp8(np.full((2, k), 0x7E, np.uint8), neg) == -448.0 * 448.0 * k)
    tiny = np.full((2, k), 0x01, np.uint8)     # 2^-9
    assert np.all(oracle.gemm_fp8(tiny, np.full((k, 3), 0x01, np.uint8)) == k * 2.0 ** -18)


from hypothesis import given, settings, strategies as st  # noqa: E402
from hypothesis.extra import numpy as hnp  # noqa: E402


@settings(max_examples=200, deadline=None)
@given(hnp.arrays(np.float32, st.tuples(st.integers(1, 5), st.integers(1, 40)),
                  elements=st.floats(width=32, allow_nan=False, allow_infinity=False)))
def test_generated_rows_quantize_like_torch_after_the_ieee_quotient(x):
    q, s = oracle.quant_per_token_fp8(x)
    amax = np.abs(x).max(axis=1)
    s_ref = (np.maximum(amax, np.float32(1e-12)) / np.float32(448.0)).astype(np.float32)
    assert np.array_equal(s, s_ref)
    with np.errstate(over="ignore", invalid="ignore"):
        ratio = (x / s_ref[:, None]).astype(np.float32)
    assert np.array_equal(q, _torch_e4m3fn(ratio))
    assert not np.any((q & 0x7F) == 0x7F)  # never NaN for finite input
