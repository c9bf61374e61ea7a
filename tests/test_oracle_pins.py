"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these compare the oracle with itself: each check is a worked value,
a closed form, an exact-rational evaluation of the IEEE definition, an
invariant of the method, a brute-force count on tiny inputs, or a special case
that reduces to a library routine.  Each is chosen so that a plausible slip in
the oracle (a dropped guard, a reciprocal instead of a division, truncation or
ties-away rounding, a clamp at -128, a transposed operand, a missing scale
factor) fails at least one of them.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# --------------------------------------------------------------------------
# step 0: widening
# --------------------------------------------------------------------------

def test_widen_bf16_matches_torch_for_every_pattern():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.widen(pats, oracle.BF16)
    ref = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_widen_f16_matches_numpy_for_every_pattern():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.widen(pats, oracle.F16)
    ref = pats.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# --------------------------------------------------------------------------
# steps 1-3: per-token quantization
# --------------------------------------------------------------------------

def test_worked_ties_round_half_to_even():
    rows = _golden_rows("quant_ties.txt")
    x = np.array([float(r[0]) for r in rows], dtype=np.float32)[None, :]
    want = np.array([int(r[1]) for r in rows], dtype=np.int8)
    q, s = oracle.quant_per_token(x)
    assert exact.f32_bits(float(s[0])) == 0x3F800000
    assert np.array_equal(q[0], want)


def test_zero_row_guard_scale():
    golden = {r[0]: int(r[1], 16) for r in _golden_rows("scale_guard.txt")}
    # the golden bits agree with the closed form evaluated exactly
    assert exact.f32_bits(exact.rn32(Fraction(1, 10**12))) == golden["guard"]
    assert exact.f32_bits(exact.scale_of(0.0)) == golden["zero_row_scale"]
    q, s = oracle.quant_per_token(np.zeros((3, 77), np.float32))
    assert all(exact.f32_bits(float(v)) == golden["zero_row_scale"] for v in s)
    assert not q.any()
    # an empty row has absmax 0 as well
    q, s = oracle.quant_per_token(np.zeros((2, 0), np.float32))
    assert all(exact.f32_bits(float(v)) == golden["zero_row_scale"] for v in s)


def test_guard_only_below_1e12():
    # a row whose absmax is below the guard uses the guard; above it, the absmax
    tiny = np.float32(3e-13)
    q, s = oracle.quant_per_token(np.array([[tiny, -tiny]], np.float32))
    assert exact.f32_bits(float(s[0])) == 0x280DD87D
    assert q[0, 0] == exact.quant_code(float(tiny), float(s[0]))
    big = np.float32(5e-12)
    q, s = oracle.quant_per_token(np.array([[big, 0]], np.float32))
    assert float(s[0]) == exact.scale_of(float(big))
    assert q[0, 0] == 127


def _random_rows(rng, m, k):
    x = rng.standard_normal((m, k)).astype(np.float32)
    mags = np.float32(10.0) ** rng.uniform(-8, 8, size=(m, 1)).astype(np.float32)
    x = (x * mags).astype(np.float32)
    idx = rng.choice(k, max(1, k // 100), replace=False)
    x[: m // 2, idx] *= np.float32(50)
    return x


def test_scale_and_codes_match_exact_division():
    rng = np.random.default_rng(1)
    x = _random_rows(rng, 24, 64)
    q, s = oracle.quant_per_token(x)
    for i in range(x.shape[0]):
        amax = float(np.max(np.abs(x[i])))
        assert float(s[i]) == exact.scale_of(amax)
        for j in range(x.shape[1]):
            assert q[i, j] == exact.quant_code(float(x[i, j]), float(s[i]))


def _reciprocal_discriminators(s: np.float32, count: int, rng) -> np.ndarray:
    """Inputs x where rint(x * RN(1/s)) differs from rint(RN(x / s)).

    Found by searching near half-integer multiples of s; the answer for each
    is then decided by the exact-rational definition, not by this search.
    """
    r = np.float32(1.0) / s
    found = []
    tries = 0
    while len(found) < count and tries < 200000:
        tries += 1
        j = int(rng.integers(-126, 127))
        base = np.float32((j + 0.5) * float(s))
        off = int(rng.integers(-3, 4))
        x = np.nextafter(base, np.float32(np.inf) if off > 0 else np.float32(-np.inf))
        for _ in range(abs(off) - 1):
            x = np.nextafter(x, np.float32(np.inf) if off > 0 else np.float32(-np.inf))
        x = np.float32(x)
        if abs(float(x)) > 127 * float(s):
            continue
        via_recip = np.rint(np.float32(x * r))
        via_div = round(exact.quant_code(float(x), float(s)))
        if via_recip != via_div:
            found.append(x)
    return np.array(found, dtype=np.float32)


def test_division_is_true_ieee_division_not_reciprocal():
    rng = np.random.default_rng(2)
    checked = 0
    for amax in [np.float32(v) for v in (1.0, 3.3, 7.77, 100.1, 0.0123, 55.5)]:
        s = np.float32(exact.scale_of(float(amax)))
        disc = _reciprocal_discriminators(s, 8, rng)
        if disc.size == 0:
            continue
        row = np.concatenate([[amax], disc]).astype(np.float32)[None, :]
        q, sc = oracle.quant_per_token(row)
        assert float(sc[0]) == float(s)
        for j, xv in enumerate(disc):
            assert q[0, j + 1] == exact.quant_code(float(xv), float(s))
        checked += disc.size
    assert checked >= 10, "discriminator search found too few cases"


def test_row_max_maps_to_plus_minus_127_and_codes_in_range():
    rng = np.random.default_rng(3)
    x = _random_rows(rng, 200, 33)
    q, s = oracle.quant_per_token(x)
    assert q.min() >= -127 and q.max() <= 127
    for i in range(x.shape[0]):
        a = np.abs(x[i])
        at_max = a == a.max()
        assert np.all(q[i][at_max] == np.sign(x[i][at_max]).astype(np.int8) * 127)


def test_codes_never_minus_128_even_at_float_extremes():
    x = np.array([[-3.4e38, 3.4e38, -1.0, 2.0e38],
                  [-1.0, -1.0, -1.0, -1.0]], np.float32)
    q, _ = oracle.quant_per_token(x)
    assert q.min() == -127 and np.all(q[1] == -127)


def test_odd_symmetry():
    rng = np.random.default_rng(4)
    x = _random_rows(rng, 40, 50)
    q1, s1 = oracle.quant_per_token(x)
    q2, s2 = oracle.quant_per_token(-x)
    assert np.array_equal(s1, s2)
    assert np.array_equal(q1, -q2)


def _all_finite_bf16() -> np.ndarray:
    """Every finite bf16 value (65,280 patterns: both signs, zero and
    subnormals included), widened to float32 by placing the bits high."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    exp = (bits >> 7) & 0xFF
    bits = bits[exp != 0xFF]
    return (bits << 16).view(np.float32)


@pytest.mark.parametrize("amax_bits", [0x0000, 0x0001, 0x0080, 0x2B8C, 0x3C00, 0x3F80, 0x4020,
                                       0x42FE, 0x447A, 0x477F, 0x5F00, 0x7F7F])
def test_quantization_of_every_bf16_value_matches_a_float32_numpy_pipeline(amax_bits):
    # a row of every finite bf16 value with |v| <= amax, plus amax itself, is
    # quantized by the oracle and by numpy's float32 arithmetic (IEEE
    # division, rint, clip): IEEE basic operations are correctly rounded, so
    # the two must agree bit for bit
    assert _all_finite_bf16().size == 65280
    amax = np.array([amax_bits << 16], np.uint32).view(np.float32)[0]
    v = _all_finite_bf16()
    row = np.concatenate([v[np.abs(v) <= amax], [amax]]).astype(np.float32)
    q, s = oracle.quant_per_token(row[None, :])
    s_ref = np.float32(np.maximum(np.float32(amax), np.float32(1e-12)) / np.float32(127.0))
    with np.errstate(over="ignore"):
        q_ref = np.clip(np.rint(row / s_ref), -127, 127).astype(np.int8)
    assert s[0].view(np.uint32) == np.float32(s_ref).view(np.uint32)
    assert np.array_equal(q[0], q_ref), np.nonzero(q[0] != q_ref)[0][:5]


def test_power_of_two_covariance():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((30, 40)).astype(np.float32)
    q1, s1 = oracle.quant_per_token(x)
    for e in (-20, -3, 1, 7, 30):
        xe = np.ldexp(x, e).astype(np.float32)
        qe, se = oracle.quant_per_token(xe)
        assert np.array_equal(qe, q1)
        assert np.array_equal(se, np.ldexp(s1, e).astype(np.float32))


def test_reconstruction_error_bound():
    # |x - q s| <= s (1/2 + 127 * 2^-24): rint moves at most 1/2, the rounded
    # quotient is within 2^-24 relative of the exact one (|x/s| <= ~127).
    rng = np.random.default_rng(6)
    x = _random_rows(rng, 64, 200)
    q, s = oracle.quant_per_token(x)
    err = np.abs(x.astype(np.float64) - q.astype(np.float64) * s[:, None].astype(np.float64))
    bound = s[:, None].astype(np.float64) * (0.5 + 127 * 2.0 ** -24)
    assert np.all(err <= bound)


def test_subnormal_inputs_are_kept():
    # no flush to zero: a row of binary32 subnormals has a guard scale, codes 0,
    # while a subnormal next to a normal max is quantized like any other value
    x = np.array([[1e-40, -2e-41, 0.0, 1e-45]], np.float32)
    q, s = oracle.quant_per_token(x)
    assert exact.f32_bits(float(s[0])) == 0x280DD87D and not q.any()
    w = oracle.widen(np.array([0x0001, 0x8001], np.uint16), oracle.BF16)
    assert w[0] > 0 and w[1] < 0  # smallest bf16 subnormals survive widening


# --------------------------------------------------------------------------
# step 0': silu(gate) * up with the binary32 exp spec
# --------------------------------------------------------------------------

def test_exp_spec_constants_are_the_nearest_binary32_values():
    from decimal import Decimal, getcontext
    getcontext().prec = 60
    ln2 = Fraction(Decimal(2).ln())
    log2e, ln2_hi, ln2_lo = (float(v) for v in oracle.spec_reduction_constants())
    assert log2e == exact.rn32(1 / ln2)
    assert ln2_hi == 0.693145751953125
    assert ln2_lo == exact.rn32(ln2 - Fraction(ln2_hi))
    taylor = oracle.spec_taylor()
    for j in range(8):
        assert float(taylor[j]) == exact.rn32(Fraction(1, math.factorial(j)))


def test_exp_spec_accuracy_against_float64_exp():
    x = np.linspace(-87.0, 88.0, 400001, dtype=np.float32)
    y = oracle.spec_expf(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    err_ulp = np.abs(y - ref) / ulp
    assert err_ulp.max() <= 2.0, err_ulp.max()


def test_exp_spec_special_values():
    y = oracle.spec_expf(np.array([0.0, -0.0, 88.5, 1000.0, -87.5, -1000.0, 1.0], np.float32))
    assert y[0] == 1.0 and y[1] == 1.0
    assert np.isinf(y[2]) and np.isinf(y[3])
    assert y[4] == 0.0 and y[5] == 0.0
    assert abs(float(y[6]) - math.e) <= 2 * float(np.spacing(np.float32(math.e)))


def test_silu_mul_special_values_and_accuracy():
    g = np.array([0.0, -0.0, 20.0, 17.5, 87.9, 100.0, -88.5, -1e30, 1.0, -1.0, 3.75, -5.5],
                 np.float32)
    u = np.ones_like(g)
    h = oracle.silu_mul(np.concatenate([g, u])[None, :])[0]
    assert h[0] == 0.0 and h[1] == 0.0
    # g >= 17.4: exp(-g) < 2^-25, so 1 + exp(-g) rounds to 1 and silu(g) = g
    assert np.array_equal(h[2:6], g[2:6])
    # g <= -88: exp(-g) overflows to +inf, silu(g) = g / inf = -0
    assert h[6] == 0.0 and np.signbit(h[6]) and h[7] == 0.0
    # elsewhere within a few ulp of the float64 function
    gg = np.linspace(-40, 40, 100001, dtype=np.float32)
    hh = oracle.silu_mul(np.concatenate([gg, np.ones_like(gg)])[None, :])[0].astype(np.float64)
    g64 = gg.astype(np.float64)
    ref = g64 / (1.0 + np.exp(-g64))
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert (np.abs(hh - ref) / ulp).max() <= 4.0


def test_silu_mul_gate_is_first_half_and_product_is_rounded_once():
    rng = np.random.default_rng(7)
    d = 37
    g = rng.standard_normal(d).astype(np.float32)
    u = rng.standard_normal(d).astype(np.float32) * np.float32(3)
    h = oracle.silu_mul(np.concatenate([g, u])[None, :])[0]
    h_swapped = oracle.silu_mul(np.concatenate([u, g])[None, :])[0]
    sil = oracle.silu_mul(np.concatenate([g, np.ones_like(g)])[None, :])[0]
    for j in range(d):
        assert float(h[j]) == exact.rn32(Fraction(float(sil[j])) * Fraction(float(u[j])))
    assert not np.array_equal(h, h_swapped)


# --------------------------------------------------------------------------
# step 4: INT8 GEMM, INT32 accumulation
# --------------------------------------------------------------------------

def _brute(a, b_kn):
    m, k = a.shape
    n = b_kn.shape[1]
    return [[sum(int(a[i, t]) * int(b_kn[t, j]) for t in range(k)) for j in range(n)]
            for i in range(m)]


@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (3, 5, 7), (8, 13, 32), (17, 9, 24), (5, 1, 48)])
def test_gemm_brute_force_both_layouts(m, n, k):
    rng = np.random.default_rng(m * 100 + n * 10 + k)
    a = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    b = rng.integers(-128, 128, size=(k, n), dtype=np.int8)
    want = np.array(_brute(a, b), dtype=np.int64)
    assert np.array_equal(oracle.gemm_i32(a, b, oracle.B_KN), want)
    assert np.array_equal(oracle.gemm_i32(a, np.ascontiguousarray(b.T), oracle.B_NK), want)
    rows = rng.integers(0, m, 11)
    cols = rng.integers(0, n, 11)
    got = oracle.gemm_entries(a, b, rows, cols, oracle.B_KN)
    assert np.array_equal(got, want[rows, cols])
    got = oracle.gemm_entries(a, np.ascontiguousarray(b.T), rows, cols, oracle.B_NK)
    assert np.array_equal(got, want[rows, cols])


def test_gemm_closed_forms_and_int32_limit():
    for K, av, bv, expect in _golden_rows("gemm_closed_forms.txt"):
        K, av, bv = int(K), int(av), int(bv)
        a = np.full((1, K), av, np.int8)
        b = np.full((K, 1), bv, np.int8)
        if expect == "OVERFLOW":
            with pytest.raises(OverflowError):
                oracle.gemm_i32(a, b)
        else:
            assert int(oracle.gemm_i32(a, b)[0, 0]) == int(expect) == K * av * bv


def test_gemm_one_hot_rows_reproduce_weight_rows_and_alternating_cancels():
    rng = np.random.default_rng(8)
    k, n = 64, 19
    w = rng.integers(-127, 128, size=(k, n), dtype=np.int8)
    a = np.zeros((k, k), np.int8)
    a[np.arange(k), np.arange(k)] = 1
    assert np.array_equal(oracle.gemm_i32(a, w), w.astype(np.int32))
    a2 = (-a).astype(np.int8)
    assert np.array_equal(oracle.gemm_i32(a2, w), -w.astype(np.int32))
    alt = np.where(np.arange(k) % 2 == 0, 1, -1).astype(np.int8)[None, :]
    assert not oracle.gemm_i32(alt, np.ones((k, n), np.int8)).any()


def test_gemm_degenerate_shapes():
    assert oracle.gemm_i32(np.zeros((0, 16), np.int8), np.zeros((16, 4), np.int8)).shape == (0, 4)
    c = oracle.gemm_i32(np.zeros((3, 0), np.int8), np.zeros((0, 4), np.int8))
    assert c.shape == (3, 4) and not c.any()


# --------------------------------------------------------------------------
# step 5: dequant epilogue and bf16 rounding
# --------------------------------------------------------------------------

def test_dequant_is_the_exact_product_to_float64_precision():
    rng = np.random.default_rng(9)
    c = rng.integers(-2**31, 2**31 - 1, size=(6, 7), dtype=np.int64).astype(np.int32)
    c[0, 0] = 0
    sa = rng.uniform(1e-4, 1, 6).astype(np.float32)
    sb = rng.uniform(1e-3, 1e-2, 7).astype(np.float32)
    for os_ in (1.0, 0.25, -3.0):
        out = oracle.dequant(c, sa, sb, os_)
        for i in range(6):
            for j in range(7):
                ex = Fraction(int(c[i, j])) * Fraction(float(sa[i])) * Fraction(float(sb[j])) \
                    * Fraction(os_)
                if ex == 0:
                    assert out[i, j] == 0
                else:
                    assert abs(Fraction(float(out[i, j])) - ex) <= abs(ex) * Fraction(4, 2**53)


def test_bf16_rounding_worked_ties():
    one = 1.0
    cases = [
        (one, 0x3F80),
        (one + 2**-8, 0x3F80),            # tie -> even (1.0)
        (one + 3 * 2**-8, 0x3F82),        # tie -> even (1 + 2^-6)
        (one + 2**-8 + 2**-20, 0x3F81),   # above the tie
        (-(one + 2**-8), 0xBF80),
        (2.0 ** -133, 0x0001),            # smallest bf16 subnormal
        (2.0 ** -134, 0x0000),            # tie at the bottom -> even (0)
        (3.4e38, 0x7F80),                 # rounds past the largest finite value
        (0.0, 0x0000),
    ]
    vals = np.array([c[0] for c in cases], np.float64)
    got = oracle.bf16_nearest(vals)
    for (v, want), g in zip(cases, got):
        assert int(g) == want, (v, hex(int(g)), hex(want))
        assert exact.rn_bf16_bits(Fraction(v)) == want


def test_bf16_rounding_matches_torch_on_binary32_values():
    rng = np.random.default_rng(10)
    v32 = (rng.standard_normal(200000) * np.float32(10.0) ** rng.uniform(-30, 30, 200000)
           ).astype(np.float32)
    v32[:1000] = (np.arange(1000, dtype=np.float32) - 500) * np.float32(2.0 ** -9)
    ours = oracle.bf16_nearest(v32.astype(np.float64))
    ref = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def _spec_expf_exact(x: float) -> float:
    """The binary32 exp spec evaluated from the IEEE definitions, one rounding per step."""
    if x > 88.0:
        return math.inf
    if x < -87.0:
        return 0.0
    log2e, ln2_hi, ln2_lo = (float(v) for v in oracle.spec_reduction_constants())
    taylor = [float(t) for t in oracle.spec_taylor()]
    n = exact.round_half_even(Fraction(exact.rn32(Fraction(x) * Fraction(log2e))))
    r = exact.rn32(Fraction(x) - n * Fraction(ln2_hi))           # fma(-n, hi, x)
    r = exact.rn32(Fraction(r) - n * Fraction(ln2_lo))           # fma(-n, lo, r)
    p = taylor[7]
    for j in range(6, -1, -1):
        p = exact.rn32(Fraction(p) * Fraction(r) + Fraction(taylor[j]))  # fma(p, r, c_j)
    return exact.rn32(Fraction(p) * Fraction(2) ** n)


def test_exp_spec_bitwise_against_stepwise_exact_evaluation():
    rng = np.random.default_rng(11)
    xs = np.concatenate([rng.uniform(-87, 88, 1500), rng.uniform(-2, 2, 500),
                         [0.0, -87.0, 88.0, 0.34657359, -0.34657359]]).astype(np.float32)
    ys = oracle.spec_expf(xs)
    for xv, yv in zip(xs, ys):
        assert exact.f32_bits(float(yv)) == exact.f32_bits(_spec_expf_exact(float(xv))), xv


def test_silu_mul_bitwise_against_stepwise_exact_evaluation():
    rng = np.random.default_rng(12)
    g = np.concatenate([rng.standard_normal(600) * 4, rng.uniform(-90, 90, 100)]).astype(np.float32)
    u = rng.standard_normal(g.size).astype(np.float32)
    h = oracle.silu_mul(np.concatenate([g, u])[None, :])[0]
    for gv, uv, hv in zip(g, u, h):
        e = _spec_expf_exact(-float(gv))
        t = exact.rn32(1 + Fraction(e)) if math.isfinite(e) else math.inf
        sg = exact.rn32(Fraction(float(gv)) / Fraction(t)) if math.isfinite(t) else -0.0 * math.copysign(1, gv)
        want = exact.rn32(Fraction(sg) * Fraction(float(uv)))
        if want == 0:
            assert float(hv) == 0.0
        else:
            assert exact.f32_bits(float(hv)) == exact.f32_bits(want), (gv, uv)


def test_dequant_entries_is_the_exact_product():
    rng = np.random.default_rng(13)
    c = rng.integers(-2**31, 2**31 - 1, size=50, dtype=np.int64).astype(np.int32)
    sa = rng.uniform(1e-4, 1, 50).astype(np.float32)
    sb = rng.uniform(1e-3, 1e-2, 50).astype(np.float32)
    out = oracle.dequant_entries(c, sa, sb, 0.5)
    for e in range(50):
        ex = Fraction(int(c[e])) * Fraction(float(sa[e])) * Fraction(float(sb[e])) / 2
        assert abs(Fraction(float(out[e])) - ex) <= abs(ex) * Fraction(4, 2**53)


# --------------------------------------------------------------------------
# property tests over generated rows (hypothesis)
# --------------------------------------------------------------------------

from hypothesis import assume, given, settings, strategies as st  # noqa: E402
from hypothesis.extra import numpy as hnp  # noqa: E402

_ROWS = hnp.arrays(np.float32, st.tuples(st.integers(1, 6), st.integers(1, 48)),
                   elements=st.floats(width=32, allow_nan=False, allow_infinity=False))


@settings(max_examples=300, deadline=None)
@given(_ROWS)
def test_generated_rows_range_symmetry_and_row_max(x):
    q, s = oracle.quant_per_token(x)
    assert q.min() >= -127 and q.max() <= 127
    q2, s2 = oracle.quant_per_token(-x)
    assert np.array_equal(s, s2) and np.array_equal(q, -q2)
    for i in range(x.shape[0]):
        a = np.abs(x[i])
        if a.max() >= np.float32(1e-12):
            at = a == a.max()
            assert np.all(q[i][at] == np.sign(x[i][at]).astype(np.int8) * 127)


@settings(max_examples=200, deadline=None)
@given(hnp.arrays(np.float32, st.tuples(st.integers(1, 4), st.integers(1, 32)),
                  elements=st.floats(-1e6, 1e6, width=32)),
       st.integers(-40, 40))
def test_generated_rows_power_of_two_covariance(x, e):
    # away from the guard and the subnormal range, scaling a row by 2^e scales
    # its scale by 2^e and leaves every code unchanged
    a = np.abs(x)
    nz = a[a > 0]
    assume(nz.size > 0 and nz.min() >= 2.0 ** -80)
    assume(np.all(a.max(axis=1) * 2.0 ** min(e, 0) >= 1e-6))
    q1, s1 = oracle.quant_per_token(x)
    xe = np.ldexp(x, e).astype(np.float32)
    qe, se = oracle.quant_per_token(xe)
    assert np.array_equal(qe, q1)
    assert np.array_equal(se, np.ldexp(s1, e).astype(np.float32))
