"""The split-K workspace words of the decode kernels, simulated on the host.

The GPU kernels settle split-K partial sums with returning 64-bit atomic adds
and let the arrival whose add returns the last-but-one count finish the
column.  Two encodings are used:
  * one row per word: count * 2^40 + sum (two's complement, wrapping at 2^64);
  * two rows per word: count * 2^56 + sum(p_hi + B) * 2^28 + sum(p_lo + B),
    with B = 2^24 for at most 4 arrivals of at most 1024 k each (matrix-core
    kernel), and B = 2^14 * slice rows for splits * slice rows <= 4096
    (dot-product kernel: 8 slices of 512 rows, or 32 of 128).
These tests replay every arrival order with partial sums at the extremes the
kernels allow and check that the decoding recovers the exact totals, i.e.
that no field ever carries into another.  (The kernels' own results are
checked against the oracle in the GPU tests.)
"""
import itertools

import numpy as np

M64 = (1 << 64) - 1


def settle_one_row(partials):
    """Returns (total seen by the last arrival, final word before reset)."""
    word = 0
    splits = len(partials)
    for p in partials:
        old = word
        word = (word + (1 << 40) + (p & M64)) & M64
        o = old - (1 << 64) if old >> 63 else old  # as signed
        count = (o + (1 << 39)) >> 40
        if count == splits - 1:
            return int(o - (count << 40)) + p
    raise AssertionError("no arrival saw the last count")


def settle_two_rows(pairs, kb=1 << 24):
    kf = (1 << 28) - 1
    word = 0
    splits = len(pairs)
    for lo, hi in pairs:
        old = word
        word = (word + (1 << 56) + (lo + kb) + ((hi + kb) << 28)) & M64
        count = old >> 56
        if count == splits - 1:
            return ((old & kf) - count * kb + lo, ((old >> 28) & kf) - count * kb + hi)
    raise AssertionError("no arrival saw the last count")


def test_one_row_words_extremes_every_order():
    ext = [-(1 << 31) // 8, (1 << 31) // 8 - 1, 0, -12345]
    for perm in itertools.permutations(ext):
        assert settle_one_row(list(perm)) == sum(ext)


def test_one_row_words_random():
    rng = np.random.default_rng(7)
    for _ in range(2000):
        splits = int(rng.integers(1, 129))
        bound = (1 << 31) // splits
        parts = [int(v) for v in rng.integers(-bound, bound, splits)]
        assert settle_one_row(parts) == sum(parts)


def test_two_row_words_extremes_every_order():
    b = 1 << 24  # |partial| <= 128 * 128 * 1024
    for lo_vals in ([b, b, b, b], [-b, -b, -b, -b], [b, -b, b, -b], [b, 0, -b, 7]):
        hi_vals = [-v for v in lo_vals]
        for perm in itertools.permutations(range(4)):
            pairs = [(lo_vals[i], hi_vals[i]) for i in perm]
            assert settle_two_rows(pairs) == (sum(lo_vals), sum(hi_vals))


def test_two_row_words_random_and_fewer_splits():
    rng = np.random.default_rng(11)
    b = 1 << 24
    for _ in range(5000):
        splits = int(rng.integers(1, 5))
        lo = [int(v) for v in rng.integers(-b, b + 1, splits)]
        hi = [int(v) for v in rng.integers(-b, b + 1, splits)]
        assert settle_two_rows(list(zip(lo, hi))) == (sum(lo), sum(hi))


def test_two_row_fields_never_carry():
    # the largest field value any arrival can see stays inside 28 bits
    b = 1 << 24
    assert 4 * (b + b) < (1 << 28)
    assert 4 < (1 << 8)  # the count field (bits 56..63) holds up to 4 arrivals


def test_two_row_words_dot_product_kernel_slices():
    # B = 2^14 * slice rows; splits * slice rows <= 4096
    rng = np.random.default_rng(13)
    for slice_rows, splits in ((512, 8), (128, 32), (512, 1), (128, 9)):
        b = 16384 * slice_rows
        assert 2 * b * splits <= 1 << 27
        for vals in ([b] * splits, [-b] * splits):
            pairs = [(v, -v) for v in vals]
            assert settle_two_rows(pairs, b) == (sum(vals), -sum(vals))
        for _ in range(500):
            lo = [int(v) for v in rng.integers(-b, b + 1, splits)]
            hi = [int(v) for v in rng.integers(-b, b + 1, splits)]
            order = rng.permutation(splits)
            pairs = [(lo[i], hi[i]) for i in order]
            assert settle_two_rows(pairs, b) == (sum(lo), sum(hi))
