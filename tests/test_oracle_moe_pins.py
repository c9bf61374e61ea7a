"""Pins of the oracle's MoE grouped GEMM ("dynquant-kernels", What is in
here: one launch for all experts): rows grouped by expert, each group
multiplied by its expert's weight.  Checked against Python integer brute
force, the plain GEMM (one expert), a permutation of the experts, and empty
experts.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle


def _case(rng, counts, k, n):
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    a = rng.integers(-127, 128, (int(off[-1]), k), dtype=np.int8)
    w = rng.integers(-127, 128, (len(counts), k, n), dtype=np.int8)
    return a, w, off


def test_moe_brute_force_both_layouts():
    rng = np.random.default_rng(1)
    a, w, off = _case(rng, [2, 0, 3, 1], 5, 4)
    want = np.zeros((a.shape[0], 4), dtype=np.int64)
    for e in range(4):
        for i in range(int(off[e]), int(off[e + 1])):
            for j in range(4):
                want[i, j] = sum(int(a[i, t]) * int(w[e, t, j]) for t in range(5))
    assert np.array_equal(oracle.moe_gemm_i32(a, w, off), want)
    w_nk = np.ascontiguousarray(w.transpose(0, 2, 1))
    assert np.array_equal(oracle.moe_gemm_i32(a, w_nk, off, oracle.B_NK), want)


def test_one_expert_is_the_plain_gemm():
    rng = np.random.default_rng(2)
    a, w, off = _case(rng, [37], 64, 48)
    assert np.array_equal(oracle.moe_gemm_i32(a, w, off), oracle.gemm_i32(a, w[0]))


def test_permuting_experts_permutes_rows():
    rng = np.random.default_rng(3)
    counts = [5, 0, 9, 2, 7]
    a, w, off = _case(rng, counts, 32, 16)
    c = oracle.moe_gemm_i32(a, w, off)
    perm = [3, 0, 4, 2, 1]
    rows = np.concatenate([np.arange(off[e], off[e + 1]) for e in perm]).astype(np.int64)
    off_p = np.concatenate([[0], np.cumsum([counts[e] for e in perm])])
    c_p = oracle.moe_gemm_i32(a[rows], w[perm], off_p)
    assert np.array_equal(c_p, c[rows])


def test_dequant_uses_each_rows_expert_scales():
    c = np.array([[2], [3], [5]], np.int32)
    sa = np.array([1.0, 0.5, 2.0], np.float32)
    sb = np.array([[0.25], [4.0]], np.float32)
    out = oracle.moe_dequant(c, sa, sb, np.array([0, 1, 3]), 2.0)
    assert np.array_equal(out, np.array([[2 * 1.0 * 0.25 * 2], [3 * 0.5 * 4 * 2], [5 * 2 * 4 * 2]], np.float64))


def test_bad_offsets_are_refused():
    a = np.zeros((4, 8), np.int8)
    w = np.zeros((2, 8, 4), np.int8)
    for off in ([0, 2], [1, 2, 4], [0, 3, 2], [0, 2, 5]):
        with pytest.raises(ValueError):
            oracle.moe_gemm_i32(a, w, np.array(off))
