"""Seeded random shapes through the INT8 and FP8 entry points, against the oracle.

The grids of the other GPU test files pick shapes by hand around each
kernel's tiles; here a fixed-seed generator draws them across those
boundaries instead (ragged rows and columns, k tails, every layout and
output type, m on both sides of the decode/tiled split), so that a shape
class nobody thought of still meets the same bar: codes, scales, zero points
and INT32 accumulators bit-exact, fp32 outputs within 1e-6 relative and bf16
within one ulp of the exact result, per-group and FP8 results within their
derived bounds.  Each case prints its shape in the assertion message.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
import w8a8_int8_quantized_qk_amd as qk
from tests.gpu_compare import DTYPE_CODE, assert_equal_exact, assert_out_close, host
from w8a8_int8_quantized_qk_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TORCH_OUT = {"f32": torch.float32, "bf16": torch.bfloat16}
U = 2.0 ** -24
# QK_SWEEP_CASES widens the sweep (the default keeps the suite short)
CASES = int(os.environ.get("QK_SWEEP_CASES", "16"))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qk.library()


def _rng(*parts) -> np.random.Generator:
    s = 0
    for p in parts:
        s = (s * 1000003 + (p if isinstance(p, int) else sum(map(ord, str(p))))) % (2**32)
    return np.random.default_rng(s)


def _dim(rng, lo, hi, mult=1) -> int:
    """A size in [lo, hi], a multiple of mult, biased towards tile edges."""
    if rng.random() < 0.3:
        edge = int(rng.choice([16, 64, 128, 256, 512, 1024]))
        v = edge * int(rng.integers(1, 4)) + int(rng.integers(-1, 2)) * mult
    else:
        v = int(rng.integers(lo, hi + 1))
    v = max(lo, min(hi, v))
    return max(lo, v // mult * mult) if mult > 1 else v


@pytest.mark.parametrize("case", range(CASES))
def test_gemm_random_shapes(case):
    rng = _rng("gemm", case)
    m = _dim(rng, 1, 16) if rng.random() < 0.35 else _dim(rng, 1, 700)
    n = _dim(rng, 1, 800)
    k = _dim(rng, 0, 2400, 16)
    layout = "kn" if rng.random() < 0.6 else "nk"
    kernel = "auto" if m > 16 else str(rng.choice(["auto", "gemv", "mfma"]))
    if kernel == "gemv" and layout == "nk":
        layout = "kn"
    out_dtype = str(rng.choice(["f32", "bf16"]))
    osc = float(rng.choice([1.0, 0.5, -2.0]))
    a = rng.integers(-128, 128, size=(m, k), dtype=np.int8)
    b_kn = rng.integers(-128, 128, size=(k, n), dtype=np.int8)
    b = b_kn if layout == "kn" else np.ascontiguousarray(b_kn.T)
    sa = rng.uniform(1e-4, 1e-1, m).astype(np.float32)
    sb = rng.uniform(1e-3, 1e-2, n).astype(np.float32)
    out, c = qk.gemm_i8_scaled(torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV),
                               torch.from_numpy(sa).to(DEV), torch.from_numpy(sb).to(DEV), osc,
                               TORCH_OUT[out_dtype], layout, return_acc=True, kernel=kernel)
    what = f"gemm {m}x{n}x{k} {layout} {kernel} {out_dtype} x{osc}"
    c_ref = oracle.gemm_i32(a, b_kn, oracle.B_KN)
    assert_equal_exact(host(c), c_ref, f"{what} acc")
    assert_out_close(host(out), oracle.dequant(c_ref, sa, sb, osc), out_dtype, what)


@pytest.mark.parametrize("case", range(CASES))
def test_linear_random_shapes(case):
    rng = _rng("linear", case)
    m = _dim(rng, 1, 48) if rng.random() < 0.7 else _dim(rng, 1, 400)
    k = _dim(rng, 16, 3000, 16)
    n = _dim(rng, 1, 700)
    x_dtype = str(rng.choice(["f32", "bf16", "f16"]))
    out_dtype = str(rng.choice(["f32", "bf16"]))
    x = wl.random_activations(rng, m, k, x_dtype, outlier_cols=max(1, k // 100))
    w = wl.random_weight(rng, k, n)
    s_ch = wl.random_channel_scales(rng, n)
    out, q, s = qk.linear_w8a8(x.to(DEV), torch.from_numpy(w).to(DEV), torch.from_numpy(s_ch).to(DEV),
                               TORCH_OUT[out_dtype], return_codes=True)
    q_ref, s_ref, c_ref, out_ref = oracle.linear(wl.bits(x), DTYPE_CODE[x_dtype], w, s_ch)
    what = f"linear {m}x{k}x{n} {x_dtype} {out_dtype}"
    assert_equal_exact(host(s), s_ref, f"{what} scale")
    assert_equal_exact(host(q), q_ref, f"{what} codes")
    assert_out_close(host(out), out_ref, out_dtype, what)


@pytest.mark.parametrize("case", range(CASES))
def test_quantization_random_shapes(case):
    rng = _rng("quant", case)
    m = _dim(rng, 1, 300)
    k = _dim(rng, 1, 6000)
    dtype = str(rng.choice(["f32", "bf16", "f16"]))
    x = wl.random_activations(rng, m, 2 * k, dtype, outlier_cols=max(1, k // 50))
    # plain rows: the first k columns; silu rows: gate | up of width k
    xp = x[:, :k].contiguous()
    q, s = qk.quant_per_token(xp.to(DEV))
    q_ref, s_ref = oracle.quantize_input(wl.bits(xp), DTYPE_CODE[dtype])
    assert_equal_exact(host(s), s_ref, f"quant {m}x{k} {dtype} scale")
    assert_equal_exact(host(q), q_ref, f"quant {m}x{k} {dtype} codes")
    q, s = qk.silu_mul_quant_per_token(x.to(DEV))
    q_ref, s_ref = oracle.silu_mul_quantize(wl.bits(x), DTYPE_CODE[dtype])
    assert_equal_exact(host(s), s_ref, f"silu quant {m}x{k} {dtype} scale")
    assert_equal_exact(host(q), q_ref, f"silu quant {m}x{k} {dtype} codes")
    qa, sa_, za = qk.quant_per_token_asym(xp.to(DEV))
    qa_ref, sa_ref, za_ref = oracle.quant_per_token_asym(oracle.widen(wl.bits(xp), DTYPE_CODE[dtype]))
    assert_equal_exact(host(sa_), sa_ref, f"asym quant {m}x{k} {dtype} scale")
    assert_equal_exact(host(za), za_ref, f"asym quant {m}x{k} {dtype} zero point")
    assert_equal_exact(host(qa), qa_ref, f"asym quant {m}x{k} {dtype} codes")
    scale = float(np.float32(rng.uniform(0.01, 0.2)))
    qs = qk.quant_static(xp.to(DEV), torch.tensor([scale], dtype=torch.float32, device=DEV))
    qs_ref = oracle.quant_static(oracle.widen(wl.bits(xp), DTYPE_CODE[dtype]), scale)
    assert_equal_exact(host(qs), qs_ref, f"static quant {m}x{k} {dtype} s={scale}")


@pytest.mark.parametrize("case", range(CASES))
def test_grouped_random_shapes(case):
    rng = _rng("grouped", case)
    group = int(rng.choice([64, 128]))
    m = _dim(rng, 1, 600)
    n = _dim(rng, 1, 600)
    k = group * int(rng.integers(1, 24))
    layout = "kn" if rng.random() < 0.6 else "nk"
    a = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    b_kn = wl.random_weight(rng, k, n)
    b = b_kn if layout == "kn" else np.ascontiguousarray(b_kn.T)
    sa = rng.uniform(1e-4, 1e-1, m).astype(np.float32)
    sb = wl.random_group_scales(rng, k // group, n)
    c = qk.gemm_i8_grouped(torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV),
                           torch.from_numpy(sa).to(DEV), torch.from_numpy(sb).to(DEV), group,
                           out_dtype=None, b_layout=layout)
    exact = oracle.gemm_i8_grouped(a, b, sb, group, oracle.B_KN if layout == "kn" else oracle.B_NK)
    t = oracle.gemm_i8_grouped(np.abs(a).astype(np.int8), np.abs(b_kn).astype(np.int8), np.abs(sb), group)
    tol = (k // group + 1) * U * t
    err = np.abs(host(c).astype(np.float64) - exact)
    assert (err <= tol).all(), (f"grouped {m}x{n}x{k} g{group} {layout}: {(err > tol).sum()} beyond "
                                f"the bound, worst excess {np.max(err - tol)!r}")


@pytest.mark.parametrize("case", range(CASES // 2))
def test_moe_random_shapes(case):
    rng = _rng("moe", case)
    experts = int(rng.integers(1, 13))
    counts = rng.integers(0, 400, experts)
    counts[rng.random(experts) < 0.2] = 0  # some experts get no rows
    if counts.sum() == 0:
        counts[0] = 1
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    m = int(offsets[-1])
    n = _dim(rng, 1, 500)
    k = _dim(rng, 16, 1200, 16)
    layout = "kn" if rng.random() < 0.6 else "nk"
    a = rng.integers(-128, 128, size=(m, k), dtype=np.int8)
    w_kn = rng.integers(-128, 128, size=(experts, k, n), dtype=np.int8)
    w = w_kn if layout == "kn" else np.ascontiguousarray(np.transpose(w_kn, (0, 2, 1)))
    sa = rng.uniform(1e-4, 1e-1, m).astype(np.float32)
    sb = rng.uniform(1e-3, 1e-2, (experts, n)).astype(np.float32)
    out, c = qk.moe_gemm_i8_scaled(torch.from_numpy(a).to(DEV), torch.from_numpy(w).to(DEV),
                                   torch.from_numpy(offsets).to(DEV), torch.from_numpy(sa).to(DEV),
                                   torch.from_numpy(sb).to(DEV), out_dtype=torch.float32,
                                   b_layout=layout, return_acc=True)
    what = f"moe {experts} experts rows {counts.tolist()} {k}->{n} {layout}"
    c_ref = oracle.moe_gemm_i32(a, w_kn, offsets, oracle.B_KN)
    assert_equal_exact(host(c), c_ref, f"{what} acc")
    assert_out_close(host(out), oracle.moe_dequant(c_ref, sa, sb, offsets), "f32", what)


@pytest.mark.parametrize("case", range(CASES // 2))
def test_asym_gemm_random_shapes(case):
    rng = _rng("asym", case)
    m = _dim(rng, 1, 500)
    n = _dim(rng, 1, 500)
    k = _dim(rng, 16, 2000, 16)
    layout = "kn" if rng.random() < 0.6 else "nk"
    a = rng.integers(-128, 128, size=(m, k), dtype=np.int8)
    zp = rng.integers(-128, 128, size=m).astype(np.int32)
    b_kn = rng.integers(-128, 128, size=(k, n), dtype=np.int8)
    b = b_kn if layout == "kn" else np.ascontiguousarray(b_kn.T)
    bd = torch.from_numpy(b).to(DEV)
    c = qk.gemm_i8_asym(torch.from_numpy(a).to(DEV), torch.from_numpy(zp).to(DEV), bd,
                        qk.weight_colsum(bd, layout), out_dtype=None, b_layout=layout)
    assert_equal_exact(host(c), oracle.gemm_asym(a, zp, b_kn, oracle.B_KN),
                       f"asym gemm {m}x{n}x{k} {layout}")


@pytest.mark.parametrize("case", range(CASES // 2))
def test_fp8_random_shapes(case):
    """FP8 quantization (codes and scales exact) and the FP8 GEMM (within the
    bound the FP8 tests derive from the matrix cores' accumulation)."""
    from tests.test_gpu_fp8 import _acc_bound, _check_acc, _check_out

    rng = _rng("fp8", case)
    m = _dim(rng, 1, 400)
    n = _dim(rng, 1, 400)
    k = _dim(rng, 16, 1500, 16)
    layout = "kn" if rng.random() < 0.6 else "nk"
    dtype = str(rng.choice(["f32", "bf16", "f16"]))
    scale_ub = float(rng.choice([0.0, 0.0, 0.002]))
    x = wl.random_activations(rng, m, k, dtype, outlier_cols=max(1, k // 100))
    q, s = qk.quant_per_token_fp8(x.to(DEV), scale_ub)
    q_ref, s_ref = oracle.quantize_input_fp8(wl.bits(x), DTYPE_CODE[dtype], scale_ub)
    what = f"fp8 {m}x{n}x{k} {layout} {dtype} ub={scale_ub}"
    assert_equal_exact(host(s), s_ref, f"{what} scale")
    assert_equal_exact(host(q.view(torch.uint8)), q_ref, f"{what} codes")
    b_kn = wl.random_weight_fp8(rng, k, n)
    b = b_kn if layout == "kn" else np.ascontiguousarray(b_kn.T)
    sb = wl.random_channel_scales(rng, n)
    out_dtype = str(rng.choice(["f32", "bf16"]))
    out, c = qk.gemm_fp8_scaled(q, torch.from_numpy(b).to(DEV).view(torch.float8_e4m3fn), s,
                                torch.from_numpy(sb).to(DEV), 1.0, TORCH_OUT[out_dtype], layout,
                                return_acc=True)
    exact = oracle.gemm_fp8(q_ref, b_kn)
    bound, _ = _acc_bound(q_ref, b_kn)
    _check_acc(host(c), exact, bound, f"{what} acc")
    _check_out(host(out), oracle.dequant_fp8(exact, s_ref, sb, 1.0), bound, s_ref, sb, 1.0,
               out_dtype, f"{what} out")
