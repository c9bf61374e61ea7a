"""GPU parity of the FP8 (float8_e4m3fn) path against the CPU oracle.

Codes and scales must match bit for bit.  The FP8 GEMM accumulates on the
matrix cores, whose FP8 dot product is not exact, so its accumulators are
compared with the oracle's exact sums within a bound derived from that
arithmetic.  Measured on gfx950 (v_mfma_f32_16x16x128_f8f6f4, e4m3 x e4m3)
with single-instruction probes of chosen operands:

  * every product of two e4m3fn values is exact (4 x 4 significant bits);
  * the products of each group of 8 consecutive k (one register pair of a
    lane) are aligned to the group's largest one: each is truncated toward
    zero to a multiple of 2^(E - 13), E = floor(log2(max |product| of the
    group)); the largest product itself is never cut;
  * the group sums and the accumulator are then added with round to nearest
    into binary32.

So one 128-deep step errs by less than 7 * 2^-13 * max_g per group g (seven
truncated products), plus binary32 rounding; allowing two roundings per step,
each at most u = 2^-24 relative to sum_t |a_t b_t|:

  |c - exact| <= 7 * 2^-13 * sum_g max_{t in g} |a_t b_t|
                 + (ceil(K / 128) + 1) * 2^-23 * sum_t |a_t b_t|.

The epilogue adds two binary32 roundings of its own (and bf16's rounding for
bf16 outputs).  Inputs are seeded and synthetic; nothing expected here comes
from the GPU.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import w8a8_int8_quantized_qk_amd as qk
from tests.gpu_compare import DTYPE_CODE, assert_equal_exact, host
from w8a8_int8_quantized_qk_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
U = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qk.library()  # raises when the HIP library is missing


def _seed(*parts) -> int:
    s = 0
    for p in parts:
        s = (s * 1000003 + (p if isinstance(p, int) else sum(map(ord, str(p))))) % (2**32)
    return s


def _codes(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.uint8).cpu().numpy()


def _check_quant(x_cpu, dtype, scale_ub=0.0, x_dev=None, what=""):
    x_dev = x_cpu.to(DEV) if x_dev is None else x_dev
    q, s = qk.quant_per_token_fp8(x_dev, scale_ub)
    q_ref, s_ref = oracle.quantize_input_fp8(wl.bits(x_cpu), DTYPE_CODE[dtype], scale_ub)
    assert q.dtype == torch.float8_e4m3fn
    assert_equal_exact(host(s), s_ref, f"{what} scale")
    assert_equal_exact(_codes(q), q_ref, f"{what} codes")


def _check_silu_quant(h_cpu, dtype, scale_ub=0.0, what=""):
    q, s = qk.silu_mul_quant_per_token_fp8(h_cpu.to(DEV), scale_ub)
    q_ref, s_ref = oracle.silu_mul_quantize_fp8(wl.bits(h_cpu), DTYPE_CODE[dtype], scale_ub)
    assert_equal_exact(host(s), s_ref, f"{what} scale")
    assert_equal_exact(_codes(q), q_ref, f"{what} codes")


# --------------------------------------------------------------------------
# per-token FP8 quantization
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("tokens", [1, 7, 64, 256])
@pytest.mark.parametrize("hidden", [64, 512, 4096])
def test_fp8_quant_token_hidden_grid(dtype, tokens, hidden):
    rng = np.random.default_rng(_seed("f8q", dtype, tokens, hidden))
    x = wl.random_activations(rng, tokens, hidden, dtype, outlier_cols=max(1, hidden // 100))
    _check_quant(x, dtype, what=f"{dtype} {tokens}x{hidden}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("tokens", [1, 7, 64, 256])
@pytest.mark.parametrize("hidden", [64, 512, 4096])
def test_fp8_silu_quant_token_hidden_grid(dtype, tokens, hidden):
    rng = np.random.default_rng(_seed("f8s", dtype, tokens, hidden))
    h = wl.random_activations(rng, tokens, 2 * hidden, dtype)
    _check_silu_quant(h, dtype, what=f"silu {dtype} {tokens}x{hidden}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("k", [0, 1, 3, 8, 100, 1000, 4104, 16392, 33000])
def test_fp8_quant_ragged_and_long_rows(dtype, k):
    rng = np.random.default_rng(_seed("f8r", dtype, k))
    x = wl.random_activations(rng, 5, k, dtype)
    _check_quant(x, dtype, what=f"{dtype} k={k}")
    _check_quant(x, dtype, scale_ub=1e-3, what=f"{dtype} k={k} bounded")


@pytest.mark.parametrize("d", [3, 100, 14336, 16392])
def test_fp8_silu_quant_ragged_and_long_rows(d):
    rng = np.random.default_rng(_seed("f8sr", d))
    h = wl.random_activations(rng, 3, 2 * d, "bf16")
    _check_silu_quant(h, "bf16", what=f"silu d={d}")
    _check_silu_quant(h, "bf16", scale_ub=2e-4, what=f"silu d={d} bounded")


def test_fp8_quant_misaligned_input_takes_the_two_pass_kernel():
    rng = np.random.default_rng(_seed("f8m"))
    m, k = 9, 1024
    x = wl.random_activations(rng, m, k, "bf16")
    buf = torch.empty(m * k + 1, dtype=x.dtype, device=DEV)
    xd = buf[1:].view(m, k)
    xd.copy_(x.to(DEV))
    _check_quant(x, "bf16", x_dev=xd, what="misaligned")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("k", [64, 333, 4096])
@pytest.mark.parametrize("scale_ub", [0.0, 1e-30, 0.01])
def test_fp8_quant_edge_rows(dtype, k, scale_ub):
    # scale_ub 1e-30 binds on every row: codes saturate and, for the largest
    # finite inputs, the quotient overflows binary32
    _check_quant(wl.edge_rows(k, dtype), dtype, scale_ub, what=f"edge {dtype} k={k} ub={scale_ub}")


@pytest.mark.parametrize("scale_ub", [1e-4, 3e-3, 0.02, 1.0, -1.0])
def test_fp8_quant_scale_bound(scale_ub):
    rng = np.random.default_rng(_seed("f8ub", scale_ub))
    x = wl.random_activations(rng, 64, 4096, "bf16", outlier_cols=41)
    _check_quant(x, "bf16", scale_ub, what=f"ub={scale_ub}")


def test_fp8_conversion_through_unit_scale_rows():
    # rows whose absmax is 448 have scale exactly 1, so their codes are the
    # plain conversion of the values: every midpoint between neighbouring
    # codes and two binary32 steps either side, plus values spread over all
    # binades the format covers and beyond
    vals = []
    for c in range(0x7E):
        lo, hi = oracle.fp8_decode(np.array([c, c + 1], np.uint8))
        mid = np.float32((lo + hi) / 2)
        for step in range(-2, 3):
            v = mid
            for _ in range(abs(step)):
                v = np.nextafter(v, np.float32(np.inf) if step > 0 else np.float32(-np.inf))
            vals.append(v)
    rng = np.random.default_rng(_seed("f8conv"))
    spread = (rng.standard_normal(1 << 20) * np.exp2(rng.uniform(-16, 9.5, 1 << 20))).astype(np.float32)
    v = np.concatenate([np.array(vals, np.float32), -np.array(vals, np.float32), spread,
                        np.array([0.0, -0.0, 1e-45, -1e-45], np.float32)])
    v = np.clip(v, -448.0, 448.0).astype(np.float32)
    per_row = 4095
    rows = math.ceil(v.size / per_row)
    x = np.zeros((rows, per_row + 1), np.float32)
    x[:, 0] = 448.0
    x[:, 1:].flat[: v.size] = v
    _check_quant(torch.from_numpy(x), "f32", what="unit-scale conversion")
    q, s = oracle.quant_per_token_fp8(x)
    assert np.all(s == 1.0)
    assert np.array_equal(q[:, 1:].reshape(-1)[: v.size], oracle.fp8_encode(v))


def test_fp8_quant_full_workloads():
    d = wl.generate("prefill_outliers")
    _check_quant(d["x"], "bf16", what="prefill_outliers")
    d = wl.generate("gated_down")
    h = d["h"][:256]
    _check_silu_quant(h, "bf16", what="gated_down rows 0-255")


def test_fp8_quant_empty():
    q, s = qk.quant_per_token_fp8(torch.empty((0, 64), dtype=torch.bfloat16, device=DEV))
    assert q.shape == (0, 64) and s.shape == (0,)


# --------------------------------------------------------------------------
# FP8 GEMM
# --------------------------------------------------------------------------

def _fp8_operands(rng, m, n, k, layout):
    x = rng.standard_normal((m, k), dtype=np.float32)
    a, sa = oracle.quant_per_token_fp8(x)  # realistic codes: each row reaches +-448
    b_kn = wl.random_weight_fp8(rng, k, n)
    b = b_kn if layout == "kn" else np.ascontiguousarray(b_kn.T)
    sb = wl.random_channel_scales(rng, n)
    return a, sa, b, b_kn, sb


_LUT = None


def _acc_bound(a, b_kn):
    global _LUT
    if _LUT is None:
        _LUT = np.abs(oracle.fp8_decode(np.arange(256, dtype=np.uint8)))
    k = a.shape[1]
    absum = oracle.gemm_fp8(a & 0x7F, b_kn & 0x7F)  # sum_t |a_t b_t|, exact
    va, vb = _LUT[a], _LUT[b_kn]
    gmax = np.zeros(absum.shape)
    for j in range(0, k, 8):  # groups of 8 consecutive k
        gmax += (va[:, j:j + 8, None] * vb[None, j:j + 8, :]).max(axis=1)
    return 7 * 2.0 ** -13 * gmax + (math.ceil(k / 128) + 1) * 2.0 ** -23 * absum, absum


def _check_acc(c_gpu, exact, bound, what):
    err = np.abs(c_gpu.astype(np.float64) - exact)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err - bound, -np.inf)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} accumulators beyond the bound; worst at {i}: "
                             f"got {c_gpu[i]!r} exact {exact[i]!r} bound {bound[i]!r}")


def _check_out(got, exact_out, acc_bound, sa, sb, osc, out_dtype, what):
    scale = np.abs(sa.astype(np.float64)[:, None] * sb.astype(np.float64)[None, :] * osc)
    tol = acc_bound * scale * (1 + 4 * U) + 4 * U * np.abs(exact_out)
    if out_dtype == "f32":
        g = got.astype(np.float64)
    else:
        g = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        tol = tol + 2.0 ** -7 * np.abs(exact_out)  # one bf16 ulp
    err = np.abs(g - exact_out)
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err - tol, -np.inf)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} outputs beyond tolerance; worst at {i}: "
                             f"got {g[i]!r} exact {exact_out[i]!r} tol {tol[i]!r}")


SHAPES = [
    (1, 128, 128, "kn"),      # one tile, one slice
    (7, 200, 272, "kn"),      # n % 16 != 0, n % 4 == 0: register-staged weight; K tail
    (300, 130, 400, "kn"),    # n % 4 != 0: byte-staged weight; ragged m and K tail
    (257, 384, 1040, "kn"),   # DMA weight, ragged m, K tail
    (256, 128, 128, "nk"),
    (513, 257, 4096, "nk"),   # [N][K] weight, ragged m and n, 32 slices
    (64, 4096, 4096, "kn"),
    (2048, 128, 4096, "kn"),  # the prefill row count
    (300, 272, 256, "kn"),    # transfer waves: two slices, fewer than the LDS stages
    (129, 144, 384, "nk"),    # transfer waves: three slices, ragged m and n
]


@pytest.mark.parametrize("m,n,k,layout", SHAPES)
def test_fp8_gemm_against_exact_sums(m, n, k, layout):
    rng = np.random.default_rng(_seed("f8g", m, n, k, layout))
    a, sa, b, b_kn, sb = _fp8_operands(rng, m, n, k, layout)
    exact = oracle.gemm_fp8(a, b_kn)
    bound, absum = _acc_bound(a, b_kn)
    ad = torch.from_numpy(a).to(DEV).view(torch.float8_e4m3fn)
    bd = torch.from_numpy(b).to(DEV).view(torch.float8_e4m3fn)
    sad, sbd = torch.from_numpy(sa).to(DEV), torch.from_numpy(sb).to(DEV)
    for out_dtype, osc in (("f32", 1.0), ("bf16", 0.5)):
        tdt = torch.float32 if out_dtype == "f32" else torch.bfloat16
        out, c = qk.gemm_fp8_scaled(ad, bd, sad, sbd, osc, tdt, layout, return_acc=True)
        c_h = host(c)
        _check_acc(c_h, exact, bound, f"{m}x{n}x{k} {layout} acc")
        used = np.max(np.abs(c_h - exact) / np.maximum(bound, 1e-300))
        print(f"{m}x{n}x{k} {layout}: largest |c - exact| is {used:.3f} of the bound")
        exact_out = oracle.dequant_fp8(exact, sa, sb, osc)
        _check_out(host(out), exact_out, bound, sa, sb, osc, out_dtype, f"{m}x{n}x{k} {out_dtype}")


def test_fp8_gemm_exact_when_sums_are_representable():
    # small-integer codes (|v| <= 8, multiples of 1/2) over K = 512: every
    # partial sum is a multiple of 1/4 below 2^15, exact in binary32 however
    # the hardware orders and rounds it
    rng = np.random.default_rng(_seed("f8x"))
    m, n, k = 300, 272, 512
    vals = np.array([0.0, 0.5, -0.5, 1.0, -1.0, 1.5, -2.0, 3.0, -4.0, 6.0, 8.0, -8.0], np.float32)
    a = oracle.fp8_encode(rng.choice(vals, (m, k)))
    b = oracle.fp8_encode(rng.choice(vals, (k, n)))
    exact = oracle.gemm_fp8(a, b)
    c = qk.gemm_fp8_scaled(torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV),
                           out_dtype=None)
    assert_equal_exact(host(c), exact.astype(np.float32), "representable sums")


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_fp8_gemm_outputs_aligned_to_their_element_only(out_dtype):
    rng = np.random.default_rng(_seed("f8al", out_dtype))
    m, n, k = 70, 96, 256
    a, sa, b, b_kn, sb = _fp8_operands(rng, m, n, k, "kn")
    exact = oracle.gemm_fp8(a, b_kn)
    bound, _ = _acc_bound(a, b_kn)
    tdt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    out_buf = torch.zeros(m * n + 1, dtype=tdt, device=DEV)
    c_buf = torch.zeros(m * n + 1, dtype=torch.float32, device=DEV)
    out, c = out_buf[1:].view(m, n), c_buf[1:].view(m, n)
    qk.gemm_fp8_scaled(torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV),
                       torch.from_numpy(sa).to(DEV), torch.from_numpy(sb).to(DEV), 1.0, tdt,
                       return_acc=True, out=out, c=c)
    _check_acc(host(c), exact, bound, "offset c")
    _check_out(host(out), oracle.dequant_fp8(exact, sa, sb, 1.0), bound, sa, sb, 1.0, out_dtype,
               "offset out")
    assert out_buf[0].item() == 0 and c_buf[0].item() == 0


def test_fp8_gemm_zero_k_and_empty():
    a = torch.empty((5, 0), dtype=torch.float8_e4m3fn, device=DEV)
    b = torch.empty((0, 32), dtype=torch.float8_e4m3fn, device=DEV)
    c = qk.gemm_fp8_scaled(a, b, out_dtype=None)
    assert torch.count_nonzero(c).item() == 0
    e = qk.gemm_fp8_scaled(torch.empty((0, 64), dtype=torch.float8_e4m3fn, device=DEV),
                           torch.zeros((64, 32), dtype=torch.float8_e4m3fn, device=DEV),
                           out_dtype=None)
    assert e.shape == (0, 32)


# --------------------------------------------------------------------------
# the FP8 layer at the prefill shape
# --------------------------------------------------------------------------

def test_fp8_linear_prefill_shape_sampled_rows():
    d = wl.generate("prefill_outliers", weight="fp8")
    x, w, s_ch = d["x"], d["w"], d["s_ch"]
    out, q, s = qk.linear_fp8(x.to(DEV), torch.from_numpy(w).to(DEV), torch.from_numpy(s_ch).to(DEV),
                              return_codes=True)
    q_ref, s_ref = oracle.quantize_input_fp8(wl.bits(x), DTYPE_CODE["bf16"])
    assert_equal_exact(host(s), s_ref, "prefill fp8 scale")
    assert_equal_exact(_codes(q), q_ref, "prefill fp8 codes")
    rows = np.array([0, 1, 255, 256, 1023, 1500, 2046, 2047])
    exact = oracle.gemm_fp8(q_ref[rows], w)
    bound, _ = _acc_bound(q_ref[rows], w)
    _check_out(host(out)[rows], oracle.dequant_fp8(exact, s_ref[rows], s_ch, 1.0), bound,
               s_ref[rows], s_ch, 1.0, "bf16", "prefill fp8 out")
