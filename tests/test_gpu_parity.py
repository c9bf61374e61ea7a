"""GPU parity: every libqk kernel against the CPU oracle, element by element.

Codes, scales and INT32 accumulators must match bit for bit; fp32 outputs
within 1e-6 relative and bf16 outputs within one ulp of the oracle's float64
dequant value.  Inputs are seeded and synthetic (w8a8_int8_quantized_qk_amd
.workloads); nothing expected here comes from the GPU.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import w8a8_int8_quantized_qk_amd as qk
from tests.gpu_compare import (DTYPE_CODE, TORCH_OUT, assert_equal_exact, assert_out_close,
                               host)
from w8a8_int8_quantized_qk_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


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


def _check_quant(x_cpu: torch.Tensor, dtype: str, x_dev: torch.Tensor | None = None, what=""):
    x_dev = x_cpu.to(DEV) if x_dev is None else x_dev
    q, s = qk.quant_per_token(x_dev)
    q_ref, s_ref = oracle.quantize_input(wl.bits(x_cpu), DTYPE_CODE[dtype])
    assert_equal_exact(host(s), s_ref, f"{what} scale")
    assert_equal_exact(host(q), q_ref, f"{what} codes")


def _check_silu_quant(h_cpu: torch.Tensor, dtype: str, what=""):
    q, s = qk.silu_mul_quant_per_token(h_cpu.to(DEV))
    q_ref, s_ref = oracle.silu_mul_quantize(wl.bits(h_cpu), DTYPE_CODE[dtype])
    assert_equal_exact(host(s), s_ref, f"{what} scale")
    assert_equal_exact(host(q), q_ref, f"{what} codes")


# --------------------------------------------------------------------------
# per-token quantization
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("tokens", [1, 7, 64, 256])
@pytest.mark.parametrize("hidden", [64, 512, 4096])
def test_quant_token_hidden_grid(dtype, tokens, hidden):
    rng = np.random.default_rng(_seed("q", dtype, tokens, hidden))
    x = wl.random_activations(rng, tokens, hidden, dtype, outlier_cols=max(1, hidden // 100))
    _check_quant(x, dtype, what=f"{dtype} {tokens}x{hidden}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("k", [0, 1, 3, 8, 100, 1000, 4104, 8200, 16392, 33000])
def test_quant_ragged_and_long_rows(dtype, k):
    rng = np.random.default_rng(_seed("qr", dtype, k))
    x = wl.random_activations(rng, 5, k, dtype)
    _check_quant(x, dtype, what=f"{dtype} k={k}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quant_misaligned_input_takes_the_two_pass_kernel(dtype):
    rng = np.random.default_rng(_seed("qm", dtype))
    m, k = 9, 1024
    x = wl.random_activations(rng, m, k, dtype)
    buf = torch.empty(m * k + 1, dtype=x.dtype, device=DEV)
    xd = buf[1:].view(m, k)
    xd.copy_(x.to(DEV))
    _check_quant(x, dtype, x_dev=xd, what="misaligned")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("k", [64, 333, 4096])
def test_quant_edge_rows(dtype, k):
    _check_quant(wl.edge_rows(k, dtype), dtype, what=f"edge {dtype} k={k}")


def test_quant_rounding_discriminators():
    # inputs next to half-integer multiples of the row scale, where a
    # reciprocal product or a different rounding would change the code
    rng = np.random.default_rng(_seed("disc"))
    rows = []
    for amax in rng.uniform(0.01, 300, 64).astype(np.float32):
        s = np.float32(max(amax, np.float32(1e-12))) / np.float32(127)
        j = rng.integers(-126, 126, 255)
        base = ((j + 0.5) * s).astype(np.float32)
        steps = rng.integers(-2, 3, 255)
        x = base.copy()
        for i in range(255):
            for _ in range(abs(int(steps[i]))):
                x[i] = np.nextafter(x[i], np.float32(np.inf) if steps[i] > 0 else np.float32(-np.inf))
        x = np.clip(x, -amax, amax)
        rows.append(np.concatenate([[amax], x]).astype(np.float32))
    xt = torch.from_numpy(np.stack(rows))
    _check_quant(xt, "f32", what="discriminators")


@pytest.mark.parametrize("name", ["prefill_outliers", "mlp_up", "decode_m8"])
def test_quant_full_workload(name):
    d = wl.generate(name)
    _check_quant(d["x"], d["workload"].x_dtype, what=name)


def test_quant_repeatable():
    rng = np.random.default_rng(_seed("rep"))
    x = wl.random_activations(rng, 300, 4096, "bf16", outlier_cols=41).to(DEV)
    q1, s1 = qk.quant_per_token(x)
    q2, s2 = qk.quant_per_token(x)
    assert torch.equal(q1, q2) and torch.equal(s1.view(torch.int32), s2.view(torch.int32))


# --------------------------------------------------------------------------
# silu(gate) * up fused with per-token quantization
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("tokens", [1, 7, 64, 256])
@pytest.mark.parametrize("hidden", [64, 512, 4096])
def test_silu_quant_token_hidden_grid(dtype, tokens, hidden):
    rng = np.random.default_rng(_seed("s", dtype, tokens, hidden))
    h = wl.random_activations(rng, tokens, 2 * hidden, dtype)
    _check_silu_quant(h, dtype, what=f"silu {dtype} {tokens}x{hidden}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [1, 3, 100, 14336, 16392])
def test_silu_quant_ragged_and_long_rows(dtype, d):
    rng = np.random.default_rng(_seed("sr", dtype, d))
    h = wl.random_activations(rng, 3, 2 * d, dtype)
    _check_silu_quant(h, dtype, what=f"silu {dtype} d={d}")


def test_silu_quant_extreme_gates():
    # gates across the exp limits (|g| up to 120) and exact zeros
    rng = np.random.default_rng(_seed("se"))
    g = rng.uniform(-120, 120, (16, 2048)).astype(np.float32)
    g[:, :16] = 0.0
    g[:, 16:32] = np.float32(-88.0)
    g[:, 32:48] = np.float32(87.5)
    u = rng.standard_normal((16, 2048)).astype(np.float32)
    for dt in ("f32", "bf16"):
        _check_silu_quant(wl.cast(np.concatenate([g, u], axis=1), dt), dt, what=f"extreme {dt}")


def test_silu_quant_full_workload():
    d = wl.generate("gated_down")
    _check_silu_quant(d["h"], "bf16", what="gated_down")


# --------------------------------------------------------------------------
# INT8 GEMM + dequant epilogue
# --------------------------------------------------------------------------

GEMM_SHAPES = [(1, 1, 16), (1, 512, 256), (2, 1000, 512), (3, 100, 64), (7, 63, 48),
               (8, 1040, 4096), (16, 77, 32), (33, 130, 272), (65, 257, 400),
               (256, 128, 128), (300, 385, 1040), (513, 200, 0)]


def _gemm_inputs(m, n, k, layout, seed):
    rng = np.random.default_rng(seed)
    a = rng.integers(-128, 128, size=(m, k), dtype=np.int8)
    b_kn = rng.integers(-128, 128, size=(k, n), dtype=np.int8)
    sa = rng.uniform(1e-4, 1e-1, m).astype(np.float32)
    sb = rng.uniform(1e-3, 1e-2, n).astype(np.float32)
    b = b_kn if layout == "kn" else np.ascontiguousarray(b_kn.T)
    return a, b, sa, sb


def _run_gemm_case(m, n, k, layout, kernel, out_dtype, output_scale=1.0):
    a, b, sa, sb = _gemm_inputs(m, n, k, layout, _seed("g", m, n, k, layout))
    out, c = qk.gemm_i8_scaled(torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV),
                               torch.from_numpy(sa).to(DEV), torch.from_numpy(sb).to(DEV),
                               output_scale, TORCH_OUT[out_dtype], layout, return_acc=True,
                               kernel=kernel)
    c_ref = oracle.gemm_i32(a, b, oracle.B_KN if layout == "kn" else oracle.B_NK)
    what = f"{m}x{n}x{k} {layout} {kernel} {out_dtype}"
    assert_equal_exact(host(c), c_ref, f"{what} acc")
    assert_out_close(host(out), oracle.dequant(c_ref, sa, sb, output_scale), out_dtype, what)
    # the launch without raw accumulators gives the same outputs
    out2 = qk.gemm_i8_scaled(torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV),
                             torch.from_numpy(sa).to(DEV), torch.from_numpy(sb).to(DEV),
                             output_scale, TORCH_OUT[out_dtype], layout, kernel=kernel)
    assert np.array_equal(host(out2).view(np.uint8), host(out).view(np.uint8))


@pytest.mark.parametrize("m,n,k", GEMM_SHAPES)
@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_gemm_mfma_kernel(m, n, k, layout, out_dtype):
    _run_gemm_case(m, n, k, layout, "mfma", out_dtype)


# outputs with at least one 256 x 256 tile per CU take the 256 x 256 tile
# kernel: exact multiples, ragged rows and columns, k tails past a 64-byte
# slice (k % 64 != 0), one slice, and slices fewer than the four LDS stages
WIDE_SHAPES = [(4096, 4096, 256), (4000, 4112, 208), (4096, 4096, 16), (4096, 4096, 48),
               (4096, 4096, 64), (4096, 4096, 128), (4096, 4096, 192), (3900, 4352, 1040),
               (8192, 2048, 320), (256, 65536, 96)]


@pytest.mark.parametrize("m,n,k", WIDE_SHAPES)
@pytest.mark.parametrize("layout", ["kn", "nk"])
def test_gemm_wide_tiles(m, n, k, layout):
    assert ((m + 255) // 256) * ((n + 255) // 256) >= 256  # the shape selects the 256 x 256 tiles
    _run_gemm_case(m, n, k, layout, "mfma", "bf16" if k % 128 else "f32", output_scale=0.5)


# outputs with fewer 256 x 256 tiles than CUs and k a multiple of 128 take
# the 256 x 128 kernel with separate transfer and matrix-core waves: one
# tile, one and two slices (fewer than its three LDS stages), as many slices
# as stages, ragged rows and columns, 16 columns, a few rows
SPEC_SHAPES = [(256, 128, 128), (300, 272, 256), (2048, 4096, 384), (1000, 1040, 1152),
               (513, 4096, 640), (7, 16, 256), (40, 2064, 2048)]


@pytest.mark.parametrize("m,n,k", SPEC_SHAPES)
@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_gemm_spec_tiles(m, n, k, layout, out_dtype):
    assert ((m + 255) // 256) * ((n + 255) // 256) < 256 and k % 128 == 0
    _run_gemm_case(m, n, k, layout, "mfma", out_dtype, output_scale=0.75)


@pytest.mark.parametrize("m,n,k", [s for s in GEMM_SHAPES if s[0] <= 16])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_gemm_decode_kernel(m, n, k, out_dtype):
    _run_gemm_case(m, n, k, "kn", "gemv", out_dtype)


# decode kernel with 4..8 rows per launch on the matrix cores (n % 16 == 0;
# 3 rows take the v_dot4 kernel):
# every row count, ragged column tiles and k splits, a single k split with
# its tail past k, 64 splits, and 9..16 rows as two launches
@pytest.mark.parametrize("m,n,k", [(3, 16, 16), (4, 272, 1040), (5, 4112, 3088), (6, 256, 1024),
                                   (7, 528, 2064), (8, 14336, 1024), (8, 48, 65536),
                                   (12, 512, 1024), (16, 256, 2048)])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_gemm_decode_kernel_matrix_core_rows(m, n, k, out_dtype):
    _run_gemm_case(m, n, k, "kn", "gemv", out_dtype)


# decode kernel with 1-2 rows on narrow weights (fewer than 128 workgroups at
# 512-row k slices): 128-row slices, ragged last slice, unaligned widths, and
# the 8-way column shard of the decode shape
@pytest.mark.parametrize("m,n,k", [(1, 1792, 4096), (2, 300, 1040), (1, 16, 65536), (2, 4112, 3088),
                                   (1, 77, 528)])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_gemm_decode_kernel_narrow_weights(m, n, k, out_dtype):
    _run_gemm_case(m, n, k, "kn", "gemv", out_dtype)


@pytest.mark.parametrize("kernel", ["auto", "mfma", "gemv"])
def test_gemm_output_scale(kernel):
    _run_gemm_case(4, 96, 64, "kn", kernel, "f32", output_scale=-0.375)


@pytest.mark.parametrize("kernel", ["mfma", "gemv"])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_gemm_outputs_aligned_to_their_element_only(kernel, out_dtype):
    # out and c start one element into their buffers: aligned to the element
    # size (all the ABI asks) but not to 16 bytes, so the kernels' 16-byte
    # stores must give way to element stores; the element before each view
    # stays untouched
    m = 300 if kernel == "mfma" else 5
    n, k = 136, 272
    a, b, sa, sb = _gemm_inputs(m, n, k, "kn", _seed("unaligned", m, n, k, kernel))
    dt = TORCH_OUT[out_dtype]
    obuf = torch.full((m * n + 1,), 7, dtype=dt, device=DEV)
    cbuf = torch.full((m * n + 1,), 7, dtype=torch.int32, device=DEV)
    out, c = qk.gemm_i8_scaled(torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV),
                               torch.from_numpy(sa).to(DEV), torch.from_numpy(sb).to(DEV),
                               1.0, dt, "kn", return_acc=True, out=obuf[1:].view(m, n),
                               c=cbuf[1:].view(m, n), kernel=kernel)
    assert out.data_ptr() % 16 != 0 and c.data_ptr() % 16 != 0
    c_ref = oracle.gemm_i32(a, b, oracle.B_KN)
    what = f"{m}x{n}x{k} {kernel} {out_dtype} element-aligned outputs"
    assert_equal_exact(host(c), c_ref, f"{what} acc")
    assert_out_close(host(out), oracle.dequant(c_ref, sa, sb, 1.0), out_dtype, what)
    assert obuf[0].item() == 7 and cbuf[0].item() == 7, what


@pytest.mark.parametrize("kernel", ["mfma", "gemv"])
def test_gemm_int32_closed_forms(kernel):
    # K * a * b with constant operands: K = 65536 at |q| <= 127, and -128 * -128
    # at the largest K accepted (the largest multiple of 16 below QK_MAX_K)
    # (the decode kernel with 2 rows takes dot products, with 8 the matrix cores;
    # at k <= 4096 the latter packs two rows' split-K sums into one word, whose
    # fields are sized for -128 * -128 over whole 1024-row splits)
    kmax = 131056
    for m in ((2, 8) if kernel == "gemv" else (2,)):
        for k, av, bv in ((65536, 127, 127), (65536, 127, -127), (kmax, -128, -128),
                          (4096, -128, -128), (4096, -128, 127), (3072, 127, -128), (1024, -128, -128)):
            a = torch.full((m, k), av, dtype=torch.int8, device=DEV)
            b = torch.full((k, 64), bv, dtype=torch.int8, device=DEV)
            c = qk.gemm_i8_scaled(a, b, out_dtype=None, kernel=kernel)
            assert bool((c == k * av * bv).all()), (kernel, m, k, av, bv)


def test_gemm_empty_and_zero_k():
    a = torch.empty((0, 32), dtype=torch.int8, device=DEV)
    b = torch.zeros((32, 8), dtype=torch.int8, device=DEV)
    out = qk.gemm_i8_scaled(a, b, torch.empty(0, device=DEV), torch.ones(8, device=DEV),
                            out_dtype=torch.float32)
    assert out.shape == (0, 8)
    for kernel in ("mfma", "gemv"):
        a = torch.empty((5, 0), dtype=torch.int8, device=DEV)
        b = torch.empty((0, 40), dtype=torch.int8, device=DEV)
        out, c = qk.gemm_i8_scaled(a, b, torch.ones(5, device=DEV), torch.ones(40, device=DEV),
                                   out_dtype=torch.float32, return_acc=True, kernel=kernel)
        assert not c.any() and not out.any()


def test_gemm_rejects_k_not_multiple_of_16():
    a = torch.zeros((4, 24), dtype=torch.int8, device=DEV)
    b = torch.zeros((24, 8), dtype=torch.int8, device=DEV)
    with pytest.raises(qk.QKError):
        qk.gemm_i8_scaled(a, b, out_dtype=None)


def test_gemm_repeatable_and_workspace_left_zero():
    d = wl.generate("decode_m8")
    x = d["x"].to(DEV)
    w = torch.from_numpy(d["w"]).to(DEV)
    s_ch = torch.from_numpy(d["s_ch"]).to(DEV)
    q, s = qk.quant_per_token(x)
    ws = qk.new_workspace(qk.gemm_workspace_size(8, w.shape[1], w.shape[0]), DEV)
    outs = [qk.gemm_i8_scaled(q, w, s, s_ch, return_acc=True, kernel="gemv", workspace=ws)
            for _ in range(3)]
    torch.cuda.synchronize()
    assert not ws.any()  # the decode kernel leaves its workspace zero
    for o, c in outs[1:]:
        assert torch.equal(c, outs[0][1]) and torch.equal(o.view(torch.int16),
                                                          outs[0][0].view(torch.int16))
    o_mfma, c_mfma = qk.gemm_i8_scaled(q, w, s, s_ch, return_acc=True, kernel="mfma")
    assert torch.equal(c_mfma, outs[0][1])


def test_gemm_on_a_side_stream():
    a, b, sa, sb = _gemm_inputs(300, 200, 256, "kn", 5)
    side = torch.cuda.Stream(DEV)
    with torch.cuda.stream(side):
        c = qk.gemm_i8_scaled(torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV),
                              out_dtype=None)
    side.synchronize()
    assert_equal_exact(host(c), oracle.gemm_i32(a, b), "side stream acc")


# --------------------------------------------------------------------------
# the named workloads, end to end, in the launch configuration of bench.py
# --------------------------------------------------------------------------

def _compare_rows_in_chunks(name, q_ref, s_ref, w_host, s_ch, c_dev, out_dev, out_dtype,
                            max_elems=1 << 26):
    """Every INT32 accumulator and every output of a GEMM against the oracle,
    a block of rows at a time so that host memory stays bounded (the MLP
    up-projection's 8192 x 28672 accumulators are 940 MB)."""
    m, n = c_dev.shape
    rows = max(1, max_elems // n)
    for r0 in range(0, m, rows):
        r1 = min(m, r0 + rows)
        c_ref = oracle.gemm_i32(q_ref[r0:r1], w_host)
        assert_equal_exact(host(c_dev[r0:r1]), c_ref, f"{name} acc rows {r0}..{r1 - 1}")
        assert_out_close(host(out_dev[r0:r1]), oracle.dequant(c_ref, s_ref[r0:r1], s_ch),
                         out_dtype, f"{name} out rows {r0}..{r1 - 1}")


@pytest.mark.parametrize("name", ["tiny_fp32", "decode_m1", "decode_m8", "prefill_outliers",
                                  "gated_down", "mlp_up"])
def test_workload_end_to_end(name):
    # The named workloads at their full sizes, in the launch configuration
    # bench.py times (quantization kernel, then the GEMM the shape selects):
    # codes, scales, every INT32 accumulator and every output element
    # against the oracle.
    d = wl.generate(name)
    w_cfg = d["workload"]
    w_host, s_ch_host = d["w"], d["s_ch"]
    w = torch.from_numpy(w_host).to(DEV)
    s_ch = torch.from_numpy(s_ch_host).to(DEV)
    if w_cfg.gated:
        q, s = qk.silu_mul_quant_per_token(d["h"].to(DEV))
        q_ref, s_ref = oracle.silu_mul_quantize(wl.bits(d["h"]), DTYPE_CODE[w_cfg.x_dtype])
    else:
        q, s = qk.quant_per_token(d["x"].to(DEV))
        q_ref, s_ref = oracle.quantize_input(wl.bits(d["x"]), DTYPE_CODE[w_cfg.x_dtype])
    assert_equal_exact(host(s), s_ref, f"{name} scale")
    assert_equal_exact(host(q), q_ref, f"{name} codes")
    del d

    out = qk.gemm_i8_scaled(q, w, s, s_ch, out_dtype=TORCH_OUT[w_cfg.out_dtype])
    out_acc, c = qk.gemm_i8_scaled(q, w, s, s_ch, out_dtype=TORCH_OUT[w_cfg.out_dtype],
                                   return_acc=True)
    # the two launches (with and without the accumulator output) agree bit for bit
    assert torch.equal(out.view(torch.int16 if out.dtype == torch.bfloat16 else torch.int32),
                       out_acc.view(torch.int16 if out.dtype == torch.bfloat16 else torch.int32))
    del out_acc, q, s
    _compare_rows_in_chunks(name, q_ref, s_ref, w_host, s_ch_host, c, out, w_cfg.out_dtype)


# --------------------------------------------------------------------------
# the whole layer in one call (fused decode launch, or quantization + tiled GEMM)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("m,k,n", [(1, 64, 64), (1, 4096, 1000), (3, 272, 130), (8, 512, 2048),
                                   (11, 1024, 320), (16, 256, 64), (40, 512, 256)])
@pytest.mark.parametrize("x_dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("kernel", ["auto", "gemv", "mfma"])
def test_linear_entry_point(m, k, n, x_dtype, kernel):
    if kernel == "gemv" and m > 16:
        pytest.skip("decode kernel takes m <= 16")
    rng = np.random.default_rng(_seed("lin", m, k, n, x_dtype))
    x = wl.random_activations(rng, m, k, x_dtype, outlier_cols=max(1, k // 100))
    w = wl.random_weight(rng, k, n)
    s_ch = wl.random_channel_scales(rng, n)
    out_dtype = "f32" if m % 2 else "bf16"
    out, q, s = qk.linear_w8a8(x.to(DEV), torch.from_numpy(w).to(DEV), torch.from_numpy(s_ch).to(DEV),
                               TORCH_OUT[out_dtype], kernel=kernel, return_codes=True)
    q_ref, s_ref, c_ref, out_ref = oracle.linear(wl.bits(x), DTYPE_CODE[x_dtype], w, s_ch)
    what = f"linear {m}x{k}x{n} {x_dtype} {kernel}"
    assert_equal_exact(host(s), s_ref, f"{what} scale")
    assert_equal_exact(host(q), q_ref, f"{what} codes")
    assert_out_close(host(out), out_ref, out_dtype, what)
    # without the optional code outputs (the fused launch then writes none)
    out2 = qk.linear_w8a8(x.to(DEV), torch.from_numpy(w).to(DEV), torch.from_numpy(s_ch).to(DEV),
                          TORCH_OUT[out_dtype], kernel=kernel)
    assert np.array_equal(host(out2).view(np.uint8), host(out).view(np.uint8))


# the fused decode launch with 4..8 rows (and 1-2 rows on narrow weights):
# rows held in registers, and rows too long for them (re-read per pass:
# k > 4096 for f32, > 8192 for bf16/f16)
@pytest.mark.parametrize("m,k,n", [(4, 1040, 272), (8, 4096, 528), (6, 4112, 64), (5, 8208, 80),
                                   (1, 4096, 1792), (2, 8208, 64), (1, 1040, 300)])
@pytest.mark.parametrize("x_dtype", ["f32", "bf16", "f16"])
def test_linear_decode_matrix_core_rows(m, k, n, x_dtype):
    rng = np.random.default_rng(_seed("lin-mc", m, k, n, x_dtype))
    x = wl.random_activations(rng, m, k, x_dtype, outlier_cols=max(1, k // 100))
    w = wl.random_weight(rng, k, n)
    s_ch = wl.random_channel_scales(rng, n)
    out, q, s = qk.linear_w8a8(x.to(DEV), torch.from_numpy(w).to(DEV), torch.from_numpy(s_ch).to(DEV),
                               torch.bfloat16, kernel="gemv", return_codes=True)
    q_ref, s_ref, c_ref, out_ref = oracle.linear(wl.bits(x), DTYPE_CODE[x_dtype], w, s_ch)
    what = f"linear {m}x{k}x{n} {x_dtype} gemv"
    assert_equal_exact(host(s), s_ref, f"{what} scale")
    assert_equal_exact(host(q), q_ref, f"{what} codes")
    assert_out_close(host(out), out_ref, "bf16", what)


@pytest.mark.parametrize("name", ["decode_m1", "decode_m8"])
def test_linear_decode_workloads(name):
    # the fused single-launch decode linear at the full decode shapes: codes,
    # scales and every INT32 accumulator bit-exact, every output within the bar
    d = wl.generate(name)
    wcfg = d["workload"]
    out, q, s, c = qk.linear_w8a8(d["x"].to(DEV), torch.from_numpy(d["w"]).to(DEV),
                                  torch.from_numpy(d["s_ch"]).to(DEV), TORCH_OUT[wcfg.out_dtype],
                                  return_codes=True, return_acc=True)
    q_ref, s_ref, c_ref, out_ref = oracle.linear(wl.bits(d["x"]), DTYPE_CODE[wcfg.x_dtype], d["w"],
                                                 d["s_ch"])
    assert_equal_exact(host(s), s_ref, f"{name} scale")
    assert_equal_exact(host(q), q_ref, f"{name} codes")
    assert_equal_exact(host(c), c_ref, f"{name} acc")
    assert_out_close(host(out), out_ref, wcfg.out_dtype, name)
    # the launch bench.py times (no optional outputs) writes the same outputs
    out2 = qk.linear_w8a8(d["x"].to(DEV), torch.from_numpy(d["w"]).to(DEV),
                          torch.from_numpy(d["s_ch"]).to(DEV), TORCH_OUT[wcfg.out_dtype])
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16))


@pytest.mark.parametrize("m,k,n,kernel", [(1, 4096, 1000, "gemv"), (8, 4096, 2048, "gemv"),
                                          (3, 1024, 272, "gemv"), (300, 1024, 512, "mfma")])
def test_linear_accumulator_output(m, k, n, kernel):
    # c_out of the whole-layer call: raw INT32 accumulators, alone or beside out
    rng = np.random.default_rng(_seed("lin-acc", m, k, n))
    x = wl.random_activations(rng, m, k, "bf16", outlier_cols=max(1, k // 100))
    w = wl.random_weight(rng, k, n)
    s_ch = wl.random_channel_scales(rng, n)
    xd, wd, sd = x.to(DEV), torch.from_numpy(w).to(DEV), torch.from_numpy(s_ch).to(DEV)
    q_ref, s_ref, c_ref, out_ref = oracle.linear(wl.bits(x), oracle.BF16, w, s_ch)
    c_only = qk.linear_w8a8(xd, wd, sd, out_dtype=None, kernel=kernel)
    assert_equal_exact(host(c_only), c_ref, f"{m}x{k}x{n} {kernel} c only")
    out, c = qk.linear_w8a8(xd, wd, sd, torch.float32, kernel=kernel, return_acc=True)
    assert_equal_exact(host(c), c_ref, f"{m}x{k}x{n} {kernel} c")
    assert_out_close(host(out), out_ref, "f32", f"{m}x{k}x{n} {kernel} out")


def test_hip_graph_replays_match_eager():
    # capture the decode linear (which uses the self-cleaning workspace) and a
    # prefill quant + GEMM; replay several times with eager work in between
    dec = wl.generate("decode_m8")
    pre = wl.generate(wl.Workload("pre_small", 300, 1024, 512, "bf16", "bf16", outlier_cols=10))
    xd, wd, sd = dec["x"].to(DEV), torch.from_numpy(dec["w"]).to(DEV), torch.from_numpy(dec["s_ch"]).to(DEV)
    xp, wp, sp = pre["x"].to(DEV), torch.from_numpy(pre["w"]).to(DEV), torch.from_numpy(pre["s_ch"]).to(DEV)
    ws = qk.new_workspace(qk.gemm_workspace_size(8, wd.shape[1], wd.shape[0]), DEV)
    out_d = torch.empty((8, wd.shape[1]), dtype=torch.bfloat16, device=DEV)
    q = torch.empty((300, 1024), dtype=torch.int8, device=DEV)
    s = torch.empty((300,), dtype=torch.float32, device=DEV)
    out_p = torch.empty((300, 512), dtype=torch.bfloat16, device=DEV)
    ref_d = qk.linear_w8a8(xd, wd, sd, workspace=ws).clone()
    qr, sr = qk.quant_per_token(xp)
    ref_p = qk.gemm_i8_scaled(qr, wp, sr, sp).clone()
    stream = torch.cuda.Stream(DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        qk.linear_w8a8(xd, wd, sd, out=out_d, workspace=ws)
        qk.quant_per_token(xp, q, s)
        qk.gemm_i8_scaled(q, wp, s, sp, out=out_p)
    for rep in range(4):
        out_d.zero_()
        out_p.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_d.view(torch.int16), ref_d.view(torch.int16)), rep
        assert torch.equal(out_p.view(torch.int16), ref_p.view(torch.int16)), rep
        # eager work on the same workspace between replays
        again = qk.linear_w8a8(xd, wd, sd, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), ref_d.view(torch.int16))
    assert not ws.any()


# --------------------------------------------------------------------------
# split-K of the tiled GEMM for outputs with few tiles (the workspace holds
# the INT32 partial sums; the reduction adds them in order and clears them)
# --------------------------------------------------------------------------

SPLIT_SHAPES = [(2048, 512, 4096), (300, 256, 2048), (513, 144, 3200), (17, 4096, 2048),
                (1024, 1024, 8192), (512, 512, 8192)]


@pytest.mark.parametrize("m,n,k", SPLIT_SHAPES)
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_gemm_split_k(m, n, k, out_dtype):
    assert qk.gemm_workspace_size(m, n, k) >= 2 * m * n * 4  # the plan splits these
    _run_gemm_case(m, n, k, "kn", "mfma", out_dtype, output_scale=0.75)


@pytest.mark.parametrize("m,n,k", [(2048, 512, 4096), (513, 144, 3200), (512, 512, 8192)])
def test_gemm_split_k_nk_weight(m, n, k):
    # the [N][K] layout splits too (B's row stride passed like A's)
    _run_gemm_case(m, n, k, "nk", "mfma", "bf16")


@pytest.mark.parametrize("m,n,k,layout", [(2048, 512, 4112, "kn"), (300, 200, 2048, "kn"),
                                          (300, 200, 2048, "nk"), (2048, 1024, 4096, "kn")])
def test_gemm_unsplit_shapes_with_workspace(m, n, k, layout):
    # k % 128 != 0, n % 16 != 0, and a shape whose split would not pay, run unsplit
    _run_gemm_case(m, n, k, layout, "mfma", "bf16")


@pytest.mark.parametrize("layout", ["kn", "nk"])
def test_gemm_split_k_closed_forms_and_workspace_left_zero(layout):
    m, n = 600, 384
    for k, av, bv in ((8192, -128, -128), (4096, 127, -128), (2048, -127, 127), (131072 - 128, -128, -128)):
        ws = qk.new_workspace(qk.gemm_workspace_size(m, n, k), DEV)
        assert ws.numel() > 0
        a = torch.full((m, k), av, dtype=torch.int8, device=DEV)
        b = torch.full((k, n) if layout == "kn" else (n, k), bv, dtype=torch.int8, device=DEV)
        c = qk.gemm_i8_scaled(a, b, out_dtype=None, kernel="mfma", workspace=ws, b_layout=layout)
        assert bool((c == k * av * bv).all()), (k, av, bv, layout)
        torch.cuda.synchronize()
        assert not ws.any(), "the split-K reduction leaves the workspace zero"
    # a [N][K] weight whose columns differ, at the largest k: the row stride of
    # B is k, so a wrong stride mixes columns
    k = 131072 - 128
    ws = qk.new_workspace(qk.gemm_workspace_size(m, n, k), DEV)
    a = torch.full((m, k), -128, dtype=torch.int8, device=DEV)
    col_vals = torch.arange(n, device=DEV, dtype=torch.int32) % 255 - 127
    b = col_vals.to(torch.int8)[:, None].expand(n, k).contiguous()
    if layout == "kn":
        b = b.t().contiguous()
    c = qk.gemm_i8_scaled(a, b, out_dtype=None, kernel="mfma", workspace=ws, b_layout=layout)
    want = (col_vals.to(torch.int64) * (-128 * k)).to(torch.int32)
    assert torch.equal(c, want[None, :].expand(m, n)), layout
    torch.cuda.synchronize()
    assert not ws.any()


def test_workspace_init_prepares_dirty_memory():
    # a workspace straight from the allocator holds arbitrary bytes:
    # qk_workspace_init zeroes it with the library's own kernel, after which
    # the decode kernel's settlement and split-K are exact and leave it zero
    rng = np.random.default_rng(_seed("dirty-ws"))
    nbytes = max(qk.gemm_workspace_size(2048, 512, 4096), qk.gemm_workspace_size(8, 14336, 4096))
    for size in (1000, 4096 + 48, nbytes):  # sizes that are not multiples of 16 or 256 too
        buf = torch.empty(size + 512, dtype=torch.uint8, device=DEV).fill_(0xA5)
        ws = buf[:size]
        qk.workspace_init(ws)
        torch.cuda.synchronize()
        assert not ws.any(), size
        assert bool((buf[size:] == 0xA5).all()), "init writes nothing past the workspace"
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    ws.copy_(torch.from_numpy(rng.integers(0, 256, nbytes, dtype=np.uint8)).to(DEV))
    qk.workspace_init(ws)
    for m, n, k, kernel in ((2048, 512, 4096, "mfma"), (8, 14336, 4096, "gemv"), (1, 4096, 4096, "gemv"),
                            (2, 512, 4096, "gemv")):
        a = rng.integers(-128, 128, size=(m, k), dtype=np.int8)
        b = rng.integers(-128, 128, size=(k, n), dtype=np.int8)
        c = qk.gemm_i8_scaled(torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV), out_dtype=None,
                              kernel=kernel, workspace=ws)
        assert_equal_exact(host(c), oracle.gemm_i32(a, b), f"{m}x{n}x{k} {kernel} after init")
    torch.cuda.synchronize()
    assert not ws.any()


@pytest.mark.parametrize("case", ["prefill_outliers", "split_k", "moe", "moe_wide"])
def test_tiled_kernels_repeat_bit_identical(case):
    # the tiled GEMM (k-group hand-over through LDS), the split-K pair of
    # launches and the MoE launch, three runs each on the same inputs: every
    # accumulator and output identical
    rng = np.random.default_rng(_seed("rep3", case))
    if case == "prefill_outliers":
        d = wl.generate(case)
        q, s = qk.quant_per_token(d["x"].to(DEV))
        w, s_ch = torch.from_numpy(d["w"]).to(DEV), torch.from_numpy(d["s_ch"]).to(DEV)
        run = lambda: qk.gemm_i8_scaled(q, w, s, s_ch, return_acc=True)
    elif case == "split_k":
        m, n, k = 2048, 512, 4096
        assert qk.gemm_workspace_size(m, n, k) > 0
        q = torch.from_numpy(rng.integers(-127, 128, size=(m, k), dtype=np.int8)).to(DEV)
        w = torch.from_numpy(rng.integers(-127, 128, size=(k, n), dtype=np.int8)).to(DEV)
        s = torch.from_numpy(rng.uniform(1e-3, 1e-1, m).astype(np.float32)).to(DEV)
        s_ch = torch.from_numpy(wl.random_channel_scales(rng, n)).to(DEV)
        run = lambda: qk.gemm_i8_scaled(q, w, s, s_ch, return_acc=True, kernel="mfma")
    else:
        # 4096 x 2048 takes the 256 x 128 tiles, 4096 x 4096 the 256 x 256 ones
        experts, m, n, k = 8, 4096, 2048 if case == "moe" else 4096, 1024
        counts = rng.multinomial(m, rng.dirichlet(np.full(experts, 2.0)))
        offsets = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).to(DEV)
        q = torch.from_numpy(rng.integers(-127, 128, size=(m, k), dtype=np.int8)).to(DEV)
        w = torch.from_numpy(rng.integers(-127, 128, size=(experts, k, n), dtype=np.int8)).to(DEV)
        s = torch.from_numpy(rng.uniform(1e-3, 1e-1, m).astype(np.float32)).to(DEV)
        s_ch = torch.from_numpy(rng.uniform(1e-3, 1e-2, (experts, n)).astype(np.float32)).to(DEV)
        run = lambda: qk.moe_gemm_i8_scaled(q, w, offsets, s, s_ch, return_acc=True)
    first_out, first_c = run()
    for _ in range(2):
        out, c = run()
        assert torch.equal(c, first_c), case
        assert torch.equal(out.view(torch.int16), first_out.view(torch.int16)), case


def test_hip_graph_replays_of_split_k_match_eager():
    # a split-K GEMM and the decode linear captured on one workspace, replayed
    # with eager split-K work in between; the reduction clears the partial
    # sums with stores (no memset nodes in the graph)
    rng = np.random.default_rng(_seed("split-graph"))
    m, n, k = 512, 512, 8192
    a = torch.from_numpy(rng.integers(-128, 128, size=(m, k), dtype=np.int8)).to(DEV)
    b = torch.from_numpy(rng.integers(-128, 128, size=(k, n), dtype=np.int8)).to(DEV)
    sa = torch.from_numpy(rng.uniform(1e-4, 1e-1, m).astype(np.float32)).to(DEV)
    sb = torch.from_numpy(rng.uniform(1e-3, 1e-2, n).astype(np.float32)).to(DEV)
    dec = wl.generate("decode_m8")
    xd, wd, sd = dec["x"].to(DEV), torch.from_numpy(dec["w"]).to(DEV), torch.from_numpy(dec["s_ch"]).to(DEV)
    ws = qk.new_workspace(max(qk.gemm_workspace_size(m, n, k), qk.gemm_workspace_size(8, wd.shape[1], wd.shape[0])), DEV)
    ref_s = qk.gemm_i8_scaled(a, b, sa, sb, kernel="mfma", workspace=ws).clone()
    ref_d = qk.linear_w8a8(xd, wd, sd, workspace=ws).clone()
    out_s = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    out_d = torch.empty((8, wd.shape[1]), dtype=torch.bfloat16, device=DEV)
    stream = torch.cuda.Stream(DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        qk.gemm_i8_scaled(a, b, sa, sb, out=out_s, kernel="mfma", workspace=ws)
        qk.linear_w8a8(xd, wd, sd, out=out_d, workspace=ws)
    for rep in range(4):
        out_s.zero_()
        out_d.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_s.view(torch.int16), ref_s.view(torch.int16)), rep
        assert torch.equal(out_d.view(torch.int16), ref_d.view(torch.int16)), rep
        again = qk.gemm_i8_scaled(a, b, sa, sb, kernel="mfma", workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), ref_s.view(torch.int16))
    assert not ws.any()
    c_ref = oracle.gemm_i32(host(a), host(b))
    assert_out_close(host(ref_s), oracle.dequant(c_ref, host(sa), host(sb)), "bf16", "split-K graph")


def test_gemm_split_k_then_decode_share_a_workspace():
    # a split-K GEMM and a decode GEMM in turn on one workspace: both exact
    rng = np.random.default_rng(_seed("split-share"))
    ws = qk.new_workspace(max(qk.gemm_workspace_size(2048, 512, 4096), qk.gemm_workspace_size(8, 4096, 4096)), DEV)
    for _ in range(2):
        for (m, n, k, kernel) in ((2048, 512, 4096, "mfma"), (8, 4096, 4096, "gemv"), (2, 512, 4096, "gemv")):
            a = rng.integers(-128, 128, size=(m, k), dtype=np.int8)
            b = rng.integers(-128, 128, size=(k, n), dtype=np.int8)
            c = qk.gemm_i8_scaled(torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV), out_dtype=None,
                                  kernel=kernel, workspace=ws)
            assert_equal_exact(host(c), oracle.gemm_i32(a, b), f"{m}x{n}x{k} {kernel} shared workspace")
    torch.cuda.synchronize()
    assert not ws.any()
