"""GPU parity of static (per-tensor) quantization, asymmetric per-token
quantization, weight column sums and the asymmetric GEMM against the oracle.
Codes, scales, zero points, column sums and INT32 accumulators bit-exact;
fp32 outputs within 1e-6 relative, bf16 within one ulp.  Inputs are seeded
and synthetic; nothing expected here comes from the GPU.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import w8a8_int8_quantized_qk_amd as qk
from tests.gpu_compare import DTYPE_CODE, assert_equal_exact, assert_out_close, host
from w8a8_int8_quantized_qk_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qk.library()


def _seed(*parts) -> int:
    s = 0
    for p in parts:
        s = (s * 1000003 + (p if isinstance(p, int) else sum(map(ord, str(p))))) % (2**32)
    return s


def _codes(t):
    return t.detach().view(torch.uint8).cpu().numpy() if t.dtype == torch.float8_e4m3fn else host(t)


def _check_static(x_cpu, dtype, scale, fp8, silu, x_dev=None, what=""):
    x_dev = x_cpu.to(DEV) if x_dev is None else x_dev
    s_dev = torch.tensor([scale], dtype=torch.float32, device=DEV)
    q = qk.quant_static(x_dev, s_dev, fp8=fp8, silu=silu)
    v = oracle.widen(wl.bits(x_cpu), DTYPE_CODE[dtype])
    if silu:
        v = oracle.silu_mul(v)
    want = oracle.quant_static_fp8(v, scale) if fp8 else oracle.quant_static(v, scale)
    assert_equal_exact(_codes(q), want, what)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("silu", [False, True])
@pytest.mark.parametrize("m,k", [(1, 64), (7, 512), (64, 4096), (5, 100), (3, 1003)])
def test_static_quant(dtype, fp8, silu, m, k):
    rng = np.random.default_rng(_seed("st", dtype, fp8, silu, m, k))
    x = wl.random_activations(rng, m, 2 * k if silu else k, dtype, outlier_cols=1)
    # a calibrated global scale: the tensor's absmax over the format's range,
    # drawn a little small so that some codes saturate
    amax = float(np.abs(oracle.widen(wl.bits(x), DTYPE_CODE[dtype])).max())
    scale = np.float32(0.8 * amax / (448.0 if fp8 else 127.0))
    _check_static(x, dtype, scale, fp8, silu, what=f"static {dtype} fp8={fp8} silu={silu} {m}x{k}")


@pytest.mark.parametrize("fp8", [False, True])
def test_static_quant_extreme_scales_and_misaligned_input(fp8):
    rng = np.random.default_rng(_seed("stx", fp8))
    x = wl.random_activations(rng, 9, 1024, "bf16", outlier_cols=3)
    for scale in (np.float32(1e-30), np.float32(1e30), np.float32(2.0 ** -7)):
        _check_static(x, "bf16", scale, fp8, False, what=f"scale {scale}")
    buf = torch.empty(9 * 1024 + 1, dtype=torch.bfloat16, device=DEV)
    xd = buf[1:].view(9, 1024)
    xd.copy_(x.to(DEV))
    _check_static(x, "bf16", np.float32(0.01), fp8, False, x_dev=xd, what="misaligned")


def test_static_quant_special_values():
    # infinities, signed zeros, subnormals and quotients at and next to the
    # half-integers around the +-127 clamp (the kernel clamps the quotient
    # before rounding it, the oracle after: the same integer)
    scale = np.float32(0.03125)
    halves = np.float32([126.5, 127.0, 127.5, 128.5, 300.0, 0.5, 1.5, 2.5]) * scale
    vals = np.concatenate([halves, -halves, np.nextafter(halves, np.float32(np.inf)),
                           np.nextafter(halves, np.float32(0)),
                           np.float32([np.inf, -np.inf, 0.0, -0.0, 1e-45, -1e-45, 3e38, -3e38])])
    x = np.resize(vals, (4, 64)).astype(np.float32)
    for dt in ("f32", "bf16"):
        for fp8 in (False, True):
            xt = wl.cast(x, dt)
            _check_static(xt, dt, scale, fp8, False, what=f"specials {dt} fp8={fp8}")


def test_static_quant_prefill_shape_and_grid_loop():
    # the prefill shape bench.py times, and a tensor one grid pass can not
    # cover (the kernel loops over units in steps of its whole grid)
    d = wl.generate("prefill_outliers")
    amax = float(np.abs(oracle.widen(wl.bits(d["x"]), oracle.BF16)).max())
    _check_static(d["x"], "bf16", np.float32(amax / 127.0), False, False, what="prefill static")
    del d
    rng = np.random.default_rng(_seed("stbig"))
    block = wl.random_activations(rng, 512, 8192, "bf16", outlier_cols=8)
    x = torch.from_numpy(np.resize(wl.bits(block), (32769, 8192)).view(np.int16)).view(torch.bfloat16)
    _check_static(x, "bf16", np.float32(0.05), False, False, what="grid loop")


def _check_asym(x_cpu, dtype, what=""):
    q, s, z = qk.quant_per_token_asym(x_cpu.to(DEV))
    q_ref, s_ref, z_ref = oracle.quant_per_token_asym(oracle.widen(wl.bits(x_cpu), DTYPE_CODE[dtype]))
    assert_equal_exact(host(s), s_ref, what + " scale")
    assert_equal_exact(host(z), z_ref, what + " zero point")
    assert_equal_exact(host(q), q_ref, what + " codes")
    return q, s, z, q_ref, s_ref, z_ref


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("m,k", [(1, 64), (7, 512), (256, 4096), (5, 100), (3, 16392), (4, 33000)])
def test_asym_quant(dtype, m, k):
    rng = np.random.default_rng(_seed("as", dtype, m, k))
    x = wl.random_activations(rng, m, k, dtype, outlier_cols=1)
    # shift rows so that some are all-positive or mostly negative
    shift = rng.uniform(-3, 3, (m, 1)).astype(np.float32)
    x = wl.cast(oracle.widen(wl.bits(x), DTYPE_CODE[dtype]) + shift, dtype)
    _check_asym(x, dtype, f"asym {dtype} {m}x{k}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("k", [64, 333, 4096])
def test_asym_quant_edge_rows(dtype, k):
    _check_asym(wl.edge_rows(k, dtype), dtype, f"asym edge {dtype} k={k}")


@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("k,n", [(16, 3), (4096, 14336), (1000 * 16, 37), (1300, 260), (513, 1024),
                                 (1, 4), (65535, 8)])
def test_weight_colsum(layout, k, n):
    rng = np.random.default_rng(_seed("cs", layout, k, n))
    w = rng.integers(-128, 128, (k, n), dtype=np.int8)
    wd = torch.from_numpy(w if layout == "kn" else np.ascontiguousarray(w.T)).to(DEV)
    assert_equal_exact(host(qk.weight_colsum(wd, layout)), w.astype(np.int64).sum(0).astype(np.int32),
                       f"colsum {layout} {k}x{n}")


@pytest.mark.parametrize("offset", [1, 2, 3])
def test_weight_colsum_unaligned(offset):
    """A weight whose first byte is not 4-byte aligned (n a multiple of 4)."""
    k, n = 700, 520
    rng = np.random.default_rng(_seed("cs-unaligned", offset))
    w = rng.integers(-128, 128, (k, n), dtype=np.int8)
    flat = torch.zeros(k * n + 16, dtype=torch.int8, device=DEV)
    wd = flat[offset:offset + k * n].view(k, n)
    wd.copy_(torch.from_numpy(w).to(DEV))
    assert wd.data_ptr() % 4 == offset
    assert_equal_exact(host(qk.weight_colsum(wd, "kn")), w.astype(np.int64).sum(0).astype(np.int32),
                       f"colsum unaligned +{offset}")


@pytest.mark.parametrize("m,n,k,layout", [
    (1, 128, 128, "kn"), (7, 200, 272, "kn"), (300, 130, 400, "kn"), (257, 384, 1040, "kn"),
    (513, 257, 4096, "nk"), (2048, 256, 4096, "kn"), (4, 128, 65520, "kn"),
    # the kernel with transfer waves (k % 128 == 0): ragged rows and columns
    (300, 272, 1152, "kn"), (129, 144, 384, "nk"),
])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_asym_gemm(m, n, k, layout, out_dtype):
    rng = np.random.default_rng(_seed("ag", m, n, k, layout))
    x = rng.standard_normal((m, k), dtype=np.float32) + rng.uniform(-1.5, 1.5, (m, 1)).astype(np.float32)
    q, sa, zp = oracle.quant_per_token_asym(x)
    w = rng.integers(-127, 128, (k, n), dtype=np.int8)
    wd = torch.from_numpy(w if layout == "kn" else np.ascontiguousarray(w.T)).to(DEV)
    sb = wl.random_channel_scales(rng, n)
    wsum = qk.weight_colsum(wd, layout)
    tdt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    out, c = qk.gemm_i8_asym(torch.from_numpy(q).to(DEV), torch.from_numpy(zp).to(DEV), wd, wsum,
                             torch.from_numpy(sa).to(DEV), torch.from_numpy(sb).to(DEV), 0.5, tdt,
                             layout, return_acc=True)
    c_ref = oracle.gemm_asym(q, zp, w)
    assert_equal_exact(host(c), c_ref, f"asym gemm {m}x{n}x{k} acc")
    assert_out_close(host(out), oracle.dequant(c_ref, sa, sb, 0.5), out_dtype, f"asym gemm {m}x{n}x{k} out")


def test_asym_layer_from_gpu_codes():
    # quantize on the GPU, then the GEMM; against the oracle end to end
    rng = np.random.default_rng(_seed("al"))
    x = wl.random_activations(rng, 300, 1024, "bf16", outlier_cols=10)
    q, s, z, q_ref, s_ref, z_ref = _check_asym(x, "bf16", "layer")
    w = rng.integers(-127, 128, (1024, 512), dtype=np.int8)
    sb = wl.random_channel_scales(rng, 512)
    wd = torch.from_numpy(w).to(DEV)
    out = qk.gemm_i8_asym(q, z, wd, qk.weight_colsum(wd), s, torch.from_numpy(sb).to(DEV))
    assert_out_close(host(out), oracle.dequant(oracle.gemm_asym(q_ref, z_ref, w), s_ref, sb), "bf16", "layer out")
