"""GPU parity of silu(gate) * up (qk_silu_mul) against the oracle, bit for bit.

The quantization kernels share this arithmetic (silu of the gate, times up).
For 16-bit gates they divide g / (1 + e^-g) by a hardware reciprocal with one
correction step instead of the IEEE sequence; that such a quotient is
correctly rounded is not a theorem for arbitrary binary32 operands, so its
exactness here rests on these tests, which cover every one of the 65536
gate values of bf16 and of fp16 (the denominator is a function of the gate).
binary32 gates keep the IEEE division and are checked at random, at the exp
limits and at special values.  NaN results must be NaN (payloads are not
compared); every other result must have the oracle's bits.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import w8a8_int8_quantized_qk_amd as qk
from tests.gpu_compare import DTYPE_CODE
from w8a8_int8_quantized_qk_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

ONE_BITS = {"bf16": 0x3F80, "f16": 0x3C00}
TORCH_16 = {"bf16": torch.bfloat16, "f16": torch.float16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qk.library()  # raises when the HIP library is missing


def _assert_same(got: np.ndarray, want: np.ndarray, what: str):
    assert got.shape == want.shape, what
    g_nan, w_nan = np.isnan(got), np.isnan(want)
    assert np.array_equal(g_nan, w_nan), f"{what}: NaN positions differ"
    gb = got.view(np.uint32)[~w_nan]
    wb = want.view(np.uint32)[~w_nan]
    bad = np.nonzero(gb != wb)[0]
    if bad.size:
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} results differ; first: got {gb[i]:#010x} "
                             f"want {wb[i]:#010x}")


def _run(h_bits: np.ndarray, dtype: str, what: str):
    """h_bits: [m, 2d] raw storage (uint16 for 16-bit formats, float32 otherwise)."""
    if dtype == "f32":
        h = torch.from_numpy(np.ascontiguousarray(h_bits, np.float32))
    else:
        h = torch.from_numpy(np.ascontiguousarray(h_bits, np.uint16).view(np.int16)).view(
            TORCH_16[dtype])
    got = qk.silu_mul(h.to(DEV)).cpu().numpy()
    want = oracle.silu_mul(oracle.widen(h_bits, DTYPE_CODE[dtype]))
    _assert_same(got, want, what)
    return got


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_silu_every_16bit_gate(dtype):
    # every bit pattern as a gate: with up = 1 the result is the quotient
    # g / (1 + e^-g) itself; with seeded random ups, the product after it
    gates = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    ones = np.full_like(gates, ONE_BITS[dtype])
    _run(np.concatenate([gates, ones], axis=1), dtype, f"{dtype} gates, up = 1")
    rng = np.random.default_rng(7)
    ups = wl.bits(wl.cast(rng.standard_normal((256, 256)).astype(np.float32) * 3, dtype))
    _run(np.concatenate([gates, ups], axis=1), dtype, f"{dtype} gates, random ups")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_silu_16bit_gates_through_the_fused_quantization(dtype):
    # the same 65536 gates through the fused kernel (row-cached path): codes
    # and scales from the oracle's silu of each row
    gates = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(64, 1024)
    finite = oracle.widen(gates, DTYPE_CODE[dtype])
    gates = np.where(np.isfinite(finite), gates, np.uint16(0))  # one scale per row needs finite rows
    rng = np.random.default_rng(11)
    ups = wl.bits(wl.cast(rng.uniform(-1, 1, gates.shape).astype(np.float32), dtype))  # |silu(g) u| <= |g|: no row overflows
    h_bits = np.ascontiguousarray(np.concatenate([gates, ups], axis=1))
    h = torch.from_numpy(h_bits.view(np.int16)).view(TORCH_16[dtype])
    q, s = qk.silu_mul_quant_per_token(h.to(DEV))
    q_ref, s_ref = oracle.silu_mul_quantize(h_bits, DTYPE_CODE[dtype])
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32)), dtype
    assert np.array_equal(q.cpu().numpy(), q_ref), dtype


def test_silu_f32_gates():
    rng = np.random.default_rng(3)
    g = np.concatenate([
        rng.uniform(-120, 120, 200000),
        rng.standard_normal(200000) * 4,
        np.ldexp(rng.uniform(0.5, 1, 20000), rng.integers(-149, 128, 20000)) *
        rng.choice([-1, 1], 20000),
        np.float32([0.0, -0.0, np.inf, -np.inf, np.nan, 88.0, -88.0, 87.0, -87.0,
                    np.nextafter(np.float32(88), np.float32(0)), np.nextafter(np.float32(-88), np.float32(0)),
                    np.nextafter(np.float32(88), np.float32(100)), np.nextafter(np.float32(-88), np.float32(-100)),
                    1e-45, -1e-45, 3.4e38, -3.4e38, 1.0, -1.0]),
    ]).astype(np.float32)
    g = np.resize(g, (g.size + 63) // 64 * 64)
    u = rng.standard_normal(g.size).astype(np.float32)
    h = np.concatenate([g.reshape(-1, 64), u.reshape(-1, 64)], axis=1)
    _run(h, "f32", "f32 gates")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("m,d", [(1, 1), (3, 7), (5, 4099)])
def test_silu_ragged_shapes(dtype, m, d):
    rng = np.random.default_rng(m * 1000 + d)
    h = wl.random_activations(rng, m, 2 * d, dtype)
    _run(wl.bits(h), dtype, f"{dtype} {m}x{d}")


def test_silu_empty():
    h = torch.empty((0, 8), dtype=torch.bfloat16, device=DEV)
    assert qk.silu_mul(h).shape == (0, 4)
    h = torch.empty((3, 0), dtype=torch.bfloat16, device=DEV)
    assert qk.silu_mul(h).shape == (3, 0)
