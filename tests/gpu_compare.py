"""Comparison rules of the GPU parity tests (test helper).

Bars: int8 codes, per-token scales and INT32 accumulators bit-exact; fp32
outputs within 1e-6 relative of the oracle's float64 value (zeros exact);
bf16 outputs within one bf16 ulp of the bf16 value nearest the oracle's.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

DTYPE_CODE = {"f32": oracle.F32, "bf16": oracle.BF16, "f16": oracle.F16}
TORCH_OUT = {"f32": torch.float32, "bf16": torch.bfloat16}
FP32_RTOL = 1e-6


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def assert_equal_exact(got: np.ndarray, want: np.ndarray, what: str):
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if got.dtype == np.float32:
        got = got.view(np.uint32)
        want = np.asarray(want, np.float32).view(np.uint32)
    diff = np.nonzero(got != want)
    if diff[0].size:
        idx = tuple(d[0] for d in diff)
        raise AssertionError(f"{what}: {diff[0].size} mismatches, first at {idx}: "
                             f"got {got[idx]} want {want[idx]}")


def _ordered_bf16(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def assert_out_close(got: np.ndarray, ref64: np.ndarray, out_dtype: str, what: str):
    """got: fp32 array or bf16 bits; ref64: the oracle's float64 values."""
    assert got.shape == ref64.shape, (what, got.shape, ref64.shape)
    if out_dtype == "f32":
        g = got.astype(np.float64)
        err = np.abs(g - ref64)
        bad = err > FP32_RTOL * np.abs(ref64)
        if bad.any():
            i = np.argmax(np.where(bad, err / np.maximum(np.abs(ref64), 1e-300), 0))
            idx = np.unravel_index(i, got.shape)
            raise AssertionError(f"{what}: {bad.sum()} fp32 outputs beyond rel {FP32_RTOL}; "
                                 f"worst at {idx}: got {g[idx]!r} want {ref64[idx]!r}")
    else:
        want = oracle.bf16_nearest(ref64)
        d = np.abs(_ordered_bf16(got) - _ordered_bf16(want))
        if (d > 1).any():
            idx = np.unravel_index(np.argmax(d), got.shape)
            raise AssertionError(f"{what}: {(d > 1).sum()} bf16 outputs beyond 1 ulp; worst at "
                                 f"{idx}: got {got[idx]:#06x} want {want[idx]:#06x}")
