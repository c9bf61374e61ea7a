"""The no-allocation whole-layer entry point (qk_linear_w8a8_noalloc, for
callers that cannot allocate device memory) against qk_linear_w8a8.

Both calls go through the C ABI.  The no-allocation call uses the library's
static per-GPU scratch in place of a caller's workspace; its codes, scales,
INT32 accumulators and outputs must equal those of qk_linear_w8a8 bit for bit
(the same kernels run), on two calls in a row on one stream, the second with
a smaller input, for the decode launch (scratch holds the split-K words) and
for quantization + tiled GEMM with split-K (scratch holds the partial sums).
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
import w8a8_int8_quantized_qk_amd as qk
from tests.gpu_compare import assert_equal_exact, host
from w8a8_int8_quantized_qk_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qk.library()


def _p(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def _buffers(m, k, n):
    return {"out": torch.empty((m, n), dtype=torch.bfloat16, device=DEV),
            "q": torch.empty((m, k), dtype=torch.int8, device=DEV),
            "s": torch.empty((m,), dtype=torch.float32, device=DEV),
            "c": torch.empty((m, n), dtype=torch.int32, device=DEV)}


def _call(noalloc, x, w, s_ch, b, kernel, ws=None):
    lib = qk.library()
    m, k = x.shape
    n = w.shape[1]
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    args = (m, n, k, _p(x), qk.BF16, _p(w), _p(s_ch), 1.0, _p(b["out"]), qk.BF16, qk.B_KN,
            _p(b["q"]), _p(b["s"]), _p(b["c"]))
    if noalloc:
        return lib.qk_linear_w8a8_noalloc(*args, kernel, stream)
    nbytes = ws.numel() if ws is not None else 0
    return lib.qk_linear_w8a8(*args, _p(ws), ctypes.c_size_t(nbytes), kernel, stream)


# (m, k, n) of two calls in a row, the second smaller
CASES = {
    "decode": [(8, 4096, 14336), (1, 1024, 1000)],
    "tiled_split_k": [(2048, 4096, 512), (300, 2048, 256)],
}


@pytest.mark.parametrize("path", sorted(CASES))
def test_noalloc_matches_linear_entry_point(path):
    rng = np.random.default_rng(20 if path == "decode" else 21)
    kernel = qk.KERNEL_GEMV if path == "decode" else qk.KERNEL_MFMA
    for i, (m, k, n) in enumerate(CASES[path]):
        if path == "tiled_split_k":
            # the tiled GEMM splits k in the scratch at these shapes
            need = qk.gemm_workspace_size(m, n, k)
            assert 0 < need <= qk.SCRATCH_BYTES, (m, k, n, need)
        x = wl.random_activations(rng, m, k, "bf16", outlier_cols=max(1, k // 100)).to(DEV)
        w = torch.from_numpy(wl.random_weight(rng, k, n)).to(DEV)
        s_ch = torch.from_numpy(wl.random_channel_scales(rng, n)).to(DEV)
        got, want = _buffers(m, k, n), _buffers(m, k, n)
        assert _call(True, x, w, s_ch, got, kernel) == qk.QK_OK
        ws = qk.new_workspace(qk.gemm_workspace_size(m, n, k), DEV)
        assert _call(False, x, w, s_ch, want, kernel, ws) == qk.QK_OK
        torch.cuda.synchronize()
        what = f"{path} call {i + 1} ({m}x{k}x{n})"
        assert torch.equal(got["q"], want["q"]), what
        assert torch.equal(got["s"].view(torch.int32), want["s"].view(torch.int32)), what
        assert torch.equal(got["c"], want["c"]), what
        assert torch.equal(got["out"].view(torch.int16), want["out"].view(torch.int16)), what
        if i == 1:  # the smaller call's accumulators against the oracle too
            q_ref, s_ref, c_ref, _ = oracle.linear(wl.bits(x.cpu()), oracle.BF16, host(w), host(s_ch))
            assert_equal_exact(host(got["c"]), c_ref, what)
