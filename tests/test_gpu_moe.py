"""GPU parity of the MoE grouped GEMM (all experts in one launch) against the
oracle's per-expert GEMM: INT32 accumulators bit-exact, fp32 outputs within
1e-6 relative, bf16 within one ulp.  Routing counts are synthetic (uneven,
with empty experts); nothing expected here comes from the GPU.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import w8a8_int8_quantized_qk_amd as qk
from tests.gpu_compare import assert_equal_exact, assert_out_close, host
from w8a8_int8_quantized_qk_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qk.library()


def _run(counts, k, n, layout, seed, out_dtype="bf16", osc=1.0):
    rng = np.random.default_rng(seed)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    m, experts = int(off[-1]), len(counts)
    a = rng.integers(-127, 128, (m, k), dtype=np.int8)
    w_kn = rng.integers(-127, 128, (experts, k, n), dtype=np.int8)
    w = w_kn if layout == "kn" else np.ascontiguousarray(w_kn.transpose(0, 2, 1))
    sa = rng.uniform(1e-3, 1e-1, m).astype(np.float32)
    sb = rng.uniform(1e-3, 1e-2, (experts, n)).astype(np.float32)
    tdt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    out, c = qk.moe_gemm_i8_scaled(torch.from_numpy(a).to(DEV), torch.from_numpy(w).to(DEV),
                                   torch.from_numpy(off).to(DEV), torch.from_numpy(sa).to(DEV),
                                   torch.from_numpy(sb).to(DEV), osc, tdt, layout, return_acc=True)
    c_ref = oracle.moe_gemm_i32(a, w_kn, off)
    what = f"moe counts={list(counts)[:6]}... k={k} n={n} {layout}"
    assert_equal_exact(host(c), c_ref, what + " acc")
    assert_out_close(host(out), oracle.moe_dequant(c_ref, sa, sb, off, osc), out_dtype, what + " out")


@pytest.mark.parametrize("counts,k,n,layout", [
    ([0, 300, 1, 257], 256, 384, "kn"),         # empty and one-row experts, ragged tiles
    ([37], 128, 128, "kn"),                       # one expert: the plain GEMM
    ([513, 0, 0, 7, 256, 255], 1040, 200, "kn"),  # K tail, register-staged weight (n % 16 != 0)
    ([64, 190, 3], 512, 130, "kn"),               # byte-staged weight (n % 4 != 0)
    ([100, 400, 29, 0, 1], 768, 512, "nk"),
    ([0, 0, 0, 600], 256, 256, "kn"),             # every row in the last expert
])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_moe_against_per_expert_oracle(counts, k, n, layout, out_dtype):
    _run(counts, k, n, layout, seed=len(counts) * 1000 + k + n, out_dtype=out_dtype, osc=0.5)


# groups whose dense GEMM of all rows has at least one 256 x 256 tile per CU
# take the 256 x 256 tile kernel: empty and one-row experts, ragged rows and
# columns, k tails past a 64-byte slice (k % 64 != 0), both layouts, all rows
# in one expert.  An expert's last row block of at most 128 rows is a light
# tile (rows 128 and 128 + 256 light, 129 full, at the boundary).
@pytest.mark.parametrize("counts,k,n,layout", [
    ([0, 1500, 1, 257, 2338], 256, 4096, "kn"),
    ([700, 0, 1300, 2100], 208, 4112, "nk"),
    ([4096], 128, 4096, "kn"),
    ([1000, 999, 1001, 1096], 320, 4096, "nk"),
    ([128, 384, 129, 3455], 192, 4096, "kn"),
    ([128, 384, 129, 3455], 208, 4096, "nk"),
    # many experts, light and full last blocks, empty ones, 17 column tiles
    # (full and light tile counts not multiples of 8: uneven XCD shares)
    ([0, 129, 128, 1, 300, 0, 640, 385, 127, 2000, 33, 0, 77, 256, 255, 257], 192, 4112, "kn"),
    ([0, 129, 128, 1, 300, 0, 640, 385, 127, 2000, 33, 0, 77, 256, 255, 257], 128, 4112, "nk"),
])
def test_moe_wide_tiles_against_per_expert_oracle(counts, k, n, layout):
    m = sum(counts)
    assert (m // 256) * ((n + 255) // 256) >= 256  # the shape selects the 256 x 256 tiles
    _run(counts, k, n, layout, seed=len(counts) * 1000 + k + n + 7, out_dtype="bf16", osc=0.75)


def test_moe_maximum_expert_count():
    rng = np.random.default_rng(7)
    counts = rng.integers(0, 5, qk.MOE_MAX_EXPERTS)
    counts[::17] = 0
    _run(counts.tolist(), 128, 128, "kn", seed=8)


def test_moe_many_tiles_per_expert():
    rng = np.random.default_rng(9)
    off = wl.moe_offsets(rng, 2048, 8)
    _run(np.diff(off).tolist(), 1024, 1024, "kn", seed=10)


def test_moe_full_workload_every_entry():
    # the MoE up-projection workload at its full size, in the launch
    # configuration bench.py times: codes and scales, then every INT32
    # accumulator and every output element, expert by expert
    d = wl.generate_moe()
    x, w, s_ch, off = d["x"], d["w"], d["s_ch"], d["offsets"]
    q, s = qk.quant_per_token(x.to(DEV))
    out, c = qk.moe_gemm_i8_scaled(q, torch.from_numpy(w).to(DEV), torch.from_numpy(off).to(DEV),
                                   s, torch.from_numpy(s_ch).to(DEV), return_acc=True)
    q_ref, s_ref = oracle.quantize_input(wl.bits(x), oracle.BF16)
    assert_equal_exact(host(q), q_ref, "moe workload codes")
    assert_equal_exact(host(s), s_ref, "moe workload scales")
    c_host, out_host = host(c), host(out)
    for e in range(d["experts"]):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        c_ref = oracle.gemm_i32(q_ref[r0:r1], w[e])
        assert_equal_exact(c_host[r0:r1], c_ref, f"moe workload acc expert {e}")
        assert_out_close(out_host[r0:r1], oracle.dequant(c_ref, s_ref[r0:r1], s_ch[e]), "bf16",
                         f"moe workload out expert {e}")
