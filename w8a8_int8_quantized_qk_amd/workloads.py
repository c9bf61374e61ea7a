"""Seeded synthetic inputs for the W8A8 INT8 linear layer.

This module only draws random numbers and casts them to the input dtypes; it
holds none of the layer's arithmetic.  The same arrays feed the GPU library
and the CPU oracle.

Named workloads (all row-major; the weight is [K, N] with N contiguous):

  tiny_fp32         X fp32 [16, 256], W [256, 128], fp32 out
  decode_m1         X bf16 [1, 4096], W [4096, 14336], bf16 out
  decode_m8         X bf16 [8, 4096], W [4096, 14336], bf16 out
  prefill_outliers  X bf16 [2048, 4096] with 41 fixed columns (1% of K) x50,
                    W [4096, 4096], bf16 out
  mlp_up            X bf16 [8192, 8192], W [8192, 28672], fp32 out
  gated_down        H bf16 [4096, 2 x 14336] (gate | up), W [14336, 4096],
                    bf16 out

Recipe (numpy ``default_rng(seed)``, draws in this order): X ~ N(0, 1) as
float32; for the outlier workload, the column set (drawn without replacement)
is multiplied by 50 in float32; X is cast to bf16/fp16 by round-to-nearest-
even (torch); W is uniform on the integers [-127, 127]; the per-channel
scales are uniform on [1e-3, 1e-2] in float32.  The gated workload draws H in
place of X.  For the FP8 layer the weight is drawn instead as N(0, 1) x 100,
clipped to +-448 and cast to float8_e4m3fn by torch; per-group weight scales
are uniform on [1e-3, 1e-2] like the per-channel ones.  The MoE workload
(generate_moe: 8 experts, 2048 tokens routed to 2 each, 4096 -> 14336) draws
its per-expert row counts as multinomial(4096, Dirichlet(2)).  These shapes and
distributions follow the workloads the pages describe (decode GEMV vs prefill
GEMM, outlier channels, fused gated MLP).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

_TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclass(frozen=True)
class Workload:
    name: str
    m: int
    k: int            # reduction length of the GEMM (d for the gated workload)
    n: int
    x_dtype: str      # "f32" | "bf16" | "f16"
    out_dtype: str    # "f32" | "bf16"
    gated: bool = False
    outlier_cols: int = 0
    outlier_mult: float = 50.0

    @property
    def ops(self) -> int:
        return 2 * self.m * self.n * self.k


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32", 16, 256, 128, "f32", "f32"),
        Workload("decode_m1", 1, 4096, 14336, "bf16", "bf16"),
        Workload("decode_m8", 8, 4096, 14336, "bf16", "bf16"),
        Workload("prefill_outliers", 2048, 4096, 4096, "bf16", "bf16", outlier_cols=41),
        Workload("mlp_up", 8192, 8192, 28672, "bf16", "f32"),
        Workload("gated_down", 4096, 14336, 4096, "bf16", "bf16", gated=True),
    ]
}


def cast(x32: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 numpy -> CPU torch tensor of `dtype` (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(_TORCH_DTYPES[dtype]).contiguous()


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a CPU tensor as numpy: float32 as is, 16-bit types as uint16."""
    t = t.contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    raise TypeError(f"unsupported dtype {t.dtype}")


def random_activations(rng: np.random.Generator, m: int, k: int, dtype: str,
                       outlier_cols: int = 0, outlier_mult: float = 50.0) -> torch.Tensor:
    x = rng.standard_normal((m, k), dtype=np.float32)
    if outlier_cols:
        idx = rng.choice(k, outlier_cols, replace=False)
        x[:, idx] *= np.float32(outlier_mult)
    return cast(x, dtype)


def random_weight(rng: np.random.Generator, k: int, n: int) -> np.ndarray:
    return rng.integers(-127, 128, size=(k, n), dtype=np.int8)


def random_weight_fp8(rng: np.random.Generator, k: int, n: int) -> np.ndarray:
    """float8_e4m3fn weight codes [k, n] as uint8: N(0, 1) draws times 100 in
    float32, clipped to +-448 and cast by torch (round to nearest even)."""
    w = rng.standard_normal((k, n), dtype=np.float32) * np.float32(100.0)
    t = torch.from_numpy(np.clip(w, -448.0, 448.0)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def random_channel_scales(rng: np.random.Generator, n: int) -> np.ndarray:
    return rng.uniform(1e-3, 1e-2, n).astype(np.float32)


def random_group_scales(rng: np.random.Generator, groups: int, n: int) -> np.ndarray:
    """Per-group weight scales [groups, n], uniform on [1e-3, 1e-2] in float32."""
    return rng.uniform(1e-3, 1e-2, (groups, n)).astype(np.float32)


def moe_offsets(rng: np.random.Generator, rows: int, experts: int, alpha: float = 2.0) -> np.ndarray:
    """Synthetic routing: row counts per expert ~ multinomial(rows, p) with
    p ~ Dirichlet(alpha) (uneven, some experts busier than others), returned
    as offsets [experts + 1] (int32, prefix sums from 0 to rows)."""
    p = rng.dirichlet(np.full(experts, alpha))
    counts = rng.multinomial(rows, p)
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def generate_moe(seed: int = 0, experts: int = 8, tokens: int = 2048, top_k: int = 2,
                 k: int = 4096, n: int = 14336) -> dict:
    """The MoE up-projection workload: tokens x top_k routed rows, grouped by
    expert, of bf16 activations [rows, k]; int8 weights [experts, k, n];
    per-channel scales [experts, n]; offsets [experts + 1]."""
    rng = np.random.default_rng(seed)
    rows = tokens * top_k
    offsets = moe_offsets(rng, rows, experts)
    x = random_activations(rng, rows, k, "bf16")
    w = rng.integers(-127, 128, size=(experts, k, n), dtype=np.int8)
    s_ch = rng.uniform(1e-3, 1e-2, (experts, n)).astype(np.float32)
    return {"x": x, "w": w, "s_ch": s_ch, "offsets": offsets, "experts": experts, "rows": rows,
            "k": k, "n": n}


def generate(name_or_workload, seed: int = 0, weight: str = "i8") -> dict:
    """Inputs of a named workload: {'x' or 'h': torch CPU, 'w': [K,N], 's_ch': f32 [N]}.

    weight "i8" draws int8 codes, "fp8" float8_e4m3fn codes (uint8 bytes); the
    activations are the same either way."""
    wl = WORKLOADS[name_or_workload] if isinstance(name_or_workload, str) else name_or_workload
    rng = np.random.default_rng(seed)
    out = {"workload": wl}
    if wl.gated:
        out["h"] = random_activations(rng, wl.m, 2 * wl.k, wl.x_dtype)
    else:
        out["x"] = random_activations(rng, wl.m, wl.k, wl.x_dtype, wl.outlier_cols,
                                      wl.outlier_mult)
    if weight == "fp8":
        out["w"] = random_weight_fp8(rng, wl.k, wl.n)
    elif weight == "i8":
        out["w"] = random_weight(rng, wl.k, wl.n)
    else:
        raise ValueError(f"weight must be 'i8' or 'fp8', got {weight!r}")
    out["s_ch"] = random_channel_scales(rng, wl.n)
    return out


def edge_rows(k: int, dtype: str) -> torch.Tensor:
    """Rows with the degenerate structures the method has, as a [R, k] tensor.

    all zeros; one nonzero element; every element equal (ties for the max);
    alternating signs of one magnitude; tiny magnitudes (binary32 subnormals
    for fp32 input, smallest normals otherwise); the largest finite value of
    the dtype; a ramp through zero; and a row whose max sits in the last column.
    """
    big = {"f32": 3.0e38, "bf16": 3.0e38, "f16": 65504.0}[dtype]
    tiny = {"f32": 1.0e-40, "bf16": 1.2e-38, "f16": 6.2e-5}[dtype]
    rows = []
    rows.append(np.zeros(k, np.float32))
    r = np.zeros(k, np.float32)
    r[k // 3] = -3.25
    rows.append(r)
    rows.append(np.full(k, 0.75, np.float32))
    rows.append(np.where(np.arange(k) % 2 == 0, 1.5, -1.5).astype(np.float32))
    rows.append(np.full(k, tiny, np.float32) * np.where(np.arange(k) % 3 == 0, -1, 1))
    r = np.linspace(-1, 1, k, dtype=np.float32)
    r[0] = big
    rows.append(r)
    rows.append(np.linspace(-2.0, 2.0, k, dtype=np.float32))
    r = np.linspace(0, 1, k, dtype=np.float32)
    r[-1] = -7.0
    rows.append(r)
    return cast(np.stack(rows), dtype)
