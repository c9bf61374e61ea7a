"""CPU oracle for the symmetric W8A8 INT8 linear layer (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never loads it and
shares no code with it.  The arithmetic lives in ``qk_oracle.c`` (plain C
loops, one step per statement); this module only marshals numpy arrays into
it and offers the composite ``linear`` that chains the steps in the order the
pages state them:

  per-token quantization  -- "kernels: fused silu_and_mul + dynamic per-token
                             FP8 quantization", Algorithm (absmax, guarded
                             scale) with the symmetric [-127, 127] range of
                             "Skill: Write an INT8 Quantized Kernel", Inputs.
  INT8 GEMM, INT32 acc    -- "16. Deploying Custom Kernels", C++ Kernel
                             Interface (GemmConfig), and "KV-cache kernels",
                             02 Scales and dequantization.
  dequant epilogue        -- the same two passages: acc * scale_a * scale_b.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qk_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, BF16, F16 = 0, 1, 2
B_KN, B_NK = 0, 1

_CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile qk_oracle.c into liboracle.so with gcc (no GPU toolchain)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.or_widen.argtypes = [ctypes.c_int, I64, P, P]
    lib.or_widen.restype = ctypes.c_int
    lib.or_quant_rows.argtypes = [I64, I64, P, P, P]
    lib.or_quant_rows.restype = None
    lib.or_spec_expf.argtypes = [ctypes.c_float]
    lib.or_spec_expf.restype = ctypes.c_float
    lib.or_expf_array.argtypes = [I64, P, P]
    lib.or_expf_array.restype = None
    lib.or_spec_taylor.argtypes = [P]
    lib.or_spec_reduction_constants.argtypes = [P]
    lib.or_silu_mul.argtypes = [I64, I64, P, P]
    lib.or_silu_mul.restype = None
    lib.or_gemm_i32.argtypes = [I64, I64, I64, P, P, ctypes.c_int, P]
    lib.or_gemm_i32.restype = I64
    lib.or_gemm_entries.argtypes = [I64, P, P, I64, I64, P, P, ctypes.c_int, P]
    lib.or_gemm_entries.restype = I64
    lib.or_dequant.argtypes = [I64, I64, P, P, P, ctypes.c_float, P]
    lib.or_dequant.restype = None
    lib.or_dequant_entries.argtypes = [I64, P, P, P, ctypes.c_float, P]
    lib.or_dequant_entries.restype = None
    lib.or_bf16_nearest.argtypes = [I64, P, P]
    lib.or_bf16_nearest.restype = None
    lib.or_fp8_encode_array.argtypes = [I64, P, P]
    lib.or_fp8_encode_array.restype = None
    lib.or_fp8_decode_array.argtypes = [I64, P, P]
    lib.or_fp8_decode_array.restype = None
    lib.or_quant_rows_fp8.argtypes = [I64, I64, P, ctypes.c_float, P, P]
    lib.or_quant_rows_fp8.restype = None
    lib.or_gemm_fp8.argtypes = [I64, I64, I64, P, P, ctypes.c_int, P]
    lib.or_gemm_fp8.restype = None
    lib.or_gemm_i8_grouped.argtypes = [I64, I64, I64, I64, P, P, ctypes.c_int, P, P]
    lib.or_gemm_i8_grouped.restype = None
    lib.or_dequant_grouped.argtypes = [I64, I64, P, P, ctypes.c_float, P]
    lib.or_dequant_grouped.restype = None
    lib.or_quant_static.argtypes = [I64, P, ctypes.c_float, P]
    lib.or_quant_static.restype = None
    lib.or_quant_static_fp8.argtypes = [I64, P, ctypes.c_float, P]
    lib.or_quant_static_fp8.restype = None
    lib.or_quant_rows_asym.argtypes = [I64, I64, P, P, P, P]
    lib.or_quant_rows_asym.restype = None
    lib.or_gemm_asym.argtypes = [I64, I64, I64, P, P, P, ctypes.c_int, P]
    lib.or_gemm_asym.restype = I64
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _contig(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------------
# step wrappers
# --------------------------------------------------------------------------

def widen(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Widen fp32 / bf16 bits / fp16 bits to binary32 (exact)."""
    lib = _load()
    if dtype == F32:
        src = _contig(bits, np.float32)
    else:
        src = _contig(bits.view(np.uint16) if bits.dtype != np.uint16 else bits, np.uint16)
    out = np.empty(src.shape, dtype=np.float32)
    rc = lib.or_widen(dtype, src.size, _ptr(src), _ptr(out))
    if rc:
        raise ValueError("unknown dtype")
    return out


def quant_per_token(x32: np.ndarray):
    """x32: [m, k] float32 -> (codes int8 [m, k], scale float32 [m])."""
    lib = _load()
    x = _contig(x32, np.float32)
    m, k = x.shape
    q = np.empty((m, k), dtype=np.int8)
    s = np.empty((m,), dtype=np.float32)
    lib.or_quant_rows(m, k, _ptr(x), _ptr(q), _ptr(s))
    return q, s


def spec_expf(x: np.ndarray) -> np.ndarray:
    lib = _load()
    xs = _contig(x, np.float32)
    y = np.empty_like(xs)
    lib.or_expf_array(xs.size, _ptr(xs), _ptr(y))
    return y


def spec_taylor() -> np.ndarray:
    out = np.empty(8, dtype=np.float32)
    _load().or_spec_taylor(_ptr(out))
    return out


def spec_reduction_constants() -> np.ndarray:
    out = np.empty(3, dtype=np.float32)
    _load().or_spec_reduction_constants(_ptr(out))
    return out


def silu_mul(h32: np.ndarray) -> np.ndarray:
    """h32: [m, 2d] float32 (gate | up) -> silu(gate) * up, float32 [m, d]."""
    lib = _load()
    h = _contig(h32, np.float32)
    m, two_d = h.shape
    if two_d % 2:
        raise ValueError("last dimension of h must be even")
    d = two_d // 2
    out = np.empty((m, d), dtype=np.float32)
    lib.or_silu_mul(m, d, _ptr(h), _ptr(out))
    return out


def gemm_i32(a: np.ndarray, b: np.ndarray, layout: int = B_KN) -> np.ndarray:
    """Exact int32 accumulators of a [m,k] x b ([k,n] if B_KN, [n,k] if B_NK)."""
    lib = _load()
    a = _contig(a, np.int8)
    b = _contig(b, np.int8)
    m, k = a.shape
    n = b.shape[1] if layout == B_KN else b.shape[0]
    kb = b.shape[0] if layout == B_KN else b.shape[1]
    if kb != k:
        raise ValueError("inner dimensions differ")
    c = np.empty((m, n), dtype=np.int32)
    ovf = lib.or_gemm_i32(m, n, k, _ptr(a), _ptr(b), layout, _ptr(c))
    if ovf:
        raise OverflowError(f"{ovf} accumulators exceed int32")
    return c


def gemm_entries(a: np.ndarray, b: np.ndarray, rows, cols, layout: int = B_KN) -> np.ndarray:
    """Exact int32 accumulators at the listed (row, col) pairs."""
    lib = _load()
    a = _contig(a, np.int8)
    b = _contig(b, np.int8)
    rows = _contig(rows, np.int64)
    cols = _contig(cols, np.int64)
    k = a.shape[1]
    n = b.shape[1] if layout == B_KN else b.shape[0]
    c = np.empty(rows.shape, dtype=np.int32)
    ovf = lib.or_gemm_entries(rows.size, _ptr(rows), _ptr(cols), n, k, _ptr(a), _ptr(b),
                              layout, _ptr(c))
    if ovf:
        raise OverflowError(f"{ovf} accumulators exceed int32")
    return c


def dequant(c: np.ndarray, scale_a: np.ndarray, scale_b: np.ndarray,
            output_scale: float = 1.0) -> np.ndarray:
    """acc * scale_a[row] * scale_b[col] * output_scale in float64."""
    lib = _load()
    c = _contig(c, np.int32)
    sa = _contig(scale_a, np.float32)
    sb = _contig(scale_b, np.float32)
    m, n = c.shape
    out = np.empty((m, n), dtype=np.float64)
    lib.or_dequant(m, n, _ptr(c), _ptr(sa), _ptr(sb), float(output_scale), _ptr(out))
    return out


def dequant_entries(c: np.ndarray, scale_a: np.ndarray, scale_b: np.ndarray,
                    output_scale: float = 1.0) -> np.ndarray:
    """Per-entry acc[e] * scale_a[e] * scale_b[e] * output_scale in float64."""
    lib = _load()
    c = _contig(c, np.int32).ravel()
    sa = _contig(scale_a, np.float32).ravel()
    sb = _contig(scale_b, np.float32).ravel()
    if not (c.size == sa.size == sb.size):
        raise ValueError("entry arrays differ in length")
    out = np.empty(c.shape, dtype=np.float64)
    lib.or_dequant_entries(c.size, _ptr(c), _ptr(sa), _ptr(sb), float(output_scale), _ptr(out))
    return out


def bf16_nearest(v: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns nearest to the float64 values (ties to even)."""
    lib = _load()
    v = _contig(v, np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib.or_bf16_nearest(v.size, _ptr(v), _ptr(out))
    return out


# --------------------------------------------------------------------------
# composites (the layer, step by step)
# --------------------------------------------------------------------------

def quantize_input(x_bits: np.ndarray, dtype: int):
    """Widen then quantize per token: returns (codes, scales)."""
    return quant_per_token(widen(x_bits, dtype))


def silu_mul_quantize(h_bits: np.ndarray, dtype: int):
    """silu(gate) * up, then per-token quantization: returns (codes, scales)."""
    return quant_per_token(silu_mul(widen(h_bits, dtype)))


def linear(x_bits: np.ndarray, dtype: int, w: np.ndarray, scale_b: np.ndarray,
           layout: int = B_KN, output_scale: float = 1.0):
    """Whole layer: returns (codes, scales, acc int32, out float64)."""
    q, s = quantize_input(x_bits, dtype)
    c = gemm_i32(q, w, layout)
    return q, s, c, dequant(c, s, scale_b, output_scale)


# --------------------------------------------------------------------------
# FP8 path: float8_e4m3fn per-token quantization and the FP8 GEMM
# --------------------------------------------------------------------------

FP8_MAX = 448.0


def fp8_encode(v: np.ndarray) -> np.ndarray:
    """binary32 -> e4m3fn codes (round to nearest even, saturating at +-448)."""
    lib = _load()
    x = _contig(v, np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib.or_fp8_encode_array(x.size, _ptr(x), _ptr(out))
    return out


def fp8_decode(c: np.ndarray) -> np.ndarray:
    """e4m3fn codes -> their exact values (float64; NaN for S.1111.111)."""
    lib = _load()
    cc = _contig(c, np.uint8)
    out = np.empty(cc.shape, dtype=np.float64)
    lib.or_fp8_decode_array(cc.size, _ptr(cc), _ptr(out))
    return out


def quant_per_token_fp8(x32: np.ndarray, scale_ub: float = 0.0):
    """x32: [m, k] float32 -> (e4m3fn codes uint8 [m, k], scale float32 [m]).
    scale_ub > 0 clamps the scales from above."""
    lib = _load()
    x = _contig(x32, np.float32)
    m, k = x.shape
    q = np.empty((m, k), dtype=np.uint8)
    s = np.empty((m,), dtype=np.float32)
    lib.or_quant_rows_fp8(m, k, _ptr(x), float(scale_ub), _ptr(q), _ptr(s))
    return q, s


def gemm_fp8(a: np.ndarray, b: np.ndarray, layout: int = B_KN) -> np.ndarray:
    """Exact sums of products of e4m3fn values (float64 [m, n])."""
    lib = _load()
    aa = _contig(a, np.uint8)
    bb = _contig(b, np.uint8)
    m, k = aa.shape
    n = bb.shape[1] if layout == B_KN else bb.shape[0]
    acc = np.empty((m, n), dtype=np.float64)
    lib.or_gemm_fp8(m, n, k, _ptr(aa), _ptr(bb), layout, _ptr(acc))
    return acc


def dequant_fp8(acc: np.ndarray, scale_a: np.ndarray, scale_b: np.ndarray,
                output_scale: float = 1.0) -> np.ndarray:
    """acc * scale_a[row] * scale_b[col] * output_scale in float64."""
    return (acc * scale_a.astype(np.float64)[:, None] * scale_b.astype(np.float64)[None, :]
            * float(np.float32(output_scale)))


def quantize_input_fp8(x_bits: np.ndarray, dtype: int, scale_ub: float = 0.0):
    """Widen then quantize per token to e4m3fn: returns (codes, scales)."""
    return quant_per_token_fp8(widen(x_bits, dtype), scale_ub)


def silu_mul_quantize_fp8(h_bits: np.ndarray, dtype: int, scale_ub: float = 0.0):
    """silu(gate) * up, then per-token e4m3fn quantization: (codes, scales)."""
    return quant_per_token_fp8(silu_mul(widen(h_bits, dtype)), scale_ub)


# --------------------------------------------------------------------------
# Per-group weight scales: "KV-cache kernels", 02 Scales and dequantization
# and 03 Where scales come from (one scale per group of 64-128 channels),
# with the groups along the reduction dimension k.
# --------------------------------------------------------------------------

def gemm_i8_grouped(a: np.ndarray, b: np.ndarray, scale_b: np.ndarray, group: int,
                    layout: int = B_KN) -> np.ndarray:
    """sum over k-groups g of scale_b[g, col] * (exact integer partial of group g),
    float64 [m, n]; scale_b is [ceil(k / group), n] float32."""
    lib = _load()
    aa = _contig(a, np.int8)
    bb = _contig(b, np.int8)
    m, k = aa.shape
    n = bb.shape[1] if layout == B_KN else bb.shape[0]
    sb = _contig(scale_b, np.float32)
    if group < 1 or sb.shape != ((k + group - 1) // group, n):
        raise ValueError("scale_b must be [ceil(k / group), n]")
    acc = np.empty((m, n), dtype=np.float64)
    lib.or_gemm_i8_grouped(m, n, k, group, _ptr(aa), _ptr(bb), layout, _ptr(sb), _ptr(acc))
    return acc


def dequant_grouped(acc: np.ndarray, scale_a: np.ndarray, output_scale: float = 1.0) -> np.ndarray:
    """acc * scale_a[row] * output_scale in float64."""
    lib = _load()
    ac = _contig(acc, np.float64)
    sa = _contig(scale_a, np.float32)
    m, n = ac.shape
    out = np.empty((m, n), dtype=np.float64)
    lib.or_dequant_grouped(m, n, _ptr(ac), _ptr(sa), float(output_scale), _ptr(out))
    return out


# --------------------------------------------------------------------------
# MoE grouped GEMM ("dynquant-kernels", What is in here: one launch for all
# experts): the rows of a are grouped by expert, rows [offsets[e],
# offsets[e + 1]) going to expert e's weight and per-channel scales.  The
# oracle is the per-expert GEMM of this module applied expert by expert.
# --------------------------------------------------------------------------

def _check_offsets(offsets: np.ndarray, experts: int, m_total: int) -> np.ndarray:
    off = np.asarray(offsets, dtype=np.int64)
    if off.shape != (experts + 1,) or off[0] != 0 or off[-1] != m_total or np.any(np.diff(off) < 0):
        raise ValueError("offsets must be [experts + 1], nondecreasing, from 0 to the row count")
    return off


def moe_gemm_i32(a: np.ndarray, w: np.ndarray, offsets: np.ndarray, layout: int = B_KN) -> np.ndarray:
    """Exact int32 accumulators: rows of expert e times w[e] ([k, n] if B_KN, [n, k] if B_NK)."""
    experts = w.shape[0]
    off = _check_offsets(offsets, experts, a.shape[0])
    n = w.shape[2] if layout == B_KN else w.shape[1]
    c = np.zeros((a.shape[0], n), dtype=np.int32)
    for e in range(experts):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 > r0:
            c[r0:r1] = gemm_i32(a[r0:r1], w[e], layout)
    return c


def moe_dequant(c: np.ndarray, scale_a: np.ndarray, scale_b: np.ndarray, offsets: np.ndarray,
                output_scale: float = 1.0) -> np.ndarray:
    """acc * scale_a[row] * scale_b[expert of row, col] * output_scale in float64."""
    experts = scale_b.shape[0]
    off = _check_offsets(offsets, experts, c.shape[0])
    out = np.zeros(c.shape, dtype=np.float64)
    for e in range(experts):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 > r0:
            out[r0:r1] = dequant(c[r0:r1], scale_a[r0:r1], scale_b[e], output_scale)
    return out


# --------------------------------------------------------------------------
# Static per-tensor scale ("kernels: fused silu_and_mul + dynamic per-token
# FP8 quantization", Purpose: silu_and_mul_quant takes one pre-calibrated
# scale) and asymmetric per-token quantization ("Skill: Write an INT8
# Quantized Kernel", Inputs: a nonzero zero point instead of the symmetric
# range).
# --------------------------------------------------------------------------

def quant_static(x32: np.ndarray, scale: float) -> np.ndarray:
    """clamp(rint(x / scale), -127, 127) with one binary32 scale."""
    lib = _load()
    x = _contig(x32, np.float32)
    q = np.empty(x.shape, dtype=np.int8)
    lib.or_quant_static(x.size, _ptr(x), float(np.float32(scale)), _ptr(q))
    return q


def quant_static_fp8(x32: np.ndarray, scale: float) -> np.ndarray:
    """e4m3fn(x / scale) with one binary32 scale."""
    lib = _load()
    x = _contig(x32, np.float32)
    q = np.empty(x.shape, dtype=np.uint8)
    lib.or_quant_static_fp8(x.size, _ptr(x), float(np.float32(scale)), _ptr(q))
    return q


def quant_per_token_asym(x32: np.ndarray):
    """x32 [m, k] -> (codes int8 [m, k], scales float32 [m], zero points int32 [m])."""
    lib = _load()
    x = _contig(x32, np.float32)
    m, k = x.shape
    q = np.empty((m, k), dtype=np.int8)
    s = np.empty(m, dtype=np.float32)
    z = np.empty(m, dtype=np.int32)
    lib.or_quant_rows_asym(m, k, _ptr(x), _ptr(q), _ptr(s), _ptr(z))
    return q, s, z


def gemm_asym(a: np.ndarray, zp: np.ndarray, b: np.ndarray, layout: int = B_KN) -> np.ndarray:
    """Exact int32 sums of (a[i, t] - zp[i]) * B(t, j)."""
    lib = _load()
    aa = _contig(a, np.int8)
    bb = _contig(b, np.int8)
    z = _contig(zp, np.int32)
    m, k = aa.shape
    n = bb.shape[1] if layout == B_KN else bb.shape[0]
    c = np.empty((m, n), dtype=np.int32)
    ovf = lib.or_gemm_asym(m, n, k, _ptr(aa), _ptr(z), _ptr(bb), layout, _ptr(c))
    if ovf:
        raise OverflowError(f"{ovf} accumulators exceed int32")
    return c
