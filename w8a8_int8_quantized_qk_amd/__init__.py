"""MI355X-native W8A8 INT8 linear layer: Python binding of libqk.

Every step runs in the HIP kernels of ``libqk.so`` (built for gfx950 by
``build.py``); this module only checks tensors, passes raw device pointers
and the current HIP stream through the C ABI of ``include/qk.h``, and raises
on a nonzero status.  PyTorch provides device memory and streams.  There is no
fallback: if the library is missing or was built for another ABI, every call
raises.

Layer (per-token dynamic INT8 activations, per-channel INT8 weights):
  q, s     = quant_per_token(x)                 # or silu_mul_quant_per_token(h)
  out      = gemm_i8_scaled(q, w, s, s_ch)       # INT32 accumulate + dequant
  out      = linear_w8a8(x, w, s_ch)             # both steps
and its FP8 (float8_e4m3fn) counterpart:
  q, s     = quant_per_token_fp8(x, scale_ub)   # or silu_mul_quant_per_token_fp8(h)
  out      = gemm_fp8_scaled(q, w8, s, s_ch)     # binary32 accumulate + dequant
  out      = linear_fp8(x, w8, s_ch)
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

ABI_VERSION = 7
F32, BF16, F16 = 0, 1, 2
B_KN, B_NK = 0, 1
KERNEL_AUTO, KERNEL_MFMA, KERNEL_GEMV = 0, 1, 2
QK_OK = 0
SCRATCH_BYTES = 16777216  # static scratch of qk_linear_w8a8_noalloc, per GPU

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqk.so")

_IN_DTYPES = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}
_OUT_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}
_LAYOUTS = {"kn": B_KN, "nk": B_NK}
_KERNELS = {"auto": KERNEL_AUTO, "mfma": KERNEL_MFMA, "gemv": KERNEL_GEMV}

EXPORTED = (
    "qk_abi_version", "qk_status_string", "qk_build_info", "qk_quant_per_token",
    "qk_silu_mul_quant_per_token", "qk_silu_mul", "qk_gemm_workspace_size", "qk_workspace_init",
    "qk_gemm_i8_scaled",
    "qk_gemm_i8_scaled_ex", "qk_linear_w8a8", "qk_linear_w8a8_noalloc", "qk_quant_per_token_fp8",
    "qk_silu_mul_quant_per_token_fp8", "qk_gemm_fp8_scaled", "qk_linear_fp8",
    "qk_gemm_i8_grouped", "qk_moe_gemm_i8_scaled", "qk_quant_static", "qk_silu_mul_quant_static",
    "qk_quant_static_fp8", "qk_silu_mul_quant_static_fp8", "qk_quant_per_token_asym",
    "qk_weight_colsum", "qk_gemm_i8_asym",
)


class QKError(RuntimeError):
    """A nonzero status from libqk."""

    def __init__(self, status: int, message: str):
        super().__init__(f"libqk status {status}: {message}")
        self.status = status


_lib = None
_lock = threading.Lock()


def _declare(lib):
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.qk_abi_version.argtypes = []
    lib.qk_abi_version.restype = I
    lib.qk_status_string.argtypes = [I]
    lib.qk_status_string.restype = ctypes.c_char_p
    lib.qk_build_info.argtypes = []
    lib.qk_build_info.restype = ctypes.c_char_p
    lib.qk_quant_per_token.argtypes = [I, I, P, I, P, P, P]
    lib.qk_quant_per_token.restype = I
    lib.qk_silu_mul_quant_per_token.argtypes = [I, I, P, I, P, P, P]
    lib.qk_silu_mul_quant_per_token.restype = I
    lib.qk_silu_mul.argtypes = [I, I, P, I, P, P]
    lib.qk_silu_mul.restype = I
    lib.qk_gemm_workspace_size.argtypes = [I, I, I]
    lib.qk_gemm_workspace_size.restype = ctypes.c_size_t
    lib.qk_workspace_init.argtypes = [P, ctypes.c_size_t, P]
    lib.qk_workspace_init.restype = I
    gemm = [I, I, I, P, P, P, P, P, F, P, I, I, P, ctypes.c_size_t]
    lib.qk_gemm_i8_scaled.argtypes = gemm + [P]
    lib.qk_gemm_i8_scaled.restype = I
    lib.qk_gemm_i8_scaled_ex.argtypes = gemm + [I, P]
    lib.qk_gemm_i8_scaled_ex.restype = I
    lib.qk_linear_w8a8.argtypes = [I, I, I, P, I, P, P, F, P, I, I, P, P, P, P, ctypes.c_size_t,
                                   I, P]
    lib.qk_linear_w8a8.restype = I
    lib.qk_linear_w8a8_noalloc.argtypes = [I, I, I, P, I, P, P, F, P, I, I, P, P, P, I, P]
    lib.qk_linear_w8a8_noalloc.restype = I
    lib.qk_quant_per_token_fp8.argtypes = [I, I, P, I, F, P, P, P]
    lib.qk_quant_per_token_fp8.restype = I
    lib.qk_silu_mul_quant_per_token_fp8.argtypes = [I, I, P, I, F, P, P, P]
    lib.qk_silu_mul_quant_per_token_fp8.restype = I
    lib.qk_gemm_fp8_scaled.argtypes = [I, I, I, P, P, P, P, P, F, P, I, I, P]
    lib.qk_gemm_fp8_scaled.restype = I
    lib.qk_linear_fp8.argtypes = [I, I, I, P, I, F, P, P, F, P, I, I, P, P, P]
    lib.qk_linear_fp8.restype = I
    lib.qk_gemm_i8_grouped.argtypes = [I, I, I, I, P, P, P, P, P, F, P, I, I, P]
    lib.qk_gemm_i8_grouped.restype = I
    lib.qk_moe_gemm_i8_scaled.argtypes = [I, I, I, I, P, P, P, P, P, P, F, P, I, I, P]
    lib.qk_moe_gemm_i8_scaled.restype = I
    for name in ("qk_quant_static", "qk_silu_mul_quant_static", "qk_quant_static_fp8",
                 "qk_silu_mul_quant_static_fp8"):
        getattr(lib, name).argtypes = [I, I, P, I, P, P, P]
        getattr(lib, name).restype = I
    lib.qk_quant_per_token_asym.argtypes = [I, I, P, I, P, P, P, P]
    lib.qk_quant_per_token_asym.restype = I
    lib.qk_weight_colsum.argtypes = [I, I, P, I, P, P]
    lib.qk_weight_colsum.restype = I
    lib.qk_gemm_i8_asym.argtypes = [I, I, I, P, P, P, P, P, P, P, F, P, I, I, P]
    lib.qk_gemm_i8_asym.restype = I


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libqk and check its ABI number; raises if absent or mismatched."""
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m w8a8_int8_quantized_qk_amd.build` "
            "(or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(path)
    for name in EXPORTED:
        if not hasattr(lib, name):
            raise ImportError(f"{path} does not export {name}")
    _declare(lib)
    got = lib.qk_abi_version()
    if got != ABI_VERSION:
        raise ImportError(
            f"{path} has ABI {got}, this binding expects ABI {ABI_VERSION}: rebuild the "
            "library from this source tree")
    return lib


def library() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                _lib = load_library()
    return _lib


def build_info() -> str:
    return library().qk_build_info().decode()


def status_string(status: int) -> str:
    return library().qk_status_string(status).decode()


def _check(status: int):
    if status != QK_OK:
        raise QKError(status, status_string(status))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, ndim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def quant_per_token(x: torch.Tensor, q: torch.Tensor | None = None,
                    scale: torch.Tensor | None = None):
    """Per-token INT8 codes and fp32 scales of x [m, k] (fp32, bf16 or fp16)."""
    _need(x, "x", ndim=2)
    if x.dtype not in _IN_DTYPES:
        raise TypeError(f"x dtype {x.dtype} not supported")
    m, k = x.shape
    q = torch.empty((m, k), dtype=torch.int8, device=x.device) if q is None else q
    scale = torch.empty((m,), dtype=torch.float32, device=x.device) if scale is None else scale
    _need(q, "q", torch.int8, 2, x.device)
    _need(scale, "scale", torch.float32, 1, x.device)
    if tuple(q.shape) != (m, k) or scale.shape[0] != m:
        raise ValueError("q must be [m, k] and scale [m]")
    _check(library().qk_quant_per_token(m, k, _ptr(x), _IN_DTYPES[x.dtype], _ptr(q),
                                        _ptr(scale), _stream(x.device)))
    return q, scale


def silu_mul_quant_per_token(h: torch.Tensor, q: torch.Tensor | None = None,
                             scale: torch.Tensor | None = None):
    """Codes and scales of silu(h[:, :d]) * h[:, d:] for h [m, 2d]."""
    _need(h, "h", ndim=2)
    if h.dtype not in _IN_DTYPES:
        raise TypeError(f"h dtype {h.dtype} not supported")
    m, two_d = h.shape
    if two_d % 2:
        raise ValueError("h must have an even number of columns (gate | up)")
    d = two_d // 2
    q = torch.empty((m, d), dtype=torch.int8, device=h.device) if q is None else q
    scale = torch.empty((m,), dtype=torch.float32, device=h.device) if scale is None else scale
    _need(q, "q", torch.int8, 2, h.device)
    _need(scale, "scale", torch.float32, 1, h.device)
    if tuple(q.shape) != (m, d) or scale.shape[0] != m:
        raise ValueError("q must be [m, d] and scale [m]")
    _check(library().qk_silu_mul_quant_per_token(m, d, _ptr(h), _IN_DTYPES[h.dtype], _ptr(q),
                                                 _ptr(scale), _stream(h.device)))
    return q, scale


def silu_mul(h: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """silu(h[:, :d]) * h[:, d:] in fp32 for h [m, 2d], unquantized (the same
    arithmetic as the fused quantization)."""
    _need(h, "h", ndim=2)
    if h.dtype not in _IN_DTYPES:
        raise TypeError(f"h dtype {h.dtype} not supported")
    m, two_d = h.shape
    if two_d % 2:
        raise ValueError("h must have an even number of columns (gate | up)")
    d = two_d // 2
    out = torch.empty((m, d), dtype=torch.float32, device=h.device) if out is None else out
    _need(out, "out", torch.float32, 2, h.device)
    if tuple(out.shape) != (m, d):
        raise ValueError("out must be [m, d]")
    _check(library().qk_silu_mul(m, d, _ptr(h), _IN_DTYPES[h.dtype], _ptr(out),
                                 _stream(h.device)))
    return out


def gemm_workspace_size(m: int, n: int, k: int) -> int:
    return int(library().qk_gemm_workspace_size(m, n, k))


_workspaces: dict = {}


def workspace_init(ws: torch.Tensor, stream=None):
    """Zero a workspace with libqk's own kernel (qk_workspace_init), on `stream`
    (default: the current stream of its device)."""
    _need(ws, "workspace")
    stream = torch.cuda.current_stream(ws.device) if stream is None else stream
    _check(library().qk_workspace_init(_ptr(ws), ws.numel() * ws.element_size(),
                                       ctypes.c_void_p(stream.cuda_stream)))
    return ws


def new_workspace(nbytes: int, device, stream=None) -> torch.Tensor | None:
    """A workspace of nbytes (256-byte aligned device memory from torch's
    allocator) prepared by qk_workspace_init; None when nbytes is 0."""
    if nbytes == 0:
        return None
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return workspace_init(ws, stream)


def workspace_for(device: torch.device, stream_handle: int, nbytes: int) -> torch.Tensor | None:
    """A prepared workspace of at least nbytes for one (device, stream).

    libqk leaves the workspace zero after every successful call, so one buffer
    serves all calls issued in order on that stream.
    """
    if nbytes == 0:
        return None
    key = (device, stream_handle)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = new_workspace(nbytes, device)
        _workspaces[key] = ws
    return ws


def _check_ws(status: int, device, stream_handle: int):
    """_check for calls that used a cached workspace: after a HIP launch error
    part of the call may have run, so the workspace is dropped (the next call
    prepares a fresh one)."""
    if status != QK_OK and status < 1000:
        _workspaces.pop((device, stream_handle), None)
    _check(status)


def gemm_i8_scaled(a: torch.Tensor, b: torch.Tensor, scale_a: torch.Tensor | None = None,
                   scale_b: torch.Tensor | None = None, output_scale: float = 1.0,
                   out_dtype: torch.dtype | None = torch.bfloat16, b_layout: str = "kn",
                   return_acc: bool = False, out: torch.Tensor | None = None,
                   c: torch.Tensor | None = None, kernel: str = "auto",
                   workspace: torch.Tensor | None = None):
    """INT8 GEMM, INT32 accumulation, dequant epilogue.

    a [m, k] int8; b [k, n] ("kn") or [n, k] ("nk") int8; scale_a [m] and
    scale_b [n] fp32.  Returns out [m, n] (out_dtype fp32 or bf16), or
    (out, c) with the raw int32 accumulators when return_acc; out_dtype None
    returns only c.
    """
    _need(a, "a", torch.int8, 2)
    dev = a.device
    _need(b, "b", torch.int8, 2, dev)
    layout = _LAYOUTS[b_layout]
    m, k = a.shape
    n, kb = (b.shape[1], b.shape[0]) if layout == B_KN else (b.shape[0], b.shape[1])
    if kb != k:
        raise ValueError(f"inner dimensions differ: a has k={k}, b has {kb}")
    want_out = out is not None or out_dtype is not None
    if want_out:
        out_dtype = out.dtype if out is not None else out_dtype
        if out_dtype not in _OUT_DTYPES:
            raise TypeError(f"out dtype {out_dtype} not supported")
        if out is None:
            out = torch.empty((m, n), dtype=out_dtype, device=dev)
        _need(out, "out", out_dtype, 2, dev)
        _need(scale_a, "scale_a", torch.float32, 1, dev)
        _need(scale_b, "scale_b", torch.float32, 1, dev)
        if scale_a.shape[0] != m or scale_b.shape[0] != n or tuple(out.shape) != (m, n):
            raise ValueError("scale_a must be [m], scale_b [n], out [m, n]")
    if return_acc or not want_out:
        if c is None:
            c = torch.empty((m, n), dtype=torch.int32, device=dev)
        _need(c, "c", torch.int32, 2, dev)
    else:
        c = None
    stream = torch.cuda.current_stream(dev)
    if workspace is None:
        workspace = workspace_for(dev, stream.cuda_stream, gemm_workspace_size(m, n, k))
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check_ws(library().qk_gemm_i8_scaled_ex(
        m, n, k, _ptr(a), _ptr(b), _ptr(c), _ptr(scale_a if want_out else None),
        _ptr(scale_b if want_out else None), float(output_scale), _ptr(out if want_out else None),
        _OUT_DTYPES[out_dtype] if want_out else F32, layout, _ptr(workspace), ws_bytes,
        _KERNELS[kernel], ctypes.c_void_p(stream.cuda_stream)), dev, stream.cuda_stream)
    if not want_out:
        return c
    return (out, c) if return_acc else out


def linear_w8a8(x: torch.Tensor, w: torch.Tensor, s_ch: torch.Tensor,
                out_dtype: torch.dtype | None = torch.bfloat16, b_layout: str = "kn",
                output_scale: float = 1.0, kernel: str = "auto", out: torch.Tensor | None = None,
                q: torch.Tensor | None = None, scale: torch.Tensor | None = None,
                return_codes: bool = False, workspace: torch.Tensor | None = None,
                return_acc: bool = False, c: torch.Tensor | None = None):
    """The whole layer in one call: per-token quantization of x, INT8 GEMM, dequant.

    Decode shapes (m <= 8, [k, n] weight) run as one fused launch.  Otherwise
    the codes and scales go through q / scale (allocated when not given).
    Returns out; with return_codes also q and scale, with return_acc also the
    raw int32 accumulators c (in that order: out, q, scale, c).  out_dtype
    None (and no out) writes only c.
    """
    _need(x, "x", ndim=2)
    if x.dtype not in _IN_DTYPES:
        raise TypeError(f"x dtype {x.dtype} not supported")
    dev = x.device
    _need(w, "w", torch.int8, 2, dev)
    layout = _LAYOUTS[b_layout]
    m, k = x.shape
    n, kb = (w.shape[1], w.shape[0]) if layout == B_KN else (w.shape[0], w.shape[1])
    if kb != k:
        raise ValueError(f"inner dimensions differ: x has k={k}, w has {kb}")
    want_out = out is not None or out_dtype is not None
    if want_out:
        out_dtype = out.dtype if out is not None else out_dtype
        if out_dtype not in _OUT_DTYPES:
            raise TypeError(f"out dtype {out_dtype} not supported")
        out = torch.empty((m, n), dtype=out_dtype, device=dev) if out is None else out
        _need(out, "out", out_dtype, 2, dev)
        _need(s_ch, "s_ch", torch.float32, 1, dev)
        if tuple(out.shape) != (m, n) or s_ch.shape[0] != n:
            raise ValueError("out must be [m, n] and s_ch [n]")
    if return_acc or not want_out:
        c = torch.empty((m, n), dtype=torch.int32, device=dev) if c is None else c
        _need(c, "c", torch.int32, 2, dev)
        if tuple(c.shape) != (m, n):
            raise ValueError("c must be [m, n]")
    else:
        c = None
    fused = (m <= 8 and layout == B_KN and kernel != "mfma") or kernel == "gemv"
    if (return_codes or not fused) and q is None:
        q = torch.empty((m, k), dtype=torch.int8, device=dev)
    if (return_codes or not fused) and scale is None:
        scale = torch.empty((m,), dtype=torch.float32, device=dev)
    if q is not None:
        _need(q, "q", torch.int8, 2, dev)
    if scale is not None:
        _need(scale, "scale", torch.float32, 1, dev)
    stream = torch.cuda.current_stream(dev)
    if workspace is None:
        workspace = workspace_for(dev, stream.cuda_stream, gemm_workspace_size(m, n, k))
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check_ws(library().qk_linear_w8a8(
        m, n, k, _ptr(x), _IN_DTYPES[x.dtype], _ptr(w), _ptr(s_ch if want_out else None),
        float(output_scale), _ptr(out if want_out else None),
        _OUT_DTYPES[out_dtype] if want_out else F32, layout, _ptr(q), _ptr(scale), _ptr(c),
        _ptr(workspace), ws_bytes, _KERNELS[kernel], ctypes.c_void_p(stream.cuda_stream)),
        dev, stream.cuda_stream)
    res = (out,) if want_out else ()
    if return_codes:
        res += (q, scale)
    if return_acc or not want_out:
        res += (c,)
    return res[0] if len(res) == 1 else res


def gated_linear_w8a8(h: torch.Tensor, w: torch.Tensor, s_ch: torch.Tensor,
                      out_dtype: torch.dtype = torch.bfloat16, b_layout: str = "kn",
                      output_scale: float = 1.0, kernel: str = "auto"):
    """silu(gate) * up with per-token quantization, then the INT8 GEMM."""
    q, s = silu_mul_quant_per_token(h)
    return gemm_i8_scaled(q, w, s, s_ch, output_scale, out_dtype, b_layout, kernel=kernel)


# ---- FP8 (float8_e4m3fn) path ----
_FP8_CODE_DTYPES = (torch.float8_e4m3fn, torch.uint8)


def _need_codes(t: torch.Tensor, name: str, ndim=None, device=None):
    _need(t, name, ndim=ndim, device=device)
    if t.dtype not in _FP8_CODE_DTYPES:
        raise TypeError(f"{name} must be torch.float8_e4m3fn (or its uint8 bytes), got {t.dtype}")


def _fp8_rows(src: torch.Tensor, name: str, silu: bool, scale_ub: float, q, scale):
    _need(src, name, ndim=2)
    if src.dtype not in _IN_DTYPES:
        raise TypeError(f"{name} dtype {src.dtype} not supported")
    m, k = src.shape
    if silu:
        if k % 2:
            raise ValueError(f"{name} must have an even number of columns (gate | up)")
        k //= 2
    q = torch.empty((m, k), dtype=torch.float8_e4m3fn, device=src.device) if q is None else q
    scale = torch.empty((m,), dtype=torch.float32, device=src.device) if scale is None else scale
    _need_codes(q, "q", 2, src.device)
    _need(scale, "scale", torch.float32, 1, src.device)
    if tuple(q.shape) != (m, k) or scale.shape[0] != m:
        raise ValueError(f"q must be [m, {'d' if silu else 'k'}] and scale [m]")
    fn = library().qk_silu_mul_quant_per_token_fp8 if silu else library().qk_quant_per_token_fp8
    _check(fn(m, k, _ptr(src), _IN_DTYPES[src.dtype], float(scale_ub), _ptr(q), _ptr(scale),
              _stream(src.device)))
    return q, scale


def quant_per_token_fp8(x: torch.Tensor, scale_ub: float = 0.0, q: torch.Tensor | None = None,
                        scale: torch.Tensor | None = None):
    """Per-token float8_e4m3fn codes and fp32 scales of x [m, k]; scale_ub > 0
    bounds the scales from above (codes then saturate at +-448)."""
    return _fp8_rows(x, "x", False, scale_ub, q, scale)


def silu_mul_quant_per_token_fp8(h: torch.Tensor, scale_ub: float = 0.0,
                                 q: torch.Tensor | None = None,
                                 scale: torch.Tensor | None = None):
    """FP8 codes and scales of silu(h[:, :d]) * h[:, d:] for h [m, 2d]."""
    return _fp8_rows(h, "h", True, scale_ub, q, scale)


def gemm_fp8_scaled(a: torch.Tensor, b: torch.Tensor, scale_a: torch.Tensor | None = None,
                    scale_b: torch.Tensor | None = None, output_scale: float = 1.0,
                    out_dtype: torch.dtype | None = torch.bfloat16, b_layout: str = "kn",
                    return_acc: bool = False, out: torch.Tensor | None = None,
                    c: torch.Tensor | None = None):
    """FP8 GEMM with binary32 accumulation and the dequant epilogue.

    a [m, k] and b [k, n] ("kn") or [n, k] ("nk") float8_e4m3fn codes; scale_a
    [m], scale_b [n] fp32.  Returns out, (out, c) with the raw fp32
    accumulators when return_acc, or c alone when out_dtype is None.
    """
    _need_codes(a, "a", 2)
    dev = a.device
    _need_codes(b, "b", 2, dev)
    layout = _LAYOUTS[b_layout]
    m, k = a.shape
    n, kb = (b.shape[1], b.shape[0]) if layout == B_KN else (b.shape[0], b.shape[1])
    if kb != k:
        raise ValueError(f"inner dimensions differ: a has k={k}, b has {kb}")
    want_out = out is not None or out_dtype is not None
    if want_out:
        out_dtype = out.dtype if out is not None else out_dtype
        if out_dtype not in _OUT_DTYPES:
            raise TypeError(f"out dtype {out_dtype} not supported")
        if out is None:
            out = torch.empty((m, n), dtype=out_dtype, device=dev)
        _need(out, "out", out_dtype, 2, dev)
        _need(scale_a, "scale_a", torch.float32, 1, dev)
        _need(scale_b, "scale_b", torch.float32, 1, dev)
        if scale_a.shape[0] != m or scale_b.shape[0] != n or tuple(out.shape) != (m, n):
            raise ValueError("scale_a must be [m], scale_b [n], out [m, n]")
    if return_acc or not want_out:
        if c is None:
            c = torch.empty((m, n), dtype=torch.float32, device=dev)
        _need(c, "c", torch.float32, 2, dev)
    else:
        c = None
    _check(library().qk_gemm_fp8_scaled(
        m, n, k, _ptr(a), _ptr(b), _ptr(c), _ptr(scale_a if want_out else None),
        _ptr(scale_b if want_out else None), float(output_scale), _ptr(out if want_out else None),
        _OUT_DTYPES[out_dtype] if want_out else F32, layout, _stream(dev)))
    if not want_out:
        return c
    return (out, c) if return_acc else out


def linear_fp8(x: torch.Tensor, w: torch.Tensor, s_ch: torch.Tensor, scale_ub: float = 0.0,
               out_dtype: torch.dtype = torch.bfloat16, b_layout: str = "kn",
               output_scale: float = 1.0, out: torch.Tensor | None = None,
               q: torch.Tensor | None = None, scale: torch.Tensor | None = None,
               return_codes: bool = False):
    """The FP8 layer: per-token FP8 quantization of x, FP8 GEMM, dequant."""
    _need(x, "x", ndim=2)
    if x.dtype not in _IN_DTYPES:
        raise TypeError(f"x dtype {x.dtype} not supported")
    dev = x.device
    _need_codes(w, "w", 2, dev)
    _need(s_ch, "s_ch", torch.float32, 1, dev)
    layout = _LAYOUTS[b_layout]
    m, k = x.shape
    n, kb = (w.shape[1], w.shape[0]) if layout == B_KN else (w.shape[0], w.shape[1])
    if kb != k:
        raise ValueError(f"inner dimensions differ: x has k={k}, w has {kb}")
    if out_dtype not in _OUT_DTYPES:
        raise TypeError(f"out dtype {out_dtype} not supported")
    out = torch.empty((m, n), dtype=out_dtype, device=dev) if out is None else out
    _need(out, "out", out_dtype, 2, dev)
    q = torch.empty((m, k), dtype=torch.float8_e4m3fn, device=dev) if q is None else q
    scale = torch.empty((m,), dtype=torch.float32, device=dev) if scale is None else scale
    _need_codes(q, "q", 2, dev)
    _need(scale, "scale", torch.float32, 1, dev)
    _check(library().qk_linear_fp8(
        m, n, k, _ptr(x), _IN_DTYPES[x.dtype], float(scale_ub), _ptr(w), _ptr(s_ch),
        float(output_scale), _ptr(out), _OUT_DTYPES[out_dtype], layout, _ptr(q), _ptr(scale),
        _stream(dev)))
    return (out, q, scale) if return_codes else out


def gated_linear_fp8(h: torch.Tensor, w: torch.Tensor, s_ch: torch.Tensor, scale_ub: float = 0.0,
                     out_dtype: torch.dtype = torch.bfloat16, b_layout: str = "kn",
                     output_scale: float = 1.0):
    """silu(gate) * up with per-token FP8 quantization, then the FP8 GEMM."""
    q, s = silu_mul_quant_per_token_fp8(h, scale_ub)
    return gemm_fp8_scaled(q, w, s, s_ch, output_scale, out_dtype, b_layout)


# ---- INT8 GEMM with per-group weight scales ----

def gemm_i8_grouped(a: torch.Tensor, b: torch.Tensor, scale_a: torch.Tensor | None,
                    scale_b: torch.Tensor, group: int, output_scale: float = 1.0,
                    out_dtype: torch.dtype | None = torch.bfloat16, b_layout: str = "kn",
                    return_acc: bool = False, out: torch.Tensor | None = None,
                    c: torch.Tensor | None = None):
    """INT8 GEMM whose weight carries one scale per group of `group` (64 or
    128) consecutive k of each output column.

    a [m, k] int8; b [k, n] ("kn") or [n, k] ("nk") int8; scale_a [m] fp32;
    scale_b [k / group, n] fp32.  acc = sum_g scale_b[g] * (INT32 partial of
    group g) in binary32; out = acc * scale_a * output_scale.  Returns out,
    (out, c) with the binary32 accumulators when return_acc, or c alone when
    out_dtype is None.
    """
    _need(a, "a", torch.int8, 2)
    dev = a.device
    _need(b, "b", torch.int8, 2, dev)
    layout = _LAYOUTS[b_layout]
    m, k = a.shape
    n, kb = (b.shape[1], b.shape[0]) if layout == B_KN else (b.shape[0], b.shape[1])
    if kb != k:
        raise ValueError(f"inner dimensions differ: a has k={k}, b has {kb}")
    _need(scale_b, "scale_b", torch.float32, 2, dev)
    if group <= 0 or k % group or tuple(scale_b.shape) != (k // group, n):
        raise ValueError("scale_b must be [k / group, n] with k a multiple of group")
    want_out = out is not None or out_dtype is not None
    if want_out:
        out_dtype = out.dtype if out is not None else out_dtype
        if out_dtype not in _OUT_DTYPES:
            raise TypeError(f"out dtype {out_dtype} not supported")
        if out is None:
            out = torch.empty((m, n), dtype=out_dtype, device=dev)
        _need(out, "out", out_dtype, 2, dev)
        _need(scale_a, "scale_a", torch.float32, 1, dev)
        if scale_a.shape[0] != m or tuple(out.shape) != (m, n):
            raise ValueError("scale_a must be [m], out [m, n]")
    if return_acc or not want_out:
        if c is None:
            c = torch.empty((m, n), dtype=torch.float32, device=dev)
        _need(c, "c", torch.float32, 2, dev)
    else:
        c = None
    _check(library().qk_gemm_i8_grouped(
        m, n, k, int(group), _ptr(a), _ptr(b), _ptr(c), _ptr(scale_a if want_out else None),
        _ptr(scale_b), float(output_scale), _ptr(out if want_out else None),
        _OUT_DTYPES[out_dtype] if want_out else F32, layout, _stream(dev)))
    if not want_out:
        return c
    return (out, c) if return_acc else out


# ---- MoE grouped GEMM ----
MOE_MAX_EXPERTS = 256


def moe_gemm_i8_scaled(a: torch.Tensor, w: torch.Tensor, offsets: torch.Tensor,
                       scale_a: torch.Tensor | None = None, scale_b: torch.Tensor | None = None,
                       output_scale: float = 1.0, out_dtype: torch.dtype | None = torch.bfloat16,
                       b_layout: str = "kn", return_acc: bool = False,
                       out: torch.Tensor | None = None, c: torch.Tensor | None = None):
    """All experts' INT8 GEMMs in one launch.

    a [m, k] int8 codes, rows grouped by expert; w [experts, k, n] ("kn") or
    [experts, n, k] ("nk") int8; offsets int32 [experts + 1] on the GPU (row
    ranges, nondecreasing from 0 to m); scale_a [m], scale_b [experts, n]
    fp32.  Returns out, (out, c) with the raw int32 accumulators, or c alone
    when out_dtype is None.
    """
    _need(a, "a", torch.int8, 2)
    dev = a.device
    _need(w, "w", torch.int8, 3, dev)
    _need(offsets, "offsets", torch.int32, 1, dev)
    layout = _LAYOUTS[b_layout]
    experts = w.shape[0]
    m, k = a.shape
    n, kb = (w.shape[2], w.shape[1]) if layout == B_KN else (w.shape[1], w.shape[2])
    if kb != k:
        raise ValueError(f"inner dimensions differ: a has k={k}, w has {kb}")
    if offsets.shape[0] != experts + 1:
        raise ValueError("offsets must have experts + 1 entries")
    want_out = out is not None or out_dtype is not None
    if want_out:
        out_dtype = out.dtype if out is not None else out_dtype
        if out_dtype not in _OUT_DTYPES:
            raise TypeError(f"out dtype {out_dtype} not supported")
        if out is None:
            out = torch.empty((m, n), dtype=out_dtype, device=dev)
        _need(out, "out", out_dtype, 2, dev)
        _need(scale_a, "scale_a", torch.float32, 1, dev)
        _need(scale_b, "scale_b", torch.float32, 2, dev)
        if scale_a.shape[0] != m or tuple(scale_b.shape) != (experts, n) or tuple(out.shape) != (m, n):
            raise ValueError("scale_a must be [m], scale_b [experts, n], out [m, n]")
    if return_acc or not want_out:
        if c is None:
            c = torch.empty((m, n), dtype=torch.int32, device=dev)
        _need(c, "c", torch.int32, 2, dev)
    else:
        c = None
    _check(library().qk_moe_gemm_i8_scaled(
        experts, m, n, k, _ptr(offsets), _ptr(a), _ptr(w), _ptr(c),
        _ptr(scale_a if want_out else None), _ptr(scale_b if want_out else None),
        float(output_scale), _ptr(out if want_out else None),
        _OUT_DTYPES[out_dtype] if want_out else F32, layout, _stream(dev)))
    if not want_out:
        return c
    return (out, c) if return_acc else out


# ---- static (per-tensor) quantization ----

def quant_static(x: torch.Tensor, scale: torch.Tensor, fp8: bool = False, silu: bool = False,
                 q: torch.Tensor | None = None) -> torch.Tensor:
    """Codes of x [m, k] (or of silu(h[:, :d]) * h[:, d:] when silu) with one
    scale for the whole tensor (a one-element fp32 GPU tensor): INT8
    clamp(rint(x / s), -127, 127), or float8_e4m3fn x / s when fp8."""
    _need(x, "x", ndim=2)
    if x.dtype not in _IN_DTYPES:
        raise TypeError(f"x dtype {x.dtype} not supported")
    _need(scale, "scale", torch.float32, None, x.device)
    if scale.numel() != 1:
        raise ValueError("scale must hold one value")
    m, k = x.shape
    if silu:
        if k % 2:
            raise ValueError("h must have an even number of columns (gate | up)")
        k //= 2
    qdt = torch.float8_e4m3fn if fp8 else torch.int8
    q = torch.empty((m, k), dtype=qdt, device=x.device) if q is None else q
    if fp8:
        _need_codes(q, "q", 2, x.device)
    else:
        _need(q, "q", torch.int8, 2, x.device)
    if tuple(q.shape) != (m, k):
        raise ValueError("q has the wrong shape")
    name = ("qk_silu_mul_quant_static" if silu else "qk_quant_static") + ("_fp8" if fp8 else "")
    _check(getattr(library(), name)(m, k, _ptr(x), _IN_DTYPES[x.dtype], _ptr(scale), _ptr(q),
                                    _stream(x.device)))
    return q


# ---- asymmetric (zero-point) activations ----
MAX_K_ASYM = 65535


def quant_per_token_asym(x: torch.Tensor):
    """Asymmetric per-token INT8 codes of x [m, k]: (q int8, scale fp32 [m], zero_point int32 [m])."""
    _need(x, "x", ndim=2)
    if x.dtype not in _IN_DTYPES:
        raise TypeError(f"x dtype {x.dtype} not supported")
    m, k = x.shape
    q = torch.empty((m, k), dtype=torch.int8, device=x.device)
    scale = torch.empty((m,), dtype=torch.float32, device=x.device)
    zp = torch.empty((m,), dtype=torch.int32, device=x.device)
    _check(library().qk_quant_per_token_asym(m, k, _ptr(x), _IN_DTYPES[x.dtype], _ptr(q),
                                             _ptr(scale), _ptr(zp), _stream(x.device)))
    return q, scale, zp


def weight_colsum(w: torch.Tensor, b_layout: str = "kn") -> torch.Tensor:
    """int32 column sums of an INT8 weight ([k, n] "kn" or [n, k] "nk")."""
    _need(w, "w", torch.int8, 2)
    layout = _LAYOUTS[b_layout]
    k, n = (w.shape[0], w.shape[1]) if layout == B_KN else (w.shape[1], w.shape[0])
    wsum = torch.empty((n,), dtype=torch.int32, device=w.device)
    _check(library().qk_weight_colsum(k, n, _ptr(w), layout, _ptr(wsum), _stream(w.device)))
    return wsum


def gemm_i8_asym(a: torch.Tensor, zero_point: torch.Tensor, b: torch.Tensor, wsum: torch.Tensor,
                 scale_a: torch.Tensor | None = None, scale_b: torch.Tensor | None = None,
                 output_scale: float = 1.0, out_dtype: torch.dtype | None = torch.bfloat16,
                 b_layout: str = "kn", return_acc: bool = False):
    """INT8 GEMM of asymmetric activations: acc = sum (a - zero_point[row]) * B,
    out = acc * scale_a * scale_b * output_scale."""
    _need(a, "a", torch.int8, 2)
    dev = a.device
    _need(b, "b", torch.int8, 2, dev)
    _need(zero_point, "zero_point", torch.int32, 1, dev)
    _need(wsum, "wsum", torch.int32, 1, dev)
    layout = _LAYOUTS[b_layout]
    m, k = a.shape
    n, kb = (b.shape[1], b.shape[0]) if layout == B_KN else (b.shape[0], b.shape[1])
    if kb != k or zero_point.shape[0] != m or wsum.shape[0] != n:
        raise ValueError("shapes differ: a [m, k], zero_point [m], b [k, n], wsum [n]")
    want_out = out_dtype is not None
    out = None
    if want_out:
        if out_dtype not in _OUT_DTYPES:
            raise TypeError(f"out dtype {out_dtype} not supported")
        out = torch.empty((m, n), dtype=out_dtype, device=dev)
        _need(scale_a, "scale_a", torch.float32, 1, dev)
        _need(scale_b, "scale_b", torch.float32, 1, dev)
    c = torch.empty((m, n), dtype=torch.int32, device=dev) if (return_acc or not want_out) else None
    _check(library().qk_gemm_i8_asym(
        m, n, k, _ptr(a), _ptr(zero_point), _ptr(b), _ptr(wsum), _ptr(c),
        _ptr(scale_a if want_out else None), _ptr(scale_b if want_out else None),
        float(output_scale), _ptr(out), _OUT_DTYPES[out_dtype] if want_out else F32, layout,
        _stream(dev)))
    if not want_out:
        return c
    return (out, c) if return_acc else out
