"""The C-ABI library loads, exports every symbol include/qk.h declares, and
rejects bad arguments on the host before anything reaches a GPU.

None of these calls launches a kernel: each returns from host-side checks, so
they run without a GPU.
"""
import ctypes
import os
import re

import pytest

import w8a8_int8_quantized_qk_amd as qk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qk.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qk_[a-z0-9_]+)\s*\(", text)))


def _header_constants():
    consts = {}
    for name, val in re.findall(r"#define\s+(QK_[A-Z0-9_]+)\s+(-?\d+)", open(HEADER).read()):
        consts[name] = int(val)
    return consts


@pytest.fixture(scope="module")
def lib():
    return qk.library()


def test_every_declared_function_is_exported(lib):
    names = _declared_functions()
    assert len(names) >= 8
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(qk.EXPORTED)


def test_binding_constants_match_header():
    c = _header_constants()
    assert c["QK_ABI_VERSION"] == qk.ABI_VERSION
    assert (c["QK_F32"], c["QK_BF16"], c["QK_F16"]) == (qk.F32, qk.BF16, qk.F16)
    assert (c["QK_B_KN"], c["QK_B_NK"]) == (qk.B_KN, qk.B_NK)
    assert (c["QK_KERNEL_AUTO"], c["QK_KERNEL_MFMA"], c["QK_KERNEL_GEMV"]) == (
        qk.KERNEL_AUTO, qk.KERNEL_MFMA, qk.KERNEL_GEMV)


def test_abi_version_and_build_info(lib):
    assert lib.qk_abi_version() == qk.ABI_VERSION
    info = qk.build_info()
    assert "gfx950" in info and f"ABI {qk.ABI_VERSION}" in info


def test_status_strings(lib):
    c = _header_constants()
    for code in ("QK_OK", "QK_ERR_INVALID_VALUE", "QK_ERR_UNSUPPORTED", "QK_ERR_WORKSPACE"):
        s = qk.status_string(c[code])
        assert s.startswith(code)


def test_abi_mismatch_refuses_to_load(monkeypatch):
    monkeypatch.setattr(qk, "ABI_VERSION", qk.ABI_VERSION + 1)
    with pytest.raises(ImportError, match="ABI"):
        qk.load_library()


def test_missing_library_raises(tmp_path):
    with pytest.raises(ImportError, match="missing"):
        qk.load_library(str(tmp_path / "libqk.so"))


def test_workspace_size(lib):
    assert qk.gemm_workspace_size(2048, 4096, 4096) == 0        # tiled kernel needs none
    ws = qk.gemm_workspace_size(1, 14336, 4096)
    assert ws >= 8 * 14336 * 4 and ws % 256 == 0
    assert qk.gemm_workspace_size(16, 100, 16) > 0
    assert qk.gemm_workspace_size(17, 100, 16) == 0
    assert qk.gemm_workspace_size(0, 100, 16) == 0


NULL = ctypes.c_void_p(0)
FAKE = ctypes.c_void_p(0x100000)      # 16-byte aligned; never dereferenced by these calls
FAKE_ODD = ctypes.c_void_p(0x100001)


def _gemm(lib, m, n, k, a=FAKE, b=FAKE, c=FAKE, sa=FAKE, sb=FAKE, out=FAKE, out_dtype=0,
          layout=0, ws=NULL, ws_bytes=0, kernel=0):
    return lib.qk_gemm_i8_scaled_ex(m, n, k, a, b, c, sa, sb, 1.0, out, out_dtype, layout, ws,
                                    ws_bytes, kernel, NULL)


def test_gemm_argument_errors_are_reported_before_launch(lib):
    c = _header_constants()
    INVALID, UNSUP, WS = c["QK_ERR_INVALID_VALUE"], c["QK_ERR_UNSUPPORTED"], c["QK_ERR_WORKSPACE"]
    assert _gemm(lib, -1, 4, 16) == INVALID
    assert _gemm(lib, 4, -1, 16) == INVALID
    assert _gemm(lib, 4, 4, -16) == INVALID
    assert _gemm(lib, 4, 4, 131072) == INVALID            # beyond QK_MAX_K
    assert _gemm(lib, 4, 4, 24) == UNSUP                  # k % 16 != 0
    assert _gemm(lib, 4, 4, 16, c=NULL, out=NULL) == INVALID
    assert _gemm(lib, 4, 4, 16, out_dtype=2) == INVALID   # fp16 out not offered
    assert _gemm(lib, 4, 4, 16, layout=7) == INVALID
    assert _gemm(lib, 4, 4, 16, kernel=9) == INVALID
    assert _gemm(lib, 40, 4, 16, a=NULL) == INVALID
    assert _gemm(lib, 40, 4, 16, sa=NULL) == INVALID      # out needs both scales
    assert _gemm(lib, 40, 4, 16, a=FAKE_ODD) == UNSUP     # 128-bit loads need alignment
    assert _gemm(lib, 17, 4, 16, kernel=2) == UNSUP       # decode kernel takes m <= 16
    assert _gemm(lib, 4, 4, 16, layout=1, kernel=2) == UNSUP
    assert _gemm(lib, 4, 4, 16, kernel=2) == WS           # decode kernel without workspace
    assert _gemm(lib, 4, 4, 16, ws=FAKE, ws_bytes=16) == WS
    # empty problems succeed without touching memory
    assert _gemm(lib, 0, 4, 16, a=NULL, b=NULL) == 0
    assert _gemm(lib, 4, 0, 16, a=NULL, b=NULL) == 0


def test_quant_argument_errors_are_reported_before_launch(lib):
    c = _header_constants()
    INVALID = c["QK_ERR_INVALID_VALUE"]
    assert lib.qk_quant_per_token(-1, 4, FAKE, 0, FAKE, FAKE, NULL) == INVALID
    assert lib.qk_quant_per_token(4, -4, FAKE, 0, FAKE, FAKE, NULL) == INVALID
    assert lib.qk_quant_per_token(4, 4, FAKE, 5, FAKE, FAKE, NULL) == INVALID
    assert lib.qk_quant_per_token(4, 4, NULL, 0, FAKE, FAKE, NULL) == INVALID
    assert lib.qk_quant_per_token(4, 4, FAKE, 0, FAKE, NULL, NULL) == INVALID
    assert lib.qk_quant_per_token(0, 4, NULL, 0, NULL, NULL, NULL) == 0
    assert lib.qk_silu_mul_quant_per_token(4, 4, FAKE, 3, FAKE, FAKE, NULL) == INVALID
    assert lib.qk_silu_mul_quant_per_token(0, 4, NULL, 1, NULL, NULL, NULL) == 0
    assert lib.qk_silu_mul(-1, 4, FAKE, 1, FAKE, NULL) == INVALID
    assert lib.qk_silu_mul(4, 4, FAKE, 3, FAKE, NULL) == INVALID
    assert lib.qk_silu_mul(4, 4, NULL, 1, FAKE, NULL) == INVALID
    assert lib.qk_silu_mul(4, 4, FAKE, 1, NULL, NULL) == INVALID
    assert lib.qk_silu_mul(0, 4, NULL, 1, NULL, NULL) == 0
    assert lib.qk_silu_mul(4, 0, NULL, 1, NULL, NULL) == 0
    assert lib.qk_silu_mul(4, 0x40000000, FAKE, 1, FAKE, NULL) == c["QK_ERR_UNSUPPORTED"]


def _linear(lib, m, n, k, x=FAKE, xdt=1, b=FAKE, sb=FAKE, out=FAKE, odt=1, layout=0, q=NULL,
            s=NULL, cc=NULL, ws=NULL, ws_bytes=0, kernel=0):
    return lib.qk_linear_w8a8(m, n, k, x, xdt, b, sb, 1.0, out, odt, layout, q, s, cc, ws,
                              ws_bytes, kernel, NULL)


def test_linear_argument_errors_are_reported_before_launch(lib):
    c = _header_constants()
    INVALID, UNSUP = c["QK_ERR_INVALID_VALUE"], c["QK_ERR_UNSUPPORTED"]
    assert _linear(lib, -1, 4, 16) == INVALID
    assert _linear(lib, 4, 4, 16, xdt=7) == INVALID
    assert _linear(lib, 4, 4, 16, odt=2) == INVALID
    assert _linear(lib, 4, 4, 24) == UNSUP
    assert _linear(lib, 4, 4, 16, out=NULL) == INVALID      # neither out nor c_out
    assert _linear(lib, 4, 4, 16, sb=NULL) == INVALID
    assert _linear(lib, 4, 4, 16, cc=FAKE_ODD) == UNSUP
    assert _linear(lib, 4, 4, 16, out=NULL, sb=NULL, cc=FAKE, odt=9) == c["QK_ERR_WORKSPACE"]
    assert _linear(lib, 4, 4, 16, b=FAKE_ODD) == UNSUP
    assert _linear(lib, 64, 4, 16) == INVALID              # tiled path needs q and scale
    assert _linear(lib, 4, 4, 16, layout=1) == INVALID     # [n][k] weight: tiled path too
    assert _linear(lib, 17, 4, 16, kernel=2) == UNSUP
    assert _linear(lib, 4, 4, 16) == c["QK_ERR_WORKSPACE"]  # fused decode launch needs one
    assert _linear(lib, 0, 4, 16, x=NULL, b=NULL) == 0


def test_noalloc_linear_errors_are_reported_before_launch(lib):
    c = _header_constants()
    assert c["QK_SCRATCH_BYTES"] == qk.SCRATCH_BYTES

    def na(m, n, k, out=FAKE, q=NULL, s=NULL, cc=NULL, kernel=0, layout=0):
        return lib.qk_linear_w8a8_noalloc(m, n, k, FAKE, 1, FAKE, FAKE, 1.0, out, 1, layout, q, s,
                                          cc, kernel, NULL)

    assert na(-1, 4, 16) == c["QK_ERR_INVALID_VALUE"]
    assert na(4, 4, 24) == c["QK_ERR_UNSUPPORTED"]
    assert na(4, 4, 16, out=NULL) == c["QK_ERR_INVALID_VALUE"]
    assert na(64, 4, 16) == c["QK_ERR_INVALID_VALUE"]          # tiled path needs q and scale
    # the decode launch needs 64 bytes of scratch per column: beyond the static
    # scratch it is refused before anything is enqueued
    cols = qk.SCRATCH_BYTES // 64
    assert na(1, cols + 16, 16) == c["QK_ERR_SCRATCH_LIMIT"]
    assert na(1, cols + 16, 16, kernel=2) == c["QK_ERR_SCRATCH_LIMIT"]
    assert na(0, 4, 16) == 0
    assert qk.status_string(c["QK_ERR_SCRATCH_LIMIT"]).startswith("QK_ERR_SCRATCH_LIMIT")


def test_workspace_init_argument_errors_are_reported_before_launch(lib):
    c = _header_constants()
    size_t = ctypes.c_size_t
    assert lib.qk_workspace_init(NULL, size_t(0), NULL) == 0          # nothing to prepare
    assert lib.qk_workspace_init(FAKE, size_t(0), NULL) == 0
    assert lib.qk_workspace_init(NULL, size_t(256), NULL) == c["QK_ERR_INVALID_VALUE"]
    assert lib.qk_workspace_init(ctypes.c_void_p(0x100010), size_t(256), NULL) == c["QK_ERR_WORKSPACE"]


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(2, 16)
    with pytest.raises(ValueError, match="GPU"):
        qk.quant_per_token(x)


def test_fp8_argument_errors_are_reported_before_launch(lib):
    c = _header_constants()
    INVALID, UNSUP = c["QK_ERR_INVALID_VALUE"], c["QK_ERR_UNSUPPORTED"]
    nan = float("nan")
    q8 = lib.qk_quant_per_token_fp8
    assert q8(-1, 4, FAKE, 0, 0.0, FAKE, FAKE, NULL) == INVALID
    assert q8(4, 4, FAKE, 5, 0.0, FAKE, FAKE, NULL) == INVALID
    assert q8(4, 4, NULL, 0, 0.0, FAKE, FAKE, NULL) == INVALID
    assert q8(4, 4, FAKE, 0, nan, FAKE, FAKE, NULL) == INVALID        # NaN scale bound
    assert q8(0, 4, NULL, 0, 0.0, NULL, NULL, NULL) == 0
    s8 = lib.qk_silu_mul_quant_per_token_fp8
    assert s8(4, 4, FAKE, 3, 0.0, FAKE, FAKE, NULL) == INVALID
    assert s8(4, 4, FAKE, 1, nan, FAKE, FAKE, NULL) == INVALID
    assert s8(0, 4, NULL, 1, 1.0, NULL, NULL, NULL) == 0

    def g8(m, n, k, a=FAKE, b=FAKE, cc=FAKE, sa=FAKE, sb=FAKE, out=FAKE, odt=0, layout=0):
        return lib.qk_gemm_fp8_scaled(m, n, k, a, b, cc, sa, sb, 1.0, out, odt, layout, NULL)

    assert g8(-1, 4, 16) == INVALID
    assert g8(4, 4, 131072) == INVALID
    assert g8(4, 4, 24) == UNSUP
    assert g8(4, 4, 16, cc=NULL, out=NULL) == INVALID
    assert g8(4, 4, 16, odt=2) == INVALID
    assert g8(4, 4, 16, layout=3) == INVALID
    assert g8(4, 4, 16, a=NULL) == INVALID
    assert g8(4, 4, 16, sb=NULL) == INVALID
    assert g8(4, 4, 16, b=FAKE_ODD) == UNSUP
    assert g8(0, 4, 16, a=NULL, b=NULL) == 0

    def l8(m, n, k, x=FAKE, xdt=1, ub=0.0, b=FAKE, sb=FAKE, out=FAKE, odt=1, q=FAKE, s=FAKE):
        return lib.qk_linear_fp8(m, n, k, x, xdt, ub, b, sb, 1.0, out, odt, 0, q, s, NULL)

    assert l8(-1, 4, 16) == INVALID
    assert l8(4, 4, 16, xdt=9) == INVALID
    assert l8(4, 4, 16, ub=nan) == INVALID
    assert l8(4, 4, 16, q=NULL) == INVALID                 # codes buffer is required
    assert l8(4, 4, 16, s=NULL) == INVALID
    assert l8(4, 4, 16, q=FAKE_ODD) == UNSUP
    assert l8(4, 4, 24) == UNSUP
    assert l8(0, 4, 16, x=NULL, b=NULL, q=NULL, s=NULL) == 0


def test_fp8_binding_rejects_wrong_dtypes():
    import torch
    with pytest.raises(ValueError, match="GPU"):
        qk.quant_per_token_fp8(torch.zeros(2, 16))
    with pytest.raises(ValueError, match="GPU"):
        qk.gemm_fp8_scaled(torch.zeros(2, 16, dtype=torch.float8_e4m3fn),
                           torch.zeros(16, 4, dtype=torch.float8_e4m3fn), out_dtype=None)


def test_grouped_argument_errors_are_reported_before_launch(lib):
    c = _header_constants()
    INVALID, UNSUP = c["QK_ERR_INVALID_VALUE"], c["QK_ERR_UNSUPPORTED"]

    def gg(m, n, k, group=128, a=FAKE, b=FAKE, cc=FAKE, sa=FAKE, sb=FAKE, out=FAKE, odt=0, layout=0):
        return lib.qk_gemm_i8_grouped(m, n, k, group, a, b, cc, sa, sb, 1.0, out, odt, layout, NULL)

    assert gg(-1, 4, 128) == INVALID
    assert gg(4, 4, 256, group=32) == UNSUP      # groups of 64 or 128 only
    assert gg(4, 4, 192, group=128) == UNSUP     # k a multiple of the group
    assert gg(4, 4, 128, sb=NULL) == INVALID
    assert gg(4, 4, 128, sa=NULL) == INVALID     # out needs the token scales
    assert gg(4, 4, 128, cc=NULL, out=NULL) == INVALID
    assert gg(4, 4, 128, layout=5) == INVALID
    assert gg(4, 4, 128, a=FAKE_ODD) == UNSUP
    assert gg(0, 4, 128, a=NULL, b=NULL) == 0


def test_moe_argument_errors_are_reported_before_launch(lib):
    c = _header_constants()
    INVALID, UNSUP = c["QK_ERR_INVALID_VALUE"], c["QK_ERR_UNSUPPORTED"]
    assert c["QK_MOE_MAX_EXPERTS"] == qk.MOE_MAX_EXPERTS

    def mm(e, m, n, k, off=FAKE, a=FAKE, b=FAKE, cc=FAKE, sa=FAKE, sb=FAKE, out=FAKE, odt=0, layout=0):
        return lib.qk_moe_gemm_i8_scaled(e, m, n, k, off, a, b, cc, sa, sb, 1.0, out, odt, layout, NULL)

    assert mm(0, 4, 4, 16) == INVALID
    assert mm(qk.MOE_MAX_EXPERTS + 1, 4, 4, 16) == INVALID
    assert mm(2, -1, 4, 16) == INVALID
    assert mm(2, 4, 4, 24) == UNSUP
    assert mm(2, 4, 4, 16, off=NULL) == INVALID
    assert mm(2, 4, 4, 16, sb=NULL) == INVALID
    assert mm(2, 4, 4, 16, cc=NULL, out=NULL) == INVALID
    assert mm(2, 4, 4, 16, b=FAKE_ODD) == UNSUP
    assert mm(2, 0, 4, 16, off=NULL, a=NULL) == 0


def test_static_and_asym_argument_errors_are_reported_before_launch(lib):
    c = _header_constants()
    INVALID, UNSUP = c["QK_ERR_INVALID_VALUE"], c["QK_ERR_UNSUPPORTED"]
    assert c["QK_MAX_K_ASYM"] == qk.MAX_K_ASYM
    for name in ("qk_quant_static", "qk_silu_mul_quant_static", "qk_quant_static_fp8",
                 "qk_silu_mul_quant_static_fp8"):
        fn = getattr(lib, name)
        assert fn(-1, 4, FAKE, 0, FAKE, FAKE, NULL) == INVALID
        assert fn(4, 4, FAKE, 9, FAKE, FAKE, NULL) == INVALID
        assert fn(4, 4, FAKE, 0, NULL, FAKE, NULL) == INVALID      # no scale
        assert fn(0, 4, NULL, 0, NULL, NULL, NULL) == 0
    aq = lib.qk_quant_per_token_asym
    assert aq(4, 4, FAKE, 0, FAKE, FAKE, NULL, NULL) == INVALID   # no zero-point buffer
    assert aq(0, 4, NULL, 0, NULL, NULL, NULL, NULL) == 0
    assert lib.qk_weight_colsum(16, 4, FAKE, 3, FAKE, NULL) == INVALID
    assert lib.qk_weight_colsum(16, 4, FAKE, 0, NULL, NULL) == INVALID
    assert lib.qk_weight_colsum(16, 0, NULL, 0, NULL, NULL) == 0

    def ag(m, n, k, zp=FAKE, ws=FAKE, a=FAKE, b=FAKE, cc=FAKE, sa=FAKE, sb=FAKE, out=FAKE):
        return lib.qk_gemm_i8_asym(m, n, k, a, zp, b, ws, cc, sa, sb, 1.0, out, 0, 0, NULL)

    assert ag(4, 4, qk.MAX_K_ASYM + 17) == INVALID
    assert ag(4, 4, 24) == UNSUP
    assert ag(4, 4, 16, zp=NULL) == INVALID
    assert ag(4, 4, 16, ws=NULL) == INVALID
    assert ag(4, 4, 16, sa=NULL) == INVALID
    assert ag(4, 4, 16, a=FAKE_ODD) == UNSUP
    assert ag(0, 4, 16, a=NULL, b=NULL) == 0
