// C ABI of libqk: argument validation, kernel choice by shape, launches on the
// caller's stream.  Declarations and the contract of each call are in qk.h.
#include <cstdint>
#include <mutex>

#include "qk_internal.h"

#define QK_STR2(x) #x
#define QK_STR(x) QK_STR2(x)

namespace qk {
namespace {

// 16 bytes per lane, grid-stride; the last (bytes % 16) bytes one per thread
// of the first workgroup.
__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* __restrict__ p, size_t n16,
                                                        unsigned char* __restrict__ tail,
                                                        unsigned ntail) {
  const size_t stride = static_cast<size_t>(gridDim.x) * 256;
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

}  // namespace

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  const size_t n16 = bytes / 16;
  const unsigned ntail = static_cast<unsigned>(bytes % 16);
  const size_t want = (n16 + 255) / 256;
  const unsigned blocks = static_cast<unsigned>(want == 0 ? 1 : (want < 4096 ? want : 4096));
  return launch(zero_fill_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<uint4*>(p), n16,
                static_cast<unsigned char*>(p) + n16 * 16, ntail);
}

}  // namespace qk

namespace {

bool aligned(const void* p, uintptr_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; }

bool known_input_dtype(int dt) { return dt == QK_F32 || dt == QK_BF16 || dt == QK_F16; }

int status_of(hipError_t e) { return e == hipSuccess ? QK_OK : static_cast<int>(e); }

bool workspace_ok(const void* ws, size_t bytes, int n) {
  return ws && aligned(ws, 256) && bytes >= qk::gemv_workspace_bytes(n);
}

int check_rows(int m, int k, const void* src, const void* q, const void* scale, int dtype) {
  if (m < 0 || k < 0) return QK_ERR_INVALID_VALUE;
  if (!known_input_dtype(dtype)) return QK_ERR_INVALID_VALUE;
  if (m > 0 && (!scale || (k > 0 && (!src || !q)))) return QK_ERR_INVALID_VALUE;
  return QK_OK;
}

int gemm_common(int m, int n, int k, const int8_t* a, const int8_t* b, int32_t* c,
                const float* scale_a, const float* scale_b, float output_scale, void* out,
                int out_dtype, int b_layout, void* workspace, size_t workspace_bytes, int kernel,
                hipStream_t stream) {
  if (m < 0 || n < 0 || k < 0 || k > QK_MAX_K) return QK_ERR_INVALID_VALUE;
  if (b_layout != QK_B_KN && b_layout != QK_B_NK) return QK_ERR_INVALID_VALUE;
  if (kernel != QK_KERNEL_AUTO && kernel != QK_KERNEL_MFMA && kernel != QK_KERNEL_GEMV)
    return QK_ERR_INVALID_VALUE;
  if (k % 16 != 0) return QK_ERR_UNSUPPORTED;
  if (m == 0 || n == 0) return QK_OK;  // empty tensors may have NULL data pointers
  if (!c && !out) return QK_ERR_INVALID_VALUE;
  if (out && out_dtype != QK_F32 && out_dtype != QK_BF16) return QK_ERR_INVALID_VALUE;
  if (k > 0 && (!a || !b)) return QK_ERR_INVALID_VALUE;
  if (out && (!scale_a || !scale_b)) return QK_ERR_INVALID_VALUE;
  if (!aligned(a, 16) || !aligned(b, 16)) return QK_ERR_UNSUPPORTED;
  if (c && !aligned(c, 4)) return QK_ERR_UNSUPPORTED;
  if (out && !aligned(out, out_dtype == QK_BF16 ? 2 : 4)) return QK_ERR_UNSUPPORTED;

  bool gemv;
  if (kernel == QK_KERNEL_GEMV) {
    if (m > qk::kGemvMaxM || b_layout != QK_B_KN) return QK_ERR_UNSUPPORTED;
    gemv = true;
  } else if (kernel == QK_KERNEL_MFMA) {
    gemv = false;
  } else {
    gemv = m <= qk::kGemvMaxRows && b_layout == QK_B_KN;
  }
  if (gemv) {
    if (!workspace_ok(workspace, workspace_bytes, n)) return QK_ERR_WORKSPACE;
    qk::GemvArgs g{m, n, k, a, -1, b, c, scale_a, scale_b, output_scale, out, out_dtype, nullptr,
                   nullptr, workspace};
    return status_of(qk::launch_gemv(g, stream));
  }
  if (!qk::gemm_mfma_supported(m, n, k)) return QK_ERR_UNSUPPORTED;
  // the workspace, when given, lets an output with few tiles split k
  const bool ws = workspace && aligned(workspace, 256);
  qk::GemmArgs g{m, n, k, a, b, c, scale_a, scale_b, output_scale, out, out_dtype, b_layout,
                 ws ? workspace : nullptr, ws ? workspace_bytes : 0};
  return status_of(qk::launch_gemm_mfma(g, stream));
}

// Host checks of the whole-layer call (both entry points).  On QK_OK, *noop
// tells that there is nothing to do (m or n is 0) and *fused which path runs:
// the single decode launch or quantization + tiled GEMM.
int linear_check(int m, int n, int k, const void* x, int x_dtype, const int8_t* b,
                 const float* scale_b, const void* out, int out_dtype, int b_layout,
                 const int8_t* q_out, const float* scale_out, const int32_t* c_out, int kernel,
                 bool* fused, bool* noop) {
  if (m < 0 || n < 0 || k < 0 || k > QK_MAX_K) return QK_ERR_INVALID_VALUE;
  if (!known_input_dtype(x_dtype)) return QK_ERR_INVALID_VALUE;
  if (b_layout != QK_B_KN && b_layout != QK_B_NK) return QK_ERR_INVALID_VALUE;
  if (kernel != QK_KERNEL_AUTO && kernel != QK_KERNEL_MFMA && kernel != QK_KERNEL_GEMV)
    return QK_ERR_INVALID_VALUE;
  if (out && out_dtype != QK_F32 && out_dtype != QK_BF16) return QK_ERR_INVALID_VALUE;
  if (k % 16 != 0) return QK_ERR_UNSUPPORTED;
  *noop = m == 0 || n == 0;
  if (*noop) return QK_OK;
  if (!out && !c_out) return QK_ERR_INVALID_VALUE;
  if ((out && !scale_b) || (k > 0 && (!x || !b))) return QK_ERR_INVALID_VALUE;
  if (!aligned(b, 16) || !aligned(x, x_dtype == QK_F32 ? 4 : 2)) return QK_ERR_UNSUPPORTED;
  if (out && !aligned(out, out_dtype == QK_BF16 ? 2 : 4)) return QK_ERR_UNSUPPORTED;
  if (c_out && !aligned(c_out, 4)) return QK_ERR_UNSUPPORTED;
  if (q_out && !aligned(q_out, 16)) return QK_ERR_UNSUPPORTED;
  if (scale_out && !aligned(scale_out, 4)) return QK_ERR_UNSUPPORTED;

  if (kernel == QK_KERNEL_GEMV) {
    if (m > qk::kGemvMaxM || b_layout != QK_B_KN) return QK_ERR_UNSUPPORTED;
    *fused = true;
  } else if (kernel == QK_KERNEL_MFMA) {
    *fused = false;
  } else {
    *fused = m <= qk::kGemvMaxRows && b_layout == QK_B_KN;
  }
  if (*fused && !aligned(x, 16)) {
    if (kernel == QK_KERNEL_GEMV) return QK_ERR_UNSUPPORTED;
    *fused = false;  // the fused launch reads x with 128-bit loads
  }
  if (!*fused) {
    // two launches: the codes and scales go through q_out / scale_out
    if (!q_out || !scale_out) return QK_ERR_INVALID_VALUE;
    if (!qk::gemm_mfma_supported(m, n, k)) return QK_ERR_UNSUPPORTED;
  }
  return QK_OK;
}

// Enqueues a checked whole-layer call; the workspace (valid and large enough
// for the decode launch when `fused`) lets the tiled GEMM split k when its
// partial sums fit.
int linear_launch(int m, int n, int k, const void* x, int x_dtype, const int8_t* b,
                  const float* scale_b, float output_scale, void* out, int out_dtype,
                  int b_layout, int8_t* q_out, float* scale_out, int32_t* c_out, bool fused,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (fused) {
    qk::GemvArgs g{m, n, k, x, x_dtype, b, c_out, nullptr, scale_b, output_scale, out,
                   out_dtype, q_out, scale_out, workspace};
    return status_of(qk::launch_gemv(g, stream));
  }
  hipError_t e = qk::launch_quant_rows(m, k, x, x_dtype, q_out, scale_out, stream);
  if (e != hipSuccess) return status_of(e);
  const bool ws = workspace && aligned(workspace, 256);
  qk::GemmArgs g{m, n, k, q_out, b, c_out, scale_out, scale_b, output_scale, out, out_dtype,
                 b_layout, ws ? workspace : nullptr, ws ? workspace_bytes : 0};
  return status_of(qk::launch_gemm_mfma(g, stream));
}

// ---- static scratch of qk_linear_w8a8_noalloc ----
// The memory the no-allocation entry point uses in place of a caller's
// workspace: a file-scope device array, one copy per GPU, held until the
// process ends.  Its name is a host-side stand-in in host code, so the device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is ever passed to kernels.  The first call
// on a device, and the first call after a failed launch, clear it on the
// caller's stream before using it (a kernel, so that a captured call stays
// valid); every successful call leaves it all zeros again.
constexpr size_t kScratchBytes = QK_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  void* ptr = nullptr;    // device address of `scratch` on this device
  bool needs_clear = true;
};
std::mutex g_scratch_mutex;
ScratchSlot g_scratch[kMaxDevices];

hipError_t scratch_for_call(hipStream_t stream, int* dev, void** ptr) {
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return e;
  if (*dev < 0 || *dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  ScratchSlot& slot = g_scratch[*dev];
  if (!slot.ptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    slot.ptr = p;
  }
  if (slot.needs_clear) {
    e = qk::launch_zero_fill(slot.ptr, kScratchBytes, stream);
    if (e != hipSuccess) return e;
    slot.needs_clear = false;
  }
  *ptr = slot.ptr;
  return hipSuccess;
}

void scratch_mark_dirty(int dev) {
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  g_scratch[dev].needs_clear = true;
}

}  // namespace

extern "C" {

int qk_abi_version(void) { return QK_ABI_VERSION; }

const char* qk_status_string(int status) {
  switch (status) {
    case QK_OK: return "QK_OK: success";
    case QK_ERR_INVALID_VALUE:
      return "QK_ERR_INVALID_VALUE: negative size, NULL pointer, or unknown dtype/layout/kernel";
    case QK_ERR_UNSUPPORTED:
      return "QK_ERR_UNSUPPORTED: k not a multiple of 16, misaligned pointer, or kernel/shape "
             "combination not provided";
    case QK_ERR_WORKSPACE:
      return "QK_ERR_WORKSPACE: workspace missing, misaligned, or smaller than "
             "qk_gemm_workspace_size()";
    case QK_ERR_SCRATCH_LIMIT:
      return "QK_ERR_SCRATCH_LIMIT: the call needs more than the QK_SCRATCH_BYTES of static "
             "scratch that qk_linear_w8a8_noalloc uses (the decode launch needs 64 bytes per "
             "output column)";
    default: return hipGetErrorString(static_cast<hipError_t>(status));
  }
}

const char* qk_build_info(void) {
  return "libqk ABI " QK_STR(QK_ABI_VERSION) "; code objects: gfx950; HIP " QK_STR(
      HIP_VERSION_MAJOR) "." QK_STR(HIP_VERSION_MINOR) "." QK_STR(HIP_VERSION_PATCH) "; built " __DATE__
                                                                                       " " __TIME__;
}

int qk_quant_per_token(int m, int k, const void* x, int x_dtype, int8_t* q, float* scale,
                       hipStream_t stream) {
  const int rc = check_rows(m, k, x, q, scale, x_dtype);
  if (rc != QK_OK || m == 0) return rc;
  return status_of(qk::launch_quant_rows(m, k, x, x_dtype, q, scale, stream));
}

int qk_silu_mul_quant_per_token(int m, int d, const void* h, int h_dtype, int8_t* q,
                                float* scale, hipStream_t stream) {
  const int rc = check_rows(m, d, h, q, scale, h_dtype);
  if (rc != QK_OK || m == 0) return rc;
  if (static_cast<long long>(d) * 2 > 0x7fffffffLL) return QK_ERR_UNSUPPORTED;
  return status_of(qk::launch_silu_quant_rows(m, d, h, h_dtype, q, scale, stream));
}

int qk_silu_mul(int m, int d, const void* h, int h_dtype, float* out, hipStream_t stream) {
  if (m < 0 || d < 0 || !known_input_dtype(h_dtype)) return QK_ERR_INVALID_VALUE;
  if (m == 0 || d == 0) return QK_OK;  // empty tensors may have NULL data pointers
  if (!h || !out) return QK_ERR_INVALID_VALUE;
  if (static_cast<long long>(d) * 2 > 0x7fffffffLL) return QK_ERR_UNSUPPORTED;
  return status_of(qk::launch_silu_mul(m, d, h, h_dtype, out, stream));
}

size_t qk_gemm_workspace_size(int m, int n, int k) {
  if (m <= 0 || n <= 0 || k < 0) return 0;
  // the decode kernel's words (m <= 16), and the tiled kernel's split-K
  // partial sums when the output has few tiles (the plan is the same for
  // either weight layout)
  const size_t gemv = m <= qk::kGemvMaxM ? qk::gemv_workspace_bytes(n) : 0;
  const size_t split = qk::splitk_plan(m, n, k, QK_B_KN).bytes;
  return gemv > split ? gemv : split;
}

int qk_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (workspace_bytes == 0) return QK_OK;
  if (!workspace) return QK_ERR_INVALID_VALUE;
  if (!aligned(workspace, 256)) return QK_ERR_WORKSPACE;
  return status_of(qk::launch_zero_fill(workspace, workspace_bytes, stream));
}

int qk_gemm_i8_scaled(int m, int n, int k, const int8_t* a, const int8_t* b, int32_t* c,
                      const float* scale_a, const float* scale_b, float output_scale, void* out,
                      int out_dtype, int b_layout, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  return gemm_common(m, n, k, a, b, c, scale_a, scale_b, output_scale, out, out_dtype, b_layout,
                     workspace, workspace_bytes, QK_KERNEL_AUTO, stream);
}

int qk_gemm_i8_scaled_ex(int m, int n, int k, const int8_t* a, const int8_t* b, int32_t* c,
                         const float* scale_a, const float* scale_b, float output_scale,
                         void* out, int out_dtype, int b_layout, void* workspace,
                         size_t workspace_bytes, int kernel, hipStream_t stream) {
  return gemm_common(m, n, k, a, b, c, scale_a, scale_b, output_scale, out, out_dtype, b_layout,
                     workspace, workspace_bytes, kernel, stream);
}

int qk_linear_w8a8(int m, int n, int k, const void* x, int x_dtype, const int8_t* b,
                   const float* scale_b, float output_scale, void* out, int out_dtype,
                   int b_layout, int8_t* q_out, float* scale_out, int32_t* c_out,
                   void* workspace, size_t workspace_bytes, int kernel, hipStream_t stream) {
  bool fused = false, noop = false;
  const int rc = linear_check(m, n, k, x, x_dtype, b, scale_b, out, out_dtype, b_layout, q_out,
                              scale_out, c_out, kernel, &fused, &noop);
  if (rc != QK_OK || noop) return rc;
  if (fused && !workspace_ok(workspace, workspace_bytes, n)) return QK_ERR_WORKSPACE;
  return linear_launch(m, n, k, x, x_dtype, b, scale_b, output_scale, out, out_dtype, b_layout,
                       q_out, scale_out, c_out, fused, workspace, workspace_bytes, stream);
}

int qk_linear_w8a8_noalloc(int m, int n, int k, const void* x, int x_dtype, const int8_t* b,
                           const float* scale_b, float output_scale, void* out, int out_dtype,
                           int b_layout, int8_t* q_out, float* scale_out, int32_t* c_out,
                           int kernel, hipStream_t stream) {
  bool fused = false, noop = false;
  const int rc = linear_check(m, n, k, x, x_dtype, b, scale_b, out, out_dtype, b_layout, q_out,
                              scale_out, c_out, kernel, &fused, &noop);
  if (rc != QK_OK || noop) return rc;
  // the decode launch needs its words; the tiled GEMM splits k only when its
  // partial sums fit, and otherwise runs unsplit
  if (fused && qk::gemv_workspace_bytes(n) > kScratchBytes) return QK_ERR_SCRATCH_LIMIT;
  int dev = 0;
  void* ptr = nullptr;
  hipError_t e = scratch_for_call(stream, &dev, &ptr);
  if (e != hipSuccess) return status_of(e);
  const int st = linear_launch(m, n, k, x, x_dtype, b, scale_b, output_scale, out, out_dtype,
                               b_layout, q_out, scale_out, c_out, fused, ptr, kScratchBytes, stream);
  if (st != QK_OK) scratch_mark_dirty(dev);  // a launch failed after others may have run
  return st;
}

int qk_quant_per_token_fp8(int m, int k, const void* x, int x_dtype, float scale_ub, uint8_t* q,
                           float* scale, hipStream_t stream) {
  const int rc = check_rows(m, k, x, q, scale, x_dtype);
  if (rc != QK_OK) return rc;
  if (scale_ub != scale_ub) return QK_ERR_INVALID_VALUE;  // NaN bound
  if (m == 0) return QK_OK;
  return status_of(qk::launch_quant_rows_fp8(m, k, x, x_dtype, q, scale, scale_ub, stream));
}

int qk_silu_mul_quant_per_token_fp8(int m, int d, const void* h, int h_dtype, float scale_ub,
                                    uint8_t* q, float* scale, hipStream_t stream) {
  const int rc = check_rows(m, d, h, q, scale, h_dtype);
  if (rc != QK_OK) return rc;
  if (scale_ub != scale_ub) return QK_ERR_INVALID_VALUE;
  if (m == 0) return QK_OK;
  if (static_cast<long long>(d) * 2 > 0x7fffffffLL) return QK_ERR_UNSUPPORTED;
  return status_of(qk::launch_silu_quant_rows_fp8(m, d, h, h_dtype, q, scale, scale_ub, stream));
}

int qk_gemm_fp8_scaled(int m, int n, int k, const uint8_t* a, const uint8_t* b, float* c,
                       const float* scale_a, const float* scale_b, float output_scale, void* out,
                       int out_dtype, int b_layout, hipStream_t stream) {
  if (m < 0 || n < 0 || k < 0 || k > QK_MAX_K) return QK_ERR_INVALID_VALUE;
  if (b_layout != QK_B_KN && b_layout != QK_B_NK) return QK_ERR_INVALID_VALUE;
  if (k % 16 != 0) return QK_ERR_UNSUPPORTED;
  if (m == 0 || n == 0) return QK_OK;
  if (!c && !out) return QK_ERR_INVALID_VALUE;
  if (out && out_dtype != QK_F32 && out_dtype != QK_BF16) return QK_ERR_INVALID_VALUE;
  if (k > 0 && (!a || !b)) return QK_ERR_INVALID_VALUE;
  if (out && (!scale_a || !scale_b)) return QK_ERR_INVALID_VALUE;
  if (!aligned(a, 16) || !aligned(b, 16)) return QK_ERR_UNSUPPORTED;
  if (c && !aligned(c, 4)) return QK_ERR_UNSUPPORTED;
  if (out && !aligned(out, out_dtype == QK_BF16 ? 2 : 4)) return QK_ERR_UNSUPPORTED;
  if (!qk::gemm_mfma_supported(m, n, k)) return QK_ERR_UNSUPPORTED;
  qk::SliceGemmArgs g{m, n, k, reinterpret_cast<const int8_t*>(a), reinterpret_cast<const int8_t*>(b),
                      c, scale_a, scale_b, output_scale, out, out_dtype, b_layout};
  return status_of(qk::launch_gemm_fp8(g, stream));
}

int qk_linear_fp8(int m, int n, int k, const void* x, int x_dtype, float scale_ub,
                  const uint8_t* b, const float* scale_b, float output_scale, void* out,
                  int out_dtype, int b_layout, uint8_t* q_out, float* scale_out,
                  hipStream_t stream) {
  if (m < 0 || n < 0 || k < 0 || k > QK_MAX_K) return QK_ERR_INVALID_VALUE;
  if (!known_input_dtype(x_dtype)) return QK_ERR_INVALID_VALUE;
  if (b_layout != QK_B_KN && b_layout != QK_B_NK) return QK_ERR_INVALID_VALUE;
  if (out_dtype != QK_F32 && out_dtype != QK_BF16) return QK_ERR_INVALID_VALUE;
  if (scale_ub != scale_ub) return QK_ERR_INVALID_VALUE;
  if (k % 16 != 0) return QK_ERR_UNSUPPORTED;
  if (m == 0 || n == 0) return QK_OK;
  if (!out || !scale_b || !q_out || !scale_out || (k > 0 && (!x || !b)))
    return QK_ERR_INVALID_VALUE;
  if (!aligned(b, 16) || !aligned(q_out, 16) || !aligned(scale_out, 4)) return QK_ERR_UNSUPPORTED;
  if (!aligned(x, x_dtype == QK_F32 ? 4 : 2)) return QK_ERR_UNSUPPORTED;
  if (!aligned(out, out_dtype == QK_BF16 ? 2 : 4)) return QK_ERR_UNSUPPORTED;
  if (!qk::gemm_mfma_supported(m, n, k)) return QK_ERR_UNSUPPORTED;
  hipError_t e = qk::launch_quant_rows_fp8(m, k, x, x_dtype, q_out, scale_out, scale_ub, stream);
  if (e != hipSuccess) return status_of(e);
  qk::SliceGemmArgs g{m, n, k, reinterpret_cast<const int8_t*>(q_out),
                      reinterpret_cast<const int8_t*>(b), nullptr, scale_out, scale_b, output_scale,
                      out, out_dtype, b_layout};
  return status_of(qk::launch_gemm_fp8(g, stream));
}

int qk_gemm_i8_grouped(int m, int n, int k, int group, const int8_t* a, const int8_t* b, float* c,
                       const float* scale_a, const float* scale_b, float output_scale, void* out,
                       int out_dtype, int b_layout, hipStream_t stream) {
  if (m < 0 || n < 0 || k < 0 || k > QK_MAX_K) return QK_ERR_INVALID_VALUE;
  if (b_layout != QK_B_KN && b_layout != QK_B_NK) return QK_ERR_INVALID_VALUE;
  if (group != 64 && group != 128) return QK_ERR_UNSUPPORTED;
  if (k % group != 0) return QK_ERR_UNSUPPORTED;
  if (m == 0 || n == 0) return QK_OK;
  if (!c && !out) return QK_ERR_INVALID_VALUE;
  if (out && out_dtype != QK_F32 && out_dtype != QK_BF16) return QK_ERR_INVALID_VALUE;
  if (k > 0 && (!a || !b || !scale_b)) return QK_ERR_INVALID_VALUE;
  if (out && !scale_a) return QK_ERR_INVALID_VALUE;
  if (!aligned(a, 16) || !aligned(b, 16) || (scale_b && !aligned(scale_b, 4)))
    return QK_ERR_UNSUPPORTED;
  if (c && !aligned(c, 4)) return QK_ERR_UNSUPPORTED;
  if (out && !aligned(out, out_dtype == QK_BF16 ? 2 : 4)) return QK_ERR_UNSUPPORTED;
  if (!qk::gemm_mfma_supported(m, n, k)) return QK_ERR_UNSUPPORTED;
  qk::SliceGemmArgs g{m, n, k, a, b, c, scale_a, scale_b, output_scale, out, out_dtype, b_layout};
  return status_of(qk::launch_gemm_i8_grouped(g, group, stream));
}

int qk_moe_gemm_i8_scaled(int experts, int m, int n, int k, const int* expert_offsets,
                          const int8_t* a, const int8_t* b, int32_t* c, const float* scale_a,
                          const float* scale_b, float output_scale, void* out, int out_dtype,
                          int b_layout, hipStream_t stream) {
  if (experts < 1 || experts > qk::moe_max_experts()) return QK_ERR_INVALID_VALUE;
  if (m < 0 || n < 0 || k < 0 || k > QK_MAX_K) return QK_ERR_INVALID_VALUE;
  if (b_layout != QK_B_KN && b_layout != QK_B_NK) return QK_ERR_INVALID_VALUE;
  if (k % 16 != 0) return QK_ERR_UNSUPPORTED;
  if (m == 0 || n == 0) return QK_OK;
  if (!expert_offsets || (!c && !out)) return QK_ERR_INVALID_VALUE;
  if (out && out_dtype != QK_F32 && out_dtype != QK_BF16) return QK_ERR_INVALID_VALUE;
  if (k > 0 && (!a || !b)) return QK_ERR_INVALID_VALUE;
  if (out && (!scale_a || !scale_b)) return QK_ERR_INVALID_VALUE;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(expert_offsets, 4)) return QK_ERR_UNSUPPORTED;
  if (c && !aligned(c, 4)) return QK_ERR_UNSUPPORTED;
  if (out && !aligned(out, out_dtype == QK_BF16 ? 2 : 4)) return QK_ERR_UNSUPPORTED;
  if (!qk::gemm_mfma_supported(m, n, k)) return QK_ERR_UNSUPPORTED;
  // k % 16 == 0 keeps every expert's weight (k n bytes apart) and every row
  // group's codes 16-byte aligned
  qk::GemmArgs g{m, n, k, a, b, c, scale_a, scale_b, output_scale, out, out_dtype, b_layout,
                 nullptr, 0};
  return status_of(qk::launch_gemm_moe(g, expert_offsets, experts, stream));
}

static int quant_static_common(int m, int k, const void* x, int x_dtype, const float* scale,
                               void* q, bool silu, bool fp8, hipStream_t stream) {
  const int rc = check_rows(m, k, x, q, scale, x_dtype);
  if (rc != QK_OK || m == 0 || k == 0) return rc;
  if (silu && static_cast<long long>(k) * 2 > 0x7fffffffLL) return QK_ERR_UNSUPPORTED;
  return status_of(qk::launch_quant_static(m, k, x, x_dtype, silu, fp8, scale,
                                           static_cast<int8_t*>(q), stream));
}

int qk_quant_static(int m, int k, const void* x, int x_dtype, const float* scale, int8_t* q,
                    hipStream_t stream) {
  return quant_static_common(m, k, x, x_dtype, scale, q, false, false, stream);
}

int qk_silu_mul_quant_static(int m, int d, const void* h, int h_dtype, const float* scale,
                             int8_t* q, hipStream_t stream) {
  return quant_static_common(m, d, h, h_dtype, scale, q, true, false, stream);
}

int qk_quant_static_fp8(int m, int k, const void* x, int x_dtype, const float* scale, uint8_t* q,
                        hipStream_t stream) {
  return quant_static_common(m, k, x, x_dtype, scale, q, false, true, stream);
}

int qk_silu_mul_quant_static_fp8(int m, int d, const void* h, int h_dtype, const float* scale,
                                 uint8_t* q, hipStream_t stream) {
  return quant_static_common(m, d, h, h_dtype, scale, q, true, true, stream);
}

int qk_quant_per_token_asym(int m, int k, const void* x, int x_dtype, int8_t* q, float* scale,
                            int32_t* zero_point, hipStream_t stream) {
  const int rc = check_rows(m, k, x, q, scale, x_dtype);
  if (rc != QK_OK) return rc;
  if (m > 0 && !zero_point) return QK_ERR_INVALID_VALUE;
  if (m == 0) return QK_OK;
  return status_of(qk::launch_quant_rows_asym(m, k, x, x_dtype, q, scale, zero_point, stream));
}

int qk_weight_colsum(int k, int n, const int8_t* b, int b_layout, int32_t* wsum, hipStream_t stream) {
  if (k < 0 || n < 0 || k > QK_MAX_K) return QK_ERR_INVALID_VALUE;
  if (b_layout != QK_B_KN && b_layout != QK_B_NK) return QK_ERR_INVALID_VALUE;
  if (n == 0) return QK_OK;
  if (!wsum || (k > 0 && !b)) return QK_ERR_INVALID_VALUE;
  return status_of(qk::launch_weight_colsum(k, n, b, b_layout, wsum, stream));
}

int qk_gemm_i8_asym(int m, int n, int k, const int8_t* a, const int32_t* zero_point,
                    const int8_t* b, const int32_t* wsum, int32_t* c, const float* scale_a,
                    const float* scale_b, float output_scale, void* out, int out_dtype,
                    int b_layout, hipStream_t stream) {
  if (m < 0 || n < 0 || k < 0 || k > QK_MAX_K_ASYM) return QK_ERR_INVALID_VALUE;
  if (b_layout != QK_B_KN && b_layout != QK_B_NK) return QK_ERR_INVALID_VALUE;
  if (k % 16 != 0) return QK_ERR_UNSUPPORTED;
  if (m == 0 || n == 0) return QK_OK;
  if (!c && !out) return QK_ERR_INVALID_VALUE;
  if (!zero_point || !wsum) return QK_ERR_INVALID_VALUE;
  if (out && out_dtype != QK_F32 && out_dtype != QK_BF16) return QK_ERR_INVALID_VALUE;
  if (k > 0 && (!a || !b)) return QK_ERR_INVALID_VALUE;
  if (out && (!scale_a || !scale_b)) return QK_ERR_INVALID_VALUE;
  if (!aligned(a, 16) || !aligned(b, 16)) return QK_ERR_UNSUPPORTED;
  if (c && !aligned(c, 4)) return QK_ERR_UNSUPPORTED;
  if (out && !aligned(out, out_dtype == QK_BF16 ? 2 : 4)) return QK_ERR_UNSUPPORTED;
  if (!qk::gemm_mfma_supported(m, n, k)) return QK_ERR_UNSUPPORTED;
  qk::GemmArgs g{m, n, k, a, b, c, scale_a, scale_b, output_scale, out, out_dtype, b_layout,
                 nullptr, 0};
  return status_of(qk::launch_gemm_asym(g, zero_point, wsum, stream));
}

}  // extern "C"
