// Internal interface between the C ABI (qk_api.hip) and the kernel files.
// Nothing here is exported; every launcher returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <tuple>
#include <utility>

#include "qk.h"

namespace qk {

// Launch `kernel` with arguments converted to its exact parameter types and
// return the launch status (hipLaunchKernel reports it directly, so no
// thread-global error state is read or cleared).
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds_bytes,
                  hipStream_t stream, Args&&... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count mismatch");
  std::tuple<KArgs...> typed(std::forward<Args>(args)...);
  return std::apply(
      [&](auto&... a) {
        void* argv[] = {static_cast<void*>(&a)...};
        return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv,
                               lds_bytes, stream);
      },
      typed);
}

// Split-K plan of the tiled INT8 GEMM (gemm_mfma.hip): splits > 1 when the
// output has few tiles; `bytes` of workspace hold the INT32 partial sums.
struct SplitKPlan {
  int splits;
  int kslice;
  size_t bytes;
};
SplitKPlan splitk_plan(int m, int n, int k, int b_layout);

struct GemmArgs {
  int m, n, k;
  const int8_t* a;
  const int8_t* b;
  int32_t* c;
  const float* scale_a;
  const float* scale_b;
  float output_scale;
  void* out;
  int out_dtype;  // QK_F32 | QK_BF16 (ignored when out == nullptr)
  int b_layout;   // QK_B_KN | QK_B_NK
  void* workspace;         // optional: the split-K partial sums (zero before and after)
  size_t workspace_bytes;
};

// Sets `bytes` bytes at p (16-byte aligned) to zero with a kernel on `stream`
// (qk_api.hip); used to prepare workspaces and to clear partial sums after a
// failed launch.
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t stream);

// Per-token quantization, one workgroup per row (quant.hip).
hipError_t launch_quant_rows(int m, int k, const void* x, int dtype, int8_t* q, float* scale,
                             hipStream_t stream);
// silu(gate) * up then per-token quantization, one workgroup per row (quant.hip).
hipError_t launch_silu_quant_rows(int m, int d, const void* h, int dtype, int8_t* q,
                                  float* scale, hipStream_t stream);
// silu(gate) * up in binary32, no quantization (quant.hip).
hipError_t launch_silu_mul(int m, int d, const void* h, int dtype, float* out,
                           hipStream_t stream);
// The same two with float8_e4m3fn codes and the optional scale bound.
hipError_t launch_quant_rows_fp8(int m, int k, const void* x, int dtype, uint8_t* q, float* scale,
                                 float scale_ub, hipStream_t stream);
hipError_t launch_silu_quant_rows_fp8(int m, int d, const void* h, int dtype, uint8_t* q,
                                      float* scale, float scale_ub, hipStream_t stream);
// Asymmetric per-token INT8 codes with zero points (quant.hip).
hipError_t launch_quant_rows_asym(int m, int k, const void* x, int dtype, int8_t* q, float* scale,
                                  int32_t* zp, hipStream_t stream);
// Static (per-tensor) quantization with a device scalar scale, INT8 or FP8,
// plain or silu-fused (quant_static.hip).
hipError_t launch_quant_static(int m, int k, const void* x, int dtype, bool silu, bool fp8,
                               const float* scale, int8_t* q, hipStream_t stream);
// Column sums of an INT8 weight (quant_static.hip): wsum[j] = sum_t B(t, j).
hipError_t launch_weight_colsum(int k, int n, const int8_t* b, int b_layout, int32_t* wsum,
                                hipStream_t stream);

// LDS-tiled INT8 MFMA GEMM with fused epilogue (gemm_mfma.hip).  Operands
// are addressed with 32-bit offsets: m*k and n*k must stay below 2^32.
bool gemm_mfma_supported(int m, int n, int k);
hipError_t launch_gemm_mfma(const GemmArgs& g, hipStream_t stream);
// The same product with 256 x 256 tiles (gemm_wide.hip), for outputs with at
// least one such tile per CU; launch_gemm_mfma picks it when it applies.
bool gemm_wide_applies(int m, int n, int k, int b_layout);
hipError_t launch_gemm_wide(const GemmArgs& g, hipStream_t stream);
// The MoE grouped GEMM on those tiles (gemm_wide.hip), for groups whose
// dense GEMM of all rows would take them; launch_gemm_moe picks it.
bool gemm_wide_moe_applies(int m, int n, int k, int b_layout);
hipError_t launch_gemm_wide_moe(const GemmArgs& g, const int* offsets, int experts,
                                hipStream_t stream);
// 256 x 128 tiles with separate transfer and matrix-core waves
// (gemm_spec.hip), for the outputs the wide kernel does not take; k a
// multiple of 128, a DMA'd weight layout.
bool gemm_spec_applies(int m, int n, int k, int b_layout);
hipError_t launch_gemm_spec(const GemmArgs& g, hipStream_t stream);
hipError_t launch_gemm_spec_asym(const GemmArgs& g, const int32_t* zp_a, const int32_t* wsum,
                                 hipStream_t stream);
// The same kernel over experts (gemm_mfma.hip): rows [offsets[e],
// offsets[e + 1]) of a (device array of experts + 1 ints) use weight
// b + e * k * n and per-channel scales scale_b + e * n; one launch.
int moe_max_experts();
// The same kernel for asymmetric activations (gemm_mfma.hip): the epilogue
// subtracts zp_a[row] * wsum[col] from the INT32 accumulators.
hipError_t launch_gemm_asym(const GemmArgs& g, const int32_t* zp_a, const int32_t* wsum,
                            hipStream_t stream);
hipError_t launch_gemm_moe(const GemmArgs& g, const int* offsets, int experts, hipStream_t stream);

// GEMMs whose waves multiply whole k slices (gemm_slice.hip): the FP8
// (e4m3fn) GEMM and the INT8 GEMM with per-group weight scales, both with
// binary32 accumulation and the fused epilogue; the same tiles, layouts and
// size limits as the INT8 GEMM.
struct SliceGemmArgs {
  int m, n, k;
  const int8_t* a;  // [m][k] codes (e4m3fn bytes or int8)
  const int8_t* b;  // [k][n] or [n][k] codes
  float* c;         // raw binary32 accumulators [m][n] or nullptr
  const float* scale_a;
  const float* scale_b;  // FP8: [n]; grouped INT8: [k / group][n]
  float output_scale;
  void* out;
  int out_dtype;  // QK_F32 | QK_BF16 (ignored when out == nullptr)
  int b_layout;   // QK_B_KN | QK_B_NK
};
hipError_t launch_gemm_fp8(const SliceGemmArgs& g, hipStream_t stream);
// group 64 or 128; k a multiple of group
hipError_t launch_gemm_i8_grouped(const SliceGemmArgs& g, int group, hipStream_t stream);

// Split-K decode GEMV (gemv.hip): m <= kGemvMaxRows rows per launch, larger m
// in row groups; exact partial sums with arrival counts in a self-cleaning
// workspace of 64-bit words.
constexpr int kGemvMaxRows = 8;
constexpr int kGemvMaxM = 16;
struct GemvArgs {
  int m, n, k;
  const void* a;   // int8 codes [m][k] (x_dtype == -1) or activations of x_dtype
  int x_dtype;
  const int8_t* b;  // [k][n]
  int32_t* c;
  const float* scale_a;  // codes' scales (x_dtype == -1)
  const float* scale_b;
  float output_scale;
  void* out;
  int out_dtype;
  int8_t* q_out;   // optional codes written by the fused path
  float* s_out;    // optional scales written by the fused path
  void* workspace; // gemv_workspace_bytes(n), zero before the first call
};
size_t gemv_workspace_bytes(int n);
hipError_t launch_gemv(const GemvArgs& g, hipStream_t stream);

}  // namespace qk
