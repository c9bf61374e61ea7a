// Static (per-tensor) quantization and weight column sums for gfx950.
//
// Static scale ("kernels: fused silu_and_mul + dynamic per-token FP8
// quantization", Purpose: silu_and_mul_quant quantizes with one
// pre-calibrated scale for the whole tensor):
//   INT8: code = clamp(rint(x / scale), -127, 127);   FP8: code = e4m3fn(x / scale)
// optionally of silu(gate) * up.  No row reduction, so the kernel streams:
// each thread converts 16-byte units (a row's units are contiguous), reading
// the input once and writing the codes once.  The scale comes from device
// memory (a calibration result need not visit the host); every thread forms
// r = RN(1 / scale) itself, and the exact quotient by the same correction as
// the dynamic kernels.
//
// Weight column sums, wsum[j] = sum_t B(t, j), once per weight: the
// zero-point correction of the asymmetric GEMM.
#include "quant_math.h"

namespace qk {
namespace {

using qm::Elem;
using qm::silu_times;

constexpr int kBlock = 256;

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

template <bool FP8>
__device__ __forceinline__ uint32_t codes4(float a, float b, float c, float d, float s, float r) {
  if constexpr (FP8) {
    return qm::pack4_fp8(qm::fp8_ratio(a, s, r), qm::fp8_ratio(b, s, r), qm::fp8_ratio(c, s, r),
                         qm::fp8_ratio(d, s, r));
  } else {
    return qm::pack4_low_bytes(qm::code_word_bounded(a, s, r), qm::code_word_bounded(b, s, r),
                               qm::code_word_bounded(c, s, r), qm::code_word_bounded(d, s, r));
  }
}

constexpr int kUnitsPerThread = 2;

// 16-byte units of P values (rows of k / P units; for SILU the up half of row
// i starts k elements after its gate half), kUnitsPerThread per thread and
// iteration: a wave's loads cover 64 consecutive units each, and all of a
// thread's loads are issued before any unit is converted, so one round of
// waves keeps the whole tensor's reads in flight.  Without SILU the units of
// the input and of the codes are both contiguous (unit u at byte 16 u and at
// code P u), so no row index is needed.
template <int DT, bool SILU, bool FP8>
__global__ __launch_bounds__(kBlock) void quant_static_units(const void* __restrict__ src,
                                                             int8_t* __restrict__ q,
                                                             const float* __restrict__ scale,
                                                             long long units, int units_per_row) {
  using E = Elem<DT>;
  constexpr int P = E::kPerUnit;
  constexpr int U = kUnitsPerThread;
  const float s = *scale;
  const float r = 1.0f / s;
  const char* in = static_cast<const char*>(src);
  const long long stride = static_cast<long long>(gridDim.x) * kBlock;
  for (long long u0 = static_cast<long long>(blockIdx.x) * kBlock + threadIdx.x; u0 < units;
       u0 += U * stride) {
    v4u raw[U], rup[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const long long u = u0 + j * stride;
      if (u >= units) continue;
      long long at = u;  // the unit's index in the input, in units
      if constexpr (SILU) {
        const long long row = units <= 0x7fffffffLL
                                  ? static_cast<long long>(static_cast<uint32_t>(u) /
                                                           static_cast<uint32_t>(units_per_row))
                                  : u / units_per_row;
        at = u + row * units_per_row;
        rup[j] = __builtin_nontemporal_load(
            reinterpret_cast<const v4u*>(in + (at + units_per_row) * 16));
      }
      raw[j] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(in + at * 16));
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const long long u = u0 + j * stride;
      if (u >= units) continue;
      float v[P];
      E::unpack(make_uint4(raw[j].x, raw[j].y, raw[j].z, raw[j].w), v);
      if constexpr (SILU) {
        float up[P];
        E::unpack(make_uint4(rup[j].x, rup[j].y, rup[j].z, rup[j].w), up);
#pragma unroll
        for (int e = 0; e < P; ++e) v[e] = silu_times<DT != QK_F32>(v[e], up[e]);
      }
      int8_t* dst = q + u * P;
      if constexpr (P == 8) {
        *reinterpret_cast<v2u*>(dst) =
            v2u{codes4<FP8>(v[0], v[1], v[2], v[3], s, r), codes4<FP8>(v[4], v[5], v[6], v[7], s, r)};
      } else {
        *reinterpret_cast<uint32_t*>(dst) = codes4<FP8>(v[0], v[1], v[2], v[3], s, r);
      }
    }
  }
}

// Any k or alignment: one thread per element.
template <int DT, bool SILU, bool FP8>
__global__ __launch_bounds__(kBlock) void quant_static_elems(const void* __restrict__ src,
                                                             int8_t* __restrict__ q,
                                                             const float* __restrict__ scale,
                                                             long long count, int k) {
  using E = Elem<DT>;
  const float s = *scale;
  const float r = 1.0f / s;
  for (long long i = static_cast<long long>(blockIdx.x) * kBlock + threadIdx.x; i < count;
       i += static_cast<long long>(gridDim.x) * kBlock) {
    const long long row = i / k;
    const long long j = i - row * k;
    const long long first = row * static_cast<long long>(SILU ? 2 : 1) * k;
    float x = E::load(src, first + j);
    if constexpr (SILU) x = silu_times<DT != QK_F32>(x, E::load(src, first + k + j));
    if constexpr (FP8) {
      q[i] = static_cast<int8_t>(
          __builtin_amdgcn_cvt_pk_fp8_f32(qm::fp8_ratio(x, s, r), 0.0f, 0, false) & 0xff);
    } else {
      q[i] = static_cast<int8_t>(qm::code_of_bounded(x, s, r));
    }
  }
}

unsigned grid_for(long long items) {
  const long long blocks = (items + kBlock - 1) / kBlock;
  return static_cast<unsigned>(blocks < 65536 ? (blocks > 0 ? blocks : 1) : 65536);
}

template <int DT, bool SILU, bool FP8>
hipError_t dispatch_static(int m, int k, const void* src, const float* scale, int8_t* q,
                           hipStream_t stream) {
  using E = Elem<DT>;
  const bool aligned = reinterpret_cast<uintptr_t>(src) % 16 == 0 &&
                       reinterpret_cast<uintptr_t>(q) % E::kPerUnit == 0 && k % E::kPerUnit == 0;
  if (aligned) {
    const int upr = k / E::kPerUnit;
    const long long units = static_cast<long long>(m) * upr;
    return launch(quant_static_units<DT, SILU, FP8>,
                  dim3(grid_for((units + kUnitsPerThread - 1) / kUnitsPerThread)), dim3(kBlock), 0,
                  stream, src, q, scale, units, upr);
  }
  const long long count = static_cast<long long>(m) * k;
  return launch(quant_static_elems<DT, SILU, FP8>, dim3(grid_for(count)), dim3(kBlock), 0, stream,
                src, q, scale, count, k);
}

template <bool SILU, bool FP8>
hipError_t static_dtype(int m, int k, const void* src, int dtype, const float* scale, int8_t* q,
                        hipStream_t stream) {
  switch (dtype) {
    case QK_F32: return dispatch_static<QK_F32, SILU, FP8>(m, k, src, scale, q, stream);
    case QK_BF16: return dispatch_static<QK_BF16, SILU, FP8>(m, k, src, scale, q, stream);
    case QK_F16: return dispatch_static<QK_F16, SILU, FP8>(m, k, src, scale, q, stream);
    default: return hipErrorInvalidValue;
  }
}

// [K][N] weight: workgroup (x, y) sums rows [y * kColsumRows, ...) of
// columns [256 x, 256 x + 256): each lane reads 4 consecutive columns of a
// row as one dword (a wave reads 1 KB of a row), the four waves take every
// fourth row, their partial sums meet in LDS, and one integer atomic per
// column adds the workgroup's sum into wsum (zeroed first).  Integer
// addition makes the order irrelevant: the result is exact.
constexpr int kColsumRows = 512;
__global__ __launch_bounds__(kBlock) void colsum_zero(int32_t* __restrict__ wsum, int n) {
  const int j = blockIdx.x * kBlock + threadIdx.x;
  if (j < n) wsum[j] = 0;
}
__global__ __launch_bounds__(kBlock) void colsum_kn(const int8_t* __restrict__ b, int k, int n,
                                                    int32_t* __restrict__ wsum) {
  __shared__ int part[kBlock / 64][256];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int j0 = blockIdx.x * 256 + 4 * lane;  // this lane's first column
  const int t0 = blockIdx.y * kColsumRows;
  const int t1 = min(t0 + kColsumRows, k);
  int acc[4] = {0, 0, 0, 0};
  if (j0 + 3 < n && ((n | static_cast<int>(reinterpret_cast<uintptr_t>(b))) & 3) == 0) {
    for (int t = t0 + w; t < t1; t += kBlock / 64) {
      const uint32_t v = *reinterpret_cast<const uint32_t*>(b + static_cast<size_t>(t) * n + j0);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += static_cast<int8_t>(v >> (8 * e));
    }
  } else {
    for (int t = t0 + w; t < t1; t += kBlock / 64)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j0 + e < n) acc[e] += b[static_cast<size_t>(t) * n + j0 + e];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) part[w][4 * lane + e] = acc[e];
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      int total = 0;
#pragma unroll
      for (int q = 0; q < kBlock / 64; ++q) total += part[q][4 * lane + e];
      if (j0 + e < n) atomicAdd(wsum + j0 + e, total);
    }
  }
}
__global__ __launch_bounds__(kBlock) void colsum_nk(const int8_t* __restrict__ b, int k, int n,
                                                    int32_t* __restrict__ wsum) {
  const int j = blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (j >= n) return;  // whole waves leave
  const int8_t* row = b + static_cast<size_t>(j) * k;
  int acc = 0;
  for (int t = lane; t < k; t += 64) acc += row[t];
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) acc += __shfl_xor(acc, d);
  if (lane == 0) wsum[j] = acc;
}

}  // namespace

hipError_t launch_quant_static(int m, int k, const void* x, int dtype, bool silu, bool fp8,
                               const float* scale, int8_t* q, hipStream_t stream) {
  if (silu) {
    return fp8 ? static_dtype<true, true>(m, k, x, dtype, scale, q, stream)
               : static_dtype<true, false>(m, k, x, dtype, scale, q, stream);
  }
  return fp8 ? static_dtype<false, true>(m, k, x, dtype, scale, q, stream)
             : static_dtype<false, false>(m, k, x, dtype, scale, q, stream);
}

hipError_t launch_weight_colsum(int k, int n, const int8_t* b, int b_layout, int32_t* wsum,
                                hipStream_t stream) {
  if (b_layout == QK_B_KN) {
    hipError_t e = launch(colsum_zero, dim3((n + kBlock - 1) / kBlock), dim3(kBlock), 0, stream, wsum, n);
    if (e != hipSuccess) return e;
    if (k == 0) return hipSuccess;
    return launch(colsum_kn, dim3((n + 255) / 256, (k + kColsumRows - 1) / kColsumRows), dim3(kBlock),
                  0, stream, b, k, n, wsum);
  }
  return launch(colsum_nk, dim3((n + kBlock / 64 - 1) / (kBlock / 64)), dim3(kBlock), 0, stream, b,
                k, n, wsum);
}

}  // namespace qk
