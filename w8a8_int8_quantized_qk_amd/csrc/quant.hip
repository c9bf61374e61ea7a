// Per-token dynamic INT8 quantization for gfx950, plain and fused with silu(gate) * up.
//
// Method ("kernels: fused silu_and_mul + dynamic per-token FP8 quantization",
// Purpose and Algorithm; symmetric [-127, 127] codes from "Skill: Write an
// INT8 Quantized Kernel", Inputs):
//   scale = max(row absmax, 1e-12) / 127, code = clamp(rint(x / scale), -127, 127).
//
// One workgroup (4 wave64s) per row.  Each lane loads its 16-byte units with
// 128-bit loads and keeps the widened values in registers, so the row is read
// from HBM exactly once: the page's second pass, which re-reads the input and
// recomputes the activation, is not needed.  The absmax is reduced across the
// wave with cross-lane max steps and across the four waves through LDS.
//
// Division: x / scale must be the correctly rounded binary32 quotient (it
// decides the integer code).  Instead of one full IEEE division per element,
// each row computes r = 1 / scale once (correctly rounded) and each element
// forms y = x * r (within one ulp of the quotient), the exact residual
// e = fma(-y, scale, x), and y' = fma(e, r, y).  By Markstein's theorem
// (P. Markstein, IBM J. Res. Dev. 34(1), 1990; see also Muller et al.,
// Handbook of Floating-Point Arithmetic, ch. on division by fma) y' is the
// correctly rounded quotient whenever the residual does not underflow, which
// holds for every element whose code can be nonzero (|x / scale| >= 1/2
// implies |x| >= 3.9e-15).  Three VALU operations replace an ~11-operation
// IEEE division sequence.
//
// Rows too long for the register cache, or not 16-byte aligned, take a
// two-pass kernel that re-reads the row (and recomputes silu * up).
#include "quant_math.h"

namespace qk {
namespace {

using qm::Elem;
using qm::code_of;
using qm::pack4;
using qm::row_scale;

constexpr int kBlock = 256;    // threads per row
constexpr int kMaxUnits = 8;   // 16-byte input units cached per thread

// e^x in binary32 by a fixed sequence so that results are reproducible bit
// for bit: x = n ln2 + r with n = rint(x / ln 2) and r reduced in two fused
// steps (ln 2 split into a 16-bit head and a tail), e^r by the degree-7
// Taylor polynomial in Horner form (coefficients: the binary32 values nearest
// 1/j!), then the exact scaling by 2^n.  Inputs above 88 give +inf, below -87
// give 0, so every finite result is a normal number.
__device__ __forceinline__ float exp_fixed(float x) {
  if (x > 88.0f) return __builtin_inff();
  if (x < -87.0f) return 0.0f;
  const float n = __builtin_rintf(x * 0x1.715476p+0f);
  float r = __builtin_fmaf(-n, 0x1.62e400p-1f, x);
  r = __builtin_fmaf(-n, 0x1.7f7d1cp-20f, r);
  float p = 0x1.a01a02p-13f;                 // 1/7!
  p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);  // 1/6!
  p = __builtin_fmaf(p, r, 0x1.111112p-7f);   // 1/5!
  p = __builtin_fmaf(p, r, 0x1.555556p-5f);   // 1/4!
  p = __builtin_fmaf(p, r, 0x1.555556p-3f);   // 1/3!
  p = __builtin_fmaf(p, r, 0.5f);             // 1/2!
  p = __builtin_fmaf(p, r, 1.0f);             // 1/1!
  p = __builtin_fmaf(p, r, 1.0f);             // 1/0!
  return __builtin_amdgcn_ldexpf(p, static_cast<int>(n));
}

// silu(g) * u = (g / (1 + e^-g)) * u, each operation rounded once.
__device__ __forceinline__ float silu_times(float g, float u) {
  const float e = exp_fixed(-g);
  const float t = 1.0f + e;
  const float sg = g / t;  // IEEE division (correctly rounded build)
  return sg * u;
}

// Register-cached path: the row (k elements, k % kPerUnit == 0) is split into
// 16-byte units; lane t holds units t, t + 256, ... (at most kMaxUnits).
// For SILU the source row has 2k elements: gate units then up units.
template <int DT, bool SILU>
__global__ __launch_bounds__(kBlock) void quant_rows_cached(const void* __restrict__ src,
                                                           int8_t* __restrict__ q,
                                                           float* __restrict__ scale, int k) {
  using E = Elem<DT>;
  constexpr int P = E::kPerUnit;
  const int units = k / P;
  const size_t row = blockIdx.x;
  const char* base =
      static_cast<const char*>(src) + row * static_cast<size_t>(SILU ? 2 : 1) * k * E::kBytes;

  float v[kMaxUnits][P];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxUnits; ++j) {
    const int u = threadIdx.x + j * kBlock;
    if (u < units) {
      const uint4 raw = *reinterpret_cast<const uint4*>(base + static_cast<size_t>(u) * 16);
      E::unpack(raw, v[j]);
      if constexpr (SILU) {
        const uint4 raw_up = *reinterpret_cast<const uint4*>(
            base + static_cast<size_t>(k) * E::kBytes + static_cast<size_t>(u) * 16);
        float up[P];
        E::unpack(raw_up, up);
#pragma unroll
        for (int e = 0; e < P; ++e) v[j][e] = silu_times(v[j][e], up[e]);
      }
#pragma unroll
      for (int e = 0; e < P; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[j][e]));
    }
  }
  amax = qm::block_max<kBlock>(amax);
  float s, r;
  row_scale(amax, s, r);
  if (threadIdx.x == 0) scale[row] = s;

  int8_t* qrow = q + row * static_cast<size_t>(k);
#pragma unroll
  for (int j = 0; j < kMaxUnits; ++j) {
    const int u = threadIdx.x + j * kBlock;
    if (u < units) {
      int c[P];
#pragma unroll
      for (int e = 0; e < P; ++e) c[e] = code_of(v[j][e], s, r);
      if constexpr (P == 8) {
        uint2 w;
        w.x = pack4(c[0], c[1], c[2], c[3]);
        w.y = pack4(c[4], c[5], c[6], c[7]);
        *reinterpret_cast<uint2*>(qrow + static_cast<size_t>(u) * 8) = w;
      } else {
        *reinterpret_cast<uint32_t*>(qrow + static_cast<size_t>(u) * 4) =
            pack4(c[0], c[1], c[2], c[3]);
      }
    }
  }
}

// Two-pass path for any k and alignment: pass 1 reduces the absmax, pass 2
// re-reads (and for SILU recomputes) each value and writes its code.
template <int DT, bool SILU>
__global__ __launch_bounds__(kBlock) void quant_rows_twopass(const void* __restrict__ src,
                                                            int8_t* __restrict__ q,
                                                            float* __restrict__ scale, int k) {
  using E = Elem<DT>;
  const size_t row = blockIdx.x;
  const size_t first = row * static_cast<size_t>(SILU ? 2 : 1) * k;
  auto value = [&](int j) -> float {
    const float x = E::load(src, first + j);
    if constexpr (SILU) return silu_times(x, E::load(src, first + k + j));
    return x;
  };
  float amax = 0.0f;
  for (int j = threadIdx.x; j < k; j += kBlock) amax = __builtin_fmaxf(amax, __builtin_fabsf(value(j)));
  amax = qm::block_max<kBlock>(amax);
  float s, r;
  row_scale(amax, s, r);
  if (threadIdx.x == 0) scale[row] = s;
  int8_t* qrow = q + row * static_cast<size_t>(k);
  for (int j = threadIdx.x; j < k; j += kBlock) qrow[j] = static_cast<int8_t>(code_of(value(j), s, r));
}

template <int DT, bool SILU>
hipError_t dispatch(int m, int k, const void* src, int8_t* q, float* scale, hipStream_t stream) {
  using E = Elem<DT>;
  const bool aligned = (reinterpret_cast<uintptr_t>(src) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(q) % E::kPerUnit == 0) &&
                       (k % E::kPerUnit == 0);
  const bool fits = k / E::kPerUnit <= kMaxUnits * kBlock;
  if (aligned && fits)
    return launch(quant_rows_cached<DT, SILU>, dim3(m), dim3(kBlock), 0, stream, src, q, scale, k);
  return launch(quant_rows_twopass<DT, SILU>, dim3(m), dim3(kBlock), 0, stream, src, q, scale, k);
}

template <bool SILU>
hipError_t dispatch_dtype(int m, int k, const void* src, int dtype, int8_t* q, float* scale,
                          hipStream_t stream) {
  switch (dtype) {
    case QK_F32: return dispatch<QK_F32, SILU>(m, k, src, q, scale, stream);
    case QK_BF16: return dispatch<QK_BF16, SILU>(m, k, src, q, scale, stream);
    case QK_F16: return dispatch<QK_F16, SILU>(m, k, src, q, scale, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_quant_rows(int m, int k, const void* x, int dtype, int8_t* q, float* scale,
                             hipStream_t stream) {
  return dispatch_dtype<false>(m, k, x, dtype, q, scale, stream);
}

hipError_t launch_silu_quant_rows(int m, int d, const void* h, int dtype, int8_t* q,
                                  float* scale, hipStream_t stream) {
  return dispatch_dtype<true>(m, d, h, dtype, q, scale, stream);
}

}  // namespace qk
