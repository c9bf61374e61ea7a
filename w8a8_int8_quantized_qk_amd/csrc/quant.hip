// Per-token dynamic quantization for gfx950, to INT8 or FP8 codes, plain and
// fused with silu(gate) * up, and asymmetric (zero-point) INT8 codes.
//
// Method ("kernels: fused silu_and_mul + dynamic per-token FP8 quantization",
// Purpose and Algorithm; symmetric [-127, 127] codes from "Skill: Write an
// INT8 Quantized Kernel", Inputs):
//   INT8: scale = max(row absmax, 1e-12) / 127, code = clamp(rint(x / scale), -127, 127);
//   FP8:  scale = min(max(row absmax, 1e-12) / 448, scale_ub if > 0),
//         code = e4m3fn(x / scale), nearest even, saturating at +-448;
//   asymmetric INT8 ("Skill: Write an INT8 Quantized Kernel", Inputs: a
//         nonzero zero point): lo = min(row min, 0), hi = max(row max, 0),
//         scale = max(hi - lo, 1e-12) / 255, zp = clamp(rint(-lo / scale) -
//         128, -128, 127), code = clamp(rint(x / scale) + zp, -128, 127).
//
// Rows of up to 128 16-byte units take one wave each (absmax by cross-lane
// max steps only); rows of up to 2048 units take one workgroup of four waves
// each (cross-lane steps, then LDS).  Either way each lane loads its units
// with 128-bit loads and keeps the widened values in registers, so the row is
// read from HBM exactly once: the page's second pass, which re-reads the
// input and recomputes the activation, is not needed.
//
// Division: x / scale must be the correctly rounded binary32 quotient (it
// decides the integer code).  Instead of one full IEEE division per element,
// each row computes r = 1 / scale once (correctly rounded) and each element
// forms y = x * r, the exact residual e = fma(-y, scale, x), and
// y' = fma(e, r, y): Markstein's correction step (P. Markstein, IBM J. Res.
// Dev. 34(1), 1990; Muller et al., Handbook of Floating-Point Arithmetic,
// division with fma).  His theorem proves y' correctly rounded when y is a
// faithful rounding of x / scale and the residual does not underflow; y here
// carries two roundings (of 1 / scale and of the product) and is not
// faithful for every input, so the theorem alone does not cover the method.
// It is checked instead: against IEEE division over every bf16 input under a
// spread of row maxima and over 2e7 random binary32 inputs, many placed next
// to half-integer multiples of the scale where a wrong quotient would change
// the code, with no difference (the division-method check of the CPU test
// suite).  Three VALU operations replace an ~11-operation IEEE division
// sequence.
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
using qm::silu_times;

enum Fmt { kI8 = 0, kF8 = 1, kI8Asym = 2 };

// Per-lane row statistics: the absmax (symmetric formats) or hi = max(x, 0)
// and nlo = max(-x, 0) (asymmetric); all non-negative.
struct Stats {
  float a = 0.0f;
  float b = 0.0f;
};
template <int FMT>
__device__ __forceinline__ void accumulate(Stats& st, float v) {
  if constexpr (FMT == kI8Asym) {
    st.a = __builtin_fmaxf(st.a, v);
    st.b = __builtin_fmaxf(st.b, -v);
  } else {
    st.a = __builtin_fmaxf(st.a, __builtin_fabsf(v));
  }
}
template <int FMT>
__device__ __forceinline__ void wave_reduce(Stats& st) {
  st.a = qm::wave_max_nonneg(st.a);
  if constexpr (FMT == kI8Asym) st.b = qm::wave_max_nonneg(st.b);
}
template <int FMT, int kBlock>
__device__ __forceinline__ void block_reduce(Stats& st) {
  if constexpr (FMT == kI8Asym)
    qm::block_max2<kBlock>(st.a, st.b);
  else
    st.a = qm::block_max<kBlock>(st.a);
}

// The row's scale s, r = RN(1 / s), and (asymmetric) the zero point.
struct RowQ {
  float s, r, zp;
  bool bounded;  // FP8: the scale bound replaced the row's own scale
};
template <int FMT>
__device__ __forceinline__ RowQ row_params(const Stats& st, float scale_ub) {
  RowQ p{0.0f, 0.0f, 0.0f, false};
  if constexpr (FMT == kI8)
    row_scale(st.a, p.s, p.r);
  else if constexpr (FMT == kF8)
    p.bounded = qm::row_scale_fp8(st.a, scale_ub, p.s, p.r);
  else
    qm::row_scale_asym(st.a, st.b, p.s, p.r, p.zp);
  return p;
}

// the code byte of one value
template <int FMT>
__device__ __forceinline__ int8_t code_byte(float x, const RowQ& p) {
  if constexpr (FMT == kI8) {
    return static_cast<int8_t>(qm::code_word_dynamic(x, p.s, p.r) & 0xffu);
  } else if constexpr (FMT == kI8Asym) {
    return static_cast<int8_t>(qm::code_of_asym(x, p.s, p.r, p.zp));
  } else {
    return static_cast<int8_t>(__builtin_amdgcn_cvt_pk_fp8_f32(qm::fp8_ratio(x, p.s, p.r), 0.0f, 0, false) & 0xff);
  }
}

// the row's outputs: scale, and the zero point for the asymmetric format
template <int FMT>
__device__ __forceinline__ void store_row_params(const RowQ& p, float* scale, int32_t* zp, size_t row) {
  scale[row] = p.s;
  if constexpr (FMT == kI8Asym) zp[row] = static_cast<int32_t>(p.zp);
}

constexpr int kBlock = 256;    // threads per workgroup
constexpr int kMaxUnits = 8;   // 16-byte input units cached per lane

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

// Codes of one 16-byte unit of P values, stored as P bytes.  Ordinary
// stores: the GEMM that consumes the codes usually runs next and finds them
// in the caches (measured on the prefill step: 0.4 us faster than
// nontemporal stores, although the quantization alone is slower).
template <int FMT, int P>
__device__ __forceinline__ void store_codes(int8_t* dst, const float (&v)[P], const RowQ& p) {
  uint32_t w[P / 4];
  const float s = p.s, r = p.r;
  if constexpr (FMT == kI8) {
    uint32_t c[P];
#pragma unroll
    for (int e = 0; e < P; ++e) c[e] = qm::code_word_dynamic(v[e], s, r);
#pragma unroll
    for (int i = 0; i < P / 4; ++i)
      w[i] = qm::pack4_low_bytes(c[4 * i], c[4 * i + 1], c[4 * i + 2], c[4 * i + 3]);
  } else if constexpr (FMT == kI8Asym) {
    const int zp_off = static_cast<int>(p.zp) - 0x4B400000;
    uint32_t c[P];
#pragma unroll
    for (int e = 0; e < P; ++e) c[e] = qm::code_word_asym(v[e], s, r, zp_off);
#pragma unroll
    for (int i = 0; i < P / 4; ++i)
      w[i] = qm::pack4_low_bytes(c[4 * i], c[4 * i + 1], c[4 * i + 2], c[4 * i + 3]);
  } else {
    float f[P];
    if (p.bounded) {  // uniform: one row per wave or workgroup
#pragma unroll
      for (int e = 0; e < P; ++e) f[e] = qm::fp8_ratio(v[e], s, r);
    } else {
#pragma unroll
      for (int e = 0; e < P; ++e) f[e] = qm::fp8_ratio_own(v[e], s, r);
    }
#pragma unroll
    for (int i = 0; i < P / 4; ++i) w[i] = qm::pack4_fp8(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3]);
  }
  if constexpr (P == 8) {
    *reinterpret_cast<v2u*>(dst) = v2u{w[0], w[1]};
  } else {
    *reinterpret_cast<uint32_t*>(dst) = w[0];
  }
}

// One 16-byte unit of the input, read once (nontemporal).
__device__ __forceinline__ uint4 load_unit(const char* p) {
  const v4u x = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(x.x, x.y, x.z, x.w);
}

// The P values of unit u of a row (for SILU: silu(gate) * up, the up half
// starting k elements after the gate half).
template <int DT, bool SILU>
__device__ __forceinline__ void unit_values(const char* base, int k, int u,
                                            float (&v)[Elem<DT>::kPerUnit]) {
  using E = Elem<DT>;
  E::unpack(load_unit(base + static_cast<size_t>(u) * 16), v);
  if constexpr (SILU) {
    const uint4 raw_up = load_unit(base + static_cast<size_t>(k) * E::kBytes + static_cast<size_t>(u) * 16);
    float up[E::kPerUnit];
    E::unpack(raw_up, up);
#pragma unroll
    for (int e = 0; e < E::kPerUnit; ++e) v[e] = silu_times<DT != QK_F32>(v[e], up[e]);
  }
}

// Short rows (up to 128 units): one wave per row, four rows per workgroup.
// Lane l holds units l, l + 64 (UPL of them) in registers; the absmax needs
// only cross-lane steps within the wave (no LDS, no barrier).
template <int DT, bool SILU, int FMT, int UPL>
__global__ __launch_bounds__(kBlock) void quant_rows_wave(const void* __restrict__ src,
                                                         int8_t* __restrict__ q,
                                                         float* __restrict__ scale, float scale_ub,
                                                         int32_t* __restrict__ zp, int m, int k) {
  using E = Elem<DT>;
  constexpr int P = E::kPerUnit;
  const int units = k / P;
  const int lane = threadIdx.x & 63;
  const size_t row = static_cast<size_t>(blockIdx.x) * (kBlock / 64) + (threadIdx.x >> 6);
  if (row >= static_cast<size_t>(m)) return;  // whole waves leave; no barriers below
  const char* base =
      static_cast<const char*>(src) + row * static_cast<size_t>(SILU ? 2 : 1) * k * E::kBytes;

  float v[UPL][P];
  Stats st;
#pragma unroll
  for (int j = 0; j < UPL; ++j) {
    const int u = lane + 64 * j;
    if (u < units) {
      unit_values<DT, SILU>(base, k, u, v[j]);
#pragma unroll
      for (int e = 0; e < P; ++e) accumulate<FMT>(st, v[j][e]);
    }
  }
  wave_reduce<FMT>(st);
  const RowQ p = row_params<FMT>(st, scale_ub);
  if (lane == 0) store_row_params<FMT>(p, scale, zp, row);

  int8_t* qrow = q + row * static_cast<size_t>(k);
#pragma unroll
  for (int j = 0; j < UPL; ++j) {
    const int u = lane + 64 * j;
    if (u < units) store_codes<FMT, P>(qrow + static_cast<size_t>(u) * P, v[j], p);
  }
}

// Longer rows: one workgroup (4 waves) per row.  Lane t holds units
// t, t + 256, ... (UPT of them) in registers, so the row is read from HBM
// exactly once: the page's second pass, which re-reads the input and
// recomputes the activation, is not needed.  (Many short-lived waves with a
// few loads each keep more of the chip's memory pipeline busy than fewer
// waves with many: measured faster than one wave per row at 512 units.)
template <int DT, bool SILU, int FMT, int UPT>
__global__ __launch_bounds__(kBlock) void quant_rows_cached(const void* __restrict__ src,
                                                           int8_t* __restrict__ q,
                                                           float* __restrict__ scale,
                                                           float scale_ub, int32_t* __restrict__ zp,
                                                           int k) {
  using E = Elem<DT>;
  constexpr int P = E::kPerUnit;
  const int units = k / P;
  const size_t row = blockIdx.x;
  const char* base =
      static_cast<const char*>(src) + row * static_cast<size_t>(SILU ? 2 : 1) * k * E::kBytes;

  float v[UPT][P];
  Stats st;
#pragma unroll
  for (int j = 0; j < UPT; ++j) {
    const int u = threadIdx.x + j * kBlock;
    if (u < units) {
      unit_values<DT, SILU>(base, k, u, v[j]);
#pragma unroll
      for (int e = 0; e < P; ++e) accumulate<FMT>(st, v[j][e]);
    }
  }
  block_reduce<FMT, kBlock>(st);
  const RowQ p = row_params<FMT>(st, scale_ub);
  if (threadIdx.x == 0) store_row_params<FMT>(p, scale, zp, row);

  int8_t* qrow = q + row * static_cast<size_t>(k);
#pragma unroll
  for (int j = 0; j < UPT; ++j) {
    const int u = threadIdx.x + j * kBlock;
    if (u < units) store_codes<FMT, P>(qrow + static_cast<size_t>(u) * P, v[j], p);
  }
}

// Two-pass path for any k and alignment: pass 1 reduces the absmax, pass 2
// re-reads (and for SILU recomputes) each value and writes its code.
template <int DT, bool SILU, int FMT>
__global__ __launch_bounds__(kBlock) void quant_rows_twopass(const void* __restrict__ src,
                                                            int8_t* __restrict__ q,
                                                            float* __restrict__ scale,
                                                            float scale_ub, int32_t* __restrict__ zp,
                                                            int k) {
  using E = Elem<DT>;
  const size_t row = blockIdx.x;
  const size_t first = row * static_cast<size_t>(SILU ? 2 : 1) * k;
  auto value = [&](int j) -> float {
    const float x = E::load(src, first + j);
    if constexpr (SILU) return silu_times<DT != QK_F32>(x, E::load(src, first + k + j));
    return x;
  };
  Stats st;
  for (int j = threadIdx.x; j < k; j += kBlock) accumulate<FMT>(st, value(j));
  block_reduce<FMT, kBlock>(st);
  const RowQ p = row_params<FMT>(st, scale_ub);
  if (threadIdx.x == 0) store_row_params<FMT>(p, scale, zp, row);
  int8_t* qrow = q + row * static_cast<size_t>(k);
  for (int j = threadIdx.x; j < k; j += kBlock) qrow[j] = code_byte<FMT>(value(j), p);
}

template <int DT, bool SILU, int FMT>
hipError_t dispatch(int m, int k, const void* src, int8_t* q, float* scale, float scale_ub,
                    int32_t* zp, hipStream_t stream) {
  using E = Elem<DT>;
  const bool aligned = (reinterpret_cast<uintptr_t>(src) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(q) % E::kPerUnit == 0) &&
                       (k % E::kPerUnit == 0);
  const int units = k / E::kPerUnit;
  if (aligned && units <= 128) {
    const dim3 grid((static_cast<unsigned>(m) + kBlock / 64 - 1) / (kBlock / 64));
    if (units <= 64)
      return launch(quant_rows_wave<DT, SILU, FMT, 1>, grid, dim3(kBlock), 0, stream, src, q, scale,
                    scale_ub, zp, m, k);
    return launch(quant_rows_wave<DT, SILU, FMT, 2>, grid, dim3(kBlock), 0, stream, src, q, scale,
                  scale_ub, zp, m, k);
  }
  if (aligned && units <= kBlock * kMaxUnits) {
    const dim3 grid(m);
    if (units <= kBlock)
      return launch(quant_rows_cached<DT, SILU, FMT, 1>, grid, dim3(kBlock), 0, stream, src, q,
                    scale, scale_ub, zp, k);
    if (units <= kBlock * 2)
      return launch(quant_rows_cached<DT, SILU, FMT, 2>, grid, dim3(kBlock), 0, stream, src, q,
                    scale, scale_ub, zp, k);
    if (units <= kBlock * 4)
      return launch(quant_rows_cached<DT, SILU, FMT, 4>, grid, dim3(kBlock), 0, stream, src, q,
                    scale, scale_ub, zp, k);
    return launch(quant_rows_cached<DT, SILU, FMT, 8>, grid, dim3(kBlock), 0, stream, src, q,
                  scale, scale_ub, zp, k);
  }
  return launch(quant_rows_twopass<DT, SILU, FMT>, dim3(m), dim3(kBlock), 0, stream, src, q, scale,
                scale_ub, zp, k);
}

// silu(gate) * up in binary32 without quantization: the activation the fused
// kernels quantize, with the same arithmetic (silu_times), for callers that
// want it unquantized.  Rows of whole 16-byte units (16-byte aligned input,
// d a multiple of the unit) take one unit of gate and one of up per thread
// and iteration; others one element.
template <int DT>
__global__ __launch_bounds__(kBlock) void silu_mul_units_kernel(const void* __restrict__ src,
                                                               float* __restrict__ out,
                                                               long long units, int units_per_row) {
  using E = Elem<DT>;
  constexpr int P = E::kPerUnit;
  const char* in = static_cast<const char*>(src);
  const long long stride = static_cast<long long>(gridDim.x) * kBlock;
  for (long long u = static_cast<long long>(blockIdx.x) * kBlock + threadIdx.x; u < units;
       u += stride) {
    const long long row = u / units_per_row;
    const long long at = u + row * units_per_row;  // the gate unit; up is units_per_row later
    float g[P], up[P];
    E::unpack(load_unit(in + at * 16), g);
    E::unpack(load_unit(in + (at + units_per_row) * 16), up);
    float* o = out + u * P;
#pragma unroll
    for (int e = 0; e < P; e += 4)
      *reinterpret_cast<float4*>(o + e) =
          make_float4(silu_times<DT != QK_F32>(g[e], up[e]), silu_times<DT != QK_F32>(g[e + 1], up[e + 1]),
                      silu_times<DT != QK_F32>(g[e + 2], up[e + 2]),
                      silu_times<DT != QK_F32>(g[e + 3], up[e + 3]));
  }
}

template <int DT>
__global__ __launch_bounds__(kBlock) void silu_mul_kernel(const void* __restrict__ src,
                                                         float* __restrict__ out,
                                                         long long total, int d) {
  using E = Elem<DT>;
  const long long stride = static_cast<long long>(gridDim.x) * kBlock;
  for (long long i = static_cast<long long>(blockIdx.x) * kBlock + threadIdx.x; i < total;
       i += stride) {
    const long long row = i / d;
    const long long j = i - row * d;
    const size_t first = static_cast<size_t>(row) * 2 * d;
    out[i] = silu_times<DT != QK_F32>(E::load(src, first + j), E::load(src, first + d + j));
  }
}

template <int DT>
hipError_t launch_silu_mul_dt(int m, int d, const void* h, float* out, hipStream_t stream) {
  constexpr int P = Elem<DT>::kPerUnit;
  const long long total = static_cast<long long>(m) * d;
  const bool units = d % P == 0 && reinterpret_cast<uintptr_t>(h) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(out) % 16 == 0;
  const long long items = units ? total / P : total;
  const long long want = (items + kBlock - 1) / kBlock;
  const dim3 grid(static_cast<unsigned>(want < 8192 ? want : 8192));
  if (units)
    return launch(silu_mul_units_kernel<DT>, grid, dim3(kBlock), 0, stream, h, out, items, d / P);
  return launch(silu_mul_kernel<DT>, grid, dim3(kBlock), 0, stream, h, out, total, d);
}

template <bool SILU, int FMT>
hipError_t dispatch_dtype(int m, int k, const void* src, int dtype, int8_t* q, float* scale,
                          float scale_ub, int32_t* zp, hipStream_t stream) {
  switch (dtype) {
    case QK_F32: return dispatch<QK_F32, SILU, FMT>(m, k, src, q, scale, scale_ub, zp, stream);
    case QK_BF16: return dispatch<QK_BF16, SILU, FMT>(m, k, src, q, scale, scale_ub, zp, stream);
    case QK_F16: return dispatch<QK_F16, SILU, FMT>(m, k, src, q, scale, scale_ub, zp, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_quant_rows(int m, int k, const void* x, int dtype, int8_t* q, float* scale,
                             hipStream_t stream) {
  return dispatch_dtype<false, kI8>(m, k, x, dtype, q, scale, 0.0f, nullptr, stream);
}

hipError_t launch_silu_quant_rows(int m, int d, const void* h, int dtype, int8_t* q,
                                  float* scale, hipStream_t stream) {
  return dispatch_dtype<true, kI8>(m, d, h, dtype, q, scale, 0.0f, nullptr, stream);
}

hipError_t launch_silu_mul(int m, int d, const void* h, int dtype, float* out,
                           hipStream_t stream) {
  if (static_cast<long long>(m) * d == 0) return hipSuccess;
  switch (dtype) {
    case QK_F32: return launch_silu_mul_dt<QK_F32>(m, d, h, out, stream);
    case QK_BF16: return launch_silu_mul_dt<QK_BF16>(m, d, h, out, stream);
    case QK_F16: return launch_silu_mul_dt<QK_F16>(m, d, h, out, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_quant_rows_fp8(int m, int k, const void* x, int dtype, uint8_t* q, float* scale,
                                 float scale_ub, hipStream_t stream) {
  return dispatch_dtype<false, kF8>(m, k, x, dtype, reinterpret_cast<int8_t*>(q), scale, scale_ub,
                                    nullptr, stream);
}

hipError_t launch_silu_quant_rows_fp8(int m, int d, const void* h, int dtype, uint8_t* q,
                                      float* scale, float scale_ub, hipStream_t stream) {
  return dispatch_dtype<true, kF8>(m, d, h, dtype, reinterpret_cast<int8_t*>(q), scale, scale_ub,
                                   nullptr, stream);
}

hipError_t launch_quant_rows_asym(int m, int k, const void* x, int dtype, int8_t* q, float* scale,
                                  int32_t* zp, hipStream_t stream) {
  return dispatch_dtype<false, kI8Asym>(m, k, x, dtype, q, scale, 0.0f, zp, stream);
}

}  // namespace qk
