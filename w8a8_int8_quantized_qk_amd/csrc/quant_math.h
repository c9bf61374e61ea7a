// Per-token quantization arithmetic shared by the quantization kernels and the
// fused decode GEMV (device code only).
//
// scale = max(row absmax, 1e-12) / 127 and code = clamp(rint(x / scale),
// -127, 127) in binary32 ("kernels: fused silu_and_mul + dynamic per-token FP8
// quantization", Algorithm; symmetric [-127, 127] codes from "Skill: Write an
// INT8 Quantized Kernel", Inputs).  x / scale is formed from r = 1 / scale
// (correctly rounded) as y = x * r, e = fma(-y, scale, x), y' = fma(e, r, y),
// Markstein's correction step (P. Markstein, IBM J. Res. Dev. 34(1), 1990;
// Muller et al., Handbook of Floating-Point Arithmetic, division with fma).
// His theorem needs y to be a faithful rounding of the quotient, which
// y = RN(x * RN(1 / scale)) is not for every input, so the method rests on
// checks against IEEE division (every bf16 input under a spread of row
// maxima, 2e7 random binary32 inputs aimed at half-integer multiples of the
// scale: no difference), not on the theorem alone.
#pragma once

#include "qk_internal.h"

namespace qk {
namespace qm {

template <int DT>
struct Elem;
template <>
struct Elem<QK_F32> {
  static constexpr int kBytes = 4;
  static constexpr int kPerUnit = 4;
  __device__ static void unpack(const uint4 v, float* f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  __device__ static float load(const void* p, size_t i) {
    return static_cast<const float*>(p)[i];
  }
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <>
struct Elem<QK_BF16> {
  static constexpr int kBytes = 2;
  static constexpr int kPerUnit = 8;
  __device__ static void unpack(const uint4 v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(w[i]);
      f[2 * i + 1] = bf16_hi(w[i]);
    }
  }
  __device__ static float load(const void* p, size_t i) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
  }
};

__device__ __forceinline__ float f16_bits(uint32_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}

template <>
struct Elem<QK_F16> {
  static constexpr int kBytes = 2;
  static constexpr int kPerUnit = 8;
  __device__ static void unpack(const uint4 v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = f16_bits(w[i] & 0xffffu);
      f[2 * i + 1] = f16_bits(w[i] >> 16);
    }
  }
  __device__ static float load(const void* p, size_t i) {
    return f16_bits(static_cast<const uint16_t*>(p)[i]);
  }
};

// clamp(rint(x / s), -127, 127) with x / s formed from r = RN(1 / s).
__device__ __forceinline__ int code_of(float x, float s, float r) {
  const float y = x * r;
  const float e = __builtin_fmaf(-y, s, x);
  float q = __builtin_fmaf(e, r, y);
  q = __builtin_rintf(q);
  q = __builtin_fminf(__builtin_fmaxf(q, -127.0f), 127.0f);
  return static_cast<int>(q);
}

// The code of x / s for a row's own dynamic scale, as the low byte of the
// returned word.  The quotient is exact (as in code_of); adding 1.5 * 2^23
// rounds it to an integer, ties to even (the sum's unit in the last place is
// 1, and 1.5 * 2^23 is even), and leaves that integer in the low mantissa
// bits: the word is 0x4B400000 + code, whose low byte is the code's two's
// complement byte.  No clamp is needed: s is the correctly rounded
// max(amax, 1e-12) / 127, so |x / s| <= 127 (1 + 2^-23) for every |x| <=
// amax, which rounds to at most 127.
__device__ __forceinline__ uint32_t code_word_dynamic(float x, float s, float r) {
  const float y = x * r;
  const float e = __builtin_fmaf(-y, s, x);
  const float q = __builtin_fmaf(e, r, y);
  return __float_as_uint(q + 12582912.0f);
}

// Four code words' low bytes packed little-endian (a in byte 0).
__device__ __forceinline__ uint32_t pack4_low_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);  // bytes: a0 b0 0 0
  const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x04000c0cu);  // bytes: 0 0 c0 d0
  return ab | cd;
}

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
  return (static_cast<uint32_t>(a) & 0xffu) | ((static_cast<uint32_t>(b) & 0xffu) << 8) |
         ((static_cast<uint32_t>(c) & 0xffu) << 16) | (static_cast<uint32_t>(d) << 24);
}

// e^x in binary32 by a fixed sequence so that results are reproducible bit
// for bit: x = n ln2 + r with n = rint(x / ln 2) and r reduced in two fused
// steps (ln 2 split into a 16-bit head and a tail), e^r by the degree-7
// Taylor polynomial in Horner form (coefficients: the binary32 values nearest
// 1/j!), then the exact scaling by 2^n.  Inputs above 88 give +inf, below -87
// give 0, so every finite result is a normal number.  This function is the
// part for x in [-87, 88]; silu_times applies the two range rules.
__device__ __forceinline__ float exp_fixed_in_range(float x) {
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

// g / t for a denominator t >= 1 (or +inf): the hardware reciprocal with
// one correction step.  v_div_scale_f32 scales both operands so that the
// reciprocal and the quotient stay clear of the subnormal range; then
// r ~ 1 / t, y = g r, the exact residual g - y t, the corrected y + residual
// * r (rescaled by v_div_fmas_f32), and v_div_fixup_f32 for infinite, zero
// and NaN operands.  Seven instructions against eleven for the IEEE sequence,
// which first refines r by a Newton step and corrects twice.  One correction
// from an unrefined reciprocal is not correctly rounded for every pair of
// binary32 operands, so this serves only 16-bit gates: there t is a function
// of g, and every one of the 65536 gates of each 16-bit format is checked
// against IEEE division on the GPU.
__device__ __forceinline__ float div_one_correction(float g, float t) {
  bool den_flag, vcc;
  const float ds = __builtin_amdgcn_div_scalef(g, t, false, &den_flag);
  const float ns = __builtin_amdgcn_div_scalef(g, t, true, &vcc);
  const float r = __builtin_amdgcn_rcpf(ds);
  const float y = ns * r;
  const float e = __builtin_fmaf(-ds, y, ns);
  const float q = __builtin_amdgcn_div_fmasf(e, r, y, vcc);
  return __builtin_amdgcn_div_fixupf(q, t, g);
}

// silu(g) * u = (g / (1 + e^-g)) * u, each operation rounded once, e^x as
// exp_fixed_in_range with its range rules, and without branches: x = -g is
// clamped to [-87, 88] first, which changes no result (below -87 the rule
// gives e = 0, the clamped x gives e = e^-87 < 2^-125, and 1 + e rounds to
// exactly 1 either way), and t = +inf replaces 1 + e where x > 88.  A NaN
// gate needs neither rule: the quotient propagates it.  kNarrow: the gate
// came from a 16-bit format (the division as div_one_correction, checked
// for all such gates); otherwise the IEEE division.
template <bool kNarrow>
__device__ __forceinline__ float silu_times(float g, float u) {
  const float x = __builtin_amdgcn_fmed3f(-g, -87.0f, 88.0f);
  float t = 1.0f + exp_fixed_in_range(x);
  t = -g > 88.0f ? __builtin_inff() : t;
  const float sg = kNarrow ? div_one_correction(g, t) : g / t;  // IEEE division (correctly rounded build)
  return sg * u;
}

// Max over the 64 lanes of a wave of non-negative binary32 values (|x|),
// left in every lane.  For x >= 0 the unsigned order of the bit patterns is
// the numeric order, so the max runs on integers (no float canonicalizing):
// DPP lane exchanges within each 16-lane row (quad partners, then the mirror
// half-row and row), then lane swaps across rows (v_permlane16_swap) and
// across the halves of the wave (v_permlane32_swap).
__device__ __forceinline__ uint32_t max_u32(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ float wave_max_nonneg(float x) {
  uint32_t v = __float_as_uint(x);
  v = max_u32(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, false)));   // quad_perm 1,0,3,2
  v = max_u32(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, false)));   // quad_perm 2,3,0,1
  v = max_u32(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x141, 0xF, 0xF, false)));  // row_half_mirror
  v = max_u32(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x140, 0xF, 0xF, false)));  // row_mirror
  const auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max_u32(static_cast<uint32_t>(r16[0]), static_cast<uint32_t>(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = max_u32(static_cast<uint32_t>(r32[0]), static_cast<uint32_t>(r32[1]));
  return __uint_as_float(v);
}

// Workgroup-wide max of non-negative values (|x|), returned to every thread.
template <int kBlock>
__device__ __forceinline__ float block_max(float v) {
  __shared__ uint32_t part[kBlock / 64];
  v = wave_max_nonneg(v);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = __float_as_uint(v);
  __syncthreads();
  uint32_t r = part[0];
#pragma unroll
  for (int w = 1; w < kBlock / 64; ++w) r = max_u32(r, part[w]);
  return __uint_as_float(r);
}

// Workgroup-wide max of two non-negative values at once (one barrier).
template <int kBlock>
__device__ __forceinline__ void block_max2(float& a, float& b) {
  __shared__ uint32_t part2[2][kBlock / 64];
  a = wave_max_nonneg(a);
  b = wave_max_nonneg(b);
  if ((threadIdx.x & 63) == 0) {
    part2[0][threadIdx.x >> 6] = __float_as_uint(a);
    part2[1][threadIdx.x >> 6] = __float_as_uint(b);
  }
  __syncthreads();
  uint32_t ra = part2[0][0], rb = part2[1][0];
#pragma unroll
  for (int w = 1; w < kBlock / 64; ++w) {
    ra = max_u32(ra, part2[0][w]);
    rb = max_u32(rb, part2[1][w]);
  }
  a = __uint_as_float(ra);
  b = __uint_as_float(rb);
}

// clamp(rint(x / s), -127, 127) for a caller-given scale s, which may be
// small enough for x * r to overflow: the first product is clamped to +-256
// (every quotient that can round inside [-127, 127] is unchanged; a clamped
// one saturates like the true quotient), which keeps the correction finite.
__device__ __forceinline__ int code_of_bounded(float x, float s, float r) {
  float y = x * r;
  y = __builtin_amdgcn_fmed3f(y, -256.0f, 256.0f);
  const float e = __builtin_fmaf(-y, s, x);
  float q = __builtin_fmaf(e, r, y);
  q = __builtin_rintf(q);
  q = __builtin_fminf(__builtin_fmaxf(q, -127.0f), 127.0f);
  return static_cast<int>(q);
}

// The same code as code_of_bounded, as the low byte of the returned word
// (packed like code_word_dynamic's): the quotient is clamped to [-127, 127]
// before it is rounded, which gives the same integer (rint and the clamp
// commute, the bounds being integers), and the rounding adds 1.5 * 2^23.
// Six instructions instead of eight plus the packing shifts.
__device__ __forceinline__ uint32_t code_word_bounded(float x, float s, float r) {
  float y = x * r;
  y = __builtin_amdgcn_fmed3f(y, -256.0f, 256.0f);
  const float e = __builtin_fmaf(-y, s, x);
  float q = __builtin_fmaf(e, r, y);
  q = __builtin_amdgcn_fmed3f(q, -127.0f, 127.0f);
  return __float_as_uint(q + 12582912.0f);
}

// Asymmetric codes: clamp(rint(x / s) + zp, -128, 127) with the exact
// quotient (|x / s| <= 255 by construction of s, so no overflow).
__device__ __forceinline__ int code_of_asym(float x, float s, float r, float zp) {
  const float y = x * r;
  const float e = __builtin_fmaf(-y, s, x);
  float q = __builtin_fmaf(e, r, y);
  q = __builtin_rintf(q) + zp;
  q = __builtin_fminf(__builtin_fmaxf(q, -128.0f), 127.0f);
  return static_cast<int>(q);
}

// The same code as code_of_asym as the low byte of the returned word: the
// exact quotient rounded by adding 1.5 * 2^23 (|x / s| <= 255, so the sum's
// bits are 0x4B400000 + rint(x / s)), then the zero point added and the clamp
// to [-128, 127] taken on that integer.  zp_off = zp - 0x4B400000 (per row).
__device__ __forceinline__ uint32_t code_word_asym(float x, float s, float r, int zp_off) {
  const float y = x * r;
  const float e = __builtin_fmaf(-y, s, x);
  const float q = __builtin_fmaf(e, r, y);
  const int c = static_cast<int>(__float_as_uint(q + 12582912.0f)) + zp_off;
  return static_cast<uint32_t>(min(max(c, -128), 127));
}

// a / d for a >= 1e-12f and a constant divisor d of 255 or 448, by the
// same correction with the constant c = RN(1 / d): checked against IEEE
// division for every binary32 a from 1e-12f to the largest finite value, as
// for 127.  An infinite a (a row holding an infinity) gives a itself, as the
// division does (the correction would give NaN).
__device__ __forceinline__ float div_by_const(float a, float d, float c) {
  const float y = a * c;
  const float e = __builtin_fmaf(-y, d, a);
  const float q = __builtin_fmaf(e, c, y);
  return __builtin_isinf(a) ? a : q;
}

// Asymmetric row parameters from hi = max(row max, 0) and nlo = -min(row
// min, 0): s = max(hi + nlo, 1e-12f) / 255 (= hi - lo; correctly rounded,
// by div_by_const), r = RN(1 / s), zp = clamp(rint(nlo / s) - 128, -128,
// 127) (IEEE divisions; once per row).
__device__ __forceinline__ void row_scale_asym(float hi, float nlo, float& s, float& r, float& zp) {
  s = div_by_const(__builtin_fmaxf(hi + nlo, 1e-12f), 255.0f, 0x1.010102p-8f);  // RN(1 / 255)
  r = 1.0f / s;
  zp = __builtin_rintf(nlo / s) - 128.0f;
  zp = __builtin_fminf(__builtin_fmaxf(zp, -128.0f), 127.0f);
}

// s = max(amax, 1e-12f) / 127 (correctly rounded) and r = RN(1 / s).  The
// division by 127 uses the same correction with the constant RN(1/127): over
// every binary32 value from 1e-12f to the largest finite one it gives the
// IEEE quotient (checked exhaustively).  r stays a true division: the code
// quotients need it correctly rounded.
__device__ __forceinline__ void row_scale(float amax, float& s, float& r) {
  constexpr float kInv127 = 0x1.020408p-7f;  // RN(1 / 127)
  const float a = __builtin_fmaxf(amax, 1e-12f);
  const float y = a * kInv127;
  const float e = __builtin_fmaf(-y, 127.0f, a);
  s = __builtin_fmaf(e, kInv127, y);
  r = 1.0f / s;
}

// ---- FP8 (float8_e4m3fn) codes ----
// "kernels: fused silu_and_mul + dynamic per-token FP8 quantization",
// Algorithm: scale = max(absmax, 1e-12) / 448 (the format's largest finite
// value), optionally clamped from above by scale_ub; the code is the e4m3fn
// value nearest x / scale (ties to even), saturating at +-448.

// s = max(amax, 1e-12f) / 448 (correctly rounded, by div_by_const), then
// min(s, scale_ub) when scale_ub > 0; r = RN(1 / s).  Returns whether the
// bound replaced the row's own scale (then quotients may exceed 448).
__device__ __forceinline__ bool row_scale_fp8(float amax, float scale_ub, float& s, float& r) {
  s = div_by_const(__builtin_fmaxf(amax, 1e-12f), 448.0f, 0x1.24924ap-9f);  // RN(1 / 448)
  const bool bounded = scale_ub > 0.0f && s > scale_ub;
  if (bounded) s = scale_ub;
  r = 1.0f / s;
  return bounded;
}

// x / s, correctly rounded (the same correction as code_of), clamped to
// [-448, 448].  With scale_ub the quotient can exceed the binary32 range:
// y is first clamped to +-1024, which leaves every y that can round to a
// finite code unchanged and keeps the residual step finite; a clamped y gives
// a quotient beyond 1000 in magnitude, which saturates like the true one.
// The residual is formed negated, e' = y s - x, and the quotient as
// y - e' r: the same values as x - y s and y + e r for every nonzero x, but
// for x = -0 the sums are -0 + -0 rather than +0 + -0, so the quotient keeps
// the sign of zero (the codes of +0 and -0 differ).
__device__ __forceinline__ float fp8_ratio(float x, float s, float r) {
  float y = x * r;
  y = __builtin_amdgcn_fmed3f(y, -1024.0f, 1024.0f);
  const float en = __builtin_fmaf(y, s, -x);
  const float q = __builtin_fmaf(-en, r, y);
  return __builtin_amdgcn_fmed3f(q, -448.0f, 448.0f);
}

// fp8_ratio for a row quantized with its own scale s = RN(max(amax, 1e-12)
// / 448) (no scale bound): every |x| <= amax gives |x * r| < 449, so the
// first clamp cannot bind and is left out (the same results).
__device__ __forceinline__ float fp8_ratio_own(float x, float s, float r) {
  const float y = x * r;
  const float en = __builtin_fmaf(y, s, -x);
  const float q = __builtin_fmaf(-en, r, y);
  return __builtin_amdgcn_fmed3f(q, -448.0f, 448.0f);
}

// Four codes packed little-endian (a in byte 0).  v_cvt_pk_fp8_f32 converts
// to OCP e4m3fn on gfx950, rounding to nearest even; its inputs are already
// within +-448, so no value reaches the overflow encodings.
__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

}  // namespace qm
}  // namespace qk
