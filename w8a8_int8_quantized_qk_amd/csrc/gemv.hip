// Decode-shaped INT8 GEMM (m <= 8 rows per launch) for gfx950: a GEMV that
// streams the [K][N] weight from HBM exactly once.
//
// What it computes is the same as the MFMA kernel ("16. Deploying Custom
// Kernels", C++ Kernel Interface; "KV-cache kernels", 02 Scales and
// dequantization).  The shape is the one "dynquant-kernels", What is in here,
// calls the memory-bound decode GEMV, and "KV-cache kernels", 04 What changes
// in the kernel's shape, is the reason for a tiling of its own: with one to
// eight tokens a GEMM tile would be almost all padding while the weight
// streams in.  One to three rows take dot-product instructions
// (gemv_kernel); four to eight take MFMAs with the rows padded to 16
// (gemv_mfma_kernel, further down), where the dot products' VALU work would
// outlast the weight's arrival.
//
// Design of gemv_kernel:
//   * Split-K: a workgroup (8 wave64s, two per SIMD) owns a 512 (k) x 512 (n)
//     block of the weight (128 x 512 for narrow weights, so that there are
//     enough workgroups).  Lane (cg, half) of wave w loads 16 contiguous
//     bytes (columns 16 cg .. 16 cg + 15) of the four rows of row quad
//     2 w + half of each 64-row round: every wave-wide load instruction reads
//     two contiguous 512-byte row segments.  Weight loads are nontemporal
//     (each byte is used once).  A lane keeps several rounds of loads in
//     flight ahead of the round it multiplies (software pipeline).  Only one
//     round (two for more than one row) is issued before the quantization: a
//     CU accepts a limited number of outstanding loads, and waves stalled
//     issuing weight loads would hold up the quantization and with it every
//     multiply.
//   * The four rows of a lane are transposed in registers (v_perm_b32) into
//     sixteen 4-byte columns and multiplied with the matching four activation
//     codes by v_dot4_i32_i8 (exact INT32).  Codes come from LDS.
//   * Partial sums are reduced across the 16 half-waves: a lane swap
//     (v_permlane32_swap) adds the two halves of each wave, each wave stores
//     its sums to LDS, and one thread per column adds the waves' sums.
//     Across the K-slice workgroups each (row, column) has one 64-bit
//     workspace word holding
//     (contributions so far) * 2^40 + (their exact sum); a workgroup adds
//     2^40 + its partial with one returning device-scope atomic.  The partial
//     sums of any subset of the k range stay within +-2^31, so the two fields
//     never interfere, and integer addition is exact in any order.  The lane
//     whose add returns a count of splits - 1 holds the last contribution: it
//     forms the total, applies the dequant epilogue for that column, and
//     returns the word to zero for the next call.  No counters, fences or
//     last-workgroup pass are needed.  (With two rows and a short k range
//     both rows share one word; the settlement code states the field bounds.)
//   * Activation codes are either given (int8 a, scale_a), or the kernel
//     quantizes the m activation rows itself from fp32/bf16/fp16 input with
//     the same arithmetic as the quantization kernels: every workgroup
//     reduces the whole row to the same bit-identical scale and encodes its
//     own k slice; one workgroup per slice writes the codes out when asked.
//     Every wave issues its activation (or code) loads before any wave issues
//     weight loads, and they are used in straight-line code, so the
//     quantization waits only for them and overlaps the weight stream.  The
//     decode linear is then a single launch.
#include "quant_math.h"


namespace qk {
namespace {

constexpr int kThreads = 512;   // 8 waves: two per SIMD
constexpr int kWaves = kThreads / 64;
constexpr int kCols = 512;      // output columns per workgroup: 32 lanes x 16 bytes
constexpr int kRowsK = 512;     // k rows per workgroup (one split-K slice), usually
constexpr int kRounds = kRowsK / 64;  // a round: 16 row quads = 8 waves x 2 half-waves
// Narrow weights (few column tiles) take slices of kNarrowRounds rounds, so
// that more k splits keep enough workgroups streaming: 1 x 4096 x 1792 makes
// 32 workgroups with 512-row slices and 128 with 128-row ones.
constexpr int kNarrowRounds = 2;
constexpr int kMinWorkgroups = 128;
constexpr int kXUnits = 2;      // 16-byte activation units a lane keeps in registers
constexpr int kCountShift = 40; // workspace word: count << 40 | sum (two's complement)
static_assert(kCols == kThreads, "one output column per thread in the reduction");

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// rounds of weight loads (4 x 16 bytes per lane each) kept in flight ahead of
// the round being multiplied; more rows need more accumulator registers.  A
// weight whose width is not a multiple of 16 is read byte by byte (64 loads
// per lane and round, each its own register until the bytes are combined),
// so with 4 or more rows only one round is kept in flight: two overflow the
// 256 registers.
template <int MR, int ROUNDS, bool N16>
constexpr int prefetch_for() {
  if (!N16 && MR >= 4) return 1;
  return (MR <= 2 ? ROUNDS - 1 : (MR == 4 ? 4 : 2)) < ROUNDS - 1
             ? (MR <= 2 ? ROUNDS - 1 : (MR == 4 ? 4 : 2))
             : ROUNDS - 1;
}
// rounds issued before the quantization: a CU accepts only so many
// outstanding loads, and a wave stalled issuing weight loads could not reach
// the quantization (and with it every wave's first multiply).  With more
// rows the quantization takes longer and a second round fits under it
// (measured: 4 rows 16.3 -> 15.9 us, 8 rows 22.4 -> 21.9 us; 1 row best
// with one).  Never more than the rounds kept in flight.
template <int MR, int ROUNDS, bool N16>
constexpr int early_rounds_for() {
  return MR == 1 || ROUNDS <= 2 || prefetch_for<MR, ROUNDS, N16>() < 2 ? 1 : 2;
}

__device__ __forceinline__ void transpose4x4(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                             uint32_t* col) {
  // a..d: rows k0..k3 (byte j = column j) -> col[j]: column j (byte i = row ki)
  const uint32_t t0 = __builtin_amdgcn_perm(b, a, 0x05010400u);
  const uint32_t t1 = __builtin_amdgcn_perm(b, a, 0x07030602u);
  const uint32_t t2 = __builtin_amdgcn_perm(d, c, 0x05010400u);
  const uint32_t t3 = __builtin_amdgcn_perm(d, c, 0x07030602u);
  col[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  col[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  col[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  col[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Workgroup-wide max of MR values at once (one barrier).
template <int MR>
__device__ __forceinline__ void block_max_rows(float (&v)[MR]) {
  __shared__ uint32_t part[MR][kWaves];
#pragma unroll
  for (int m = 0; m < MR; ++m) v[m] = qm::wave_max_nonneg(v[m]);
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int m = 0; m < MR; ++m) part[m][threadIdx.x >> 6] = __float_as_uint(v[m]);
  __syncthreads();
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    uint32_t r = part[m][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) r = qm::max_u32(r, part[m][w]);
    v[m] = __uint_as_float(r);
  }
}

// The k slice's activation codes, staged into LDS: int8 codes with their
// scales (XDT < 0), or activations of dtype XDT quantized here (every
// workgroup reduces whole rows to the same bit-identical scales and encodes
// its own slice; q_w, when given, receives this slice's codes).  Rows M..MR-1
// and k past K get zero codes.  `early` issues the first weight loads: it
// runs after every wave has issued its activation loads and before the
// quantization (K > 0).
template <int MR, int XDT, int ROWSK, typename Early>
__device__ __forceinline__ void stage_codes(const void* __restrict__ a,
                                            const float* __restrict__ scale_a, int M, int K,
                                            int k0, int8_t* __restrict__ q_w,
                                            float* __restrict__ s_out,
                                            int32_t (&q_lds)[MR][ROWSK / 4], float (&s_row)[MR],
                                            Early&& early) {
  constexpr int kSliceWords = ROWSK / 4;  // code words of one row's k slice
  constexpr int kCodeWords = MR * kSliceWords;
  constexpr int kCodeRegs = (kCodeWords + kThreads - 1) / kThreads;
  using E = qm::Elem<XDT < 0 ? QK_F32 : XDT>;
  constexpr int P = E::kPerUnit;
  const int t = threadIdx.x;

  const int units = K / P;  // 16-byte activation units per row (fused path)
  const bool x_in_regs = units <= kThreads * kXUnits;
  uint4 xr[MR][kXUnits];
  int32_t cr[kCodeRegs];
  if constexpr (XDT >= 0) {
    if (x_in_regs) {
#pragma unroll
      for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int j = 0; j < kXUnits; ++j) {
          const int mm = min(m, M - 1);
          const int u = min(t + kThreads * j, units - 1);  // duplicates add nothing to a max
          xr[m][j] = *reinterpret_cast<const uint4*>(
              static_cast<const char*>(a) + (static_cast<size_t>(mm) * K + static_cast<size_t>(u) * P) * E::kBytes);
        }
    }
  } else {
    const int8_t* q = static_cast<const int8_t*>(a);
#pragma unroll
    for (int j = 0; j < kCodeRegs; ++j) {
      const int idx = t + kThreads * j;
      const int m = idx / kSliceWords;
      const int k = k0 + 4 * (idx % kSliceWords);
      cr[j] = (idx < kCodeWords && m < M && k < K)
                  ? *reinterpret_cast<const int32_t*>(q + static_cast<size_t>(m) * K + k)
                  : 0;
    }
    if (t < MR) s_row[t] = (t < M && scale_a) ? scale_a[t] : 0.0f;
  }
  // the slice units this thread encodes: unit su of row m, with
  // m * kSliceUnits + su = t + kThreads * i, spread over every thread (one
  // wave per row would serialize the divisions of all rows)
  constexpr int kSliceUnits = ROWSK / P;
  constexpr int kEncRegs = (MR * kSliceUnits + kThreads - 1) / kThreads;
  uint4 er[kEncRegs];
  if constexpr (XDT >= 0) {
    if (x_in_regs) {
#pragma unroll
      for (int i = 0; i < kEncRegs; ++i) {
        const int idx = min(t + kThreads * i, MR * kSliceUnits - 1);
        const int mm = min(idx / kSliceUnits, M - 1);
        const int u = min(k0 / P + idx % kSliceUnits, units - 1);
        er[i] = *reinterpret_cast<const uint4*>(
            static_cast<const char*>(a) + (static_cast<size_t>(mm) * K + static_cast<size_t>(u) * P) * E::kBytes);
      }
    }
  }
  // A CU serves its loads in issue order: without this barrier the later
  // waves' activation loads would queue behind the earlier waves' weight
  // loads.  (Execution barrier only; nothing needs to be visible yet.)
  __builtin_amdgcn_s_barrier();
  early();

  // ---- codes of rows k0 .. k0 + 511 into LDS ----
  if constexpr (XDT < 0) {
#pragma unroll
    for (int j = 0; j < kCodeRegs; ++j) {
      const int idx = t + kThreads * j;
      if (idx < kCodeWords) q_lds[idx / kSliceWords][idx % kSliceWords] = cr[j];
    }
  } else if (x_in_regs) {
    // the scale needs the whole row: every workgroup reduces it (identical bits)
    float amax[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      amax[m] = 0.0f;
#pragma unroll
      for (int j = 0; j < kXUnits; ++j) {
        float v[P];
        E::unpack(xr[m][j], v);
#pragma unroll
        for (int e = 0; e < P; ++e) amax[m] = __builtin_fmaxf(amax[m], __builtin_fabsf(v[e]));
      }
    }
    block_max_rows<MR>(amax);
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      float s, r;
      qm::row_scale(amax[m], s, r);
      if (t == 0) s_row[m] = s;
      if (blockIdx.x == 0 && t == 0 && s_out && m < M) s_out[m] = s;
    }
#pragma unroll
    for (int i = 0; i < kEncRegs; ++i) {
      const int idx = t + kThreads * i;
      if (idx >= MR * kSliceUnits) continue;
      const int m = idx / kSliceUnits;
      const int su = idx % kSliceUnits;
      const int u = k0 / P + su;
      float am = amax[0];
#pragma unroll
      for (int mm = 1; mm < MR; ++mm) am = m == mm ? amax[mm] : am;
      float s, r;
      qm::row_scale(am, s, r);
      float v[P];
      E::unpack(er[i], v);
      // padding rows and units past K (the tail of the last slice): zero words
      const bool live = m < M && u < units;
#pragma unroll
      for (int e4 = 0; e4 < P / 4; ++e4) {
        const uint32_t word =
            live ? qm::pack4(qm::code_of(v[4 * e4], s, r), qm::code_of(v[4 * e4 + 1], s, r),
                             qm::code_of(v[4 * e4 + 2], s, r), qm::code_of(v[4 * e4 + 3], s, r))
                 : 0u;
        const int kw = su * (P / 4) + e4;  // codes of elements k0 + 4 kw .. + 3
        q_lds[m][kw] = static_cast<int32_t>(word);
        if (q_w && live)  // one workgroup per k slice writes the codes
          *reinterpret_cast<uint32_t*>(q_w + static_cast<size_t>(m) * K + k0 + 4 * kw) = word;
      }
    }
  } else {
    // rows too long to hold in registers: re-read them (from L2) per pass
    for (int m = 0; m < MR; ++m) {
      if (m >= M) {  // padding rows: zero codes
        for (int wd = t; wd < kSliceWords; wd += kThreads) q_lds[m][wd] = 0;
        continue;
      }
      const char* xrow = static_cast<const char*>(a) + static_cast<size_t>(m) * K * E::kBytes;
      auto unit = [&](int u) -> uint4 {
        return *reinterpret_cast<const uint4*>(xrow + static_cast<size_t>(u) * 16);
      };
      float amax = 0.0f;
      for (int u = t; u < units; u += kThreads) {
        float v[P];
        E::unpack(unit(u), v);
#pragma unroll
        for (int e = 0; e < P; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[e]));
      }
      amax = qm::block_max<kThreads>(amax);
      float s, r;
      qm::row_scale(amax, s, r);
      if (t == 0) s_row[m] = s;
      if (blockIdx.x == 0 && t == 0 && s_out) s_out[m] = s;
      for (int wd = t; wd < kSliceWords; wd += kThreads)
        if (k0 + 4 * wd >= K) q_lds[m][wd] = 0;
      const int u_lo = k0 / P;
      const int u_hi = min(units, (k0 + ROWSK) / P);
      for (int u = u_lo + t; u < u_hi; u += kThreads) {
        float v[P];
        E::unpack(unit(u), v);
#pragma unroll
        for (int e4 = 0; e4 < P / 4; ++e4) {
          const uint32_t word =
              qm::pack4(qm::code_of(v[4 * e4], s, r), qm::code_of(v[4 * e4 + 1], s, r),
                        qm::code_of(v[4 * e4 + 2], s, r), qm::code_of(v[4 * e4 + 3], s, r));
          const int kw = u * (P / 4) + e4;
          q_lds[m][kw - k0 / 4] = static_cast<int32_t>(word);
          if (q_w)
            *reinterpret_cast<uint32_t*>(q_w + static_cast<size_t>(m) * K + 4 * kw) = word;
        }
      }
      __syncthreads();  // block_max reuses its LDS between rows
    }
  }
  __syncthreads();

}

// XDT < 0: `a` holds int8 codes [M][K] and scale_a their scales.
// XDT >= 0: `a` holds activations [M][K] of that dtype (16-byte aligned rows,
// K % 16 == 0), quantized here.
template <int MR, int XDT, bool N16, int ROUNDS>
__global__ __launch_bounds__(kThreads) void gemv_kernel(
    const void* __restrict__ a, const int8_t* __restrict__ w, int32_t* __restrict__ c,
    const float* __restrict__ scale_a, const float* __restrict__ scale_b, float output_scale,
    void* __restrict__ out, int out_dtype, int M, int N, int K, int8_t* __restrict__ q_out,
    float* __restrict__ s_out, unsigned long long* __restrict__ ws, int col_tiles, int splits) {
  constexpr int kRowsK = 64 * ROUNDS;  // this instance's k slice
  constexpr int kRounds = ROUNDS;
  constexpr int PD = prefetch_for<MR, ROUNDS, N16>();
  constexpr int kEarlyRounds = early_rounds_for<MR, ROUNDS, N16>();
  static_assert(PD >= kEarlyRounds && PD < kRounds, "prefetch distance");
  __shared__ int32_t q_lds[MR][kRowsK / 4];  // codes of this k slice, 4 per word
  __shared__ float s_row[MR];
  // per-wave partial sums: column c of row m of wave w at [w][m][c ^ ((c >> 6) & 7)]
  __shared__ int wsum[kWaves][MR][kCols];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int ct = blockIdx.x % col_tiles;
  const int ks = blockIdx.x / col_tiles;
  const int n0 = ct * kCols;
  const int k0 = ks * kRowsK;
  const int cg = lane & 31;                  // 16-column group
  const int quad = 2 * wave + (lane >> 5);   // row quad within a 64-row round
  const int gn = n0 + 16 * cg;

  if (K == 0) {
    // empty reduction: acc = 0 (one workgroup per column tile, no workspace);
    // the scale of an empty row is the guard's
    const int n = n0 + t;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      if (m >= M) continue;
      float s_m, r_m;
      if constexpr (XDT < 0) {
        s_m = scale_a ? scale_a[m] : 0.0f;
      } else {
        qm::row_scale(0.0f, s_m, r_m);
        if (blockIdx.x == 0 && t == 0 && s_out) s_out[m] = s_m;
      }
      if (n >= N) continue;
      const size_t o_idx = static_cast<size_t>(m) * N + n;
      if (c) c[o_idx] = 0;
      if (out) {
        const float f = (0.0f * s_m) * (scale_b[n] * output_scale);
        if (out_dtype == QK_BF16)
          static_cast<uint16_t*>(out)[o_idx] = to_bf16(f);
        else
          static_cast<float*>(out)[o_idx] = f;
      }
    }
    return;
  }

  // weight loads of one round (all loop indices below are compile-time after
  // unrolling, so wr stays in registers); rows past K (zero codes) and
  // columns past N (never stored) read clamped, valid addresses instead of
  // branching
  uint32_t wr[kRounds][4][4];
  auto load_round = [&](int round) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int k = min(k0 + round * 64 + 4 * quad + r, K - 1);
      const int8_t* row = w + static_cast<size_t>(k) * N;
      if constexpr (N16) {
        const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(row + min(gn, N - 16)));
        wr[round][r][0] = v.x;
        wr[round][r][1] = v.y;
        wr[round][r][2] = v.z;
        wr[round][r][3] = v.w;
      } else {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          uint32_t x = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            x |= static_cast<uint32_t>(static_cast<uint8_t>(row[min(gn + 4 * q4 + e, N - 1)])) << (8 * e);
          wr[round][r][q4] = x;
        }
      }
    }
  };

  // ---- activation (or code) loads first, then the weight (K > 0 from here) ----
  stage_codes<MR, XDT, kRowsK>(a, scale_a, M, K, k0, ct == 0 ? q_out : nullptr, s_out, q_lds, s_row,
                               [&] {
#pragma unroll
                                 for (int round = 0; round < kEarlyRounds; ++round) load_round(round);
                               });

  // ---- multiply the streamed weight with the codes ----
  int acc[MR][16];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[m][j] = 0;

  // software pipeline: round `round` is multiplied while rounds up to
  // round + PD are in flight
#pragma unroll
  for (int round = 0; round < kRounds; ++round) {
    if (round == 0) {
#pragma unroll
      for (int q = kEarlyRounds; q <= PD; ++q) load_round(q);
    } else if (round + PD < kRounds) {
      load_round(round + PD);
    }
    uint32_t col[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      transpose4x4(wr[round][0][q4], wr[round][1][q4], wr[round][2][q4], wr[round][3][q4], &col[4 * q4]);
    const int kw = round * 16 + quad;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const int qd = q_lds[m][kw];
#pragma unroll
      for (int j = 0; j < 16; ++j)
        acc[m][j] = __builtin_amdgcn_sdot4(static_cast<int>(col[j]), qd, acc[m][j], false);
    }
  }

  // ---- reduce within the workgroup ----
  // The two half-waves hold the same 512 columns (row quads 2w and 2w + 1):
  // a lane swap across the halves adds them, lanes < 32 ending with columns
  // 16 cg + jj and lanes >= 32 with 16 cg + 8 + jj (jj < 8).  Each wave then
  // stores its partial sums with plain LDS stores, and after one barrier
  // thread t adds the kWaves partials of column t.  The XOR swizzle keeps
  // both the stores and the column-major reads free of bank conflicts.
  auto wsum_slot = [](int col) { return col ^ ((col >> 6) & 7); };
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const auto sw = __builtin_amdgcn_permlane32_swap(acc[m][jj], acc[m][jj + 8], false, false);
      const int col = 16 * cg + jj + 8 * (lane >> 5);
      wsum[wave][m][wsum_slot(col)] = static_cast<int>(sw[0]) + static_cast<int>(sw[1]);
    }
  __syncthreads();
  int part_sum[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    int v = 0;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) v += wsum[w2][m][wsum_slot(t)];
    part_sum[m] = v;
  }

  // ---- across the split-K workgroups: one returning 64-bit add per (row,
  //      column) carrying the arrival count and the exact partial sum ----
  const int n = n0 + t;
  if (n >= N) return;
  auto finish = [&](int m, int v) {
    const size_t o_idx = static_cast<size_t>(m) * N + n;
    if (c) c[o_idx] = v;
    if (out) {
      const float f = (static_cast<float>(v) * s_row[m]) * (scale_b[n] * output_scale);
      if (out_dtype == QK_BF16)
        static_cast<uint16_t*>(out)[o_idx] = to_bf16(f);
      else
        static_cast<float*>(out)[o_idx] = f;
    }
  };
  if constexpr (MR == 2) {
    // Two rows share one word while splits * kRowsK <= 4096: bits 56-63
    // count the arrivals, bits 28-55 and 0-27 hold, for rows 1 and 0, the sum
    // of (partial + B) with B = 2^14 kRowsK >= |partial|, so each biased term
    // lies in [0, 2 B] and all of them together stay below 2 B splits <= 2^27:
    // no field carries into the next, and subtracting count * B recovers the
    // exact earlier sum.  (Half the returning atomics of two words.)
    constexpr long long kB = 16384ll * kRowsK;
    constexpr unsigned long long kF = (1ull << 28) - 1;
    if (static_cast<long long>(splits) * kRowsK <= 4096) {
      const unsigned long long add =
          (1ull << 56) + static_cast<unsigned long long>(part_sum[0] + kB) +
          (static_cast<unsigned long long>(part_sum[1] + kB) << 28);
      const unsigned long long o = __hip_atomic_fetch_add(&ws[n], add, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
      const long long count = static_cast<long long>(o >> 56);
      if (count != splits - 1) return;
      __hip_atomic_store(&ws[n], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      finish(0, static_cast<int>(static_cast<long long>(o & kF) - count * kB) + part_sum[0]);
      if (M > 1)
        finish(1, static_cast<int>(static_cast<long long>((o >> 28) & kF) - count * kB) + part_sum[1]);
      return;
    }
  }
  unsigned long long prev[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (m >= M) continue;
    const unsigned long long add =
        (1ull << kCountShift) + static_cast<unsigned long long>(static_cast<long long>(part_sum[m]));
    prev[m] = __hip_atomic_fetch_add(&ws[static_cast<size_t>(m) * N + n], add, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
  }
  const float sb = out ? scale_b[n] * output_scale : 0.0f;
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (m >= M) continue;
    const long long o = static_cast<long long>(prev[m]);
    const long long count = (o + (1ll << (kCountShift - 1))) >> kCountShift;
    if (count != splits - 1) continue;
    // last contribution: total = earlier sum + this partial; word back to zero
    const int v = static_cast<int>(o - (count << kCountShift)) + part_sum[m];
    __hip_atomic_store(&ws[static_cast<size_t>(m) * N + n], 0ull, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    const size_t o_idx = static_cast<size_t>(m) * N + n;
    if (c) c[o_idx] = v;
    if (out) {
      const float f = (static_cast<float>(v) * s_row[m]) * sb;
      if (out_dtype == QK_BF16)
        static_cast<uint16_t*>(out)[o_idx] = to_bf16(f);
      else
        static_cast<float*>(out)[o_idx] = f;
    }
  }
  (void)finish;
}

// Four to eight rows: the products on the matrix cores.  With v_dot4 the
// VALU work grows with the row count (eight rows: 1024 dot instructions per
// wave, more than the weight's arrival time); one v_mfma_i32_16x16x64_i8
// multiplies 64 k of 16 columns by up to 16 rows (rows 8..15 are zero
// here), so the multiply no longer grows with m.
//   * Each lane loads CB bytes (CB consecutive columns) per weight row, so a
//     workgroup covers 16 CB columns and, at the same 256 KB per workgroup,
//     16384 / CB k rows (16 B: 256 columns x 1024 k; 4 B: 64 columns x 4096
//     k, where one workgroup holds a column's whole k range and no split-K
//     settlement is needed for k <= 4096).
//   * Wave w multiplies k rows kWaveRows w .. kWaveRows (w + 1) - 1 of the
//     block in 64-deep steps.  Lane (p = lane % 16, g = lane / 16) loads
//     columns CB p .. CB p + CB - 1 of the 16 rows 16 g .. 16 g + 15 of a
//     step: every wave-wide load reads four contiguous 16 CB-byte row
//     segments.
//   * 4 x 4 byte transposes turn a lane's 16 rows x CB columns into CB
//     16-byte column operands (byte t = row 16 g + t).  MFMA j takes column
//     CB p + j from lane p, and from every lane the 16 activation codes of its
//     row p (from LDS) at the same k, 16 g .. 16 g + 15: A and B pair the same
//     k in every byte, so each output is an exact INT32 dot product whatever
//     order the instruction sums in.
//   * Output of MFMA j: lane (p, g) holds rows 4 g .. 4 g + 3 of column
//     CB p + j.  The eight waves' partial sums meet in LDS; each thread then
//     owns CB / 4 rows of one column and either writes them (one k split) or
//     settles them through the workspace as gemv_kernel does.
//   Measured at 8 x 4096 x 14336: 16-byte loads (4 splits) 17.2 us per call,
//   8-byte (2 splits) 17.8, 4-byte (no split) 28.3; the split-K settlement
//   costs ~3.5 us of the 17.2 (v_dot4 kernel: 21.9 us).
constexpr int kMEarlyBytes = 128;  // weight bytes per lane issued before the quantization

template <int CB>
struct MfmaTiling {
  static constexpr int kCols = 16 * CB;            // columns per workgroup
  static constexpr int kRowsK = 16384 / CB;        // k rows per workgroup (256 KB of weight)
  static constexpr int kWaveRows = kRowsK / kWaves;
  static constexpr int kSteps = kWaveRows / 64;    // 64-deep MFMA steps per wave
  static constexpr int kRowsPerThread = CB / 4;    // rows of one column each thread settles
  static_assert(CB == 4 || CB == 8 || CB == 16, "load width");
  static_assert(8 * kCols == kThreads * kRowsPerThread, "one (row, column) per thread and row");
};

template <int CB>
struct WeightLoad;
template <>
struct WeightLoad<16> {
  static __device__ __forceinline__ void get(const int8_t* src, uint32_t* d) {
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(src));
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
  }
};
template <>
struct WeightLoad<8> {
  typedef unsigned v2u __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ void get(const int8_t* src, uint32_t* d) {
    const v2u v = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(src));
    d[0] = v.x; d[1] = v.y;
  }
};
template <>
struct WeightLoad<4> {
  static __device__ __forceinline__ void get(const int8_t* src, uint32_t* d) {
    d[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(src));
  }
};

template <int XDT, int CB>
__global__ __launch_bounds__(kThreads) void gemv_mfma_kernel(
    const void* __restrict__ a, const int8_t* __restrict__ w, int32_t* __restrict__ c,
    const float* __restrict__ scale_a, const float* __restrict__ scale_b, float output_scale,
    void* __restrict__ out, int out_dtype, int M, int N, int K, int8_t* __restrict__ q_out,
    float* __restrict__ s_out, unsigned long long* __restrict__ ws, int col_tiles, int splits) {
  using T = MfmaTiling<CB>;
  constexpr int MR = 8;
  constexpr int D = CB / 4;  // dwords per lane per weight row
  typedef int v4i __attribute__((ext_vector_type(4)));
  __shared__ int32_t q_lds[MR][T::kRowsK / 4];
  __shared__ float s_row[MR];
  // partial sums of wave w: row m, column col at [w][m][slot(m, col)]
  __shared__ int wsum[kWaves][MR][T::kCols];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int p = lane & 15;
  const int g = lane >> 4;
  const int ct = blockIdx.x % col_tiles;
  const int ks = blockIdx.x / col_tiles;
  const int n0 = ct * T::kCols;
  const int k0 = ks * T::kRowsK;
  // columns past N (never stored) and rows past K (zero codes) read
  // clamped, valid addresses; N % 16 == 0 here
  const int gn = min(n0 + CB * p, N - CB);

  uint32_t wr[T::kSteps][16][D];
  auto load_row = [&](int st, int tt) {
    const int k = min(k0 + T::kWaveRows * wave + 64 * st + 16 * g + tt, K - 1);
    WeightLoad<CB>::get(w + static_cast<size_t>(k) * N + gn, wr[st][tt]);
  };
  constexpr int kEarly = kMEarlyBytes / CB;  // loads, in (step, row) order
  static_assert(kEarly <= 16 * T::kSteps, "early loads");

  stage_codes<MR, XDT, T::kRowsK>(a, scale_a, M, K, k0, ct == 0 ? q_out : nullptr, s_out, q_lds,
                                  s_row, [&] {
#pragma unroll
                                    for (int e = 0; e < kEarly; ++e) load_row(e / 16, e % 16);
                                  });
#pragma unroll
  for (int e = kEarly; e < 16 * T::kSteps; ++e) load_row(e / 16, e % 16);

  v4i acc[CB];
#pragma unroll
  for (int j = 0; j < CB; ++j) acc[j] = v4i{0, 0, 0, 0};
#pragma unroll
  for (int st = 0; st < T::kSteps; ++st) {
    // codes of row p at k = kWaveRows w + 64 st + 16 g .. + 15 of the block
    const v4i av = p < MR ? *reinterpret_cast<const v4i*>(
                                &q_lds[p & (MR - 1)][(T::kWaveRows * wave + 64 * st + 16 * g) / 4])
                          : v4i{0, 0, 0, 0};
    uint32_t col[4][CB];  // [4-row batch][column]: bytes = rows 4 b .. 4 b + 3
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int q4 = 0; q4 < D; ++q4)
        transpose4x4(wr[st][4 * b][q4], wr[st][4 * b + 1][q4], wr[st][4 * b + 2][q4],
                     wr[st][4 * b + 3][q4], &col[b][4 * q4]);
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const v4i bv = v4i{static_cast<int>(col[0][j]), static_cast<int>(col[1][j]),
                         static_cast<int>(col[2][j]), static_cast<int>(col[3][j])};
      acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, acc[j], 0, 0, 0);
    }
  }

  // ---- reduce within the workgroup ----
  // slot: the column's CB-block index XORed into its low bits, and bit 4
  // flipped for rows 4..7, so that the 32 lanes of a store (columns CB p + j
  // of two row groups) and 64 consecutive columns of a read hit distinct
  // banks
  auto slot = [](int m, int col) { return col ^ ((col / CB) & (CB - 1)) ^ ((m & 4) << 2); };
  if (g < 2) {
#pragma unroll
    for (int j = 0; j < CB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * g + i;
        wsum[wave][m][slot(m, CB * p + j)] = acc[j][i];
      }
  }
  __syncthreads();
  constexpr int R = T::kRowsPerThread;
  const int colx = t % T::kCols;
  const int m0 = R * (t / T::kCols);  // rows m0 .. m0 + R - 1
  int part_sum[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int m = m0 + i;
    int v = 0;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) v += wsum[w2][m][slot(m, colx)];
    part_sum[i] = v;
  }

  const int n = n0 + colx;
  if (n >= N) return;
  const float sb = out ? scale_b[n] * output_scale : 0.0f;
  auto finish = [&](int m, int v) {
    const size_t o_idx = static_cast<size_t>(m) * N + n;
    if (c) c[o_idx] = v;
    if (out) {
      const float f = (static_cast<float>(v) * s_row[m]) * sb;
      if (out_dtype == QK_BF16)
        static_cast<uint16_t*>(out)[o_idx] = to_bf16(f);
      else
        static_cast<float*>(out)[o_idx] = f;
    }
  };
  if (splits == 1) {  // the whole k range is here
#pragma unroll
    for (int i = 0; i < R; ++i)
      if (m0 + i < M) finish(m0 + i, part_sum[i]);
    return;
  }
  // ---- across the split-K workgroups ----
  // With at most 4 splits (k <= 4096) two rows share one 64-bit workspace
  // word, halving the returning atomics (measured at 8 x 4096 x 14336: 16.9
  // -> 15.8 us): bits 56-58 count the arrivals, bits 28-55 and 0-27 hold,
  // for rows 2p + 1 and 2p, the sum of (partial + 2^24) over the arrivals.
  // A split covers at most 1024 k, so |partial| <= 128 * 128 * 1024 = 2^24:
  // each biased term lies in [0, 2^25] and four of them stay below 2^28, so
  // no field carries into the next, and subtracting count * 2^24 from a
  // field recovers the exact sum of the earlier partials.
  static_assert(T::kRowsK <= 1024, "packed fields hold partial sums of at most 1024 k");
  if (R == 4 && splits <= 4) {
    constexpr unsigned long long kB = 1ull << 24, kF = (1ull << 28) - 1;
    unsigned long long prev2[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int m = m0 + 2 * h;
      if (m >= M) continue;
      const unsigned long long add =
          (1ull << 56) + (static_cast<unsigned long long>(part_sum[2 * h] + static_cast<long long>(kB))) +
          (static_cast<unsigned long long>(part_sum[2 * h + 1] + static_cast<long long>(kB)) << 28);
      prev2[h] = __hip_atomic_fetch_add(&ws[static_cast<size_t>(m / 2) * N + n], add,
                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int m = m0 + 2 * h;
      if (m >= M) continue;
      const unsigned long long o = prev2[h];
      const long long count = static_cast<long long>(o >> 56);
      if (count != splits - 1) continue;
      __hip_atomic_store(&ws[static_cast<size_t>(m / 2) * N + n], 0ull, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      const long long lo = static_cast<long long>(o & kF) - count * static_cast<long long>(kB);
      const long long hi = static_cast<long long>((o >> 28) & kF) - count * static_cast<long long>(kB);
      finish(m, static_cast<int>(lo) + part_sum[2 * h]);
      if (m + 1 < M) finish(m + 1, static_cast<int>(hi) + part_sum[2 * h + 1]);
    }
    return;
  }
  // ---- across the split-K workgroups (as in gemv_kernel) ----
  unsigned long long prev[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int m = m0 + i;
    if (m >= M) continue;
    const unsigned long long add =
        (1ull << kCountShift) + static_cast<unsigned long long>(static_cast<long long>(part_sum[i]));
    prev[i] = __hip_atomic_fetch_add(&ws[static_cast<size_t>(m) * N + n], add, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int m = m0 + i;
    if (m >= M) continue;
    const long long o = static_cast<long long>(prev[i]);
    const long long count = (o + (1ll << (kCountShift - 1))) >> kCountShift;
    if (count != splits - 1) continue;
    __hip_atomic_store(&ws[static_cast<size_t>(m) * N + n], 0ull, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    finish(m, static_cast<int>(o - (count << kCountShift)) + part_sum[i]);
  }
}

// Row-group pointers of one launch.
struct RowGroup {
  const void* a;
  int32_t* c;
  const float* sa;
  void* out;
  int8_t* q_out;
  float* s_out;
};

template <int XDT>
RowGroup row_group(const GemvArgs& g, int row0) {
  const size_t xsz = XDT == QK_F32 ? 4 : (XDT < 0 ? 1 : 2);
  RowGroup r;
  r.a = static_cast<const char*>(g.a) + static_cast<size_t>(row0) * g.k * xsz;
  r.c = g.c ? g.c + static_cast<size_t>(row0) * g.n : nullptr;
  r.sa = g.scale_a ? g.scale_a + row0 : nullptr;
  r.out = nullptr;
  if (g.out) {
    const size_t esz = g.out_dtype == QK_BF16 ? 2 : 4;
    r.out = static_cast<char*>(g.out) + static_cast<size_t>(row0) * g.n * esz;
  }
  r.q_out = g.q_out ? g.q_out + static_cast<size_t>(row0) * g.k : nullptr;
  r.s_out = g.s_out ? g.s_out + row0 : nullptr;
  return r;
}

constexpr int kMfmaLoadBytes = 16;

template <int XDT>
hipError_t launch_mfma(const GemvArgs& g, int row0, int rows, hipStream_t stream) {
  using T = MfmaTiling<kMfmaLoadBytes>;
  const RowGroup r = row_group<XDT>(g, row0);
  const int col_tiles = (g.n + T::kCols - 1) / T::kCols;
  const int splits = (g.k + T::kRowsK - 1) / T::kRowsK;
  auto* ws = static_cast<unsigned long long*>(g.workspace);
  const dim3 grid(static_cast<unsigned>(col_tiles) * static_cast<unsigned>(splits));
  return launch(gemv_mfma_kernel<XDT, kMfmaLoadBytes>, grid, dim3(kThreads), 0, stream, r.a, g.b, r.c, r.sa,
                g.scale_b, g.output_scale, r.out, g.out_dtype, rows, g.n, g.k, r.q_out, r.s_out,
                ws, col_tiles, splits);
}

template <int MR, int XDT, int ROUNDS>
hipError_t launch_rounds(const GemvArgs& g, int row0, int rows, hipStream_t stream) {
  const RowGroup r = row_group<XDT>(g, row0);
  const int col_tiles = (g.n + kCols - 1) / kCols;
  const int splits = g.k > 0 ? (g.k + 64 * ROUNDS - 1) / (64 * ROUNDS) : 1;
  auto* ws = static_cast<unsigned long long*>(g.workspace);
  const dim3 grid(static_cast<unsigned>(col_tiles) * static_cast<unsigned>(splits));
  if (g.n % 16 == 0 && reinterpret_cast<uintptr_t>(g.b) % 16 == 0)
    return launch(gemv_kernel<MR, XDT, true, ROUNDS>, grid, dim3(kThreads), 0, stream, r.a, g.b,
                  r.c, r.sa, g.scale_b, g.output_scale, r.out, g.out_dtype, rows, g.n, g.k, r.q_out,
                  r.s_out, ws, col_tiles, splits);
  return launch(gemv_kernel<MR, XDT, false, ROUNDS>, grid, dim3(kThreads), 0, stream, r.a, g.b,
                r.c, r.sa, g.scale_b, g.output_scale, r.out, g.out_dtype, rows, g.n, g.k, r.q_out,
                r.s_out, ws, col_tiles, splits);
}

template <int MR, int XDT>
hipError_t launch_mr(const GemvArgs& g, int row0, int rows, hipStream_t stream) {
  if constexpr (MR <= 2) {
    const long long wide = static_cast<long long>((g.n + kCols - 1) / kCols) *
                           ((g.k + kRowsK - 1) / kRowsK);
    if (g.k > kRowsK && wide < kMinWorkgroups)
      return launch_rounds<MR, XDT, kNarrowRounds>(g, row0, rows, stream);
  }
  return launch_rounds<MR, XDT, kRounds>(g, row0, rows, stream);
}

template <int XDT>
hipError_t launch_rows(const GemvArgs& g, hipStream_t stream) {
  for (int row0 = 0; row0 < g.m; row0 += kGemvMaxRows) {
    const int rows = g.m - row0 < kGemvMaxRows ? g.m - row0 : kGemvMaxRows;
    hipError_t e;
    const bool mfma_ok =
        g.k > 0 && g.n >= 16 && g.n % 16 == 0 && reinterpret_cast<uintptr_t>(g.b) % 16 == 0;
    if (rows >= 4 && mfma_ok)  // measured: v_dot4 ahead at 3 rows, level at 4, behind from 5
      e = launch_mfma<XDT>(g, row0, rows, stream);
    else if (rows == 1)
      e = launch_mr<1, XDT>(g, row0, rows, stream);
    else if (rows == 2)
      e = launch_mr<2, XDT>(g, row0, rows, stream);
    else if (rows <= 4)
      e = launch_mr<4, XDT>(g, row0, rows, stream);
    else
      e = launch_mr<8, XDT>(g, row0, rows, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

size_t gemv_workspace_bytes(int n) {
  const size_t bytes = static_cast<size_t>(kGemvMaxRows) * static_cast<size_t>(n) * 8;
  return (bytes + 255) / 256 * 256;
}

hipError_t launch_gemv(const GemvArgs& g, hipStream_t stream) {
  switch (g.x_dtype) {
    case -1: return launch_rows<-1>(g, stream);
    case QK_F32: return launch_rows<QK_F32>(g, stream);
    case QK_BF16: return launch_rows<QK_BF16>(g, stream);
    case QK_F16: return launch_rows<QK_F16>(g, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qk
