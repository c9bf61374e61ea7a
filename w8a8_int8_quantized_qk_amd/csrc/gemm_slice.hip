// GEMMs in which every wave multiplies whole 128-byte k slices, on CDNA4
// matrix cores, with binary32 accumulators and the dequant epilogue fused:
//
//   FP8 (float8_e4m3fn) x FP8 (the FP8 codes of "kernels: fused silu_and_mul
//   + dynamic per-token FP8 quantization", Purpose and Algorithm, fed to the
//   scaled GEMM of "16. Deploying Custom Kernels", C++ Kernel Interface):
//     acc[i][j] = sum_t value(a[i][t]) * value(B(t, j))
//     out[i][j] = (acc * scale_a[i]) * (scale_b[j] * output_scale)
//
//   INT8 x INT8 with per-group weight scales ("KV-cache kernels", 02 Scales
//   and dequantization and 03 Where scales come from: one scale per group of
//   64-128 channels), the groups of G consecutive k of each output column:
//     acc[i][j] = sum_g scale_b[g][j] * P_g[i][j],  P_g the INT32 partial of group g
//     out[i][j] = (acc * scale_a[i]) * output_scale
//
//   c[i][j] = acc (optional, binary32) for both.
//
// Design for gfx950:
//   * Workgroup tile, k slices, LDS layouts, global-to-LDS transfers and
//     XCD-aware tile order are the INT8 kernel's (gemm_tile.h).  The eight
//     waves each own a 64 x 64 sub-tile (4 x 2 of them) over whole slices,
//     and a lane holds 32 bytes of a row (A) or column (B): the 16-byte
//     chunks l / 16 (k 0..63 of the slice across the lane groups) and
//     4 + l / 16 (k 64..127).  No partial sums cross waves.
//   * FP8: one v_mfma_f32_16x16x128_f8f6f4 (both operands e4m3, no block
//     scales) per fragment pair and slice; the older 16x16x32 FP8 form
//     issues at half its rate on this chip.  Any assignment of k to (lane
//     group, register byte) is a correct product as long as A and B use the
//     same one, which holds because both are built the same way.
//   * INT8 with group scales: per fragment pair and slice two
//     v_mfma_i32_16x16x64_i8 on the two 64-byte halves.  With G = 128 the
//     second accumulates onto the first (one group per slice); with G = 64
//     each starts from zero (two groups per slice).  The INT32 partial of a
//     group is exact and below 2^24 in magnitude, so its conversion to
//     binary32 is exact; it is added into the binary32 accumulator with one
//     fused multiply-add by the group's scale, issued two MFMA units later so
//     the conversion does not wait for the matrix core.  A lane's four
//     accumulator registers share one column, so a lane needs one scale per
//     fragment column and group; the next slice's scales are loaded during
//     the current slice, ahead of the DMA parts, so the barrier's wait on
//     the vector-memory counter covers them.  This layout gives each wave 64
//     accumulators (the INT8 kernel's 128 x 64 sub-tiles would need twice
//     the conversion work per slice).
//   * Per slice: 16 MFMA units (one fragment pair each), the first 8 with
//     DMA parts of slice kt + 2 in between, then the barrier, then 8, each
//     followed by the read of one of slice kt + 1's fragments into registers
//     already done with, and the remaining DMA parts.
//   * The LDS ring is split (the three A blocks, then the three weight
//     blocks) and the loop is unrolled over the stages so that every
//     fragment read is a base register plus a constant:
//     vector-ALU instructions do not overlap the MFMAs on this chip but add
//     to the SIMD's time, and the conversions are the only ones left.
//   * Bytes past K in the final slice are zeroed in LDS for A; the weight
//     rows or chunks read past K meet those zeros.  A NaN code in an FP8
//     weight there would still poison the sum, as it would inside K.
#include "gemm_tile.h"

namespace qk {
namespace {

using namespace tile;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int WTM = 64;       // wave tile rows
constexpr int WTN = 64;       // wave tile columns
constexpr int FM = WTM / 16;  // 16x16 fragments per wave along M
constexpr int FN = WTN / 16;  // ... along N
static_assert((BM / WTM) * (BN / WTN) == kWaves, "every wave owns one sub-tile");

enum Kind { kFp8 = 0, kI8Group64 = 1, kI8Group128 = 2 };

// groups of weight scales per 128-byte slice
template <int KIND>
constexpr int groups_per_slice() { return KIND == kI8Group64 ? 2 : (KIND == kI8Group128 ? 1 : 0); }

__device__ __forceinline__ v4i lo_half(const v8i& x) { return v4i{x[0], x[1], x[2], x[3]}; }
__device__ __forceinline__ v4i hi_half(const v8i& x) { return v4i{x[4], x[5], x[6], x[7]}; }

// acc += float(p) * s, elementwise (p exact in binary32).  The empty
// volatile asm takes acc as an operand, which keeps the arithmetic at this
// point of the instruction sequence: scheduling barriers bind only the
// machine scheduler, and without it the optimizer sinks these operations
// past the following MFMAs, which then all hold their results at once.
__device__ __forceinline__ void add_scaled(v4f& acc, const v4i& p, float s) {
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(static_cast<float>(p[r]), s, acc[r]);
  asm volatile("" : "+v"(acc));
}

template <int KIND, int MODE, bool KTAIL>
__global__ __launch_bounds__(kThreads, 1) void gemm_slice_kernel(
    const int8_t* __restrict__ a, const int8_t* __restrict__ b, float* __restrict__ c,
    const float* __restrict__ scale_a, const float* __restrict__ scale_b, float output_scale,
    void* __restrict__ out, int out_dtype, int M, int N, int K, int tiles_m, int tiles_n) {
  constexpr bool kRegB = MODE == kBknReg4 || MODE == kBknReg1;
  constexpr int GPS = groups_per_slice<KIND>();
  constexpr bool kGrouped = GPS > 0;
  __shared__ __attribute__((aligned(1024))) char smem[kStages * STAGE];

  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM;
  const int n0 = tn * BN;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave / (BN / WTN);
  const int wn = wave % (BN / WTN);

  // epilogue scales: per token, then per channel (FP8) or 1 (group scales
  // are applied in the main loop) times output_scale; written to LDS before
  // the k loop so that no register holds them across it (read after its
  // barriers)
  static_assert(BM + BN <= kThreads, "one scale per thread");
  __shared__ float s_scale[BM + BN];
  if (out && t < BM + BN) {
    float v = 1.0f;
    if (t < BM) {
      v = m0 + t < M ? scale_a[m0 + t] : 0.0f;
    } else if (!kGrouped) {
      v = n0 + t - BM < N ? scale_b[n0 + t - BM] : 0.0f;
    }
    s_scale[t] = t < BM ? v : v * output_scale;
  }

  // the split LDS ring (gemm_tile.h): the three A blocks, then the three
  // weight blocks, so that one base register reaches a weight fragment in
  // every stage within a DS instruction's immediate offset
  auto a_lds = [&](int s) { return smem + (s % kStages) * A_STAGE; };
  auto b_lds = [&](int s) { return smem + kStages * A_STAGE + (s % kStages) * B_STAGE; };

  using RegTile = std::conditional_t<MODE == kBknReg4, KnRegTile<true>,
                                     std::conditional_t<MODE == kBknReg1, KnRegTile<false>, NoRegTile>>;
  RegTile breg;

  auto fetch = [&](int s) {
    dma_rowk<BM>(a, a_lds(s), M, K, m0, s * BK);
    if constexpr (MODE == kBnkDma) dma_rowk<BN>(b, b_lds(s), N, K, n0, s * BK);
    if constexpr (MODE == kBknDma) dma_kn(b, b_lds(s), N, K, n0, s * BK);
  };
  constexpr int kFetchOps = BM * BK / 1024 / kWaves + (kRegB ? 0 : BN * BK / 1024 / kWaves);
  constexpr int kOpsA = rowk_ops<BM>();
  constexpr bool kFixedParts = !KTAIL && !kRegB;
  const uint32_t lds_smem = lds_addr(smem);
  using Parts = std::conditional_t<kFixedParts, FixedParts<MODE == kBnkDma ? kBnkDma : kBknDma, true>,
                                   NoParts>;
  Parts parts;
  if constexpr (kFixedParts) {
    static_assert(Parts::kOps == kFetchOps, "one DMA instruction per part");
    parts.init(a, b, M, N, K, m0, n0);
  }
  auto fetch_part = [&](int s, int part) {
    if constexpr (kFixedParts) {
      parts.issue(lds_smem, s, part);
    } else if (part < kOpsA) {
      dma_rowk_one<BM>(a, a_lds(s), M, K, m0, s * BK, part);
    } else if constexpr (MODE == kBnkDma) {
      dma_rowk_one<BN>(b, b_lds(s), N, K, n0, s * BK, part - kOpsA);
    } else if constexpr (MODE == kBknDma) {
      dma_kn_one(b, b_lds(s), N, K, n0, s * BK, part - kOpsA);
    }
  };

  // the lane's two 16-byte k chunks of a slice and its fragment row / column
  const int c0 = lane >> 4;
  const int c1 = 4 + (lane >> 4);
  const int i16 = lane & 15;
  const int a_row = wm * WTM + i16;
  const int b_row = wn * WTN + i16;
  // Fragment reads of stage S.  kConstStage: the DMA-mode loop below is
  // unrolled over the stages and every read is a base register plus a
  // constant, so the loop issues no address arithmetic (vector-ALU
  // instructions do not overlap the MFMAs on this chip but add to the
  // SIMD's time).  The empty asm makes each base opaque, so that the
  // compiler keeps it in its own register instead of deriving one from
  // another with offsets past the 16-bit immediate's reach.  The
  // register-staged weight's loop is not unrolled: there the stage is a
  // run-time value and each read's address is formed from it.
  constexpr bool kConstStage = !kRegB;
  auto opaque = [](uint32_t x) {
    asm("" : "+v"(x));
    return x;
  };
  const uint32_t lds0 = lds_addr(smem);
  const uint32_t b_ring = lds0 + kStages * A_STAGE;
  // A: chunks c0 and c1 of fragment 0; fragment i at + 2048 i.  Set 0
  // serves stages 0 and 1 (stage 1 at + A_STAGE), set 1 stage 2, which lies
  // past the immediate's reach from set 0.
  uint32_t a_base[2][2] = {{0, 0}, {0, 0}};
  // [k][n] weight: a transpose read covers k rows kr .. kr + 7 (kr = 16 ch +
  // 8 h + (i16 >> 1) for lane i16 of a 16-lane group) of fragment column
  // block j, and lane i16 receives column i16's eight bytes.  The row
  // swizzle kn_swz(kr) = (i16 >> 1) ^ (ch & 1) is the same for the lane's
  // chunks c0 and c1 = c0 + 4 and both halves h, so the four reads of a
  // fragment share one base and differ by 64 rows (c1) and 8 rows (h); the
  // bases serve all three stages.
  uint32_t b_base[FN];
  // [N][K] or register-staged weight: like A, fragment j at + 2048 j
  uint32_t bk_base[2] = {0, 0};
#pragma unroll
  for (int j = 0; j < FN; ++j)
    b_base[j] = b_ring + kn_offset(16 * c0 + (i16 >> 1), (wn * WTN + j * 16) >> 4) + 8 * (i16 & 1);
  if constexpr (kConstStage) {
#pragma unroll
    for (int set = 0; set < 2; ++set) {
      a_base[set][0] = opaque(lds0 + set * 2 * A_STAGE + rowk_offset(a_row, c0));
      a_base[set][1] = opaque(lds0 + set * 2 * A_STAGE + rowk_offset(a_row, c1));
    }
    if constexpr (MODE == kBknDma) {
#pragma unroll
      for (int j = 0; j < FN; ++j) b_base[j] = opaque(b_base[j]);
    } else {
      bk_base[0] = opaque(b_ring + rowk_offset(b_row, c0));
      bk_base[1] = opaque(b_ring + rowk_offset(b_row, c1));
    }
  }
  typedef __attribute__((address_space(3))) const v4i* lds_v4i;
  auto a_addr = [&](int S, int h, uint32_t off) -> uint32_t {
    return a_base[S / 2][h] + (S == 1 ? A_STAGE : 0) + off;
  };
  auto read_a = [&](int S, int i) -> v8i {
    v4i lo, hi;
    if constexpr (kConstStage) {
      lo = *reinterpret_cast<lds_v4i>(a_addr(S, 0, 2048 * i));
      hi = *reinterpret_cast<lds_v4i>(a_addr(S, 1, 2048 * i));
    } else {
      const char* As = a_lds(S);
      lo = *reinterpret_cast<const v4i*>(As + rowk_offset(a_row + i * 16, c0));
      hi = *reinterpret_cast<const v4i*>(As + rowk_offset(a_row + i * 16, c1));
    }
    return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  };
  auto read_b_tr = [&](int S, int j, int row_off) -> v2i {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) v2i*)(b_base[j] + S * B_STAGE + row_off * BN));
  };
  auto read_b_rowk = [&](int S, int j) -> v8i {
    v4i lo, hi;
    if constexpr (kConstStage) {
      const uint32_t off = S * B_STAGE + 2048 * j;
      lo = *reinterpret_cast<lds_v4i>(bk_base[0] + off);
      hi = *reinterpret_cast<lds_v4i>(bk_base[1] + off);
    } else {
      const char* Bs = b_lds(S);
      lo = *reinterpret_cast<const v4i*>(Bs + rowk_offset(b_row + j * 16, c0));
      hi = *reinterpret_cast<const v4i*>(Bs + rowk_offset(b_row + j * 16, c1));
    }
    return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  };
  auto read_b = [&](int S, int j) -> v8i {
    if constexpr (MODE == kBknDma) {
      const v2i p0 = read_b_tr(S, j, 0);
      const v2i p1 = read_b_tr(S, j, 8);
      const v2i p2 = read_b_tr(S, j, 64);
      const v2i p3 = read_b_tr(S, j, 72);
      return v8i{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
    } else {
      return read_b_rowk(S, j);
    }
  };

  // group scales of a slice: lane column of fragment block j, group h of the
  // slice (the column is clamped to N - 1 and the group to the last one:
  // such values multiply partials that are never stored, or are zero)
  const int groups = kGrouped ? K / (BK / GPS) : 1;
  int sc_col[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) sc_col[j] = min(n0 + wn * WTN + j * 16 + (lane & 15), N - 1);
  auto load_scales = [&](int s, float (&dst)[FN][GPS > 0 ? GPS : 1]) {
    if constexpr (kGrouped) {
#pragma unroll
      for (int h = 0; h < GPS; ++h) {
        const size_t g = static_cast<size_t>(min(s * GPS + h, groups - 1));
#pragma unroll
        for (int j = 0; j < FN; ++j) dst[j][h] = scale_b[g * N + sc_col[j]];
      }
    }
  };
  float sc[FN][GPS > 0 ? GPS : 1];   // scales of the slice being multiplied
  float scn[FN][GPS > 0 ? GPS : 1];  // ... of the next slice

  v4f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v4f{};

  const int KT = (K + BK - 1) / BK;

  auto zero_tail = [&](int s) {
    char* Az = a_lds(s);
#pragma unroll
    for (int i = 0; i < BM * 8 / kThreads; ++i) {
      const int row = (t >> 3) + (kThreads / 8) * i;
      if (s * BK + 16 * (t & 7) >= K)
        *reinterpret_cast<uint4*>(Az + rowk_offset(row, t & 7)) = make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
  };

  v8i fa[FM], fb[FN];  // fragments of the slice being multiplied
  if (KT > 0) {
    fetch(0);
    load_scales(0, sc);
    if constexpr (kRegB) breg.load(b, N, K, n0, 0);
    if (KT > 1) fetch(1);
    if constexpr (kRegB) {
      wait_vmcnt<0>();
      breg.store(b_lds(0));
    } else {
      if (KT > 1) wait_vmcnt<kFetchOps>(); else wait_vmcnt<0>();
    }
    __syncthreads();
    if (KTAIL && KT == 1) zero_tail(0);
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = read_a(0, i);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[j] = read_b(0, j);
  }

  // ---- one MFMA unit: one fragment pair ----
  // Units 0-7 take A fragments 0-1 against B 0-3 (A-fragment-major); unit
  // 8 + q takes A 2 + (q & 1) against B q / 2, so that B fragment j is free
  // for the next slice after unit 9 + 2 j.  INT8 kinds leave the unit's INT32
  // partials in part[] and add the previous unit's partials (prev[]) into the
  // accumulators.
  constexpr int kUnits = FM * FN;
  static_assert(FM == 4 && FN == 4, "unit order below");
  constexpr int kPartsPerUnit = GPS == 2 ? 2 : 1;
  // a unit's partials are scaled kLag units after its MFMAs, by when the
  // matrix core has written them (no wait states before the conversions)
  constexpr int kLag = 2;
  v4i pend[kLag][kPartsPerUnit];  // unit u's partials in pend[u % kLag]
  auto unit_pair = [](int u, int& i, int& j) {
    if (u < 8) {
      i = u / FN;
      j = u % FN;
    } else {
      i = 2 + ((u - 8) & 1);
      j = (u - 8) >> 1;
    }
  };
  auto unit_mfma = [&](int u) {
    int i, j;
    unit_pair(u, i, j);
    [[maybe_unused]] v4i(&part)[kPartsPerUnit] = pend[u % kLag];
    if constexpr (KIND == kFp8) {
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0, 0, 0, 0);
    } else if constexpr (KIND == kI8Group128) {
      const v4i zero = {0, 0, 0, 0};
      part[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(lo_half(fa[i]), lo_half(fb[j]), zero, 0, 0, 0);
      part[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(hi_half(fa[i]), hi_half(fb[j]), part[0], 0, 0, 0);
    } else {
      const v4i zero = {0, 0, 0, 0};
      part[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(lo_half(fa[i]), lo_half(fb[j]), zero, 0, 0, 0);
      part[1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(hi_half(fa[i]), hi_half(fb[j]), zero, 0, 0, 0);
    }
  };
  // add the partials of unit u (held in pend[u % kLag]) with the scales `s`
  auto unit_scale = [&](int u, const float (&s)[FN][GPS > 0 ? GPS : 1]) {
    if constexpr (kGrouped) {
      int i, j;
      unit_pair(u, i, j);
#pragma unroll
      for (int h = 0; h < kPartsPerUnit; ++h) add_scaled(acc[i][j], pend[u % kLag][h], s[j][h]);
    }
  };
  // the scaling of unit u - kLag, then the MFMAs of unit u into the
  // partials it freed; the slice's last kLag units are scaled after the
  // loop over units
  auto unit = [&](int u) {
    if constexpr (kGrouped) {
      if (u >= kLag) unit_scale(u - kLag, sc);
    }
    unit_mfma(u);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto slice_end = [&]() {
    if constexpr (kGrouped) {
#pragma unroll
      for (int d = kLag; d >= 1; --d) unit_scale(kUnits - d, sc);
    }
  };

  if constexpr (kRegB) {
    // register-staged weight (N not a multiple of 16): one slice per
    // iteration, the next slice's B staged through registers and written in
    // the [n][k] layout
    for (int kt = 0; kt < KT; ++kt) {
      if (kt + 1 < KT) load_scales(kt + 1, scn);
      if (kt + 2 < KT) fetch(kt + 2);
      if (kt + 1 < KT) breg.load(b, N, K, n0, (kt + 1) * BK);
#pragma unroll
      for (int u = 0; u < kUnits; ++u) unit(u);
      slice_end();
      if (kt + 1 < KT) {
        wait_vmcnt<0>();
        breg.store(b_lds(kt + 1));
        __syncthreads();
        if (KTAIL && kt + 1 == KT - 1) zero_tail(kt + 1);
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[i] = read_a((kt + 1) % kStages, i);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[j] = read_b_rowk((kt + 1) % kStages, j);
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int h = 0; h < (GPS > 0 ? GPS : 1); ++h) sc[j][h] = scn[j][h];
      }
    }
  } else {
    // DMA modes, one k slice per iteration in two phases:
    //   phase 0: the first kPhase0 units with DMA parts [0, kSplit) of slice
    //            kt + 2 in between (its LDS stage held slice kt - 1, whose
    //            fragments every wave read before the barrier of iteration
    //            kt - 1), after the loads of slice kt + 1's group scales;
    //   barrier: this wave's DMA of slice kt + 1 (and the scale loads before
    //            it) have landed (vmcnt), then all waves' (s_barrier);
    //   phase 1: the other units, each followed by a read of one of slice
    //            kt + 1's fragments: B j into the registers unit 9 + 2 j has
    //            just finished with, A 0-1 into registers free since phase 0,
    //            A 2-3 into a spare pair; and the remaining DMA parts.
    constexpr int kPhase0 = kUnits / 2;
    constexpr int kPhase1 = kUnits - kPhase0;
    constexpr int kSplit = kFetchOps / 2;
    static_assert(kFetchOps == 2 * kSplit, "DMA parts split evenly over the two phases");
    static_assert(kPhase0 >= kSplit && kPhase1 >= kFetchOps - kSplit, "one DMA part per unit");
    // slice kt, in stage S = kt % 3 (a constant in the unrolled loop)
    auto slice = [&](int S, int kt) __attribute__((always_inline)) {
      const int SN = (S + 1) % kStages;
      const bool prefetch = kt + 2 < KT;
      auto dma = [&](int part_idx) {
        if (prefetch) fetch_part(kt + 2, part_idx);
        __builtin_amdgcn_sched_barrier(0);
      };
      // ---- phase 0 ----
      if (kt + 1 < KT) load_scales(kt + 1, scn);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kPhase0; ++u) {
        unit(u);
        if (u < kSplit) dma(u);
      }
      // ---- barrier for slice kt + 1 ----
      if (kt + 1 < KT) {
        if (prefetch) wait_vmcnt<kSplit>(); else wait_vmcnt<0>();
        __syncthreads();
        if (KTAIL && kt + 1 == KT - 1) zero_tail(kt + 1);
      }
      // ---- phase 1 ----
      {
        // after the last slice these reads come from a valid, unused LDS
        // slice and are not used: no branches around LDS reads
        v8i na2, na3;
#pragma unroll
        for (int q = 0; q < kPhase1; ++q) {
          unit(kPhase0 + q);
          if (q & 1) {
            fb[q >> 1] = read_b(SN, q >> 1);
          } else if (q < 4) {
            fa[q >> 1] = read_a(SN, q >> 1);
          } else if (q == 4) {
            na2 = read_a(SN, 2);
          } else {
            na3 = read_a(SN, 3);
          }
          __builtin_amdgcn_sched_barrier(0);
          if (q < kFetchOps - kSplit) dma(kSplit + q);
        }
        slice_end();
        fa[2] = na2;
        fa[3] = na3;
        if (kt + 1 < KT) {
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int h = 0; h < (GPS > 0 ? GPS : 1); ++h) sc[j][h] = scn[j][h];
        }
      }
    };
    static_assert(kStages == 3, "three stages");
    if constexpr (KTAIL || !kConstStage) {
      for (int kt = 0; kt < KT; ++kt) slice(kt % kStages, kt);
    } else {
      int kt = 0;
      for (; kt + kStages <= KT; kt += kStages) {
        slice(0, kt);
        slice(1, kt + 1);
        slice(2, kt + 2);
      }
      if (kt < KT) slice(0, kt);
      if (kt + 1 < KT) slice(1, kt + 1);
    }
  }

  // ---- epilogue ----
  // Each wave holds the final sums of its 64 x 64 sub-tile; it
  // stages them row-major in LDS (the operand slices are free after the
  // barrier) and stores whole 128-byte row segments with nontemporal stores.
  constexpr int kStageBytes = WTM * WTN * 4;
  static_assert(WTN == kStageCols, "staging rows are one wave tile wide");
  static_assert(kWaves * kStageBytes <= kStages * STAGE, "staging fits in the ring");
  __syncthreads();  // every wave is done with the k slices
  const float* s_sa = s_scale;
  const float* s_sb = s_scale + BM;
  int* stage = reinterpret_cast<int*>(smem + wave * kStageBytes);
  // the lane index again from the exec mask, so that no register keeps it
  // over the k loop
  const int elane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const v4i bits = {__float_as_int(acc[i][j][0]), __float_as_int(acc[i][j][1]),
                          __float_as_int(acc[i][j][2]), __float_as_int(acc[i][j][3])};
        stage_fragment(stage, elane, i, j, bits);
      }
  }
  __syncthreads();  // each wave reads back only its own staging

  const int lrow0 = wm * WTM;
  const int lcol0 = wn * WTN;
  if (c) store4<WTM, true, true>(stage, elane, m0, n0, lrow0, lcol0, M, N, s_sa, s_sb, c);
  if (out) {
    if (out_dtype == QK_BF16)
      store_bf16<WTM, true>(stage, elane, m0, n0, lrow0, lcol0, M, N, s_sa, s_sb, out);
    else
      store4<WTM, true, false>(stage, elane, m0, n0, lrow0, lcol0, M, N, s_sa, s_sb, out);
  }
}

template <int KIND, int MODE>
hipError_t launch_mode(const SliceGemmArgs& g, dim3 grid, int tiles_m, int tiles_n,
                       hipStream_t stream) {
  // whole slices of a DMA'd weight take the fixed transfer parts, whose lane
  // offsets are 32-bit; the k-tail kernel forms its addresses per slice
  constexpr bool kDma = MODE == kBnkDma || MODE == kBknDma;
  if (g.k % BK != 0 || (kDma && !xfer_parts_fit(g.n, g.k)))
    return launch(gemm_slice_kernel<KIND, MODE, true>, grid, dim3(kThreads), 0, stream, g.a, g.b,
                  g.c, g.scale_a, g.scale_b, g.output_scale, g.out, g.out_dtype, g.m, g.n, g.k,
                  tiles_m, tiles_n);
  return launch(gemm_slice_kernel<KIND, MODE, false>, grid, dim3(kThreads), 0, stream, g.a, g.b,
                g.c, g.scale_a, g.scale_b, g.output_scale, g.out, g.out_dtype, g.m, g.n, g.k,
                tiles_m, tiles_n);
}

template <int KIND>
hipError_t launch_kind(const SliceGemmArgs& g, hipStream_t stream) {
  const int tiles_m = (g.m + BM - 1) / BM;
  const int tiles_n = (g.n + BN - 1) / BN;
  const long long tiles = static_cast<long long>(tiles_m) * tiles_n;
  if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(tiles));
  if (g.b_layout == QK_B_NK) return launch_mode<KIND, kBnkDma>(g, grid, tiles_m, tiles_n, stream);
  if (g.n % 16 == 0) return launch_mode<KIND, kBknDma>(g, grid, tiles_m, tiles_n, stream);
  if (g.n % 4 == 0) return launch_mode<KIND, kBknReg4>(g, grid, tiles_m, tiles_n, stream);
  return launch_mode<KIND, kBknReg1>(g, grid, tiles_m, tiles_n, stream);
}

}  // namespace

hipError_t launch_gemm_fp8(const SliceGemmArgs& g, hipStream_t stream) {
  return launch_kind<kFp8>(g, stream);
}

hipError_t launch_gemm_i8_grouped(const SliceGemmArgs& g, int group, hipStream_t stream) {
  if (group == 64) return launch_kind<kI8Group64>(g, stream);
  if (group == 128) return launch_kind<kI8Group128>(g, stream);
  return hipErrorInvalidValue;
}

}  // namespace qk
