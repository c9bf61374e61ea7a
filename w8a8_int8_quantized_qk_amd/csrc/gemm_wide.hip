// INT8 x INT8 -> INT32 GEMM with 256 x 256 workgroup tiles, for outputs with
// many tiles (the large MLP projections), on CDNA4 matrix cores with the
// dequant epilogue fused.
//
// What it computes is the tiled INT8 kernel's ("16. Deploying Custom
// Kernels", C++ Kernel Interface; "KV-cache kernels", 02 Scales and
// dequantization; INT32 accumulation from "Skill: Write an INT8 Quantized
// Kernel", Inputs):
//   acc[i][j] = sum_t a[i][t] * B(t, j)        exact INT32
//   c[i][j]   = acc                            (optional)
//   out[i][j] = ((float)acc * scale_a[i]) * (scale_b[j] * output_scale)   (optional)
// Re-tiling for the shape class is what "KV-cache kernels", 04 What changes
// in the kernel's shape, asks for: a larger tile halves the global-to-LDS
// bytes per multiply-accumulate of the 256 x 128 tile's k-split design.
//
// Design for gfx950:
//   * Workgroup tile 256 (M) x 256 (N), k slices of 64 bytes, four LDS
//     stages of 32 KiB (A 256 x 64, B 64 x 256), eight wave64s (two per SIMD),
//     each owning a 128 x 64 sub-tile (2 x 4 of them) over the whole k range
//     with v_mfma_i32_16x16x64_i8: per slice and wave 8 x 4 instructions, 8
//     A and 4 B fragment reads, exactly the per-wave work of the 256 x 128
//     kernel's half slice, with 32 KiB of global-to-LDS transfer per slice
//     instead of 48 and no k-group hand-over at the end.
//   * Transfers go global -> LDS with 128-bit global_load_lds (four per wave
//     and slice), issued for slice kt + 3 while slice kt is multiplied: the
//     wait before slice kt + 1's fragments covers loads issued two slices
//     earlier.  One execution barrier per slice, without a memory fence, and
//     every fragment read several MFMAs ahead of its first use, so neither
//     the barrier nor an MFMA waits on LDS latency.
//   * Measured: the loop's time per slice is the same at 1.8 and 2.4 GHz, so
//     memory, not the matrix cores, paces it: with four stages, each slice's
//     lines that miss L2 have about two slices' time to arrive.
//   * A (and a weight stored [N][K]) is kept k-contiguous, 64-byte rows with
//     the 16-byte chunk index XORed by (row >> 2) & 3: the 16 consecutive
//     rows a 128-bit fragment read serves together hit 16 distinct 16-byte
//     bank groups.  A weight stored [K][N] stays [k][n] (256-byte rows, chunk
//     XORed by (k & 7) | ((k >> 4) & 1) << 3) and is read with
//     ds_read_b64_tr_b8, which hands each lane its column's k bytes; the 16
//     rows two lane groups read together land in 16 distinct bank groups.
//   * Rows past M or N re-read a valid row (never stored); a k tail (K not a
//     multiple of 64) has its A chunks at k >= K zeroed in LDS before use.
//   * XCD-aware tile order as in the 256 x 128 kernel.
//   * MoE: an expert's last row block of at most 128 rows is a light tile:
//     every wave multiplies a 64 x 64 block of the first 128 rows (half the
//     MFMAs) and only those A rows are transferred (three 1-KiB parts per
//     wave and slice instead of four).  The loop is paced by its transfers,
//     so the light tile costs about three quarters of a full one.
//   * Epilogue: each wave stages its 128 x 64 block in two 64-row halves
//     row-major in LDS and stores whole 128-byte row segments with the
//     shared store helpers (scales in binary32, bf16 rounded to nearest even).
#include "gemm_tile.h"

namespace qk {
namespace {

namespace wide {

using tile::v2i;
using tile::v4i;

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int kStages = 4;
constexpr int A_STAGE = BM * BK;          // 16 KiB
constexpr int B_STAGE = BN * BK;          // 16 KiB
constexpr int STAGE = A_STAGE + B_STAGE;  // 32 KiB
constexpr int WTM = 128;                  // wave sub-tile rows
constexpr int WTN = 64;                   // wave sub-tile columns
constexpr int FM = WTM / 16;
constexpr int FN = WTN / 16;
static_assert((BM / WTM) * (BN / WTN) == kWaves, "one sub-tile per wave");
constexpr int kOpsA = BM * BK / 1024 / kWaves;  // 1 KiB transfers per wave and slice
constexpr int kOpsB = BN * BK / 1024 / kWaves;
constexpr int kOps = kOpsA + kOpsB;
static_assert(kOpsA == 2 && kOpsB == 2, "two A and two B transfers per wave and slice");

// k-contiguous rows of 64 bytes (A, [N][K] weight)
__device__ __forceinline__ int rowk_offset(int row, int chunk) {
  return row * BK + ((chunk ^ ((row >> 2) & 3)) << 4);
}
// [k][n] weight rows of 256 bytes
__device__ __forceinline__ int kn_swz(int k) { return (k & 7) | (((k >> 4) & 1) << 3); }
__device__ __forceinline__ int kn_offset(int k, int chunk) {
  return k * BN + ((chunk ^ kn_swz(k)) << 4);
}

// Source address and LDS slot (wave-uniform, for m0; relative to the stage's
// block of its operand) of this thread's transfer `part` of a slice.
// A part: 16 rows x 64 bytes (lane l: row l / 4, LDS chunk l % 4).  [K][N]
// weight part: 4 k rows x 256 bytes (lane l: k row l / 16, LDS chunk l % 16).
// Global rows, columns and k are clamped into the operands (the values
// there are never used, or meet zero codes).
template <int MODE>
__device__ __forceinline__ void part_source(const int8_t* __restrict__ a,
                                            const int8_t* __restrict__ b, int M, int N, int K,
                                            int m0, int n0, int k0, int lda, int ldb, int part,
                                            const int8_t*& src, uint32_t& lds, int a_blk = -1) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  if (part < kOpsA || MODE == tile::kBnkDma) {
    const bool is_a = part < kOpsA;
    const int blk = is_a && a_blk >= 0 ? a_blk : wave * kOpsA + (is_a ? part : part - kOpsA);
    const int row = blk * 16 + (lane >> 2);
    const int gchunk = (lane & 3) ^ ((row >> 2) & 3);
    const uint32_t gr = static_cast<uint32_t>(min((is_a ? m0 : n0) + row, (is_a ? M : N) - 1));
    const uint32_t gk = static_cast<uint32_t>(min(k0 + 16 * gchunk, K - 16));
    src = (is_a ? a : b) + (gr * static_cast<uint32_t>(is_a ? lda : ldb) + gk);
    lds = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(blk * 1024));
  } else {
    const int blk = wave * kOpsB + (part - kOpsA);
    const int k = blk * 4 + (lane >> 4);
    const int gchunk = (lane & 15) ^ kn_swz(k);
    const uint32_t gk = static_cast<uint32_t>(min(k0 + k, K - 1));
    const uint32_t gn = static_cast<uint32_t>(min(n0 + 16 * gchunk, N - 16));
    src = b + (gk * static_cast<uint32_t>(N) + gn);
    lds = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(blk * 1024));
  }
}

// One workgroup's 256 x 256 output tile (tm, tn).  light: the tile has at
// most 128 rows below M (an expert's last row block in the MoE launch); its
// eight waves then each multiply a 64 x 64 block of the first 128 rows, half
// the MFMAs of a full tile.
template <int MODE, bool KTAIL>
__device__ __forceinline__ void gemm_wide_tile(
    const int8_t* __restrict__ a, const int8_t* __restrict__ b, int32_t* __restrict__ c,
    const float* __restrict__ scale_a, const float* __restrict__ scale_b, float output_scale,
    void* __restrict__ out, int out_dtype, int M, int N, int K, int tm, int tn,
    bool light = false) {
  static_assert(MODE == tile::kBnkDma || MODE == tile::kBknDma, "DMA weight layouts");
  constexpr int kStageRows = 64;                         // rows per epilogue pass
  constexpr int kStageBytes = kStageRows * WTN * 4;      // 16 KiB per wave
  constexpr int kSmem = kStages * STAGE > kWaves * kStageBytes + 8 * (BM + BN)
                            ? kStages * STAGE
                            : kWaves * kStageBytes + 8 * (BM + BN);
  __shared__ __attribute__((aligned(1024))) char smem[kSmem];

  const int m0 = tm * BM;
  const int n0 = tn * BN;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave >> 2;  // 2 sub-tiles along M
  const int wn = wave & 3;   // 4 along N

  // this thread's per-token or per-channel scale, loaded now so that its
  // latency hides behind the main loop
  static_assert(BM + BN == kThreads, "one scale per thread");
  float scale_reg = 0.0f;
  if (out) {
    if (t < BM) {
      if (m0 + t < M) scale_reg = scale_a[m0 + t];
    } else if (n0 + t - BM < N) {
      scale_reg = scale_b[n0 + t - BM];  // times output_scale later
    }
  }

  // The LDS ring is split: the A blocks of the four stages first (stage s at
  // s * A_STAGE), then the weight blocks (at kStages * A_STAGE + s * B_STAGE),
  // so that one base register reaches an operand's block in every stage
  // within a DS instruction's 16-bit immediate offset.
  auto stage_a = [](int s) { return static_cast<uint32_t>((s % kStages) * A_STAGE); };
  auto stage_b = [](int s) {
    return static_cast<uint32_t>(kStages * A_STAGE + (s % kStages) * B_STAGE);
  };
  static_assert((kStages - 1) * A_STAGE + 1024 * (FM - 1) < 65536 &&
                    (kStages - 1) * B_STAGE + 2048 < 65536 &&
                    (kStages - 1) * B_STAGE + 1024 * (FN - 1) < 65536,
                "every stage within the immediate offsets of one base");

  // transfer sources and LDS slots, formed once.  Whole slices (no k tail):
  // each part is a wave-uniform base (the tile's A rows or weight block at
  // slice 0, advanced per slice in scalar registers) plus a fixed 32-bit
  // lane offset (gemm_wide_applies bounds it).  A k tail changes the clamps
  // in its final slice, so there every slice forms its addresses again.
  const uint32_t lds_smem = lds_addr(smem);
  const int8_t* const base_a = a + static_cast<size_t>(m0) * K;
  const int8_t* const base_b = MODE == tile::kBknDma ? b + n0 : b + static_cast<size_t>(n0) * K;
  const size_t stride_b = MODE == tile::kBknDma ? static_cast<size_t>(BK) * N : BK;
  uint32_t voff[kOps];
  uint32_t slot[kOps];
#pragma unroll
  for (int q = 0; q < kOps; ++q) {
    const int8_t* src;
    part_source<MODE>(a, b, M, N, K, m0, n0, 0, K, K, q, src, slot[q]);
    voff[q] = static_cast<uint32_t>(src - (q < kOpsA ? base_a : base_b));
  }
  auto issue = [&](int s, int q) {
    const uint32_t lds = lds_smem + (q < kOpsA ? stage_a(s) : stage_b(s));
    if constexpr (KTAIL) {
      const int8_t* p;
      uint32_t l;
      part_source<MODE>(a, b, M, N, K, m0, n0, s * BK, K, K, q, p, l);
      lds_dma16(p, lds + l);
    } else {
      const int8_t* sbase = q < kOpsA ? base_a + static_cast<size_t>(s) * BK
                                      : base_b + static_cast<size_t>(s) * stride_b;
      lds_dma16_split(sbase, voff[q], lds + slot[q]);
    }
  };
  // A light tile needs only A rows 0 .. 127: its transfers per slice are one
  // A part per wave (rows 16 w .. 16 w + 15) and the wave's two weight parts
  constexpr int kOpsLight = 1 + kOpsB;
  uint32_t voff_la = 0, slot_la = 0;
  {
    const int8_t* src;
    part_source<MODE>(a, b, M, N, K, m0, n0, 0, K, K, 0, src, slot_la, wave);
    voff_la = static_cast<uint32_t>(src - base_a);
  }
  auto issue_light = [&](int s, int p) {
    if (p > 0) {
      issue(s, kOpsA + p - 1);
      return;
    }
    const uint32_t lds = lds_smem + stage_a(s);
    if constexpr (KTAIL) {
      const int8_t* src;
      uint32_t l;
      part_source<MODE>(a, b, M, N, K, m0, n0, s * BK, K, K, 0, src, l, wave);
      lds_dma16(src, lds + l);
    } else {
      lds_dma16_split(base_a + static_cast<size_t>(s) * BK, voff_la, lds + slot_la);
    }
  };

  // Fragments of v_mfma_i32_16x16x64_i8: lane l holds 16 k-consecutive bytes,
  // k = 16 (l / 16) .. + 15 of the slice, of row l % 16 (A) or column l % 16
  // (B) of the fragment.  Every read is a base register plus a constant (the
  // stage is a template constant below): A fragment i at + 1024 i; the [K][N]
  // weight's column block j from its own base (kn_swz of k rows 16 (l / 16) +
  // (l % 16) / 2 + 8 h does not depend on h, so half h is at + 8 rows); the
  // [N][K] weight's fragment j at + 1024 j.  The empty asm makes each base
  // opaque, so that the compiler keeps it in its own register instead of
  // deriving one from another with offsets past the immediate's reach.
  auto opaque = [](uint32_t x) {
    asm("" : "+v"(x));
    return x;
  };
  const int kchunk = lane >> 4;
  const int i16 = lane & 15;
  const uint32_t a_base = opaque(lds_smem + rowk_offset(wm * WTM + i16, kchunk));
  uint32_t b_base[FN];
  uint32_t bk_base = 0;
  if constexpr (MODE == tile::kBknDma) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
      b_base[j] = opaque(lds_smem + kStages * A_STAGE +
                         kn_offset(16 * kchunk + (i16 >> 1), wn * (WTN / 16) + j) + 8 * (i16 & 1));
  } else {
    bk_base = opaque(lds_smem + kStages * A_STAGE + rowk_offset(wn * WTN + i16, kchunk));
  }
  typedef __attribute__((address_space(3))) const v4i* lds_v4i;
  // stage S of the ring (a constant wherever the loop below is unrolled)
  auto read_a = [&](int S, int i) -> v4i {
    return *reinterpret_cast<lds_v4i>(a_base + S * A_STAGE + 1024 * i);
  };
  auto read_b_tr = [&](int S, int j, int h) -> v2i {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) v2i*)(b_base[j] + S * B_STAGE + BN * 8 * h));
  };
  auto read_b_rowk = [&](int S, int j) -> v4i {
    return *reinterpret_cast<lds_v4i>(bk_base + S * B_STAGE + 1024 * j);
  };
  auto read_b = [&](int S, int j) -> v4i {
    if constexpr (MODE == tile::kBknDma) {
      const v2i lo = read_b_tr(S, j, 0);
      const v2i hi = read_b_tr(S, j, 1);
      return v4i{lo.x, lo.y, hi.x, hi.y};
    } else {
      return read_b_rowk(S, j);
    }
  };

  v4i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v4i{};

  const int KT = (K + BK - 1) / BK;

  // zero the A chunks of the final slice that lie at k >= K, then publish
  auto zero_tail = [&](int s) {
    char* Az = smem + stage_a(s);
    // 256 rows x 4 chunks = 1024 chunks, two per thread
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = t + kThreads * i;
      const int row = idx >> 2;
      const int ch = idx & 3;
      if (s * BK + 16 * ch >= K)
        *reinterpret_cast<uint4*>(Az + rowk_offset(row, ch)) = make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
  };

  v4i fa[FM], fb[FN];
  if (KT > 0) {
    if (light) {
#pragma unroll
      for (int s = 0; s < 3; ++s)
        if (s < KT)
#pragma unroll
          for (int p = 0; p < kOpsLight; ++p) issue_light(s, p);
      if (KT > 2) wait_vmcnt<2 * kOpsLight>(); else if (KT > 1) wait_vmcnt<kOpsLight>(); else wait_vmcnt<0>();
    } else {
#pragma unroll
      for (int s = 0; s < 3; ++s)
        if (s < KT)
#pragma unroll
          for (int q = 0; q < kOps; ++q) issue(s, q);
      // slice 0 landed: at most the later prologue slices are outstanding
      if (KT > 2) wait_vmcnt<2 * kOps>(); else if (KT > 1) wait_vmcnt<kOps>(); else wait_vmcnt<0>();
    }
    __syncthreads();
    if (KTAIL && KT == 1) zero_tail(0);
    if (!light) {
#pragma unroll
      for (int i = 0; i < FM / 2; ++i) fa[i] = read_a(0, i);
#pragma unroll
      for (int j = 0; j < FN / 2; ++j) fb[j] = read_b(0, j);
    }
  }

  // An execution barrier without a memory fence: the waits it needs are
  // explicit (vmcnt for this wave's transfers), and LDS reads issued before it
  // stay in flight until the MFMA that uses them waits for them.
  auto barrier = [] {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // One slice (in stage S = kt % 4) in two phases, every instruction's place
  // pinned by sched_barrier, each fragment read several MFMAs before its
  // first use:
  //   phase 0: MFMAs of A 0..3 x B 0..1 (fragments read in the previous
  //            slice), interleaved with the reads of this slice's A 4..7,
  //            then B 2..3;
  //   barrier: slice kt + 1 has landed (this wave's transfers by vmcnt, every
  //            wave's by s_barrier).  Every wave has also consumed slice
  //            kt - 1 by now, so the transfers of slice kt + 3 into its stage
  //            follow the barrier;
  //   phase 1: A 4..7 x B 0 and B 1 (then B 0 and B 1 are free and slice
  //            kt + 1's B 0..1 are read into them), A 0..3 x B 2..3 (each A
  //            register is read for slice kt + 1 once its last MFMA issued),
  //            A 4..7 x B 2..3, with the four transfers of slice kt + 3
  //            spread between.
  static_assert(FM == 8 && FN == 4, "interleave pattern below");
  auto slice = [&](int S, int kt) __attribute__((always_inline)) {
    const int SN = (S + 1) % kStages;
    const bool prefetch = kt + 3 < KT;
    auto mfma = [&](int i, int j) {
      acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    };
    auto dma = [&](int q) {
      if (prefetch) issue(kt + 3, q);
      __builtin_amdgcn_sched_barrier(0);
    };
    // ---- phase 0 ----
    {
      mfma(0, 0);
      fa[4] = read_a(S, 4);
      mfma(0, 1);
      fa[5] = read_a(S, 5);
      mfma(1, 0);
      fa[6] = read_a(S, 6);
      mfma(1, 1);
      fa[7] = read_a(S, 7);
      if constexpr (MODE == tile::kBknDma) {
        v2i lo[2], hi[2];
        mfma(2, 0);
        lo[0] = read_b_tr(S, 2, 0);
        mfma(2, 1);
        hi[0] = read_b_tr(S, 2, 1);
        mfma(3, 0);
        lo[1] = read_b_tr(S, 3, 0);
        mfma(3, 1);
        hi[1] = read_b_tr(S, 3, 1);
        fb[2] = v4i{lo[0].x, lo[0].y, hi[0].x, hi[0].y};
        fb[3] = v4i{lo[1].x, lo[1].y, hi[1].x, hi[1].y};
      } else {
        mfma(2, 0);
        fb[2] = read_b_rowk(S, 2);
        mfma(2, 1);
        mfma(3, 0);
        fb[3] = read_b_rowk(S, 3);
        mfma(3, 1);
      }
    }
    // ---- barrier for slice kt + 1 ----
    if (kt + 1 < KT) {
      // outstanding after slice kt + 1: slice kt + 2's transfers, if issued
      if (kt + 2 < KT) wait_vmcnt<kOps>(); else wait_vmcnt<0>();
      barrier();
      if (KTAIL && kt + 1 == KT - 1) zero_tail(kt + 1);
    }
    // ---- phase 1 ----
    {
      // after the last slice these reads come from a valid, unused stage and
      // are not used: no branches around LDS reads
      v4i na[4], nb[2];
      mfma(4, 0);
      mfma(5, 0);
      dma(0);
      mfma(6, 0);
      mfma(7, 0);
      if constexpr (MODE == tile::kBknDma) {
        v2i lo[2], hi[2];
        lo[0] = read_b_tr(SN, 0, 0);
        mfma(4, 1);
        hi[0] = read_b_tr(SN, 0, 1);
        mfma(5, 1);
        dma(1);
        mfma(6, 1);
        mfma(7, 1);
        lo[1] = read_b_tr(SN, 1, 0);
        mfma(0, 2);
        hi[1] = read_b_tr(SN, 1, 1);
        nb[0] = v4i{lo[0].x, lo[0].y, hi[0].x, hi[0].y};
        nb[1] = v4i{lo[1].x, lo[1].y, hi[1].x, hi[1].y};
      } else {
        nb[0] = read_b_rowk(SN, 0);
        mfma(4, 1);
        mfma(5, 1);
        dma(1);
        mfma(6, 1);
        mfma(7, 1);
        nb[1] = read_b_rowk(SN, 1);
        mfma(0, 2);
      }
      mfma(0, 3);
      na[0] = read_a(SN, 0);
      mfma(1, 2);
      dma(2);
      mfma(1, 3);
      na[1] = read_a(SN, 1);
      mfma(2, 2);
      mfma(2, 3);
      na[2] = read_a(SN, 2);
      mfma(3, 2);
      dma(3);
      mfma(3, 3);
      na[3] = read_a(SN, 3);
      mfma(4, 2);
      mfma(4, 3);
      mfma(5, 2);
      mfma(5, 3);
      mfma(6, 2);
      mfma(6, 3);
      mfma(7, 2);
      mfma(7, 3);
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = na[i];
      fb[0] = nb[0];
      fb[1] = nb[1];
    }
  };
  // A light tile: wave w multiplies rows 64 (w / 4) .. + 63 of the tile by
  // its 64 columns, 16 MFMAs per slice from 4 A and 4 B fragments.  At the
  // top of slice kt the wave holds kt's fragments (xa, xb); after the barrier
  // for slice kt + 1 (every wave has also consumed slice kt - 1, whose stage
  // slice kt + 3 then takes) it reads kt + 1's into (ya, yb) between the
  // MFMAs, with the three transfers of slice kt + 3.
  const uint32_t la_base = opaque(lds_smem + rowk_offset(wm * 64 + i16, kchunk));
  auto lread_a = [&](int S, int i) -> v4i {
    return *reinterpret_cast<lds_v4i>(la_base + S * A_STAGE + 1024 * i);
  };
  v4i xa[4], xb[FN], ya[4], yb[FN];
  auto lslice = [&](int S, int kt) __attribute__((always_inline)) {
    const int SN = (S + 1) % kStages;
    const bool prefetch = kt + 3 < KT;
    if (kt + 1 < KT) {
      if (kt + 2 < KT) wait_vmcnt<kOpsLight>(); else wait_vmcnt<0>();
      barrier();
      if (KTAIL && kt + 1 == KT - 1) zero_tail(kt + 1);
    }
    v2i lo[FN], hi[FN];
#pragma unroll
    for (int n = 0; n < 4 * FN; ++n) {
      const int i = n / FN;
      const int j = n % FN;
      acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa[i], xb[j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      // after the last slice these reads come from a valid, unused stage
      if (n < 4) {
        ya[n] = lread_a(SN, n);
      } else if (n < 4 + 2 * FN) {
        const int r = n - 4;
        if constexpr (MODE == tile::kBknDma) {
          if (r & 1) hi[r >> 1] = read_b_tr(SN, r >> 1, 1);
          else lo[r >> 1] = read_b_tr(SN, r >> 1, 0);
        } else if ((r & 1) == 0) {
          yb[r >> 1] = read_b_rowk(SN, r >> 1);
        }
      }
      if ((n & 3) == 3 && (n >> 2) < kOpsLight) {
        if (prefetch) issue_light(kt + 3, n >> 2);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (MODE == tile::kBknDma) {
#pragma unroll
      for (int j = 0; j < FN; ++j) yb[j] = v4i{lo[j].x, lo[j].y, hi[j].x, hi[j].y};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) xa[i] = ya[i];
#pragma unroll
    for (int j = 0; j < FN; ++j) xb[j] = yb[j];
  };

  static_assert(kStages == 4, "four stages");
  if (light) {
    if (KT > 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) xa[i] = lread_a(0, i);
#pragma unroll
      for (int j = 0; j < FN; ++j) xb[j] = read_b(0, j);
    }
    if constexpr (KTAIL) {
      for (int kt = 0; kt < KT; ++kt) lslice(kt % kStages, kt);
    } else {
      int kt = 0;
      for (; kt + kStages <= KT; kt += kStages) {
        lslice(0, kt);
        lslice(1, kt + 1);
        lslice(2, kt + 2);
        lslice(3, kt + 3);
      }
      if (kt < KT) lslice(0, kt);
      if (kt + 1 < KT) lslice(1, kt + 1);
      if (kt + 2 < KT) lslice(2, kt + 2);
    }
  } else if constexpr (KTAIL) {
    for (int kt = 0; kt < KT; ++kt) slice(kt % kStages, kt);
  } else {
    // unrolled over the four stages, so that each slice's stage is a constant
    int kt = 0;
    for (; kt + kStages <= KT; kt += kStages) {
      slice(0, kt);
      slice(1, kt + 1);
      slice(2, kt + 2);
      slice(3, kt + 3);
    }
    if (kt < KT) slice(0, kt);
    if (kt + 1 < KT) slice(1, kt + 1);
    if (kt + 2 < KT) slice(2, kt + 2);
  }

  // ---- epilogue ----
  // Each wave stages its 128 x 64 block in two 64-row halves, row-major in
  // LDS (the stages are free once every wave is past the loop), and stores
  // whole 128-byte row segments.  Output stores are nontemporal.
  __syncthreads();
  float* s_sa = reinterpret_cast<float*>(smem + kWaves * kStageBytes);
  float* s_sb = s_sa + BM;
  if (out) s_sa[t] = t < BM ? scale_reg : scale_reg * output_scale;  // s_sb follows s_sa
  int* stage = reinterpret_cast<int*>(smem + wave * kStageBytes);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    // a light tile's wave holds one 64-row block (rows 64 wm .. + 63)
    if (half == 1 && light) break;
    if (half == 1) __syncthreads();  // the first half's rows are read back by now
    constexpr int kHalfFrags = kStageRows / 16;
#pragma unroll
    for (int ii = 0; ii < kHalfFrags; ++ii)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        tile::stage_fragment(stage, lane, ii, j, acc[half * kHalfFrags + ii][j]);
    __syncthreads();  // staged blocks and scales visible
    const int lrow0 = light ? wm * kStageRows : wm * WTM + half * kStageRows;
    const int lcol0 = wn * WTN;
    if (c)
      tile::store4<kStageRows, false, true>(stage, lane, m0, n0, lrow0, lcol0, M, N, s_sa, s_sb, c);
    if (out) {
      if (out_dtype == QK_BF16)
        tile::store_bf16<kStageRows, false>(stage, lane, m0, n0, lrow0, lcol0, M, N, s_sa, s_sb,
                                            out);
      else
        tile::store4<kStageRows, false, false>(stage, lane, m0, n0, lrow0, lcol0, M, N, s_sa,
                                               s_sb, out);
    }
  }
}

template <int MODE, bool KTAIL>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_wide_kernel(
    const int8_t* __restrict__ a, const int8_t* __restrict__ b, int32_t* __restrict__ c,
    const float* __restrict__ scale_a, const float* __restrict__ scale_b, float output_scale,
    void* __restrict__ out, int out_dtype, int M, int N, int K, int tiles_m, int tiles_n) {
  int tm, tn;
  tile::tile_coords(tiles_m, tiles_n, tm, tn);
  gemm_wide_tile<MODE, KTAIL>(a, b, c, scale_a, scale_b, output_scale, out, out_dtype, M, N, K,
                              tm, tn);
}

// The MoE grouped GEMM on 256 x 256 tiles: expert e's rows [offsets[e],
// offsets[e + 1]) times its weight b + e * expert_stride, with its
// per-channel scales scale_b + e * N; moe_pick (gemm_tile.h) gives each
// workgroup its expert and tile.
template <int MODE, bool KTAIL>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_wide_moe_kernel(
    const int8_t* __restrict__ a, const int8_t* __restrict__ b, int32_t* __restrict__ c,
    const float* __restrict__ scale_a, const float* __restrict__ scale_b, float output_scale,
    void* __restrict__ out, int out_dtype, int M, int N, int K, int tiles_n,
    const int* __restrict__ offsets, int experts, long long expert_stride) {
  int e, local, r0, Me;
  if (!tile::moe_pick<BM, QK_MOE_MAX_EXPERTS>(offsets, experts, M, tiles_n, e, local, r0, Me))
    return;
  int tm, tn;
  tile::group_order(local, (Me + BM - 1) / BM, tiles_n, tm, tn);
  // an expert's last row block of at most 128 rows: a light tile
  const bool light = Me - tm * BM <= BM / 2;
  const size_t row_off = static_cast<size_t>(r0);
  void* out_e = out ? static_cast<char*>(out) + row_off * N * (out_dtype == QK_BF16 ? 2 : 4) : nullptr;
  gemm_wide_tile<MODE, KTAIL>(a + row_off * K, b + e * expert_stride, c ? c + row_off * N : nullptr,
                              scale_a ? scale_a + row_off : nullptr,
                              scale_b ? scale_b + static_cast<size_t>(e) * N : nullptr,
                              output_scale, out_e, out_dtype, Me, N, K, tm, tn, light);
}

template <int MODE>
hipError_t launch_wide_moe_mode(const GemmArgs& g, const int* offsets, int experts, dim3 grid,
                                int tiles_n, hipStream_t stream) {
  const long long stride = static_cast<long long>(g.k) * g.n;
  if (g.k % BK != 0)
    return launch(gemm_i8_wide_moe_kernel<MODE, true>, grid, dim3(kThreads), 0, stream, g.a, g.b,
                  g.c, g.scale_a, g.scale_b, g.output_scale, g.out, g.out_dtype, g.m, g.n, g.k,
                  tiles_n, offsets, experts, stride);
  return launch(gemm_i8_wide_moe_kernel<MODE, false>, grid, dim3(kThreads), 0, stream, g.a, g.b,
                g.c, g.scale_a, g.scale_b, g.output_scale, g.out, g.out_dtype, g.m, g.n, g.k,
                tiles_n, offsets, experts, stride);
}

template <int MODE>
hipError_t launch_wide_mode(const GemmArgs& g, dim3 grid, int tiles_m, int tiles_n,
                            hipStream_t stream) {
  if (g.k % BK != 0)
    return launch(gemm_i8_wide_kernel<MODE, true>, grid, dim3(kThreads), 0, stream, g.a, g.b,
                  g.c, g.scale_a, g.scale_b, g.output_scale, g.out, g.out_dtype, g.m, g.n, g.k,
                  tiles_m, tiles_n);
  return launch(gemm_i8_wide_kernel<MODE, false>, grid, dim3(kThreads), 0, stream, g.a, g.b, g.c,
                g.scale_a, g.scale_b, g.output_scale, g.out, g.out_dtype, g.m, g.n, g.k, tiles_m,
                tiles_n);
}

}  // namespace wide
}  // namespace

bool gemm_wide_applies(int m, int n, int k, int b_layout) {
  // k, n <= 2^24: the transfers' 32-bit lane offsets (256 rows of k bytes,
  // 64 k rows of n bytes) fit
  if (k <= 0 || n < 16 || k > (1 << 24) || n > (1 << 24)) return false;
  if (b_layout == QK_B_KN && n % 16 != 0) return false;  // DMA of [k][n] rows in 16-byte chunks
  const long long tiles = static_cast<long long>((m + wide::BM - 1) / wide::BM) *
                          ((n + wide::BN - 1) / wide::BN);
  return tiles >= 256;  // at least one 256 x 256 tile per CU
}

bool gemm_wide_moe_applies(int m, int n, int k, int b_layout) {
  // the dense GEMM of all rows would take the 256 x 256 tiles
  return gemm_wide_applies(m, n, k, b_layout);
}

hipError_t launch_gemm_wide_moe(const GemmArgs& g, const int* offsets, int experts,
                                hipStream_t stream) {
  // at most floor(m / BM) + experts tile rows over all experts
  const int tiles_n = (g.n + wide::BN - 1) / wide::BN;
  const long long tiles = (static_cast<long long>(g.m) / wide::BM + experts) * tiles_n;
  if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(tiles));
  if (g.b_layout == QK_B_NK)
    return wide::launch_wide_moe_mode<tile::kBnkDma>(g, offsets, experts, grid, tiles_n, stream);
  return wide::launch_wide_moe_mode<tile::kBknDma>(g, offsets, experts, grid, tiles_n, stream);
}

hipError_t launch_gemm_wide(const GemmArgs& g, hipStream_t stream) {
  const int tiles_m = (g.m + wide::BM - 1) / wide::BM;
  const int tiles_n = (g.n + wide::BN - 1) / wide::BN;
  const long long tiles = static_cast<long long>(tiles_m) * tiles_n;
  if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(tiles));
  if (g.b_layout == QK_B_NK) return wide::launch_wide_mode<tile::kBnkDma>(g, grid, tiles_m, tiles_n, stream);
  return wide::launch_wide_mode<tile::kBknDma>(g, grid, tiles_m, tiles_n, stream);
}

}  // namespace qk
