// INT8 x INT8 -> INT32 GEMM on CDNA4 matrix cores with the dequant epilogue fused.
//
// What it computes ("16. Deploying Custom Kernels", C++ Kernel Interface;
// "KV-cache kernels", 02 Scales and dequantization; INT32 accumulation from
// "Skill: Write an INT8 Quantized Kernel", Inputs):
//   acc[i][j] = sum_t a[i][t] * B(t, j)        exact INT32
//   c[i][j]   = acc                            (optional)
//   out[i][j] = ((float)acc * scale_a[i]) * (scale_b[j] * output_scale)   (optional)
//
// Design for gfx950:
//   * Workgroup tile 256 (M) x 128 (N), k slice 128 bytes, eight wave64s (two
//     per SIMD).  The waves form two groups of four: each group covers the
//     whole tile as four 128 x 64 sub-tiles computed with
//     v_mfma_i32_16x16x64_i8 (8 x 4 instructions per 64-deep k step, 128
//     INT32 accumulators per lane), group g multiplying bytes [64 g, 64 g + 64)
//     of every slice.  M=2048, N=4096 is 256 tiles: one per CU.
//   * 16x16x64 rather than 32x32x32: the chip runs power-limited here, and on
//     this workload's operands the same MACs issued as 16x16x64 draw less
//     power per MAC (a pure MFMA loop measured 24% faster at equal work; with
//     all-zero operands both shapes run at the same rate).
//   * Operands go from global memory straight into LDS with 128-bit
//     global_load_lds (no register staging): lane l of a wave writes LDS
//     bytes [16 l, 16 l + 16) above the wave's base address, so each lane
//     fetches the global chunk that belongs at its LDS slot.  Three LDS
//     slices (3 x 48 KiB) let slice s + 2 stream in while slice s is
//     multiplied; one barrier per slice.
//   * A (and a weight stored [N][K]) is kept k-contiguous, 128-byte rows with
//     the 16-byte chunk index XORed by (row >> 1) & 7: the 16 lanes served
//     together by a 128-bit fragment read (16 consecutive rows, one chunk)
//     hit 16 distinct 16-byte bank groups.
//   * A weight stored [K][N] (n contiguous) stays [k][n] in LDS (chunk index
//     XORed by (k & 7) ^ ((k >> 4) & 1)) and is read with ds_read_b64_tr_b8: a
//     16-lane group reads an 8 (k) x 16 (n) byte block and lane j receives
//     column j's eight k values, which is the k-contiguous MFMA operand; two
//     such reads give the 16 bytes of a lane.  No VALU transposes are needed.
//   * For a [K][N] weight whose N is not a multiple of 16, B falls back to
//     register staging (dword or byte loads, 4 x 4 byte transposes with
//     v_perm_b32, LDS writes in the [n][k] layout).
//   * Rows past M or N re-read a valid row (those outputs are never stored).
//     When K is not a multiple of 128 the final slice's A chunks at k >= K are
//     zeroed in LDS before use, so they add nothing.
//   * Workgroups are dispatched to the 8 XCDs round robin; tiles are renumbered
//     so the ones running together on one XCD form a compact 4 x 8 block that
//     shares A rows and B columns in that XCD's L2.
//   * Epilogue: the two wave groups swap half of their partial sums through
//     LDS as 16-byte chunks; each lane transposes 4 x 4 blocks across its
//     lane quad (DPP) and writes 4 consecutive columns of one row to a
//     row-major staging block in LDS; the block is read back row-contiguous,
//     the per-token and per-channel scales are applied in binary32, and fp32
//     or bf16 (round to nearest even), or the raw accumulators, are stored as
//     whole 128-byte row segments with nontemporal stores.
//   * Operands are addressed with 32-bit offsets (m*k, n*k < 2^32).
#include "gemm_tile.h"

namespace qk {
namespace {

using namespace tile;

constexpr int kGroups = 2;              // wave groups splitting each k slice
constexpr int WTM = 128;       // wave tile rows
constexpr int WTN = 64;        // wave tile columns
constexpr int FM = WTM / 16;   // 16x16 fragments per wave along M
constexpr int FN = WTN / 16;   // ... along N
constexpr int kSubTiles = (BM / WTM) * (BN / WTN);  // wave sub-tiles per workgroup tile
static_assert(kSubTiles * kGroups == kWaves, "every wave owns one (sub-tile, k group)");

// One workgroup's 256 x 128 output tile (tm, tn) of an M x N x K product.
// ASYM: the activations carry per-row zero points zp_a, and the epilogue
// subtracts zp_a[row] * wsum[col] (wsum: the weight's column sums) from the
// INT32 accumulators before storing or scaling them.
template <int MODE, bool KTAIL, bool ASYM = false>
__device__ __forceinline__ void gemm_i8_tile(
    const int8_t* __restrict__ a, const int8_t* __restrict__ b, int32_t* __restrict__ c,
    const float* __restrict__ scale_a, const float* __restrict__ scale_b, float output_scale,
    void* __restrict__ out, int out_dtype, int M, int N, int K, int tm, int tn,
    const int32_t* __restrict__ zp_a = nullptr, const int32_t* __restrict__ wsum = nullptr,
    int lda = -1, int ldb = -1) {
  constexpr bool kRegB = MODE == kBknReg4 || MODE == kBknReg1;
  __shared__ __attribute__((aligned(1024))) char smem[kStages * STAGE];

  const int m0 = tm * BM;
  const int n0 = tn * BN;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int grp = (t >> 6) / kSubTiles;  // which 64-byte half of each k slice this wave multiplies
  const int wsub = (t >> 6) % kSubTiles;  // which 128 x 64 sub-tile it owns
  const int wm = wsub / (BN / WTN);
  const int wn = wsub % (BN / WTN);

  // this thread's per-token or per-channel scale of the tile, loaded now so
  // that its latency hides behind the main loop; the epilogue stages it to LDS
  static_assert(BM + BN <= kThreads, "one scale per thread");
  float scale_reg = 0.0f;
  if (out) {
    if (t < BM) {
      if (m0 + t < M) scale_reg = scale_a[m0 + t];
    } else if (t < BM + BN) {
      if (n0 + t - BM < N) scale_reg = scale_b[n0 + t - BM];  // times output_scale later
    }
  }
  int corr_reg = 0;  // this thread's row zero point or column sum (ASYM)
  if constexpr (ASYM) {
    if (t < BM) {
      if (m0 + t < M) corr_reg = zp_a[m0 + t];
    } else if (t < BM + BN) {
      if (n0 + t - BM < N) corr_reg = wsum[n0 + t - BM];
    }
  }

  auto a_lds = [&](int s) { return smem + (s % kStages) * STAGE; };
  auto b_lds = [&](int s) { return smem + (s % kStages) * STAGE + A_STAGE; };

  using RegTile = std::conditional_t<MODE == kBknReg4, KnRegTile<true>,
                                     std::conditional_t<MODE == kBknReg1, KnRegTile<false>, NoRegTile>>;
  RegTile breg;

  // issue the global reads of k slice s (DMA: straight into its LDS slice)
  auto fetch = [&](int s) {
    dma_rowk<BM>(a, a_lds(s), M, K, m0, s * BK, lda);
    if constexpr (MODE == kBnkDma) dma_rowk<BN>(b, b_lds(s), N, K, n0, s * BK, ldb);
    if constexpr (MODE == kBknDma) dma_kn(b, b_lds(s), N, K, n0, s * BK);
  };
  constexpr int kFetchOps = BM * BK / 1024 / kWaves + (kRegB ? 0 : BN * BK / 1024 / kWaves);
  // one DMA instruction of slice s: parts [0, kOpsA) are A, the rest B.
  // Without a K tail no clamp changes from slice to slice, so each part's
  // source address and LDS slot are formed once: slice s adds s times the
  // part's stride (BK bytes along k) and the stage offset.
  constexpr int kOpsA = rowk_ops<BM>();
  constexpr bool kFixedParts = !KTAIL && !kRegB;
  const uint32_t lds_smem = lds_addr(smem);
  using Parts = std::conditional_t<kFixedParts, FixedParts<MODE == kBnkDma ? kBnkDma : kBknDma>,
                                   NoParts>;
  Parts parts;
  if constexpr (kFixedParts) {
    static_assert(Parts::kOps == kFetchOps, "one DMA instruction per part");
    parts.init(a, b, M, N, K, m0, n0, lda, ldb);
  }
  auto fetch_part = [&](int s, int part) {
    if constexpr (kFixedParts) {
      parts.issue(lds_smem, s, part);
    } else if (part < kOpsA) {
      dma_rowk_one<BM>(a, a_lds(s), M, K, m0, s * BK, part, lda);
    } else if constexpr (MODE == kBnkDma) {
      dma_rowk_one<BN>(b, b_lds(s), N, K, n0, s * BK, part - kOpsA, ldb);
    } else if constexpr (MODE == kBknDma) {
      dma_kn_one(b, b_lds(s), N, K, n0, s * BK, part - kOpsA);
    }
  };

  // Fragments of v_mfma_i32_16x16x64_i8: lane l holds 16 k-consecutive bytes,
  // k = 16 (l / 16) .. + 15 of the wave group's 64-byte k step, of row l % 16
  // (A) or column l % 16 (B) of the fragment.  A (and [N][K] / register-staged
  // B) take one 128-bit read; a DMA'd [K][N] B takes two transpose reads.
  const int kchunk = 4 * grp + (lane >> 4);  // the lane's 16-byte chunk of a slice row
  const int a_row = wm * WTM + (lane & 15);
  const int b_row = wn * WTN + (lane & 15);
  auto read_a = [&](const char* As, int i) -> v4i {
    return *reinterpret_cast<const v4i*>(As + rowk_offset(a_row + i * 16, kchunk));
  };
  // B fragment j of a [K][N] weight: transpose read h covers k rows 8h .. 8h + 7
  // of the lane's 16
  auto read_b_tr = [&](const char* Bs, int j, int h) -> v2i {
    const int i16 = lane & 15;
    const int kr = 64 * grp + 16 * (lane >> 4) + (i16 >> 1) + 8 * h;
    const int cb = (wn * WTN + j * 16) >> 4;
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) v2i*)(Bs + kn_offset(kr, cb) + 8 * (i16 & 1)));
  };
  auto read_b_rowk = [&](const char* Bs, int j) -> v4i {
    return *reinterpret_cast<const v4i*>(Bs + rowk_offset(b_row + j * 16, kchunk));
  };
  auto read_b = [&](const char* Bs, int j) -> v4i {
    if constexpr (MODE == kBknDma) {
      const v2i lo = read_b_tr(Bs, j, 0);
      const v2i hi = read_b_tr(Bs, j, 1);
      return v4i{lo.x, lo.y, hi.x, hi.y};
    } else {
      return read_b_rowk(Bs, j);
    }
  };

  v4i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v4i{};

  const int KT = (K + BK - 1) / BK;

  // Zero the A chunks of slice s that lie at k >= K (final slice of a K that
  // is not a multiple of BK), then publish with a barrier.
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

  v4i fa[FM], fb[FN];  // fragments of the slice being multiplied
  if (KT > 0) {
    fetch(0);
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
    // the DMA schedule below reads fragments A 4..7 and B 2..3 of a slice
    // while it multiplies the others
    constexpr int kFirstA = kRegB ? FM : FM / 2;
    constexpr int kFirstB = kRegB ? FN : FN / 2;
#pragma unroll
    for (int i = 0; i < kFirstA; ++i) fa[i] = read_a(a_lds(0), i);
#pragma unroll
    for (int j = 0; j < kFirstB; ++j) fb[j] = read_b(b_lds(0), j);
  }

  if constexpr (kRegB) {
    // register-staged weight (N not a multiple of 16): one slice per
    // iteration, the next slice's B staged through registers
    for (int kt = 0; kt < KT; ++kt) {
      if (kt + 2 < KT) fetch(kt + 2);
      if (kt + 1 < KT) breg.load(b, N, K, n0, (kt + 1) * BK);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
      if (kt + 1 < KT) {
        wait_vmcnt<0>();
        breg.store(b_lds(kt + 1));
        __syncthreads();
        if (KTAIL && kt + 1 == KT - 1) zero_tail(kt + 1);
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[i] = read_a(a_lds(kt + 1), i);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[j] = read_b_rowk(b_lds(kt + 1), j);
      }
    }
  } else {
    // DMA modes, one k slice per iteration in two phases, every instruction's
    // place pinned by sched_barrier and every fragment read several MFMAs
    // ahead of its first use:
    //   phase 0: MFMAs of A 0..3 x B 0..1 (fragments read in the previous
    //            iteration); this slice's A 4..7 and B 2..3 are read in its
    //            first half, so the barrier's wait for LDS reads finds them
    //            done, and DMA parts [0, kSplit) of slice kt + 2 follow (its
    //            LDS stage held slice kt - 1, whose last reads every wave
    //            completed before the previous iteration's barrier);
    //   barrier: this wave's DMA of slice kt + 1 has landed (vmcnt), then all
    //            waves' (s_barrier);
    //   phase 1: A 4..7 x B 0 and B 1 (then slice kt + 1's B 0..1 are read
    //            into the freed registers), A 0..3 x B 2..3 (each A register
    //            refilled with slice kt + 1's fragment after its last MFMA),
    //            A 4..7 x B 2..3, with the remaining DMA parts in between.
    // The DMA instructions are spread through the MFMA stream because a CU
    // accepts its loads at a limited rate, and a wave waiting to issue one
    // cannot issue its MFMAs either.
    static_assert(FM == 8 && FN == 4, "interleave pattern below");
    constexpr int kSplit = kFetchOps / 2;
    static_assert(kFetchOps == 2 * kSplit && kSplit == 3, "three DMA slots per phase");
    for (int kt = 0; kt < KT; ++kt) {
      const bool prefetch = kt + 2 < KT;
      auto mfma = [&](int i, int j) {
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      };
      auto dma = [&](int part) {
        if (prefetch) fetch_part(kt + 2, part);
        __builtin_amdgcn_sched_barrier(0);
      };
      auto sb = [] { __builtin_amdgcn_sched_barrier(0); };
      // ---- phase 0 ----
      {
        const char* As = a_lds(kt);
        const char* Bs = b_lds(kt);
        fa[4] = read_a(As, 4);
        sb();
        mfma(0, 0);
        fa[5] = read_a(As, 5);
        sb();
        fa[6] = read_a(As, 6);
        sb();
        mfma(0, 1);
        fa[7] = read_a(As, 7);
        sb();
        if constexpr (MODE == kBknDma) {
          v2i lo[2], hi[2];
          lo[0] = read_b_tr(Bs, 2, 0);
          sb();
          mfma(1, 0);
          hi[0] = read_b_tr(Bs, 2, 1);
          sb();
          lo[1] = read_b_tr(Bs, 3, 0);
          sb();
          mfma(1, 1);
          hi[1] = read_b_tr(Bs, 3, 1);
          sb();
          fb[2] = v4i{lo[0].x, lo[0].y, hi[0].x, hi[0].y};
          fb[3] = v4i{lo[1].x, lo[1].y, hi[1].x, hi[1].y};
        } else {
          fb[2] = read_b_rowk(Bs, 2);
          sb();
          mfma(1, 0);
          fb[3] = read_b_rowk(Bs, 3);
          sb();
          mfma(1, 1);
        }
        dma(0);
        mfma(2, 0);
        dma(1);
        mfma(2, 1);
        dma(2);
        mfma(3, 0);
        mfma(3, 1);
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
        // slice and are not used: no branches around LDS reads, so the
        // compiler's waits for them stay exact
        const char* As = a_lds(kt + 1);
        const char* Bs = b_lds(kt + 1);
        v4i na[4], nb[2];
        mfma(4, 0);
        mfma(5, 0);
        dma(kSplit + 0);
        mfma(6, 0);
        mfma(7, 0);
        if constexpr (MODE == kBknDma) {
          v2i lo[2], hi[2];
          lo[0] = read_b_tr(Bs, 0, 0);
          mfma(4, 1);
          hi[0] = read_b_tr(Bs, 0, 1);
          mfma(5, 1);
          mfma(6, 1);
          mfma(7, 1);
          lo[1] = read_b_tr(Bs, 1, 0);
          mfma(0, 2);
          hi[1] = read_b_tr(Bs, 1, 1);
          nb[0] = v4i{lo[0].x, lo[0].y, hi[0].x, hi[0].y};
          nb[1] = v4i{lo[1].x, lo[1].y, hi[1].x, hi[1].y};
        } else {
          nb[0] = read_b_rowk(Bs, 0);
          mfma(4, 1);
          mfma(5, 1);
          mfma(6, 1);
          mfma(7, 1);
          nb[1] = read_b_rowk(Bs, 1);
          mfma(0, 2);
        }
        mfma(0, 3);
        na[0] = read_a(As, 0);
        mfma(1, 2);
        dma(kSplit + 1);
        mfma(1, 3);
        na[1] = read_a(As, 1);
        mfma(2, 2);
        mfma(2, 3);
        na[2] = read_a(As, 2);
        mfma(3, 2);
        dma(kSplit + 2);
        mfma(3, 3);
        na[3] = read_a(As, 3);
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
    }
  }

  // ---- epilogue ----
  // The two wave groups hold partial sums of the same 128 x 64 sub-tile.
  // Group g finishes fragment rows i in [4g, 4g + 4): it hands the other
  // group's fragments over through LDS as 16-byte chunks (the 4 accumulator
  // registers of a lane) and adds the chunks it receives.  A fragment's
  // register r of lane l is element (4 (l / 16) + r, l % 16); a 4 x 4
  // transpose across each lane quad (DPP) gives every lane four consecutive
  // columns of one row for the staging below.  Output stores are
  // nontemporal: nothing here reads them.
  constexpr int kHalfM = FM / kGroups;  // fragment rows finished per group
  constexpr int kChunkBytes = kHalfM * FN * 64 * 16;  // one group's hand-over
  static_assert(2 * kSubTiles * kChunkBytes + 8 * (BM + BN) <= kStages * STAGE,
                "epilogue hand-over, scales and zero-point terms fit in LDS");
  __syncthreads();  // every wave is done with the k slices
  float* s_sa = reinterpret_cast<float*>(smem + 2 * kSubTiles * kChunkBytes);
  float* s_sb = s_sa + BM;
  if (out && t < BM + BN) s_sa[t] = t < BM ? scale_reg : scale_reg * output_scale;  // s_sb follows s_sa
  int* s_zp = reinterpret_cast<int*>(s_sa + BM + BN);  // row zero points, then column sums (ASYM)
  int* s_ws = s_zp + BM;
  if (ASYM && t < BM + BN) s_zp[t] = corr_reg;
  // hand-over region written for group `to` of this sub-tile
  auto chunk_at = [&](int to, int ii, int j) -> v4i* {
    return reinterpret_cast<v4i*>(smem + (wsub * 2 + to) * kChunkBytes +
                                  ((ii * FN + j) * 64 + lane) * 16);
  };
  auto give = [&](auto i_off) {  // fragments i_off .. i_off + kHalfM - 1 go to the other group
#pragma unroll
    for (int ii = 0; ii < kHalfM; ++ii)
#pragma unroll
      for (int j = 0; j < FN; ++j) *chunk_at(1 - grp, ii, j) = acc[i_off + ii][j];
  };
  auto take = [&](auto i_off) {  // add the other group's sums for my fragments
#pragma unroll
    for (int ii = 0; ii < kHalfM; ++ii)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i_off + ii][j] += *chunk_at(grp, ii, j);
  };
  if (grp == 0) give(std::integral_constant<int, kHalfM>{}); else give(std::integral_constant<int, 0>{});
  __syncthreads();  // hand-over and scales visible
  if (grp == 0) take(std::integral_constant<int, 0>{}); else take(std::integral_constant<int, kHalfM>{});

  // Each wave now holds the final sums of a 64 x 64 block: rows
  // [16 i_off, 16 i_off + 64) of its sub-tile.  It stages them row-major in
  // LDS (the hand-over region, free after this barrier) and reads them back
  // row-contiguous, so that every store instruction writes whole 128-byte
  // row segments.
  __syncthreads();
  constexpr int kFinRows = kHalfM * 16;
  constexpr int kStageBytes = kFinRows * WTN * 4;
  static_assert(kWaves * kStageBytes <= 2 * kSubTiles * kChunkBytes, "staging fits in the hand-over region");
  static_assert(WTN == kStageCols, "staging rows are one wave tile wide");
  int* stage = reinterpret_cast<int*>(smem + (t >> 6) * kStageBytes);
  auto stage_out = [&](auto i_off) {
#pragma unroll
    for (int ii = 0; ii < kHalfM; ++ii)
#pragma unroll
      for (int j = 0; j < FN; ++j) stage_fragment(stage, lane, ii, j, acc[i_off + ii][j]);
  };
  if (grp == 0) stage_out(std::integral_constant<int, 0>{}); else stage_out(std::integral_constant<int, kHalfM>{});

  const int lrow0 = wm * WTM + (grp == 0 ? 0 : kFinRows);  // tile-local first row of the block
  const int lcol0 = wn * WTN;
  if (c)
    store4<kFinRows, false, true, ASYM>(stage, lane, m0, n0, lrow0, lcol0, M, N, s_sa, s_sb, c,
                                        s_zp, s_ws);
  if (out) {
    if (out_dtype == QK_BF16)
      store_bf16<kFinRows, false, ASYM>(stage, lane, m0, n0, lrow0, lcol0, M, N, s_sa, s_sb, out,
                                        s_zp, s_ws);
    else
      store4<kFinRows, false, false, ASYM>(stage, lane, m0, n0, lrow0, lcol0, M, N, s_sa, s_sb,
                                           out, s_zp, s_ws);
  }
}

template <int MODE, bool KTAIL>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_mfma_kernel(
    const int8_t* __restrict__ a, const int8_t* __restrict__ b, int32_t* __restrict__ c,
    const float* __restrict__ scale_a, const float* __restrict__ scale_b, float output_scale,
    void* __restrict__ out, int out_dtype, int M, int N, int K, int tiles_m, int tiles_n) {
  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  gemm_i8_tile<MODE, KTAIL>(a, b, c, scale_a, scale_b, output_scale, out, out_dtype, M, N, K, tm,
                            tn);
}

// MoE grouped GEMM ("dynquant-kernels", What is in here: one launch for all
// experts): rows [offsets[e], offsets[e + 1]) of a belong to expert e, whose
// weight is b + e * expert_stride and per-channel scales scale_b + e * N.
// Each workgroup finds its expert and tile with moe_pick (gemm_tile.h).
constexpr int kMoeMaxExperts = QK_MOE_MAX_EXPERTS;
template <int MODE, bool KTAIL>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_moe_kernel(
    const int8_t* __restrict__ a, const int8_t* __restrict__ b, int32_t* __restrict__ c,
    const float* __restrict__ scale_a, const float* __restrict__ scale_b, float output_scale,
    void* __restrict__ out, int out_dtype, int M, int N, int K, int tiles_n,
    const int* __restrict__ offsets, int experts, long long expert_stride) {
  int e, local, r0, Me;
  if (!moe_pick<BM, kMoeMaxExperts>(offsets, experts, M, tiles_n, e, local, r0, Me)) return;
  int tm, tn;
  group_order(local, (Me + BM - 1) / BM, tiles_n, tm, tn);
  const size_t row_off = static_cast<size_t>(r0);
  void* out_e = out ? static_cast<char*>(out) + row_off * N * (out_dtype == QK_BF16 ? 2 : 4) : nullptr;
  gemm_i8_tile<MODE, KTAIL>(a + row_off * K, b + e * expert_stride, c ? c + row_off * N : nullptr,
                            scale_a ? scale_a + row_off : nullptr,
                            scale_b ? scale_b + static_cast<size_t>(e) * N : nullptr, output_scale,
                            out_e, out_dtype, Me, N, K, tm, tn);
}

// Asymmetric activations: codes with per-row zero points; the result is
// sum_t (a[i][t] - zp_a[i]) * B(t, j) = acc - zp_a[i] * wsum[j].
template <int MODE, bool KTAIL>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_asym_kernel(
    const int8_t* __restrict__ a, const int8_t* __restrict__ b, int32_t* __restrict__ c,
    const float* __restrict__ scale_a, const float* __restrict__ scale_b, float output_scale,
    void* __restrict__ out, int out_dtype, int M, int N, int K, int tiles_m, int tiles_n,
    const int32_t* __restrict__ zp_a, const int32_t* __restrict__ wsum) {
  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  gemm_i8_tile<MODE, KTAIL, true>(a, b, c, scale_a, scale_b, output_scale, out, out_dtype, M, N, K,
                                  tm, tn, zp_a, wsum);
}

template <int MODE>
hipError_t launch_mode(const GemmArgs& g, dim3 grid, int tiles_m, int tiles_n,
                       hipStream_t stream) {
  if (g.k % BK != 0)
    return launch(gemm_i8_mfma_kernel<MODE, true>, grid, dim3(kThreads), 0, stream, g.a, g.b, g.c,
                  g.scale_a, g.scale_b, g.output_scale, g.out, g.out_dtype, g.m, g.n, g.k,
                  tiles_m, tiles_n);
  return launch(gemm_i8_mfma_kernel<MODE, false>, grid, dim3(kThreads), 0, stream, g.a, g.b, g.c,
                g.scale_a, g.scale_b, g.output_scale, g.out, g.out_dtype, g.m, g.n, g.k, tiles_m,
                tiles_n);
}

template <int MODE>
hipError_t launch_moe_mode(const GemmArgs& g, const int* offsets, int experts, dim3 grid,
                           int tiles_n, hipStream_t stream) {
  const long long stride = static_cast<long long>(g.k) * g.n;
  if (g.k % BK != 0)
    return launch(gemm_i8_moe_kernel<MODE, true>, grid, dim3(kThreads), 0, stream, g.a, g.b, g.c,
                  g.scale_a, g.scale_b, g.output_scale, g.out, g.out_dtype, g.m, g.n, g.k, tiles_n,
                  offsets, experts, stride);
  return launch(gemm_i8_moe_kernel<MODE, false>, grid, dim3(kThreads), 0, stream, g.a, g.b, g.c,
                g.scale_a, g.scale_b, g.output_scale, g.out, g.out_dtype, g.m, g.n, g.k, tiles_n,
                offsets, experts, stride);
}

}  // namespace

int moe_max_experts() { return kMoeMaxExperts; }

namespace {
template <int MODE>
hipError_t launch_asym_mode(const GemmArgs& g, const int32_t* zp_a, const int32_t* wsum, dim3 grid,
                            int tiles_m, int tiles_n, hipStream_t stream) {
  if (g.k % BK != 0)
    return launch(gemm_i8_asym_kernel<MODE, true>, grid, dim3(kThreads), 0, stream, g.a, g.b, g.c,
                  g.scale_a, g.scale_b, g.output_scale, g.out, g.out_dtype, g.m, g.n, g.k, tiles_m,
                  tiles_n, zp_a, wsum);
  return launch(gemm_i8_asym_kernel<MODE, false>, grid, dim3(kThreads), 0, stream, g.a, g.b, g.c,
                g.scale_a, g.scale_b, g.output_scale, g.out, g.out_dtype, g.m, g.n, g.k, tiles_m,
                tiles_n, zp_a, wsum);
}
}  // namespace

hipError_t launch_gemm_asym(const GemmArgs& g, const int32_t* zp_a, const int32_t* wsum,
                            hipStream_t stream) {
  const int tiles_m = (g.m + BM - 1) / BM;
  const int tiles_n = (g.n + BN - 1) / BN;
  const long long tiles = static_cast<long long>(tiles_m) * tiles_n;
  if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(tiles));
  // the kernel with transfer waves apart where it applies (as for the plain GEMM)
  if (gemm_spec_applies(g.m, g.n, g.k, g.b_layout)) return launch_gemm_spec_asym(g, zp_a, wsum, stream);
  if (g.b_layout == QK_B_NK) return launch_asym_mode<kBnkDma>(g, zp_a, wsum, grid, tiles_m, tiles_n, stream);
  if (g.n % 16 == 0) return launch_asym_mode<kBknDma>(g, zp_a, wsum, grid, tiles_m, tiles_n, stream);
  if (g.n % 4 == 0) return launch_asym_mode<kBknReg4>(g, zp_a, wsum, grid, tiles_m, tiles_n, stream);
  return launch_asym_mode<kBknReg1>(g, zp_a, wsum, grid, tiles_m, tiles_n, stream);
}

hipError_t launch_gemm_moe(const GemmArgs& g, const int* offsets, int experts, hipStream_t stream) {
  if (gemm_wide_moe_applies(g.m, g.n, g.k, g.b_layout)) return launch_gemm_wide_moe(g, offsets, experts, stream);
  // at most floor(m / BM) + experts tile rows over all experts
  const int tiles_n = (g.n + BN - 1) / BN;
  const long long tiles = (static_cast<long long>(g.m) / BM + experts) * tiles_n;
  if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(tiles));
  if (g.b_layout == QK_B_NK) return launch_moe_mode<kBnkDma>(g, offsets, experts, grid, tiles_n, stream);
  if (g.n % 16 == 0) return launch_moe_mode<kBknDma>(g, offsets, experts, grid, tiles_n, stream);
  if (g.n % 4 == 0) return launch_moe_mode<kBknReg4>(g, offsets, experts, grid, tiles_n, stream);
  return launch_moe_mode<kBknReg1>(g, offsets, experts, grid, tiles_n, stream);
}

namespace {

// ---- split-K for outputs with few tiles ----
// An output of fewer than 128 tiles (e.g. 2048 x 512: 32 tiles) leaves most
// CUs idle while each tile runs the whole k range.  Workgroup (s, t) then
// multiplies tile t over the k slice [s * kslice, (s + 1) * kslice) and
// stores its raw INT32 partial sums to slice s of the workspace; a second
// kernel adds the slices in order (exact, and the same bits on every run),
// returns the workspace to zero, and applies the epilogue.
template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_splitk_kernel(
    const int8_t* __restrict__ a, const int8_t* __restrict__ b, int32_t* __restrict__ part,
    int M, int N, int K, int tiles_m, int tiles_n, int kslice) {
  const int tiles = tiles_m * tiles_n;
  const int s = static_cast<int>(blockIdx.x) / tiles;
  const int t = static_cast<int>(blockIdx.x) - s * tiles;
  int tm, tn;
  group_order(xcd_order(t, tiles), tiles_m, tiles_n, tm, tn);
  const int k0 = s * kslice;
  // a [K][N] weight's k range starts k0 rows down; a [N][K] one's k0 bytes in
  const int8_t* bk = MODE == kBknDma ? b + static_cast<size_t>(k0) * N : b + k0;
  gemm_i8_tile<MODE, false>(a + k0, bk, part + static_cast<size_t>(s) * M * N, nullptr, nullptr,
                            1.0f, nullptr, QK_F32, M, N, min(kslice, K - k0), tm, tn, nullptr,
                            nullptr, K, K);
}

// Four consecutive outputs of one row per thread (N % 16 == 0).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(
    int32_t* __restrict__ part, int splits, long long quads, int N, int32_t* __restrict__ c,
    const float* __restrict__ scale_a, const float* __restrict__ scale_b, float output_scale,
    void* __restrict__ out, int out_dtype) {
  const long long mn = quads * 4;
  for (long long v = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x; v < quads;
       v += static_cast<long long>(gridDim.x) * 256) {
    const long long e = 4 * v;
    v4i acc = {0, 0, 0, 0};
    for (int s = 0; s < splits; ++s) {
      v4i* p = reinterpret_cast<v4i*>(part + s * mn + e);
      acc += __builtin_nontemporal_load(p);
      __builtin_nontemporal_store(v4i{0, 0, 0, 0}, p);
    }
    if (c)
#pragma unroll
      for (int i = 0; i < 4; ++i) c[e + i] = acc[i];
    if (out) {
      const int row = static_cast<int>(e / N);
      const int col = static_cast<int>(e - static_cast<long long>(row) * N);
      const float sa = scale_a[row];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float f = (static_cast<float>(acc[i]) * sa) * (scale_b[col + i] * output_scale);
        if (out_dtype == QK_BF16)
          static_cast<uint16_t*>(out)[e + i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
        else
          static_cast<float*>(out)[e + i] = f;
      }
    }
  }
}

}  // namespace

SplitKPlan splitk_plan(int m, int n, int k, int b_layout) {
  SplitKPlan p{1, k, 0};
  if (m <= 0 || (b_layout != QK_B_KN && b_layout != QK_B_NK) || n % 16 != 0 || k % BK != 0 ||
      k < 2048)
    return p;
  const long long tiles = static_cast<long long>((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  if (tiles >= 128) return p;
  const int want = static_cast<int>(256 / tiles);  // (slice, tile) workgroups in one round
  // at least 1024 k per split: a tile's fixed cost (prologue, k-group hand-over,
  // stores) is ~8 slices' worth (measured: 2048 x 512 x 4096 with 512-k
  // splits 34.2 us against 33.4 unsplit)
  const int splits = min(want, k / 1024);
  if (splits < 2) return p;
  const int kt = k / BK;
  const int per = (kt + splits - 1) / splits;
  const int kslice = per * BK;
  const int nsplit = (kt + per - 1) / per;
  // worth it only when the loop time saved outweighs the partial sums' round
  // trip (written, read, cleared); fitted to eight measured shapes: ~6.2 ns per
  // k of a tile's loop, ~3.3 ps per partial-sum element (e.g. 2048 x 1024 x
  // 4096 split 4 ways measured 39.5 against 33.6 us unsplit, and is refused)
  const double saved_us = 6.2e-3 * (k - kslice);
  const double cost_us = 3.3e-6 * nsplit * static_cast<double>(m) * n;
  if (saved_us < 1.25 * cost_us) return p;
  p.splits = nsplit;
  p.kslice = kslice;
  p.bytes = (static_cast<size_t>(p.splits) * m * n * 4 + 255) / 256 * 256;
  return p;
}

namespace {

hipError_t launch_splitk(const GemmArgs& g, const SplitKPlan& p, hipStream_t stream) {
  const int tiles_m = (g.m + BM - 1) / BM;
  const int tiles_n = (g.n + BN - 1) / BN;
  auto* part = static_cast<int32_t*>(g.workspace);
  const dim3 grid(static_cast<unsigned>(p.splits * tiles_m * tiles_n));
  hipError_t e = g.b_layout == QK_B_NK
                     ? launch(gemm_i8_splitk_kernel<kBnkDma>, grid, dim3(kThreads), 0, stream, g.a,
                              g.b, part, g.m, g.n, g.k, tiles_m, tiles_n, p.kslice)
                     : launch(gemm_i8_splitk_kernel<kBknDma>, grid, dim3(kThreads), 0, stream, g.a,
                              g.b, part, g.m, g.n, g.k, tiles_m, tiles_n, p.kslice);
  if (e != hipSuccess) return e;
  const long long quads = static_cast<long long>(g.m) * g.n / 4;
  const long long blocks = (quads + 255) / 256;
  e = launch(splitk_reduce_kernel, dim3(static_cast<unsigned>(blocks < 16384 ? blocks : 16384)),
             dim3(256), 0, stream, part, p.splits, quads, g.n, g.c, g.scale_a, g.scale_b,
             g.output_scale, g.out, g.out_dtype);
  // the partial sums are already enqueued: without the reduction nothing
  // would clear them, so try to return the workspace to zero (the caller is
  // told to re-initialize it after a launch error in any case)
  if (e != hipSuccess) (void)launch_zero_fill(part, p.bytes, stream);
  return e;
}

}  // namespace

bool gemm_mfma_supported(int m, int n, int k) {
  return static_cast<unsigned long long>(m) * k < (1ull << 32) &&
         static_cast<unsigned long long>(n) * k < (1ull << 32);
}

hipError_t launch_gemm_mfma(const GemmArgs& g, hipStream_t stream) {
  const int tiles_m = (g.m + BM - 1) / BM;
  const int tiles_n = (g.n + BN - 1) / BN;
  const long long tiles = static_cast<long long>(tiles_m) * tiles_n;
  if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(tiles));
  const SplitKPlan p = splitk_plan(g.m, g.n, g.k, g.b_layout);
  if (p.splits > 1 && g.workspace && g.workspace_bytes >= p.bytes)
    return launch_splitk(g, p, stream);
  if (gemm_wide_applies(g.m, g.n, g.k, g.b_layout)) return launch_gemm_wide(g, stream);
  if (gemm_spec_applies(g.m, g.n, g.k, g.b_layout)) return launch_gemm_spec(g, stream);
  if (g.b_layout == QK_B_NK) return launch_mode<kBnkDma>(g, grid, tiles_m, tiles_n, stream);
  if (g.n % 16 == 0) return launch_mode<kBknDma>(g, grid, tiles_m, tiles_n, stream);
  if (g.n % 4 == 0) return launch_mode<kBknReg4>(g, grid, tiles_m, tiles_n, stream);
  return launch_mode<kBknReg1>(g, grid, tiles_m, tiles_n, stream);
}

}  // namespace qk
