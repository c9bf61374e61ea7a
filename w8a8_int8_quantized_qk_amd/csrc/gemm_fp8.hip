// FP8 (float8_e4m3fn) x FP8 GEMM with binary32 accumulation on CDNA4 matrix
// cores, the dequant epilogue fused.
//
// What it computes (the FP8 codes of "kernels: fused silu_and_mul + dynamic
// per-token FP8 quantization", Purpose and Algorithm, fed to the scaled GEMM
// of "16. Deploying Custom Kernels", C++ Kernel Interface, with the
// scale-then-multiply epilogue of "KV-cache kernels", 02 Scales and
// dequantization):
//   acc[i][j] = sum_t value(a[i][t]) * value(B(t, j))     binary32 accumulation
//   c[i][j]   = acc                                       (optional, binary32)
//   out[i][j] = (acc * scale_a[i]) * (scale_b[j] * output_scale)   (optional)
// Every product of two e4m3fn values is exact in binary32; the sums are
// rounded by the matrix cores, once per 128-deep step or finer.
//
// Design for gfx950:
//   * v_mfma_f32_16x16x128_f8f6f4 with both operands e4m3: a 16 x 16 x 128
//     step per instruction (the older 16x16x32 FP8 form issues at half the
//     rate on this chip).  A lane holds 32 bytes of a row (A) or column (B):
//     its two 16-byte k chunks of a 128-byte slice, chunk l / 16 in registers
//     0-3 and chunk 4 + l / 16 in registers 4-7.  Any assignment of k to
//     (lane group, register byte) is a correct product as long as A and B use
//     the same one, which holds because both are built the same way.
//   * Same workgroup tile, k slices, LDS layouts, global-to-LDS transfers and
//     XCD-aware tile order as the INT8 kernel (one-byte operands in both).
//     The eight waves each own a 64 x 64 sub-tile (4 x 2 of them) over the
//     whole k slice: a 128-deep instruction consumes the full slice, so the
//     INT8 kernel's split of each slice between two wave groups does not
//     apply, and no partial sums are handed over in the epilogue.
//   * Per slice a wave issues 16 MFMAs; the next slice's fragments are read
//     into a second register set while the second half of them runs.
//   * Bytes past K in the final slice are zeroed in LDS for A (+0.0 codes);
//     the weight rows or chunks read past K meet those zeros.  A NaN code in
//     the weight there would still poison the sum, as it would inside K.
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

// e4m3 x e4m3 -> binary32, 16 x 16 x 128 (format code 0 = e4m3 for both
// operands; no block scales)
__device__ __forceinline__ v4f mfma_f8(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int MODE, bool KTAIL>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp8_mfma_kernel(
    const uint8_t* __restrict__ a8, const uint8_t* __restrict__ b8, float* __restrict__ c,
    const float* __restrict__ scale_a, const float* __restrict__ scale_b, float output_scale,
    void* __restrict__ out, int out_dtype, int M, int N, int K, int tiles_m, int tiles_n) {
  constexpr bool kRegB = MODE == kBknReg4 || MODE == kBknReg1;
  __shared__ __attribute__((aligned(1024))) char smem[kStages * STAGE];
  const int8_t* a = reinterpret_cast<const int8_t*>(a8);
  const int8_t* b = reinterpret_cast<const int8_t*>(b8);

  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM;
  const int n0 = tn * BN;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave / (BN / WTN);
  const int wn = wave % (BN / WTN);

  static_assert(BM + BN <= kThreads, "one scale per thread");
  float scale_reg = 0.0f;
  if (out) {
    if (t < BM) {
      if (m0 + t < M) scale_reg = scale_a[m0 + t];
    } else if (t < BM + BN) {
      if (n0 + t - BM < N) scale_reg = scale_b[n0 + t - BM];  // times output_scale later
    }
  }

  auto a_lds = [&](int s) { return smem + (s % kStages) * STAGE; };
  auto b_lds = [&](int s) { return smem + (s % kStages) * STAGE + A_STAGE; };

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
  using Parts = std::conditional_t<kFixedParts, FixedParts<MODE == kBnkDma ? kBnkDma : kBknDma>,
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
  const int a_row = wm * WTM + (lane & 15);
  const int b_row = wn * WTN + (lane & 15);
  auto read_a = [&](const char* As, int i) -> v8i {
    const v4i lo = *reinterpret_cast<const v4i*>(As + rowk_offset(a_row + i * 16, c0));
    const v4i hi = *reinterpret_cast<const v4i*>(As + rowk_offset(a_row + i * 16, c1));
    return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  };
  // Transpose reads of a [k][n] weight: a read covers k rows kr .. kr + 7
  // (kr = 16 ch + 8 h + (i16 >> 1) for lane i16 of a 16-lane group) of
  // fragment column block j, and lane i16 receives column i16's eight bytes.
  // The row swizzle kn_swz(kr) = (i16 >> 1) ^ (ch & 1) is the same for the
  // lane's chunks c0 and c1 = c0 + 4 and both halves h, so the four reads
  // of a fragment share one per-lane base and differ by constants
  // (64 rows for c1, 8 rows for h).
  int b_tr_base[FN];
  {
    const int i16 = lane & 15;
    const int kr0 = 16 * c0 + (i16 >> 1);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      b_tr_base[j] = kn_offset(kr0, (wn * WTN + j * 16) >> 4) + 8 * (i16 & 1);
  }
  auto read_b_tr = [&](const char* Bs, int j, int row_off) -> v2i {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) v2i*)(Bs + b_tr_base[j] + row_off * BN));
  };
  auto read_b = [&](const char* Bs, int j) -> v8i {
    if constexpr (MODE == kBknDma) {
      const v2i p0 = read_b_tr(Bs, j, 0);
      const v2i p1 = read_b_tr(Bs, j, 8);
      const v2i p2 = read_b_tr(Bs, j, 64);
      const v2i p3 = read_b_tr(Bs, j, 72);
      return v8i{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
    } else {
      const v4i lo = *reinterpret_cast<const v4i*>(Bs + rowk_offset(b_row + j * 16, c0));
      const v4i hi = *reinterpret_cast<const v4i*>(Bs + rowk_offset(b_row + j * 16, c1));
      return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
  };

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
    for (int i = 0; i < FM; ++i) fa[i] = read_a(a_lds(0), i);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[j] = read_b(b_lds(0), j);
  }

  if constexpr (kRegB) {
    // register-staged weight (N not a multiple of 16): one slice per
    // iteration, the next slice's B staged through registers and written in
    // the [n][k] layout
    auto read_b_rowk = [&](const char* Bs, int j) -> v8i {
      const v4i lo = *reinterpret_cast<const v4i*>(Bs + rowk_offset(b_row + j * 16, c0));
      const v4i hi = *reinterpret_cast<const v4i*>(Bs + rowk_offset(b_row + j * 16, c1));
      return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    };
    for (int kt = 0; kt < KT; ++kt) {
      if (kt + 2 < KT) fetch(kt + 2);
      if (kt + 1 < KT) breg.load(b, N, K, n0, (kt + 1) * BK);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma_f8(fa[i], fb[j], acc[i][j]);
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
    // DMA modes, one k slice per iteration in two phases:
    //   phase 0: the first kPhase0 MFMAs (A-fragment-major order) with DMA
    //            parts [0, kSplit) of slice kt + 2 in between (its LDS stage
    //            held slice kt - 1, whose fragments every wave read before
    //            the barrier of iteration kt - 1);
    //   barrier: this wave's DMA of slice kt + 1 has landed (vmcnt), then all
    //            waves' (s_barrier);
    //   phase 1: the other MFMAs with the reads of slice kt + 1's fragments
    //            into the second register set spread between them, and the
    //            remaining DMA parts.
    constexpr int kPhase0 = 8;
    constexpr int kPhase1 = FM * FN - kPhase0;
    constexpr int kReads = FM + FN;
    constexpr int kSplit = kFetchOps / 2;
    static_assert(kFetchOps == 2 * kSplit, "DMA parts split evenly over the two phases");
    static_assert(kPhase0 >= kSplit && kPhase1 >= kFetchOps - kSplit, "one DMA part per MFMA slot");
    for (int kt = 0; kt < KT; ++kt) {
      const bool prefetch = kt + 2 < KT;
      auto mfma = [&](int q) {
        acc[q / FN][q % FN] = mfma_f8(fa[q / FN], fb[q % FN], acc[q / FN][q % FN]);
        __builtin_amdgcn_sched_barrier(0);
      };
      auto dma = [&](int part) {
        if (prefetch) fetch_part(kt + 2, part);
        __builtin_amdgcn_sched_barrier(0);
      };
      // ---- phase 0 ----
#pragma unroll
      for (int q = 0; q < kPhase0; ++q) {
        mfma(q);
        if (q < kSplit) dma(q);
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
        const char* As = a_lds(kt + 1);
        const char* Bs = b_lds(kt + 1);
        v8i na[FM], nb[FN];
#pragma unroll
        for (int q = 0; q < kPhase1; ++q) {
          mfma(kPhase0 + q);
#pragma unroll
          for (int r = q * kReads / kPhase1; r < (q + 1) * kReads / kPhase1; ++r) {
            if (r < FM)
              na[r] = read_a(As, r);
            else
              nb[r - FM] = read_b(Bs, r - FM);
          }
          __builtin_amdgcn_sched_barrier(0);
          if (q < kFetchOps - kSplit) dma(kSplit + q);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[i] = na[i];
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[j] = nb[j];
      }
    }
  }

  // ---- epilogue ----
  // Each wave holds the final sums of its 64 x 64 sub-tile; it stages them
  // row-major in LDS (the operand slices are free after the barrier) and
  // stores whole 128-byte row segments with nontemporal stores.
  constexpr int kStageBytes = WTM * WTN * 4;
  static_assert(WTN == kStageCols, "staging rows are one wave tile wide");
  static_assert(kWaves * kStageBytes + 4 * (BM + BN) <= kStages * STAGE, "staging fits in LDS");
  __syncthreads();  // every wave is done with the k slices
  float* s_sa = reinterpret_cast<float*>(smem + kWaves * kStageBytes);
  float* s_sb = s_sa + BM;
  if (out && t < BM + BN) s_sa[t] = t < BM ? scale_reg : scale_reg * output_scale;  // s_sb follows s_sa
  int* stage = reinterpret_cast<int*>(smem + wave * kStageBytes);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const v4i bits = {__float_as_int(acc[i][j][0]), __float_as_int(acc[i][j][1]),
                        __float_as_int(acc[i][j][2]), __float_as_int(acc[i][j][3])};
      stage_fragment(stage, lane, i, j, bits);
    }
  __syncthreads();  // scales visible (each wave reads back only its own staging)

  const int lrow0 = wm * WTM;
  const int lcol0 = wn * WTN;
  if (c) store4<WTM, true, true>(stage, lane, m0, n0, lrow0, lcol0, M, N, s_sa, s_sb, c);
  if (out) {
    if (out_dtype == QK_BF16)
      store_bf16<WTM, true>(stage, lane, m0, n0, lrow0, lcol0, M, N, s_sa, s_sb, out);
    else
      store4<WTM, true, false>(stage, lane, m0, n0, lrow0, lcol0, M, N, s_sa, s_sb, out);
  }
}

template <int MODE>
hipError_t launch_mode(const GemmFp8Args& g, dim3 grid, int tiles_m, int tiles_n,
                       hipStream_t stream) {
  if (g.k % BK != 0)
    return launch(gemm_fp8_mfma_kernel<MODE, true>, grid, dim3(kThreads), 0, stream, g.a, g.b,
                  g.c, g.scale_a, g.scale_b, g.output_scale, g.out, g.out_dtype, g.m, g.n, g.k,
                  tiles_m, tiles_n);
  return launch(gemm_fp8_mfma_kernel<MODE, false>, grid, dim3(kThreads), 0, stream, g.a, g.b,
                g.c, g.scale_a, g.scale_b, g.output_scale, g.out, g.out_dtype, g.m, g.n, g.k,
                tiles_m, tiles_n);
}

}  // namespace

hipError_t launch_gemm_fp8(const GemmFp8Args& g, hipStream_t stream) {
  const int tiles_m = (g.m + BM - 1) / BM;
  const int tiles_n = (g.n + BN - 1) / BN;
  const long long tiles = static_cast<long long>(tiles_m) * tiles_n;
  if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(tiles));
  if (g.b_layout == QK_B_NK) return launch_mode<kBnkDma>(g, grid, tiles_m, tiles_n, stream);
  if (g.n % 16 == 0) return launch_mode<kBknDma>(g, grid, tiles_m, tiles_n, stream);
  if (g.n % 4 == 0) return launch_mode<kBknReg4>(g, grid, tiles_m, tiles_n, stream);
  return launch_mode<kBknReg1>(g, grid, tiles_m, tiles_n, stream);
}

}  // namespace qk
