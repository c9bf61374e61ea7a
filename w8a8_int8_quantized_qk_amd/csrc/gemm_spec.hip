// INT8 x INT8 -> INT32 GEMM on 256 x 128 tiles with transfer waves and
// matrix-core waves kept apart, dequant epilogue fused.
//
// What it computes is the tiled INT8 kernel's ("16. Deploying Custom
// Kernels", C++ Kernel Interface; "KV-cache kernels", 02 Scales and
// dequantization; INT32 accumulation from "Skill: Write an INT8 Quantized
// Kernel", Inputs):
//   acc[i][j] = sum_t a[i][t] * B(t, j)        exact INT32
//   c[i][j]   = acc                            (optional)
//   out[i][j] = ((float)acc * scale_a[i]) * (scale_b[j] * output_scale)   (optional)
//
// Design for gfx950 (measured on the 256 x 128 k-group kernel: with the same
// LDS reads and MFMAs, leaving out the in-loop global-to-LDS instructions
// made its loop 31% faster, leaving out only the waits for them 6%; a wave
// held up issuing a transfer cannot issue its MFMAs either):
//   * Workgroup tile 256 (M) x 128 (N), k slices of 128 bytes, three LDS
//     stages (the 256 x 128 kernel's row layouts, swizzles and fragment
//     reads, gemm_tile.h) in a split ring: the three A blocks first, then
//     the three weight blocks.
//   * Twelve waves, three per SIMD: waves 0..7 multiply (two per SIMD: one
//     wave issues a 16x16x64 MFMA only every ~25 cycles, measured, so a
//     single wave cannot keep a matrix core busy), waves 8..11 only move
//     data.  Transfer wave d issues 12 of a slice's 48 1-KiB
//     global_load_lds_dwordx4 (A rows 64 d .. 64 d + 63 and a quarter of the
//     weight block) from a scalar base plus fixed per-lane offsets, waits for
//     them and meets the others at the slice barrier.  Matrix-core wave w
//     owns a 64 x 64 sub-tile over the whole k range (three waves per SIMD
//     leave ~168 registers each): per slice two 64-deep steps of 4 x 4
//     v_mfma_i32_16x16x64_i8, reading the next step's 8 fragments while it
//     multiplies the current one.  No partial sums cross waves, so there is
//     no k-group hand-over.
//   * No vector-ALU work in the k loop: on this chip such instructions do
//     not overlap a wave's MFMAs but add to the SIMD's time (a probe: 4
//     conversions or FMAs per 16x16x64 MFMA, from the same or another wave,
//     raise its cycle count from 16.5 to 25-27).  The loop is unrolled over
//     the three stages so that every fragment read is a base register plus an
//     immediate offset, and the transfer waves advance their sources in
//     scalar registers.
//   * One barrier per slice, between its two steps: before it the transfer
//     waves have seen slice kt + 1 land; after it they issue slice kt + 2
//     into the stage of slice kt - 1, whose last fragments the matrix-core
//     waves read before that barrier (a fenced barrier: their LDS reads are
//     complete when they arrive).
//   * Rows past M or N re-read a valid row (never stored).  K must be a
//     multiple of 128 (the 256 x 128 k-group kernel takes the others).
//   * Epilogue: each matrix-core wave stages its 64 x 64 block row-major in
//     LDS and stores it as whole 128-byte row segments, scales in binary32.
#include "gemm_tile.h"

namespace qk {
namespace {

namespace spec {

using namespace tile;

constexpr int kMma = 8;                       // matrix-core waves 0..7, two per SIMD
constexpr int kXfer = 4;                      // transfer waves 8..11, one per SIMD
constexpr int kSpecThreads = 64 * (kMma + kXfer);
constexpr int WTM = 64;                       // matrix-core wave sub-tile rows
constexpr int WTN = 64;                       // ... columns
constexpr int FM = WTM / 16;
constexpr int FN = WTN / 16;
static_assert((BM / WTM) * (BN / WTN) == kMma, "one sub-tile per matrix-core wave");
static_assert(kXfer == kXferWaves, "the transfer waves of gemm_tile.h");

// ASYM: the activations carry per-row zero points zp_a, and the epilogue
// subtracts zp_a[row] * wsum[col] (wsum: the weight's column sums) from the
// INT32 accumulators before storing or scaling them ("KV-cache kernels", 02
// Scales and dequantization: asymmetric codes with a zero point).
template <int MODE, bool ASYM>
__device__ __forceinline__ void gemm_spec_tile(
    const int8_t* __restrict__ a, const int8_t* __restrict__ b, int32_t* __restrict__ c,
    const float* __restrict__ scale_a, const float* __restrict__ scale_b, float output_scale,
    void* __restrict__ out, int out_dtype, int M, int N, int K, int tm, int tn,
    const int32_t* __restrict__ zp_a, const int32_t* __restrict__ wsum) {
  static_assert(MODE == kBnkDma || MODE == kBknDma, "DMA weight layouts");
  constexpr int kStageBytes = WTM * WTN * 4;  // one matrix-core wave's staged block (16 KiB)
  static_assert(kMma * kStageBytes <= kStages * STAGE, "epilogue staging fits in the ring");
  __shared__ __attribute__((aligned(1024))) char smem[kStages * STAGE];
  // per-token scales, then per-channel ones times output_scale; written
  // before the k loop so that no register holds them across it
  __shared__ float s_scale[BM + BN];
  // row zero points, then column sums (ASYM)
  __shared__ int s_corr[ASYM ? BM + BN : 1];

  const int m0 = tm * BM;
  const int n0 = tn * BN;
  const int t = threadIdx.x;
  const int lane = t & 63;
  // wave-uniform for the compiler too, so the two kinds branch, not mask
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);

  if (out && t < BM + BN) {
    float v = 0.0f;
    if (t < BM) {
      if (m0 + t < M) v = scale_a[m0 + t];
    } else if (n0 + t - BM < N) {
      v = scale_b[n0 + t - BM] * output_scale;
    }
    s_scale[t] = v;  // read after the barriers below
  }
  if constexpr (ASYM) {
    if (t < BM + BN) {
      int z = 0;
      if (t < BM) {
        if (m0 + t < M) z = zp_a[m0 + t];
      } else if (n0 + t - BM < N) {
        z = wsum[n0 + t - BM];
      }
      s_corr[t] = z;
    }
  }

  const int KT = K / BK;  // K % BK == 0

  v4i acc[FM][FN];
  const int wm = wave >> 1;  // matrix-core wave's 64 x 64 sub-tile
  const int wn = wave & 1;

  if (wave >= kMma) {
    // ---------------- transfer wave ----------------
    XferParts<MODE> parts;
    parts.init(a, b, M, N, K, m0, n0, wave - kMma);
    parts.run(lds_addr(smem), KT);
  } else {
    // ---------------- matrix-core wave ----------------
    // Every fragment read is a per-lane base plus a constant: the loop below
    // is unrolled over the three stages of the split ring (A stages at
    // s * A_STAGE, weight stages after them at kStages * A_STAGE + s *
    // B_STAGE), and a DS instruction's immediate offset reaches 65535 bytes:
    // one set of A bases serves stages 0 and 1, a second stage 2, and one set
    // of weight bases all three.  No address arithmetic is left in the loop,
    // whose vector-ALU issue cycles the MFMAs share.
    static_assert(kStages == 3, "three stages");
    static_assert(A_STAGE + 2048 * (FM - 1) < 65536, "A: stage 1 from the stage-0 bases");
    static_assert(2 * B_STAGE + BN * (64 + 8) < 65536 && 2 * B_STAGE + 2048 * (FN - 1) < 65536,
                  "weight: every stage from one base");
    const int c = lane >> 4;     // the lane's 16-byte chunk of a 64-deep step
    const int i16 = lane & 15;
    // LDS byte addresses; the empty asm makes each base opaque, so that the
    // compiler keeps it in its own register instead of deriving one base
    // from another with offsets beyond the immediate's reach
    auto opaque = [](uint32_t x) {
      asm("" : "+v"(x));
      return x;
    };
    const uint32_t lds0 = lds_addr(smem);
    const uint32_t b_ring = lds0 + kStages * A_STAGE;
    uint32_t a_base[2][2];    // [set][step g]: A fragment 0; fragment i at + 2048 i
    uint32_t b_base[FN];      // [j] ([K][N] weight): column block j, k row 16 c + i16 / 2
    uint32_t bk_base[2];      // [g] ([N][K] weight): fragment 0; fragment j at + 2048 j
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const uint32_t a_off = rowk_offset(wm * WTM + i16, 4 * g + c);
      a_base[0][g] = opaque(lds0 + a_off);
      a_base[1][g] = opaque(lds0 + 2 * A_STAGE + a_off);
      if constexpr (MODE == kBnkDma) bk_base[g] = opaque(b_ring + rowk_offset(wn * WTN + i16, 4 * g + c));
    }
    // kn_swz of k rows 64 g + 16 c + i16 / 2 + 8 h is that of 16 c + i16 / 2
    // for every g and h, so they differ from it by (64 g + 8 h) rows
    if constexpr (MODE == kBknDma) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
        b_base[j] = opaque(b_ring + kn_offset(16 * c + (i16 >> 1), (wn * WTN + j * 16) >> 4) +
                           8 * (i16 & 1));
    }
    typedef __attribute__((address_space(3))) const v4i* lds_v4i;
    // fragments of 64-deep step g of a slice in stage S: lane l holds k = 64 g
    // + 16 (l / 16) .. + 15 of row (A) or column (B) l % 16 of the fragment
    auto read_a = [&](auto S_, int i, int g) -> v4i {
      constexpr int S = decltype(S_)::value;
      return *reinterpret_cast<lds_v4i>(a_base[S / 2][g] + (S == 1 ? A_STAGE : 0) + 2048 * i);
    };
    auto read_b_tr = [&](auto S_, int j, int h, int g) -> v2i {
      constexpr int S = decltype(S_)::value;
      return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) v2i*)(b_base[j] + S * B_STAGE + BN * (64 * g + 8 * h)));
    };
    auto read_b_rowk = [&](auto S_, int j, int g) -> v4i {
      constexpr int S = decltype(S_)::value;
      return *reinterpret_cast<lds_v4i>(bk_base[g] + S * B_STAGE + 2048 * j);
    };
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = v4i{};

    v4i f0a[FM], f0b[FN], f1a[FM], f1b[FN];
    // 16 MFMAs of (xa, xb); after each of the first 12 one read of (ya, yb)
    // from step g of stage S: the A fragments, then the weight's
    auto mfma_step = [&](auto S_, auto G_, v4i (&xa)[FM], v4i (&xb)[FN], v4i (&ya)[FM],
                         v4i (&yb)[FN]) {
      constexpr int g = decltype(G_)::value;
      v2i lo[FN], hi[FN];
#pragma unroll
      for (int n = 0; n < FM * FN; ++n) {
        const int i = n / FN;
        const int j = n % FN;
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa[i], xb[j], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (n < FM) {
          ya[n] = read_a(S_, n, g);
        } else if (n < FM + 2 * FN) {
          const int r = n - FM;
          if constexpr (MODE == kBknDma) {
            if (r & 1) hi[r >> 1] = read_b_tr(S_, r >> 1, 1, g);
            else lo[r >> 1] = read_b_tr(S_, r >> 1, 0, g);
          } else if ((r & 1) == 0) {
            yb[r >> 1] = read_b_rowk(S_, r >> 1, g);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (MODE == kBknDma) {
#pragma unroll
        for (int j = 0; j < FN; ++j) yb[j] = v4i{lo[j].x, lo[j].y, hi[j].x, hi[j].y};
      }
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;

    __syncthreads();  // slice 0 in LDS
    if (KT > 0) {
#pragma unroll
      for (int i = 0; i < FM; ++i) f0a[i] = read_a(S0{}, i, 0);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (MODE == kBknDma) {
          const v2i lo = read_b_tr(S0{}, j, 0, 0);
          const v2i hi = read_b_tr(S0{}, j, 1, 0);
          f0b[j] = v4i{lo.x, lo.y, hi.x, hi.y};
        } else {
          f0b[j] = read_b_rowk(S0{}, j, 0);
        }
      }
    }
    // slice kt, which sits in stage S = kt % 3
    auto slice = [&](auto S_, int kt) {
      constexpr int S = decltype(S_)::value;
      // step 0 of slice kt, reading its step 1
      mfma_step(S_, S1{}, f0a, f0b, f1a, f1b);
      // slice kt + 1 landed; this wave's reads of slice kt are complete
      if (kt + 1 < KT) __syncthreads();
      // step 1 of slice kt, reading step 0 of slice kt + 1 (after the last
      // slice: a valid, unused stage; not used)
      mfma_step(std::integral_constant<int, (S + 1) % kStages>{}, S0{}, f1a, f1b, f0a, f0b);
    };
    int kt = 0;
    for (; kt + kStages <= KT; kt += kStages) {
      slice(S0{}, kt);
      slice(S1{}, kt + 1);
      slice(S2{}, kt + 2);
    }
    if (kt < KT) slice(S0{}, kt);
    if (kt + 1 < KT) slice(S1{}, kt + 1);
  }

  // ---- epilogue ----
  __syncthreads();  // every wave is done with the stages
  const float* s_sa = s_scale;
  const float* s_sb = s_scale + BM;
  int* stage = reinterpret_cast<int*>(smem + (wave & 7) * kStageBytes);
  if (wave < kMma) {
    // the lane index again from the exec mask, so that no register keeps it
    // over the k loop
    const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) stage_fragment(stage, lane, i, j, acc[i][j]);
  }
  __syncthreads();  // staged blocks visible
  if (wave < kMma) {
    const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int lrow0 = wm * WTM;
    const int lcol0 = wn * WTN;
    const int* s_zp = s_corr;
    const int* s_ws = s_corr + BM;
    if (c)
      store4<64, false, true, ASYM>(stage, lane, m0, n0, lrow0, lcol0, M, N, s_sa, s_sb, c, s_zp,
                                    s_ws);
    if (out) {
      if (out_dtype == QK_BF16)
        store_bf16<64, false, ASYM>(stage, lane, m0, n0, lrow0, lcol0, M, N, s_sa, s_sb, out, s_zp,
                                    s_ws);
      else
        store4<64, false, false, ASYM>(stage, lane, m0, n0, lrow0, lcol0, M, N, s_sa, s_sb, out,
                                       s_zp, s_ws);
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(kSpecThreads, 1) void gemm_i8_spec_kernel(
    const int8_t* __restrict__ a, const int8_t* __restrict__ b, int32_t* __restrict__ c,
    const float* __restrict__ scale_a, const float* __restrict__ scale_b, float output_scale,
    void* __restrict__ out, int out_dtype, int M, int N, int K, int tiles_m, int tiles_n) {
  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  gemm_spec_tile<MODE, false>(a, b, c, scale_a, scale_b, output_scale, out, out_dtype, M, N, K,
                              tm, tn, nullptr, nullptr);
}

// Asymmetric activations: the result is sum_t (a[i][t] - zp_a[i]) * B(t, j)
// = acc - zp_a[i] * wsum[j].
template <int MODE>
__global__ __launch_bounds__(kSpecThreads, 1) void gemm_i8_spec_asym_kernel(
    const int8_t* __restrict__ a, const int8_t* __restrict__ b, int32_t* __restrict__ c,
    const float* __restrict__ scale_a, const float* __restrict__ scale_b, float output_scale,
    void* __restrict__ out, int out_dtype, int M, int N, int K, int tiles_m, int tiles_n,
    const int32_t* __restrict__ zp_a, const int32_t* __restrict__ wsum) {
  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  gemm_spec_tile<MODE, true>(a, b, c, scale_a, scale_b, output_scale, out, out_dtype, M, N, K, tm,
                             tn, zp_a, wsum);
}

}  // namespace spec
}  // namespace

bool gemm_spec_applies(int m, int n, int k, int b_layout) {
  if (k <= 0 || k % tile::BK != 0 || n < 16 || !tile::xfer_parts_fit(n, k)) return false;
  if (b_layout == QK_B_KN && n % 16 != 0) return false;  // DMA of [k][n] rows in 16-byte chunks
  return true;
}

hipError_t launch_gemm_spec_asym(const GemmArgs& g, const int32_t* zp_a, const int32_t* wsum,
                                 hipStream_t stream) {
  const int tiles_m = (g.m + tile::BM - 1) / tile::BM;
  const int tiles_n = (g.n + tile::BN - 1) / tile::BN;
  const long long tiles = static_cast<long long>(tiles_m) * tiles_n;
  if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(tiles));
  if (g.b_layout == QK_B_NK)
    return launch(spec::gemm_i8_spec_asym_kernel<tile::kBnkDma>, grid, dim3(spec::kSpecThreads), 0,
                  stream, g.a, g.b, g.c, g.scale_a, g.scale_b, g.output_scale, g.out, g.out_dtype,
                  g.m, g.n, g.k, tiles_m, tiles_n, zp_a, wsum);
  return launch(spec::gemm_i8_spec_asym_kernel<tile::kBknDma>, grid, dim3(spec::kSpecThreads), 0,
                stream, g.a, g.b, g.c, g.scale_a, g.scale_b, g.output_scale, g.out, g.out_dtype,
                g.m, g.n, g.k, tiles_m, tiles_n, zp_a, wsum);
}

hipError_t launch_gemm_spec(const GemmArgs& g, hipStream_t stream) {
  const int tiles_m = (g.m + tile::BM - 1) / tile::BM;
  const int tiles_n = (g.n + tile::BN - 1) / tile::BN;
  const long long tiles = static_cast<long long>(tiles_m) * tiles_n;
  if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(tiles));
  if (g.b_layout == QK_B_NK)
    return launch(spec::gemm_i8_spec_kernel<tile::kBnkDma>, grid, dim3(spec::kSpecThreads), 0, stream,
                  g.a, g.b, g.c, g.scale_a, g.scale_b, g.output_scale, g.out, g.out_dtype, g.m,
                  g.n, g.k, tiles_m, tiles_n);
  return launch(spec::gemm_i8_spec_kernel<tile::kBknDma>, grid, dim3(spec::kSpecThreads), 0, stream,
                g.a, g.b, g.c, g.scale_a, g.scale_b, g.output_scale, g.out, g.out_dtype, g.m, g.n,
                g.k, tiles_m, tiles_n);
}

}  // namespace qk
