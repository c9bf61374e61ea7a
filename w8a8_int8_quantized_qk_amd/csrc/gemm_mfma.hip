// INT8 x INT8 -> INT32 GEMM on CDNA4 matrix cores with the dequant epilogue fused.
//
// What it computes ("16. Deploying Custom Kernels", C++ Kernel Interface;
// "KV-cache kernels", 02 Scales and dequantization; INT32 accumulation from
// "Skill: Write an INT8 Quantized Kernel", Inputs):
//   acc[i][j] = sum_t a[i][t] * B(t, j)        exact INT32
//   c[i][j]   = acc                            (optional)
//   out[i][j] = ((float)acc * scale_a[i]) * scale_b[j] * output_scale   (optional)
//
// Design for gfx950:
//   * Workgroup tile 256 (M) x 128 (N), reduction step 128 bytes of K.  Four
//     wave64s in a 2 x 2 grid each own a 128 x 64 sub-tile computed with
//     v_mfma_i32_32x32x32_i8 (4 x 2 instructions per 32-deep k slice, 128
//     INT32 accumulators per lane).  One tile per CU covers M=2048, N=4096 in
//     a single wave of 256 workgroups.
//   * Both operands are staged through LDS, double buffered (2 x 48 KiB):
//     the next k slice is fetched into registers with 128-bit (A) loads while
//     the matrix cores work on the current one.
//   * LDS rows are 128 bytes; the 16-byte chunk index is XORed with a function
//     of the row so that the eight lanes served together by a 128-bit LDS
//     access touch eight different chunks, both when a row is written and
//     when eight consecutive rows are read as MFMA operands.
//   * MFMA wants 16 consecutive k values per lane for both operands.  A is
//     [M][K] (k contiguous) and is copied as is.  A weight stored [K][N]
//     (n contiguous) is loaded as 4-column x 16-row byte blocks and transposed
//     in registers with v_perm_b32 before it is written to LDS as [N][K];
//     a weight stored [N][K] is copied like A.
//   * Rows past M or N re-read the last valid row (results discarded); k past
//     K loads zeros, so partial k slices add nothing.
//   * The epilogue converts each accumulator to binary32 in registers,
//     multiplies by the per-token and per-channel scales, and stores fp32 or
//     bf16 (round to nearest even); raw accumulators are stored when asked.
#include "qk_internal.h"

namespace qk {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int BM = 256;
constexpr int BN = 128;
constexpr int BK = 128;
constexpr int WTM = 128;       // wave tile rows
constexpr int WTN = 64;        // wave tile columns
constexpr int FM = WTM / 32;   // 32x32 fragments per wave along M
constexpr int FN = WTN / 32;   // ... along N
constexpr int A_STAGE = BM * BK;
constexpr int B_STAGE = BN * BK;
constexpr int A_CHUNKS = BM * BK / 16 / kThreads;  // 16-byte chunks per thread: 8
constexpr int BNK_CHUNKS = BN * BK / 16 / kThreads;  // 4

__device__ __forceinline__ int lds_offset(int row, int chunk) {
  const int swz = (row & 7) ^ ((row >> 2) & 7);
  return row * BK + ((chunk ^ swz) << 4);
}

// ---- A (and a [N][K] weight): 16-byte chunks, 8 consecutive lanes per row ----
template <int ROWS>
struct RowTile {
  static constexpr int kChunks = ROWS * BK / 16 / kThreads;
  uint4 v[kChunks];

  __device__ void load(const int8_t* __restrict__ p, int rows_valid, int K, int r0, int k0) {
    const int t = threadIdx.x;
    const int gk = k0 + (t & 7) * 16;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int row = (t >> 3) + 32 * i;
      const int gr = min(r0 + row, rows_valid - 1);
      if (gk < K)
        v[i] = *reinterpret_cast<const uint4*>(p + static_cast<size_t>(gr) * K + gk);
      else
        v[i] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ void store(char* lds) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int row = (t >> 3) + 32 * i;
      *reinterpret_cast<uint4*>(lds + lds_offset(row, t & 7)) = v[i];
    }
  }
};

// ---- a [K][N] weight: each thread loads 16 k-rows x 4 columns ----
__device__ __forceinline__ void transpose4x4(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                             uint32_t& c0, uint32_t& c1, uint32_t& c2,
                                             uint32_t& c3) {
  // input: a..d are rows k0..k3, byte j = column j; output cj = column j, byte i = row ki
  const uint32_t t0 = __builtin_amdgcn_perm(b, a, 0x05010400u);  // a0 b0 a1 b1
  const uint32_t t1 = __builtin_amdgcn_perm(b, a, 0x07030602u);  // a2 b2 a3 b3
  const uint32_t t2 = __builtin_amdgcn_perm(d, c, 0x05010400u);  // c0 d0 c1 d1
  const uint32_t t3 = __builtin_amdgcn_perm(d, c, 0x07030602u);  // c2 d2 c3 d3
  c0 = __builtin_amdgcn_perm(t2, t0, 0x05040100u);               // a0 b0 c0 d0
  c1 = __builtin_amdgcn_perm(t2, t0, 0x07060302u);               // a1 b1 c1 d1
  c2 = __builtin_amdgcn_perm(t3, t1, 0x05040100u);               // a2 b2 c2 d2
  c3 = __builtin_amdgcn_perm(t3, t1, 0x07060302u);               // a3 b3 c3 d3
}

template <bool N4>
struct KnTile {
  uint32_t v[16];  // v[r] = columns 4cg..4cg+3 of k row 16rg + r

  __device__ void load(const int8_t* __restrict__ b, int N, int K, int n0, int k0) {
    const int t = threadIdx.x;
    const int gn = n0 + 4 * (t & 31);
    const int kb = k0 + 16 * (t >> 5);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int gk = kb + r;
      const int8_t* row = b + static_cast<size_t>(gk) * N;
      if constexpr (N4) {
        v[r] = (gk < K && gn < N) ? *reinterpret_cast<const uint32_t*>(row + gn) : 0u;
      } else {
        uint32_t w = 0;
        if (gk < K) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (gn + j < N) w |= (static_cast<uint32_t>(static_cast<uint8_t>(row[gn + j]))) << (8 * j);
        }
        v[r] = w;
      }
    }
  }
  __device__ void store(char* lds) const {
    const int t = threadIdx.x;
    const int cg = t & 31;
    const int rg = t >> 5;
    uint32_t col[4][4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
      transpose4x4(v[4 * d], v[4 * d + 1], v[4 * d + 2], v[4 * d + 3], col[0][d], col[1][d],
                   col[2][d], col[3][d]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<uint4*>(lds + lds_offset(4 * cg + j, rg)) =
          make_uint4(col[j][0], col[j][1], col[j][2], col[j][3]);
  }
};

__device__ __forceinline__ uint16_t to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

template <bool B_NK, bool N4>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_mfma_kernel(
    const int8_t* __restrict__ a, const int8_t* __restrict__ b, int32_t* __restrict__ c,
    const float* __restrict__ scale_a, const float* __restrict__ scale_b, float output_scale,
    void* __restrict__ out, int out_dtype, int M, int N, int K, int tiles_m) {
  __shared__ __attribute__((aligned(16))) char smem[2 * (A_STAGE + B_STAGE)];
  char* const As0 = smem;
  char* const Bs0 = smem + 2 * A_STAGE;

  const int tile = blockIdx.x;
  const int m0 = (tile % tiles_m) * BM;
  const int n0 = (tile / tiles_m) * BN;
  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int lane = t & 63;
  const int wm = wave >> 1;
  const int wn = wave & 1;

  RowTile<BM> at;
  using BTile = std::conditional_t<B_NK, RowTile<BN>, KnTile<N4>>;
  BTile bt;
  auto load_b = [&](int k0) {
    if constexpr (B_NK)
      bt.load(b, N, K, n0, k0);
    else
      bt.load(b, N, K, n0, k0);
  };

  v16i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16i{};

  const int KT = (K + BK - 1) / BK;
  if (KT > 0) {
    at.load(a, M, K, m0, 0);
    load_b(0);
    at.store(As0);
    bt.store(Bs0);
  }
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const char* As = As0 + (kt & 1) * A_STAGE;
    const char* Bs = Bs0 + (kt & 1) * B_STAGE;
    const bool more = kt + 1 < KT;
    if (more) {
      at.load(a, M, K, m0, (kt + 1) * BK);
      load_b((kt + 1) * BK);
    }
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      const int chunk = 2 * kk + (lane >> 5);
      v4i af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const v4i*>(As + lds_offset(wm * WTM + i * 32 + (lane & 31), chunk));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bf[j] = *reinterpret_cast<const v4i*>(Bs + lds_offset(wn * WTN + j * 32 + (lane & 31), chunk));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      at.store(As0 + ((kt + 1) & 1) * A_STAGE);
      bt.store(Bs0 + ((kt + 1) & 1) * B_STAGE);
    }
    __syncthreads();
  }

  // epilogue: lane owns column (lane & 31) of each fragment and rows
  // 8 * (r / 4) + 4 * (lane / 32) + r % 4 for accumulator register r
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int col = n0 + wn * WTN + j * 32 + (lane & 31);
    if (col >= N) continue;
    const float sb = out ? scale_b[col] * output_scale : 0.0f;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= M) continue;
        const int v = acc[i][j][r];
        const size_t idx = static_cast<size_t>(row) * N + col;
        if (c) c[idx] = v;
        if (out) {
          const float f = (static_cast<float>(v) * scale_a[row]) * sb;
          if (out_dtype == QK_BF16)
            static_cast<uint16_t*>(out)[idx] = to_bf16(f);
          else
            static_cast<float*>(out)[idx] = f;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_mfma(const GemmArgs& g, hipStream_t stream) {
  const int tiles_m = (g.m + BM - 1) / BM;
  const int tiles_n = (g.n + BN - 1) / BN;
  const long long tiles = static_cast<long long>(tiles_m) * tiles_n;
  if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(tiles));
  const dim3 block(kThreads);
  if (g.b_layout == QK_B_NK)
    return launch(gemm_i8_mfma_kernel<true, true>, grid, block, 0, stream, g.a, g.b, g.c,
                  g.scale_a, g.scale_b, g.output_scale, g.out, g.out_dtype, g.m, g.n, g.k, tiles_m);
  if (g.n % 4 == 0)
    return launch(gemm_i8_mfma_kernel<false, true>, grid, block, 0, stream, g.a, g.b, g.c,
                  g.scale_a, g.scale_b, g.output_scale, g.out, g.out_dtype, g.m, g.n, g.k, tiles_m);
  return launch(gemm_i8_mfma_kernel<false, false>, grid, block, 0, stream, g.a, g.b, g.c,
                g.scale_a, g.scale_b, g.output_scale, g.out, g.out_dtype, g.m, g.n, g.k, tiles_m);
}

}  // namespace qk
