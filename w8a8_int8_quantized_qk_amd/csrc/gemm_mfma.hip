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
//     v_mfma_i32_32x32x32_i8 (4 x 2 instructions per 32-deep k step, 128
//     INT32 accumulators per lane), group g multiplying k steps 2g and 2g + 1
//     of every slice.  M=2048, N=4096 is 256 tiles: one per CU.
//   * Operands go from global memory straight into LDS with 128-bit
//     global_load_lds (no register staging): lane l of a wave writes LDS
//     bytes [16 l, 16 l + 16) above the wave's base address, so each lane
//     fetches the global chunk that belongs at its LDS slot.  Three LDS
//     slices (3 x 48 KiB) let slice s + 2 stream in while slice s is
//     multiplied; one barrier per slice.
//   * A (and a weight stored [N][K]) is kept k-contiguous, 128-byte rows with
//     the 16-byte chunk index XORed by (row & 7) ^ ((row >> 2) & 7): the eight
//     lanes served together by a 128-bit LDS read see eight distinct chunks.
//   * A weight stored [K][N] (n contiguous) stays [k][n] in LDS (chunk index
//     XORed by k & 7) and is read with ds_read_b64_tr_b8: a 16-lane group
//     reads an 8 (k) x 16 (n) byte block and lane j receives column j's eight
//     k values, which is the k-contiguous MFMA operand; two such reads give
//     the 16 bytes of a lane.  No VALU transposes are needed.
//   * For a [K][N] weight whose N is not a multiple of 16, B falls back to
//     register staging (dword or byte loads, 4 x 4 byte transposes with
//     v_perm_b32, LDS writes in the [n][k] layout).
//   * Rows past M or N re-read a valid row (those outputs are never stored).
//     When K is not a multiple of 128 the final slice's A chunks at k >= K are
//     zeroed in LDS before use, so they add nothing.
//   * Workgroups are dispatched to the 8 XCDs round robin; tiles are renumbered
//     so the ones running together on one XCD form a compact 4 x 8 block that
//     shares A rows and B columns in that XCD's L2.
//   * Epilogue without a row-major staging pass: the two wave groups swap
//     half of their partial sums through LDS as 16-byte chunks, then each
//     lane transposes 4 x 4 blocks across its lane quad (DPP) so that it holds
//     4 consecutive columns of one row, applies the per-token and per-channel
//     scales in binary32 and stores fp32 or bf16 (round to nearest even), or
//     the raw accumulators, with nontemporal stores.
//   * Operands are addressed with 32-bit offsets (m*k, n*k < 2^32).
#include "lds_dma.h"
#include "qk_internal.h"

#include <type_traits>

namespace qk {
namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;   // 8: two per SIMD
constexpr int kGroups = 2;              // wave groups splitting each k slice
constexpr int BM = 256;
constexpr int BN = 128;
constexpr int BK = 128;
constexpr int WTM = 128;       // wave tile rows
constexpr int WTN = 64;        // wave tile columns
constexpr int FM = WTM / 32;   // 32x32 fragments per wave along M
constexpr int FN = WTN / 32;   // ... along N
constexpr int kSubTiles = (BM / WTM) * (BN / WTN);  // wave sub-tiles per workgroup tile
static_assert(kSubTiles * kGroups == kWaves, "every wave owns one (sub-tile, k group)");
constexpr int kStages = 3;     // LDS k slices in flight
constexpr int A_STAGE = BM * BK;
constexpr int B_STAGE = BN * BK;
constexpr int STAGE = A_STAGE + B_STAGE;

enum BMode {
  kBnkDma = 0,    // weight [N][K], DMA, read like A
  kBknDma = 1,    // weight [K][N], N % 16 == 0: DMA into [k][n], transpose reads
  kBknReg4 = 2,   // weight [K][N], N % 4 == 0: dword loads, register transpose
  kBknReg1 = 3,   // weight [K][N], other N: byte loads, register transpose
};

// k-contiguous tiles (A, [N][K] weight): 128-byte rows
__device__ __forceinline__ int rowk_offset(int row, int chunk) {
  return row * BK + ((chunk ^ ((row & 7) ^ ((row >> 2) & 7))) << 4);
}
// [k][n] weight tile: 128-byte rows of n
__device__ __forceinline__ int kn_offset(int k, int chunk) {
  return k * BN + ((chunk ^ (k & 7)) << 4);
}

// DMA of a k-contiguous tile of ROWS rows x 128 bytes (global rows clamped to
// rows_valid - 1, k offset clamped into the row): instruction i of this
// wave's share (1 KiB = 8 rows each).
template <int ROWS>
constexpr int rowk_ops() { return ROWS * BK / 1024 / kWaves; }
template <int ROWS>
__device__ __forceinline__ void dma_rowk_one(const int8_t* __restrict__ g, char* lds,
                                             int rows_valid, int K, int r0, int k0, int i) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int blk = wave * rowk_ops<ROWS>() + i;
  const int row = blk * 8 + (lane >> 3);
  const int lchunk = (lane & 7) ^ ((row & 7) ^ ((row >> 2) & 7));
  const uint32_t gr = static_cast<uint32_t>(min(r0 + row, rows_valid - 1));
  const uint32_t gk = static_cast<uint32_t>(min(k0 + 16 * lchunk, K - 16));
  lds_dma16(g + (gr * static_cast<uint32_t>(K) + gk), lds_addr(lds + blk * 1024));
}
template <int ROWS>
__device__ __forceinline__ void dma_rowk(const int8_t* __restrict__ g, char* lds, int rows_valid,
                                         int K, int r0, int k0) {
#pragma unroll
  for (int i = 0; i < rowk_ops<ROWS>(); ++i) dma_rowk_one<ROWS>(g, lds, rows_valid, K, r0, k0, i);
}

// DMA of a [K][N] weight tile: 128 k rows x 128 bytes of n; instruction i of
// this wave's share.
constexpr int kn_ops() { return BK * BN / 1024 / kWaves; }
__device__ __forceinline__ void dma_kn_one(const int8_t* __restrict__ b, char* lds, int N, int K,
                                           int n0, int k0, int i) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int blk = wave * kn_ops() + i;
  const int k = blk * 8 + (lane >> 3);
  const int lchunk = (lane & 7) ^ (k & 7);
  const uint32_t gk = static_cast<uint32_t>(min(k0 + k, K - 1));
  const uint32_t gn = static_cast<uint32_t>(min(n0 + 16 * lchunk, N - 16));
  lds_dma16(b + (gk * static_cast<uint32_t>(N) + gn), lds_addr(lds + blk * 1024));
}
__device__ __forceinline__ void dma_kn(const int8_t* __restrict__ b, char* lds, int N, int K,
                                       int n0, int k0) {
#pragma unroll
  for (int i = 0; i < kn_ops(); ++i) dma_kn_one(b, lds, N, K, n0, k0, i);
}

// ---- register-staged [K][N] weight (N not a multiple of 16) ----
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
struct KnRegTile {
  uint32_t v[16];  // v[r] = columns 4cg..4cg+3 of k row 16rg + r; thread = (cg, rg) = (t%32, t/32)

  __device__ __forceinline__ void load(const int8_t* __restrict__ b, int N, int K, int n0, int k0) {
    const int t = threadIdx.x;
    if (t >= 256) return;  // waves 0-3 stage the 128 x 128 tile
    const int gn = n0 + 4 * (t & 31);
    const int kb = k0 + 16 * (t >> 5);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t gk = static_cast<uint32_t>(min(kb + r, K - 1));
      if constexpr (N4) {
        const uint32_t gnc = static_cast<uint32_t>(min(gn, N - 4));
        v[r] = *reinterpret_cast<const uint32_t*>(b + (gk * static_cast<uint32_t>(N) + gnc));
      } else {
        const int8_t* row = b + gk * static_cast<uint32_t>(N);
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          w |= static_cast<uint32_t>(static_cast<uint8_t>(row[min(gn + j, N - 1)])) << (8 * j);
        v[r] = w;
      }
    }
  }
  // written as k-contiguous [n][k] rows (read like A)
  __device__ __forceinline__ void store(char* lds) const {
    const int t = threadIdx.x;
    if (t >= 256) return;
    const int cg = t & 31;
    const int rg = t >> 5;
    uint32_t col[4][4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
      transpose4x4(v[4 * d], v[4 * d + 1], v[4 * d + 2], v[4 * d + 3], col[0][d], col[1][d],
                   col[2][d], col[3][d]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<uint4*>(lds + rowk_offset(4 * cg + j, rg)) =
          make_uint4(col[j][0], col[j][1], col[j][2], col[j][3]);
  }
};

struct NoRegTile {
  __device__ __forceinline__ void load(const int8_t*, int, int, int, int) {}
  __device__ __forceinline__ void store(char*) const {}
};

__device__ __forceinline__ uint16_t to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// 4 x 4 transpose across each quad of lanes: lane i of the quad holds x[k]
// = element (k, i) of a 4 x 4 block; afterwards y[k] = element (i, k).  Two
// butterfly steps (partner lane i ^ 1, then i ^ 2), each exchanging the
// off-diagonal 2 x 2 blocks with DPP quad permutations.
__device__ __forceinline__ void quad_transpose(int x0, int x1, int x2, int x3, int i, int* y) {
  // quad_perm(1, 0, 3, 2) = 0xB1: read lane i ^ 1; quad_perm(2, 3, 0, 1) = 0x4E: read lane i ^ 2
  const bool odd = i & 1;
  const int p0 = __builtin_amdgcn_mov_dpp(x0, 0xB1, 0xF, 0xF, false);
  const int p1 = __builtin_amdgcn_mov_dpp(x1, 0xB1, 0xF, 0xF, false);
  const int p2 = __builtin_amdgcn_mov_dpp(x2, 0xB1, 0xF, 0xF, false);
  const int p3 = __builtin_amdgcn_mov_dpp(x3, 0xB1, 0xF, 0xF, false);
  const int a0 = odd ? p1 : x0;
  const int a1 = odd ? x1 : p0;
  const int a2 = odd ? p3 : x2;
  const int a3 = odd ? x3 : p2;
  const bool hi = i & 2;
  const int r0 = __builtin_amdgcn_mov_dpp(a0, 0x4E, 0xF, 0xF, false);
  const int r1 = __builtin_amdgcn_mov_dpp(a1, 0x4E, 0xF, 0xF, false);
  const int r2 = __builtin_amdgcn_mov_dpp(a2, 0x4E, 0xF, 0xF, false);
  const int r3 = __builtin_amdgcn_mov_dpp(a3, 0x4E, 0xF, 0xF, false);
  y[0] = hi ? r2 : a0;
  y[1] = hi ? r3 : a1;
  y[2] = hi ? a2 : r0;
  y[3] = hi ? a3 : r1;
}

constexpr int kGroupM = 4;

__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  int b = blockIdx.x;
  if (T % 8 == 0) b = (b % 8) * (T / 8) + b / 8;
  const int group_tiles = kGroupM * tiles_n;
  const int g = b / group_tiles;
  const int first_m = g * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int r = b - g * group_tiles;
  tm = first_m + r % gm;
  tn = r / gm;
}

template <int MODE, bool KTAIL>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_mfma_kernel(
    const int8_t* __restrict__ a, const int8_t* __restrict__ b, int32_t* __restrict__ c,
    const float* __restrict__ scale_a, const float* __restrict__ scale_b, float output_scale,
    void* __restrict__ out, int out_dtype, int M, int N, int K, int tiles_m, int tiles_n) {
  constexpr bool kRegB = MODE == kBknReg4 || MODE == kBknReg1;
  __shared__ __attribute__((aligned(1024))) char smem[kStages * STAGE];

  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM;
  const int n0 = tn * BN;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int grp = (t >> 6) / kSubTiles;  // which k steps of a slice this wave multiplies
  const int wsub = (t >> 6) % kSubTiles;  // which 128 x 64 sub-tile it owns
  const int wm = wsub / (BN / WTN);
  const int wn = wsub % (BN / WTN);

  auto a_lds = [&](int s) { return smem + (s % kStages) * STAGE; };
  auto b_lds = [&](int s) { return smem + (s % kStages) * STAGE + A_STAGE; };

  using RegTile = std::conditional_t<MODE == kBknReg4, KnRegTile<true>,
                                     std::conditional_t<MODE == kBknReg1, KnRegTile<false>, NoRegTile>>;
  RegTile breg;

  // issue the global reads of k slice s (DMA: straight into its LDS slice)
  auto fetch = [&](int s) {
    dma_rowk<BM>(a, a_lds(s), M, K, m0, s * BK);
    if constexpr (MODE == kBnkDma) dma_rowk<BN>(b, b_lds(s), N, K, n0, s * BK);
    if constexpr (MODE == kBknDma) dma_kn(b, b_lds(s), N, K, n0, s * BK);
  };
  constexpr int kFetchOps = BM * BK / 1024 / kWaves + (kRegB ? 0 : BN * BK / 1024 / kWaves);
  // one DMA instruction of slice s: parts [0, kOpsA) are A, the rest B.
  // Without a K tail no clamp changes from slice to slice, so each part's
  // source address and LDS slot are formed once: slice s adds s times the
  // part's stride (BK bytes along k) and the stage offset.
  constexpr int kOpsA = rowk_ops<BM>();
  constexpr bool kFixedParts = !KTAIL && !kRegB;
  const int8_t* part_src[kFetchOps];
  uint32_t part_lds[kFetchOps];  // wave-uniform (m0 operand)
  size_t part_stride[kFetchOps];
  const uint32_t lds_smem = lds_addr(smem);
  if constexpr (kFixedParts) {
    const int wave = t >> 6;
#pragma unroll
    for (int q = 0; q < kFetchOps; ++q) {
      if (q < kOpsA) {
        const int blk = wave * kOpsA + q;
        const int row = blk * 8 + (lane >> 3);
        const int lchunk = (lane & 7) ^ ((row & 7) ^ ((row >> 2) & 7));
        const uint32_t gr = static_cast<uint32_t>(min(m0 + row, M - 1));
        part_src[q] = a + (gr * static_cast<uint32_t>(K) + 16 * lchunk);
        part_lds[q] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(blk * 1024));
        part_stride[q] = BK;
      } else if constexpr (MODE == kBnkDma) {
        const int blk = wave * rowk_ops<BN>() + (q - kOpsA);
        const int row = blk * 8 + (lane >> 3);
        const int lchunk = (lane & 7) ^ ((row & 7) ^ ((row >> 2) & 7));
        const uint32_t gr = static_cast<uint32_t>(min(n0 + row, N - 1));
        part_src[q] = b + (gr * static_cast<uint32_t>(K) + 16 * lchunk);
        part_lds[q] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(A_STAGE + blk * 1024));
        part_stride[q] = BK;
      } else {
        const int blk = wave * kn_ops() + (q - kOpsA);
        const int k = blk * 8 + (lane >> 3);
        const int lchunk = (lane & 7) ^ (k & 7);
        const uint32_t gn = static_cast<uint32_t>(min(n0 + 16 * lchunk, N - 16));
        part_src[q] = b + (static_cast<uint32_t>(k) * static_cast<uint32_t>(N) + gn);
        part_lds[q] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(A_STAGE + blk * 1024));
        part_stride[q] = static_cast<size_t>(BK) * N;
      }
    }
  }
  auto fetch_part = [&](int s, int part) {
    if constexpr (kFixedParts) {
      lds_dma16(part_src[part] + static_cast<size_t>(s) * part_stride[part],
                lds_smem + static_cast<uint32_t>((s % kStages) * STAGE) + part_lds[part]);
    } else if (part < kOpsA) {
      dma_rowk_one<BM>(a, a_lds(s), M, K, m0, s * BK, part);
    } else if constexpr (MODE == kBnkDma) {
      dma_rowk_one<BN>(b, b_lds(s), N, K, n0, s * BK, part - kOpsA);
    } else if constexpr (MODE == kBknDma) {
      dma_kn_one(b, b_lds(s), N, K, n0, s * BK, part - kOpsA);
    }
  };

  // fragment reads: A (and [N][K] / register-staged B) with 128-bit reads;
  // a DMA'd [K][N] B with two transpose reads per lane
  const int a_row = wm * WTM + (lane & 31);
  const int b_row = wn * WTN + (lane & 31);
  // single-fragment reads for the interleaved schedule
  auto read_a = [&](const char* As, int kk, int i) -> v4i {
    return *reinterpret_cast<const v4i*>(As + rowk_offset(a_row + i * 32, 2 * kk + (lane >> 5)));
  };
  // B fragment j: a [K][N] weight takes two transpose reads (half 0 and 1)
  auto read_b_tr = [&](const char* Bs, int kk, int j, int h) -> v2i {
    const int g = lane >> 4;
    const int i16 = lane & 15;
    const int kr = 32 * kk + 16 * (g >> 1) + (i16 >> 1) + 8 * h;
    const int cb = (wn * WTN + j * 32 + 16 * (g & 1)) >> 4;
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) v2i*)(Bs + kn_offset(kr, cb) + 8 * (i16 & 1)));
  };
  auto read_b_rowk = [&](const char* Bs, int kk, int j) -> v4i {
    return *reinterpret_cast<const v4i*>(Bs + rowk_offset(b_row + j * 32, 2 * kk + (lane >> 5)));
  };
  auto read_frags = [&](const char* As, const char* Bs, int kk, v4i* fa, v4i* fb) {
    const int chunk = 2 * kk + (lane >> 5);
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[i] = *reinterpret_cast<const v4i*>(As + rowk_offset(a_row + i * 32, chunk));
    if constexpr (MODE == kBknDma) {
      const int g = lane >> 4;        // 16-lane group
      const int i16 = lane & 15;
      const int kr = 32 * kk + 16 * (g >> 1) + (i16 >> 1);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int cb = (wn * WTN + j * 32 + 16 * (g & 1)) >> 4;  // chunk of 16 columns
        const int half = 8 * (i16 & 1);
        const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) v2i*)(Bs + kn_offset(kr, cb) + half));
        const v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) v2i*)(Bs + kn_offset(kr + 8, cb) + half));
        fb[j] = v4i{lo.x, lo.y, hi.x, hi.y};
      }
    } else {
#pragma unroll
      for (int j = 0; j < FN; ++j)
        fb[j] = *reinterpret_cast<const v4i*>(Bs + rowk_offset(b_row + j * 32, chunk));
    }
  };

  v16i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16i{};


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

  constexpr int kSteps = BK / 32 / kGroups;  // MFMA steps per wave per slice
  v4i af[2][FM], bf[2][FN];
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
    read_frags(a_lds(0), b_lds(0), kSteps * grp, af[0], bf[0]);
  }

  // Software pipeline, one k slice per iteration.  A slice has 4 MFMA steps
  // of 32 k; wave group g multiplies steps 2g and 2g + 1 (both groups cover
  // the same output sub-tiles, their sums are added at the end).  Per slice:
  //   top:      issue the DMA of slice kt + 2 (its LDS slice was last read in
  //             iteration kt - 1, before that iteration's barrier);
  //   step 1st: 8 MFMAs on the fragments in registers, interleaved with the
  //             LDS reads of the second step's fragments;
  //   step 2nd: wait for this wave's DMA of slice kt + 1, barrier (all DMA
  //             landed, all reads of slice kt done), then 8 MFMAs interleaved
  //             with the reads of slice kt + 1's first step.
  if constexpr (kRegB) {
    for (int kt = 0; kt < KT; ++kt) {
      if (kt + 2 < KT) fetch(kt + 2);
      if constexpr (kRegB) {
        if (kt + 1 < KT) breg.load(b, N, K, n0, (kt + 1) * BK);
      }
      const char* As = a_lds(kt);
      const char* Bs = b_lds(kt);
  #pragma unroll
      for (int st = 0; st < kSteps; ++st) {
        const int cur = st & 1;
        const int nxt = cur ^ 1;
        if (st + 1 < kSteps) {
          read_frags(As, Bs, kSteps * grp + st + 1, af[nxt], bf[nxt]);
        } else if (kt + 1 < KT) {
          if constexpr (kRegB) {
            wait_vmcnt<0>();
            breg.store(b_lds(kt + 1));
          } else {
            if (kt + 2 < KT) wait_vmcnt<kFetchOps>(); else wait_vmcnt<0>();
          }
          __syncthreads();
          if (KTAIL && kt + 1 == KT - 1) zero_tail(kt + 1);
          read_frags(a_lds(kt + 1), b_lds(kt + 1), kSteps * grp, af[nxt], bf[nxt]);
        }
  #pragma unroll
        for (int i = 0; i < FM; ++i)
  #pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[cur][i], bf[cur][j], acc[i][j], 0,
                                                              0, 0);
        // issue order: two LDS reads, one MFMA, ... then the remaining MFMAs
  #pragma unroll
        for (int x = 0; x < 4; ++x) {
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      }
    }
  } else {
    // DMA modes: the slice's DMA instructions are spread through the MFMA
    // stream (one after every few MFMAs) instead of issued together: a CU
    // accepts its loads at a limited rate, and a wave waiting to issue one
    // cannot issue its MFMAs either.  Step 0 issues parts [0, kSplit) of
    // slice kt + 2, step 1 (after the barrier) the rest.
    static_assert(FM == 4 && FN == 2 && kSteps == 2, "interleave pattern below");
    constexpr int kSplit = kFetchOps / 2;
    for (int kt = 0; kt < KT; ++kt) {
      const bool prefetch = kt + 2 < KT;
#pragma unroll
      for (int st = 0; st < kSteps; ++st) {
        const int cur = st & 1;
        const int nxt = cur ^ 1;
        const char* As = a_lds(kt);
        const char* Bs = b_lds(kt);
        // the next step's fragments are read unconditionally (after the last
        // slice they come from a valid, unused LDS slice and are not used):
        // no branches around LDS reads, so their waits stay exact
        int kk_next = kSteps * grp + st + 1;
        if (st + 1 == kSteps) {
          if (kt + 1 < KT) {
            if (prefetch) wait_vmcnt<kSplit>(); else wait_vmcnt<0>();
            __syncthreads();
            if (KTAIL && kt + 1 == KT - 1) zero_tail(kt + 1);
          }
          As = a_lds(kt + 1);
          Bs = b_lds(kt + 1);
          kk_next = kSteps * grp;
        }
        const int part0 = st * kSplit;
        auto mfma = [&](int i, int j) {
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[cur][i], bf[cur][j], acc[i][j], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        };
        auto dma = [&](int q) {
          if (prefetch && q < kSplit) fetch_part(kt + 2, part0 + q);
          __builtin_amdgcn_sched_barrier(0);
        };
        v2i blo[FN], bhi[FN];
        mfma(0, 0);
        af[nxt][0] = read_a(As, kk_next, 0);
        mfma(0, 1);
        af[nxt][1] = read_a(As, kk_next, 1);
        dma(0);
        mfma(1, 0);
        af[nxt][2] = read_a(As, kk_next, 2);
        mfma(1, 1);
        af[nxt][3] = read_a(As, kk_next, 3);
        dma(1);
        mfma(2, 0);
        if constexpr (MODE == kBknDma) {
          blo[0] = read_b_tr(Bs, kk_next, 0, 0);
          mfma(2, 1);
          bhi[0] = read_b_tr(Bs, kk_next, 0, 1);
          dma(2);
          mfma(3, 0);
          blo[1] = read_b_tr(Bs, kk_next, 1, 0);
          mfma(3, 1);
          bhi[1] = read_b_tr(Bs, kk_next, 1, 1);
#pragma unroll
          for (int j = 0; j < FN; ++j) bf[nxt][j] = v4i{blo[j].x, blo[j].y, bhi[j].x, bhi[j].y};
        } else {
          bf[nxt][0] = read_b_rowk(Bs, kk_next, 0);
          mfma(2, 1);
          dma(2);
          mfma(3, 0);
          bf[nxt][1] = read_b_rowk(Bs, kk_next, 1);
          mfma(3, 1);
        }
#pragma unroll
        for (int q = 3; q < kSplit; ++q) dma(q);
      }
    }
  }

  // ---- epilogue ----
  // The two wave groups hold partial sums of the same 128 x 64 sub-tile.
  // Group g finishes fragment rows i in [2g, 2g + 2): it hands the other
  // group's fragments over through LDS as 16-byte chunks (4 accumulator
  // registers), adds the chunks it receives, and stores straight from
  // registers.  A fragment's register r of lane l is element
  // (8 (r / 4) + 4 (l / 32) + r % 4, l % 32); a 4 x 4 transpose across each
  // lane quad (DPP) turns the four registers 4q .. 4q + 3 into four
  // consecutive columns of one row, so every lane writes 8 (bf16) or 16 (fp32)
  // contiguous bytes.  Output stores are nontemporal: nothing here reads them.
  constexpr int kHalfM = FM / kGroups;  // fragment rows finished per group
  constexpr int kChunkBytes = kHalfM * FN * 4 * 64 * 16;  // one group's hand-over
  static_assert(2 * kSubTiles * kChunkBytes + 4 * (BM + BN) <= kStages * STAGE,
                "epilogue hand-over fits in LDS");
  __syncthreads();  // every wave is done with the k slices
  float* s_sa = reinterpret_cast<float*>(smem + 2 * kSubTiles * kChunkBytes);
  float* s_sb = s_sa + BM;
  if (out) {
    for (int idx = t; idx < BM + BN; idx += kThreads) {
      if (idx < BM)
        s_sa[idx] = m0 + idx < M ? scale_a[m0 + idx] : 0.0f;
      else
        s_sb[idx - BM] = n0 + idx - BM < N ? scale_b[n0 + idx - BM] * output_scale : 0.0f;
    }
  }
  // hand-over region written for group `to` of this sub-tile
  auto chunk_at = [&](int to, int ii, int j, int q) -> int4* {
    return reinterpret_cast<int4*>(smem + (wsub * 2 + to) * kChunkBytes +
                                   (((ii * FN + j) * 4 + q) * 64 + lane) * 16);
  };
  auto give = [&](auto i_off) {  // fragments i_off .. i_off + kHalfM - 1 go to the other group
#pragma unroll
    for (int ii = 0; ii < kHalfM; ++ii)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const v16i& v = acc[i_off + ii][j];
          *chunk_at(1 - grp, ii, j, q) = make_int4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
        }
  };
  auto take = [&](auto i_off) {  // add the other group's sums for my fragments
#pragma unroll
    for (int ii = 0; ii < kHalfM; ++ii)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int4 v = *chunk_at(grp, ii, j, q);
          acc[i_off + ii][j][4 * q] += v.x;
          acc[i_off + ii][j][4 * q + 1] += v.y;
          acc[i_off + ii][j][4 * q + 2] += v.z;
          acc[i_off + ii][j][4 * q + 3] += v.w;
        }
  };
  if (grp == 0) give(std::integral_constant<int, kHalfM>{}); else give(std::integral_constant<int, 0>{});
  __syncthreads();  // hand-over and scales visible
  if (grp == 0) take(std::integral_constant<int, 0>{}); else take(std::integral_constant<int, kHalfM>{});

  const int quad_i = lane & 3;          // row within the 4-row group after the transpose
  const int col4 = 4 * ((lane & 31) >> 2);  // first of the lane's 4 columns in a fragment
  auto finish = [&](auto i_off) {
#pragma unroll
    for (int ii = 0; ii < kHalfM; ++ii)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int lcol = wn * WTN + j * 32 + col4;  // tile-local column
        const int gcol = n0 + lcol;
        float sb4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) sb4[e] = out ? s_sb[lcol + e] : 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          int v[4];
          quad_transpose(acc[i_off + ii][j][4 * q], acc[i_off + ii][j][4 * q + 1],
                         acc[i_off + ii][j][4 * q + 2], acc[i_off + ii][j][4 * q + 3], quad_i, v);
          const int lrow = wm * WTM + (i_off + ii) * 32 + 8 * q + 4 * (lane >> 5) + quad_i;
          const int grow = m0 + lrow;
          if (grow >= M) continue;
          const size_t base = static_cast<size_t>(grow) * N + gcol;
          const bool vec_ok = (N % 4 == 0) && (gcol + 4 <= N);
          if (c) {
            if (vec_ok) {
              __builtin_nontemporal_store(v4i{v[0], v[1], v[2], v[3]}, reinterpret_cast<v4i*>(c + base));
            } else {
              for (int e = 0; e < 4; ++e)
                if (gcol + e < N) c[base + e] = v[e];
            }
          }
          if (out) {
            const float sa = s_sa[lrow];
            float f[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) f[e] = (static_cast<float>(v[e]) * sa) * sb4[e];
            if (out_dtype == QK_BF16) {
              uint16_t* o = static_cast<uint16_t*>(out) + base;
              if (vec_ok) {
                const v2i w = {static_cast<int>(to_bf16(f[0]) | (static_cast<uint32_t>(to_bf16(f[1])) << 16)),
                               static_cast<int>(to_bf16(f[2]) | (static_cast<uint32_t>(to_bf16(f[3])) << 16))};
                __builtin_nontemporal_store(w, reinterpret_cast<v2i*>(o));
              } else {
                for (int e = 0; e < 4; ++e)
                  if (gcol + e < N) o[e] = to_bf16(f[e]);
              }
            } else {
              float* o = static_cast<float*>(out) + base;
              if (vec_ok) {
                typedef float v4f __attribute__((ext_vector_type(4)));
                __builtin_nontemporal_store(v4f{f[0], f[1], f[2], f[3]}, reinterpret_cast<v4f*>(o));
              } else {
                for (int e = 0; e < 4; ++e)
                  if (gcol + e < N) o[e] = f[e];
              }
            }
          }
        }
      }
  };
  if (grp == 0) finish(std::integral_constant<int, 0>{}); else finish(std::integral_constant<int, kHalfM>{});
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
  if (g.b_layout == QK_B_NK) return launch_mode<kBnkDma>(g, grid, tiles_m, tiles_n, stream);
  if (g.n % 16 == 0) return launch_mode<kBknDma>(g, grid, tiles_m, tiles_n, stream);
  if (g.n % 4 == 0) return launch_mode<kBknReg4>(g, grid, tiles_m, tiles_n, stream);
  return launch_mode<kBknReg1>(g, grid, tiles_m, tiles_n, stream);
}

}  // namespace qk
