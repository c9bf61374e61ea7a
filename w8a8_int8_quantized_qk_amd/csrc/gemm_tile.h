// Workgroup tile machinery shared by the INT8 and FP8 MFMA GEMMs (gfx950):
// tile sizes, LDS layouts and their swizzles, global-to-LDS transfers of the
// operand tiles, the register-staged weight tile, the XCD-aware tile order and
// the LDS-staged epilogue stores.  Both kernels run 512 threads on a 256 x 128
// output tile with 128-byte k slices of one-byte operands.
#pragma once

#include "lds_dma.h"
#include "qk_internal.h"

#include <type_traits>

namespace qk {
namespace tile {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;   // 8: two per SIMD
constexpr int BM = 256;
constexpr int BN = 128;
constexpr int BK = 128;
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
__device__ __forceinline__ int rowk_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int rowk_offset(int row, int chunk) {
  return row * BK + ((chunk ^ rowk_swz(row)) << 4);
}
// [k][n] weight tile: 128-byte rows of n
__device__ __forceinline__ int kn_swz(int k) { return (k & 7) ^ ((k >> 4) & 1); }
__device__ __forceinline__ int kn_offset(int k, int chunk) {
  return k * BN + ((chunk ^ kn_swz(k)) << 4);
}

// DMA of a k-contiguous tile of ROWS rows x 128 bytes (global rows clamped to
// rows_valid - 1, k offset clamped into the row): instruction i of this
// wave's share (1 KiB = 8 rows each).
template <int ROWS>
constexpr int rowk_ops() { return ROWS * BK / 1024 / kWaves; }
// Row-major [rows][K] operand; ld, when given, is the row stride (a k range
// of a longer row), else K.
template <int ROWS>
__device__ __forceinline__ void dma_rowk_one(const int8_t* __restrict__ g, char* lds,
                                             int rows_valid, int K, int r0, int k0, int i,
                                             int ld = -1) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int blk = wave * rowk_ops<ROWS>() + i;
  const int row = blk * 8 + (lane >> 3);
  const int lchunk = (lane & 7) ^ rowk_swz(row);
  const uint32_t gr = static_cast<uint32_t>(min(r0 + row, rows_valid - 1));
  const uint32_t gk = static_cast<uint32_t>(min(k0 + 16 * lchunk, K - 16));
  lds_dma16(g + (gr * static_cast<uint32_t>(ld < 0 ? K : ld) + gk), lds_addr(lds + blk * 1024));
}
template <int ROWS>
__device__ __forceinline__ void dma_rowk(const int8_t* __restrict__ g, char* lds, int rows_valid,
                                         int K, int r0, int k0, int ld = -1) {
#pragma unroll
  for (int i = 0; i < rowk_ops<ROWS>(); ++i)
    dma_rowk_one<ROWS>(g, lds, rows_valid, K, r0, k0, i, ld);
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
  const int lchunk = (lane & 7) ^ kn_swz(k);
  const uint32_t gk = static_cast<uint32_t>(min(k0 + k, K - 1));
  const uint32_t gn = static_cast<uint32_t>(min(n0 + 16 * lchunk, N - 16));
  lds_dma16(b + (gk * static_cast<uint32_t>(N) + gn), lds_addr(lds + blk * 1024));
}
__device__ __forceinline__ void dma_kn(const int8_t* __restrict__ b, char* lds, int N, int K,
                                       int n0, int k0) {
#pragma unroll
  for (int i = 0; i < kn_ops(); ++i) dma_kn_one(b, lds, N, K, n0, k0, i);
}

// Source addresses and LDS slots of one thread's DMA instructions of a k
// slice (A parts first, then the weight's), formed once per kernel: slice s
// adds s times the part's stride (BK bytes along k) and its stage offset.
// Valid when no clamp changes from slice to slice: K a multiple of BK and a
// DMA'd weight (MODE kBnkDma or kBknDma).
//
// SPLIT false: the interleaved ring (stage s at s * STAGE, the weight block
// at A_STAGE within it), each source a 64-bit per-lane address.  SPLIT true:
// the split ring of XferParts below, each source a wave-uniform base in
// scalar registers (advanced per slice there) plus a fixed 32-bit lane
// offset (needs xfer_parts_fit; lda and ldb are K).
template <int MODE, bool SPLIT = false>
struct FixedParts {
  static constexpr int kOpsA = rowk_ops<BM>();
  static constexpr int kOps = kOpsA + (MODE == kBnkDma ? rowk_ops<BN>() : kn_ops());
  static constexpr uint32_t kBSlot0 = SPLIT ? 0 : A_STAGE;  // weight block within its stage
  const int8_t* src[SPLIT ? 1 : kOps];
  size_t stride[SPLIT ? 1 : kOps];
  const int8_t* base_a;
  const int8_t* base_b;
  size_t stride_b;
  uint32_t voff[SPLIT ? kOps : 1];
  uint32_t lds[kOps];  // wave-uniform (m0 operand)

  // lda, ldb: the row strides of A and of a [N][K] B when they are a k range
  // of longer rows (else K)
  __device__ __forceinline__ void init(const int8_t* __restrict__ a, const int8_t* __restrict__ b,
                                       int M, int N, int K, int m0, int n0, int lda = -1,
                                       int ldb = -1) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const uint32_t la = static_cast<uint32_t>(lda < 0 ? K : lda);
    const uint32_t lb = static_cast<uint32_t>(ldb < 0 ? K : ldb);
    if constexpr (SPLIT) {
      base_a = a + static_cast<size_t>(m0) * la;
      base_b = MODE == kBknDma ? b + n0 : b + static_cast<size_t>(n0) * lb;
      stride_b = MODE == kBknDma ? static_cast<size_t>(BK) * N : BK;
    }
#pragma unroll
    for (int q = 0; q < kOps; ++q) {
      uint32_t rel;        // offset from the tile's base (SPLIT)
      const int8_t* full;  // whole address (interleaved)
      if (q < kOpsA) {
        const int blk = wave * kOpsA + q;
        const int row = blk * 8 + (lane >> 3);
        const int lchunk = (lane & 7) ^ rowk_swz(row);
        const uint32_t gr = static_cast<uint32_t>(min(m0 + row, M - 1));
        rel = (gr - m0) * la + 16 * lchunk;
        full = a + (gr * la + 16 * lchunk);
        lds[q] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(blk * 1024));
        if constexpr (!SPLIT) stride[q] = BK;
      } else if constexpr (MODE == kBnkDma) {
        const int blk = wave * rowk_ops<BN>() + (q - kOpsA);
        const int row = blk * 8 + (lane >> 3);
        const int lchunk = (lane & 7) ^ rowk_swz(row);
        const uint32_t gr = static_cast<uint32_t>(min(n0 + row, N - 1));
        rel = (gr - n0) * lb + 16 * lchunk;
        full = b + (gr * lb + 16 * lchunk);
        lds[q] = __builtin_amdgcn_readfirstlane(kBSlot0 + static_cast<uint32_t>(blk * 1024));
        if constexpr (!SPLIT) stride[q] = BK;
      } else {
        const int blk = wave * kn_ops() + (q - kOpsA);
        const int k = blk * 8 + (lane >> 3);
        const int lchunk = (lane & 7) ^ kn_swz(k);
        const uint32_t gn = static_cast<uint32_t>(min(n0 + 16 * lchunk, N - 16));
        rel = static_cast<uint32_t>(k) * static_cast<uint32_t>(N) + (gn - n0);
        full = b + (static_cast<uint32_t>(k) * static_cast<uint32_t>(N) + gn);
        lds[q] = __builtin_amdgcn_readfirstlane(kBSlot0 + static_cast<uint32_t>(blk * 1024));
        if constexpr (!SPLIT) stride[q] = static_cast<size_t>(BK) * N;
      }
      if constexpr (SPLIT) voff[q] = rel;
      else src[q] = full;
    }
  }
  // DMA part `part` of slice s into its stage of the LDS ring at lds_smem
  __device__ __forceinline__ void issue(uint32_t lds_smem, int s, int part) const {
    if constexpr (SPLIT) {
      const uint32_t st = static_cast<uint32_t>(
          part < kOpsA ? (s % kStages) * A_STAGE : kStages * A_STAGE + (s % kStages) * B_STAGE);
      const int8_t* sbase = part < kOpsA ? base_a + static_cast<size_t>(s) * BK
                                         : base_b + static_cast<size_t>(s) * stride_b;
      lds_dma16_split(sbase, voff[part], lds_smem + st + lds[part]);
    } else {
      lds_dma16(src[part] + static_cast<size_t>(s) * stride[part],
                lds_smem + static_cast<uint32_t>((s % kStages) * STAGE) + lds[part]);
    }
  }
};

struct NoParts {};

// The transfer waves' per-lane source offsets (below 256 rows of K bytes, or
// 128 k rows of N bytes) fit in 32 bits.
__host__ __device__ constexpr bool xfer_parts_fit(int n, int k) {
  return k > 0 && n > 0 && k <= (1 << 24) && n <= (1 << 24);
}

// Transfer waves' parts, for kernels whose global-to-LDS transfers are issued
// by kXferWaves waves of their own: transfer wave d (0 .. kXferWaves - 1)
// issues kXferOps of a slice's 48 1-KiB parts, A blocks kXferOpsA d ..
// kXferOpsA d + 7 (8 rows of 128 bytes each), then a quarter of the weight
// block.  Valid for K a multiple of BK, a DMA'd weight and xfer_parts_fit.
constexpr int kXferWaves = 4;
constexpr int kXferOps = (BM + BN) * BK / 1024 / kXferWaves;  // 12
constexpr int kXferOpsA = BM * BK / 1024 / kXferWaves;        // 8
// The parts fill the split LDS ring: the A blocks of the stages at
// s * A_STAGE and the weight blocks after all of them, at kStages * A_STAGE +
// s * B_STAGE, so that the three weight stages lie within one 64 KiB reach
// of a DS immediate offset.
template <int MODE>
struct XferParts {
  static_assert(MODE == kBnkDma || MODE == kBknDma, "DMA weight layouts");
  // A part's source is a wave-uniform base (the tile's A rows or weight
  // block at slice 0, advanced per slice in scalar registers) plus this
  // lane's 32-bit offset, which stays fixed over the k loop; xfer_parts_fit
  // bounds the offsets.
  const int8_t* base_a;
  const int8_t* base_b;
  size_t stride_b;             // weight bytes per slice (A: BK)
  uint32_t voff[kXferOps];
  uint32_t slot[kXferOps];

  __device__ __forceinline__ void init(const int8_t* __restrict__ a, const int8_t* __restrict__ b,
                                       int M, int N, int K, int m0, int n0, int d) {
    // the lane index from the exec mask (the whole wave runs this), not from
    // threadIdx, which the kernel then need not keep in a register
    const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    base_a = a + static_cast<size_t>(m0) * K;
    base_b = MODE == kBknDma ? b + n0 : b + static_cast<size_t>(n0) * K;
    stride_b = MODE == kBknDma ? static_cast<size_t>(BK) * N : BK;
#pragma unroll
    for (int q = 0; q < kXferOps; ++q) {
      if (q < kXferOpsA) {  // A block kXferOpsA d + q: 8 rows of 128 bytes
        const int blk = kXferOpsA * d + q;
        const int row = blk * 8 + (lane >> 3);
        const int lchunk = (lane & 7) ^ rowk_swz(row);
        voff[q] = static_cast<uint32_t>(min(m0 + row, M - 1) - m0) * static_cast<uint32_t>(K) +
                  16 * lchunk;
        slot[q] = static_cast<uint32_t>(blk * 1024);
      } else if constexpr (MODE == kBnkDma) {  // [N][K] weight block: 8 rows of 128 bytes
        const int blk = (kXferOps - kXferOpsA) * d + (q - kXferOpsA);
        const int row = blk * 8 + (lane >> 3);
        const int lchunk = (lane & 7) ^ rowk_swz(row);
        voff[q] = static_cast<uint32_t>(min(n0 + row, N - 1) - n0) * static_cast<uint32_t>(K) +
                  16 * lchunk;
        slot[q] = static_cast<uint32_t>(blk * 1024);
      } else {  // [K][N] weight block: 8 k rows of 128 bytes (n0 <= N - 16)
        const int blk = (kXferOps - kXferOpsA) * d + (q - kXferOpsA);
        const int k = blk * 8 + (lane >> 3);
        const int lchunk = (lane & 7) ^ kn_swz(k);
        voff[q] = static_cast<uint32_t>(k) * static_cast<uint32_t>(N) +
                  static_cast<uint32_t>(min(n0 + 16 * lchunk, N - 16) - n0);
        slot[q] = static_cast<uint32_t>(blk * 1024);
      }
    }
  }
  // offset of part q's stage of slice s in the ring
  __device__ __forceinline__ static uint32_t stage_offset(int s, int q) {
    return static_cast<uint32_t>(q < kXferOpsA ? (s % kStages) * A_STAGE
                                               : kStages * A_STAGE + (s % kStages) * B_STAGE);
  }
  // every part of slice s into its stage of the LDS ring at lds_smem
  __device__ __forceinline__ void issue(uint32_t lds_smem, int s) const {
    const int8_t* sa = base_a + static_cast<size_t>(s) * BK;
    const int8_t* sb = base_b + static_cast<size_t>(s) * stride_b;
#pragma unroll
    for (int q = 0; q < kXferOps; ++q)
      lds_dma16_split(q < kXferOpsA ? sa : sb, voff[q],
                      __builtin_amdgcn_readfirstlane(lds_smem + stage_offset(s, q) + slot[q]));
  }
  // The transfer wave's whole k loop, matching a consumer that waits at one
  // barrier after slice 0 has landed and then one per slice kt < KT - 1, by
  // which slice kt + 1 has landed and every wave has read its last fragments
  // of slice kt - 1 (whose stage slice kt + 2 then takes).  KT <= 0: no
  // transfer and no barrier (the operands may be empty).
  __device__ __forceinline__ void run(uint32_t lds_smem, int KT) const {
    if (KT <= 0) return;
    issue(lds_smem, 0);
    if (KT > 1) {
      issue(lds_smem, 1);
      wait_vmcnt<kXferOps>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();  // slice 0 in LDS
    for (int kt = 0; kt < KT; ++kt) {
      const bool more = kt + 2 < KT;
      if (more) issue(lds_smem, kt + 2);
      if (kt + 1 < KT) {
        if (more) wait_vmcnt<kXferOps>(); else wait_vmcnt<0>();  // slice kt + 1 landed
        __syncthreads();
      }
    }
  }
};

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

// Tile b of T workgroups, renumbered so that the ones dispatched together to
// one XCD (b, b + 8, ... run on the same XCD) are consecutive.
__device__ __forceinline__ int xcd_order(int b, int T) {
  return T % 8 == 0 ? (b % 8) * (T / 8) + b / 8 : b;
}

// (tm, tn) of tile b of a tiles_m x tiles_n grid: groups of kGroupM tile rows,
// column-major inside a group, so that consecutive tiles share A rows and B
// columns.
__device__ __forceinline__ void group_order(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int group_tiles = kGroupM * tiles_n;
  const int g = b / group_tiles;
  const int first_m = g * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int r = b - g * group_tiles;
  tm = first_m + r % gm;
  tn = r / gm;
}

__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  group_order(xcd_order(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, tm, tn);
}

// ---- grouped (MoE) launches ----
// Rows [offsets[e], offsets[e + 1]) of the activations belong to expert e
// (offsets clamped to [0, M]: invalid ones give unspecified results but no
// access out of bounds).  Expert e has ceil(rows / TILE_M) x tiles_n tiles,
// numbered expert by expert; the grid is an upper bound on their total (the
// offsets live on the device).  Every workgroup (kThreads threads, one per
// expert and at most MAX_EXPERTS experts) counts each expert's tiles with a
// block-wide prefix sum and takes the tile its index falls on: expert e,
// index `local` within e's tiles, e's first row r0 and row count Me.  The
// XCD renumbering runs over the real total, so the surplus workgroups, all
// at the end of the grid, do not unbalance the XCDs.  Returns false (for the
// whole workgroup) past the last tile.
template <int TILE_M, int MAX_EXPERTS>
__device__ __forceinline__ bool moe_pick(const int* __restrict__ offsets, int experts, int M,
                                         int tiles_n, int& e, int& local, int& r0, int& Me) {
  static_assert(MAX_EXPERTS <= kThreads && MAX_EXPERTS % 64 == 0, "one thread per expert");
  __shared__ int s_wave_sum[MAX_EXPERTS / 64];
  __shared__ int s_pick[2];  // the workgroup's expert and that expert's first tile
  const int t = threadIdx.x;
  int tiles = 0;
  if (t < experts) {
    const int row0 = min(max(offsets[t], 0), M);
    const int row1 = min(max(offsets[t + 1], 0), M);
    tiles = row1 > row0 ? ((row1 - row0 + TILE_M - 1) / TILE_M) * tiles_n : 0;
  }
  // inclusive prefix sum of the tile counts: within each wave, then across
  // the waves
  int incl = tiles;
  if (t < MAX_EXPERTS) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if ((t & 63) >= d) incl += v;
    }
    if ((t & 63) == 63) s_wave_sum[t >> 6] = incl;
  }
  if (t == 0) s_pick[0] = -1;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < MAX_EXPERTS / 64; ++w) {
    if (w < (t >> 6)) before += s_wave_sum[w];
    total += s_wave_sum[w];
  }
  const int v = xcd_order(blockIdx.x, total);  // meaningful for blockIdx.x < total
  const int excl = before + incl - tiles;
  if (t < experts && tiles > 0 && v >= excl && v < excl + tiles) {
    s_pick[0] = t;
    s_pick[1] = excl;
  }
  __syncthreads();
  e = s_pick[0];
  if (static_cast<int>(blockIdx.x) >= total || e < 0) return false;
  local = v - s_pick[1];
  r0 = min(max(offsets[e], 0), M);
  Me = min(max(offsets[e + 1], 0), M) - r0;
  return true;
}

// ---- LDS-staged epilogue ----
// A wave stages a block of kRows x 64 32-bit results row-major in LDS (the
// operand slices are free by then) and reads it back row-contiguous, so that
// every store instruction writes whole 128-byte row segments.  16-byte chunk
// q (columns 4q .. 4q + 3) of staged row r; the XOR keeps the transposed
// writes and both read patterns below free of bank conflicts.
constexpr int kStageCols = 64;
__device__ __forceinline__ v4i* stage_at(int* stage, int r, int q) {
  return reinterpret_cast<v4i*>(stage + r * kStageCols + ((q ^ (((r & 3) << 2) | (r & 1))) << 2));
}

// Writes fragment (ii, j) of a wave's block into its staging rows: a
// fragment's register r of lane l is element (4 (l / 16) + r, l % 16); a 4 x 4
// transpose across each lane quad gives every lane four consecutive columns
// of one row.
__device__ __forceinline__ void stage_fragment(int* stage, int lane, int ii, int j, const v4i& f) {
  const int quad_i = lane & 3;  // row within the 4-row group after the transpose
  int v[4];
  quad_transpose(f[0], f[1], f[2], f[3], quad_i, v);
  *stage_at(stage, ii * 16 + 4 * (lane >> 4) + quad_i, 4 * j + ((lane & 15) >> 2)) =
      v4i{v[0], v[1], v[2], v[3]};
}

// The value of a staged 32-bit result: an INT32 accumulator converted to
// binary32, or the binary32 accumulator itself.
template <bool ACC_F32>
__device__ __forceinline__ float acc_value(int v) {
  if constexpr (ACC_F32)
    return __int_as_float(v);
  else
    return static_cast<float>(v);
}

// Zero-point correction of INT32 accumulators (asymmetric activations):
// acc - zp[row] * wsum[col], with the tile's zero points and column sums in
// LDS.  Without CORR the accumulators are used as they are.
template <bool CORR>
__device__ __forceinline__ v4i corrected(v4i v, const int* s_zp, const int* s_ws, int lrow, int lcol) {
  if constexpr (CORR) {
    const int z = s_zp[lrow];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] -= z * s_ws[lcol + e];
  }
  return v;
}

// Raw accumulators (IS_C: INT32 or binary32 bit patterns to c) or fp32
// results: 4 columns (16 bytes) per lane, 4 rows per pass.  The block covers
// tile-local rows [lrow0, lrow0 + kRows) and columns [lcol0, lcol0 + 64) of
// the tile at (m0, n0); s_sa and s_sb are the tile's row and column scales,
// s_zp and s_ws its zero points and column sums (CORR only).
template <int kRows, bool ACC_F32, bool IS_C, bool CORR = false>
__device__ __forceinline__ void store4(int* stage, int lane, int m0, int n0, int lrow0, int lcol0,
                                       int M, int N, const float* s_sa, const float* s_sb,
                                       void* __restrict__ dst, const int* s_zp = nullptr,
                                       const int* s_ws = nullptr) {
  const int q = lane & 15;
  const int lcol = lcol0 + 4 * q;
  const int gcol = n0 + lcol;
  float sb4[4];
  if constexpr (!IS_C) {
#pragma unroll
    for (int e = 0; e < 4; ++e) sb4[e] = s_sb[lcol + e];
  }
#pragma unroll 4
  for (int pass = 0; pass < kRows / 4; ++pass) {
    const int r = 4 * pass + (lane >> 4);
    const int grow = m0 + lrow0 + r;
    const v4i v = corrected<CORR>(*stage_at(stage, r, q), s_zp, s_ws, lrow0 + r, lcol);
    if (grow >= M) continue;
    const size_t base = static_cast<size_t>(grow) * N + gcol;
    if constexpr (IS_C) {
      int32_t* o = static_cast<int32_t*>(dst) + base;
      if (gcol + 4 <= N && reinterpret_cast<uintptr_t>(o) % 16 == 0) {
        __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(o));
      } else {
        for (int e = 0; e < 4; ++e)
          if (gcol + e < N) o[e] = v[e];
      }
    } else {
      typedef float v4f __attribute__((ext_vector_type(4)));
      const float sa = s_sa[lrow0 + r];
      v4f f;
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = (acc_value<ACC_F32>(v[e]) * sa) * sb4[e];
      float* o = static_cast<float*>(dst) + base;
      if (gcol + 4 <= N && reinterpret_cast<uintptr_t>(o) % 16 == 0) {
        __builtin_nontemporal_store(f, reinterpret_cast<v4f*>(o));
      } else {
        for (int e = 0; e < 4; ++e)
          if (gcol + e < N) o[e] = f[e];
      }
    }
  }
}

// bf16 results: 8 columns (16 bytes) per lane, 8 rows per pass.
template <int kRows, bool ACC_F32, bool CORR = false>
__device__ __forceinline__ void store_bf16(int* stage, int lane, int m0, int n0, int lrow0,
                                           int lcol0, int M, int N, const float* s_sa,
                                           const float* s_sb, void* __restrict__ out,
                                           const int* s_zp = nullptr, const int* s_ws = nullptr) {
  const int q2 = lane & 7;
  const int lcol = lcol0 + 8 * q2;
  const int gcol = n0 + lcol;
  float sb8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sb8[e] = s_sb[lcol + e];
#pragma unroll 4
  for (int pass = 0; pass < kRows / 8; ++pass) {
    const int r = 8 * pass + (lane >> 3);
    const int grow = m0 + lrow0 + r;
    const v4i v0 = corrected<CORR>(*stage_at(stage, r, 2 * q2), s_zp, s_ws, lrow0 + r, lcol);
    const v4i v1 = corrected<CORR>(*stage_at(stage, r, 2 * q2 + 1), s_zp, s_ws, lrow0 + r, lcol + 4);
    if (grow >= M) continue;
    const float sa = s_sa[lrow0 + r];
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      h[e] = to_bf16((acc_value<ACC_F32>(e < 4 ? v0[e] : v1[e - 4]) * sa) * sb8[e]);
    uint16_t* o = static_cast<uint16_t*>(out) + static_cast<size_t>(grow) * N + gcol;
    if (gcol + 8 <= N && reinterpret_cast<uintptr_t>(o) % 16 == 0) {
      const v4i w = {static_cast<int>(h[0] | (h[1] << 16)), static_cast<int>(h[2] | (h[3] << 16)),
                     static_cast<int>(h[4] | (h[5] << 16)), static_cast<int>(h[6] | (h[7] << 16))};
      __builtin_nontemporal_store(w, reinterpret_cast<v4i*>(o));
    } else {
      for (int e = 0; e < 8; ++e)
        if (gcol + e < N) o[e] = static_cast<uint16_t>(h[e]);
    }
  }
}

}  // namespace tile
}  // namespace qk
