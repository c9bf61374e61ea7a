// Decode-shaped INT8 GEMM (m <= 8 rows per launch) for gfx950: a split-K GEMV
// that streams the [K][N] weight once from HBM.
//
// What it computes is the same as the MFMA kernel ("16. Deploying Custom
// Kernels", C++ Kernel Interface; "KV-cache kernels", 02 Scales and
// dequantization); the shape is the one "dynquant-kernels", What is in here,
// calls the memory-bound decode GEMV, and "KV-cache kernels", 04 What changes
// in the kernel's shape, is the reason for a second tiling: with one or a few
// tokens the matrix cores would idle while the weight streams in.
//
// Design:
//   * A workgroup (256 lanes) owns a 256-row (k) x 512-column (n) block of
//     the weight.  Lane (cg, rg) = (t % 32, t / 32) loads 16 contiguous
//     bytes (columns 16cg..16cg+15) of rows k0 + 32 it + 4 rg + {0..3},
//     it = 0..7: every wave-wide load instruction reads two 512-byte row
//     segments, and each lane has 512 bytes in flight.
//   * The four rows of a lane are transposed in registers (v_perm_b32) into
//     sixteen 4-byte columns, each multiplied with the matching 4 activation
//     codes by v_dot4_i32_i8 (exact INT32).  Activation codes come from LDS.
//   * Partial sums are reduced across the wave's two row groups by a lane
//     swap, across the four waves with LDS atomics, and across the K splits
//     with device-scope INT32 atomics into the workspace: integer addition is
//     exact in any order, so the result is bit-identical to one sequential
//     sum.  The last workgroup to finish a column block (arrival counter)
//     reads the sums, applies the dequant epilogue, and returns the
//     workspace and the counter to zero for the next call.
#include "qk_internal.h"

namespace qk {
namespace {

constexpr int kThreads = 256;
constexpr int kCols = 512;               // columns per workgroup
constexpr int kRowsK = 256;              // k rows per workgroup
constexpr int kIters = kRowsK / 32;      // 8 row groups x 4 rows per iteration

__device__ __forceinline__ void transpose4x4(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                             uint32_t* col) {
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

template <int MR, bool N16>
__global__ __launch_bounds__(kThreads) void gemv_i8_splitk_kernel(
    const int8_t* __restrict__ a, const int8_t* __restrict__ w, int32_t* __restrict__ c,
    const float* __restrict__ scale_a, const float* __restrict__ scale_b, float output_scale,
    void* __restrict__ out, int out_dtype, int M, int N, int K, int col_tiles, int splits,
    int32_t* __restrict__ ws_acc, int32_t* __restrict__ ws_cnt) {
  __shared__ int32_t q_lds[MR][kRowsK / 4];
  __shared__ int32_t red[MR][kCols];
  __shared__ int last_flag;

  const int t = threadIdx.x;
  const int ct = blockIdx.x % col_tiles;
  const int ks = blockIdx.x / col_tiles;
  const int n0 = ct * kCols;
  const int k0 = ks * kRowsK;
  const int cg = t & 31;
  const int rg = t >> 5;

  for (int idx = t; idx < MR * (kRowsK / 4); idx += kThreads) {
    const int m = idx / (kRowsK / 4);
    const int k = k0 + 4 * (idx % (kRowsK / 4));
    q_lds[m][idx % (kRowsK / 4)] =
        (m < M && k < K) ? *reinterpret_cast<const int32_t*>(a + static_cast<size_t>(m) * K + k) : 0;
  }
  for (int idx = t; idx < MR * kCols; idx += kThreads) red[idx / kCols][idx % kCols] = 0;
  __syncthreads();

  int acc[MR][16];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[m][j] = 0;

  const int gn = n0 + 16 * cg;
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int kb = k0 + 32 * it + 4 * rg;
    uint32_t wr[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int k = kb + r;
      const int8_t* row = w + static_cast<size_t>(k) * N;
      if constexpr (N16) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (k < K && gn < N) v = *reinterpret_cast<const uint4*>(row + gn);
        wr[r][0] = v.x;
        wr[r][1] = v.y;
        wr[r][2] = v.z;
        wr[r][3] = v.w;
      } else {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          uint32_t x = 0;
          if (k < K) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int n = gn + 4 * q4 + e;
              if (n < N) x |= static_cast<uint32_t>(static_cast<uint8_t>(row[n])) << (8 * e);
            }
          }
          wr[r][q4] = x;
        }
      }
    }
    uint32_t col[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      transpose4x4(wr[0][q4], wr[1][q4], wr[2][q4], wr[3][q4], &col[4 * q4]);
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const int qd = q_lds[m][8 * it + rg];
#pragma unroll
      for (int j = 0; j < 16; ++j)
        acc[m][j] = __builtin_amdgcn_sdot4(static_cast<int>(col[j]), qd, acc[m][j], false);
    }
  }

  // lanes l and l + 32 hold the same columns for adjacent row groups
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[m][j] += __shfl_xor(acc[m][j], 32, 64);
  if ((t & 63) < 32) {
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int j = 0; j < 16; ++j) atomicAdd(&red[m][16 * cg + j], acc[m][j]);
  }
  __syncthreads();

  for (int idx = t; idx < MR * kCols; idx += kThreads) {
    const int m = idx / kCols;
    const int n = n0 + idx % kCols;
    if (m < M && n < N)
      __hip_atomic_fetch_add(&ws_acc[static_cast<size_t>(m) * N + n], red[m][idx % kCols],
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __threadfence();
  __syncthreads();
  if (t == 0) {
    const int prev =
        __hip_atomic_fetch_add(&ws_cnt[ct], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (prev == splits - 1);
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();

  for (int idx = t; idx < M * kCols; idx += kThreads) {
    const int m = idx / kCols;
    const int n = n0 + idx % kCols;
    if (n >= N) continue;
    int32_t* p = &ws_acc[static_cast<size_t>(m) * N + n];
    const int v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const size_t o = static_cast<size_t>(m) * N + n;
    if (c) c[o] = v;
    if (out) {
      const float f = (static_cast<float>(v) * scale_a[m]) * (scale_b[n] * output_scale);
      if (out_dtype == QK_BF16)
        static_cast<uint16_t*>(out)[o] = to_bf16(f);
      else
        static_cast<float*>(out)[o] = f;
    }
  }
  if (t == 0) __hip_atomic_store(&ws_cnt[ct], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int MR>
hipError_t launch_rows(const GemmArgs& g, int row0, int rows, hipStream_t stream) {
  const int col_tiles = (g.n + kCols - 1) / kCols;
  const int splits = g.k > 0 ? (g.k + kRowsK - 1) / kRowsK : 1;
  int32_t* ws_acc = static_cast<int32_t*>(g.workspace);
  int32_t* ws_cnt = ws_acc + static_cast<size_t>(kGemvMaxRows) * g.n;
  const int8_t* a = g.a + static_cast<size_t>(row0) * g.k;
  int32_t* c = g.c ? g.c + static_cast<size_t>(row0) * g.n : nullptr;
  const float* sa = g.scale_a ? g.scale_a + row0 : nullptr;
  void* out = nullptr;
  if (g.out) {
    const size_t esz = g.out_dtype == QK_BF16 ? 2 : 4;
    out = static_cast<char*>(g.out) + static_cast<size_t>(row0) * g.n * esz;
  }
  const dim3 grid(static_cast<unsigned>(col_tiles) * static_cast<unsigned>(splits));
  if (g.n % 16 == 0 && reinterpret_cast<uintptr_t>(g.b) % 16 == 0)
    return launch(gemv_i8_splitk_kernel<MR, true>, grid, dim3(kThreads), 0, stream, a, g.b, c, sa,
                  g.scale_b, g.output_scale, out, g.out_dtype, rows, g.n, g.k, col_tiles, splits,
                  ws_acc, ws_cnt);
  return launch(gemv_i8_splitk_kernel<MR, false>, grid, dim3(kThreads), 0, stream, a, g.b, c, sa,
                g.scale_b, g.output_scale, out, g.out_dtype, rows, g.n, g.k, col_tiles, splits,
                ws_acc, ws_cnt);
}

}  // namespace

size_t gemv_workspace_bytes(int n) {
  const size_t col_tiles = (static_cast<size_t>(n) + kCols - 1) / kCols;
  const size_t bytes = (static_cast<size_t>(kGemvMaxRows) * n + col_tiles) * sizeof(int32_t);
  return (bytes + 255) / 256 * 256;
}

hipError_t launch_gemv(const GemmArgs& g, hipStream_t stream) {
  for (int row0 = 0; row0 < g.m; row0 += kGemvMaxRows) {
    const int rows = g.m - row0 < kGemvMaxRows ? g.m - row0 : kGemvMaxRows;
    hipError_t e;
    if (rows == 1)
      e = launch_rows<1>(g, row0, rows, stream);
    else if (rows == 2)
      e = launch_rows<2>(g, row0, rows, stream);
    else if (rows <= 4)
      e = launch_rows<4>(g, row0, rows, stream);
    else
      e = launch_rows<8>(g, row0, rows, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qk
