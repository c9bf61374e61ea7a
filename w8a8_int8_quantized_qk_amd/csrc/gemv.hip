// Decode-shaped INT8 GEMM (m <= 8 rows per launch) for gfx950: a GEMV that
// streams the [K][N] weight from HBM exactly once.
//
// What it computes is the same as the MFMA kernel ("16. Deploying Custom
// Kernels", C++ Kernel Interface; "KV-cache kernels", 02 Scales and
// dequantization).  The shape is the one "dynquant-kernels", What is in here,
// calls the memory-bound decode GEMV, and "KV-cache kernels", 04 What changes
// in the kernel's shape, is the reason for a tiling of its own: with one to
// eight tokens the matrix cores would idle while the weight streams in.
//
// Design:
//   * Split-K: a workgroup (8 wave64s, two per SIMD) owns a 512 (k) x 512 (n)
//     block of the weight.  Lane (cg, half) of wave w loads 16 contiguous
//     bytes (columns 16 cg .. 16 cg + 15) of the four rows of row quad
//     2 w + half of each 64-row round: every wave-wide load instruction reads
//     two contiguous 512-byte row segments.  A lane issues the loads of all
//     eight rounds (32 x 128-bit) before using any.
//   * The four rows of a lane are transposed in registers (v_perm_b32) into
//     sixteen 4-byte columns and multiplied with the matching four activation
//     codes by v_dot4_i32_i8 (exact INT32).  Codes come from LDS.
//   * Partial sums are reduced across the two half-waves by a lane swap,
//     across the eight waves with LDS atomics, and across the K-slice
//     workgroups with device-scope INT32 atomic adds into a workspace:
//     integer addition is exact in any order, so the result is the same bits
//     as one sequential sum.  Each lane waits for its adds to complete, then
//     one lane per workgroup counts the arrival (acquire-release, device
//     scope).  The last workgroup of a column tile reads the sums, applies
//     the dequant epilogue, and returns its workspace words and counter to
//     zero for the next call.
//   * Activation codes are either given (int8 a, scale_a), or the kernel
//     quantizes the m activation rows itself from fp32/bf16/fp16 input with
//     the same arithmetic as the quantization kernels: every workgroup
//     reduces the whole row to the same bit-identical scale and encodes its
//     own k slice; one workgroup per slice writes the codes out when asked.
//     The activation loads are issued first and the weight loads right
//     after, so the quantization overlaps the weight stream.  The decode
//     linear is then a single launch.
#include "quant_math.h"

namespace qk {
namespace {

constexpr int kThreads = 512;   // 8 waves: two per SIMD
constexpr int kWaves = kThreads / 64;
constexpr int kCols = 512;      // output columns per workgroup: 32 lanes x 16 bytes
constexpr int kRowsK = 512;     // k rows per workgroup (one split-K slice)
constexpr int kRounds = kRowsK / 64;  // a round: 16 row quads = 8 waves x 2 half-waves
constexpr int kXUnits = 2;      // 16-byte activation units a lane keeps in registers

// rounds whose weight loads a lane keeps in flight (4 x 16 bytes each)
template <int MR>
constexpr int unroll_for() { return MR <= 2 ? 8 : (MR == 4 ? 4 : 2); }

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

// XDT < 0: `a` holds int8 codes [M][K] and scale_a their scales.
// XDT >= 0: `a` holds activations [M][K] of that dtype (16-byte aligned rows,
// K % 16 == 0), quantized here.
template <int MR, int XDT, bool N16>
__global__ __launch_bounds__(kThreads) void gemv_kernel(
    const void* __restrict__ a, const int8_t* __restrict__ w, int32_t* __restrict__ c,
    const float* __restrict__ scale_a, const float* __restrict__ scale_b, float output_scale,
    void* __restrict__ out, int out_dtype, int M, int N, int K, int8_t* __restrict__ q_out,
    float* __restrict__ s_out, int32_t* __restrict__ ws_acc, int32_t* __restrict__ ws_cnt,
    int col_tiles, int splits) {
  constexpr int U = unroll_for<MR>();
  __shared__ int32_t q_lds[MR][kRowsK / 4];  // codes of this k slice, 4 per word
  __shared__ float s_row[MR];
  __shared__ int red[MR][kCols];
  __shared__ int last_flag;

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

  for (int idx = t; idx < MR * kCols; idx += kThreads) red[idx / kCols][idx % kCols] = 0;

  // weight loads of U rounds; rows past K (zero codes) and columns past N
  // (never stored) read clamped, valid addresses instead of branching
  uint32_t wr[U][4][4];
  auto load_batch = [&](int round0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int k = min(k0 + (round0 + u) * 64 + 4 * quad + r, K - 1);
        const int8_t* row = w + static_cast<size_t>(k) * N;
        if constexpr (N16) {
          const uint4 v = *reinterpret_cast<const uint4*>(row + min(gn, N - 16));
          wr[u][r][0] = v.x;
          wr[u][r][1] = v.y;
          wr[u][r][2] = v.z;
          wr[u][r][3] = v.w;
        } else {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            uint32_t x = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              x |= static_cast<uint32_t>(static_cast<uint8_t>(row[min(gn + 4 * q4 + e, N - 1)])) << (8 * e);
            wr[u][r][q4] = x;
          }
        }
      }
    }
  };

  // ---- activation loads first, then the weight, so the activation work
  //      below overlaps the weight stream ----
  using E = qm::Elem<XDT < 0 ? QK_F32 : XDT>;
  constexpr int P = E::kPerUnit;
  const int units = K / P;  // 16-byte activation units per row (fused path)
  uint4 xr[MR][kXUnits];
  const bool x_in_regs = units <= kThreads * kXUnits;
  if constexpr (XDT >= 0) {
    if (x_in_regs && units > 0) {
#pragma unroll
      for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int j = 0; j < kXUnits; ++j) {
          const int mm = min(m, M - 1);
          const int u = min(t + kThreads * j, units - 1);
          xr[m][j] = *reinterpret_cast<const uint4*>(
              static_cast<const char*>(a) + (static_cast<size_t>(mm) * K + static_cast<size_t>(u) * P) * E::kBytes);
        }
    }
  }
  if (K > 0) load_batch(0);

  // ---- codes of rows k0 .. k0 + 511 into LDS ----
  if constexpr (XDT < 0) {
    const int8_t* q = static_cast<const int8_t*>(a);
    for (int idx = t; idx < MR * (kRowsK / 4); idx += kThreads) {
      const int m = idx / (kRowsK / 4);
      const int k = k0 + 4 * (idx % (kRowsK / 4));
      q_lds[m][idx % (kRowsK / 4)] =
          (m < M && k < K) ? *reinterpret_cast<const int32_t*>(q + static_cast<size_t>(m) * K + k) : 0;
    }
    if (t < MR) s_row[t] = (t < M && scale_a) ? scale_a[t] : 0.0f;
  } else {
    for (int m = 0; m < MR; ++m) {
      if (m >= M) {  // padding rows: zero codes
        for (int idx = t; idx < kRowsK / 4; idx += kThreads) q_lds[m][idx] = 0;
        continue;
      }
      const char* xrow = static_cast<const char*>(a) + static_cast<size_t>(m) * K * E::kBytes;
      auto unit = [&](int j, int u) -> uint4 {  // unit u of this row, from registers if held
        if (x_in_regs) return xr[m][j];
        return *reinterpret_cast<const uint4*>(xrow + static_cast<size_t>(u) * 16);
      };
      // the scale needs the whole row: every workgroup reduces it (identical bits)
      float amax = 0.0f;
      for (int u0 = 0; u0 < units; u0 += kThreads * kXUnits) {
#pragma unroll
        for (int j = 0; j < kXUnits; ++j) {
          const int u = min(u0 + t + kThreads * j, units - 1);  // duplicates add nothing to a max
          float v[P];
          E::unpack(unit(j, u), v);
#pragma unroll
          for (int e = 0; e < P; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[e]));
        }
      }
      amax = qm::block_max<kThreads>(amax);
      float s, r;
      qm::row_scale(amax, s, r);
      if (t == 0) s_row[m] = s;
      if (blockIdx.x == 0 && t == 0 && s_out) s_out[m] = s;
      // codes of this workgroup's k slice only
      for (int idx = t; idx < kRowsK / 4; idx += kThreads) q_lds[m][idx] = 0;
      __syncthreads();
      const int u_lo = k0 / P;
      const int u_hi = min(units, (k0 + kRowsK) / P);
      for (int u0 = 0; u0 < units; u0 += kThreads * kXUnits) {
#pragma unroll
        for (int j = 0; j < kXUnits; ++j) {
          const int u = u0 + t + kThreads * j;
          if (u < u_lo || u >= u_hi) continue;
          float v[P];
          E::unpack(unit(j, u), v);
#pragma unroll
          for (int e4 = 0; e4 < P / 4; ++e4) {
            const uint32_t word =
                qm::pack4(qm::code_of(v[4 * e4], s, r), qm::code_of(v[4 * e4 + 1], s, r),
                          qm::code_of(v[4 * e4 + 2], s, r), qm::code_of(v[4 * e4 + 3], s, r));
            const int kw = u * (P / 4) + e4;  // codes of elements 4 kw .. 4 kw + 3
            q_lds[m][kw - k0 / 4] = static_cast<int32_t>(word);
            if (ct == 0 && q_out)  // one workgroup per k slice writes the codes
              *reinterpret_cast<uint32_t*>(q_out + static_cast<size_t>(m) * K + 4 * kw) = word;
          }
        }
      }
      __syncthreads();  // block_max reuses its LDS between rows
    }
  }
  __syncthreads();

  // ---- multiply the streamed weight with the codes ----
  int acc[MR][16];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[m][j] = 0;

  for (int round0 = 0; K > 0 && round0 < kRounds; round0 += U) {
    if (round0 > 0) load_batch(round0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint32_t col[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        transpose4x4(wr[u][0][q4], wr[u][1][q4], wr[u][2][q4], wr[u][3][q4], &col[4 * q4]);
      const int kw = (round0 + u) * 16 + quad;
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const int qd = q_lds[m][kw];
#pragma unroll
        for (int j = 0; j < 16; ++j)
          acc[m][j] = __builtin_amdgcn_sdot4(static_cast<int>(col[j]), qd, acc[m][j], false);
      }
    }
  }

  // ---- reduce within the workgroup: the two half-waves, then LDS ----
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int v = acc[m][j] + __shfl_xor(acc[m][j], 32, 64);
      if (lane < 32) atomicAdd(&red[m][16 * cg + j], v);
    }
  __syncthreads();

  // ---- across the split-K workgroups: exact INT32 adds into the workspace ----
  for (int idx = t; idx < MR * kCols; idx += kThreads) {
    const int m = idx / kCols;
    const int n = n0 + idx % kCols;
    if (m < M && n < N)
      __hip_atomic_fetch_add(&ws_acc[static_cast<size_t>(m) * N + n], red[m][idx % kCols],
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // every lane's adds have completed before the workgroup's arrival is counted
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (t == 0) {
    const int prev =
        __hip_atomic_fetch_add(&ws_cnt[ct], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = prev == splits - 1;
  }
  __syncthreads();
  if (!last_flag) return;

  // ---- last workgroup of this column tile: epilogue, workspace back to zero ----
  __atomic_thread_fence(__ATOMIC_ACQUIRE);
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
      const float f = (static_cast<float>(v) * s_row[m]) * (scale_b[n] * output_scale);
      if (out_dtype == QK_BF16)
        static_cast<uint16_t*>(out)[o] = to_bf16(f);
      else
        static_cast<float*>(out)[o] = f;
    }
  }
  if (t == 0) __hip_atomic_store(&ws_cnt[ct], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int MR, int XDT>
hipError_t launch_mr(const GemvArgs& g, int row0, int rows, hipStream_t stream) {
  const size_t xsz = XDT == QK_F32 ? 4 : (XDT < 0 ? 1 : 2);
  const void* a = static_cast<const char*>(g.a) + static_cast<size_t>(row0) * g.k * xsz;
  int32_t* c = g.c ? g.c + static_cast<size_t>(row0) * g.n : nullptr;
  const float* sa = g.scale_a ? g.scale_a + row0 : nullptr;
  void* out = nullptr;
  if (g.out) {
    const size_t esz = g.out_dtype == QK_BF16 ? 2 : 4;
    out = static_cast<char*>(g.out) + static_cast<size_t>(row0) * g.n * esz;
  }
  int8_t* q_out = g.q_out ? g.q_out + static_cast<size_t>(row0) * g.k : nullptr;
  float* s_out = g.s_out ? g.s_out + row0 : nullptr;
  const int col_tiles = (g.n + kCols - 1) / kCols;
  const int splits = g.k > 0 ? (g.k + kRowsK - 1) / kRowsK : 1;
  int32_t* ws_acc = static_cast<int32_t*>(g.workspace);
  int32_t* ws_cnt = ws_acc + static_cast<size_t>(kGemvMaxRows) * g.n;
  const dim3 grid(static_cast<unsigned>(col_tiles) * static_cast<unsigned>(splits));
  if (g.n % 16 == 0 && reinterpret_cast<uintptr_t>(g.b) % 16 == 0)
    return launch(gemv_kernel<MR, XDT, true>, grid, dim3(kThreads), 0, stream, a, g.b, c, sa,
                  g.scale_b, g.output_scale, out, g.out_dtype, rows, g.n, g.k, q_out, s_out,
                  ws_acc, ws_cnt, col_tiles, splits);
  return launch(gemv_kernel<MR, XDT, false>, grid, dim3(kThreads), 0, stream, a, g.b, c, sa,
                g.scale_b, g.output_scale, out, g.out_dtype, rows, g.n, g.k, q_out, s_out,
                ws_acc, ws_cnt, col_tiles, splits);
}

template <int XDT>
hipError_t launch_rows(const GemvArgs& g, hipStream_t stream) {
  for (int row0 = 0; row0 < g.m; row0 += kGemvMaxRows) {
    const int rows = g.m - row0 < kGemvMaxRows ? g.m - row0 : kGemvMaxRows;
    hipError_t e;
    if (rows == 1)
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
  const size_t col_tiles = (static_cast<size_t>(n) + kCols - 1) / kCols;
  const size_t bytes = (static_cast<size_t>(kGemvMaxRows) * n + col_tiles) * sizeof(int32_t);
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
