// bf16 MFMA projection GEMM for the joint block: C = A W^T (+ per-batch bias).
//
// Used for the per-modality input projections (with the time embedding tau,
// or its derivative for tangent rows, as the bias), the concatenated Q/K/V
// projection sharing one input (the deep read of TurboT2VA, section 6.2,
// concatenates projections that share an input; here W_qkv is one [3d, d]
// matrix), and the per-modality output projections.  Primal and tangent rows
// are separate batches of the same launch, so the weights are read once for
// both.
//
// Both operands are K-contiguous, so every MFMA operand is one 16-byte LDS
// read.  Tile 128x128x64, 4 waves in 2x2, each wave 64x64 as 2x2 tiles of
// v_mfma_f32_32x32x16_bf16; LDS double-buffered with one barrier per k-tile.
// Columns at or beyond n_split can be written transposed per head
// (V^T[b][h][c][row]), the layout the attention kernel stages V from.
#include "common.h"

namespace t2va {

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LROW = BK + 8;  // padded LDS row (elements): 144 B, conflict-free 16-B reads
constexpr int kThreads = 256;
constexpr int kStageElems = (BM + BN) * LROW;
constexpr size_t kLdsBytes = 2 * kStageElems * sizeof(bf16);

__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(GemmParams p, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16 *smem = reinterpret_cast<bf16 *>(smem_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int tn = blockIdx.x % tiles_n, tm = blockIdx.x / tiles_n;
  const int bz = blockIdx.y;
  const int m0 = tm * BM, n0 = tn * BN;

  const bf16 *A = p.A + (int64_t)bz * p.a_bs;
  const bf16 *W = p.W;

  // global -> register staging: 4 16-byte chunks of A and of W per thread
  uint4 ra[4], rw[4];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = tid + kThreads * r;
      const int row = c >> 3, kc = (c & 7) * 8;
      const int gm = m0 + row, gn = n0 + row;
      ra[r] = (gm < p.M) ? *reinterpret_cast<const uint4 *>(A + (int64_t)gm * p.lda + k0 + kc)
                         : make_uint4(0, 0, 0, 0);
      rw[r] = (gn < p.N) ? *reinterpret_cast<const uint4 *>(W + (int64_t)gn * p.ldw + k0 + kc)
                         : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&](int stage) {
    bf16 *sA = smem + stage * kStageElems;
    bf16 *sW = sA + BM * LROW;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = tid + kThreads * r;
      const int row = c >> 3, kc = (c & 7) * 8;
      *reinterpret_cast<uint4 *>(sA + row * LROW + kc) = ra[r];
      *reinterpret_cast<uint4 *>(sW + row * LROW + kc) = rw[r];
    }
  };

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int KT = p.K / BK;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < KT) load_tile((kt + 1) * BK);
    const bf16 *sA = smem + stage * kStageElems;
    const bf16 *sW = sA + BM * LROW;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8 *>(sA + (wm * 64 + i * 32 + l32) * LROW + s * 16 + hi * 8);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const bf16x8 *>(sW + (wn * 64 + j * 32 + l32) * LROW + s * 16 + hi * 8);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) store_tile(stage ^ 1);
    __syncthreads();
  }

  // Epilogue.  MFMA 32x32 output: lane holds column l32 and rows 8*(v/4) + 4*hi + v%4.
  const float *bias = p.bias ? p.bias + (int64_t)bz * p.bias_bs : nullptr;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = n0 + wn * 64 + j * 32 + l32;
    if (col >= p.N) continue;
    const float bcol = bias ? bias[col] : 0.f;
    if (col < p.n_split) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * hi + (v & 3);
          if (row < p.M) {
            const float val = acc[i][j][v] + bcol;
            const int64_t off = (int64_t)bz * p.c_bs + (int64_t)row * p.ldc + col;
            if (p.c_dt == 0)
              reinterpret_cast<bf16 *>(p.C)[off] = (bf16)val;
            else
              reinterpret_cast<float *>(p.C)[off] = val;
          }
        }
      }
    } else {
      const int cc = col - p.n_split;
      const int h = cc / p.dh, e = cc % p.dh;
      bf16 *vt = p.VT + (int64_t)bz * p.vt_bs + (int64_t)h * p.vt_hs + (int64_t)e * p.vt_rs;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int row = m0 + wm * 64 + i * 32 + 8 * g + 4 * hi;
          // rows in [M, vt_rows) read zero A rows: they store the zero padding
          if (row + 3 < p.vt_rows) {
            bf16x4 pk;
#pragma unroll
            for (int u = 0; u < 4; ++u) pk[u] = (bf16)(acc[i][j][4 * g + u] + bcol);
            *reinterpret_cast<bf16x4 *>(vt + row) = pk;
          } else {
#pragma unroll
            for (int u = 0; u < 4; ++u)
              if (row + u < p.vt_rows) vt[row + u] = (bf16)(acc[i][j][4 * g + u] + bcol);
          }
        }
      }
    }
  }
}

bool g_attr_set = false;

}  // namespace

hipError_t launch_gemm(const GemmParams &p, hipStream_t s) {
  if (p.M <= 0 || p.batch <= 0) return hipSuccess;
  if (!g_attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)gemm_bf16_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
    if (e != hipSuccess) return e;
    g_attr_set = true;
  }
  const int tiles_n = (p.N + BN - 1) / BN;
  const int tiles_m = (max(p.M, p.VT ? p.vt_rows : 0) + BM - 1) / BM;
  dim3 grid(tiles_n * tiles_m, p.batch);
  hipLaunchKernelGGL(gemm_bf16_kernel, grid, dim3(kThreads), kLdsBytes, s, p, tiles_n);
  return hipGetLastError();
}

}  // namespace t2va
