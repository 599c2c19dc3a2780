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

#include <type_traits>

namespace t2va {

namespace {

constexpr int BM = 128, BN = 128, BK = 64;

// One element of C at offset `off`: bf16, fp32, or a split pair (bf16(x) at
// off, bf16(x - bf16(x)) at off + n_split).
__device__ __forceinline__ void store_c(const GemmParams &p, int64_t off, float val) {
  if (p.c_dt == 0) {
    reinterpret_cast<bf16 *>(p.C)[off] = (bf16)val;
  } else if (p.c_dt == 1) {
    reinterpret_cast<float *>(p.C)[off] = val;
  } else {
    const bf16 hi = (bf16)val;
    reinterpret_cast<bf16 *>(p.C)[off] = hi;
    reinterpret_cast<bf16 *>(p.C)[off + p.n_split] = (bf16)(val - (float)hi);
  }
}
constexpr int LROW = BK + 8;  // padded LDS row (elements): 144 B, conflict-free 16-B reads
constexpr int kThreads = 256;
constexpr int kStageElems = (BM + BN) * LROW;
constexpr size_t kLdsBytes = 2 * kStageElems * sizeof(bf16);

// Output of a 128x128 tile held as 2x2 v_mfma_f32_32x32x16_bf16 results per
// wave (wave (wm, wn) owns rows wm*64.., columns wn*64..): bias, then the
// element stores of store_c, or columns past n_split dh-major into V^T.
__device__ __forceinline__ void small_epilogue(const GemmParams &p, int bz, int m0, int n0, int wm, int wn,
                                               int l32, int hi, const floatx16 (&acc)[2][2]) {
  // MFMA 32x32 output: lane holds column l32 and rows 8*(v/4) + 4*hi + v%4.
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
            store_c(p, off, val);
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
          // (V^T may start at any token: a vector store needs an aligned address)
          if (row + 3 < p.vt_rows && (((uintptr_t)(vt + row)) & 7) == 0) {
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

// Two independent problems can share one launch (the first tiles1 workgroups
// of each batch row run p1, the rest p2): a problem with few tiles then runs
// beside a larger one instead of after it.
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(GemmParams p1, GemmParams p2, int tiles_n1,
                                                             int tiles_n2, int tiles1) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16 *smem = reinterpret_cast<bf16 *>(smem_raw);

  const bool second = (int)blockIdx.x >= tiles1;
  const GemmParams &p = second ? p2 : p1;
  const int tiles_n = second ? tiles_n2 : tiles_n1;
  const int bx = second ? (int)blockIdx.x - tiles1 : (int)blockIdx.x;
  const int bz = blockIdx.y;
  if (bz >= p.batch) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int tn = bx % tiles_n, tm = bx / tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;

  const bf16 *A = p.A + (int64_t)bz * p.a_bs;
  const bf16 *W = p.W + (int64_t)bz * p.w_bs;

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

  small_epilogue(p, bz, m0, n0, wm, wn, l32, hi, acc);
}

// ---------------------------------------------------------------------------
// Large-tile variant for the wide projections (the fused QKV and the input
// projections): 256x256x64 tiles, 8 waves in 2x4, each wave 128x64 as 4x2
// tiles of v_mfma_f32_32x32x16_bf16 (or 4 waves of 128x128).  Every A fragment
// a wave reads from LDS feeds two MFMAs and every W fragment four, and two
// waves per SIMD hide one another's LDS and barrier waits.  Tiles go from global memory straight
// into LDS with buffer_load_dwordx4 ... lds: one instruction moves 8 rows x
// 128 B, its 16-byte chunks XOR-swizzled within each row (lslot below) so
// that operand reads are free of bank conflicts.  Rows past M (or N) lie past
// the buffer descriptor's end and load as zeros.
// ---------------------------------------------------------------------------
constexpr int LBM = 256, LBN = 256;
constexpr int kLStageElems = (LBM + LBN) * BK;                      // unpadded rows
constexpr int kEpiElems = 128 * 64;   // staged epilogue: one wave's 128x64 bf16 tile (16 KB)
constexpr size_t kLLdsBytes = 2 * kLStageElems * sizeof(bf16) > (size_t)8 * kEpiElems * sizeof(bf16)
                                  ? 2 * kLStageElems * sizeof(bf16)                 // 128 KB of stages
                                  : (size_t)8 * kEpiElems * sizeof(bf16);

typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource over [base, base + bytes) (loads past the end return zeros).
// Both arguments are wave-uniform; readfirstlane keeps the descriptor in SGPRs
// (a VGPR descriptor makes the compiler wrap each load in a waterfall loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemm_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(lo | (hi << 32)), (short)0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000);
}
// 16-byte slot of chunk c (of 8) of a 128-byte tile row.  A 32x32x16 operand
// read takes one chunk from 32 consecutive rows; with this XOR key any 8
// consecutive rows cover all 8 slots (distinct banks when the LDS serves 128 B
// per clock) and any 16 rows are distinct in (row parity, slot) (distinct
// banks at 256 B per clock).  The map is an involution.
__device__ __forceinline__ int lxor(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int lslot(int row, int c) { return c ^ lxor(row); }

// Staged epilogue layouts (per wave, 16 KB, no padding): 8-byte units (4 bf16)
// are XOR-swizzled within each line by a key of the line index, so that the
// 8-byte stores of 16 (or 32) consecutive lanes, one line each, hit distinct
// banks.  A 16-byte read of chunk c of a line then finds both of its halves in
// chunk c ^ (key >> 1), swapped when the key is odd.
__device__ __forceinline__ int ekey_row(int m) { return (m & 15) ^ ((m >> 4) & 1); }   // 16 units per line
__device__ __forceinline__ int ekey_col(int n) { return n & 31; }                       // 32 units per line
__device__ __forceinline__ bf16x8 read_chunk(const bf16 *line, int c, int key) {
  bf16x8 v = *reinterpret_cast<const bf16x8 *>(line + 8 * (c ^ (key >> 1)));
  if (key & 1) {
    bf16x8 w;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      w[u] = v[u + 4];
      w[u + 4] = v[u];
    }
    v = w;
  }
  return v;
}

#ifndef T2VA_GEMM_LARGE_WAVES
#define T2VA_GEMM_LARGE_WAVES 8
#endif
constexpr int kLWaves = T2VA_GEMM_LARGE_WAVES;        // 4 (2x2 of 128x128) or 8 (2x4 of 128x64)
constexpr int kLThreads = 64 * kLWaves;
constexpr int kLJ = kLWaves == 4 ? 4 : 2;             // 32-column tiles per wave
constexpr int kLGroups = 32 / kLWaves;                // 8-row load groups per wave and operand

// One workgroup per CU (its LDS), so two waves per SIMD: the register budget is
// 256 per wave, which the fragment double buffer below uses.
__global__ __launch_bounds__(kLThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_bf16_large_kernel(GemmParams p, int tiles_n,
                                                                     int tiles_m) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16 *smem = reinterpret_cast<bf16 *>(smem_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int wm = kLWaves == 4 ? wave >> 1 : wave >> 2;
  const int wn = kLWaves == 4 ? wave & 1 : wave & 3;
  // Hardware places workgroup w on XCD w % 8, and each XCD has its own L2:
  // give each XCD a contiguous range of logical tiles (batch-major), so the
  // tiles an XCD runs at once form a compact block.  Logical order within a
  // batch: column-tile-major within bands of 8 row tiles, so 32 consecutive
  // tiles are 8 row tiles x 4 column tiles sharing their A and W slices in L2.
  const int tiles = tiles_n * tiles_m;
  const int total = tiles * p.batch;
  const int per_xcd = (total + 7) / 8;
  const int L = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (L >= total) return;
  const int bz = L / tiles;
  const int bid = L - bz * tiles;
  const int group = bid / (8 * tiles_n);
  const int first_m = group * 8;
  const int gsize = min(tiles_m - first_m, 8);
  const int tm = first_m + (bid % (8 * tiles_n)) % gsize;
  const int tn = (bid % (8 * tiles_n)) / gsize;
  const int m0 = tm * LBM, n0 = tn * LBN;

  // descriptors end after the last valid row: rows >= M (N) read zeros
  const int m_rows = max(min(p.M - m0, LBM), 0), n_rows = max(min(p.N - n0, LBN), 0);
  const bf16 *A = p.A + (int64_t)bz * p.a_bs + (int64_t)m0 * p.lda;
  const bf16 *W = p.W + (int64_t)bz * p.w_bs + (int64_t)n0 * p.ldw;
  const __amdgpu_buffer_rsrc_t rA = gemm_rsrc(A, (uint32_t)(m_rows > 0 ? ((int64_t)(m_rows - 1) * p.lda + p.K) * 2 : 0));
  const __amdgpu_buffer_rsrc_t rW = gemm_rsrc(W, (uint32_t)(n_rows > 0 ? ((int64_t)(n_rows - 1) * p.ldw + p.K) * 2 : 0));

  // each wave loads kLGroups of the 32 row groups (8 rows each) of A and of W per stage
  uint32_t aoff[kLGroups], woff[kLGroups];
#pragma unroll
  for (int r = 0; r < kLGroups; ++r) {
    const int grp = wave * kLGroups + r;
    const int row = grp * 8 + (lane >> 3);
    const int c = lslot(row, lane & 7);          // the slot map is an involution
    aoff[r] = (uint32_t)((row * p.lda + 8 * c) * 2);
    woff[r] = (uint32_t)((row * p.ldw + 8 * c) * 2);
  }
  auto issue = [&](int stage, int k0) {
    bf16 *sA = smem + stage * kLStageElems;
    bf16 *sW = sA + LBM * BK;
    const uint32_t kb = (uint32_t)(k0 * 2);
#pragma unroll
    for (int r = 0; r < kLGroups; ++r) {
      const int grp = wave * kLGroups + r;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void *)(sA + grp * 512), 16, aoff[r] + kb, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rW, (lds_void *)(sW + grp * 512), 16, woff[r] + kb, 0, 0, 0);
    }
  };

  // fragment read offsets (elements) for k-step s: row R, chunk 2 s + hi
  int abase[4], wbase[kLJ], ax[4], wx[kLJ];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ra = wm * 128 + i * 32 + l32;
    abase[i] = ra * BK;
    ax[i] = lxor(ra);
  }
#pragma unroll
  for (int j = 0; j < kLJ; ++j) {
    const int rw = wn * 32 * kLJ + j * 32 + l32;
    wbase[j] = rw * BK;
    wx[j] = lxor(rw);
  }

  floatx16 acc[4][kLJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kLJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // bf16 tiles staged through LDS on the way out (8 waves): row-major outputs
  // take the product transposed (W fragments as the A operand), so that a lane
  // holds one output row and four consecutive columns per register group;
  // V^T outputs keep the plain order (a lane holds one column, runs of rows).
  const int wcol0 = n0 + wn * 32 * kLJ, wrow0 = m0 + wm * 128;
  // (split outputs c_dt = 2 stage their hi and lo parts one after the other)
  const bool staged = kLWaves == 8 && (p.c_dt == 0 || p.c_dt == 2) && (p.n_split % 64 == 0 || p.n_split >= p.N);
  const bool rowmajor = staged && wcol0 < p.n_split;

  const int KT = p.K / BK;
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (KT > 1) issue(1, BK);
  // Two LDS stages, one barrier per k-tile, placed before the tile's last
  // k-step: that step's fragments are already in registers, so after the
  // barrier (which publishes tile kt+1 and frees tile kt's stage for tile kt+2)
  // the first fragments of tile kt+1 are read while the last MFMAs of tile kt
  // run, and no k-tile starts by waiting for an LDS read.
  auto main_loop = [&](auto order) {
  constexpr bool kSwap = decltype(order)::value;
  bf16x8 a[2][4], b[2][kLJ];
  auto read_frags = [&](const bf16 *sA, int s, int x) {
    const bf16 *sW = sA + LBM * BK;
    const int c = 2 * s + hi;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[x][i] = *reinterpret_cast<const bf16x8 *>(sA + abase[i] + 8 * (c ^ ax[i]));
#pragma unroll
    for (int j = 0; j < kLJ; ++j) b[x][j] = *reinterpret_cast<const bf16x8 *>(sW + wbase[j] + 8 * (c ^ wx[j]));
  };
  static_assert((BK / 16) % 2 == 0, "the next tile's first fragments go to register set 0");
  read_frags(smem, 0, 0);
  for (int kt = 0; kt < KT; ++kt) {
    const int stage = kt & 1;
    const bf16 *sA = smem + stage * kLStageElems;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      if (s + 1 < BK / 16) {
        // fragments of k-step s+1 are read while the MFMAs of k-step s run
        read_frags(sA, s + 1, (s + 1) & 1);
      } else {
        // this wave's loads of tile kt+1 have landed and every wave has read
        // its last fragments of tile kt
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (kt + 1 < KT) read_frags(smem + (stage ^ 1) * kLStageElems, 0, 0);
      }
      // keep the reads ahead of this k-step's MFMAs (the scheduler would
      // otherwise sink each read next to its first use)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < kLJ; ++j)
          acc[i][j] = kSwap ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[s & 1][j], a[s & 1][i], acc[i][j], 0, 0, 0)
                            : __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s & 1][i], b[s & 1][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      // tile kt+2 into the stage every wave has finished reading, issued
      // behind the last k-step's MFMAs
      if (s + 1 == BK / 16 && kt + 2 < KT) issue(stage, (kt + 2) * BK);
    }
  }
  };
  if (rowmajor) main_loop(std::true_type{});
  else main_loop(std::false_type{});

  // Epilogue.  MFMA 32x32 output: lane holds column l32 and rows 8*(v/4) + 4*hi + v%4
  // of each 32x32 tile (with the transposed product: row l32, columns 8*(v/4) + 4*hi + v%4).
  const float *bias = p.bias ? p.bias + (int64_t)bz * p.bias_bs : nullptr;
  if (staged) {
    // LDS is free after the main loop's last barrier; each wave stages its own
    // 128x64 tile and writes it out in 16-byte chunks
    bf16 *st = smem + wave * kEpiElems;
    if (rowmajor) {
      // pass 0: the values (split: their bf16 hi parts); pass 1 (split only):
      // the lo parts bf16(x - hi), n_split columns further along the row
      for (int pass = 0; pass < (p.c_dt == 2 ? 2 : 1); ++pass) {
      // the wave's lanes exchange values through its own LDS tile: keep the
      // compiler from moving one lane's stores across another lane's loads
      __builtin_amdgcn_wave_barrier();
      // [128 rows][64 columns]: row m = 32 i + l32; unit 8 j + 2 k + hi holds
      // columns 32 j + 8 k + 4 hi .. + 3
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = i * 32 + l32, key = ekey_row(m);
#pragma unroll
        for (int j = 0; j < kLJ; ++j)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int c0 = j * 32 + 8 * k + 4 * hi;
            bf16x4 pk;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const float bc = (bias && wcol0 + c0 + u < p.N) ? bias[wcol0 + c0 + u] : 0.f;
              const float x = acc[i][j][4 * k + u] + bc;
              pk[u] = pass == 0 ? (bf16)x : (bf16)(x - (float)(bf16)x);
            }
            *reinterpret_cast<bf16x4 *>(st + m * 64 + 4 * ((8 * j + 2 * k + hi) ^ key)) = pk;
          }
      }
      __builtin_amdgcn_wave_barrier();
      // chunk q = row q / 8, columns 8 (q % 8) .. + 7
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int q = lane + 64 * k;
        const int r = q >> 3, c = q & 7;
        const int row = wrow0 + r, col = wcol0 + 8 * c;
        if (row >= p.M || col >= p.N) continue;
        const bf16x8 v = read_chunk(st + r * 64, c, ekey_row(r));
        bf16 *dst = reinterpret_cast<bf16 *>(p.C) + (int64_t)bz * p.c_bs + (int64_t)row * p.ldc + col +
                    (pass ? p.n_split : 0);
        if (col + 8 <= p.N && ((p.ldc | col | (pass ? p.n_split : 0)) & 7) == 0) {
          *reinterpret_cast<bf16x8 *>(dst) = v;
        } else {
          for (int u = 0; u < 8; ++u)
            if (col + u < p.N) dst[u] = v[u];
        }
      }
      }
    } else {
      // V^T, [64 columns][128 rows]: column n = 32 j + l32; unit 8 i + 2 g + hi
      // holds rows 32 i + 8 g + 4 hi .. + 3
#pragma unroll
      for (int j = 0; j < kLJ; ++j) {
        const int cl = j * 32 + l32, key = ekey_col(cl);
        const float bcol = (bias && wcol0 + cl < p.N) ? bias[wcol0 + cl] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            bf16x4 pk;
#pragma unroll
            for (int u = 0; u < 4; ++u) pk[u] = (bf16)(acc[i][j][4 * g + u] + bcol);
            *reinterpret_cast<bf16x4 *>(st + cl * 128 + 4 * ((8 * i + 2 * g + hi) ^ key)) = pk;
          }
      }
      // chunk q = column q / 16, tokens 8 (q % 16) .. + 7
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int q = lane + 64 * k;
        const int c = q >> 4, rc = q & 15;
        const int col = wcol0 + c, row = wrow0 + 8 * rc;
        if (col >= p.N || row >= p.vt_rows) continue;
        const bf16x8 v = read_chunk(st + c * 128, rc, ekey_col(c));
        const int cc = col - p.n_split;
        bf16 *vt = p.VT + (int64_t)bz * p.vt_bs + (int64_t)(cc / p.dh) * p.vt_hs + (int64_t)(cc % p.dh) * p.vt_rs;
        if (row + 8 <= p.vt_rows && (((uintptr_t)(vt + row)) & 15) == 0) {
          *reinterpret_cast<bf16x8 *>(vt + row) = v;
        } else {
          for (int u = 0; u < 8; ++u)
            if (row + u < p.vt_rows) vt[row + u] = v[u];
        }
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < kLJ; ++j) {
    const int col = n0 + wn * 32 * kLJ + j * 32 + l32;
    if (col >= p.N) continue;
    const float bcol = bias ? bias[col] : 0.f;
    if (col < p.n_split) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = m0 + wm * 128 + i * 32 + 8 * (v >> 2) + 4 * hi + (v & 3);
          if (row < p.M) {
            const float val = acc[i][j][v] + bcol;
            const int64_t off = (int64_t)bz * p.c_bs + (int64_t)row * p.ldc + col;
            store_c(p, off, val);
          }
        }
      }
    } else {
      const int cc = col - p.n_split;
      const int h = cc / p.dh, e = cc % p.dh;
      bf16 *vt = p.VT + (int64_t)bz * p.vt_bs + (int64_t)h * p.vt_hs + (int64_t)e * p.vt_rs;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int row = m0 + wm * 128 + i * 32 + 8 * g + 4 * hi;
          // rows in [M, vt_rows) read zero A rows: they store the zero padding
          // (V^T may start at any token: a vector store needs an aligned address)
          if (row + 3 < p.vt_rows && (((uintptr_t)(vt + row)) & 7) == 0) {
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

bool g_attr_set = false, g_lattr_set = false;


// ---------------------------------------------------------------------------
// 128x128 tiles with a deep direct-to-LDS ring, for products with long K and
// few tiles (the output projections, K = d; the text rows' QKV; the weight
// fold).  With the tile held one k-step ahead in registers (the kernel above)
// such launches wait on memory most of the time: a workgroup's loads of the
// next k-tile take longer than its MFMAs on the current one.  Here the operand
// tiles go straight into a ring of kRing LDS stages, kRing - 1 k-tiles in
// flight, in the 256x256 kernel's layout (unpadded 128-byte rows, 16-byte
// chunks XOR-swizzled by lslot; rows past M or N lie past the descriptor's end
// and read zeros).  4 waves of 64x64 as 2x2 v_mfma_f32_32x32x16_bf16 tiles;
// output through small_epilogue.
// ---------------------------------------------------------------------------
// Workgroup barrier for the ring: a fence (as in __syncthreads()) would wait
// for every load in flight, since the ring's loads write LDS; each wave has
// already waited for its own loads of the tile it is about to read, so only
// the compiler must keep memory accesses on their side of the barrier.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

constexpr int kRing = 4;
constexpr int kRStageElems = (BM + BN) * BK;                                  // 32 KB
constexpr size_t kRLdsBytes = (size_t)kRing * kRStageElems * sizeof(bf16);   // 128 KB
constexpr int kRGroups = BM / 8 / (kThreads / 64);   // 8-row chunks per wave and operand: 4

// s_waitcnt with the vector-memory count n (0..63) and the other counters
// left alone (expcnt 7, lgkmcnt 15)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__global__ __launch_bounds__(kThreads) void gemm_bf16_ring_kernel(GemmParams p1, GemmParams p2, int tiles_n1,
                                                                  int tiles_n2, int tiles1) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16 *smem = reinterpret_cast<bf16 *>(smem_raw);

  const bool second = (int)blockIdx.x >= tiles1;
  const GemmParams &p = second ? p2 : p1;
  const int tiles_n = second ? tiles_n2 : tiles_n1;
  const int bx = second ? (int)blockIdx.x - tiles1 : (int)blockIdx.x;
  const int bz = blockIdx.y;
  if (bz >= p.batch) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int tn = bx % tiles_n, tm = bx / tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;

  const int m_rows = max(min(p.M - m0, BM), 0), n_rows = max(min(p.N - n0, BN), 0);
  const bf16 *A = p.A + (int64_t)bz * p.a_bs + (int64_t)m0 * p.lda;
  const bf16 *W = p.W + (int64_t)bz * p.w_bs + (int64_t)n0 * p.ldw;
  const __amdgpu_buffer_rsrc_t rA =
      gemm_rsrc(A, (uint32_t)(m_rows > 0 ? ((int64_t)(m_rows - 1) * p.lda + p.K) * 2 : 0));
  const __amdgpu_buffer_rsrc_t rW =
      gemm_rsrc(W, (uint32_t)(n_rows > 0 ? ((int64_t)(n_rows - 1) * p.ldw + p.K) * 2 : 0));

  // wave w moves the 8-row chunks w*kRGroups .. of A and of W of each stage
  uint32_t aoff[kRGroups], woff[kRGroups];
#pragma unroll
  for (int r = 0; r < kRGroups; ++r) {
    const int row = (wave * kRGroups + r) * 8 + (lane >> 3);
    const int c = lslot(row, lane & 7);   // the slot map is an involution
    aoff[r] = (uint32_t)((row * p.lda + 8 * c) * 2);
    woff[r] = (uint32_t)((row * p.ldw + 8 * c) * 2);
  }
  auto issue = [&](int stage, int k0) {
    bf16 *sA = smem + stage * kRStageElems;
    bf16 *sW = sA + BM * BK;
    const uint32_t kb = (uint32_t)(k0 * 2);
#pragma unroll
    for (int r = 0; r < kRGroups; ++r) {
      const int grp = wave * kRGroups + r;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void *)(sA + grp * 512), 16, aoff[r] + kb, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rW, (lds_void *)(sW + grp * 512), 16, woff[r] + kb, 0, 0, 0);
    }
  };
  // fragment rows and their swizzle keys
  int abase[2], wbase[2], ax[2], wx[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ra = wm * 64 + i * 32 + l32, rw = wn * 64 + i * 32 + l32;
    abase[i] = ra * BK;
    ax[i] = lxor(ra);
    wbase[i] = rw * BK;
    wx[i] = lxor(rw);
  }

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int KT = p.K / BK;
#pragma unroll
  for (int t = 0; t < kRing - 1; ++t)
    if (t < KT) issue(t, t * BK);
  for (int kt = 0; kt < KT; ++kt) {
    // this wave's loads of tile kt have landed once at most the loads of the
    // tiles issued after it (up to kRing - 2 of them, 2 kRGroups each) remain
    const int newer = min(KT - 1 - kt, kRing - 2);
    static_assert(kRing == 4, "the waits below count up to two newer tiles");
    if (newer >= 2) wait_vm<4 * kRGroups>();
    else if (newer == 1) wait_vm<2 * kRGroups>();
    else wait_vm<0>();
    // every wave's tile kt is in LDS, and every wave is done reading tile
    // kt - 1, whose stage the tile kRing - 1 ahead now takes
    ring_barrier();
    if (kt + kRing - 1 < KT) issue((kt + kRing - 1) % kRing, (kt + kRing - 1) * BK);
    const bf16 *sA = smem + (kt % kRing) * kRStageElems;
    const bf16 *sW = sA + BM * BK;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int c = 2 * s + hi;
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = *reinterpret_cast<const bf16x8 *>(sA + abase[i] + 8 * (c ^ ax[i]));
        b[i] = *reinterpret_cast<const bf16x8 *>(sW + wbase[i] + 8 * (c ^ wx[i]));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
  small_epilogue(p, bz, m0, n0, wm, wn, l32, hi, acc);
}

}  // namespace

namespace {
// the large tile for wide outputs with many rows; per-(batch, tile) byte
// extents must fit the 32-bit buffer descriptors
// The 256x256 tiles for wide outputs with many rows: 2048 rows per problem, or
// a batch of at least 2048 rows in all whose row tiles are at least 80 % full.
bool use_large(const GemmParams &p) {
  const int rows = max(p.M, p.VT ? p.vt_rows : 0);
  const int64_t padded = (int64_t)(rows + LBM - 1) / LBM * LBM;
  const bool many = rows >= 2048 || ((int64_t)rows * p.batch >= 2048 && 5 * (int64_t)rows >= 4 * padded);
  return p.N >= 1024 && many && (int64_t)LBM * p.lda * 2 < ((int64_t)1 << 31) &&
         (int64_t)LBN * p.ldw * 2 < ((int64_t)1 << 31);
}
// The ring kernel for long K (at least 8 k-tiles) when the launch has few
// workgroups (its 128 KB of LDS allow one per CU); 32-bit tile offsets.
bool use_ring(const GemmParams &p) {
  const int64_t tiles = (int64_t)((p.N + BN - 1) / BN) * ((max(p.M, p.VT ? p.vt_rows : 0) + BM - 1) / BM);
  return p.K >= 8 * BK && tiles * p.batch <= 1024;
}
bool tile_offsets_fit(const GemmParams &p) {
  return (int64_t)BM * max(p.lda, p.ldw) * 2 < ((int64_t)1 << 31);
}
hipError_t set_ring_attr() {
  static bool done = false;
  if (!done) {
    hipError_t e = hipFuncSetAttribute((const void *)gemm_bf16_ring_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kRLdsBytes);
    if (e != hipSuccess) return e;
    done = true;
  }
  return hipSuccess;
}
int small_tiles(const GemmParams &p) {
  return ((p.N + BN - 1) / BN) * ((max(p.M, p.VT ? p.vt_rows : 0) + BM - 1) / BM);
}
hipError_t set_small_attr() {
  if (!g_attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)gemm_bf16_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
    if (e != hipSuccess) return e;
    g_attr_set = true;
  }
  return hipSuccess;
}
}  // namespace

hipError_t launch_gemm(const GemmParams &p, hipStream_t s) {
  // M = 0 still writes the V^T padding rows [0, vt_rows) as zeros
  if ((p.M <= 0 && !(p.VT && p.vt_rows > 0)) || p.batch <= 0) return hipSuccess;
  const int rows = max(p.M, p.VT ? p.vt_rows : 0);
  if (use_large(p)) {
    if (!g_lattr_set) {
      hipError_t e = hipFuncSetAttribute((const void *)gemm_bf16_large_kernel,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLLdsBytes);
      if (e != hipSuccess) return e;
      g_lattr_set = true;
    }
    const int tiles_n = (p.N + LBN - 1) / LBN;
    const int tiles_m = (rows + LBM - 1) / LBM;
    const int64_t total = (int64_t)tiles_n * tiles_m * p.batch;
    hipLaunchKernelGGL(gemm_bf16_large_kernel, dim3((unsigned)((total + 7) / 8 * 8)), dim3(kLThreads), kLLdsBytes,
                       s, p, tiles_n, tiles_m);
    return hipGetLastError();
  }
  const int tiles_n = (p.N + BN - 1) / BN;
  const int tiles = small_tiles(p);
  if (use_ring(p) && tile_offsets_fit(p)) {
    if (hipError_t e = set_ring_attr()) return e;
    hipLaunchKernelGGL(gemm_bf16_ring_kernel, dim3(tiles, p.batch), dim3(kThreads), kRLdsBytes, s, p, p, tiles_n,
                       tiles_n, tiles);
    return hipGetLastError();
  }
  if (hipError_t e = set_small_attr()) return e;
  hipLaunchKernelGGL(gemm_bf16_kernel, dim3(tiles, p.batch), dim3(kThreads), kLdsBytes, s, p, p, tiles_n, tiles_n,
                     tiles);
  return hipGetLastError();
}

hipError_t launch_gemm_pair(const GemmParams &a, const GemmParams &b, hipStream_t s) {
  const bool a_on = a.M > 0 && a.batch > 0, b_on = b.M > 0 && b.batch > 0;
  if (!a_on || !b_on || use_large(a) || use_large(b)) {
    if (hipError_t e = launch_gemm(a, s)) return e;
    return launch_gemm(b, s);
  }
  const int ta = small_tiles(a);
  if ((use_ring(a) || use_ring(b)) && tile_offsets_fit(a) && tile_offsets_fit(b)) {
    if (hipError_t e = set_ring_attr()) return e;
    hipLaunchKernelGGL(gemm_bf16_ring_kernel, dim3(ta + small_tiles(b), max(a.batch, b.batch)), dim3(kThreads),
                       kRLdsBytes, s, a, b, (a.N + BN - 1) / BN, (b.N + BN - 1) / BN, ta);
    return hipGetLastError();
  }
  if (hipError_t e = set_small_attr()) return e;
  hipLaunchKernelGGL(gemm_bf16_kernel, dim3(ta + small_tiles(b), max(a.batch, b.batch)), dim3(kThreads),
                     kLdsBytes, s, a, b, (a.N + BN - 1) / BN, (b.N + BN - 1) / BN, ta);
  return hipGetLastError();
}

}  // namespace t2va
