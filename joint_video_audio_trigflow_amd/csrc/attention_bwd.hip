// Joint attention backward on bf16 MFMA (gfx950), for the training backward of
// the joint sCM loss: the loss reaches the student's weights only through its
// primal forward pass (the target gbar is under stop-gradient; deep read of
// TurboT2VA, section 3.1), so the attention backward is the ordinary one of
// the primal softmax attention:
//   P = softmax(scale Q K^T) (keys >= nk[b] excluded), dP = dO V^T,
//   dS = P * (dP - D) with D_i = sum_e dO_ie O_ie,
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
// P is recomputed from the forward's log-sum-exp (log2 units), so no running
// max is needed.  Two kernels, both deterministic (no atomics):
//
// * dQ: a wave owns two blocks of 16 query rows and streams key tiles; in
//   registers it keeps Q and dO as B operands; per 32-key sub-tile it forms S^T = K Q^T and
//   dP^T = V dO^T (A: K and V rows from LDS, read in the permuted row order
//   that makes the 8 values a lane holds the 8 keys of its B operand), then
//   dQ^T += K^T dS^T (A: K^T rows from LDS, B: dS^T from registers).
// * dK/dV: a wave (12 per workgroup) owns 16 keys and streams query tiles; in registers it keeps
//   K and V as B operands; per 32-query sub-tile it forms S = Q K^T and
//   dP = dO V^T (A: Q and dO rows from LDS, permuted), then
//   dV^T += dO^T P and dK^T += Q^T dS (A: dO^T and Q^T rows from LDS).
//
// Each kernel therefore reads its streamed operand in both layouts (rows for
// the contraction over the head dimension, transposed for the contraction over
// tokens); the transposed copies are written beforehand by a transpose kernel.
// Tiles go straight from global memory into LDS (buffer_load ... lds),
// double-buffered in 64-token stages, with the swizzles of attn_tiles.h.
#include "attn_tiles.h"
#include "common.h"

#include <algorithm>

#include <math.h>

namespace t2va {

namespace {

#ifndef T2VA_BWD_WAVES_DQ
#define T2VA_BWD_WAVES_DQ 8
#endif
#ifndef T2VA_BWD_WAVES_DKV
#define T2VA_BWD_WAVES_DKV 12
#endif
#ifndef T2VA_BWD_MB_DQ
#define T2VA_BWD_MB_DQ 2
#endif
#ifndef T2VA_BWD_MB_DKV
#define T2VA_BWD_MB_DKV 1
#endif
constexpr int BT = 64;   // streamed tokens per LDS stage

template <int DH>
struct BwdCfg {
  static constexpr int NW_DQ = T2VA_BWD_WAVES_DQ, NW_DKV = T2VA_BWD_WAVES_DKV;
  static constexpr int THREADS_DQ = 64 * NW_DQ, THREADS_DKV = 64 * NW_DKV;
  // blocks of 16 rows per wave (queries for dQ, keys for dK/dV): every
  // fragment a wave reads from LDS feeds MB MFMAs
  static constexpr int MB_DQ = T2VA_BWD_MB_DQ, MB_DKV = T2VA_BWD_MB_DKV;
  static constexpr int BW_DQ = 16 * MB_DQ * NW_DQ;     // queries per dQ workgroup
  static constexpr int BW_DKV = 16 * MB_DKV * NW_DKV;  // keys per dK/dV workgroup
  static constexpr int KSTEPS = DH / 32;
  static constexpr int DT = DH / 16;
  static constexpr int CPR = DH / 8;
  static constexpr int ROW_ELEMS = BT * DH;   // row tile [BT][DH]
  static constexpr int T_ELEMS = DH * BT;     // transposed tile [DH][BT]
  // waves that issue a stage's LDS loads (at most 8)
  static constexpr int LD_DQ = NW_DQ < 8 ? NW_DQ : 8, LD_DKV = NW_DKV < 8 ? NW_DKV : 8;
  static constexpr int ROWS_PER_CHUNK = 512 / DH;
  // dQ stage: K rows, V rows, K^T; dK/dV stage: Q rows, dO rows, Q^T, dO^T, lse2, D
  static constexpr int DQ_STAGE = 2 * ROW_ELEMS + T_ELEMS;
  static constexpr int DKV_STAGE = 2 * ROW_ELEMS + 2 * T_ELEMS + 2 * BT * 2;  // + 2 x 64 floats
  static constexpr size_t DQ_LDS = (size_t)2 * DQ_STAGE * sizeof(bf16);
  static constexpr size_t DKV_LDS = (size_t)2 * DKV_STAGE * sizeof(bf16);
  // partial results of one piece of a split tile (floats): for each row of
  // the tile and lane group g (index 4 row + g), the lane's four columns of
  // each d-tile, already scaled; dK/dV: the dK part, then the dV part
  static constexpr int PIECE_DQ = 4 * MB_DQ * DT * THREADS_DQ;
  static constexpr int PIECE_DKV_HALF = 4 * MB_DKV * DT * THREADS_DKV;
  static constexpr int PIECE_DKV = 2 * PIECE_DKV_HALF;
};

// Per-lane byte offsets (at token 0) of the chunks loading wave lw of LD moves
// into a row tile / a transposed tile; chunk j of the tile holds 512 elements.
template <int DH, int LD>
struct TileOffsets {
  using C = BwdCfg<DH>;
  static constexpr int RCH = C::ROW_ELEMS / 512 / LD, TCH = C::T_ELEMS / 512 / LD;
  static_assert(RCH * LD * 512 == C::ROW_ELEMS && TCH * LD * 512 == C::T_ELEMS, "whole chunks per loader");
  uint32_t row[RCH], tr[TCH];
  __device__ void init(int lw, int lane, int64_t rs, int64_t trs) {
#pragma unroll
    for (int r = 0; r < RCH; ++r) {
      const int chunk = lw + LD * r;
      const int rr = chunk * C::ROWS_PER_CHUNK + lane / C::CPR;
      const int c = kslot<C::CPR>(rr, lane % C::CPR);
      row[r] = (uint32_t)((rr * rs + 8 * c) * 2);
    }
#pragma unroll
    for (int r = 0; r < TCH; ++r) {
      const int chunk = lw + LD * r;
      const int e = chunk * 8 + lane / 8;
      tr[r] = (uint32_t)((e * trs + 8 * vslot(e, lane % 8)) * 2);
    }
  }
};

// A-operand read offsets (elements) of a row tile: half t, k-step s of a
// 32-row sub-tile (add 32 * DH per sub-tile); rows in the order 8(i/4)+4t+i%4.
template <int DH>
struct RowReader {
  int base[2], xs[2];
  __device__ void init(int l16, int g) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = 8 * (l16 >> 2) + 4 * t + (l16 & 3);
      const int x = kslot<DH / 8>(row, 0);
      base[t] = row * DH + 8 * (g ^ (x & 3));
      xs[t] = x >> 2;
    }
  }
  __device__ int off(int u, int t, int s) const { return 32 * u * DH + base[t] + 32 * (s ^ xs[t]); }
};

// A-operand read offsets of a transposed tile: row e = 16 et + l16, token
// chunk g of 32-token sub-tile u.
struct TrReader {
  int base[2];
  __device__ void init(int l16, int g) {
#pragma unroll
    for (int u = 0; u < 2; ++u) base[u] = l16 * BT + 8 * vslot(l16, 4 * u + g);
  }
  __device__ int off(int u, int et) const { return base[u] + 16 * et * BT; }
};

// Eight consecutive floats from each of two LDS rows (16-byte aligned).  The
// reads are plain ds_read_b128 written out, with their wait in the same
// block: left to the compiler, a read of LDS that buffer-to-LDS loads also
// write gets an s_waitcnt vmcnt(0) in front, which would make every sub-tile
// wait for the next stage's prefetch (these rows were published by the
// stage's barrier; the loads in flight target the other stage buffer).
__device__ __forceinline__ void read_stage_stats(const float *a, const float *b, float4 &a0, float4 &a1,
                                                 float4 &b0, float4 &b1) {
  typedef __attribute__((address_space(3))) const float lds_float;
  const uint32_t pa = (uint32_t)(uintptr_t)(lds_float *)a, pb = (uint32_t)(uintptr_t)(lds_float *)b;
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:16\n\t"
      "ds_read_b128 %2, %5\n\t"
      "ds_read_b128 %3, %5 offset:16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a0), "=&v"(a1), "=&v"(b0), "=&v"(b1)
      : "v"(pa), "v"(pb)
      : "memory");
}


// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__((BwdCfg<DH>::THREADS_DQ), 1) void attn_bwd_dq_kernel(AttnBwdParams p, int nqb,
                                                                              int per_xcd, int total, SplitArgs sp) {
  using C = BwdCfg<DH>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16 *const lds = reinterpret_cast<bf16 *>(smem_raw);
  auto sK = [&](int buf) { return lds + buf * C::DQ_STAGE; };
  auto sV = [&](int buf) { return lds + buf * C::DQ_STAGE + C::ROW_ELEMS; };
  auto sKT = [&](int buf) { return lds + buf * C::DQ_STAGE + 2 * C::ROW_ELEMS; };

  // XCD-aware order; a split tile's pieces cover consecutive key stages
  const SplitItem it = split_item(blockIdx.x, per_xcd, sp);
  if (it.L >= total) return;
  const int qb = it.L % nqb, bh = it.L / nqb;
  const int b = bh / p.H, h = bh % p.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  constexpr int MB = C::MB_DQ;
  const int q_row0 = qb * C::BW_DQ + wave * 16 * MB + l16;   // + 16 mb for row block mb
  const int nk_b = min(max(p.nk[b], 1), p.Nk);
  // this workgroup's keys [key0, key0 + nk)
  int key0 = 0, nk = nk_b;
  float *part = nullptr;
  if (it.slot >= 0) {
    int s0, s1;
    piece_stages((nk_b + BT - 1) / BT, it.piece, sp.k, s0, s1);
    key0 = s0 * BT;
    nk = min(nk_b, s1 * BT) - key0;
    part = p.part + (size_t)(it.slot * sp.k + it.piece) * C::PIECE_DQ;
  }
  if (nk <= 0) {   // an empty piece (a sample shorter than the longest) adds zero
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int pi = 4 * (q_row0 + 16 * mb - qb * C::BW_DQ) + g;
#pragma unroll
      for (int e = 0; e < C::DT; ++e)
        *reinterpret_cast<float4 *>(part + 4 * (e * MB * C::THREADS_DQ + pi)) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    return;
  }
  const float c_log2 = p.scale * 1.4426950408889634f;

  bf16x8 qf[MB][C::KSTEPS], dof[MB][C::KSTEPS];
  float lse2[MB], Dq[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int q_ld = min(q_row0 + 16 * mb, p.Nq - 1);
    const bf16 *qp = p.q + (int64_t)b * p.q_bs + (int64_t)q_ld * p.q_rs + h * DH + 8 * g;
    const bf16 *dp = p.dout + (int64_t)b * p.do_bs + (int64_t)q_ld * p.do_rs + h * DH + 8 * g;
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) {
      qf[mb][s] = *reinterpret_cast<const bf16x8 *>(qp + 32 * s);
      dof[mb][s] = *reinterpret_cast<const bf16x8 *>(dp + 32 * s);
    }
    const int64_t sidx = ((int64_t)b * p.H + h) * p.Nq + q_ld;
    lse2[mb] = p.lse2[sidx];
    Dq[mb] = p.D[sidx];
  }

  // Descriptors start at key key0.  K and V row descriptors end after key
  // row nk-1 (rows past it load as zeros); K^T columns past nk hold finite
  // values (zeros or padded text keys) and meet zero weights.
  const uint32_t k_bytes = (uint32_t)(((int64_t)(nk - 1) * p.k_rs + DH) * 2);
  const uint32_t v_bytes = (uint32_t)(((int64_t)(nk - 1) * p.v_rs + DH) * 2);
  const uint32_t kt_bytes = (uint32_t)(((int64_t)DH * p.kt_rs - key0) * 2);
  const __amdgpu_buffer_rsrc_t rK = make_rsrc(p.k + (int64_t)b * p.k_bs + (int64_t)key0 * p.k_rs + h * DH, k_bytes);
  const __amdgpu_buffer_rsrc_t rV = make_rsrc(p.v + (int64_t)b * p.v_bs + (int64_t)key0 * p.v_rs + h * DH, v_bytes);
  const __amdgpu_buffer_rsrc_t rKT =
      make_rsrc(p.kt + (int64_t)b * p.kt_bs + (int64_t)h * p.kt_hs + key0, kt_bytes);
  constexpr int LD = C::LD_DQ;
  using TO = TileOffsets<DH, LD>;
  const int lw = wave % LD;
  const bool loader = wave < LD;
  TO ko, vo;
  ko.init(lw, lane, p.k_rs, p.kt_rs);
  vo.init(lw, lane, p.v_rs, p.kt_rs);
  auto issue = [&](int buf, int k0) {
    if (!loader) return;
    const uint32_t kst = (uint32_t)(k0 * p.k_rs * 2), vst = (uint32_t)(k0 * p.v_rs * 2), tst = (uint32_t)(k0 * 2);
#pragma unroll
    for (int r = 0; r < TO::RCH; ++r) {
      const int chunk = lw + LD * r;
      load_lds16(rK, ko.row[r] + kst, sK(buf) + chunk * 512);
      load_lds16(rV, vo.row[r] + vst, sV(buf) + chunk * 512);
    }
#pragma unroll
    for (int r = 0; r < TO::TCH; ++r) {
      const int chunk = lw + LD * r;
      load_lds16(rKT, ko.tr[r] + tst, sKT(buf) + chunk * 512);
    }
  };

  RowReader<DH> rr;
  rr.init(l16, g);
  TrReader tr;
  tr.init(l16, g);

  floatx4 acc[MB][C::DT];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < C::DT; ++e)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[mb][e][r] = 0.f;
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};

  const int nst = (nk + BT - 1) / BT;
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int cur = st & 1;
    if (st + 1 < nst) issue(cur ^ 1, (st + 1) * BT);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // the wave that reaches its logits issues first (raised priority over the
      // S and dP products and the exponentials, dropped for the dQ products)
      __builtin_amdgcn_s_setprio(1);
      floatx4 S[MB][2], dP[MB][2];
      // both key halves at each k-step: the accumulation chains alternate
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) {
        bf16x8 ka[2], va[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          ka[t] = *reinterpret_cast<const bf16x8 *>(sK(cur) + rr.off(u, t, s));
          va[t] = *reinterpret_cast<const bf16x8 *>(sV(cur) + rr.off(u, t, s));
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            S[mb][t] = mfma16(ka[t], qf[mb][s], s == 0 ? zero4 : S[mb][t]);
            dP[mb][t] = mfma16(va[t], dof[mb][s], s == 0 ? zero4 : dP[mb][t]);
          }
      }
      // keys past nk (last stage only) get zero weight
      if (st == nst - 1) {
        const int kbase = st * BT + 32 * u + 8 * g;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int m = 0; m < 8; ++m)
            if (kbase + m >= nk) S[mb][m >> 2][m & 3] = -INFINITY;
      }
      bf16x8 dS[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const int t = m >> 2, r = m & 3;
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(S[mb][t][r], c_log2, -lse2[mb]));
          dS[mb][m] = (bf16)(pv * (dP[mb][t][r] - Dq[mb]));
        }
      __builtin_amdgcn_s_setprio(0);
      // K^T fragments of d-tile e+1 read ahead of the MFMAs of d-tile e
      bf16x8 kta[2];
      kta[0] = *reinterpret_cast<const bf16x8 *>(sKT(cur) + tr.off(u, 0));
#pragma unroll
      for (int e = 0; e < C::DT; ++e) {
        if (e + 1 < C::DT) kta[(e + 1) & 1] = *reinterpret_cast<const bf16x8 *>(sKT(cur) + tr.off(u, e + 1));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb][e] = mfma16(kta[e & 1], dS[mb], acc[mb][e]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // this wave's loads of the next stage have landed and every wave is done
    // with the current stage before it is refilled
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int q_row = q_row0 + 16 * mb;
    if (part) {   // a piece of a split tile: its scaled partial dQ, every row
      const int pi = 4 * (q_row - qb * C::BW_DQ) + g;
#pragma unroll
      for (int e = 0; e < C::DT; ++e)
        *reinterpret_cast<float4 *>(part + 4 * (e * MB * C::THREADS_DQ + pi)) =
            make_float4(acc[mb][e][0] * p.scale, acc[mb][e][1] * p.scale, acc[mb][e][2] * p.scale,
                        acc[mb][e][3] * p.scale);
    } else if (q_row < p.Nq) {
      bf16 *dst = p.dq + (int64_t)b * p.dq_bs + (int64_t)q_row * p.dq_rs + h * DH + 4 * g;
#pragma unroll
      for (int e = 0; e < C::DT; ++e) {
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (bf16)(acc[mb][e][r] * p.scale);
        *reinterpret_cast<bf16x4 *>(dst + 16 * e) = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__((BwdCfg<DH>::THREADS_DKV), 1) void attn_bwd_dkv_kernel(AttnBwdParams p, int nkb,
                                                                               int per_xcd, int total, SplitArgs sp) {
  using C = BwdCfg<DH>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16 *const lds = reinterpret_cast<bf16 *>(smem_raw);
  auto sQ = [&](int buf) { return lds + buf * C::DKV_STAGE; };
  auto sDO = [&](int buf) { return lds + buf * C::DKV_STAGE + C::ROW_ELEMS; };
  auto sQT = [&](int buf) { return lds + buf * C::DKV_STAGE + 2 * C::ROW_ELEMS; };
  auto sDOT = [&](int buf) { return lds + buf * C::DKV_STAGE + 2 * C::ROW_ELEMS + C::T_ELEMS; };
  auto sL = [&](int buf) {
    return reinterpret_cast<float *>(lds + buf * C::DKV_STAGE + 2 * C::ROW_ELEMS + 2 * C::T_ELEMS);
  };
  auto sD = [&](int buf) { return sL(buf) + BT; };

  // XCD-aware order; a split tile's pieces cover consecutive query stages
  const SplitItem it = split_item(blockIdx.x, per_xcd, sp);
  if (it.L >= total) return;
  const int kb = it.L % nkb, bh = it.L / nkb;
  const int b = bh / p.H, h = bh % p.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  constexpr int MB = C::MB_DKV;
  const int k_row0 = kb * C::BW_DKV + wave * 16 * MB + l16;   // + 16 mb for key block mb
  const int nk = min(max(p.nk[b], 1), p.Nk);
  // this workgroup's queries [q0, q0 + Nq)
  int q0 = 0, Nq = p.Nq;
  float *part = nullptr;
  if (it.slot >= 0) {
    int s0, s1;
    piece_stages((p.Nq + BT - 1) / BT, it.piece, sp.k, s0, s1);
    q0 = s0 * BT;
    Nq = min(p.Nq, s1 * BT) - q0;
    part = p.part + (size_t)(it.slot * sp.k + it.piece) * C::PIECE_DKV;
  }
  if (Nq <= 0) {   // an empty piece adds zero
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int pi = 4 * (k_row0 + 16 * mb - kb * C::BW_DKV) + g;
#pragma unroll
      for (int e = 0; e < C::DT; ++e) {
        *reinterpret_cast<float4 *>(part + 4 * (e * MB * C::THREADS_DKV + pi)) = make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4 *>(part + C::PIECE_DKV_HALF + 4 * (e * MB * C::THREADS_DKV + pi)) =
            make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    return;
  }
  const float c_log2 = p.scale * 1.4426950408889634f;

  bf16x8 kf[MB][C::KSTEPS], vf[MB][C::KSTEPS];
  // Keys past nk get dK = dV = 0, applied when they are stored: a lane's
  // weights P and dS only ever reach its own key's dK and dV columns.
  bool kvalid[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int k_ld = min(k_row0 + 16 * mb, p.Nk - 1);
    kvalid[mb] = k_row0 + 16 * mb < nk;
    const bf16 *kp = p.k + (int64_t)b * p.k_bs + (int64_t)k_ld * p.k_rs + h * DH + 8 * g;
    const bf16 *vp = p.v + (int64_t)b * p.v_bs + (int64_t)k_ld * p.v_rs + h * DH + 8 * g;
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) {
      kf[mb][s] = *reinterpret_cast<const bf16x8 *>(kp + 32 * s);
      vf[mb][s] = *reinterpret_cast<const bf16x8 *>(vp + 32 * s);
    }
  }

  // Descriptors start at query q0.  Q and dO row descriptors end after query
  // row Nq-1; the transposed copies are zero past the last query; lse2 and D
  // past Nq load as zeros and those queries' weights are masked.
  const uint32_t q_bytes = (uint32_t)(((int64_t)(Nq - 1) * p.q_rs + DH) * 2);
  const uint32_t do_bytes = (uint32_t)(((int64_t)(Nq - 1) * p.do_rs + DH) * 2);
  const uint32_t qt_bytes = (uint32_t)(((int64_t)DH * p.qt_rs - q0) * 2);
  const uint32_t s_bytes = (uint32_t)(Nq * 4);
  const __amdgpu_buffer_rsrc_t rQ = make_rsrc(p.q + (int64_t)b * p.q_bs + (int64_t)q0 * p.q_rs + h * DH, q_bytes);
  const __amdgpu_buffer_rsrc_t rDO =
      make_rsrc(p.dout + (int64_t)b * p.do_bs + (int64_t)q0 * p.do_rs + h * DH, do_bytes);
  const int64_t qt_at = (int64_t)b * p.qt_bs + (int64_t)h * p.qt_hs + q0;
  const __amdgpu_buffer_rsrc_t rQT = make_rsrc(p.qt + qt_at, qt_bytes);
  const __amdgpu_buffer_rsrc_t rDOT = make_rsrc(p.dot + qt_at, qt_bytes);
  const int64_t srow = ((int64_t)b * p.H + h) * p.Nq + q0;
  const __amdgpu_buffer_rsrc_t rL = make_rsrc(p.lse2 + srow, s_bytes);
  const __amdgpu_buffer_rsrc_t rD = make_rsrc(p.D + srow, s_bytes);
  constexpr int LD = C::LD_DKV;
  using TO = TileOffsets<DH, LD>;
  const int lw = wave % LD;
  const bool loader = wave < LD;
  TO qo, doo;
  qo.init(lw, lane, p.q_rs, p.qt_rs);
  doo.init(lw, lane, p.do_rs, p.qt_rs);
  auto issue = [&](int buf, int q0) {
    if (!loader) return;
    const uint32_t qst = (uint32_t)(q0 * p.q_rs * 2), dst = (uint32_t)(q0 * p.do_rs * 2), tst = (uint32_t)(q0 * 2);
#pragma unroll
    for (int r = 0; r < TO::RCH; ++r) {
      const int chunk = lw + LD * r;
      load_lds16(rQ, qo.row[r] + qst, sQ(buf) + chunk * 512);
      load_lds16(rDO, doo.row[r] + dst, sDO(buf) + chunk * 512);
    }
#pragma unroll
    for (int r = 0; r < TO::TCH; ++r) {
      const int chunk = lw + LD * r;
      load_lds16(rQT, qo.tr[r] + tst, sQT(buf) + chunk * 512);
      load_lds16(rDOT, qo.tr[r] + tst, sDOT(buf) + chunk * 512);
    }
    if (lw == 0) {   // 64 lanes x 4 B: the stage's lse2 and D
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rL, (lds_void *)sL(buf), 4, (uint32_t)((q0 + lane) * 4), 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rD, (lds_void *)sD(buf), 4, (uint32_t)((q0 + lane) * 4), 0, 0, 0);
    }
  };

  RowReader<DH> rr;
  rr.init(l16, g);
  TrReader tr;
  tr.init(l16, g);

  floatx4 dK[MB][C::DT], dV[MB][C::DT];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < C::DT; ++e)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        dK[mb][e][r] = 0.f;
        dV[mb][e][r] = 0.f;
      }
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};

  const int nst = (Nq + BT - 1) / BT;
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int cur = st & 1;
    if (st + 1 < nst) issue(cur ^ 1, (st + 1) * BT);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // raised priority over the S and dP products and the exponentials, as in
      // the dQ kernel, dropped for the dK and dV products
      __builtin_amdgcn_s_setprio(1);
      floatx4 S[MB][2], dP[MB][2];
      // both query halves at each k-step: four accumulation chains alternate
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) {
        bf16x8 qa[2], da[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          qa[t] = *reinterpret_cast<const bf16x8 *>(sQ(cur) + rr.off(u, t, s));
          da[t] = *reinterpret_cast<const bf16x8 *>(sDO(cur) + rr.off(u, t, s));
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            S[mb][t] = mfma16(qa[t], kf[mb][s], s == 0 ? zero4 : S[mb][t]);
            dP[mb][t] = mfma16(da[t], vf[mb][s], s == 0 ? zero4 : dP[mb][t]);
          }
      }
      // this lane's queries: 32 u + 8 g + m of the stage, m = 4 t + r.
      // Queries past Nq (in the last stage of the last piece; other pieces end
      // at a stage boundary) need no mask: their Q and dO rows, lse2 and D lie
      // past the descriptors' ends and load as zeros, so S = dP = 0, P = 1 and
      // dS = 0, and their Q^T and dO^T columns are the zeros the transposes
      // pad with up to a whole stage, so both products add 0.
      float4 l0, l1, d0, d1;
      read_stage_stats(sL(cur) + 32 * u + 8 * g, sD(cur) + 32 * u + 8 * g, l0, l1, d0, d1);
      const float lq[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
      const float dq[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
      bf16x8 P[MB], dS[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const int t = m >> 2, r = m & 3;
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(S[mb][t][r], c_log2, -lq[m]));
          P[mb][m] = (bf16)pv;
          dS[mb][m] = (bf16)(pv * (dP[mb][t][r] - dq[m]));
        }
      // the dO^T and Q^T fragments of d-tile e+1 are read before the MFMAs of
      // d-tile e (held in that order by scheduling barriers; left alone, the
      // scheduler sinks each read next to its use and every MFMA pair waits
      // for an LDS round trip)
      __builtin_amdgcn_s_setprio(0);
      bf16x8 doa[2], qta[2];
      doa[0] = *reinterpret_cast<const bf16x8 *>(sDOT(cur) + tr.off(u, 0));
      qta[0] = *reinterpret_cast<const bf16x8 *>(sQT(cur) + tr.off(u, 0));
#pragma unroll
      for (int e = 0; e < C::DT; ++e) {
        if (e + 1 < C::DT) {
          doa[(e + 1) & 1] = *reinterpret_cast<const bf16x8 *>(sDOT(cur) + tr.off(u, e + 1));
          qta[(e + 1) & 1] = *reinterpret_cast<const bf16x8 *>(sQT(cur) + tr.off(u, e + 1));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          dV[mb][e] = mfma16(doa[e & 1], P[mb], dV[mb][e]);
          dK[mb][e] = mfma16(qta[e & 1], dS[mb], dK[mb][e]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int k_row = k_row0 + 16 * mb;
    if (part) {   // a piece of a split tile: its partial dK (scaled) and dV, every row
      const int pi = 4 * (k_row - kb * C::BW_DKV) + g;
#pragma unroll
      for (int e = 0; e < C::DT; ++e) {
        float *pk = part + 4 * (e * MB * C::THREADS_DKV + pi);
        float k4[4], v4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          k4[r] = kvalid[mb] ? dK[mb][e][r] * p.scale : 0.f;
          v4[r] = kvalid[mb] ? dV[mb][e][r] : 0.f;
        }
        *reinterpret_cast<float4 *>(pk) = make_float4(k4[0], k4[1], k4[2], k4[3]);
        *reinterpret_cast<float4 *>(pk + C::PIECE_DKV_HALF) = make_float4(v4[0], v4[1], v4[2], v4[3]);
      }
    } else if (k_row < p.Nk) {
      const int64_t o = (int64_t)b * p.dk_bs + (int64_t)k_row * p.dk_rs + h * DH + 4 * g;
#pragma unroll
      for (int e = 0; e < C::DT; ++e) {
        bf16x4 vk, vv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          vk[r] = (bf16)(kvalid[mb] ? dK[mb][e][r] * p.scale : 0.f);
          vv[r] = (bf16)(kvalid[mb] ? dV[mb][e][r] : 0.f);
        }
        *reinterpret_cast<bf16x4 *>(p.dk + o + 16 * e) = vk;
        *reinterpret_cast<bf16x4 *>(p.dv + o + 16 * e) = vv;
      }
    }
  }
}

// Sum of the pieces of each split dQ tile (one workgroup per split tile and
// 16-column d-tile, each thread the rows and columns of that d-tile it held in
// the dQ kernel), in piece order.
template <int DH>
__global__ __launch_bounds__((BwdCfg<DH>::THREADS_DQ), 1) void attn_bwd_dq_merge_kernel(AttnBwdParams p, int nqb,
                                                                                    int per_xcd, int total,
                                                                                    SplitArgs sp) {
  using C = BwdCfg<DH>;
  constexpr int MB = C::MB_DQ;
  const int slot = blockIdx.x;
  const int L = split_tile(slot, per_xcd, sp);
  if (L >= total) return;
  const int qb = L % nqb, bh = L / nqb;
  const int b = bh / p.H, h = bh % p.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int e = blockIdx.y;   // the d-tile this workgroup sums
  const float *part = p.part + (size_t)slot * sp.k * C::PIECE_DQ;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int row = wave * 16 * MB + 16 * mb + l16;
    const int q_row = qb * C::BW_DQ + row;
    if (q_row >= p.Nq) continue;
    const int pi = 4 * row + g;
    bf16 *dst = p.dq + (int64_t)b * p.dq_bs + (int64_t)q_row * p.dq_rs + h * DH + 4 * g;
    {
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int i = 0; i < sp.k; ++i) {
        const float4 v = *reinterpret_cast<const float4 *>(part + (size_t)i * C::PIECE_DQ +
                                                           4 * (e * MB * C::THREADS_DQ + pi));
        a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
      }
      bf16x4 o;
      o[0] = (bf16)a.x; o[1] = (bf16)a.y; o[2] = (bf16)a.z; o[3] = (bf16)a.w;
      *reinterpret_cast<bf16x4 *>(dst + 16 * e) = o;
    }
  }
}

// Sum of the pieces of each split dK/dV tile, in piece order.
template <int DH>
__global__ __launch_bounds__((BwdCfg<DH>::THREADS_DKV), 1) void attn_bwd_dkv_merge_kernel(AttnBwdParams p,
                                                                                      int nkb, int per_xcd,
                                                                                      int total, SplitArgs sp) {
  using C = BwdCfg<DH>;
  constexpr int MB = C::MB_DKV;
  const int slot = blockIdx.x;
  const int L = split_tile(slot, per_xcd, sp);
  if (L >= total) return;
  const int kb = L % nkb, bh = L / nkb;
  const int b = bh / p.H, h = bh % p.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int e = blockIdx.y;   // the d-tile this workgroup sums
  const float *part = p.part + (size_t)slot * sp.k * C::PIECE_DKV;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int row = wave * 16 * MB + 16 * mb + l16;
    const int k_row = kb * C::BW_DKV + row;
    if (k_row >= p.Nk) continue;
    const int pi = 4 * row + g;
    const int64_t o = (int64_t)b * p.dk_bs + (int64_t)k_row * p.dk_rs + h * DH + 4 * g;
    {
      float4 ak = make_float4(0.f, 0.f, 0.f, 0.f), av = ak;
      for (int i = 0; i < sp.k; ++i) {
        const float *pk = part + (size_t)i * C::PIECE_DKV + 4 * (e * MB * C::THREADS_DKV + pi);
        const float4 vk = *reinterpret_cast<const float4 *>(pk);
        const float4 vv = *reinterpret_cast<const float4 *>(pk + C::PIECE_DKV_HALF);
        ak.x += vk.x; ak.y += vk.y; ak.z += vk.z; ak.w += vk.w;
        av.x += vv.x; av.y += vv.y; av.z += vv.z; av.w += vv.w;
      }
      bf16x4 ok, ov;
      ok[0] = (bf16)ak.x; ok[1] = (bf16)ak.y; ok[2] = (bf16)ak.z; ok[3] = (bf16)ak.w;
      ov[0] = (bf16)av.x; ov[1] = (bf16)av.y; ov[2] = (bf16)av.z; ov[3] = (bf16)av.w;
      *reinterpret_cast<bf16x4 *>(p.dk + o + 16 * e) = ok;
      *reinterpret_cast<bf16x4 *>(p.dv + o + 16 * e) = ov;
    }
  }
}

constexpr size_t kCapPiecesBwd = 768;   // scratch for at most this many pieces

template <int DH>
size_t bwd_split_bytes(int B, int H, int Nq, int Nk) {
  using C = BwdCfg<DH>;
  auto need = [](int64_t tiles, int piece_floats) {
    return std::min<size_t>(kCapPiecesBwd, (size_t)kMaxPiecesBwd * 8 * ((tiles + 7) / 8)) * piece_floats *
           sizeof(float);
  };
  const int64_t tq = (int64_t)B * H * ((Nq + C::BW_DQ - 1) / C::BW_DQ);
  const int64_t tk = (int64_t)B * H * ((Nk + C::BW_DKV - 1) / C::BW_DKV);
  return std::max(need(tq, C::PIECE_DQ), need(tk, C::PIECE_DKV));
}

template <int DH>
hipError_t launch_bwd_impl(const AttnBwdParams &p, hipStream_t s) {
  using C = BwdCfg<DH>;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void *)attn_bwd_dq_kernel<DH>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::DQ_LDS);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void *)attn_bwd_dkv_kernel<DH>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::DKV_LDS);
    if (e != hipSuccess) return e;
    attr = true;
  }
  static int slots_dq[kMaxDevices], slots_dkv[kMaxDevices];
  // dQ: query tiles, split over key stages
  const int nqb = (p.Nq + C::BW_DQ - 1) / C::BW_DQ;
  int total = nqb * p.H * p.B;
  int per_xcd = (total + 7) / 8;
  size_t cap = p.part ? p.part_bytes / (sizeof(float) * C::PIECE_DQ) : 0;
  SplitArgs sp = cap ? plan_split(per_xcd, xcd_slots(attn_bwd_dq_kernel<DH>, C::THREADS_DQ, C::DQ_LDS, slots_dq),
                                  (p.Nk + BT - 1) / BT, cap, kMinPieceKeys / BT, kMaxPiecesBwd)
                     : SplitArgs{per_xcd, 0, 1};
  hipLaunchKernelGGL((attn_bwd_dq_kernel<DH>), dim3(8 * (sp.n_full + sp.rem * sp.k)), dim3(C::THREADS_DQ),
                     C::DQ_LDS, s, p, nqb, per_xcd, total, sp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (sp.rem > 0) {
    hipLaunchKernelGGL((attn_bwd_dq_merge_kernel<DH>), dim3(8 * sp.rem, C::DT), dim3(C::THREADS_DQ), 0, s, p, nqb,
                       per_xcd, total, sp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // dK/dV: key tiles, split over query stages (the same scratch: the dQ merge
  // has read it by the time these pieces write, on the one stream)
  const int nkb = (p.Nk + C::BW_DKV - 1) / C::BW_DKV;
  total = nkb * p.H * p.B;
  per_xcd = (total + 7) / 8;
  cap = p.part ? p.part_bytes / (sizeof(float) * C::PIECE_DKV) : 0;
  sp = cap ? plan_split(per_xcd, xcd_slots(attn_bwd_dkv_kernel<DH>, C::THREADS_DKV, C::DKV_LDS, slots_dkv),
                        (p.Nq + BT - 1) / BT, cap, kMinPieceKeys / BT, kMaxPiecesBwd)
           : SplitArgs{per_xcd, 0, 1};
  hipLaunchKernelGGL((attn_bwd_dkv_kernel<DH>), dim3(8 * (sp.n_full + sp.rem * sp.k)), dim3(C::THREADS_DKV),
                     C::DKV_LDS, s, p, nkb, per_xcd, total, sp);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (sp.rem > 0)
    hipLaunchKernelGGL((attn_bwd_dkv_merge_kernel<DH>), dim3(8 * sp.rem, C::DT), dim3(C::THREADS_DKV), 0, s, p, nkb,
                       per_xcd, total, sp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_bwd(int dh, const AttnBwdParams &p, hipStream_t s) {
  if (dh == 128) return launch_bwd_impl<128>(p, s);
  if (dh == 64) return launch_bwd_impl<64>(p, s);
  return hipErrorInvalidValue;
}

size_t attention_bwd_split_bytes(int dh, int B, int H, int Nq, int Nk) {
  if (dh == 128) return bwd_split_bytes<128>(B, H, Nq, Nk);
  if (dh == 64) return bwd_split_bytes<64>(B, H, Nq, Nk);
  return 0;
}

}  // namespace t2va
