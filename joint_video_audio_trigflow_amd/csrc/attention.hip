// Joint attention forward + forward-mode JVP on bf16 MFMA (gfx950).
//
// The joint block of TurboT2VA runs one self-attention over video, audio and
// valid text tokens; the sCM stage needs its JVP in the same pass (deep read,
// section 3.1, J_theta equation; section 4.2: the JVP passes through the
// cross-modal transformer).  Per (sample, head) and query row i:
//   s_j  = scale q_i.k_j            ds_j = scale (dq_i.k_j + q_i.dk_j)
//   p_j  = softmax_j(s)             mu   = sum_j p_j ds_j
//   o_i  = sum_j p_j v_j            do_i = sum_j p_j (ds_j - mu) v_j + p_j dv_j
// streamed over key tiles with fp32 online-softmax state.  With running max
// m, alpha = exp(m_old - m_new) rescales l = sum p, mu~ = sum p ds,
// A = sum p v and dA = sum (p ds) v + p dv; at the end o = A/l,
// do = dA/l - (mu~/l) o.  Keys j >= nk[b] (padded text, section 6.3 of the
// deep read) get logit -inf.
//
// Layout of the work: one workgroup = 4 waves = 128 query rows of one
// (sample, head); each wave owns 32 query rows.  Every product is computed
// transposed so that one lane owns one query row throughout:
//   S^T  = K Q^T           A operand: K rows from LDS, B operand: Q^T in registers
//   dS^T = dK Q^T + K dQ^T
//   O^T += V^T P^T         A operand: V^T rows from LDS, B operand: P^T in registers
//   dO^T += V^T (P*dS)^T + dV^T P^T
// With v_mfma_f32_32x32x16_bf16 a lane l holds output column l%32 and rows
// 8*(v/4) + 4*(l/32) + v%4.  Reading the K rows in the permuted order
// sigma(r) (bits 2 and 3 of r swapped) makes register v of lane l hold key
// 8*(l/32) + v (v < 8) or 16 + 8*(l/32) + (v-8), which is exactly the B
// operand layout the P^T V^T product needs: no shuffles between the two MFMAs.
// The key-tile (K, dK, V^T, dV^T) is staged through LDS with padded rows
// (conflict-free 16-byte reads); the next tile is fetched into registers while
// the current one is consumed.
#include "common.h"

#include <math.h>

namespace t2va {

namespace {

constexpr int BM = 128;     // query rows per workgroup
constexpr int BN = 64;      // keys per tile
constexpr int kThreads = 256;

template <int DH, bool TAN>
struct AttnCfg {
  static constexpr int KSTEPS = DH / 16;     // MFMA k-steps over the head dimension
  static constexpr int DT = DH / 32;         // 32-wide tiles of the head dimension
  static constexpr int KROW = DH + 8;        // LDS row (elements) of K / dK
  static constexpr int VROW = BN + 8;        // LDS row (elements) of V^T / dV^T
  static constexpr int K_ELEMS = BN * KROW;
  static constexpr int V_ELEMS = DH * VROW;
  static constexpr int NSTREAM = TAN ? 2 : 1;
  static constexpr size_t LDS_BYTES = (size_t)NSTREAM * (K_ELEMS + V_ELEMS) * sizeof(bf16);
  // 16-byte chunks per thread per operand tile
  static constexpr int KCH = BN * DH / 8 / kThreads;
  static constexpr int VCH = DH * BN / 8 / kThreads;
};

__device__ __forceinline__ int sigma(int r) {
  // swap bits 2 and 3
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// key offset (within a 32-key sub-tile) held in register v of a lane with half hi
__device__ __forceinline__ int key_of(int v, int hi) {
  return (v < 8) ? (8 * hi + v) : (16 + 8 * hi + (v - 8));
}

template <int DH, bool TAN>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_jvp_kernel(AttnParams p, int nqb,
                                                                   int per_xcd, int total) {
  using C = AttnCfg<DH, TAN>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16 *sK = reinterpret_cast<bf16 *>(smem_raw);
  bf16 *sVT = sK + C::K_ELEMS;
  bf16 *sKd = sVT + C::V_ELEMS;            // valid when TAN
  bf16 *sVdT = sKd + C::K_ELEMS;

  // XCD-aware order: hardware places workgroup w on XCD w % 8; give each XCD a
  // contiguous range of logical tiles so one head's K/V stay in that XCD's L2.
  const int w = blockIdx.x;
  const int L = (w & 7) * per_xcd + (w >> 3);
  if (L >= total) return;
  const int qb = L % nqb;
  const int bh = L / nqb;
  const int b = bh / p.H, h = bh % p.H;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int q_row = qb * BM + wave * 32 + l32;
  const int q_ld = min(q_row, p.Nq - 1);
  const int nk = min(max(p.nk[b], 1), p.Nk);

  const float scale = p.scale;
  const float c_log2 = scale * 1.4426950408889634f;

  // Q^T (and dQ^T) as B operands: lane holds Q[q_row][16 s + 8 hi .. +7].
  bf16x8 qf[C::KSTEPS], qdf[TAN ? C::KSTEPS : 1];
  {
    const bf16 *qp = p.q + (int64_t)b * p.q_bs + (int64_t)q_ld * p.q_rs + h * DH + 8 * hi;
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) qf[s] = *reinterpret_cast<const bf16x8 *>(qp + 16 * s);
    if constexpr (TAN) {
      const bf16 *qdp = p.qd + (int64_t)b * p.q_bs + (int64_t)q_ld * p.q_rs + h * DH + 8 * hi;
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) qdf[s] = *reinterpret_cast<const bf16x8 *>(qdp + 16 * s);
    }
  }

  const bf16 *kbase = p.k + (int64_t)b * p.k_bs + h * DH;
  const bf16 *vtbase = p.vt + (int64_t)b * p.vt_bs + (int64_t)h * p.vt_hs;
  const bf16 *kdbase = TAN ? p.kd + (int64_t)b * p.k_bs + h * DH : nullptr;
  const bf16 *vdtbase = TAN ? p.vdt + (int64_t)b * p.vt_bs + (int64_t)h * p.vt_hs : nullptr;

  uint4 rk[C::KCH], rv[C::VCH], rkd[TAN ? C::KCH : 1], rvd[TAN ? C::VCH : 1];

  auto fetch = [&](int k0) {
#pragma unroll
    for (int r = 0; r < C::KCH; ++r) {
      const int c = tid + kThreads * r;
      const int key = c / (DH / 8), col = (c % (DH / 8)) * 8;
      const bool ok = (k0 + key) < nk;
      const int64_t off = (int64_t)(k0 + key) * p.k_rs + col;
      rk[r] = ok ? *reinterpret_cast<const uint4 *>(kbase + off) : make_uint4(0, 0, 0, 0);
      if constexpr (TAN)
        rkd[r] = ok ? *reinterpret_cast<const uint4 *>(kdbase + off) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < C::VCH; ++r) {
      const int c = tid + kThreads * r;
      const int e = c / (BN / 8), kc = (c % (BN / 8)) * 8;
      const int j0 = k0 + kc;
      const int64_t off = (int64_t)e * p.vt_rs + j0;
      uint4 x = make_uint4(0, 0, 0, 0), xd = make_uint4(0, 0, 0, 0);
      if (j0 < nk) {
        x = *reinterpret_cast<const uint4 *>(vtbase + off);
        if constexpr (TAN) xd = *reinterpret_cast<const uint4 *>(vdtbase + off);
        if (j0 + 8 > nk) {  // partial chunk: zero the keys past nk
          bf16x8 a = __builtin_bit_cast(bf16x8, x), ad = __builtin_bit_cast(bf16x8, xd);
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (j0 + u >= nk) { a[u] = (bf16)0.f; ad[u] = (bf16)0.f; }
          x = __builtin_bit_cast(uint4, a);
          xd = __builtin_bit_cast(uint4, ad);
        }
      }
      rv[r] = x;
      if constexpr (TAN) rvd[r] = xd;
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int r = 0; r < C::KCH; ++r) {
      const int c = tid + kThreads * r;
      const int key = c / (DH / 8), col = (c % (DH / 8)) * 8;
      *reinterpret_cast<uint4 *>(sK + key * C::KROW + col) = rk[r];
      if constexpr (TAN) *reinterpret_cast<uint4 *>(sKd + key * C::KROW + col) = rkd[r];
    }
#pragma unroll
    for (int r = 0; r < C::VCH; ++r) {
      const int c = tid + kThreads * r;
      const int e = c / (BN / 8), kc = (c % (BN / 8)) * 8;
      *reinterpret_cast<uint4 *>(sVT + e * C::VROW + kc) = rv[r];
      if constexpr (TAN) *reinterpret_cast<uint4 *>(sVdT + e * C::VROW + kc) = rvd[r];
    }
  };

  floatx16 O[C::DT], Od[TAN ? C::DT : 1];
#pragma unroll
  for (int e = 0; e < C::DT; ++e)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      O[e][v] = 0.f;
      if constexpr (TAN) Od[e][v] = 0.f;
    }
  float m_run = -INFINITY, l_part = 0.f, mu_part = 0.f;

  const int ntiles = (nk + BN - 1) / BN;
  fetch(0);
  for (int tile = 0; tile < ntiles; ++tile) {
    const int k0 = tile * BN;
    stage();
    __syncthreads();
    if (tile + 1 < ntiles) fetch(k0 + BN);

    // ---- S^T (and dS^T) for two 32-key sub-tiles ----
    floatx16 S[2], Sd[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        S[t][v] = 0.f;
        Sd[t][v] = 0.f;
      }
      const bf16 *krow = sK + (32 * t + sigma(l32)) * C::KROW + 8 * hi;
      const bf16 *kdrow = sKd + (32 * t + sigma(l32)) * C::KROW + 8 * hi;
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(krow + 16 * s);
        S[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[s], S[t], 0, 0, 0);
        if constexpr (TAN) {
          const bf16x8 kda = *reinterpret_cast<const bf16x8 *>(kdrow + 16 * s);
          Sd[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kda, qf[s], Sd[t], 0, 0, 0);
          Sd[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qdf[s], Sd[t], 0, 0, 0);
        }
      }
    }

    // ---- mask, online softmax ----
    if (k0 + BN > nk) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (k0 + 32 * t + key_of(v, hi) >= nk) {
            S[t][v] = -INFINITY;
            Sd[t][v] = 0.f;
          }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, S[t][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * c_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;

    bf16x8 P[2][2], PS[2][2];
    float lsum = 0.f, musum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int v = 8 * u + j;
          const float pv = __builtin_amdgcn_exp2f(S[t][v] * c_log2 - m_new);
          lsum += pv;
          P[t][u][j] = (bf16)pv;
          if constexpr (TAN) {
            const float ps = pv * (Sd[t][v] * scale);
            musum += ps;
            PS[t][u][j] = (bf16)ps;
          }
        }
    l_part = alpha * l_part + lsum;
    if constexpr (TAN) mu_part = alpha * mu_part + musum;

    // ---- O^T = alpha O^T + V^T P^T (and the tangent) ----
#pragma unroll
    for (int e = 0; e < C::DT; ++e) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        O[e][v] *= alpha;
        if constexpr (TAN) Od[e][v] *= alpha;
      }
      const bf16 *vrow = sVT + (32 * e + l32) * C::VROW + 8 * hi;
      const bf16 *vdrow = sVdT + (32 * e + l32) * C::VROW + 8 * hi;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const bf16x8 va = *reinterpret_cast<const bf16x8 *>(vrow + 32 * t + 16 * u);
          O[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, P[t][u], O[e], 0, 0, 0);
          if constexpr (TAN) {
            const bf16x8 vda = *reinterpret_cast<const bf16x8 *>(vdrow + 32 * t + 16 * u);
            Od[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, PS[t][u], Od[e], 0, 0, 0);
            Od[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vda, P[t][u], Od[e], 0, 0, 0);
          }
        }
    }
    __syncthreads();
  }

  // ---- epilogue ----
  const float l_tot = l_part + __shfl_xor(l_part, 32);
  const float inv_l = 1.f / l_tot;
  float mu = 0.f;
  if constexpr (TAN) mu = (mu_part + __shfl_xor(mu_part, 32)) * inv_l;
  if (q_row < p.Nq) {
    if (p.lse && hi == 0)
      p.lse[((int64_t)b * p.H + h) * p.Nq + q_row] = m_run * 0.6931471805599453f + logf(l_tot);
    const int64_t obase = (int64_t)b * p.o_bs + (int64_t)q_row * p.o_rs + h * DH;
#pragma unroll
    for (int e = 0; e < C::DT; ++e)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * e + 8 * g + 4 * hi;
        float o4[4], od4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          o4[u] = O[e][4 * g + u] * inv_l;
          if constexpr (TAN) od4[u] = Od[e][4 * g + u] * inv_l - mu * o4[u];
        }
        if (p.out_dt == 0) {
          bf16x4 a;
#pragma unroll
          for (int u = 0; u < 4; ++u) a[u] = (bf16)o4[u];
          *reinterpret_cast<bf16x4 *>(reinterpret_cast<bf16 *>(p.o) + obase + col) = a;
          if constexpr (TAN) {
#pragma unroll
            for (int u = 0; u < 4; ++u) a[u] = (bf16)od4[u];
            *reinterpret_cast<bf16x4 *>(reinterpret_cast<bf16 *>(p.od) + obase + col) = a;
          }
        } else {
          *reinterpret_cast<float4 *>(reinterpret_cast<float *>(p.o) + obase + col) =
              make_float4(o4[0], o4[1], o4[2], o4[3]);
          if constexpr (TAN)
            *reinterpret_cast<float4 *>(reinterpret_cast<float *>(p.od) + obase + col) =
                make_float4(od4[0], od4[1], od4[2], od4[3]);
        }
      }
  }
}

template <int DH, bool TAN>
hipError_t launch_impl(const AttnParams &p, hipStream_t s) {
  using C = AttnCfg<DH, TAN>;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void *)attn_fwd_jvp_kernel<DH, TAN>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int nqb = (p.Nq + BM - 1) / BM;
  const int total = nqb * p.H * p.B;
  const int per_xcd = (total + 7) / 8;
  hipLaunchKernelGGL((attn_fwd_jvp_kernel<DH, TAN>), dim3(per_xcd * 8), dim3(kThreads),
                     C::LDS_BYTES, s, p, nqb, per_xcd, total);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(int dh, bool tangent, const AttnParams &p, hipStream_t s) {
  if (dh == 128) return tangent ? launch_impl<128, true>(p, s) : launch_impl<128, false>(p, s);
  if (dh == 64) return tangent ? launch_impl<64, true>(p, s) : launch_impl<64, false>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace t2va
