// Joint attention forward + forward-mode JVP on bf16 MFMA (gfx950).
//
// The joint block of TurboT2VA runs one self-attention over video, audio and
// valid text tokens; the sCM stage needs its JVP in the same pass (deep read,
// section 3.1, J_theta equation; section 4.2: the JVP passes through the
// cross-modal transformer).  Per (sample, head) and query row i:
//   s_j  = scale q_i.k_j            ds_j = scale (dq_i.k_j + q_i.dk_j)
//   p_j  = softmax_j(s)             mu   = sum_j p_j ds_j
//   o_i  = sum_j p_j v_j            do_i = sum_j p_j (ds_j - mu) v_j + p_j dv_j
// streamed over key tiles with fp32 softmax state: with a reference max m,
// l = sum 2^(s'-m), mu~ = sum 2^(s'-m) ds, A = sum 2^(s'-m) v and
// dA = sum 2^(s'-m) (ds v + dv) (s' = s log2 e); at the end o = A/l,
// do = dA/l - (mu~/l) o.  Keys j >= nk[b] (padded text, section 6.3 of the
// deep read) get logit -inf.
//
// Work decomposition: a workgroup of 12 waves (three per SIMD) owns the query
// rows of one (sample, head); a JVP wave owns 16 rows, a forward-only wave two
// blocks of 16 that share every K and V^T fragment it reads from LDS (so each
// 1 KB fragment feeds two MFMAs; with one block per wave the forward kernel
// measured 36 % of the bf16 peak instead of 41 %).  Products are computed
// transposed so that one lane column owns one query row throughout, using
// v_mfma_f32_16x16x32_bf16 (A: lane l holds row l%16, k = 8(l/16)..+7;
// B: k = 8(l/16)..+7, column l%16; C: column l%16, rows 4(l/16)+r):
//   S^T  = K Q^T, dS^T = dK Q^T + K dQ^T    (A: K rows from LDS, B: Q^T in registers)
//   O^T += V^T P^T, dO^T += V^T (P dS)^T + dV^T P^T   (A: V^T rows from LDS, B: P^T)
// For 32-key sub-tile half t the K rows are read in the order
// 8(i/4) + 4t + i%4, which makes register r of half t of a lane with g = l/16
// hold key 8g + 4t + r: the 8 values a lane owns are then exactly the
// B-operand keys 8g..8g+7 of the P^T V^T product, with no lane exchange.
//
// Key tiles (K, dK, V^T, dV^T) go from global memory straight into LDS with
// buffer_load_dwordx4 ... lds (no staging registers; SGPR descriptors and
// 32-bit lane offsets), in stages of BN keys (64 in the JVP kernel, 128 in the
// forward kernel, which halves its barriers): a three-slot ring for K (and dK)
// and a two-slot ring for V^T (and dV^T), one barrier per stage.  16-byte slots are
// XOR-swizzled so that every 16-lane group of an operand read hits 16
// different bank groups.
#include "attn_tiles.h"
#include "common.h"

#include <math.h>

#include <algorithm>

namespace t2va {

namespace {

#ifndef T2VA_ATTN_WAVES_JVP
#define T2VA_ATTN_WAVES_JVP 12
#endif
#ifndef T2VA_ATTN_WAVES_FWD
#define T2VA_ATTN_WAVES_FWD 12
#endif
#ifndef T2VA_ATTN_MB_FWD
#define T2VA_ATTN_MB_FWD 2
#endif
constexpr int kLoadWaves = 8;         // waves that issue the LDS loads

// 16-byte slot of key chunk kc of V^T row e for rows of VCPR chunks: 8 chunks
// (64 keys): the shared swizzle; 16 chunks (128 keys, rows 256 B apart, i.e.
// on the same banks): XOR with the row's low four bits, so the 16 rows a
// 16-lane group reads at one chunk index fall on 16 distinct slots; 4 chunks
// (32 keys, rows 64 B apart: rows e and e + 4 share banks): XOR with row bits
// 2-3, so the 16 rows again cover all 16 bank groups.
template <int VCPR>
__device__ __forceinline__ int vslot_n(int e, int kc) {
  if constexpr (VCPR == 4) return kc ^ ((e >> 2) & 3);   // 32 keys: rows 64 B apart
  else if constexpr (VCPR == 8) return vslot(e, kc);
  else return kc ^ (e & 15);
}

// SPLIT: the split-precision kernels (logits from q + q_lo and k + k_lo).  They
// hold Q_lo in registers and stage K_lo beside K, so they use one row block
// per wave, 64-key stages in the forward kernel and 4096-element K tiles in
// the JVP kernel (32 keys at dh 128), and the JVP kernel runs 8 waves (two per
// SIMD, with room for the extra registers).
template <int DH, bool TAN, bool SPLIT = false>
struct AttnCfg {
  // waves per workgroup: 12 (three per SIMD) by default; MB blocks of 16
  // query rows per wave.  In the forward kernel every K / V^T fragment a wave
  // reads from LDS feeds MB MFMAs; in the JVP kernel each pair of fragments
  // (K and dK, or V^T and dV^T) feeds three (S, dS twice; O, dO twice).
  static constexpr int NW = SPLIT ? (TAN ? 8 : 12) : (TAN ? T2VA_ATTN_WAVES_JVP : T2VA_ATTN_WAVES_FWD);
  static constexpr int MB = (TAN || SPLIT) ? 1 : T2VA_ATTN_MB_FWD;
  // row sums on the matrix cores (forward); the JVP kernel keeps them on the
  // VALU, where its register budget has room and the matrix cores do not
  static constexpr bool MFMA_SUMS = !TAN;
  static constexpr int THREADS = 64 * NW;
  // keys per LDS stage (one barrier each): 64 for the JVP kernel, whose
  // tangent tiles double its LDS; 128 for the forward, which then also fills
  // the 160 KB and needs half as many barriers
  static constexpr int BN = SPLIT ? (TAN ? 4096 / DH : 64) : (TAN ? 64 : 128);
  static constexpr int SUB = BN / 32;      // 32-key sub-tiles per stage
  static constexpr int VCPR = BN / 8;      // 16-byte chunks per V^T row
  static constexpr int BM = 16 * MB * NW;  // query rows per workgroup
  static constexpr int KSTEPS = DH / 32;   // MFMA k-steps over the head dimension
  static constexpr int DT = DH / 16;       // 16-row tiles of the head dimension
  static constexpr int CPR = DH / 8;       // 16-byte chunks per K row
  static constexpr int K_ELEMS = BN * DH;  // K tile [BN][DH], swizzled slots
  static constexpr int V_ELEMS = DH * BN;  // V^T tile [DH][BN], swizzled slots
  static constexpr int NSTREAM = TAN ? 2 : 1;
  // rings of three K stages ([K | dK | K_lo] each, as present) and two V^T
  // stages ([V^T | dV^T])
  static constexpr int KBUF_ELEMS = (NSTREAM + (SPLIT ? 1 : 0)) * K_ELEMS;
  static constexpr int VBUF_ELEMS = NSTREAM * V_ELEMS;
  static constexpr int KLO_AT = NSTREAM * K_ELEMS;   // K_lo's offset in a K stage
  static constexpr size_t LDS_BYTES = (size_t)(3 * KBUF_ELEMS + 2 * VBUF_ELEMS) * sizeof(bf16);
  // one direct load instruction moves 64 lanes x 16 B = 1 KB = 512 elements
  static constexpr int KCH = K_ELEMS / 512 / kLoadWaves;   // per loading wave, per operand tile
  static constexpr int VCH = V_ELEMS / 512 / kLoadWaves;
  static constexpr int K_ROWS_PER_CHUNK = 512 / DH;
  // partial result of one piece of a split tile (floats): for each of the
  // BM rows and its four lanes g (index 4 row + g, row within the tile),
  // (lse, mu) and the normalised o (and do) of the lane's four columns of each
  // d-tile
  static constexpr int PIECE_STATS = 2 * MB * THREADS;
  static constexpr int PIECE_O = 4 * MB * DT * THREADS;
  static constexpr int PIECE_FLOATS = PIECE_STATS + PIECE_O + (TAN ? 4 * DT * THREADS : 0);
  static_assert(KCH >= 1 && VCH >= 1, "every loading wave moves at least one 1 KB chunk per tile");
  static_assert(BN % 32 == 0 && (VCPR == 4 || VCPR == 8 || VCPR == 16), "32-key sub-tiles, known V^T swizzle");
};


// Four consecutive output columns of one row (and of its tangent): bf16 or
// fp32 as p.out_dt says, at element offset `at` of o (od).
// The value x, opaque to the optimiser: address arithmetic that starts from
// it stays where it is used instead of being hoisted above the key loop, where
// the forward kernel has no registers to hold it (it then spilled ~40 output
// addresses per lane, 344 bytes of scratch, on every launch).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// max(a, b, c) in one v_max3_f32 (written out: fmaxf's NaN rules make the
// compiler quieten every operand of an MFMA result first)
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

template <bool TAN>
__device__ __forceinline__ void store_out4(const AttnParams &p, int64_t at, const float (&o4)[4],
                                           const float (&od4)[4]) {
  if (p.out_dt == 0) {
    bf16x4 a;
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = (bf16)o4[r];
    *reinterpret_cast<bf16x4 *>(reinterpret_cast<bf16 *>(p.o) + at) = a;
    if constexpr (TAN) {
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = (bf16)od4[r];
      *reinterpret_cast<bf16x4 *>(reinterpret_cast<bf16 *>(p.od) + at) = a;
    }
  } else {
    *reinterpret_cast<float4 *>(reinterpret_cast<float *>(p.o) + at) = make_float4(o4[0], o4[1], o4[2], o4[3]);
    if constexpr (TAN)
      *reinterpret_cast<float4 *>(reinterpret_cast<float *>(p.od) + at) =
          make_float4(od4[0], od4[1], od4[2], od4[3]);
  }
}

template <int DH, bool TAN, bool SPLIT>
__global__ __launch_bounds__((AttnCfg<DH, TAN, SPLIT>::THREADS), 1) void attn_fwd_jvp_kernel(
    AttnParams p, int nqb, int per_xcd, int total, SplitArgs sp) {
  using C = AttnCfg<DH, TAN, SPLIT>;
  constexpr int BN = C::BN;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16 *const lds = reinterpret_cast<bf16 *>(smem_raw);
  // LDS: K ring [3][K | dK | K_lo], then V^T ring [2][V^T | dV^T]
  auto sK = [&](int kb) { return lds + kb * C::KBUF_ELEMS; };
  auto sKd = [&](int kb) { return lds + kb * C::KBUF_ELEMS + C::K_ELEMS; };
  auto sKlo = [&](int kb) { return lds + kb * C::KBUF_ELEMS + C::KLO_AT; };
  auto sVT = [&](int vb) { return lds + 3 * C::KBUF_ELEMS + vb * C::VBUF_ELEMS; };
  auto sVdT = [&](int vb) { return lds + 3 * C::KBUF_ELEMS + vb * C::VBUF_ELEMS + C::V_ELEMS; };

  // XCD-aware order, with the XCD's last tiles split (split_item)
  const SplitItem it = split_item(blockIdx.x, per_xcd, sp);
  const int L = it.L, piece = it.piece, slot = it.slot;
  if (L >= total) return;
  const int qb = L % nqb;
  const int bh = L / nqb;
  const int b = bh / p.H, h = bh % p.H;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int q_row0 = qb * C::BM + wave * 16 * C::MB + l16;   // + 16 mb for row block mb
  const int nk_b = min(max(p.nk[b], 1), p.Nk);
  // this workgroup's keys [key0, key0 + nk): all of them, or piece `piece` of
  // sp.k over whole BN-key stages (empty when the sample has fewer stages)
  int key0 = 0, nk = nk_b;
  float *part = nullptr;
  if (slot >= 0) {
    int s0, s1;
    piece_stages((nk_b + BN - 1) / BN, piece, sp.k, s0, s1);
    key0 = s0 * BN;
    nk = min(nk_b, s1 * BN) - key0;
    part = p.part + (size_t)(slot * sp.k + piece) * C::PIECE_FLOATS;
  }
  // forward only: also store the output over the first nk_split keys (a
  // multiple of 32, at most nk) into o2.  A split tile's piece that holds key
  // nk_split - 1 but not all its keys stores its partial result over the keys
  // before it into the prefix bank (the merge takes the other pieces' full
  // partials, or nothing, by their key ranges).
  int nk_split = -1;
  float *ppart = nullptr;
  if (!TAN && p.o2) {
    if (slot < 0) {
      nk_split = p.nk_split;
    } else if (key0 < p.nk_split && p.nk_split < key0 + nk) {
      nk_split = p.nk_split - key0;
      ppart = part + (size_t)sp.pbank * C::PIECE_FLOATS;
    }
  }
  if (nk <= 0) {
    // an empty piece: weight zero in the combination
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      const int pi = 4 * (q_row0 + 16 * mb - qb * C::BM) + g;
      *reinterpret_cast<float2 *>(part + 2 * pi) = make_float2(-INFINITY, 0.f);
#pragma unroll
      for (int e = 0; e < C::DT; ++e) {
        *reinterpret_cast<float4 *>(part + C::PIECE_STATS + 4 * (e * C::MB * C::THREADS + pi)) =
            make_float4(0.f, 0.f, 0.f, 0.f);
        if constexpr (TAN)
          *reinterpret_cast<float4 *>(part + C::PIECE_STATS + C::PIECE_O + 4 * (e * C::THREADS + pi)) =
              make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    return;
  }

  const float scale = p.scale;
  const float c_log2 = scale * 1.4426950408889634f;

  // Q^T (and dQ^T, Q_lo^T) as B operands: lane holds Q[q_row][32 s + 8 g .. +7].
  bf16x8 qf[C::MB][C::KSTEPS], qdf[TAN ? C::KSTEPS : 1], qlf[SPLIT ? C::MB : 1][SPLIT ? C::KSTEPS : 1];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) {
    const int q_ld = min(q_row0 + 16 * mb, p.Nq - 1);
    const int64_t q_at = (int64_t)b * p.q_bs + (int64_t)q_ld * p.q_rs + h * DH + 8 * g;
    const bf16 *qp = p.q + q_at;
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) qf[mb][s] = *reinterpret_cast<const bf16x8 *>(qp + 32 * s);
    if constexpr (SPLIT) {
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) qlf[mb][s] = *reinterpret_cast<const bf16x8 *>(p.q_lo + q_at + 32 * s);
    }
    if constexpr (TAN) {
      const bf16 *qdp = p.qd + (int64_t)b * p.q_bs + (int64_t)q_ld * p.q_rs + h * DH + 8 * g;
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) qdf[s] = *reinterpret_cast<const bf16x8 *>(qdp + 32 * s);
    }
  }

  // ---- global -> LDS staging of one BN-key stage ----
  // The K descriptors end after key row nk-1, so rows >= nk load as zeros
  // (their logits are masked).  V^T columns in [nk, round_up(nk, BN)) are read
  // as stored; the caller keeps them finite, and their weights are zero.
  // Descriptors start at key key0 (so stage offsets below are relative to it).
  const uint32_t k_bytes = (uint32_t)(((int64_t)(nk - 1) * p.k_rs + DH) * 2);
  const uint32_t v_bytes = (uint32_t)(((int64_t)DH * p.vt_rs - key0) * 2);
  const int64_t k_at = (int64_t)b * p.k_bs + (int64_t)key0 * p.k_rs + h * DH;
  const int64_t v_at = (int64_t)b * p.vt_bs + (int64_t)h * p.vt_hs + key0;
  const __amdgpu_buffer_rsrc_t rK = make_rsrc(p.k + k_at, k_bytes);
  const __amdgpu_buffer_rsrc_t rV = make_rsrc(p.vt + v_at, v_bytes);
  __amdgpu_buffer_rsrc_t rKd = rK, rVd = rV, rKlo = rK;
  if constexpr (TAN) {
    rKd = make_rsrc(p.kd + k_at, k_bytes);
    rVd = make_rsrc(p.vdt + v_at, v_bytes);
  }
  if constexpr (SPLIT) rKlo = make_rsrc(p.k_lo + k_at, k_bytes);
  const int lw = wave % kLoadWaves;
  const bool loader = wave < kLoadWaves;
  // Per-lane byte offsets of this lane's 16-byte chunks (at key 0).  Chunk r
  // of a loading wave lies a uniform number of rows after chunk 0
  // (8 r K_ROWS_PER_CHUNK key rows, 8 r 512 / BN V^T rows) and has the same
  // XOR key (the swizzles read only low row bits), so only chunk 0's offset
  // lives in a VGPR and the rest is a uniform per-stage offset.
  uint32_t kvo[C::KCH], vvo[C::VCH];
#pragma unroll
  for (int r = 0; r < C::KCH; ++r) {
    const int chunk = lw + kLoadWaves * r;
    const int row = chunk * C::K_ROWS_PER_CHUNK + lane / C::CPR;
    const int c = kslot<C::CPR>(row, lane % C::CPR);   // the XOR swizzle is an involution
    kvo[r] = (uint32_t)((row * p.k_rs + 8 * c) * 2);
  }
#pragma unroll
  for (int r = 0; r < C::VCH; ++r) {
    const int chunk = lw + kLoadWaves * r;
    const int e = chunk * (512 / BN) + lane / C::VCPR;   // a 1 KB chunk holds 512 / BN rows
    vvo[r] = (uint32_t)((e * p.vt_rs + 8 * vslot_n<C::VCPR>(e, lane % C::VCPR)) * 2);
  }
  // offset of chunk r of stage k0: per-lane part + uniform part
  auto k_off = [&](int r, int k0) -> uint32_t {
    return kvo[0] + (uint32_t)__builtin_amdgcn_readfirstlane(
                        (int)((k0 + kLoadWaves * C::K_ROWS_PER_CHUNK * r) * p.k_rs * 2));
  };
  auto v_off = [&](int r, int k0) -> uint32_t {
    return vvo[0] + (uint32_t)__builtin_amdgcn_readfirstlane(
                        (int)((k0 + kLoadWaves * (512 / BN) * r * p.vt_rs) * 2));
  };
  auto issue_k = [&](int kb, int k0) {
    if (!loader) return;
#pragma unroll
    for (int r = 0; r < C::KCH; ++r) {
      const int chunk = lw + kLoadWaves * r;
      load_lds16(rK, k_off(r, k0), sK(kb) + chunk * 512);
      if constexpr (TAN) load_lds16(rKd, k_off(r, k0), sKd(kb) + chunk * 512);
      if constexpr (SPLIT) load_lds16(rKlo, k_off(r, k0), sKlo(kb) + chunk * 512);
    }
  };
  auto issue_v = [&](int vb, int k0) {
    if (!loader) return;
#pragma unroll
    for (int r = 0; r < C::VCH; ++r) {
      const int chunk = lw + kLoadWaves * r;
      load_lds16(rV, v_off(r, k0), sVT(vb) + chunk * 512);
      if constexpr (TAN) load_lds16(rVd, v_off(r, k0), sVdT(vb) + chunk * 512);
    }
  };
  auto wait_loads = [&]() { __builtin_amdgcn_s_waitcnt(0); };

  // Per-lane swizzled read offsets (elements).  K: half t, k-step s, within a
  // 32-key sub-tile (add 32 * DH per sub-tile).  V^T: rows l16 (+16 per d-tile),
  // key chunk g of 32-key sub-tile u (add 16 * BN per d-tile).
  // K slot of k-step s is 4 s + g; with the XOR key x of the row it is
  // (4 s + g) ^ x = 4 (s ^ (x >> 2)) + (g ^ (x & 3)), so one XOR per read.
  // Rows 8 (l16 / 4) + 4 t + l16 % 4 of the two halves t share their key (it
  // depends on row bits the half does not touch), so half 1 is half 0 moved
  // by four rows.
  const int krow = 8 * (l16 >> 2) + (l16 & 3);
  const int kx = kslot<C::CPR>(krow, 0);                 // the rows' XOR key
  const int kbase_off = krow * DH + 8 * (g ^ (kx & 3));
  auto koff = [&](int t, int s) { return kbase_off + 4 * DH * t + 32 * (s ^ (kx >> 2)); };
  // V^T chunk 4 u + g of row l16: with g < 4, slot(4 u + g) = slot(g) ^ 4 u
  // (both swizzles XOR with a row key), i.e. element offset XOR 32 u
  const int voff0 = l16 * BN + 8 * vslot_n<C::VCPR>(l16, g);
  auto voff = [&](int u) { return voff0 ^ (32 * u); };

  // ---- logits of one 32-key sub-tile u of a stage buffer ----
  // S[mb][t][r] holds key 32 u + 8 g + 4 t + r of row block mb.
  // Split kernels add K_lo Q^T and K Q_lo^T to each logit chain.
  auto compute_s = [&](int buf, int u, floatx4 (&S)[C::MB][2], floatx4 (&Sd)[2]) {
    const bf16 *kt = sK(buf) + 32 * u * DH;
    const bf16 *kdt = sKd(buf) + 32 * u * DH;
    const bf16 *klt = sKlo(buf) + 32 * u * DH;
    // the first k-step starts from a zero accumulator operand (no VALU clears)
    const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
    // Both key halves at each k-step: the accumulation chains of the two
    // halves (logits, and tangent logits in the JVP kernel) interleave, so no
    // MFMA waits on the one just before it.
    if constexpr (TAN) {
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) {
        bf16x8 ka[2], kda[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          ka[t] = *reinterpret_cast<const bf16x8 *>(kt + koff(t, s));
          kda[t] = *reinterpret_cast<const bf16x8 *>(kdt + koff(t, s));
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) Sd[t] = mfma16(kda[t], qf[0][s], s == 0 ? zero4 : Sd[t]);
#pragma unroll
        for (int t = 0; t < 2; ++t) S[0][t] = mfma16(ka[t], qf[0][s], s == 0 ? zero4 : S[0][t]);
#pragma unroll
        for (int t = 0; t < 2; ++t) Sd[t] = mfma16(ka[t], qdf[s], Sd[t]);
        if constexpr (SPLIT) {
          bf16x8 kla[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) kla[t] = *reinterpret_cast<const bf16x8 *>(klt + koff(t, s));
#pragma unroll
          for (int t = 0; t < 2; ++t) S[0][t] = mfma16(kla[t], qf[0][s], S[0][t]);
#pragma unroll
          for (int t = 0; t < 2; ++t) S[0][t] = mfma16(ka[t], qlf[0][s], S[0][t]);
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) {
        bf16x8 ka[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) ka[t] = *reinterpret_cast<const bf16x8 *>(kt + koff(t, s));
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int mb = 0; mb < C::MB; ++mb) S[mb][t] = mfma16(ka[t], qf[mb][s], s == 0 ? zero4 : S[mb][t]);
        if constexpr (SPLIT) {
          bf16x8 kla[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) kla[t] = *reinterpret_cast<const bf16x8 *>(klt + koff(t, s));
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int mb = 0; mb < C::MB; ++mb) {
              S[mb][t] = mfma16(kla[t], qf[mb][s], S[mb][t]);
              S[mb][t] = mfma16(ka[t], qlf[mb][s], S[mb][t]);
            }
        }
      }
    }
  };
  auto mask_s = [&](int kb, floatx4 (&S)[C::MB][2], floatx4 (&Sd)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (kb + 8 * g + 4 * t + r >= nk) {
#pragma unroll
          for (int mb = 0; mb < C::MB; ++mb) S[mb][t][r] = -INFINITY;
          if constexpr (TAN) Sd[t][r] = 0.f;
        }
  };
  // row max over the sub-tile, in log2 units of the scaled logits
  auto row_max = [&](const floatx4 (&S)[2]) {
    float mx = fmaxf(fmaxf(S[0][0], S[0][1]), fmaxf(S[0][2], S[0][3]));
    mx = fmaxf(mx, fmaxf(fmaxf(S[1][0], S[1][1]), fmaxf(S[1][2], S[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    return mx * c_log2;
  };

  // row max (log2 units) and the tangent logit of the key attaining it; ties
  // go to the larger tangent so the four lanes of a row agree
  auto row_max_arg = [&](const floatx4 (&S)[2], const floatx4 (&Sd)[2], float &sd_at_max) {
    float mx = S[0][0], sd = Sd[0][0];
#pragma unroll
    for (int m = 1; m < 8; ++m) {
      const float v = S[m >> 2][m & 3], vd = Sd[m >> 2][m & 3];
      const bool gt = v > mx || (v == mx && vd > sd);
      mx = gt ? v : mx;
      sd = gt ? vd : sd;
    }
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const float om = __shfl_xor(mx, off), od = __shfl_xor(sd, off);
      const bool gt = om > mx || (om == mx && od > sd);
      mx = gt ? om : mx;
      sd = gt ? od : sd;
    }
    sd_at_max = sd * scale;
    return mx * c_log2;
  };

  floatx4 O[C::MB][C::DT], Od[TAN ? C::DT : 1];
#pragma unroll
  for (int e = 0; e < C::DT; ++e)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) O[mb][e][r] = 0.f;
      if constexpr (TAN) Od[e][r] = 0.f;
    }
  // m_run is a reference max (log2 units), not the exact running max: it is
  // raised only when a row's logits exceed it by more than kLazy, so every p is
  // at most 2^kLazy.  Raising it (and rescaling the accumulators) happens
  // outside the inner loop, which therefore never touches O/dO with the VALU.
  //
  // The tangent weights are centred: the kernel accumulates p (ds - c) with c
  // the tangent logit of the row's max key at the last raise, and
  // mu~ = sum p (ds - c).  Then do = dA/l - (mu~/l) o still holds, and when
  // softmax is nearly one-hot (large logits) the dominant key contributes
  // p (ds - c) ~ 0 instead of a large p ds that the final subtraction would
  // have to cancel after bf16 rounding.  For that the JVP kernel raises (and
  // re-centres) once a row's max grows by more than 4 (a factor of 16).
#ifndef T2VA_ATTN_LAZY_JVP
#define T2VA_ATTN_LAZY_JVP 4.f
#endif
  constexpr float kLazy = TAN ? T2VA_ATTN_LAZY_JVP : 16.f;
  // Forward: the row sums l = sum p run on the matrix cores: an all-ones A
  // operand times the bf16 weights P^T gives the sum over the sub-tile's 32
  // keys in every row of the 16x16 result, so each lane gets the full sum of
  // its query row with no lane exchange, from the same bf16-rounded weights
  // as O.  JVP: l and mu~ = sum p (ds - c) are per-lane VALU partial sums,
  // combined over the four lanes of a row at the end.
  float m_run[C::MB], thr[C::MB], c_ref = 0.f, l_part[C::MB], mu_part = 0.f;
  floatx4 Lacc[C::MFMA_SUMS ? C::MB : 1];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) {
    l_part[mb] = 0.f;
    if constexpr (C::MFMA_SUMS)
#pragma unroll
      for (int r = 0; r < 4; ++r) Lacc[mb][r] = 0.f;
  }
  bf16x8 ones;
#pragma unroll
  for (int m = 0; m < 8; ++m) ones[m] = (bf16)1.f;
  {
    // opaque to the compiler, so the forward kernel keeps the operand in four
    // registers instead of rebuilding it with two moves per sub-tile in the
    // key loop (its VALU issue slots are the scarce ones; teacher attention
    // 0.4 % faster, same box)
    typedef int intx4 __attribute__((ext_vector_type(4)));
    intx4 bits = *reinterpret_cast<intx4 *>(&ones);
    asm volatile("" : "+v"(bits));
    ones = *reinterpret_cast<bf16x8 *>(&bits);
  }
  // a row needs a raise once a raw logit exceeds (m_run + kLazy)/c_log2
  auto set_thr = [&](int mb) { thr[mb] = (m_run[mb] + kLazy) / c_log2; };

  // p = 2^(s c - m_run) and p (ds - c) as bf16 B operands (keys 8g..8g+7)
  auto softmax = [&](const floatx4 (&S)[C::MB][2], const floatx4 (&Sd)[2], bf16x8 (&P)[C::MB],
                     bf16x8 &PS) {
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      // the sums start at -0, the identity of fp addition, so the first add folds away
      float lsum = -0.f, musum = -0.f;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int t = m >> 2, r = m & 3;
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(S[mb][t][r], c_log2, -m_run[mb]));
        P[mb][m] = (bf16)pv;
        if constexpr (!C::MFMA_SUMS) lsum += pv;
        if constexpr (TAN) {
          const float ps = pv * __builtin_fmaf(Sd[t][r], scale, -c_ref);   // p (ds - c)
          musum += ps;
          PS[m] = (bf16)ps;
        }
      }
      if constexpr (!C::MFMA_SUMS) l_part[mb] += lsum;
      if constexpr (TAN) mu_part += musum;
    }
  };
  // The forward kernel reads the V^T fragments of d-tile e+1 before the MFMAs
  // of d-tile e, held in that order by scheduling barriers (left alone, the
  // scheduler sinks each read next to its first use); 3 % faster.  The JVP
  // kernel has no registers to spare for it (the same change spills in its
  // loop) and keeps the compiler's order.
  auto pv_accum = [&](int buf, int u, const bf16x8 (&P)[C::MB], const bf16x8 &PS) {
    const bf16 *vt = sVT(buf) + voff(u);
    const bf16 *vdt = sVdT(buf) + voff(u);
    if constexpr (C::MFMA_SUMS)
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) Lacc[mb] = mfma16(ones, P[mb], Lacc[mb]);
    if constexpr (TAN) {
#pragma unroll
      for (int e = 0; e < C::DT; ++e) {
        const bf16x8 va = *reinterpret_cast<const bf16x8 *>(vt + 16 * e * BN);
        O[0][e] = mfma16(va, P[0], O[0][e]);
        const bf16x8 vda = *reinterpret_cast<const bf16x8 *>(vdt + 16 * e * BN);
        Od[e] = mfma16(va, PS, Od[e]);
        Od[e] = mfma16(vda, P[0], Od[e]);
      }
    } else {
      bf16x8 va[2];
      va[0] = *reinterpret_cast<const bf16x8 *>(vt);
#pragma unroll
      for (int e = 0; e < C::DT; ++e) {
        if (e + 1 < C::DT) va[(e + 1) & 1] = *reinterpret_cast<const bf16x8 *>(vt + 16 * (e + 1) * BN);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) O[mb][e] = mfma16(va[e & 1], P[mb], O[mb][e]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // any lane's own logits past its row's threshold (no lane exchange): the
  // lane's largest logit per row block from four three-way maxima, then one
  // compare (v_max3 ignores a quiet NaN operand, as the compare does).  Eight
  // compares per row block cost more VALU issue slots, which the forward
  // kernel is short of (teacher attention 2.5 % slower).
  auto outgrown = [&](const floatx4 (&S)[C::MB][2]) {
    // one ballot per compare: the compares' lane masks OR together in scalar
    // registers (a vote on an OR-ed bool first copies it to a vector register)
    uint64_t votes = 0;
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      const float m = max3f(max3f(S[mb][0][0], S[mb][0][1], S[mb][0][2]), max3f(S[mb][0][3], S[mb][1][0], S[mb][1][1]),
                            max3f(S[mb][1][2], S[mb][1][3], S[mb][1][3]));
      votes |= __builtin_amdgcn_ballot_w64(m > thr[mb]);
    }
    return votes != 0;
  };

  // Forward only: the normalised output of the keys seen so far into o2 (o's
  // strides), or for a piece, its partial result into the prefix bank.  Used
  // mid-loop for the prefix snapshot and not for the JVP.
  auto store_prefix = [&](void *dst) {
    if constexpr (!TAN) {
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        const int q_row = opaque(q_row0 + 16 * mb);
        if (ppart) {
          const float inv_l = 1.f / Lacc[mb][0];
          const int pi = 4 * (q_row - qb * C::BM) + g;
          *reinterpret_cast<float2 *>(ppart + 2 * pi) =
              make_float2(m_run[mb] * 0.6931471805599453f + logf(Lacc[mb][0]), 0.f);
#pragma unroll
          for (int e = 0; e < C::DT; ++e)
            *reinterpret_cast<float4 *>(ppart + C::PIECE_STATS + 4 * (e * C::MB * C::THREADS + pi)) =
                make_float4(O[mb][e][0] * inv_l, O[mb][e][1] * inv_l, O[mb][e][2] * inv_l, O[mb][e][3] * inv_l);
        } else if (q_row < p.Nq) {
          const float inv_l = 1.f / Lacc[mb][0];
          const int64_t obase = (int64_t)b * p.o_bs + (int64_t)q_row * p.o_rs + h * DH + 4 * g;
#pragma unroll
          for (int e = 0; e < C::DT; ++e) {
            if (p.out_dt == 0) {
              bf16x4 a;
#pragma unroll
              for (int r = 0; r < 4; ++r) a[r] = (bf16)(O[mb][e][r] * inv_l);
              *reinterpret_cast<bf16x4 *>(reinterpret_cast<bf16 *>(dst) + obase + 16 * e) = a;
            } else {
              *reinterpret_cast<float4 *>(reinterpret_cast<float *>(dst) + obase + 16 * e) =
                  make_float4(O[mb][e][0] * inv_l, O[mb][e][1] * inv_l, O[mb][e][2] * inv_l,
                              O[mb][e][3] * inv_l);
            }
          }
        }
      }
    }
  };

  // ---- main loop over 32-key sub-tiles of BN-key stages ----
  // The logits of sub-tile j+1 are computed in the same basic block as the
  // softmax of sub-tile j, so the matrix cores work while the VALU exponentiates.
  // Stage st's K sits in ring slot st % 3 and its V^T in slot st % 2.  The
  // sub-tiles of stage st read K of st (first) and of st+1 (second) and V^T of
  // st (both), so one barrier per stage, at its start, suffices: it publishes
  // K of st+1 and V^T of st (loaded during stage st-1) and frees the slots of
  // K and V^T of st-1, which then receive K of st+2 and V^T of st+1.
  const int nst = (nk + BN - 1) / BN;
  const int nsub = C::SUB * nst;
  issue_k(0, 0);
  wait_loads();
  __syncthreads();
  if (nst > 1) issue_k(1, BN);
  issue_v(0, 0);
  floatx4 S[C::MB][2], Sd[2];
  bf16x8 P[C::MB], PS;
  compute_s(0, 0, S, Sd);
  if (nst == 1) mask_s(0, S, Sd);
  // key 0 is always valid, so this is finite
  if constexpr (TAN) m_run[0] = row_max_arg(S[0], Sd, c_ref);
  else {
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) m_run[mb] = row_max(S[mb]);
  }
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) set_thr(mb);
  int j = 0;
  floatx4 Sn[C::MB][2], Sdn[2];
  // the prefix output (forward with o2) is stored between two runs of the
  // inner loop, after the sub-tile that ends at key nk_split, so the loop
  // body carries no store code
  bool prefix_due = !TAN && nk_split > 0;
  for (;;) {
    const int jend = prefix_due ? nk_split / 32 : nsub;
    for (; j < jend; ++j) {
      const int u = C::SUB == 2 ? (j & 1) : j % C::SUB, st = C::SUB == 2 ? (j >> 1) : j / C::SUB;
      if (outgrown(S)) break;   // rare: raise m_run outside
      if (u == 0) {
        wait_loads();
        __syncthreads();
        if (st + 2 < nst) issue_k((st + 2) % 3, (st + 2) * BN);
        if (st + 1 < nst) issue_v((st + 1) & 1, (st + 1) * BN);
      }
      // K of the next sub-tile (unused past the end).  The logit MFMAs and
      // the exponentials run at raised wave priority, so a wave that reaches
      // them issues ahead of waves busy in their P V products (forward 3 %,
      // JVP 1.7 % faster).
      __builtin_amdgcn_s_setprio(1);
      if constexpr (C::SUB == 2) compute_s(u == 0 ? st % 3 : (st + 1) % 3, u ^ 1, Sn, Sdn);
      else compute_s(((j + 1) / C::SUB) % 3, (j + 1) % C::SUB, Sn, Sdn);
      softmax(S, Sd, P, PS);
      __builtin_amdgcn_s_setprio(0);
      pv_accum(st & 1, u, P, PS);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) S[mb][t] = Sn[mb][t];
        if constexpr (TAN) Sd[t] = Sdn[t];
      }
      if (j + 1 < nsub && (C::SUB == 2 ? ((j + 1) >> 1) : (j + 1) / C::SUB) == nst - 1)
        mask_s(32 * (j + 1), S, Sd);
    }
    if (j >= jend) {
      if (!prefix_due) break;
      store_prefix(p.o2);
      prefix_due = false;
      continue;
    }
    // raise the reference max of the rows that outgrew it; rescale the
    // accumulators and re-centre the tangent weights on the new max key
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      float sd_max = 0.f;
      const float mx = TAN ? row_max_arg(S[mb], Sd, sd_max) : row_max(S[mb]);
      const float m_new = fmaxf(m_run[mb], mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run[mb] - m_new);
      const float c_new = (TAN && mx > m_run[mb]) ? sd_max : c_ref;
      const float delta = c_ref - c_new;   // dA += delta A, mu~ += delta l
      m_run[mb] = m_new;
      set_thr(mb);
      if constexpr (C::MFMA_SUMS) {
#pragma unroll
        for (int r = 0; r < 4; ++r) Lacc[mb][r] *= alpha;
      } else {
        if constexpr (TAN) mu_part = alpha * (mu_part + delta * l_part[mb]);
        l_part[mb] *= alpha;
      }
      if constexpr (TAN) c_ref = c_new;
#pragma unroll
      for (int e = 0; e < C::DT; ++e)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (TAN) Od[e][r] = alpha * __builtin_fmaf(delta, O[mb][e][r], Od[e][r]);
          O[mb][e][r] *= alpha;
        }
    }
  }

  // ---- epilogue: combine the four lanes of a row, normalise, store ----
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) {
  const int q_row = opaque(q_row0 + 16 * mb);
  float l_tot;
  if constexpr (C::MFMA_SUMS) {
    l_tot = Lacc[mb][0];
  } else {
    l_tot = l_part[mb] + __shfl_xor(l_part[mb], 16);
    l_tot += __shfl_xor(l_tot, 32);
  }
  const float inv_l = 1.f / l_tot;
  float mu = 0.f;
  if constexpr (TAN) {
    mu = mu_part + __shfl_xor(mu_part, 16);
    mu = (mu + __shfl_xor(mu, 32)) * inv_l;
  }
  const float lse = m_run[mb] * 0.6931471805599453f + logf(l_tot);
  if (part) {
    // a piece of a split tile: its own normalised result, for every row; the
    // mean tangent logit is mu (centred on c_ref) plus c_ref
    const int pi = 4 * (q_row - qb * C::BM) + g;
    *reinterpret_cast<float2 *>(part + 2 * pi) = make_float2(lse, TAN ? mu + c_ref : 0.f);
#pragma unroll
    for (int e = 0; e < C::DT; ++e) {
      float o4[4], od4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        o4[r] = O[mb][e][r] * inv_l;
        if constexpr (TAN) od4[r] = Od[e][r] * inv_l - mu * o4[r];
      }
      *reinterpret_cast<float4 *>(part + C::PIECE_STATS + 4 * (e * C::MB * C::THREADS + pi)) =
          make_float4(o4[0], o4[1], o4[2], o4[3]);
      if constexpr (TAN)
        *reinterpret_cast<float4 *>(part + C::PIECE_STATS + C::PIECE_O + 4 * (e * C::THREADS + pi)) =
            make_float4(od4[0], od4[1], od4[2], od4[3]);
    }
    continue;
  }
  if (q_row < p.Nq) {
    if (p.lse && g == 0) p.lse[((int64_t)b * p.H + h) * p.Nq + q_row] = lse;
    const int64_t obase = (int64_t)b * p.o_bs + (int64_t)q_row * p.o_rs + h * DH + 4 * g;
#pragma unroll
    for (int e = 0; e < C::DT; ++e) {
      float o4[4], od4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        o4[r] = O[mb][e][r] * inv_l;
        if constexpr (TAN) od4[r] = Od[e][r] * inv_l - mu * o4[r];
      }
      store_out4<TAN>(p, obase + 16 * e, o4, od4);
    }
  }
  }
}

// Merges the pieces of the split tiles (one workgroup per split tile and
// 16-column d-tile, each thread the rows and columns of that d-tile it held in
// the attention kernel).  A piece holds
// its own normalised result o_i, do_i, log-sum-exp and mean tangent logit
// mu_i; with w_i the softmax of the log-sum-exps over the pieces,
// o = sum w_i o_i, mu = sum w_i mu_i and do = sum w_i (do_i + (mu_i - mu) o_i)
// (each do_i is centred on its own mu_i).  Pieces are taken in key order, so
// the result does not depend on which finished first.
template <int DH, bool TAN, bool SPLIT>
__global__ __launch_bounds__((AttnCfg<DH, TAN, SPLIT>::THREADS), 1) void attn_combine_kernel(
    AttnParams p, int nqb, int per_xcd, int total, SplitArgs sp) {
  using C = AttnCfg<DH, TAN, SPLIT>;
  constexpr int BN = C::BN;
  const int slot = blockIdx.x;
  const int L = split_tile(slot, per_xcd, sp);
  if (L >= total) return;
  const int qb = L % nqb, bh = L / nqb;
  const int b = bh / p.H, h = bh % p.H;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int e = blockIdx.y;   // the d-tile this workgroup merges
  const float *part = p.part + (size_t)slot * sp.k * C::PIECE_FLOATS;
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) {
    const int row = wave * 16 * C::MB + 16 * mb + l16;   // within the tile
    const int q_row = qb * C::BM + row;
    if (q_row >= p.Nq) continue;
    const int pi = 4 * row + g;
    float lse[kMaxPieces], mu[kMaxPieces], wgt[kMaxPieces];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kMaxPieces; ++i) {
      lse[i] = -INFINITY;
      mu[i] = 0.f;
      if (i < sp.k) {
        const float2 v = *reinterpret_cast<const float2 *>(part + (size_t)i * C::PIECE_FLOATS + 2 * pi);
        lse[i] = v.x;
        mu[i] = v.y;
      }
      mx = fmaxf(mx, lse[i]);
    }
    float wsum = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPieces; ++i) {
      wgt[i] = expf(lse[i] - mx);   // 0 for an empty piece (and pieces past k)
      wsum += wgt[i];
    }
    const float inv = 1.f / wsum;
    float mu_all = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPieces; ++i) {
      wgt[i] *= inv;
      mu_all += wgt[i] * mu[i];
    }
    if (p.lse && g == 0 && e == 0) p.lse[((int64_t)b * p.H + h) * p.Nq + q_row] = mx + logf(wsum);
    const int64_t obase = (int64_t)b * p.o_bs + (int64_t)q_row * p.o_rs + h * DH + 4 * g;
    {
      float o4[4] = {0.f, 0.f, 0.f, 0.f}, od4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < kMaxPieces; ++i) {
        if (i >= sp.k) break;
        const float *pp = part + (size_t)i * C::PIECE_FLOATS + C::PIECE_STATS;
        const float4 a = *reinterpret_cast<const float4 *>(pp + 4 * (e * C::MB * C::THREADS + pi));
        const float av[4] = {a.x, a.y, a.z, a.w};
        float dv[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (TAN) {
          const float4 d = *reinterpret_cast<const float4 *>(pp + C::PIECE_O + 4 * (e * C::THREADS + pi));
          dv[0] = d.x; dv[1] = d.y; dv[2] = d.z; dv[3] = d.w;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          o4[r] += wgt[i] * av[r];
          if constexpr (TAN) od4[r] += wgt[i] * (dv[r] + (mu[i] - mu_all) * av[r]);
        }
      }
      store_out4<TAN>(p, obase + 16 * e, o4, od4);
    }
    if constexpr (!TAN) {
      if (p.o2) {
        // the output over the first nk_split keys: per piece its full partial
        // (keys all before nk_split), its prefix partial (the piece holding
        // the boundary) or nothing (keys all after)
        const int nk_b = min(max(p.nk[b], 1), p.Nk);
        float plse[kMaxPieces];
        const float *src[kMaxPieces];
        float pmx = -INFINITY;
#pragma unroll
        for (int i = 0; i < kMaxPieces; ++i) {
          plse[i] = -INFINITY;
          src[i] = nullptr;
          if (i < sp.k) {
            int s0, s1;
            piece_stages((nk_b + BN - 1) / BN, i, sp.k, s0, s1);
            const int k0 = s0 * BN, k1 = min(nk_b, s1 * BN);
            const float *bank0 = part + (size_t)i * C::PIECE_FLOATS;
            src[i] = k1 <= p.nk_split ? bank0
                     : (k0 < p.nk_split ? bank0 + (size_t)sp.pbank * C::PIECE_FLOATS : nullptr);
            if (src[i]) plse[i] = reinterpret_cast<const float2 *>(src[i] + 2 * pi)->x;
          }
          pmx = fmaxf(pmx, plse[i]);
        }
        float pw[kMaxPieces], psum = 0.f;
#pragma unroll
        for (int i = 0; i < kMaxPieces; ++i) {
          pw[i] = expf(plse[i] - pmx);
          psum += pw[i];
        }
        const float pinv = 1.f / psum;
        {
          float o4[4] = {0.f, 0.f, 0.f, 0.f}, unused[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < kMaxPieces; ++i) {
            if (!src[i]) continue;
            const float4 a = *reinterpret_cast<const float4 *>(src[i] + C::PIECE_STATS +
                                                               4 * (e * C::MB * C::THREADS + pi));
            const float w = pw[i] * pinv;
            o4[0] += w * a.x; o4[1] += w * a.y; o4[2] += w * a.z; o4[3] += w * a.w;
          }
          AttnParams q = p;
          q.o = p.o2;
          store_out4<false>(q, obase + 16 * e, o4, unused);
        }
      }
    }
  }
}



constexpr size_t kCapPieces = 768;   // scratch for at most this many pieces

template <int DH, bool TAN, bool SPLIT>
size_t split_bytes(int B, int H, int Nq, bool prefix) {
  using C = AttnCfg<DH, TAN, SPLIT>;
  const int64_t total = (int64_t)B * H * ((Nq + C::BM - 1) / C::BM);
  const size_t pieces = std::min<size_t>(kCapPieces, (size_t)kMaxPieces * 8 * ((total + 7) / 8));
  return pieces * C::PIECE_FLOATS * sizeof(float) * (prefix && !TAN ? 2 : 1);
}

template <int DH, bool TAN, bool SPLIT>
hipError_t launch_impl(const AttnParams &p, hipStream_t s) {
  using C = AttnCfg<DH, TAN, SPLIT>;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void *)attn_fwd_jvp_kernel<DH, TAN, SPLIT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int nqb = (p.Nq + C::BM - 1) / C::BM;
  const int total = nqb * p.H * p.B;
  const int per_xcd = (total + 7) / 8;
  // split the tail only with scratch; with the prefix output (forward) every
  // piece needs a second partial in the prefix bank
  const bool two_banks = !TAN && p.o2;
  const size_t cap =
      p.part ? p.part_bytes / (sizeof(float) * C::PIECE_FLOATS) / (two_banks ? 2 : 1) : 0;
  static int slots[kMaxDevices];
  SplitArgs sp =
      cap ? plan_split(per_xcd,
                       xcd_slots(attn_fwd_jvp_kernel<DH, TAN, SPLIT>, C::THREADS, C::LDS_BYTES, slots),
                       (p.Nk + C::BN - 1) / C::BN, cap, kMinPieceKeys / C::BN)
          : SplitArgs{per_xcd, 0, 1, 0};
  sp.pbank = 8 * sp.rem * sp.k;
  hipLaunchKernelGGL((attn_fwd_jvp_kernel<DH, TAN, SPLIT>), dim3(8 * (sp.n_full + sp.rem * sp.k)),
                     dim3(C::THREADS), C::LDS_BYTES, s, p, nqb, per_xcd, total, sp);
  if (sp.rem > 0) {
    if (hipError_t e = hipGetLastError()) return e;
    // one workgroup per (split tile, d-tile): a tile's pieces hold up to a few
    // MB of partials, which one workgroup alone would stream slowly
    hipLaunchKernelGGL((attn_combine_kernel<DH, TAN, SPLIT>), dim3(8 * sp.rem, C::DT), dim3(C::THREADS), 0, s, p,
                       nqb, per_xcd, total, sp);
  }
  return hipGetLastError();
}

template <int DH, bool SPLIT>
hipError_t launch_dh(bool tangent, const AttnParams &p, hipStream_t s) {
  return tangent ? launch_impl<DH, true, SPLIT>(p, s) : launch_impl<DH, false, SPLIT>(p, s);
}

template <int DH>
size_t split_bytes_dh(int B, int H, int Nq, bool prefix) {
  return std::max({split_bytes<DH, true, false>(B, H, Nq, prefix), split_bytes<DH, false, false>(B, H, Nq, prefix),
                   split_bytes<DH, true, true>(B, H, Nq, prefix), split_bytes<DH, false, true>(B, H, Nq, prefix)});
}

}  // namespace

hipError_t launch_attention(int dh, bool tangent, const AttnParams &p, hipStream_t s) {
  const bool split = p.q_lo != nullptr;
  if (split != (p.k_lo != nullptr)) return hipErrorInvalidValue;
  if (dh == 128) return split ? launch_dh<128, true>(tangent, p, s) : launch_dh<128, false>(tangent, p, s);
  if (dh == 64) return split ? launch_dh<64, true>(tangent, p, s) : launch_dh<64, false>(tangent, p, s);
  return hipErrorInvalidValue;
}

size_t attention_split_bytes(int dh, int B, int H, int Nq, bool prefix) {
  if (dh == 128) return split_bytes_dh<128>(B, H, Nq, prefix);
  if (dh == 64) return split_bytes_dh<64>(B, H, Nq, prefix);
  return 0;
}

}  // namespace t2va
