// HBM-bound kernels of the joint sCM target and the joint DMD term: TrigFlow
// noising and fields, the sinusoidal time embedding, text-key compaction, the
// sCM direction with its per-block sums of squares, the guided DMD direction
// with its per-block sums, and the normalisations with the losses.
//
// Method: TurboT2VA deep read (robotworld.top, arXiv 2608.24674), section 3
// (noising) and section 3.1 (fields, joint JVP, sCM direction, per-sample
// per-modality L2 normalisation, residual, joint loss); section 4 (DMD
// direction with a guided teacher, residual-scale normaliser, summed loss),
// 4.1 (stage-3 mix); section 6.3 (padded text positions are removed before
// attention).
#include "common.h"

namespace t2va {

namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 8;
constexpr int kChunk = kThreads * kPerThread;  // elements per block

template <typename T>
__device__ __forceinline__ void load_n(const T *p, int64_t i0, int64_t n, bool vec, float *f) {
  if (vec && i0 + kPerThread <= n) {
    load8(p + i0, f);
  } else {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) f[j] = (i0 + j < n) ? to_f32(p[i0 + j]) : 0.f;
  }
}

template <typename T>
__device__ __forceinline__ void store_n(T *p, int64_t i0, int64_t n, bool vec, const float *f) {
  if (vec && i0 + kPerThread <= n) {
    store8(p + i0, f);
  } else {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
      if (i0 + j < n) p[i0 + j] = Store<T>::cvt(f[j]);
  }
}

// op 0: r (cos a + sin b); op 1: (cos a - b)/sin; op 2: with z = cos a + sin b and
// the teacher's x0-prediction x0 = rf ? r z - t_emb x : x, F_T = (cos z - x0)/sin
// and out = r F_T + rdot z (the tangent of the student's token input).
template <typename TA, typename TB, typename TO, bool SPLIT_ROWS = false>
__global__ __launch_bounds__(kThreads) void trigflow_kernel(int op, CoefTable coef, TrigSeg s1, TrigSeg s2,
                                                            int blocks1) {
  // the first blocks1 blocks of each sample's row take segment 1, the rest segment 2
  const bool second = (int)blockIdx.x >= blocks1;
  const TrigSeg &sg = second ? s2 : s1;
  const int bi = blockIdx.y;
  const Coef c = coef.c[bi];
  const int64_t n = sg.n;
  const int64_t i0 = ((int64_t)((int)blockIdx.x - (second ? blocks1 : 0)) * kThreads + threadIdx.x) * kPerThread;
  if (i0 >= n) return;
  const TA *a = (const TA *)sg.a + bi * sg.a_bs;
  const TB *b = (const TB *)sg.b + bi * sg.b_bs;
  TO *out = (TO *)sg.out + bi * sg.o_bs;
  const int vec = sg.vec;
  float fa[8], fb[8], fx[8], fo[8];
  load_n(a, i0, n, vec, fa);
  load_n(b, i0, n, vec, fb);
  if (op == 2) load_n(sg.x + bi * sg.x_bs, i0, n, vec, fx);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (op == 0) {
      fo[j] = c.r * (c.cos_t * fa[j] + c.sin_t * fb[j]);
    } else if (op == 1) {
      fo[j] = (c.cos_t * fa[j] - fb[j]) * c.inv_sin;
    } else {
      const float z = c.cos_t * fa[j] + c.sin_t * fb[j];
      const float x0 = coef.rf ? c.r * z - c.t_emb * fx[j] : fx[j];
      const float F = (c.cos_t * z - x0) * c.inv_sin;
      fo[j] = coef.rf ? c.r * F + c.rdot * z : F;
    }
  }
  if constexpr (SPLIT_ROWS) {
    // the 8 values lie in one row (w and i0 multiples of 8)
    const int64_t r = i0 / sg.w, col = i0 - r * sg.w;
    bf16 *o = reinterpret_cast<bf16 *>(out) + r * 3 * sg.w + col;
    float lo[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) lo[j] = fo[j] - (float)(bf16)fo[j];
    store8(o, fo);
    store8(o + sg.w, lo);
    store8(o + 2 * sg.w, fo);
  } else {
    store_n(out, i0, n, vec, fo);
  }
}

template <typename TA, typename TB, typename TO, bool SPLIT_ROWS = false>
hipError_t trigflow_launch3(int op, const CoefTable &coef, TrigSeg s1, TrigSeg s2, hipStream_t s) {
  for (TrigSeg *g : {&s1, &s2}) {
    g->vec = (g->n % 8 == 0) && (g->a_bs % 8 == 0) && (g->b_bs % 8 == 0) && (g->o_bs % 8 == 0) &&
             (g->x == nullptr || g->x_bs % 8 == 0);
    if (SPLIT_ROWS && g->n > 0 && (!g->vec || g->w <= 0 || g->w % 8 || g->n % g->w)) return hipErrorInvalidValue;
  }
  const int b1 = (int)((max(s1.n, (int64_t)0) + kChunk - 1) / kChunk);
  const int b2 = (int)((max(s2.n, (int64_t)0) + kChunk - 1) / kChunk);
  if (b1 + b2 == 0) return hipSuccess;
  hipLaunchKernelGGL((trigflow_kernel<TA, TB, TO, SPLIT_ROWS>), dim3(b1 + b2, coef.B), dim3(kThreads), 0, s, op,
                     coef, s1, s2, b1);
  return hipGetLastError();
}

template <typename TA, typename TB>
hipError_t trigflow_launch2(int op, const CoefTable &coef, int out_dt, const TrigSeg &s1, const TrigSeg &s2,
                            hipStream_t s) {
  if (out_dt == 0) return trigflow_launch3<TA, TB, bf16>(op, coef, s1, s2, s);
  if (out_dt == kTrigSplitRows) return trigflow_launch3<TA, TB, bf16, true>(op, coef, s1, s2, s);
  return trigflow_launch3<TA, TB, float>(op, coef, s1, s2, s);
}

template <typename TA>
hipError_t trigflow_launch1(int op, const CoefTable &coef, int b_dt, int out_dt, const TrigSeg &s1,
                            const TrigSeg &s2, hipStream_t s) {
  if (b_dt == 0) return trigflow_launch2<TA, bf16>(op, coef, out_dt, s1, s2, s);
  return trigflow_launch2<TA, float>(op, coef, out_dt, s1, s2, s);
}

// ---------------------------------------------------------------------------
// Time embedding: e_k = cos(s w_k), e_{d/2+k} = sin(s w_k), w_k = 10000^(-k/(d/2)),
// at the block's time input s = t_emb, and its derivative along dt = 1
// (de/ds * t_emb_dot).  Rows 0..B-1 hold e, rows B..2B-1 the derivative.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void time_embedding_kernel(CoefTable coef, int d, float *E) {
  const int half = d / 2;
  const int k = blockIdx.x * kThreads + threadIdx.x;
  const int bi = blockIdx.y;
  if (k >= half) return;
  const float w = exp2f(-(float)k / (float)half * 13.287712379549449f);  // log2(10000)
  const float arg = coef.c[bi].t_emb * w;
  const float wd = w * coef.c[bi].t_emb_dot;
  float sn, cs;
  sincosf(arg, &sn, &cs);
  float *e = E + (int64_t)bi * d;
  float *de = E + (int64_t)(coef.B + bi) * d;
  e[k] = cs;
  e[half + k] = sn;
  de[k] = -wd * sn;
  de[half + k] = wd * cs;
}

// One wave per output feature i: out[r][i] = sum_k W[i][k] E[r][k] (W [n_out][d]),
// for two independent problems in one launch: blocks [0, blocks1) compute
// problem 1, the rest problem 2 (same d and n_out).
__global__ __launch_bounds__(kThreads) void time_linear_kernel(int d, int n_out, RowLinSeg s1, RowLinSeg s2,
                                                               int blocks1) {
  const bool second = (int)blockIdx.x >= blocks1;
  const float *E = second ? s2.E : s1.E;
  const bf16 *w_t = second ? s2.W : s1.W;
  float *tau = second ? s2.out : s1.out;
  const int rows = second ? s2.rows : s1.rows;
  const int lane = threadIdx.x & 63;
  const int i = ((int)blockIdx.x - (second ? blocks1 : 0)) * 4 + (threadIdx.x >> 6);
  if (i >= n_out) return;
  const bf16 *wr = w_t + (int64_t)i * d;
  // rows in groups of kR: each weight chunk is read once per group, and the
  // group's kR sums are reduced together (independent shuffle chains)
  constexpr int kR = 8;
  for (int r0 = 0; r0 < rows; r0 += kR) {
    float acc[kR];
#pragma unroll
    for (int q = 0; q < kR; ++q) acc[q] = 0.f;
    for (int k0 = lane * 8; k0 < d; k0 += 64 * 8) {
      float w8[8];
      load8(wr + k0, w8);
#pragma unroll
      for (int q = 0; q < kR; ++q) {
        if (r0 + q < rows) {
          float e8[8];
          load8(E + (int64_t)(r0 + q) * d + k0, e8);
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[q] += w8[j] * e8[j];
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
      for (int q = 0; q < kR; ++q) acc[q] += __shfl_xor(acc[q], off);
    if (lane == 0) {
#pragma unroll
      for (int q = 0; q < kR; ++q)
        if (r0 + q < rows) tau[(int64_t)(r0 + q) * n_out + i] = acc[q];
    }
  }
}

// ---------------------------------------------------------------------------
// Text rows: block (j, b) writes row Nq + j of sample b: the j-th valid text
// position if there is one, else zeros.  With split, the row holds the value
// rounded to bf16 in columns [0, d) and the rounding remainder, rounded to
// bf16, in columns [d, 2d).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void text_rows_kernel(int Nq, int Nt, int d, const T *text,
                                                             const uint8_t *mask, bf16 *X,
                                                             int64_t x_bs, int64_t x_rs, int split,
                                                             int copy_b, int32_t *nk) {
  const int j = blockIdx.x, bi = blockIdx.y;
  const bool zero_only = bi >= copy_b;   // a tangent problem: zero text rows
  __shared__ int src;
  __shared__ int count;
  if (threadIdx.x < 64) {
    // the first wave ranks the valid positions 64 at a time: position i of
    // this chunk is valid row c + (valid lanes below it)
    const int lane = threadIdx.x;
    const uint64_t below = (1ull << lane) - 1;
    int c = 0, found = -1;
    if (!zero_only) {
      const uint8_t *m = mask + (int64_t)bi * Nt;
      for (int base = 0; base < Nt; base += 64) {
        const int i = base + lane;
        const bool v = i < Nt && m[i] != 0;
        const uint64_t bal = __ballot(v);
        if (v && c + __popcll(bal & below) == j) found = i;
        c += __popcll(bal);
      }
    }
    const uint64_t hit = __ballot(found >= 0);   // at most one lane
    const int from = hit ? __ffsll((unsigned long long)hit) - 1 : 0;
    const int f = __shfl(found, from);             // every lane takes part
    if (lane == 0) {
      src = hit ? f : -1;
      count = c;
    }
  }
  __syncthreads();
  if (j == 0 && threadIdx.x == 0 && nk != nullptr && !zero_only) nk[bi] = Nq + count;
  bf16 *dst = X + (int64_t)bi * x_bs + (int64_t)(Nq + j) * x_rs;
  const T *row = src < 0 ? nullptr : text + ((int64_t)bi * Nt + src) * d;
  for (int c0 = threadIdx.x * 8; c0 < d; c0 += kThreads * 8) {
    float f[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (row) load8(row + c0, f);
    store8(dst + c0, f);
    if (split) {
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] -= (float)(bf16)f[i];
      store8(dst + d + c0, f);
    }
  }
}

// Guided attention output: u + s (c - u) per element, s by the row's modality.
__global__ __launch_bounds__(kThreads) void guide_kernel(const float *c, const float *u, bf16 *out, int64_t per,
                                                         int D, int Nv, float s_v, float s_a) {
  const int64_t i0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 8;
  if (i0 >= per) return;
  const int64_t at = (int64_t)blockIdx.y * per + i0;
  const float sc = (i0 / D) < Nv ? s_v : s_a;   // D is a multiple of 8: one row per group
  float fc[8], fu[8];
  load8(c + at, fc);
  load8(u + at, fu);
#pragma unroll
  for (int i = 0; i < 8; ++i) fc[i] = fu[i] + sc * (fc[i] - fu[i]);
  store8(out + at, fc);
}

// [W | W]: row i of W2 holds row i of W twice.
__global__ __launch_bounds__(kThreads) void dup_cols_kernel(const bf16 *W0, const bf16 *W1, bf16 *D0, bf16 *D1,
                                                            int n, int k) {
  const bf16 *W = blockIdx.y ? W1 : W0;   // problem blockIdx.y
  bf16 *W2 = blockIdx.y ? D1 : D0;
  const int64_t i0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 8;
  if (i0 >= (int64_t)n * k) return;
  const int64_t r = i0 / k, c = i0 - r * k;
  const uint4 v = *reinterpret_cast<const uint4 *>(W + i0);
  *reinterpret_cast<uint4 *>(W2 + r * 2 * k + c) = v;
  *reinterpret_cast<uint4 *>(W2 + r * 2 * k + k + c) = v;
}

// Folded weights from split-K partials: part [splits][rows][Cv + Ca] fp32,
// summed over the splits in order.  bf16: Wf [rows][Cv + Ca].  split: per
// modality [rows][3 C_m] = [hi | hi | lo] (video first, audio at 3 rows Cv).
__global__ __launch_bounds__(kThreads) void fold_finish_kernel(const float *part, int splits, int rows, int Cv,
                                                               int Ca, bool split, bf16 *Wf, int64_t part_bs,
                                                               int64_t wf_bs) {
  part += blockIdx.y * part_bs;   // block blockIdx.y of the launch
  Wf += blockIdx.y * wf_bs;
  const int CC = Cv + Ca;
  const int64_t n = (int64_t)rows * CC;
  const int64_t i0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 8;
  if (i0 >= n) return;
  float f[8], g[8];
  load8(part + i0, f);
  for (int k = 1; k < splits; ++k) {
    load8(part + (int64_t)k * n + i0, g);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] += g[i];
  }
  if (!split) {
    store8(Wf + i0, f);
    return;
  }
  const int64_t r = i0 / CC;
  const int c = (int)(i0 - r * CC);   // Cv, Ca multiples of 8: the group stays in one modality
  const bool vid = c < Cv;
  const int cm = vid ? Cv : Ca, j = vid ? c : c - Cv;
  bf16 *o = Wf + (vid ? 0 : (int64_t)3 * rows * Cv) + r * 3 * cm + j;
  float lo[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) lo[i] = f[i] - (float)(bf16)f[i];
  store8(o, f);
  store8(o + cm, f);
  store8(o + 2 * cm, lo);
}

// Up to kMaxCasts fp32 -> bf16 copies in one launch: segment k owns blocks
// [start[k], start[k + 1]).
__global__ __launch_bounds__(kThreads) void cast_set_kernel(CastSet cs) {
  int k = 0;
  while (k + 1 < cs.count && (int64_t)blockIdx.x >= cs.start[k + 1]) ++k;
  const int64_t n = cs.n[k];
  const int64_t i0 = (((int64_t)blockIdx.x - cs.start[k]) * kThreads + threadIdx.x) * 8;
  if (i0 >= n) return;
  float f[8];
  load_n(cs.src[k], i0, n, (n % 8) == 0, f);
  store_n(cs.dst[k], i0, n, (n % 8) == 0, f);
}

// ---------------------------------------------------------------------------
// Deterministic block reduction (fixed order): wave butterfly, then waves in order.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ T block_sum(T v, T *smem) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) smem[w] = v;
  __syncthreads();
  T r = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) r += smem[i];
  return r;
}

// g = boost (F_T - F_S) - gamma c_t z_t - J with
//   F_T - F_S = (x0_S - x0_T)/sin t,
//   J = c_t dF_S = -c_t z_t + cos^2 t (F_T - F_S) - cos t dG,
// the closed form of the JVP of F_S = (cos t z - G(z, t))/sin t along
// (dt = 1, dz = F_T) given dG, the JVP of G.
template <typename T>
__global__ __launch_bounds__(kThreads) void scm_direction_kernel(CoefTable coef, GParams p) {
  __shared__ float red[kThreads / 64];
  int blk = blockIdx.x;
  const int m = (blk >= coef.B * p.nblk[0]) ? 1 : 0;
  if (m) blk -= coef.B * p.nblk[0];
  const int bi = blk / p.nblk[m], cb = blk % p.nblk[m];
  const Coef c = coef.c[bi];
  const int64_t n = p.n[m];
  const int64_t off = (int64_t)bi * n;
  const int64_t xo = (int64_t)bi * p.x_bs[m];
  const int64_t i0 = (int64_t)cb * kChunk + threadIdx.x * kPerThread;
  float ss = 0.f;
  if (i0 < n) {  // n is a multiple of 64: whole 8-element groups
    float z0[8], ep[8], xt[8], xs[8], gd[8], J[8], g[8];
    load8((const T *)p.z0[m] + off + i0, z0);
    load8((const T *)p.eps[m] + off + i0, ep);
    load8(p.x0T[m] + xo + i0, xt);
    load8(p.x0S[m] + xo + i0, xs);
    load8(p.Gd[m] + xo + i0, gd);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float z = c.cos_t * z0[j] + c.sin_t * ep[j];
      if (coef.rf) {
        // velocities -> x0-predictions through the wrapper, and the JVP of x0_S
        const float zin = c.r * z;
        xt[j] = zin - c.t_emb * xt[j];
        const float FT = (c.cos_t * z - xt[j]) * c.inv_sin;
        gd[j] = (c.r * FT + c.rdot * z) - c.t_emb_dot * xs[j] - c.t_emb * gd[j];
        xs[j] = zin - c.t_emb * xs[j];
      }
      const float D = (xs[j] - xt[j]) * c.inv_sin;
      J[j] = -c.ct_st * z + c.cos2 * D - c.cos_t * gd[j];
      g[j] = c.boost * D - c.gamma_ct_st * z - J[j];
      ss += g[j] * g[j];
    }
    if (p.J[m]) store8(p.J[m] + off + i0, J);
    store8(p.g[m] + off + i0, g);
  }
  const float tot = block_sum(ss, red);
  if (threadIdx.x == 0) p.partial[m][(int64_t)bi * p.nblk[m] + cb] = tot;
}

// Guided teacher prediction, DMD direction g = x0_F - x0_T, and per-block sums
// of |x0 - x0_T| (the residual scale's numerator) and of g^2.
template <typename T>
__global__ __launch_bounds__(kThreads) void dmd_direction_kernel(CoefTable coef, DmdParams p) {
  __shared__ float red[kThreads / 64];
  const int B = coef.B;
  int blk = blockIdx.x;
  const int m = (blk >= B * p.nblk[0]) ? 1 : 0;
  if (m) blk -= B * p.nblk[0];
  const int bi = blk / p.nblk[m], cb = blk % p.nblk[m];
  const int64_t n = p.n[m];
  const int64_t off = (int64_t)bi * n;
  const int64_t xo = (int64_t)bi * p.x_bs[m];
  const int64_t i0 = (int64_t)cb * kChunk + threadIdx.x * kPerThread;
  float sa = 0.f, ss = 0.f;
  if (i0 < n) {  // n is a multiple of 64: whole 8-element groups
    float x0[8], tc[8], tu[8], fk[8], g[8];
    load8((const T *)p.x0[m] + off + i0, x0);
    load8(p.tc[m] + xo + i0, tc);
    load8(p.fk[m] + xo + i0, fk);
    if (p.tu[m]) {
      load8(p.tu[m] + xo + i0, tu);
#pragma unroll
      for (int j = 0; j < 8; ++j) tc[j] = tu[j] + p.scale[m] * (tc[j] - tu[j]);
    }
    if (coef.rf) {
      // velocities -> x0-predictions through the wrapper (affine, so guidance
      // commutes with it): x0 = r z_t - t_rf v
      const Coef c = coef.c[bi];
      float ep[8];
      load8((const T *)p.eps[m] + off + i0, ep);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float zin = c.r * (c.cos_t * x0[j] + c.sin_t * ep[j]);
        tc[j] = zin - c.t_emb * tc[j];
        fk[j] = zin - c.t_emb * fk[j];
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      g[j] = fk[j] - tc[j];
      sa += fabsf(x0[j] - tc[j]);
      ss += g[j] * g[j];
    }
    store8(p.g[m] + off + i0, g);
  }
  const float ta = block_sum(sa, red);
  const float ts = block_sum(ss, red);
  if (threadIdx.x == 0) {
    p.part_abs[m][(int64_t)bi * p.nblk[m] + cb] = ta;
    p.part_sq[m][(int64_t)bi * p.nblk[m] + cb] = ts;
  }
}

__device__ __forceinline__ double sum_partials(const float *pp, int nblk, double *red) {
  double acc = 0.0;
  for (int i = threadIdx.x; i < nblk; i += kThreads) acc += (double)pp[i];
  return block_sum(acc, red);
}

__global__ __launch_bounds__(kThreads) void normalise_kernel(int B, NormParams p) {
  __shared__ double red[kThreads / 64];
  int blk = blockIdx.x;
  const int m = (blk >= B * p.nblk[0]) ? 1 : 0;
  if (m) blk -= B * p.nblk[0];
  const int bi = blk / p.nblk[m], cb = blk % p.nblk[m];
  double S[2], Q[2], scl[2];
#pragma unroll
  for (int mm = 0; mm < 2; ++mm) {
    S[mm] = sum_partials(p.partial[mm] + (int64_t)bi * p.nblk[mm], p.nblk[mm], red);
    if (p.mode == 0) {
      Q[mm] = S[mm];
      scl[mm] = sqrt(S[mm]);
    } else {
      Q[mm] = sum_partials(p.partial2[mm] + (int64_t)bi * p.nblk[mm], p.nblk[mm], red);
      scl[mm] = S[mm] / (double)p.n[mm];
    }
  }
  const float inv = (float)(1.0 / (scl[m] + p.eps));
  if (m == 0 && cb == 0 && threadIdx.x == 0) {
    if (p.norms) {
      p.norms[2 * bi] = (float)scl[0];
      p.norms[2 * bi + 1] = (float)scl[1];
    }
    p.loss[bi] = (float)(p.w[0] * Q[0] / ((scl[0] + p.eps) * (scl[0] + p.eps)) +
                         p.w[1] * Q[1] / ((scl[1] + p.eps) * (scl[1] + p.eps)));
  }
  const int64_t n = p.n[m];
  const int64_t i0 = (int64_t)cb * kChunk + threadIdx.x * kPerThread;
  if (i0 < n) {
    float *g = p.g[m] + (int64_t)bi * n + i0;
    float f[8];
    load8(g, f);
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] *= inv;
    store8(g, f);
    if (p.r[m]) {
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = -f[j];
      store8(p.r[m] + (int64_t)bi * n + i0, f);
    }
  }
}

}  // namespace

int elementwise_blocks(int64_t n) { return (int)((n + kChunk - 1) / kChunk); }

hipError_t launch_trigflow_pair(int op, const CoefTable &coef, int a_dt, int b_dt, int out_dt, const TrigSeg &s1,
                                const TrigSeg &s2, hipStream_t s) {
  if (a_dt == 0) return trigflow_launch1<bf16>(op, coef, b_dt, out_dt, s1, s2, s);
  return trigflow_launch1<float>(op, coef, b_dt, out_dt, s1, s2, s);
}

hipError_t launch_trigflow(int op, const CoefTable &coef, int64_t n, int a_dt, int b_dt,
                           int out_dt, const void *a, const void *b, const float *x, void *out,
                           int64_t a_bs, int64_t b_bs, int64_t x_bs, int64_t out_bs,
                           hipStream_t s) {
  const TrigSeg s1{a, b, x, out, n, a_bs, b_bs, x_bs, out_bs, 0};
  const TrigSeg none{nullptr, nullptr, nullptr, nullptr, 0, 0, 0, 0, 0, 0};
  return launch_trigflow_pair(op, coef, a_dt, b_dt, out_dt, s1, none, s);
}

hipError_t launch_time_embedding(const CoefTable &coef, int d, float *E, hipStream_t s) {
  dim3 grid((d / 2 + kThreads - 1) / kThreads, coef.B);
  hipLaunchKernelGGL(time_embedding_kernel, grid, dim3(kThreads), 0, s, coef, d, E);
  return hipGetLastError();
}

hipError_t launch_row_linear_pair(int d, int n_out, const RowLinSeg &s1, const RowLinSeg &s2, hipStream_t s) {
  const int per = (n_out + 3) / 4;
  const int blocks1 = s1.rows > 0 ? per : 0, blocks2 = s2.rows > 0 ? per : 0;
  if (blocks1 + blocks2 == 0) return hipSuccess;
  hipLaunchKernelGGL(time_linear_kernel, dim3(blocks1 + blocks2), dim3(kThreads), 0, s, d, n_out, s1, s2, blocks1);
  return hipGetLastError();
}

hipError_t launch_text_rows(int B, int Nq, int Nt, int d, const void *text, int text_dt,
                            const uint8_t *mask, bf16 *X, int64_t x_batch_stride, int64_t x_row_stride,
                            int split, int copy_b, int32_t *nk, hipStream_t s) {
  if (Nt == 0) return hipSuccess;  // no text rows; the host sets nk = Nq itself
  dim3 grid(Nt, B);
  if (text_dt == 0)
    hipLaunchKernelGGL(text_rows_kernel<bf16>, grid, dim3(kThreads), 0, s, Nq, Nt, d,
                       (const bf16 *)text, mask, X, x_batch_stride, x_row_stride, split, copy_b, nk);
  else
    hipLaunchKernelGGL(text_rows_kernel<float>, grid, dim3(kThreads), 0, s, Nq, Nt, d,
                       (const float *)text, mask, X, x_batch_stride, x_row_stride, split, copy_b, nk);
  return hipGetLastError();
}

hipError_t launch_fold_finish(const float *part, int splits, int rows, int Cv, int Ca, bool split, bf16 *Wf,
                              int nblk, int64_t part_bs, int64_t wf_bs, hipStream_t s) {
  const int64_t total = (int64_t)rows * (Cv + Ca);
  if (total <= 0 || nblk <= 0) return hipSuccess;
  hipLaunchKernelGGL(fold_finish_kernel, dim3((unsigned)((total + kChunk - 1) / kChunk), nblk), dim3(kThreads), 0,
                     s, part, splits, rows, Cv, Ca, split, Wf, part_bs, wf_bs);
  return hipGetLastError();
}

hipError_t launch_guide(const float *c, const float *u, bf16 *out, int B, int Nq, int Nv, int D, float s_v,
                        float s_a, hipStream_t s) {
  const int64_t per = (int64_t)Nq * D;
  if (per <= 0 || B <= 0) return hipSuccess;
  dim3 grid((unsigned)((per + kChunk - 1) / kChunk), B);
  hipLaunchKernelGGL(guide_kernel, grid, dim3(kThreads), 0, s, c, u, out, per, D, Nv, s_v, s_a);
  return hipGetLastError();
}

hipError_t launch_dup_cols(const bf16 *W0, const bf16 *W1, bf16 *D0, bf16 *D1, int n, int k, hipStream_t s) {
  const int64_t total = (int64_t)n * k;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(dup_cols_kernel, dim3((unsigned)((total + kChunk - 1) / kChunk), W1 ? 2 : 1), dim3(kThreads), 0,
                     s, W0, W1, D0, D1, n, k);
  return hipGetLastError();
}

namespace {
__global__ void fill_nk_kernel(int32_t *nk, int B, int v) {
  const int i = threadIdx.x;
  if (i < B) nk[i] = v;
}
}  // namespace

hipError_t launch_fill_nk(int32_t *nk, int B, int value, hipStream_t s) {
  hipLaunchKernelGGL(fill_nk_kernel, dim3(1), dim3(64), 0, s, nk, B, value);
  return hipGetLastError();
}

hipError_t launch_cast_set(const float *const *src, bf16 *const *dst, const int64_t *n, int count, hipStream_t s) {
  if (count < 0 || count > kMaxCasts) return hipErrorInvalidValue;
  CastSet cs = {};
  int64_t blocks = 0;
  for (int k = 0; k < count; ++k) {
    cs.src[cs.count] = src[k];
    cs.dst[cs.count] = dst[k];
    cs.n[cs.count] = n[k];
    cs.start[cs.count] = blocks;
    if (n[k] <= 0) continue;   // nothing to copy: no segment
    blocks += (n[k] + kChunk - 1) / kChunk;
    ++cs.count;
  }
  if (blocks == 0) return hipSuccess;
  cs.start[cs.count] = blocks;
  hipLaunchKernelGGL(cast_set_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, cs);
  return hipGetLastError();
}

hipError_t launch_scm_direction(const CoefTable &coef, const GParams &p, hipStream_t s) {
  const unsigned blocks = (unsigned)(coef.B * (p.nblk[0] + p.nblk[1]));
  if (p.in_dt == 0)
    hipLaunchKernelGGL(scm_direction_kernel<bf16>, dim3(blocks), dim3(kThreads), 0, s, coef, p);
  else
    hipLaunchKernelGGL(scm_direction_kernel<float>, dim3(blocks), dim3(kThreads), 0, s, coef, p);
  return hipGetLastError();
}

hipError_t launch_dmd_direction(const CoefTable &coef, const DmdParams &p, hipStream_t s) {
  const unsigned blocks = (unsigned)(coef.B * (p.nblk[0] + p.nblk[1]));
  if (p.in_dt == 0)
    hipLaunchKernelGGL(dmd_direction_kernel<bf16>, dim3(blocks), dim3(kThreads), 0, s, coef, p);
  else
    hipLaunchKernelGGL(dmd_direction_kernel<float>, dim3(blocks), dim3(kThreads), 0, s, coef, p);
  return hipGetLastError();
}

namespace {
__global__ void mix_kernel(int B, float a, const float *x, float c, const float *y, float *out) {
  const int i = threadIdx.x;
  if (i < B) out[i] = a * x[i] + c * y[i];
}
}  // namespace

hipError_t launch_mix(int B, float a, const float *x, float c, const float *y, float *out,
                      hipStream_t s) {
  hipLaunchKernelGGL(mix_kernel, dim3(1), dim3(64), 0, s, B, a, x, c, y, out);
  return hipGetLastError();
}

hipError_t launch_normalise(int B, const NormParams &p, hipStream_t s) {
  const unsigned blocks = (unsigned)(B * (p.nblk[0] + p.nblk[1]));
  hipLaunchKernelGGL(normalise_kernel, dim3(blocks), dim3(kThreads), 0, s, B, p);
  return hipGetLastError();
}

}  // namespace t2va
