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
template <typename TA, typename TB, typename TO>
__global__ __launch_bounds__(kThreads) void trigflow_kernel(int op, CoefTable coef, int64_t n,
                                                            const TA *a, const TB *b,
                                                            const float *x, TO *out, int64_t a_bs,
                                                            int64_t b_bs, int64_t x_bs,
                                                            int64_t o_bs, int vec) {
  const int bi = blockIdx.y;
  const Coef c = coef.c[bi];
  const int64_t i0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * kPerThread;
  if (i0 >= n) return;
  a += bi * a_bs;
  b += bi * b_bs;
  out += bi * o_bs;
  float fa[8], fb[8], fx[8], fo[8];
  load_n(a, i0, n, vec, fa);
  load_n(b, i0, n, vec, fb);
  if (op == 2) load_n(x + bi * x_bs, i0, n, vec, fx);
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
  store_n(out, i0, n, vec, fo);
}

template <typename TA, typename TB, typename TO>
hipError_t trigflow_launch3(int op, const CoefTable &coef, int64_t n, const void *a, const void *b,
                            const float *x, void *out, int64_t a_bs, int64_t b_bs, int64_t x_bs,
                            int64_t o_bs, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const bool vec = (n % 8 == 0) && (a_bs % 8 == 0) && (b_bs % 8 == 0) && (o_bs % 8 == 0) &&
                   (x == nullptr || x_bs % 8 == 0);
  dim3 grid((unsigned)((n + kChunk - 1) / kChunk), coef.B);
  hipLaunchKernelGGL((trigflow_kernel<TA, TB, TO>), grid, dim3(kThreads), 0, s, op, coef, n,
                     (const TA *)a, (const TB *)b, x, (TO *)out, a_bs, b_bs, x_bs, o_bs, (int)vec);
  return hipGetLastError();
}

template <typename TA, typename TB>
hipError_t trigflow_launch2(int op, const CoefTable &coef, int64_t n, int out_dt, const void *a,
                            const void *b, const float *x, void *out, int64_t a_bs, int64_t b_bs,
                            int64_t x_bs, int64_t o_bs, hipStream_t s) {
  if (out_dt == 0)
    return trigflow_launch3<TA, TB, bf16>(op, coef, n, a, b, x, out, a_bs, b_bs, x_bs, o_bs, s);
  return trigflow_launch3<TA, TB, float>(op, coef, n, a, b, x, out, a_bs, b_bs, x_bs, o_bs, s);
}

template <typename TA>
hipError_t trigflow_launch1(int op, const CoefTable &coef, int64_t n, int b_dt, int out_dt,
                            const void *a, const void *b, const float *x, void *out, int64_t a_bs,
                            int64_t b_bs, int64_t x_bs, int64_t o_bs, hipStream_t s) {
  if (b_dt == 0)
    return trigflow_launch2<TA, bf16>(op, coef, n, out_dt, a, b, x, out, a_bs, b_bs, x_bs, o_bs, s);
  return trigflow_launch2<TA, float>(op, coef, n, out_dt, a, b, x, out, a_bs, b_bs, x_bs, o_bs, s);
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

// One wave per output feature i: tau[r][i] = sum_k W_t[i][k] E[r][k].
__global__ __launch_bounds__(kThreads) void time_linear_kernel(const float *E, int rows, int d,
                                                               const bf16 *w_t, float *tau) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= d) return;
  const bf16 *wr = w_t + (int64_t)i * d;
  for (int r = 0; r < rows; ++r) {
    const float *er = E + (int64_t)r * d;
    float acc = 0.f;
    for (int k0 = lane * 8; k0 < d; k0 += 64 * 8) {
      float w8[8], e8[8];
      load8(wr + k0, w8);
      load8(er + k0, e8);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += w8[j] * e8[j];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) tau[(int64_t)r * d + i] = acc;
  }
}

// ---------------------------------------------------------------------------
// Text rows: block (j, b) writes row Nq + j of sample b: the j-th valid text
// position if there is one, else zeros.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void text_rows_kernel(int Nq, int Nt, int d, const T *text,
                                                             const uint8_t *mask, bf16 *X,
                                                             int64_t x_bs, int zero_only,
                                                             int32_t *nk) {
  const int j = blockIdx.x, bi = blockIdx.y;
  __shared__ int src;
  __shared__ int count;
  if (threadIdx.x == 0) {
    int c = 0, found = -1;
    if (!zero_only) {
      const uint8_t *m = mask + (int64_t)bi * Nt;
      for (int i = 0; i < Nt; ++i) {
        if (m[i]) {
          if (c == j) found = i;
          ++c;
        }
      }
    }
    src = found;
    count = c;
  }
  __syncthreads();
  if (j == 0 && threadIdx.x == 0 && nk != nullptr) nk[bi] = Nq + count;
  bf16 *dst = X + (int64_t)bi * x_bs + (int64_t)(Nq + j) * d;
  if (src < 0) {
    for (int c0 = threadIdx.x * 8; c0 < d; c0 += kThreads * 8) {
      float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      store8(dst + c0, z);
    }
  } else {
    const T *row = text + ((int64_t)bi * Nt + src) * d;
    for (int c0 = threadIdx.x * 8; c0 < d; c0 += kThreads * 8) {
      float f[8];
      load8(row + c0, f);
      store8(dst + c0, f);
    }
  }
}

__global__ __launch_bounds__(kThreads) void cast_kernel(const float *src, bf16 *dst, int64_t n) {
  const int64_t i0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 8;
  if (i0 >= n) return;
  float f[8];
  load_n(src, i0, n, (n % 8) == 0, f);
  store_n(dst, i0, n, (n % 8) == 0, f);
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

hipError_t launch_trigflow(int op, const CoefTable &coef, int64_t n, int a_dt, int b_dt,
                           int out_dt, const void *a, const void *b, const float *x, void *out,
                           int64_t a_bs, int64_t b_bs, int64_t x_bs, int64_t out_bs,
                           hipStream_t s) {
  if (a_dt == 0)
    return trigflow_launch1<bf16>(op, coef, n, b_dt, out_dt, a, b, x, out, a_bs, b_bs, x_bs, out_bs, s);
  return trigflow_launch1<float>(op, coef, n, b_dt, out_dt, a, b, x, out, a_bs, b_bs, x_bs, out_bs, s);
}

hipError_t launch_time_embedding(const CoefTable &coef, int d, float *E, hipStream_t s) {
  dim3 grid((d / 2 + kThreads - 1) / kThreads, coef.B);
  hipLaunchKernelGGL(time_embedding_kernel, grid, dim3(kThreads), 0, s, coef, d, E);
  return hipGetLastError();
}

hipError_t launch_time_linear(const float *E, int rows, int d, const bf16 *w_t, float *tau,
                              hipStream_t s) {
  hipLaunchKernelGGL(time_linear_kernel, dim3((d + 3) / 4), dim3(kThreads), 0, s, E, rows, d, w_t, tau);
  return hipGetLastError();
}

hipError_t launch_text_rows(int B, int Nq, int Nt, int d, const void *text, int text_dt,
                            const uint8_t *mask, bf16 *X, int64_t x_batch_stride, int zero_only,
                            int32_t *nk, hipStream_t s) {
  if (Nt == 0) return hipSuccess;  // no text rows; the host sets nk = Nq itself
  dim3 grid(Nt, B);
  if (text_dt == 0)
    hipLaunchKernelGGL(text_rows_kernel<bf16>, grid, dim3(kThreads), 0, s, Nq, Nt, d,
                       (const bf16 *)text, mask, X, x_batch_stride, zero_only, nk);
  else
    hipLaunchKernelGGL(text_rows_kernel<float>, grid, dim3(kThreads), 0, s, Nq, Nt, d,
                       (const float *)text, mask, X, x_batch_stride, zero_only, nk);
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

hipError_t launch_cast_bf16(const float *src, bf16 *dst, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n + kChunk - 1) / kChunk);
  hipLaunchKernelGGL(cast_kernel, dim3(blocks), dim3(kThreads), 0, s, src, dst, n);
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
