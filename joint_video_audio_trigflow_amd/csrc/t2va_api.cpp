// Host side of libt2va: argument validation, workspace layouts, the launch
// sequences of the joint sCM target and the joint DMD term, and phase timing.
//
// Method: TurboT2VA deep read (robotworld.top, arXiv 2608.24674), sections 3
// and 3.1 (sCM), 4 and 4.1 (DMD, stage-3 mix); the block G and its JVP as
// described in t2va.h.
#include "../../include/t2va.h"
#include "common.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

using namespace t2va;

namespace {

thread_local std::string g_err;

t2va_status fail(t2va_status code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

t2va_status hip_fail(hipError_t e, const char *what) {
  return fail(T2VA_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(expr, what)                     \
  do {                                          \
    hipError_t _e = (expr);                     \
    if (_e != hipSuccess) return hip_fail(_e, what); \
  } while (0)

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool valid_dtype(int dt) { return dt == T2VA_DTYPE_BF16 || dt == T2VA_DTYPE_FP32; }

int dt_size(int dt) { return dt == T2VA_DTYPE_BF16 ? 2 : 4; }

t2va_status check_t(int B, const double *t_host) {
  if (!t_host) return fail(T2VA_INVALID_ARG, "t_host is NULL");
  for (int b = 0; b < B; ++b) {
    const double t = t_host[b];
    if (!(t > 0.0 && t < M_PI / 2) || !isfinite(t))
      return fail(T2VA_INVALID_ARG, "t[%d] = %g is outside the open interval (0, pi/2)", b, t);
  }
  return T2VA_OK;
}

// Coefficients of the sCM target and of the block's parameterisation in fp64,
// rounded once to fp32.
CoefTable make_coef(int B, const double *t_host, double beta, double gamma, int param) {
  CoefTable c;
  memset(&c, 0, sizeof(c));
  c.B = B;
  c.rf = param == T2VA_PARAM_RF ? 1 : 0;
  for (int b = 0; b < B; ++b) {
    const double t = t_host[b];
    const double ct = cos(t), st = sin(t);
    // beta cos t / sqrt(1 - gamma^2 sin^2 t), with the root written as
    // sqrt(cos^2 t + (1 - gamma^2) sin^2 t) to avoid cancellation near pi/2.
    const double root = sqrt(ct * ct + (1.0 - gamma * gamma) * st * st);
    c.c[b].cos_t = (float)ct;
    c.c[b].sin_t = (float)st;
    c.c[b].inv_sin = (float)(1.0 / st);
    c.c[b].ct_st = (float)(ct * st);
    c.c[b].cos2 = (float)(ct * ct);
    c.c[b].boost = (float)(beta * ct / root);
    c.c[b].gamma_ct_st = (float)(gamma * ct * st);
    if (c.rf) {
      // TrigFlow wrapper: z_rf = z/(cos t + sin t), t_rf = sin t/(cos t + sin t)
      const double cs = ct + st;
      c.c[b].r = (float)(1.0 / cs);
      c.c[b].rdot = (float)((st - ct) / (cs * cs));
      c.c[b].t_emb = (float)(st / cs);
      c.c[b].t_emb_dot = (float)(1.0 / (cs * cs));
    } else {
      c.c[b].r = 1.f;
      c.c[b].rdot = 0.f;
      c.c[b].t_emb = (float)t;
      c.c[b].t_emb_dot = 1.f;
    }
  }
  return c;
}

t2va_status check_shape(int B, int Nv, int Na, int Nt, int Cv, int Ca, int d, int H, int in_dt,
                        int w_dt) {
  if (B < 1 || B > T2VA_MAX_BATCH)
    return fail(T2VA_UNSUPPORTED_SHAPE, "B = %d outside [1, %d]", B, T2VA_MAX_BATCH);
  if (Nv < 1 || Na < 1 || Nt < 0)
    return fail(T2VA_UNSUPPORTED_SHAPE, "need Nv >= 1, Na >= 1, Nt >= 0 (got %d, %d, %d)", Nv, Na, Nt);
  if (Cv < 64 || Cv % 64 || Ca < 64 || Ca % 64)
    return fail(T2VA_UNSUPPORTED_SHAPE, "Cv = %d and Ca = %d must be positive multiples of 64", Cv, Ca);
  if (H < 1 || d < 1 || d % H)
    return fail(T2VA_UNSUPPORTED_SHAPE, "d = %d is not a multiple of H = %d", d, H);
  const int dh = d / H;
  if (dh != 64 && dh != 128)
    return fail(T2VA_UNSUPPORTED_SHAPE, "head dim d/H = %d must be 64 or 128", dh);
  // The attention kernels address one sample's token rows (up to 3d elements
  // apart, plus a stage past the last key) with 32-bit buffer offsets.
  const int64_t tokens = (int64_t)Nv + Na + Nt;
  if ((tokens + 128) * 3 * d * 2 >= ((int64_t)1 << 31))
    return fail(T2VA_UNSUPPORTED_SHAPE, "%lld tokens x d = %d: a sample's rows exceed 2 GiB of 32-bit offsets",
                (long long)tokens, d);
  if (!valid_dtype(in_dt) || !valid_dtype(w_dt))
    return fail(T2VA_INVALID_ARG, "in_dtype / weight_dtype must be T2VA_DTYPE_BF16 or _FP32");
  return T2VA_OK;
}

// Element counts of the six weights of one block, in t2va_block_weights order.
void block_weight_elems(int Cv, int Ca, int d, size_t *n) {
  const size_t D = d;
  n[0] = D * Cv;
  n[1] = D * Ca;
  n[2] = D * D;
  n[3] = 3 * D * D;
  n[4] = (size_t)Cv * D;
  n[5] = (size_t)Ca * D;
}

// bf16 views of `count` blocks' weights: fp32 weights are rounded into dst
// (one after another, 128-element aligned), bf16 weights are used in place.
hipError_t prepare_weights(const t2va_block_weights *const *wb, int count, int weight_dtype,
                           const size_t *elems, bf16 *dst, const bf16 *W[][6], hipStream_t s) {
  // fp32 weights: every tensor of every block cast in one launch
  const float *srcs[kMaxCasts];
  bf16 *dsts[kMaxCasts];
  int64_t ns[kMaxCasts];
  int nc = 0;
  for (int i = 0; i < count; ++i) {
    const void *src[6] = {wb[i]->w_in_v, wb[i]->w_in_a, wb[i]->w_t, wb[i]->w_qkv, wb[i]->w_out_v, wb[i]->w_out_a};
    for (int j = 0; j < 6; ++j) {
      if (weight_dtype == T2VA_DTYPE_FP32) {
        if (nc == kMaxCasts) return hipErrorInvalidValue;
        srcs[nc] = (const float *)src[j];
        dsts[nc] = dst;
        ns[nc++] = (int64_t)elems[j];
        W[i][j] = dst;
        dst += align_up(elems[j], 128);
      } else {
        W[i][j] = (const bf16 *)src[j];
      }
    }
  }
  return nc ? launch_cast_set(srcs, dsts, ns, nc, s) : hipSuccess;
}

// Split precision: the text rows' QKV product contracts [X_hi | X_lo] rows, so
// its weight is used as [W_qkv | W_qkv] ([3d, 2d]), built into the workspace
// per call for each block (both blocks in one launch).
size_t dup_qkv_elems(int d) { return align_up((size_t)3 * d * 2 * d, 128); }
hipError_t prepare_dup(const bf16 *W[][6], int count, int d, bf16 *dst, const bf16 *Wd[], hipStream_t s) {
  if (count < 1 || count > 2) return hipErrorInvalidValue;
  for (int i = 0; i < count; ++i) Wd[i] = dst + i * dup_qkv_elems(d);
  return launch_dup_cols(W[0][3], count == 2 ? W[1][3] : nullptr, (bf16 *)Wd[0], count == 2 ? (bf16 *)Wd[1] : nullptr,
                         3 * d, d, s);
}

// ---------------------------------------------------------------------------
// Workspace layout of t2va_scm_target.
// ---------------------------------------------------------------------------
struct Layout {
  int Nq, N_all, dh, ldv, nblk_v, nblk_a;
  bool split;   // T2VA_PREC_SPLIT: [hi | lo | hi] z rows, [hi | lo] rows for X and Q|K
  size_t wts, wdup, wfold, wint, fpart, bqkv, zv, za, E, tau, X, QK, VT, nk, O, x0T_v, x0T_a, x0S_v,
      x0S_a,
      part_v, part_a, apart;
  size_t total, apart_bytes;
  size_t w_elems[6];  // per-block weight element counts
};

// The folded weights of one block (W_qkv W_in_m, [3d, C_m] per modality; in
// split precision [3d, 3 C_m] per modality, see Block::fold_weights).
size_t fold_elems(int Cv, int Ca, int d, bool split) {
  return align_up((size_t)3 * d * (Cv + Ca) * (split ? 3 : 1), 128);
}
// The fold's product (3d rows, Cv + Ca columns, K = d) has few output tiles:
// it runs split-K into fp32 partials, in chunks of d of at least 512 (the
// deep-ring GEMM's long-K case) and multiples of 64, at most 8 of them.
int fold_splits(int d) {
  int s = 8;
  while (s > 1 && (d % (64 * s) || d / s < 512)) s /= 2;
  return s;
}
size_t fold_part_bytes(int Cv, int Ca, int d) {
  return (size_t)fold_splits(d) * 3 * d * (Cv + Ca) * sizeof(float);
}

// whole_tiles: no scratch for split attention tails (every tile runs whole).
Layout make_layout(const t2va_scm_desc &d, bool whole_tiles = false) {
  Layout L;
  L.Nq = d.Nv + d.Na;
  L.N_all = L.Nq + d.Nt;
  L.dh = d.d / d.H;
  L.ldv = (int)align_up((size_t)L.N_all, 64);
  L.nblk_v = elementwise_blocks((int64_t)d.Nv * d.Cv);
  L.nblk_a = elementwise_blocks((int64_t)d.Na * d.Ca);
  const size_t B = d.B, D = d.d;
  block_weight_elems(d.Cv, d.Ca, d.d, L.w_elems);
  size_t wcount = 0;
  for (int i = 0; i < 6; ++i) wcount += align_up(L.w_elems[i], 128);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  L.split = d.precision == T2VA_PREC_SPLIT;
  const size_t sp = L.split ? 2 : 1;   // [hi | lo] rows are twice as wide
  const size_t spz = L.split ? 3 : 1;  // z rows [hi | lo | hi]
  L.wts = take(d.weight_dtype == T2VA_DTYPE_FP32 ? 2 * wcount * sizeof(bf16) : 0);
  L.wdup = take(L.split ? 2 * dup_qkv_elems(d.d) * sizeof(bf16) : 0);
  L.wfold = take(2 * fold_elems(d.Cv, d.Ca, d.d, L.split) * sizeof(bf16));
  L.wint = take(2 * (size_t)(d.Cv + d.Ca) * D * sizeof(bf16));
  L.fpart = take(2 * fold_part_bytes(d.Cv, d.Ca, d.d));
  L.bqkv = take(3 * B * 3 * D * sizeof(float));   // student [0, 2B), teacher [2B, 3B)
  L.zv = take(2 * B * d.Nv * d.Cv * spz * sizeof(bf16));
  L.za = take(2 * B * d.Na * d.Ca * spz * sizeof(bf16));
  L.E = take(2 * B * D * sizeof(float));
  L.tau = take(3 * B * D * sizeof(float));   // student [tau; dtau] [0, 2B), teacher [2B, 3B)
  L.X = take(2 * B * L.N_all * D * sp * sizeof(bf16));
  L.QK = take(2 * B * L.N_all * 2 * D * sp * sizeof(bf16));
  L.VT = take(2 * B * D * (size_t)L.ldv * sizeof(bf16));
  L.nk = take(B * sizeof(int32_t));
  L.O = take(2 * B * L.Nq * D * sizeof(bf16));
  L.x0T_v = take(B * d.Nv * d.Cv * sizeof(float));
  L.x0T_a = take(B * d.Na * d.Ca * sizeof(float));
  L.x0S_v = take(2 * B * d.Nv * d.Cv * sizeof(float));
  L.x0S_a = take(2 * B * d.Na * d.Ca * sizeof(float));
  L.part_v = take(B * L.nblk_v * sizeof(float));
  L.part_a = take(B * L.nblk_a * sizeof(float));
  L.apart_bytes = whole_tiles ? 0 : attention_split_bytes(L.dh, d.B, d.H, L.Nq);
  L.apart = take(L.apart_bytes);
  L.total = off;
  return L;
}

// Workspace of t2va_scm_grad: the target's layout, then the backward's buffers.
struct GradLayout {
  Layout base;
  int ldq, split_v, split_a, split_all;
  int64_t kc_v, kc_a, kc_all, kp_v, kp_a, kp_all;   // split-K chunk and padded token counts
  size_t lse, lse2, Dq, wt_out_v, wt_out_a, wt_qkv, dy_v, dy_a, dO, dOT, QT, KT, Vrm, dQKV, dX;
  size_t dyT_v, oT_v, dyT_a, oT_a, dqkvT, xT, dxT_v, zT_v, dxT_a, zT_a, tpart, part;
  size_t total, part_bytes;
};

// Split-K factor for a weight gradient contracted over `tokens` rows with
// `tiles` output tiles: enough workgroups to fill the chip, chunks of >= 512 tokens.
int grad_splits(int64_t tokens, int tiles) {
  int s = (int)std::min<int64_t>(std::max<int64_t>(tokens / 512, 1), 32);
  while (s > 1 && (int64_t)tiles * (s / 2) >= 512) s /= 2;
  return s;
}

GradLayout make_grad_layout(const t2va_scm_desc &d) {
  GradLayout G;
  G.base = make_layout(d);
  const Layout &L = G.base;
  const size_t B = d.B, D = d.d, H = d.H;
  const int64_t Nv = d.Nv, Na = d.Na, Nq = L.Nq, NA = L.N_all;
  G.ldq = (int)align_up((size_t)Nq, 64);
  const int tiles_out_v = (d.Cv + 127) / 128 * ((d.d + 127) / 128);
  const int tiles_out_a = (d.Ca + 127) / 128 * ((d.d + 127) / 128);
  const int tiles_qkv = (3 * d.d + 255) / 256 * ((d.d + 255) / 256);
  G.split_v = grad_splits(B * Nv, tiles_out_v);
  G.split_a = grad_splits(B * Na, tiles_out_a);
  G.split_all = grad_splits(B * NA, tiles_qkv);
  G.kc_v = (int64_t)align_up((size_t)((B * Nv + G.split_v - 1) / G.split_v), 64);
  G.kc_a = (int64_t)align_up((size_t)((B * Na + G.split_a - 1) / G.split_a), 64);
  G.kc_all = (int64_t)align_up((size_t)((B * NA + G.split_all - 1) / G.split_all), 64);
  G.kp_v = G.kc_v * G.split_v;
  G.kp_a = G.kc_a * G.split_a;
  G.kp_all = G.kc_all * G.split_all;
  size_t off = L.total;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  const size_t bfs = sizeof(bf16), fs = sizeof(float);
  G.lse = take(B * H * Nq * fs);
  G.lse2 = take(B * H * Nq * fs);
  G.Dq = take(B * H * Nq * fs);
  G.wt_out_v = take(D * d.Cv * bfs);
  G.wt_out_a = take(D * d.Ca * bfs);
  G.wt_qkv = take(D * 3 * D * bfs);
  G.dy_v = take(B * Nv * d.Cv * bfs);
  G.dy_a = take(B * Na * d.Ca * bfs);
  G.dO = take(B * Nq * D * bfs);
  G.dOT = take(B * D * G.ldq * bfs);
  G.QT = take(B * D * G.ldq * bfs);
  G.KT = take(B * D * (size_t)L.ldv * bfs);
  G.Vrm = take(B * NA * D * bfs);
  G.dQKV = take(B * NA * 3 * D * bfs);
  G.dX = take(B * Nq * D * bfs);
  G.dyT_v = take((size_t)d.Cv * G.kp_v * bfs);
  G.oT_v = take(D * G.kp_v * bfs);
  G.dyT_a = take((size_t)d.Ca * G.kp_a * bfs);
  G.oT_a = take(D * G.kp_a * bfs);
  G.dqkvT = take(3 * D * G.kp_all * bfs);
  G.xT = take(D * G.kp_all * bfs);
  G.dxT_v = take(D * G.kp_v * bfs);
  G.zT_v = take((size_t)d.Cv * G.kp_v * bfs);
  G.dxT_a = take(D * G.kp_a * bfs);
  G.zT_a = take((size_t)d.Ca * G.kp_a * bfs);
  G.tpart = take(B * (size_t)(colsum_chunks((int)Nq) + 1) * D * fs);   // partial sums, then dtau
  const size_t part_elems = std::max({(size_t)G.split_v * d.Cv * D, (size_t)G.split_a * d.Ca * D,
                                      (size_t)G.split_all * 3 * D * D});
  // also the attention backward's scratch (used before the weight gradients, on one stream)
  G.part_bytes = std::max(part_elems * fs, attention_bwd_split_bytes(L.dh, d.B, d.H, L.Nq, L.N_all));
  G.part = take(G.part_bytes);
  G.total = off;
  return G;
}

t2va_status check_desc(const t2va_scm_desc *d) {
  if (!d) return fail(T2VA_INVALID_ARG, "desc is NULL");
  if (t2va_status st = check_shape(d->B, d->Nv, d->Na, d->Nt, d->Cv, d->Ca, d->d, d->H,
                                   d->in_dtype, d->weight_dtype))
    return st;
  if (d->param != T2VA_PARAM_X0 && d->param != T2VA_PARAM_RF)
    return fail(T2VA_INVALID_ARG, "param = %d must be T2VA_PARAM_X0 or T2VA_PARAM_RF", d->param);
  if (d->precision != T2VA_PREC_BF16 && d->precision != T2VA_PREC_SPLIT)
    return fail(T2VA_INVALID_ARG, "precision = %d must be T2VA_PREC_BF16 or T2VA_PREC_SPLIT", d->precision);
  if (!(d->gamma >= 0.0 && d->gamma <= 1.0))
    return fail(T2VA_INVALID_ARG, "gamma = %g outside [0, 1]", d->gamma);
  if (!(d->eps_scm > 0.0) || !isfinite(d->eps_scm))
    return fail(T2VA_INVALID_ARG, "eps_scm = %g must be positive and finite", d->eps_scm);
  if (!isfinite(d->beta) || !isfinite(d->w_v) || !isfinite(d->w_a))
    return fail(T2VA_INVALID_ARG, "beta, w_v and w_a must be finite");
  return T2VA_OK;
}

t2va_status check_weights(const t2va_block_weights *const *wb, int n, const char *name0,
                          const char *name1) {
  for (int i = 0; i < n; ++i) {
    const char *name = i ? name1 : name0;
    if (!wb[i]) return fail(T2VA_INVALID_ARG, "%s weights are NULL", name);
    const void *w[6] = {wb[i]->w_in_v, wb[i]->w_in_a, wb[i]->w_t, wb[i]->w_qkv, wb[i]->w_out_v, wb[i]->w_out_a};
    for (const void *p : w) {
      if (!p) return fail(T2VA_INVALID_ARG, "%s weight pointer is NULL", name);
      if (!aligned16(p)) return fail(T2VA_INVALID_ARG, "weights must be 16-byte aligned");
    }
  }
  return T2VA_OK;
}

// Workspace layout of t2va_dmd_target.
struct DmdLayout {
  int ldv, nblk_v, nblk_a;
  bool split;
  size_t wts, wdup, wfold, wint, fpart, bqkv, zv, za, E, tau, X, QK, VT, nk, nk_null, O, Of, xT_v,
      xT_a, xF_v,
      xF_a, pa_v, pa_a, ps_v, ps_a, apart;
  size_t total, apart_bytes;
  size_t w_elems[6];
};

DmdLayout make_dmd_layout(const t2va_dmd_desc &d) {
  DmdLayout L;
  const int Nq = d.Nv + d.Na, N_all = Nq + d.Nt;
  L.ldv = (int)align_up((size_t)N_all, 64);
  L.nblk_v = elementwise_blocks((int64_t)d.Nv * d.Cv);
  L.nblk_a = elementwise_blocks((int64_t)d.Na * d.Ca);
  const size_t B = d.B, D = d.d;
  const size_t nv = (size_t)d.Nv * d.Cv, na = (size_t)d.Na * d.Ca;
  block_weight_elems(d.Cv, d.Ca, d.d, L.w_elems);
  size_t wcount = 0;
  for (int i = 0; i < 6; ++i) wcount += align_up(L.w_elems[i], 128);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  L.split = d.precision == T2VA_PREC_SPLIT;
  const size_t sp = L.split ? 2 : 1;
  const size_t spz = L.split ? 3 : 1;
  L.wts = take(d.weight_dtype == T2VA_DTYPE_FP32 ? 2 * wcount * sizeof(bf16) : 0);
  L.wdup = take(L.split ? 2 * dup_qkv_elems(d.d) * sizeof(bf16) : 0);
  L.wfold = take(2 * fold_elems(d.Cv, d.Ca, d.d, L.split) * sizeof(bf16));
  L.wint = take(2 * (size_t)(d.Cv + d.Ca) * D * sizeof(bf16));
  L.fpart = take(2 * fold_part_bytes(d.Cv, d.Ca, d.d));
  L.bqkv = take(2 * B * 3 * D * sizeof(float));   // teacher [0, B), fake [B, 2B)
  L.zv = take(B * nv * spz * sizeof(bf16));
  L.za = take(B * na * spz * sizeof(bf16));
  L.E = take(2 * B * D * sizeof(float));
  L.tau = take(2 * B * D * sizeof(float));   // teacher [0, B), fake [B, 2B)
  L.X = take(B * N_all * D * sp * sizeof(bf16));
  L.QK = take(B * N_all * 2 * D * sp * sizeof(bf16));
  L.VT = take(B * D * (size_t)L.ldv * sizeof(bf16));
  L.nk = take(B * sizeof(int32_t));
  L.nk_null = take(B * sizeof(int32_t));
  L.O = take(B * Nq * D * sizeof(bf16));
  L.Of = take(2 * B * Nq * D * sizeof(float));   // guided teacher: conditional and null outputs, fp32
  L.xT_v = take(B * nv * sizeof(float));
  L.xT_a = take(B * na * sizeof(float));
  L.xF_v = take(B * nv * sizeof(float));
  L.xF_a = take(B * na * sizeof(float));
  L.pa_v = take(B * L.nblk_v * sizeof(float));
  L.pa_a = take(B * L.nblk_a * sizeof(float));
  L.ps_v = take(B * L.nblk_v * sizeof(float));
  L.ps_a = take(B * L.nblk_a * sizeof(float));
  L.apart_bytes = attention_split_bytes(d.d / d.H, d.B, d.H, Nq, true);
  L.apart = take(L.apart_bytes);
  L.total = off;
  return L;
}

t2va_status check_dmd_desc(const t2va_dmd_desc *d) {
  if (!d) return fail(T2VA_INVALID_ARG, "desc is NULL");
  if (t2va_status st = check_shape(d->B, d->Nv, d->Na, d->Nt, d->Cv, d->Ca, d->d, d->H,
                                   d->in_dtype, d->weight_dtype))
    return st;
  if (d->param != T2VA_PARAM_X0 && d->param != T2VA_PARAM_RF)
    return fail(T2VA_INVALID_ARG, "param = %d must be T2VA_PARAM_X0 or T2VA_PARAM_RF", d->param);
  if (d->precision != T2VA_PREC_BF16 && d->precision != T2VA_PREC_SPLIT)
    return fail(T2VA_INVALID_ARG, "precision = %d must be T2VA_PREC_BF16 or T2VA_PREC_SPLIT", d->precision);
  if (!isfinite(d->cfg_v) || !isfinite(d->cfg_a))
    return fail(T2VA_INVALID_ARG, "guidance scales must be finite");
  if (!(d->eps_dmd > 0.0) || !isfinite(d->eps_dmd))
    return fail(T2VA_INVALID_ARG, "eps_dmd = %g must be positive and finite", d->eps_dmd);
  if (!isfinite(d->w_v) || !isfinite(d->w_a)) return fail(T2VA_INVALID_ARG, "w_v and w_a must be finite");
  return T2VA_OK;
}

// ---------------------------------------------------------------------------
// Phase timing.
// ---------------------------------------------------------------------------
struct Profiler {
  int max_calls = 0, calls = 0;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  struct Rec { int phase; hipEvent_t a, b; };
  std::vector<Rec> recs;
  bool active() const { return max_calls > 0 && calls < max_calls; }
  hipEvent_t next() { return used < pool.size() ? pool[used++] : nullptr; }
};
Profiler g_prof;
unsigned g_prof_phases = ~0u;   // phases whose events are recorded (t2va_profile_set_phases)

struct PhaseScope {
  hipStream_t s;
  int phase;
  hipEvent_t a = nullptr, b = nullptr;
  bool on;
  PhaseScope(hipStream_t s_, int ph, bool on_) : s(s_), phase(ph), on(on_ && ((g_prof_phases >> ph) & 1u)) {
    if (on) {
      a = g_prof.next();
      b = g_prof.next();
      if (a && b) hipEventRecord(a, s);
    }
  }
  ~PhaseScope() {
    if (on && a && b) {
      hipEventRecord(b, s);
      g_prof.recs.push_back({phase, a, b});
    }
  }
};

// The steps of one joint block on the caller's stream: the per-modality input
// projections (+ tau) and the fused QKV projection, attention, and the
// per-modality output projections.  `batch` stacks independent problems that
// share the weights (primal and tangent rows, or conditional and
// unconditional outputs).
struct Block {
  int B, Nv, Na, Cv, Ca, D, H, dh, Nq, NA, ldv;
  bool split;        // T2VA_PREC_SPLIT: z rows [hi | lo | hi], X and Q|K rows [hi | lo]
  int64_t xs, qks;   // row strides of X (d, or 2d split) and QK (2d, or 4d split)
  int64_t nv, na, x_bs, qk_bs, vt_hs, vt_bs, o_bs;
  hipStream_t s;
  bool prof;
  float *apart = nullptr;   // attention scratch for split tails (nullable)
  size_t apart_bytes = 0;

  Block(int B_, int Nv_, int Na_, int Nt, int Cv_, int Ca_, int d, int H_, int ldv_, hipStream_t s_,
        bool prof_, bool split_ = false)
      : B(B_), Nv(Nv_), Na(Na_), Cv(Cv_), Ca(Ca_), D(d), H(H_), dh(d / H_), Nq(Nv_ + Na_),
        NA(Nv_ + Na_ + Nt), ldv(ldv_), split(split_), s(s_), prof(prof_) {
    nv = (int64_t)Nv * Cv;
    na = (int64_t)Na * Ca;
    xs = split ? 2 * D : D;
    qks = split ? 4 * D : 2 * D;
    x_bs = (int64_t)NA * xs;
    qk_bs = (int64_t)NA * qks;
    vt_hs = (int64_t)dh * ldv;
    vt_bs = (int64_t)H * vt_hs;
    o_bs = (int64_t)Nq * D;
  }

  GemmParams params(const bf16 *A, int64_t lda, int64_t a_bs, const bf16 *Wt, int64_t ldw, void *Cp,
                    int64_t ldc, int64_t c_bs, int c_dt, const float *bias, int64_t bias_bs, int M, int N,
                    int K, int batch, bf16 *vt, int n_split, int64_t w_bs = 0, int vt_rows = -1) const {
    GemmParams g;
    g.A = A; g.lda = lda; g.a_bs = a_bs;
    g.W = Wt; g.ldw = ldw; g.w_bs = w_bs;
    g.C = Cp; g.ldc = ldc; g.c_bs = c_bs; g.c_dt = c_dt;
    g.bias = bias; g.bias_bs = bias_bs;
    g.VT = vt; g.vt_bs = vt_bs; g.vt_hs = vt_hs; g.vt_rs = ldv; g.vt_rows = vt_rows < 0 ? ldv : vt_rows;
    g.n_split = n_split; g.dh = dh;
    g.M = M; g.N = N; g.K = K; g.batch = batch;
    return g;
  }

  // vt_rows: V^T token columns [0, vt_rows) from vt are written (rows past M as zeros); -1: up to ldv
  t2va_status gemm(const bf16 *A, int64_t lda, int64_t a_bs, const bf16 *Wt, int64_t ldw, void *Cp,
                   int64_t ldc, int64_t c_bs, int c_dt, const float *bias, int64_t bias_bs, int M,
                   int N, int K, int batch, bf16 *vt, int n_split, int64_t w_bs = 0, int vt_rows = -1) const {
    const GemmParams g = params(A, lda, a_bs, Wt, ldw, Cp, ldc, c_bs, c_dt, bias, bias_bs, M, N, K, batch, vt,
                                n_split, w_bs, vt_rows);
    PhaseScope ps(s, T2VA_PHASE_GEMM, prof);
    HIP_TRY(launch_gemm(g, s), "gemm");
    return T2VA_OK;
  }

  // Folded weights of both blocks: Wf = W_qkv [W_in_v | W_in_a].  Before
  // attention the block is linear, so for video and audio rows Q|K|V =
  // (z W_in^T + tau) W_qkv^T = z (W_qkv W_in)^T + tau W_qkv^T: a product with
  // K = C_m instead of the input projection and a K = d product.  Block i
  // (weights W[i]) writes Wf + i fold_elems; wint: scratch for
  // [W_in_v^T; W_in_a^T] of each block, 2 [Cv + Ca, d]; fpart: 2
  // fold_part_bytes of split-K partials.
  //   bf16: Wf [3d, Cv + Ca] (row stride Cv + Ca; the video part is its first
  //     Cv columns).
  //   split: per modality Wf_m [3d, 3 C_m] = [Wf_hi | Wf_hi | Wf_lo] (video,
  //     then audio at 9 d Cv), the hi/lo pair of the fp32 product; against z
  //     rows [z_hi | z_lo | z_hi] one K = 3 C_m product then sums
  //     z_hi Wf_hi + z_lo Wf_hi + z_hi Wf_lo, the pair product less its
  //     lo x lo term (relative 2^-18).
  // Three launches for both blocks: the four transposes, the two split-K
  // products, the two sums.
  t2va_status fold_weights(const bf16 *const (&W)[2][6], bf16 *Wf, bf16 *wint, float *fpart) const {
    const int C[2] = {Cv, Ca}, CC = Cv + Ca;
    const int64_t wint_bs = (int64_t)CC * D;
    TransposeParams tp[4];
    for (int i = 0; i < 2; ++i)
      for (int m = 0; m < 2; ++m) {
        TransposeParams &t = tp[2 * i + m];
        t.src = W[i][m]; t.s_bs = 0; t.s_hs = 0; t.s_rs = C[m];
        t.dst = wint + i * wint_bs + (m ? (int64_t)Cv * D : 0); t.d_bs = 0; t.d_hs = 0; t.d_rs = D;
        t.B = 1; t.H = 1; t.R = D; t.C = C[m]; t.Rpad = D;
      }
    HIP_TRY(launch_transpose_set(tp, 4, s), "transpose");
    // split-K: chunk k of W_qkv's columns against the same chunk of W_in^T's
    const int splits = fold_splits(D), kc = D / splits;
    const int64_t part_bs = (int64_t)fold_part_bytes(Cv, Ca, D) / sizeof(float);
    GemmParams g[2];
    for (int i = 0; i < 2; ++i)
      g[i] = params(W[i][3], D, kc, wint + i * wint_bs, D, fpart + i * part_bs, CC, (int64_t)3 * D * CC, 1,
                    nullptr, 0, 3 * D, CC, kc, splits, nullptr, CC, kc);
    {
      PhaseScope ps(s, T2VA_PHASE_GEMM, prof);
      HIP_TRY(launch_gemm_pair(g[0], g[1], s), "gemm");
    }
    HIP_TRY(launch_fold_finish(fpart, splits, 3 * D, Cv, Ca, split, Wf, 2, part_bs,
                               (int64_t)fold_elems(Cv, Ca, D, split), s),
            "fold");
    return T2VA_OK;
  }

  // X rows [0, Nq) = [z^v W_in_v^T; z^a W_in_a^T] + tau[b] for `batch` problems.
  t2va_status in_proj(const bf16 *const *W, const bf16 *zv, const bf16 *za, const float *tau, bf16 *X,
                      int batch) const {
    if (t2va_status st = gemm(zv, Cv, nv, W[0], Cv, X, D, x_bs, 0, tau, D, Nv, D, Cv, batch, nullptr, D))
      return st;
    return gemm(za, Ca, na, W[1], Ca, X + (int64_t)Nv * D, D, x_bs, 0, tau, D, Na, D, Ca,
                batch, nullptr, D);
  }

  // Q|K (row-major into QK) and V^T (dh-major into VT) of `batch` problems:
  // the video and audio rows straight from z with the folded weights Wf
  // (fold_weights; bias bqkv [batch][3d] = W_qkv tau per batch), the text
  // rows [Nq, NA) from X with W_qkv (no bias; their V^T columns and the zero
  // padding up to ldv).  Split precision: z rows are [hi | lo | hi] (3 C_m
  // wide), the text rows of X [hi | lo] against Wd_qkv = [W_qkv | W_qkv], and
  // Q|K rows are written [Q_hi | K_hi | Q_lo | K_lo].  The audio and text
  // products are small and run as one two-problem launch.
  t2va_status project_in_folded(const bf16 *const *W, const bf16 *Wd_qkv, const bf16 *Wf, const bf16 *zv,
                                const bf16 *za, const float *bqkv, const bf16 *X, bf16 *QK, bf16 *VT,
                                int batch) const {
    const int kz = split ? 3 : 1, cdt = split ? 2 : 0;
    const bf16 *Wv = Wf, *Wa = split ? Wf + (int64_t)9 * D * Cv : Wf + Cv;
    const int64_t ldwv = split ? 3 * Cv : Cv + Ca, ldwa = split ? 3 * Ca : Cv + Ca;
    const bf16 *Wt = split ? Wd_qkv : W[3];
    const int kt = split ? 2 * D : D;
    if (t2va_status st = gemm(zv, kz * Cv, kz * nv, Wv, ldwv, QK, qks, qk_bs, cdt, bqkv, 3 * D, Nv, 3 * D, kz * Cv,
                              batch, VT, 2 * D, 0, Nv))
      return st;
    const GemmParams ga = params(za, kz * Ca, kz * na, Wa, ldwa, QK + (int64_t)Nv * qks, qks, qk_bs, cdt, bqkv,
                                 3 * D, Na, 3 * D, kz * Ca, batch, VT + Nv, 2 * D, 0, Na);
    const GemmParams gt = params(X + (int64_t)Nq * xs, xs, x_bs, Wt, kt, QK + (int64_t)Nq * qks, qks, qk_bs, cdt,
                                 nullptr, 0, NA - Nq, 3 * D, kt, batch, VT + Nq, 2 * D, 0, ldv - Nq);
    PhaseScope ps(s, T2VA_PHASE_GEMM, prof);
    HIP_TRY(launch_gemm_pair(ga, gt, s), "gemm");
    return T2VA_OK;
  }

  // O [batch, Nq, D] -> fp32 x0^v [batch, Nv, Cv] and x0^a [batch, Na, Ca], in one launch: the
  // audio rows are few, and alone they would leave most of the chip idle.
  t2va_status project_out(const bf16 *const *W, const bf16 *O, float *xv, float *xa, int batch) const {
    const GemmParams gv = params(O, D, o_bs, W[4], D, xv, Cv, nv, 1, nullptr, 0, Nv, Cv, D, batch, nullptr, Cv);
    const GemmParams ga = params(O + (int64_t)Nv * D, D, o_bs, W[5], D, xa, Ca, na, 1, nullptr, 0, Na, Ca, D,
                                 batch, nullptr, Ca);
    PhaseScope ps(s, T2VA_PHASE_GEMM, prof);
    HIP_TRY(launch_gemm_pair(gv, ga, s), "gemm");
    return T2VA_OK;
  }

  // Attention of the B problems in QK/VT over nk[b] keys into O; with `tan`,
  // the tangent operands are the batches that follow (QK + B qk_bs, VT + B
  // vt_bs) and the tangent output goes to O + B o_bs.
  // out_dt: the dtype of O (and O_prefix); elements at the same strides either way.
  t2va_status attention(const bf16 *QK, const bf16 *VT, const int32_t *nk, void *O, bool tan,
                        int phase, float *lse = nullptr, void *O_prefix = nullptr, int nk_split = 0,
                        int out_dt = T2VA_DTYPE_BF16) const {
    AttnParams p;
    p.q = QK; p.k = QK + D; p.vt = VT;
    p.q_lo = split ? QK + 2 * D : nullptr;
    p.k_lo = split ? QK + 3 * D : nullptr;
    p.qd = tan ? QK + (int64_t)B * qk_bs : nullptr;
    p.kd = tan ? QK + (int64_t)B * qk_bs + D : nullptr;
    p.vdt = tan ? VT + (int64_t)B * vt_bs : nullptr;
    p.nk = nk; p.o = O; p.od = tan ? (bf16 *)O + (int64_t)B * o_bs : nullptr; p.lse = lse;
    p.o2 = O_prefix; p.nk_split = nk_split;
    p.q_bs = qk_bs; p.q_rs = qks; p.k_bs = qk_bs; p.k_rs = qks;
    p.vt_bs = vt_bs; p.vt_hs = vt_hs; p.vt_rs = ldv;
    p.o_bs = o_bs; p.o_rs = D;
    p.B = B; p.H = H; p.Nq = Nq; p.Nk = NA;
    p.out_dt = out_dt;
    p.scale = (float)(1.0 / sqrt((double)dh));
    p.part = apart;
    p.part_bytes = apart_bytes;
    PhaseScope ps(s, phase, prof);
    HIP_TRY(launch_attention(dh, tan, p, s), "attention");
    return T2VA_OK;
  }
};

// Argument checks shared by t2va_scm_target and t2va_scm_grad (no HIP calls).
t2va_status validate_scm(const t2va_scm_desc *desc, const t2va_block_weights *const *wb,
                         const void *z0_v, const void *z0_a, const void *eps_v, const void *eps_a,
                         const void *text, const uint8_t *text_mask, const double *t_host,
                         const float *J_v, const float *J_a, const float *gbar_v, const float *gbar_a,
                         const float *r_v, const float *r_a, const float *loss, const void *workspace,
                         size_t workspace_bytes, size_t needed) {
  if (t2va_status st = check_desc(desc)) return st;
  const t2va_scm_desc &d = *desc;
  if (t2va_status st = check_t(d.B, t_host)) return st;
  if (t2va_status st = check_weights(wb, 2, "teacher", "student")) return st;
  const void *req[] = {z0_v, z0_a, eps_v, eps_a, gbar_v, gbar_a, loss};
  for (const void *p : req)
    if (!p) return fail(T2VA_INVALID_ARG, "z0, eps, gbar and loss pointers are required");
  if (d.Nt > 0 && (!text || !text_mask))
    return fail(T2VA_INVALID_ARG, "text and text_mask are required when Nt > 0");
  const void *al[] = {z0_v, z0_a, eps_v, eps_a, text, J_v, J_a, gbar_v, gbar_a, r_v, r_a};
  for (const void *p : al)
    if (p && !aligned16(p)) return fail(T2VA_INVALID_ARG, "tensor operands must be 16-byte aligned");
  if (!workspace) return fail(T2VA_INVALID_ARG, "workspace is NULL");
  if (((uintptr_t)workspace & 255u) != 0) return fail(T2VA_INVALID_ARG, "workspace must be 256-byte aligned");
  if (workspace_bytes < needed)
    return fail(T2VA_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, needed);
  return T2VA_OK;
}

// The launch sequence of the joint sCM target (validated arguments).  With
// lse_student, the student's attention also writes its primal log-sum-exp
// (for the backward).  W receives the bf16 views of both blocks' weights.
t2va_status run_scm(const t2va_scm_desc &d, const Layout &L, const t2va_block_weights *const *wb,
                    const void *z0_v, const void *z0_a, const void *eps_v, const void *eps_a,
                    const void *text, const uint8_t *text_mask, const double *t_host, float *J_v,
                    float *J_a, float *gbar_v, float *gbar_a, float *r_v, float *r_a, float *norms,
                    float *loss, void *workspace, float *lse_student, const bf16 *(&W)[2][6],
                    hipStream_t s, bool prof) {
  char *ws = (char *)workspace;
  Block blk(d.B, d.Nv, d.Na, d.Nt, d.Cv, d.Ca, d.d, d.H, L.ldv, s, prof, L.split);
  blk.apart = (float *)(ws + L.apart);
  blk.apart_bytes = L.apart_bytes;
  const int B = d.B, D = d.d, Nq = L.Nq;
  const int64_t nv = blk.nv, na = blk.na;
  const CoefTable coef = make_coef(B, t_host, d.beta, d.gamma, d.param);

  HIP_TRY(prepare_weights(wb, 2, d.weight_dtype, L.w_elems, (bf16 *)(ws + L.wts), W, s), "cast");
  const bf16 *Wd[2] = {nullptr, nullptr};
  if (L.split) HIP_TRY(prepare_dup(W, 2, D, (bf16 *)(ws + L.wdup), Wd, s), "weight pairs");
  // fold W_qkv W_in_m for both blocks
  float *bqkv = (float *)(ws + L.bqkv);
  bf16 *const wfold = (bf16 *)(ws + L.wfold);
  if (t2va_status st = blk.fold_weights(W, wfold, (bf16 *)(ws + L.wint), (float *)(ws + L.fpart))) return st;
  const bf16 *Wf[2] = {wfold, wfold + fold_elems(d.Cv, d.Ca, D, L.split)};

  bf16 *zv = (bf16 *)(ws + L.zv), *za = (bf16 *)(ws + L.za);
  float *E = (float *)(ws + L.E), *tau = (float *)(ws + L.tau);
  bf16 *X = (bf16 *)(ws + L.X), *QK = (bf16 *)(ws + L.QK), *VT = (bf16 *)(ws + L.VT);
  bf16 *O = (bf16 *)(ws + L.O);
  int32_t *nk = (int32_t *)(ws + L.nk);
  float *x0T_v = (float *)(ws + L.x0T_v), *x0T_a = (float *)(ws + L.x0T_a);
  float *x0S_v = (float *)(ws + L.x0S_v), *x0S_a = (float *)(ws + L.x0S_a);
  float *part_v = (float *)(ws + L.part_v), *part_a = (float *)(ws + L.part_a);

  // The block's latent token rows of batch half `half` (0: z_t, 1: F_T) from
  // the trigflow op: bf16, or in split precision the fp32 value split into
  // bf16 rows [hi | lo | hi].
  auto token_rows = [&](int op, int half, const float *x0_v, const float *x0_a) -> t2va_status {
    const int64_t xs_v = op == 2 ? nv : 0, xs_a = op == 2 ? na : 0;
    // video and audio rows in one launch
    if (!L.split) {
      const TrigSeg sv{z0_v, eps_v, x0_v, zv + (int64_t)half * B * nv, nv, nv, nv, xs_v, nv, 0};
      const TrigSeg sa{z0_a, eps_a, x0_a, za + (int64_t)half * B * na, na, na, na, xs_a, na, 0};
      HIP_TRY(launch_trigflow_pair(op, coef, d.in_dtype, d.in_dtype, T2VA_DTYPE_BF16, sv, sa, s), "token rows");
      return T2VA_OK;
    }
    const TrigSeg sv{z0_v, eps_v, x0_v, zv + (int64_t)half * B * 3 * nv, nv, nv, nv, xs_v, 3 * nv, 0, d.Cv};
    const TrigSeg sa{z0_a, eps_a, x0_a, za + (int64_t)half * B * 3 * na, na, na, na, xs_a, 3 * na, 0, d.Ca};
    HIP_TRY(launch_trigflow_pair(op, coef, d.in_dtype, d.in_dtype, kTrigSplitRows, sv, sa, s), "token rows");
    return T2VA_OK;
  };

#define T2VA_CALL(x) do { t2va_status _st = (x); if (_st) return _st; } while (0)
  // z_t = cos t z0 + sin t eps (the GEMM input), half 0 of zv / za.
  T2VA_CALL(token_rows(0, 0, nullptr, nullptr));
  HIP_TRY(launch_time_embedding(coef, D, E, s), "time embedding");
  // tau = W_t e(t) of both blocks in one launch, then both blocks' QKV bias
  // rows W_qkv tau in a second; the student's [tau; dtau] rows are [0, 2B)
  // (where the backward reads them), the teacher's [2B, 3B)
  float *tau_T = tau + (int64_t)2 * B * D, *bqkv_T = bqkv + (int64_t)2 * B * 3 * D;
  HIP_TRY(launch_row_linear_pair(D, D, RowLinSeg{E, W[0][2], tau_T, B}, RowLinSeg{E, W[1][2], tau, 2 * B}, s),
          "time linear");
  HIP_TRY(launch_row_linear_pair(D, 3 * D, RowLinSeg{tau_T, W[0][3], bqkv_T, B},
                                 RowLinSeg{tau, W[1][3], bqkv, 2 * B}, s),
          "QKV bias");
  if (d.Nt > 0)
    // the primal text rows of both blocks' batches [0, B) and the zero tangent
    // rows [B, 2B) of the student's, in one launch
    HIP_TRY(launch_text_rows(2 * B, Nq, d.Nt, D, text, d.in_dtype, text_mask, X, blk.x_bs, blk.xs, L.split, B, nk,
                             s), "text rows");
  else
    HIP_TRY(launch_fill_nk(nk, B, Nq, s), "fill nk");

  // ---------------- teacher: x0_T = G_T(z_t, t, c) ----------------
  T2VA_CALL(blk.project_in_folded(W[0], Wd[0], Wf[0], zv, za, bqkv_T, X, QK, VT, B));
  T2VA_CALL(blk.attention(QK, VT, nk, O, false, T2VA_PHASE_TEACHER_ATTN));
  T2VA_CALL(blk.project_out(W[0], O, x0T_v, x0T_a, B));

  // ---------------- F_T (tangent of the student's latent inputs), half 1 ----------------
  T2VA_CALL(token_rows(2, 1, x0T_v, x0T_a));

  // ---------------- student: G_S and its JVP ----------------
  // Batches [0, B) carry the primal rows, [B, 2B) their tangents.
  T2VA_CALL(blk.project_in_folded(W[1], Wd[1], Wf[1], zv, za, bqkv, X, QK, VT, 2 * B));
  T2VA_CALL(blk.attention(QK, VT, nk, O, true, T2VA_PHASE_STUDENT_ATTN, lse_student));
  T2VA_CALL(blk.project_out(W[1], O, x0S_v, x0S_a, 2 * B));
#undef T2VA_CALL

  // ---------------- g, norms, gbar, r, loss ----------------
  GParams gp;
  gp.z0[0] = z0_v; gp.z0[1] = z0_a; gp.eps[0] = eps_v; gp.eps[1] = eps_a;
  gp.x0T[0] = x0T_v; gp.x0T[1] = x0T_a;
  gp.x0S[0] = x0S_v; gp.x0S[1] = x0S_a;
  gp.Gd[0] = x0S_v + (int64_t)B * nv; gp.Gd[1] = x0S_a + (int64_t)B * na;
  gp.x_bs[0] = nv; gp.x_bs[1] = na;
  gp.J[0] = J_v; gp.J[1] = J_a;
  gp.g[0] = gbar_v; gp.g[1] = gbar_a;
  gp.partial[0] = part_v; gp.partial[1] = part_a;
  gp.n[0] = nv; gp.n[1] = na;
  gp.nblk[0] = L.nblk_v; gp.nblk[1] = L.nblk_a;
  gp.in_dt = d.in_dtype;
  HIP_TRY(launch_scm_direction(coef, gp, s), "sCM direction");
  NormParams np;
  np.mode = 0;
  np.g[0] = gbar_v; np.g[1] = gbar_a; np.r[0] = r_v; np.r[1] = r_a;
  np.partial[0] = part_v; np.partial[1] = part_a;
  np.partial2[0] = np.partial2[1] = nullptr;
  np.n[0] = nv; np.n[1] = na;
  np.nblk[0] = L.nblk_v; np.nblk[1] = L.nblk_a;
  np.norms = norms; np.loss = loss;
  np.eps = d.eps_scm; np.w[0] = d.w_v; np.w[1] = d.w_a;
  HIP_TRY(launch_normalise(B, np, s), "normalise");
  return T2VA_OK;
}

// The standalone attention entry points (validated here; no workspace, so
// every tile runs whole).  split: the logits also take q_lo and k_lo.
t2va_status attn_entry(const t2va_attn_desc *desc, const void *q, const void *q_lo, const void *k,
                       const void *k_lo, const void *vt, const void *qd, const void *kd, const void *vdt,
                       const int32_t *nk_valid, void *o, void *od, float *lse, t2va_stream stream, bool split) {
  if (!desc) return fail(T2VA_INVALID_ARG, "desc is NULL");
  const t2va_attn_desc &d = *desc;
  if (d.dh != 64 && d.dh != 128) return fail(T2VA_UNSUPPORTED_SHAPE, "dh = %d must be 64 or 128", d.dh);
  if (d.B < 1 || d.H < 1 || d.Nq < 1 || d.Nk < 1)
    return fail(T2VA_UNSUPPORTED_SHAPE, "B, H, Nq and Nk must be >= 1");
  if (!q || !k || !vt || !nk_valid || !o) return fail(T2VA_INVALID_ARG, "q, k, vt, nk_valid and o are required");
  if (split && (!q_lo || !k_lo)) return fail(T2VA_INVALID_ARG, "q_lo and k_lo are required");
  const bool tan = d.has_tangent != 0;
  if (tan && (!qd || !kd || !vdt || !od))
    return fail(T2VA_INVALID_ARG, "has_tangent needs qd, kd, vdt and od");
  if (!tan && (qd || kd || vdt || od))
    return fail(T2VA_INVALID_ARG, "tangent pointers given with has_tangent = 0");
  if (!valid_dtype(d.out_dtype)) return fail(T2VA_INVALID_ARG, "bad out_dtype");
  if (!(d.scale >= 0.f) || !isfinite(d.scale))
    return fail(T2VA_INVALID_ARG, "scale = %g must be finite and >= 0 (0: 1/sqrt(dh))", (double)d.scale);
  const void *ptrs[] = {q, q_lo, k, k_lo, vt, qd, kd, vdt, nk_valid, o, od};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return fail(T2VA_INVALID_ARG, "operands must be 16-byte aligned");
  const int64_t strides[] = {d.q_batch_stride, d.q_row_stride, d.k_batch_stride, d.k_row_stride,
                             d.vt_batch_stride, d.vt_head_stride, d.vt_row_stride,
                             d.o_batch_stride, d.o_row_stride};
  for (int64_t st : strides)
    if (st < 0 || st % 8) return fail(T2VA_INVALID_ARG, "strides must be non-negative multiples of 8");
  if (d.vt_row_stride < ((d.Nk + 63) / 64) * 64)
    return fail(T2VA_INVALID_ARG, "vt_row_stride %lld < round_up(Nk, 64)", (long long)d.vt_row_stride);
  // Per-(sample, head) byte offsets must fit the 32-bit buffer addressing: the
  // kernels address K rows up to one 128-key stage past the last key, and
  // every V^T row of a head.
  if ((int64_t)(d.Nk + 128) * d.k_row_stride * 2 >= ((int64_t)1 << 31) ||
      (int64_t)d.dh * d.vt_row_stride * 2 >= ((int64_t)1 << 31))
    return fail(T2VA_UNSUPPORTED_SHAPE, "K or V^T extent per (sample, head) exceeds 2 GiB");
  if (d.q_row_stride < (int64_t)d.H * d.dh || d.k_row_stride < (int64_t)d.H * d.dh ||
      d.o_row_stride < (int64_t)d.H * d.dh)
    return fail(T2VA_INVALID_ARG, "row strides must cover H*dh elements");
  AttnParams p;
  p.q = (const bf16 *)q; p.k = (const bf16 *)k; p.vt = (const bf16 *)vt;
  p.q_lo = (const bf16 *)q_lo; p.k_lo = (const bf16 *)k_lo;
  p.qd = (const bf16 *)qd; p.kd = (const bf16 *)kd; p.vdt = (const bf16 *)vdt;
  p.nk = nk_valid; p.o = o; p.od = od; p.lse = lse;
  p.o2 = nullptr; p.nk_split = 0;
  p.q_bs = d.q_batch_stride; p.q_rs = d.q_row_stride;
  p.k_bs = d.k_batch_stride; p.k_rs = d.k_row_stride;
  p.vt_bs = d.vt_batch_stride; p.vt_hs = d.vt_head_stride; p.vt_rs = d.vt_row_stride;
  p.o_bs = d.o_batch_stride; p.o_rs = d.o_row_stride;
  p.B = d.B; p.H = d.H; p.Nq = d.Nq; p.Nk = d.Nk;
  p.out_dt = d.out_dtype;
  p.scale = d.scale != 0.f ? d.scale : (float)(1.0 / sqrt((double)d.dh));
  HIP_TRY(launch_attention(d.dh, tan, p, (hipStream_t)stream), "attention kernel launch");
  return T2VA_OK;
}

// ---------------------------------------------------------------------------
// The allocation-free entry point's workspace: one file-scope device array per
// GPU, held from the library's load until the process ends.  Host code never
// uses the array's name as an address: it takes the device address from
// hipGetSymbolAddress, once per device, with that device current.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = (size_t)128 << 20;   // T2VA_NOALLOC_SCRATCH_BYTES
static_assert(kNoAllocScratchBytes == (size_t)T2VA_NOALLOC_SCRATCH_BYTES, "header and library agree");
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxScratchDevices = 64;
void *g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch array (nullptr and a message on failure).
void *device_scratch(t2va_status *st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *st = hip_fail(e, "hipGetDevice");
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxScratchDevices) {
    *st = fail(T2VA_UNSUPPORTED_SHAPE, "device %d is beyond the %d devices the scratch table holds", dev,
               kMaxScratchDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      *st = e != hipSuccess ? hip_fail(e, "hipGetSymbolAddress(scratch)")
                            : fail(T2VA_HIP_ERROR, "hipGetSymbolAddress(scratch) returned NULL");
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *st = T2VA_OK;
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int t2va_abi_version(void) { return T2VA_ABI_VERSION; }

const char *t2va_last_error(void) { return g_err.c_str(); }

t2va_status t2va_trigflow_field(int mode, int B, int64_t n_per_sample, int a_dtype, int b_dtype,
                                int out_dtype, const double *t_host, const void *a, const void *b,
                                void *out, t2va_stream stream) {
  g_err.clear();
  if (mode != T2VA_NOISE && mode != T2VA_FIELD) return fail(T2VA_INVALID_ARG, "bad mode %d", mode);
  if (B < 1 || B > T2VA_MAX_BATCH)
    return fail(T2VA_UNSUPPORTED_SHAPE, "B = %d outside [1, %d]", B, T2VA_MAX_BATCH);
  if (n_per_sample < 0) return fail(T2VA_INVALID_ARG, "n_per_sample < 0");
  if (!valid_dtype(a_dtype) || !valid_dtype(b_dtype) || !valid_dtype(out_dtype))
    return fail(T2VA_INVALID_ARG, "dtypes must be T2VA_DTYPE_BF16 or T2VA_DTYPE_FP32");
  if (t2va_status st = check_t(B, t_host)) return st;
  if (n_per_sample == 0) return T2VA_OK;
  if (!a || !b || !out) return fail(T2VA_INVALID_ARG, "a, b and out must be non-NULL");
  if (!aligned16(a) || !aligned16(b) || !aligned16(out))
    return fail(T2VA_INVALID_ARG, "a, b and out must be 16-byte aligned");
  const CoefTable coef = make_coef(B, t_host, 0.0, 0.0, T2VA_PARAM_X0);
  HIP_TRY(launch_trigflow(mode, coef, n_per_sample, a_dtype, b_dtype, out_dtype, a, b, nullptr,
                          out, n_per_sample, n_per_sample, 0, n_per_sample, (hipStream_t)stream),
          "trigflow kernel launch");
  return T2VA_OK;
}

t2va_status t2va_joint_attn_fwd_jvp(const t2va_attn_desc *desc, const void *q, const void *k,
                                    const void *vt, const void *qd, const void *kd,
                                    const void *vdt, const int32_t *nk_valid, void *o, void *od,
                                    float *lse, t2va_stream stream) {
  g_err.clear();
  return attn_entry(desc, q, nullptr, k, nullptr, vt, qd, kd, vdt, nk_valid, o, od, lse, stream, false);
}

t2va_status t2va_v_transpose(int B, int N, int H, int dh, const void *v, int64_t v_batch_stride,
                             int64_t v_row_stride, void *vt, int64_t vt_batch_stride, int64_t vt_head_stride,
                             int64_t vt_row_stride, t2va_stream stream) {
  g_err.clear();
  if (B < 1 || N < 1 || H < 1) return fail(T2VA_UNSUPPORTED_SHAPE, "B, N and H must be >= 1");
  if (dh != 64 && dh != 128) return fail(T2VA_UNSUPPORTED_SHAPE, "dh = %d must be 64 or 128", dh);
  if (!v || !vt) return fail(T2VA_INVALID_ARG, "v and vt are required");
  if (!aligned16(v) || !aligned16(vt)) return fail(T2VA_INVALID_ARG, "v and vt must be 16-byte aligned");
  const int64_t strides[] = {v_batch_stride, v_row_stride, vt_batch_stride, vt_head_stride, vt_row_stride};
  for (int64_t st : strides)
    if (st < 0 || st % 8) return fail(T2VA_INVALID_ARG, "strides must be non-negative multiples of 8");
  if (v_row_stride < (int64_t)H * dh) return fail(T2VA_INVALID_ARG, "v_row_stride must cover H*dh elements");
  const int npad = (N + 63) / 64 * 64;
  if (vt_row_stride < npad)
    return fail(T2VA_INVALID_ARG, "vt_row_stride %lld < round_up(N, 64)", (long long)vt_row_stride);
  TransposeParams tp;
  tp.src = v; tp.s_bs = v_batch_stride; tp.s_hs = dh; tp.s_rs = v_row_stride;
  tp.dst = (bf16 *)vt; tp.d_bs = vt_batch_stride; tp.d_hs = vt_head_stride; tp.d_rs = vt_row_stride;
  tp.B = B; tp.H = H; tp.R = N; tp.C = dh; tp.Rpad = npad;
  HIP_TRY(launch_transpose(tp, 0, (hipStream_t)stream), "transpose kernel launch");
  return T2VA_OK;
}

t2va_status t2va_joint_attn_fwd_jvp_split(const t2va_attn_desc *desc, const void *q, const void *q_lo,
                                          const void *k, const void *k_lo, const void *vt, const void *qd,
                                          const void *kd, const void *vdt, const int32_t *nk_valid, void *o,
                                          void *od, float *lse, t2va_stream stream) {
  g_err.clear();
  return attn_entry(desc, q, q_lo, k, k_lo, vt, qd, kd, vdt, nk_valid, o, od, lse, stream, true);
}

size_t t2va_scm_workspace_bytes(const t2va_scm_desc *desc) {
  g_err.clear();
  if (check_desc(desc) != T2VA_OK) return 0;
  return make_layout(*desc).total;
}

t2va_status t2va_profile_enable(int max_calls) {
  g_err.clear();
  if (max_calls < 0) return fail(T2VA_INVALID_ARG, "max_calls < 0");
  for (hipEvent_t e : g_prof.pool) hipEventDestroy(e);
  g_prof = Profiler();
  if (max_calls == 0) return T2VA_OK;
  const size_t n = (size_t)max_calls * 64;   // up to 32 timed phases per call
  g_prof.pool.resize(n, nullptr);
  for (size_t i = 0; i < n; ++i) HIP_TRY(hipEventCreate(&g_prof.pool[i]), "hipEventCreate");
  g_prof.max_calls = max_calls;
  return T2VA_OK;
}

t2va_status t2va_profile_set_phases(unsigned phase_mask) {
  g_err.clear();
  if (!g_prof.recs.empty()) return fail(T2VA_INVALID_ARG, "read the recorded events first");
  g_prof_phases = phase_mask;
  return T2VA_OK;
}

t2va_status t2va_profile_read(double *ms_out, int *n_calls) {
  g_err.clear();
  if (!ms_out || !n_calls) return fail(T2VA_INVALID_ARG, "NULL output");
  for (int i = 0; i < T2VA_NUM_PHASES; ++i) ms_out[i] = 0.0;
  double other = 0.0;
  for (const auto &r : g_prof.recs) {
    HIP_TRY(hipEventSynchronize(r.b), "hipEventSynchronize");
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, r.a, r.b), "hipEventElapsedTime");
    ms_out[r.phase] += ms;
    (void)other;
  }
  double parts = ms_out[T2VA_PHASE_TEACHER_ATTN] + ms_out[T2VA_PHASE_STUDENT_ATTN] + ms_out[T2VA_PHASE_GEMM] +
                 ms_out[T2VA_PHASE_BWD_ATTN];
  // the remainder of the call, when the call and every timed part were recorded
  const unsigned need = (1u << T2VA_PHASE_TOTAL) | (1u << T2VA_PHASE_TEACHER_ATTN) |
                        (1u << T2VA_PHASE_STUDENT_ATTN) | (1u << T2VA_PHASE_GEMM) | (1u << T2VA_PHASE_BWD_ATTN);
  ms_out[T2VA_PHASE_OTHER] = (g_prof_phases & need) == need ? ms_out[T2VA_PHASE_TOTAL] - parts : 0.0;
  *n_calls = g_prof.calls;
  g_prof.recs.clear();
  g_prof.used = 0;
  g_prof.calls = 0;
  return T2VA_OK;
}

t2va_status t2va_scm_target(const t2va_scm_desc *desc, const t2va_block_weights *teacher,
                            const t2va_block_weights *student, const void *z0_v, const void *z0_a,
                            const void *eps_v, const void *eps_a, const void *text,
                            const uint8_t *text_mask, const double *t_host, float *J_v, float *J_a,
                            float *gbar_v, float *gbar_a, float *r_v, float *r_a, float *norms,
                            float *loss, void *workspace, size_t workspace_bytes,
                            t2va_stream stream) {
  g_err.clear();
  const t2va_block_weights *wb[2] = {teacher, student};
  const size_t needed = check_desc(desc) == T2VA_OK ? make_layout(*desc).total : 0;
  if (t2va_status st = validate_scm(desc, wb, z0_v, z0_a, eps_v, eps_a, text, text_mask, t_host, J_v, J_a,
                                    gbar_v, gbar_a, r_v, r_a, loss, workspace, workspace_bytes, needed))
    return st;
  hipStream_t s = (hipStream_t)stream;
  const bool prof = g_prof.active();
  if (prof) g_prof.calls++;
  PhaseScope total(s, T2VA_PHASE_TOTAL, prof);
  const bf16 *W[2][6];
  return run_scm(*desc, make_layout(*desc), wb, z0_v, z0_a, eps_v, eps_a, text, text_mask, t_host, J_v, J_a,
                 gbar_v, gbar_a, r_v, r_a, norms, loss, workspace, nullptr, W, s, prof);
}

t2va_status t2va_scm_target_noalloc(const t2va_scm_desc *desc, const t2va_block_weights *teacher,
                                    const t2va_block_weights *student, const void *z0_v, const void *z0_a,
                                    const void *eps_v, const void *eps_a, const void *text,
                                    const uint8_t *text_mask, const double *t_host, float *J_v, float *J_a,
                                    float *gbar_v, float *gbar_a, float *r_v, float *r_a, float *norms,
                                    float *loss, t2va_stream stream) {
  g_err.clear();
  const t2va_block_weights *wb[2] = {teacher, student};
  if (t2va_status st = check_desc(desc)) return st;
  const Layout L = make_layout(*desc, true);
  if (L.total > kNoAllocScratchBytes)
    return fail(T2VA_WORKSPACE_TOO_SMALL,
                "t2va_scm_target_noalloc: this shape needs %zu bytes of workspace; its static scratch holds %zu "
                "(use t2va_scm_target with a caller workspace)",
                L.total, kNoAllocScratchBytes);
  // validation with a stand-in address (the scratch is 256-byte aligned and large enough)
  if (t2va_status st = validate_scm(desc, wb, z0_v, z0_a, eps_v, eps_a, text, text_mask, t_host, J_v, J_a,
                                    gbar_v, gbar_a, r_v, r_a, loss, (void *)(uintptr_t)256, L.total, L.total))
    return st;
  t2va_status st = T2VA_OK;
  void *ws = device_scratch(&st);
  if (!ws) return st;
  hipStream_t s = (hipStream_t)stream;
  const bool prof = g_prof.active();
  if (prof) g_prof.calls++;
  PhaseScope total(s, T2VA_PHASE_TOTAL, prof);
  const bf16 *W[2][6];
  return run_scm(*desc, L, wb, z0_v, z0_a, eps_v, eps_a, text, text_mask, t_host, J_v, J_a, gbar_v, gbar_a, r_v,
                 r_a, norms, loss, ws, nullptr, W, s, prof);
}

// ---------------------------------------------------------------------------
// Training backward of the joint sCM loss.
// ---------------------------------------------------------------------------
size_t t2va_scm_grad_workspace_bytes(const t2va_scm_desc *desc) {
  g_err.clear();
  if (check_desc(desc) != T2VA_OK) return 0;
  if (desc->precision != T2VA_PREC_BF16) {
    fail(T2VA_INVALID_ARG, "t2va_scm_grad supports precision T2VA_PREC_BF16 only");
    return 0;
  }
  return make_grad_layout(*desc).total;
}

t2va_status t2va_scm_grad(const t2va_scm_desc *desc, const t2va_block_weights *teacher,
                          const t2va_block_weights *student, const void *z0_v, const void *z0_a,
                          const void *eps_v, const void *eps_a, const void *text,
                          const uint8_t *text_mask, const double *t_host, float *gbar_v, float *gbar_a,
                          float *norms, float *loss, const t2va_block_grads *grads, void *workspace,
                          size_t workspace_bytes, t2va_stream stream) {
  g_err.clear();
  const t2va_block_weights *wb[2] = {teacher, student};
  const bool ok_desc = check_desc(desc) == T2VA_OK;
  const size_t needed = ok_desc ? make_grad_layout(*desc).total : 0;
  if (t2va_status st = validate_scm(desc, wb, z0_v, z0_a, eps_v, eps_a, text, text_mask, t_host, nullptr,
                                    nullptr, gbar_v, gbar_a, nullptr, nullptr, loss, workspace,
                                    workspace_bytes, needed))
    return st;
  if (desc->precision != T2VA_PREC_BF16)
    return fail(T2VA_INVALID_ARG, "t2va_scm_grad supports precision T2VA_PREC_BF16 only");
  if (!grads) return fail(T2VA_INVALID_ARG, "grads is NULL");
  float *gout[6] = {grads->w_in_v, grads->w_in_a, grads->w_t, grads->w_qkv, grads->w_out_v, grads->w_out_a};
  for (float *g : gout)
    if (!g) return fail(T2VA_INVALID_ARG, "every gradient pointer is required");
  const t2va_scm_desc &d = *desc;
  const GradLayout G = make_grad_layout(d);
  const Layout &L = G.base;

  hipStream_t s = (hipStream_t)stream;
  const bool prof = g_prof.active();
  if (prof) g_prof.calls++;
  PhaseScope total(s, T2VA_PHASE_TOTAL, prof);
  char *ws = (char *)workspace;
  const bf16 *W[2][6];
  float *lse = (float *)(ws + G.lse);
  if (t2va_status st = run_scm(d, L, wb, z0_v, z0_a, eps_v, eps_a, text, text_mask, t_host, nullptr, nullptr,
                               gbar_v, gbar_a, nullptr, nullptr, norms, loss, workspace, lse, W, s, prof))
    return st;

  const Block blk(d.B, d.Nv, d.Na, d.Nt, d.Cv, d.Ca, d.d, d.H, L.ldv, s, prof);
  const int B = d.B, D = d.d, H = d.H, dh = L.dh, Nv = d.Nv, Na = d.Na, Nq = L.Nq, NA = L.N_all;
  const int64_t nv = blk.nv, na = blk.na;
  const CoefTable coef = make_coef(B, t_host, d.beta, d.gamma, d.param);
  const bf16 *const *Ws = W[1];
  bf16 *zv = (bf16 *)(ws + L.zv), *za = (bf16 *)(ws + L.za);   // primal halves: the block's inputs
  const float *E = (const float *)(ws + L.E);
  bf16 *X = (bf16 *)(ws + L.X), *QK = (bf16 *)(ws + L.QK), *VT = (bf16 *)(ws + L.VT);
  bf16 *O = (bf16 *)(ws + L.O);
  const int32_t *nk = (const int32_t *)(ws + L.nk);
  float *lse2 = (float *)(ws + G.lse2), *Dq = (float *)(ws + G.Dq);
  bf16 *wt_out_v = (bf16 *)(ws + G.wt_out_v), *wt_out_a = (bf16 *)(ws + G.wt_out_a);
  bf16 *wt_qkv = (bf16 *)(ws + G.wt_qkv);
  bf16 *dy_v = (bf16 *)(ws + G.dy_v), *dy_a = (bf16 *)(ws + G.dy_a);
  bf16 *dO = (bf16 *)(ws + G.dO), *dOT = (bf16 *)(ws + G.dOT), *QT = (bf16 *)(ws + G.QT);
  bf16 *KT = (bf16 *)(ws + G.KT), *Vrm = (bf16 *)(ws + G.Vrm), *dQKV = (bf16 *)(ws + G.dQKV);
  bf16 *dX = (bf16 *)(ws + G.dX);
  float *part = (float *)(ws + G.part);
  const int64_t o_bs = (int64_t)Nq * D, x_bs = (int64_t)NA * D, g_bs = (int64_t)NA * 3 * D;

  // dst[c][r] = src[r][c] per (b, h); see TransposeParams
  auto transpose = [&](const void *src, int src_f32, int64_t s_bs, int64_t s_hs, int64_t s_rs, bf16 *dst,
                       int64_t d_bs, int64_t d_hs, int64_t d_rs, int nb, int nh, int R, int C,
                       int Rpad) -> t2va_status {
    TransposeParams tp;
    tp.src = src; tp.s_bs = s_bs; tp.s_hs = s_hs; tp.s_rs = s_rs;
    tp.dst = dst; tp.d_bs = d_bs; tp.d_hs = d_hs; tp.d_rs = d_rs;
    tp.B = nb; tp.H = nh; tp.R = R; tp.C = C; tp.Rpad = Rpad;
    HIP_TRY(launch_transpose(tp, src_f32, s), "transpose");
    return T2VA_OK;
  };
  // rows [0, R) of B samples (batch stride s_bs, row stride s_rs, C columns)
  // -> dst [C][kp] with sample b at columns [b R, (b + 1) R) and zeros up to kp
  auto gather_t = [&](const bf16 *src, int64_t s_bs, int64_t s_rs, int R, int C, bf16 *dst,
                      int64_t kp) -> t2va_status {
    if (t2va_status st = transpose(src, 0, s_bs, 0, s_rs, dst, R, 0, kp, B, 1, R, C, R)) return st;
    const int tail = (int)(kp - (int64_t)B * R);
    if (tail > 0)
      return transpose(src, 0, 0, 0, s_rs, dst + (int64_t)B * R, 0, 0, kp, 1, 1, 0, C, tail);
    return T2VA_OK;
  };
  // out [M][N] fp32 = A [M][kp] . Wt [N][kp]^T, split-K over `splits` chunks of kc
  auto wgrad = [&](const bf16 *A, const bf16 *Wt, int64_t kp, int64_t kc, int splits, int M, int N,
                   float *out) -> t2va_status {
    if (splits == 1)
      return blk.gemm(A, kp, 0, Wt, kp, out, N, 0, 1, nullptr, 0, M, N, (int)kc, 1, nullptr, N, 0);
    if (t2va_status st = blk.gemm(A, kp, kc, Wt, kp, part, N, (int64_t)M * N, 1, nullptr, 0, M, N, (int)kc,
                                  splits, nullptr, N, kc))
      return st;
    HIP_TRY(launch_reduce_splits(part, splits, (int64_t)M * N, out, s), "split-K reduce");
    return T2VA_OK;
  };
#define T2VA_CALL(x) do { t2va_status _st = (x); if (_st) return _st; } while (0)

  // The token rows X of the student's primal batch (the folded forward never
  // forms them): the weight gradients contract over them.  tau holds the
  // student's [tau; dtau] rows.
  T2VA_CALL(blk.in_proj(Ws, zv, za, (const float *)(ws + L.tau), X, B));

  // ---- dL/dy at the block's outputs, and dO = dy W_out ----
  HIP_TRY(launch_seed(coef, (float)d.w_v, gbar_v, dy_v, nv, s), "seed");
  HIP_TRY(launch_seed(coef, (float)d.w_a, gbar_a, dy_a, na, s), "seed");
  T2VA_CALL(transpose(Ws[4], 0, 0, 0, D, wt_out_v, 0, 0, d.Cv, 1, 1, d.Cv, D, d.Cv));
  T2VA_CALL(transpose(Ws[5], 0, 0, 0, D, wt_out_a, 0, 0, d.Ca, 1, 1, d.Ca, D, d.Ca));
  T2VA_CALL(transpose(Ws[3], 0, 0, 0, D, wt_qkv, 0, 0, 3 * D, 1, 1, 3 * D, D, 3 * D));
  T2VA_CALL(blk.gemm(dy_v, d.Cv, nv, wt_out_v, d.Cv, dO, D, o_bs, 0, nullptr, 0, Nv, D, d.Cv, B, nullptr, D));
  T2VA_CALL(blk.gemm(dy_a, d.Ca, na, wt_out_a, d.Ca, dO + (int64_t)Nv * D, D, o_bs, 0, nullptr, 0, Na, D,
                     d.Ca, B, nullptr, D));

  // ---- attention backward ----
  HIP_TRY(launch_rowterms(dO, O, o_bs, D, B, H, dh, Nq, lse, lse2, Dq, s), "row terms");
  T2VA_CALL(transpose(QK, 0, blk.qk_bs, dh, 2 * D, QT, (int64_t)D * G.ldq, (int64_t)dh * G.ldq, G.ldq, B, H,
                      Nq, dh, G.ldq));
  T2VA_CALL(transpose(QK + D, 0, blk.qk_bs, dh, 2 * D, KT, (int64_t)D * L.ldv, (int64_t)dh * L.ldv, L.ldv, B,
                      H, NA, dh, L.ldv));
  T2VA_CALL(transpose(VT, 0, blk.vt_bs, blk.vt_hs, L.ldv, Vrm, x_bs, dh, D, B, H, dh, NA, dh));
  T2VA_CALL(transpose(dO, 0, o_bs, dh, D, dOT, (int64_t)D * G.ldq, (int64_t)dh * G.ldq, G.ldq, B, H, Nq, dh,
                      G.ldq));
  HIP_TRY(launch_zero_rows(dQKV, g_bs, 3 * D, B, Nq, NA, D, s), "zero rows");
  {
    AttnBwdParams ap;
    ap.q = QK; ap.k = QK + D; ap.v = Vrm; ap.dout = dO;
    ap.qt = QT; ap.kt = KT; ap.dot = dOT;
    ap.lse2 = lse2; ap.D = Dq; ap.nk = nk;
    ap.dq = dQKV; ap.dk = dQKV + D; ap.dv = dQKV + 2 * D;
    ap.q_bs = blk.qk_bs; ap.q_rs = 2 * D; ap.k_bs = blk.qk_bs; ap.k_rs = 2 * D;
    ap.v_bs = x_bs; ap.v_rs = D; ap.do_bs = o_bs; ap.do_rs = D;
    ap.qt_bs = (int64_t)D * G.ldq; ap.qt_hs = (int64_t)dh * G.ldq; ap.qt_rs = G.ldq;
    ap.kt_bs = (int64_t)D * L.ldv; ap.kt_hs = (int64_t)dh * L.ldv; ap.kt_rs = L.ldv;
    ap.dq_bs = g_bs; ap.dq_rs = 3 * D; ap.dk_bs = g_bs; ap.dk_rs = 3 * D;
    ap.B = B; ap.H = H; ap.Nq = Nq; ap.Nk = NA;
    ap.scale = (float)(1.0 / sqrt((double)dh));
    ap.part = (float *)(ws + G.part);
    ap.part_bytes = G.part_bytes;
    PhaseScope ps(s, T2VA_PHASE_BWD_ATTN, prof);
    HIP_TRY(launch_attention_bwd(dh, ap, s), "attention backward");
  }

  // ---- dX = dQKV W_qkv (video and audio rows), dW_qkv = dQKV^T X ----
  T2VA_CALL(blk.gemm(dQKV, 3 * D, g_bs, wt_qkv, 3 * D, dX, D, o_bs, 0, nullptr, 0, Nq, D, 3 * D, B, nullptr, D));
  bf16 *dqkvT = (bf16 *)(ws + G.dqkvT), *xT = (bf16 *)(ws + G.xT);
  T2VA_CALL(gather_t(dQKV, g_bs, 3 * D, NA, 3 * D, dqkvT, G.kp_all));
  T2VA_CALL(gather_t(X, x_bs, D, NA, D, xT, G.kp_all));
  T2VA_CALL(wgrad(dqkvT, xT, G.kp_all, G.kc_all, G.split_all, 3 * D, D, grads->w_qkv));

  // ---- output projections: dW_out = dy^T O ----
  bf16 *dyT_v = (bf16 *)(ws + G.dyT_v), *oT_v = (bf16 *)(ws + G.oT_v);
  bf16 *dyT_a = (bf16 *)(ws + G.dyT_a), *oT_a = (bf16 *)(ws + G.oT_a);
  T2VA_CALL(gather_t(dy_v, nv, d.Cv, Nv, d.Cv, dyT_v, G.kp_v));
  T2VA_CALL(gather_t(O, o_bs, D, Nv, D, oT_v, G.kp_v));
  T2VA_CALL(wgrad(dyT_v, oT_v, G.kp_v, G.kc_v, G.split_v, d.Cv, D, grads->w_out_v));
  T2VA_CALL(gather_t(dy_a, na, d.Ca, Na, d.Ca, dyT_a, G.kp_a));
  T2VA_CALL(gather_t(O + (int64_t)Nv * D, o_bs, D, Na, D, oT_a, G.kp_a));
  T2VA_CALL(wgrad(dyT_a, oT_a, G.kp_a, G.kc_a, G.split_a, d.Ca, D, grads->w_out_a));

  // ---- input projections: dW_in = dX^T z_in; time embedding: dW_t = (sum_rows dX) e^T ----
  bf16 *dxT_v = (bf16 *)(ws + G.dxT_v), *zT_v = (bf16 *)(ws + G.zT_v);
  bf16 *dxT_a = (bf16 *)(ws + G.dxT_a), *zT_a = (bf16 *)(ws + G.zT_a);
  T2VA_CALL(gather_t(dX, o_bs, D, Nv, D, dxT_v, G.kp_v));
  T2VA_CALL(gather_t(zv, nv, d.Cv, Nv, d.Cv, zT_v, G.kp_v));
  T2VA_CALL(wgrad(dxT_v, zT_v, G.kp_v, G.kc_v, G.split_v, D, d.Cv, grads->w_in_v));
  T2VA_CALL(gather_t(dX + (int64_t)Nv * D, o_bs, D, Na, D, dxT_a, G.kp_a));
  T2VA_CALL(gather_t(za, na, d.Ca, Na, d.Ca, zT_a, G.kp_a));
  T2VA_CALL(wgrad(dxT_a, zT_a, G.kp_a, G.kc_a, G.split_a, D, d.Ca, grads->w_in_a));
  HIP_TRY(launch_time_grad(dX, o_bs, D, B, Nq, D, E, (float *)(ws + G.tpart), grads->w_t, s), "time grad");
#undef T2VA_CALL
  return T2VA_OK;
}

// ---------------------------------------------------------------------------
// Joint DMD term and the stage-3 mix.
// ---------------------------------------------------------------------------
size_t t2va_dmd_workspace_bytes(const t2va_dmd_desc *desc) {
  g_err.clear();
  if (check_dmd_desc(desc) != T2VA_OK) return 0;
  return make_dmd_layout(*desc).total;
}

t2va_status t2va_dmd_target(const t2va_dmd_desc *desc, const t2va_block_weights *teacher,
                            const t2va_block_weights *fake, const void *x0_v, const void *x0_a,
                            const void *eps_v, const void *eps_a, const void *text,
                            const uint8_t *text_mask, const double *t_host, float *delta_v,
                            float *delta_a, float *scales, float *loss, void *workspace,
                            size_t workspace_bytes, t2va_stream stream) {
  g_err.clear();
  // ---------------- validation (before any HIP call) ----------------
  if (t2va_status st = check_dmd_desc(desc)) return st;
  const t2va_dmd_desc &d = *desc;
  if (t2va_status st = check_t(d.B, t_host)) return st;
  const t2va_block_weights *wb[2] = {teacher, fake};
  if (t2va_status st = check_weights(wb, 2, "teacher", "fake")) return st;
  const void *req[] = {x0_v, x0_a, eps_v, eps_a, delta_v, delta_a, loss};
  for (const void *p : req)
    if (!p) return fail(T2VA_INVALID_ARG, "x0, eps, delta and loss pointers are required");
  if (d.Nt > 0 && (!text || !text_mask))
    return fail(T2VA_INVALID_ARG, "text and text_mask are required when Nt > 0");
  const void *al[] = {x0_v, x0_a, eps_v, eps_a, text, delta_v, delta_a};
  for (const void *p : al)
    if (p && !aligned16(p)) return fail(T2VA_INVALID_ARG, "tensor operands must be 16-byte aligned");
  const DmdLayout L = make_dmd_layout(d);
  if (!workspace) return fail(T2VA_INVALID_ARG, "workspace is NULL");
  if (((uintptr_t)workspace & 255u) != 0) return fail(T2VA_INVALID_ARG, "workspace must be 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(T2VA_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);

  // ---------------- launch sequence ----------------
  hipStream_t s = (hipStream_t)stream;
  const bool prof = g_prof.active();
  if (prof) g_prof.calls++;
  PhaseScope total(s, T2VA_PHASE_TOTAL, prof);

  char *ws = (char *)workspace;
  Block blk(d.B, d.Nv, d.Na, d.Nt, d.Cv, d.Ca, d.d, d.H, L.ldv, s, prof, L.split);
  blk.apart = (float *)(ws + L.apart);
  blk.apart_bytes = L.apart_bytes;
  const int B = d.B, D = d.d, Nq = d.Nv + d.Na;
  const int64_t nv = blk.nv, na = blk.na;
  const CoefTable coef = make_coef(B, t_host, 0.0, 0.0, d.param);
  const bool guided = !(d.cfg_v == 1.0 && d.cfg_a == 1.0);

  const bf16 *W[2][6];
  HIP_TRY(prepare_weights(wb, 2, d.weight_dtype, L.w_elems, (bf16 *)(ws + L.wts), W, s), "cast");
  const bf16 *Wd[2] = {nullptr, nullptr};
  if (L.split) HIP_TRY(prepare_dup(W, 2, D, (bf16 *)(ws + L.wdup), Wd, s), "weight pairs");
  float *bqkv = (float *)(ws + L.bqkv);
  bf16 *const wfold = (bf16 *)(ws + L.wfold);
  if (t2va_status st = blk.fold_weights(W, wfold, (bf16 *)(ws + L.wint), (float *)(ws + L.fpart))) return st;
  const bf16 *Wf[2] = {wfold, wfold + fold_elems(d.Cv, d.Ca, D, L.split)};

  bf16 *zv = (bf16 *)(ws + L.zv), *za = (bf16 *)(ws + L.za);
  float *E = (float *)(ws + L.E), *tau = (float *)(ws + L.tau);
  bf16 *X = (bf16 *)(ws + L.X), *QK = (bf16 *)(ws + L.QK), *VT = (bf16 *)(ws + L.VT);
  bf16 *O = (bf16 *)(ws + L.O);
  int32_t *nk = (int32_t *)(ws + L.nk), *nk_null = (int32_t *)(ws + L.nk_null);
  float *xT_v = (float *)(ws + L.xT_v), *xT_a = (float *)(ws + L.xT_a);
  float *xF_v = (float *)(ws + L.xF_v), *xF_a = (float *)(ws + L.xF_a);

  // z_t = cos t x0 + sin t eps of the student's sample (the GEMM input: bf16,
  // or in split precision fp32 split into [hi | lo | hi] rows).
  if (!L.split) {
    const TrigSeg sv{x0_v, eps_v, nullptr, zv, nv, nv, nv, 0, nv, 0};
    const TrigSeg sa{x0_a, eps_a, nullptr, za, na, na, na, 0, na, 0};
    HIP_TRY(launch_trigflow_pair(0, coef, d.in_dtype, d.in_dtype, T2VA_DTYPE_BF16, sv, sa, s), "noise");
  } else {
    const TrigSeg sv{x0_v, eps_v, nullptr, zv, nv, nv, nv, 0, 3 * nv, 0, d.Cv};
    const TrigSeg sa{x0_a, eps_a, nullptr, za, na, na, na, 0, 3 * na, 0, d.Ca};
    HIP_TRY(launch_trigflow_pair(0, coef, d.in_dtype, d.in_dtype, kTrigSplitRows, sv, sa, s), "noise");
  }
  HIP_TRY(launch_time_embedding(coef, D, E, s), "time embedding");
  // tau and the QKV bias of the teacher (rows [0, B)) and the fake-score block ([B, 2B))
  float *tau_F = tau + (int64_t)B * D, *bqkv_F = bqkv + (int64_t)B * 3 * D;
  HIP_TRY(launch_row_linear_pair(D, D, RowLinSeg{E, W[0][2], tau, B}, RowLinSeg{E, W[1][2], tau_F, B}, s),
          "time linear");
  HIP_TRY(launch_row_linear_pair(D, 3 * D, RowLinSeg{tau, W[0][3], bqkv, B}, RowLinSeg{tau_F, W[1][3], bqkv_F, B},
                                 s),
          "QKV bias");
  if (d.Nt > 0)
    HIP_TRY(launch_text_rows(B, Nq, d.Nt, D, text, d.in_dtype, text_mask, X, blk.x_bs, blk.xs, L.split, B, nk, s),
            "text rows");
  else
    HIP_TRY(launch_fill_nk(nk, B, Nq, s), "fill nk");
  if (guided && Nq % 32 != 0) HIP_TRY(launch_fill_nk(nk_null, B, Nq, s), "fill nk");

#define T2VA_CALL(x) do { t2va_status _st = (x); if (_st) return _st; } while (0)
  // ---------------- teacher: conditional and null-condition passes ----------------
  // Both passes share Q, K and V; the null condition masks every text key, so
  // its attention runs over the video and audio keys only.  Guided, both
  // outputs stay fp32 (Of: batches [0, B) conditional, [B, 2B) unconditional)
  // and are combined, O = O_u + s_m (O_c - O_u), before the one bf16 rounding
  // of the output projection's input: the output projection is linear, so
  // this is the guided prediction, and the large scales (5 for audio) no
  // longer amplify two separate roundings.
  T2VA_CALL(blk.project_in_folded(W[0], Wd[0], Wf[0], zv, za, bqkv, X, QK, VT, B));
  if (guided) {
    float *Of = (float *)(ws + L.Of);
    if (Nq % 32 == 0) {
      // the text keys follow the video and audio keys, so the null-condition
      // output is the running state after the first Nq keys: one pass stores both
      T2VA_CALL(blk.attention(QK, VT, nk, Of, false, T2VA_PHASE_TEACHER_ATTN, nullptr, Of + (int64_t)B * blk.o_bs,
                              Nq, T2VA_DTYPE_FP32));
    } else {
      T2VA_CALL(blk.attention(QK, VT, nk, Of, false, T2VA_PHASE_TEACHER_ATTN, nullptr, nullptr, 0,
                              T2VA_DTYPE_FP32));
      T2VA_CALL(blk.attention(QK, VT, nk_null, Of + (int64_t)B * blk.o_bs, false, T2VA_PHASE_TEACHER_ATTN, nullptr,
                              nullptr, 0, T2VA_DTYPE_FP32));
    }
    HIP_TRY(launch_guide(Of, Of + (int64_t)B * blk.o_bs, O, B, Nq, d.Nv, D, (float)d.cfg_v, (float)d.cfg_a, s),
            "guidance");
  } else {
    T2VA_CALL(blk.attention(QK, VT, nk, O, false, T2VA_PHASE_TEACHER_ATTN));
  }
  T2VA_CALL(blk.project_out(W[0], O, xT_v, xT_a, B));

  // ---------------- fake-score block ----------------
  T2VA_CALL(blk.project_in_folded(W[1], Wd[1], Wf[1], zv, za, bqkv_F, X, QK, VT, B));
  T2VA_CALL(blk.attention(QK, VT, nk, O, false, T2VA_PHASE_TEACHER_ATTN));
  T2VA_CALL(blk.project_out(W[1], O, xF_v, xF_a, B));
#undef T2VA_CALL

  // ---------------- direction, residual scale, Delta, loss ----------------
  DmdParams dp;
  dp.x0[0] = x0_v; dp.x0[1] = x0_a;
  dp.eps[0] = eps_v; dp.eps[1] = eps_a;
  dp.tc[0] = xT_v; dp.tc[1] = xT_a;
  dp.tu[0] = nullptr;   // the teacher's prediction is already guided
  dp.tu[1] = nullptr;
  dp.fk[0] = xF_v; dp.fk[1] = xF_a;
  dp.x_bs[0] = nv; dp.x_bs[1] = na;
  dp.scale[0] = (float)d.cfg_v; dp.scale[1] = (float)d.cfg_a;
  dp.g[0] = delta_v; dp.g[1] = delta_a;
  dp.part_abs[0] = (float *)(ws + L.pa_v); dp.part_abs[1] = (float *)(ws + L.pa_a);
  dp.part_sq[0] = (float *)(ws + L.ps_v); dp.part_sq[1] = (float *)(ws + L.ps_a);
  dp.n[0] = nv; dp.n[1] = na;
  dp.nblk[0] = L.nblk_v; dp.nblk[1] = L.nblk_a;
  dp.in_dt = d.in_dtype;
  HIP_TRY(launch_dmd_direction(coef, dp, s), "DMD direction");
  NormParams np;
  np.mode = 1;
  np.g[0] = delta_v; np.g[1] = delta_a; np.r[0] = np.r[1] = nullptr;
  np.partial[0] = dp.part_abs[0]; np.partial[1] = dp.part_abs[1];
  np.partial2[0] = dp.part_sq[0]; np.partial2[1] = dp.part_sq[1];
  np.n[0] = nv; np.n[1] = na;
  np.nblk[0] = L.nblk_v; np.nblk[1] = L.nblk_a;
  np.norms = scales; np.loss = loss;
  np.eps = d.eps_dmd; np.w[0] = d.w_v; np.w[1] = d.w_a;
  HIP_TRY(launch_normalise(B, np, s), "normalise");
  return T2VA_OK;
}

t2va_status t2va_stage3_mix(int B, double lam_scm, double lam_dmd, const float *loss_scm,
                            const float *loss_dmd, float *out, t2va_stream stream) {
  g_err.clear();
  if (B < 1 || B > T2VA_MAX_BATCH)
    return fail(T2VA_UNSUPPORTED_SHAPE, "B = %d outside [1, %d]", B, T2VA_MAX_BATCH);
  if (!isfinite(lam_scm) || !isfinite(lam_dmd)) return fail(T2VA_INVALID_ARG, "lam must be finite");
  if (!loss_scm || !loss_dmd || !out) return fail(T2VA_INVALID_ARG, "NULL loss pointer");
  HIP_TRY(launch_mix(B, (float)lam_scm, loss_scm, (float)lam_dmd, loss_dmd, out, (hipStream_t)stream),
          "stage-3 mix");
  return T2VA_OK;
}

}  // extern "C"
