// Shared device helpers and the internal launch interface of libt2va.
// gfx950 (CDNA4) only: 64-lane wavefronts, bf16 MFMA, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace t2va {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kMaxBatch = 64;
constexpr int kWave = 64;

// fp32 <-> bf16.  The fp32 -> bf16 conversion compiles to gfx950's
// v_cvt_pk_bf16_f32 (round to nearest even).
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }

template <typename T> struct Store;
template <> struct Store<float> {
  __device__ __forceinline__ static float cvt(float x) { return x; }
};
template <> struct Store<bf16> {
  __device__ __forceinline__ static bf16 cvt(float x) { return (bf16)x; }
};

// 8 consecutive elements <-> 8 floats.
__device__ __forceinline__ void load8(const bf16 *p, float *f) {
  uint4 u = *reinterpret_cast<const uint4 *>(p);
  const bf16x8 v = __builtin_bit_cast(bf16x8, u);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (float)v[i];
}
__device__ __forceinline__ void load8(const float *p, float *f) {
  const float4 a = reinterpret_cast<const float4 *>(p)[0];
  const float4 b = reinterpret_cast<const float4 *>(p)[1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
__device__ __forceinline__ void store8(bf16 *p, const float *f) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (bf16)f[i];
  *reinterpret_cast<uint4 *>(p) = __builtin_bit_cast(uint4, v);
}
__device__ __forceinline__ void store8(float *p, const float *f) {
  reinterpret_cast<float4 *>(p)[0] = make_float4(f[0], f[1], f[2], f[3]);
  reinterpret_cast<float4 *>(p)[1] = make_float4(f[4], f[5], f[6], f[7]);
}

// Per-sample coefficients, rounded once from fp64 on the host; travels as a
// kernel argument so no host-to-device copy is needed.
//
// The block's inputs and outputs under its parameterisation:
//   token input   z_in = r z_t,   its tangent  r F_T + rdot z_t
//   time input    t_emb,          its tangent  t_emb_dot
//   x0-prediction x0 = rf ? z_in - t_emb y : y     (y = the block's output)
//   its tangent   rf ? (r F_T + rdot z_t) - t_emb_dot y - t_emb dy : dy
// x0-prediction block: r = 1, rdot = 0, t_emb = t, t_emb_dot = 1.
// Rectified-flow velocity block behind the TrigFlow wrapper: r = 1/(cos t + sin t),
// rdot = dr/dt, t_emb = t_rf = sin t/(cos t + sin t), t_emb_dot = r^2.
struct Coef {
  float cos_t, sin_t, inv_sin, ct_st, cos2, boost, gamma_ct_st;
  float r, rdot, t_emb, t_emb_dot;
};
struct CoefTable {
  int B;
  int rf;  // 1: rectified-flow velocity block behind the wrapper
  Coef c[kMaxBatch];
};

// ---------------------------------------------------------------------------
// Internal launchers (implemented in the .hip files).
// ---------------------------------------------------------------------------

// Elementwise TrigFlow maps.  op: 0 the block's token input r (cos a + sin b)
// (a=z0, b=eps; r = 1 for an x0-prediction block), 1 field (cos a - b)/sin
// (a=z_t, b=x0), 2 the tangent of the block's token input from the teacher's
// output x: with z = cos a + sin b, F_T = (cos z - x0(x))/sin, out = r F_T + rdot z.
hipError_t launch_trigflow(int op, const CoefTable &coef, int64_t n, int a_dt, int b_dt, int out_dt,
                           const void *a, const void *b, const float *x, void *out,
                           int64_t a_bs, int64_t b_bs, int64_t x_bs, int64_t out_bs,
                           hipStream_t s);
// Two such maps in one launch (the video and the audio rows): per sample,
// n elements from a, b (and x for op 2) into out, each with its own batch
// strides; vec is set by the launcher (16-byte accesses when n and the strides
// allow them).
struct TrigSeg {
  const void *a, *b;
  const float *x;
  void *out;
  int64_t n, a_bs, b_bs, x_bs, o_bs;
  int vec;
  int w;   // out_dt kTrigSplitRows only: the row width (a multiple of 8)
};
// out_dt of launch_trigflow_pair for split-precision GEMM rows: each row of w
// values becomes the bf16 row [hi | lo | hi] (3 w wide; hi = bf16(x),
// lo = bf16(x - hi)); o_bs counts output elements.
constexpr int kTrigSplitRows = 2;
hipError_t launch_trigflow_pair(int op, const CoefTable &coef, int a_dt, int b_dt, int out_dt, const TrigSeg &s1,
                                const TrigSeg &s2, hipStream_t s);

// Sinusoidal time embedding e(t_b) (rows 0..B-1) and de/dt (rows B..2B-1), fp32 [2B, d].
hipError_t launch_time_embedding(const CoefTable &coef, int d, float *E, hipStream_t s);

// out[r] = W e_r for r in [0, rows): fp32 [rows, n_out] from bf16 W [n_out, d] and fp32 E [rows, d]
// (tau = W_t e(t), and the QKV bias W_qkv tau).
// Two such products (same d and n_out) per launch; a problem with rows = 0 is skipped.
struct RowLinSeg {
  const float *E;
  const bf16 *W;
  float *out;
  int rows;
};
hipError_t launch_row_linear_pair(int d, int n_out, const RowLinSeg &s1, const RowLinSeg &s2, hipStream_t s);

// Text rows of X for B problems: for each sample b < copy_b, the valid text
// positions (mask != 0) in order, converted to bf16, at rows [Nq, Nq + count);
// rows up to Nq + Nt are zero.  Problems b >= copy_b get zero text rows (the
// tangent of the text, for the stacked primal and tangent batches).
// nk[b] = Nq + count for b < copy_b (written when nk != nullptr).  Rows are
// x_row_stride elements apart; with split, columns [d, 2d) of a row receive
// the low half bf16(x - bf16(x)) of each value (zero for bf16 text).
hipError_t launch_text_rows(int B, int Nq, int Nt, int d, const void *text, int text_dt,
                            const uint8_t *mask, bf16 *X, int64_t x_batch_stride, int64_t x_row_stride,
                            int split, int copy_b, int32_t *nk, hipStream_t s);

// Guided attention output of B samples [Nq][D] (fp32 conditional c and
// unconditional u, batch stride Nq D): out = bf16(u + s (c - u)) with s = s_v
// for rows < Nv, s_a for the rest.
hipError_t launch_guide(const float *c, const float *u, bf16 *out, int B, int Nq, int Nv, int D, float s_v,
                        float s_a, hipStream_t s);

// Folded weights from split-K partials part [splits][rows][Cv + Ca] (fp32,
// summed in split order): bf16 Wf [rows][Cv + Ca], or with split per modality
// [rows][3 C_m] = [hi | hi | lo] (hi = bf16(x), lo = bf16(x - hi); video
// first, audio at 3 rows Cv).  Cv, Ca multiples of 8.  nblk blocks' folds
// in one launch: block i reads part + i part_bs and writes Wf + i wf_bs.
hipError_t launch_fold_finish(const float *part, int splits, int rows, int Cv, int Ca, bool split, bf16 *Wf,
                              int nblk, int64_t part_bs, int64_t wf_bs, hipStream_t s);

// D [n][2k] = [W | W] for bf16 W [n][k] (k a multiple of 8): the weight of a
// product whose operand rows are [hi | lo] pairs; W0 -> D0 and, unless W1 is
// null, W1 -> D1 in the same launch.
hipError_t launch_dup_cols(const bf16 *W0, const bf16 *W1, bf16 *D0, bf16 *D1, int n, int k, hipStream_t s);

// nk[b] = value for every sample (used when there is no text).
hipError_t launch_fill_nk(int32_t *nk, int B, int value, hipStream_t s);

// Blocks the per-sample elementwise kernels use for n elements.
int elementwise_blocks(int64_t n);

// fp32 -> bf16 copies of count (at most kMaxCasts) arrays src[k] -> dst[k] of
// n[k] elements, in one launch.
constexpr int kMaxCasts = 12;
struct CastSet {
  const float *src[kMaxCasts];
  bf16 *dst[kMaxCasts];
  int64_t n[kMaxCasts];
  int64_t start[kMaxCasts + 1];
  int count;
};
hipError_t launch_cast_set(const float *const *src, bf16 *const *dst, const int64_t *n, int count, hipStream_t s);

// g, J and per-block partial sums of g^2 for both modalities.
struct GParams {
  const void *z0[2], *eps[2];
  const float *x0T[2], *x0S[2], *Gd[2];
  int64_t x_bs[2];   // batch stride (elements) of x0T/x0S/Gd
  float *J[2];       // nullable
  float *g[2];       // g (later normalised in place)
  float *partial[2]; // [B, nblk[m]]
  int64_t n[2];      // elements per sample per modality
  int nblk[2];
  int in_dt;
};
hipError_t launch_scm_direction(const CoefTable &coef, const GParams &p, hipStream_t s);

// DMD direction g = x0_F - x0_T with the guided teacher prediction
// x0_T = u + s (c - u) (c only when u is null), and per-block partial sums of
// |x0 - x0_T| and of g^2 for both modalities.
struct DmdParams {
  const void *x0[2], *eps[2];  // eps is read only for a rectified-flow block
  const float *tc[2], *tu[2], *fk[2];  // conditional / unconditional teacher, fake; tu nullable
  int64_t x_bs[2];     // batch stride (elements) of tc/tu/fk
  float scale[2];      // guidance scale per modality
  float *g[2];         // g (later normalised in place)
  float *part_abs[2];  // [B, nblk[m]]
  float *part_sq[2];   // [B, nblk[m]]
  int64_t n[2];
  int nblk[2];
  int in_dt;
};
hipError_t launch_dmd_direction(const CoefTable &coef, const DmdParams &p, hipStream_t s);

// Normalisation in place with the loss.
//   mode 0 (sCM): n = sqrt(sum partial), g /= n + eps, r = -g, norms = n,
//                 loss = sum_m w_m n_m^2/(n_m + eps)^2
//   mode 1 (DMD): c = (sum partial)/n_elems, g /= c + eps, norms = c,
//                 loss = sum_m w_m (sum partial2)/(c_m + eps)^2
struct NormParams {
  int mode;
  float *g[2];
  float *r[2];        // nullable
  const float *partial[2];
  const float *partial2[2];  // mode 1: partial sums of g^2
  int64_t n[2];
  int nblk[2];
  float *norms;       // nullable [B, 2]
  float *loss;        // [B]
  double eps, w[2];
};
hipError_t launch_normalise(int B, const NormParams &p, hipStream_t s);

// out[b] = a * x[b] + c * y[b] for b < B.
hipError_t launch_mix(int B, float a, const float *x, float c, const float *y, float *out,
                      hipStream_t s);

// C = A W^T (+ bias) for `batch` independent problems.
// c_dt: 0 bf16, 1 fp32, 2 split bf16: column c < n_split of a row receives
// hi = bf16(x) and column c + n_split lo = bf16(x - hi).
struct GemmParams {
  const bf16 *A; int64_t lda, a_bs;
  const bf16 *W; int64_t ldw, w_bs;       // W [N, K]; w_bs = 0 shares it across batches
  void *C; int64_t ldc, c_bs; int c_dt;   // columns [0, n_split) go to C
  const float *bias; int64_t bias_bs;     // nullable, fp32 [batch][N]
  bf16 *VT; int64_t vt_bs, vt_hs, vt_rs;  // columns >= n_split: V^T[b][h][c][row]
  int vt_rows;                            // V^T rows [M, vt_rows) are written as zeros
  int n_split, dh;
  int M, N, K, batch;
};
hipError_t launch_gemm(const GemmParams &p, hipStream_t s);
// Two GEMMs in one launch when both take the 128x128 tile (else one after the
// other): a small one then runs beside the other instead of after it.
hipError_t launch_gemm_pair(const GemmParams &a, const GemmParams &b, hipStream_t s);

// Attention forward (+JVP).  With q_lo and k_lo (q's and k's strides) the
// logits are scale (q k^T + q k_lo^T + q_lo k^T): the split-precision kernels.
struct AttnParams {
  const bf16 *q, *k, *vt, *qd, *kd, *vdt;
  const bf16 *q_lo = nullptr, *k_lo = nullptr;
  const int32_t *nk;
  void *o, *od;
  // forward only (nullable): o2 receives the output over the first nk_split
  // keys, a multiple of 32 no larger than any nk[b] (same strides as o)
  void *o2;
  int nk_split;
  float *lse;
  int64_t q_bs, q_rs, k_bs, k_rs, vt_bs, vt_hs, vt_rs, o_bs, o_rs;
  int B, H, Nq, Nk;
  int out_dt;
  float scale;
  // nullable scratch of part_bytes bytes: with it, the last tiles of each
  // XCD's range may run split over key ranges and be merged by a second kernel
  // (with o2, each piece needs room for two partial results)
  float *part = nullptr;
  size_t part_bytes = 0;
};
hipError_t launch_attention(int dh, bool tangent, const AttnParams &p, hipStream_t s);
// Scratch bytes that let launch_attention split the tail of a B x H x Nq launch
// (forward or JVP; `prefix`: forward launches with the o2 output) as far as it
// would.
size_t attention_split_bytes(int dh, int B, int H, int Nq, bool prefix = false);

// Attention backward for one (sample, head) grid: dQ, dK, dV from Q, K, V, dO,
// the forward's log2-unit log-sum-exp and D = rowsum(dO * O).  Row-major
// operands [b][row][h*dh + e] (strides *_bs, *_rs); transposed operands
// [b][h][e][token] (strides *_bs, *_hs, *_rs).
struct AttnBwdParams {
  const bf16 *q, *k, *v, *dout;          // row-major
  const bf16 *qt, *kt, *dot;             // transposed (Q^T, K^T, dO^T)
  const float *lse2, *D;                 // [B][H][Nq]
  const int32_t *nk;
  bf16 *dq, *dk, *dv;                    // row-major outputs
  int64_t q_bs, q_rs, k_bs, k_rs, v_bs, v_rs, do_bs, do_rs;
  int64_t qt_bs, qt_hs, qt_rs, kt_bs, kt_hs, kt_rs;
  int64_t dq_bs, dq_rs, dk_bs, dk_rs;    // dv uses dk's strides
  int B, H, Nq, Nk;
  float scale;
  // nullable scratch of part_bytes bytes: with it, the last tiles of each
  // XCD's range may run split (dQ over keys, dK/dV over queries) and be summed
  // by a second kernel
  float *part = nullptr;
  size_t part_bytes = 0;
};
hipError_t launch_attention_bwd(int dh, const AttnBwdParams &p, hipStream_t s);
// Scratch bytes that let launch_attention_bwd split the tails of its two kernels.
size_t attention_bwd_split_bytes(int dh, int B, int H, int Nq, int Nk);

// ---- the training backward's HBM-bound steps ----
// dy = bf16(2 w bo / sin t * gbar) per sample (bo = 1, or -t_rf behind the wrapper).
hipError_t launch_seed(const CoefTable &coef, float w, const float *gbar, bf16 *dy, int64_t n, hipStream_t s);
// dst[c][r] = src[r][c] per (b, h) slice; dst rows r in [R, Rpad) are zeros.
struct TransposeParams {
  const void *src; int64_t s_bs, s_hs, s_rs;
  bf16 *dst; int64_t d_bs, d_hs, d_rs;
  int B, H, R, C, Rpad;
};
hipError_t launch_transpose(const TransposeParams &p, int src_fp32, hipStream_t s);
// n (at most 4) bf16 transposes in one launch when each is eligible for the
// vectorised kernel (16-byte aligned source rows), else one launch each.
hipError_t launch_transpose_set(const TransposeParams *ps, int n, hipStream_t s);
// D = rowsum(dO * O) per (b, h, q) and lse2 = lse * log2(e).
hipError_t launch_rowterms(const bf16 *dO, const bf16 *O, int64_t bs, int64_t rs, int B, int H, int dh, int Nq,
                           const float *lse, float *lse2, float *D, hipStream_t s);
hipError_t launch_zero_rows(bf16 *X, int64_t bs, int64_t rs, int B, int r0, int r1, int cols, hipStream_t s);
// dW_t = sum_b (sum_rows dX[b]) e_b^T with fixed-order partial sums
// (part: B * (colsum_chunks(rows) + 1) * d floats).
int colsum_chunks(int rows);
hipError_t launch_time_grad(const bf16 *dX, int64_t bs, int64_t rs, int B, int rows, int d, const float *E,
                            float *part, float *dWt, hipStream_t s);
hipError_t launch_reduce_splits(const float *part, int splits, int64_t n, float *out, hipStream_t s);

}  // namespace t2va
