/*
 * t2va.h - C ABI of the MI355X (gfx950) joint sCM target library (libt2va.so).
 *
 * The library computes the training target of TurboT2VA's joint
 * continuous-time consistency (sCM) stage for paired video and audio latents
 * (arXiv 2608.24674; "TurboT2VA：分数正则化一致性蒸馏加速 19B 视频音频联合生成",
 * robotworld.top deep read, sections 3 and 3.1).  All GPU work is hand-written
 * HIP for gfx950 and is enqueued on the caller's stream.
 *
 * Conventions shared by every entry point
 *   - Device pointers are plain HIP device addresses; host pointers are named
 *     *_host.  Nothing is allocated on the hot path: the caller owns every
 *     buffer, including the workspace.  Inputs are never written; outputs are
 *     fully overwritten (never accumulated into).
 *   - Matrices are row-major.  "bf16" is bfloat16 (1-8-7), "fp32" IEEE single.
 *   - Weights follow the nn.Linear convention [out_features, in_features]:
 *     y = x W^T.
 *   - All host-side validation happens before the first launch.  A failing
 *     call returns a non-zero status, launches nothing and records a message
 *     that t2va_last_error() returns (thread-local).  No exception or abort
 *     crosses the ABI.  A failure reported by the HIP runtime at launch maps to
 *     T2VA_HIP_ERROR; work already enqueued by that call may have run.
 *   - Work is asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  Outputs are valid once the caller synchronises that stream.
 *   - Results are deterministic: no floating-point atomics; reductions run in
 *     a fixed order, so identical inputs give bitwise-identical outputs on a
 *     given device configuration.  (The attention launches of the entry points
 *     that take a workspace cut the last tiles of each XCD into key or query
 *     ranges merged in a fixed order; how they cut depends on the device's
 *     compute-unit count, so a GPU with another count, or another partition
 *     mode, may differ in the last bits.)
 *   - Calls on the same stream are ordered; calls on different streams that
 *     share a workspace race.
 */
#ifndef T2VA_H
#define T2VA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define T2VA_ABI_VERSION 3

typedef int t2va_status;
#define T2VA_OK 0
#define T2VA_INVALID_ARG 1
#define T2VA_UNSUPPORTED_SHAPE 2
#define T2VA_WORKSPACE_TOO_SMALL 3
#define T2VA_HIP_ERROR 4

#define T2VA_DTYPE_BF16 0
#define T2VA_DTYPE_FP32 1

/* The joint block's parameterisation (deep read, section 4.2).
 * T2VA_PARAM_X0: the block predicts x0 directly at the TrigFlow inputs (z_t, t).
 * T2VA_PARAM_RF: the block is a rectified-flow velocity model behind the
 *   TrigFlow wrapper: it sees z_rf = z_t/(cos t + sin t) and
 *   t_rf = sin t/(cos t + sin t) (the time embedding takes t_rf), and its
 *   output v is turned into x0 = z_rf - t_rf v (the rectified-flow relation
 *   z_rf = (1 - t_rf) x0 + t_rf eps, v = eps - x0, solved for x0).  The JVP
 *   passes through the wrapper and the time embedding. */
#define T2VA_PARAM_X0 0
#define T2VA_PARAM_RF 1

/* Precision of the primal logit path (the descriptors' `precision` field).
 * T2VA_PREC_BF16: every activation between kernels is stored in bf16 (fp32
 *   accumulation inside each kernel).
 * T2VA_PREC_SPLIT: the primal values that decide the attention logits -- the
 *   noised latents, the folded weights W_qkv W_in (and the token rows X of the
 *   text) and the projections Q and K -- are carried as pairs hi + lo of bf16
 *   values (hi = bf16(x), lo = bf16(x - hi), about 16 significant bits).  The
 *   projections contract the pairs on the matrix cores with fp32 accumulation
 *   (dropping only the lo x lo product), and the attention kernels form the
 *   logits as Q_hi K_hi^T + Q_hi K_lo^T + Q_lo K_hi^T.
 *   Tangents, V and the attention outputs stay bf16.  This is for inputs whose
 *   logits are large enough that a bf16 rounding of Q or K (a relative 2^-9)
 *   moves a logit by a sizeable fraction of one unit, which makes softmax,
 *   and with it J, sensitive to the storage rounding: scaled latents at small t
 *   (deep read, section 3.1, the J_theta equation near t -> 0).  It costs three
 *   times the latent-row projection work, twice the text rows', and 1.5 to 2
 *   times the logit work. */
#define T2VA_PREC_BF16 0
#define T2VA_PREC_SPLIT 1

/* Largest batch one call accepts (per-sample coefficients travel as kernel
 * arguments). */
#define T2VA_MAX_BATCH 64

typedef void *t2va_stream; /* hipStream_t */

/* Returns T2VA_ABI_VERSION of the loaded library. */
int t2va_abi_version(void);

/* Message describing the last failing call on this thread ("" if none).
 * The pointer stays valid until the next call on this thread. */
const char *t2va_last_error(void);

/* ------------------------------------------------------------------------ */
/* Elementwise TrigFlow maps                                                 */
/* ------------------------------------------------------------------------ */
#define T2VA_NOISE 0 /* out = cos(t) a + sin(t) b          (a = z0,  b = eps)     */
#define T2VA_FIELD 1 /* out = (cos(t) a - b) / sin(t)      (a = z_t, b = x0_hat)  */

/*
 * t2va_trigflow_field - TrigFlow noising z_t = cos t z0 + sin t eps (deep read,
 * section 3, noising equation) or the TrigFlow field
 * F = (cos t z_t - x0_hat)/sin t (section 3.1, field equation), per sample.
 *
 *   mode            T2VA_NOISE or T2VA_FIELD.
 *   B               samples, 1..T2VA_MAX_BATCH.
 *   n_per_sample    elements per sample (>= 0); a, b, out are [B, n_per_sample],
 *                   contiguous, 16-byte aligned device buffers.
 *   a_dtype, b_dtype, out_dtype   T2VA_DTYPE_BF16 or T2VA_DTYPE_FP32.
 *   t_host          host array of B timesteps, each finite with 0 < t < pi/2.
 * Arithmetic is fp32 with coefficients rounded once from fp64.
 * Errors: T2VA_INVALID_ARG (null pointer, bad mode/dtype, t out of range,
 * misalignment), T2VA_UNSUPPORTED_SHAPE (B out of range).
 */
t2va_status t2va_trigflow_field(int mode, int B, int64_t n_per_sample, int a_dtype, int b_dtype,
                                int out_dtype, const double *t_host, const void *a, const void *b,
                                void *out, t2va_stream stream);

/* ------------------------------------------------------------------------ */
/* Joint attention forward + forward-mode JVP                                */
/* ------------------------------------------------------------------------ */
/*
 * Operand layouts (all strides in elements, all bf16):
 *   q, qd   element (b, i, h, c) at  b*q_batch_stride + i*q_row_stride + h*dh + c
 *           (sequence-major; the projection's [B, N, H*dh] output works as is)
 *   k, kd   element (b, j, h, c) at  b*k_batch_stride + j*k_row_stride + h*dh + c
 *   vt, vdt V stored dh-major per head ("V transposed"; t2va_v_transpose
 *           converts a sequence-major V):
 *           element (b, j, h, c) at  b*vt_batch_stride + h*vt_head_stride + c*vt_row_stride + j
 *           vt_row_stride must be a multiple of 8 and >= round_up(Nk, 64).  Keys
 *           are read in blocks of 64: columns j in [nk_valid[b], round_up(nk_valid[b], 64))
 *           must hold finite values (zeros, say); they get zero weight.
 *   o, od   element (b, i, h, c) at  b*o_batch_stride + i*o_row_stride + h*dh + c,
 *           dtype out_dtype.
 *   lse     fp32 [B, H, Nq] (nullable): natural-log log-sum-exp of the scaled
 *           logits of each query row.
 * Tangent operands use the same strides as their primal operands.
 */
typedef struct {
  int B, H, dh;  /* dh in {64, 128} */
  int Nq;        /* query rows per sample (>= 1) */
  int Nk;        /* key rows present per sample (>= 1); nk_valid[b] <= Nk */
  int64_t q_batch_stride, q_row_stride;
  int64_t k_batch_stride, k_row_stride;
  int64_t vt_batch_stride, vt_head_stride, vt_row_stride;
  int64_t o_batch_stride, o_row_stride;
  int has_tangent; /* 0: forward only (qd, kd, vdt, od must be NULL) */
  int out_dtype;   /* T2VA_DTYPE_BF16 or T2VA_DTYPE_FP32 */
  float scale;     /* logit scale, finite and >= 0; 0 selects 1/sqrt(dh) */
} t2va_attn_desc;

/*
 * t2va_joint_attn_fwd_jvp - O = softmax(scale Q K^T + mask) V and its tangent
 * dO along (dQ, dK, dV) for every (sample, head):
 *   dO = P (dS - mu) V + P dV,  dS = scale (dQ K^T + Q dK^T),  mu = rowsum(P * dS),
 * where keys j >= nk_valid[b] are excluded (logit -inf).  This is the attention
 * step of the joint block through which the joint JVP of the sCM stage passes
 * (deep read, section 3.1, J_theta equation; section 4.2: the JVP passes
 * through the cross-modal transformer; section 6.3: padded text positions are
 * removed from the keys).  Softmax state and accumulators are fp32; P and
 * P*dS enter the matrix cores as bf16.  This entry point has no workspace and
 * always runs every tile whole (the workspace-carrying entry points may split
 * the last tiles, which changes rounding in the last bits only).
 *   nk_valid  device int32 [B], each in [1, Nk].  Values outside that range
 *             are clamped to it by the kernel.
 * Errors: T2VA_INVALID_ARG (null/misaligned pointers, strides not multiples
 * of 8, vt_row_stride too small, tangent pointers inconsistent with
 * has_tangent), T2VA_UNSUPPORTED_SHAPE (dh not 64/128, B/H/Nq/Nk < 1, or the
 * K or V^T extent of one (sample, head) at or above 2 GiB).
 */
t2va_status t2va_joint_attn_fwd_jvp(const t2va_attn_desc *desc, const void *q, const void *k,
                                    const void *vt, const void *qd, const void *kd,
                                    const void *vdt, const int32_t *nk_valid, void *o, void *od,
                                    float *lse, t2va_stream stream);

/*
 * t2va_v_transpose - V (or dV) from the sequence-major layout of q and k to
 * the dh-major layout the attention entry points take for V:
 *   vt[b*vt_batch_stride + h*vt_head_stride + c*vt_row_stride + j]
 *       = v[b*v_batch_stride + j*v_row_stride + h*dh + c]        for j < N,
 * and columns j in [N, round_up(N, 64)) are written as zeros.  The joint
 * block's own QKV projection writes V in the dh-major layout directly; this is
 * for callers holding V sequence-major, e.g. in place in a fused [B, N, 3 H dh]
 * projection output (v then points at its V columns).
 *   B, N, H >= 1; dh in {64, 128}; all strides in elements, non-negative
 *   multiples of 8; v_row_stride >= H*dh; vt_row_stride >= round_up(N, 64);
 *   v and vt 16-byte aligned device buffers that do not overlap.
 * Errors: T2VA_INVALID_ARG (null/misaligned pointers, strides),
 * T2VA_UNSUPPORTED_SHAPE (B, N, H < 1 or dh not 64/128).
 */
t2va_status t2va_v_transpose(int B, int N, int H, int dh, const void *v, int64_t v_batch_stride,
                             int64_t v_row_stride, void *vt, int64_t vt_batch_stride, int64_t vt_head_stride,
                             int64_t vt_row_stride, t2va_stream stream);

/*
 * t2va_joint_attn_fwd_jvp_split - as t2va_joint_attn_fwd_jvp, with the logits
 * taken from split operands (T2VA_PREC_SPLIT): the query is q + q_lo and the key
 * k + k_lo (q_lo and k_lo bf16 with q's and k's strides), and
 *   s = scale (q k^T + q k_lo^T + q_lo k^T)
 * in fp32 (the lo x lo term, 2^-16 of the product, is left out).  The tangent
 * logits and P V use q, k, vt and their tangents as in t2va_joint_attn_fwd_jvp.
 * Errors: as t2va_joint_attn_fwd_jvp, plus T2VA_INVALID_ARG for a NULL or
 * misaligned q_lo or k_lo.
 */
t2va_status t2va_joint_attn_fwd_jvp_split(const t2va_attn_desc *desc, const void *q, const void *q_lo,
                                          const void *k, const void *k_lo, const void *vt, const void *qd,
                                          const void *kd, const void *vdt, const int32_t *nk_valid, void *o,
                                          void *od, float *lse, t2va_stream stream);

/* ------------------------------------------------------------------------ */
/* The joint sCM target                                                      */
/* ------------------------------------------------------------------------ */
typedef struct {
  int B;        /* samples, 1..T2VA_MAX_BATCH */
  int Nv, Na;   /* video and audio tokens per sample (>= 1 each) */
  int Nt;       /* text positions per sample (>= 0) */
  int Cv, Ca;   /* latent channels, multiples of 64 */
  int d, H;     /* block width and heads; d = H*dh with dh in {64, 128} */
  int in_dtype; /* dtype of z0, eps and text: T2VA_DTYPE_BF16 or T2VA_DTYPE_FP32 */
  int weight_dtype; /* dtype of all weights: T2VA_DTYPE_BF16 or T2VA_DTYPE_FP32
                       (fp32 weights are rounded to bf16 into the workspace) */
  double beta;  /* consistency boost (section 3.1) */
  double gamma; /* tangent warm-up ratio, 0 <= gamma <= 1 */
  double eps_scm; /* > 0, added to the L2 norm */
  double w_v, w_a; /* modality weights of the joint loss */
  int param;       /* T2VA_PARAM_X0 or T2VA_PARAM_RF (the block's parameterisation) */
  int precision;   /* T2VA_PREC_BF16 or T2VA_PREC_SPLIT (zero-initialised: bf16) */
} t2va_scm_desc;

/* One copy of the joint block (teacher or student); device pointers. */
typedef struct {
  const void *w_in_v;  /* [d, Cv] */
  const void *w_in_a;  /* [d, Ca] */
  const void *w_t;     /* [d, d]  linear layer after the sinusoidal time embedding */
  const void *w_qkv;   /* [3d, d] rows 0..d-1: W_q, d..2d-1: W_k, 2d..3d-1: W_v */
  const void *w_out_v; /* [Cv, d] */
  const void *w_out_a; /* [Ca, d] */
} t2va_block_weights;

/* Exact workspace size in bytes for t2va_scm_target with this descriptor
 * (0 if the descriptor is invalid; t2va_last_error() says why).  It covers the
 * activations and tangents of both blocks, partial sums, and the scratch in
 * which the attention launches merge the pieces of their split last tiles. */
size_t t2va_scm_workspace_bytes(const t2va_scm_desc *desc);

/*
 * t2va_scm_target - the joint sCM target (deep read, section 3 and 3.1):
 *   z_t^m  = cos t z0^m + sin t eps^m                         (shared t, m in {v, a})
 *   x0_T   = G_T(z_t^v, z_t^a, t, c),  F_T^m = (cos t z_t^m - x0_T^m)/sin t
 *   x0_S, dG = G_S and its JVP along (dt = 1, dz^v = F_T^v, dz^a = F_T^a, dc = 0)
 *   F_S^m  = (cos t z_t^m - x0_S^m)/sin t
 *   J^m    = cos t sin t * d/ds F_S^m along that tangent
 *   g^m    = -beta cos t/sqrt(1 - gamma^2 sin^2 t) (F_S^m - F_T^m) - gamma cos t sin t z_t^m - J^m
 *   n^m    = ||g^m||_2 over all Nm*Cm elements of one sample's modality
 *   gbar^m = g^m/(n^m + eps_scm),  r^m = F_S - sg(F_S) - gbar^m = -gbar^m (value)
 *   loss_b = w_v ||r^v||^2 + w_a ||r^a||^2
 * G is the joint block: per-modality input projection plus a sinusoidal
 * time embedding (base 10000, [cos | sin]) through w_t; one multi-head
 * self-attention whose queries are the video and audio tokens and whose keys
 * are video, audio and the valid text tokens; per-modality output projection.
 * With desc->param == T2VA_PARAM_RF both blocks are rectified-flow velocity
 * models behind the TrigFlow wrapper (see T2VA_PARAM_RF): G above is then the
 * wrapped x0-prediction, and the JVP runs through the wrapper.
 *
 * Inputs (device):
 *   z0_v, eps_v  [B, Nv, Cv] in_dtype     z0_a, eps_a [B, Na, Ca] in_dtype
 *   text         [B, Nt, d]  in_dtype     text_mask   uint8 [B, Nt], nonzero = valid
 *   t_host       host double [B], each finite with 0 < t < pi/2
 * Outputs (device, fp32):
 *   J_v [B, Nv, Cv], J_a [B, Na, Ca]           nullable
 *   gbar_v, gbar_a  same shapes                 required
 *   r_v, r_a        same shapes                 nullable
 *   norms [B, 2]  (n^v, n^a)                    nullable
 *   loss  [B]                                   required
 * workspace: device buffer of at least t2va_scm_workspace_bytes(desc) bytes,
 * 256-byte aligned; its contents on entry are irrelevant.
 * Errors: T2VA_INVALID_ARG (null required pointers, misalignment, t out of
 * range, gamma outside [0, 1], eps_scm <= 0, bad dtypes, unknown precision),
 * T2VA_UNSUPPORTED_SHAPE (d != H*dh, dh not 64/128, Cv/Ca not multiples of 64,
 * B out of range, or (Nv + Na + Nt + 128) * 3d * 2 bytes >= 2 GiB: one
 * sample's rows must fit 32-bit buffer offsets), T2VA_WORKSPACE_TOO_SMALL.
 */
t2va_status t2va_scm_target(const t2va_scm_desc *desc, const t2va_block_weights *teacher,
                            const t2va_block_weights *student, const void *z0_v, const void *z0_a,
                            const void *eps_v, const void *eps_a, const void *text,
                            const uint8_t *text_mask, const double *t_host, float *J_v, float *J_a,
                            float *gbar_v, float *gbar_a, float *r_v, float *r_a, float *norms,
                            float *loss, void *workspace, size_t workspace_bytes,
                            t2va_stream stream);

/*
 * t2va_scm_target_noalloc - t2va_scm_target for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It allocates nothing: its workspace is a static
 * device array of T2VA_NOALLOC_SCRATCH_BYTES bytes in the library, one per GPU
 * the library runs on, held until the process ends.  Arguments and outputs are
 * those of t2va_scm_target without the workspace; the stream must belong to
 * the current device.  Every attention tile runs whole (no split tails), so
 * results may differ from t2va_scm_target's in the last bits.
 * Shapes whose workspace exceeds the scratch (for one sample at d = 1024,
 * roughly 3,000 tokens; the small workload fits, the standard one does not)
 * are rejected with T2VA_WORKSPACE_TOO_SMALL before any launch.
 * All calls on one GPU share its scratch: calls that overlap on one GPU (two
 * streams, or two host threads) race and must be ordered by the caller.  Its
 * contents on entry are irrelevant (every buffer is written before it is
 * read).  The first call on a device looks up the scratch's device address.
 * Errors: as t2va_scm_target, plus T2VA_WORKSPACE_TOO_SMALL for shapes beyond
 * the scratch and T2VA_HIP_ERROR if the address lookup fails.
 */
#define T2VA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
t2va_status t2va_scm_target_noalloc(const t2va_scm_desc *desc, const t2va_block_weights *teacher,
                                    const t2va_block_weights *student, const void *z0_v, const void *z0_a,
                                    const void *eps_v, const void *eps_a, const void *text,
                                    const uint8_t *text_mask, const double *t_host, float *J_v, float *J_a,
                                    float *gbar_v, float *gbar_a, float *r_v, float *r_a, float *norms,
                                    float *loss, t2va_stream stream);

/* ------------------------------------------------------------------------ */
/* Training backward of the joint sCM loss                                   */
/* ------------------------------------------------------------------------ */

/* Gradients of the student's weights, fp32 device arrays shaped like the
 * weights of t2va_block_weights (overwritten, not accumulated into). */
typedef struct {
  float *w_in_v;  /* [d, Cv] */
  float *w_in_a;  /* [d, Ca] */
  float *w_t;     /* [d, d]  */
  float *w_qkv;   /* [3d, d] */
  float *w_out_v; /* [Cv, d] */
  float *w_out_a; /* [Ca, d] */
} t2va_block_grads;

/* Exact workspace size in bytes for t2va_scm_grad (0 if the descriptor is invalid). */
size_t t2va_scm_grad_workspace_bytes(const t2va_scm_desc *desc);

/*
 * t2va_scm_grad - the joint sCM target (as t2va_scm_target: gbar, norms, loss)
 * and the gradient of sum_b L_b with respect to every student weight
 * (deep read, section 3.1: r = F_S - sg(F_S) - gbar, L_b = sum_m w_m ||r^m||^2).
 * gbar is a constant (stop-gradient) target, so the gradient flows only
 * through the student's primal forward pass:
 *   dL/dF_S^m = -2 w_m gbar^m,  dL/dx0_S^m = 2 w_m gbar^m / sin t
 *   (behind the TrigFlow wrapper, dL/dv = -t_rf dL/dx0),
 * then back through the output projections, the joint attention (softmax
 * backward, keys = video, audio and valid text), the fused QKV projection,
 * the input projections and the time-embedding linear layer.  Divide by B
 * for the gradient of the batch mean.
 * Inputs and the target's outputs as in t2va_scm_target (J and r are not
 * produced); grads: all six pointers required.
 * workspace: at least t2va_scm_grad_workspace_bytes(desc) bytes, 256-byte aligned.
 * The backward is built for desc->precision == T2VA_PREC_BF16 only (it
 * recomputes the softmax from bf16 Q and K): T2VA_PREC_SPLIT is rejected.
 * Errors: as t2va_scm_target, plus T2VA_INVALID_ARG for NULL gradient pointers
 * and for T2VA_PREC_SPLIT.
 * Deterministic: no atomics; every reduction runs in a fixed order.
 */
t2va_status t2va_scm_grad(const t2va_scm_desc *desc, const t2va_block_weights *teacher,
                          const t2va_block_weights *student, const void *z0_v, const void *z0_a,
                          const void *eps_v, const void *eps_a, const void *text,
                          const uint8_t *text_mask, const double *t_host, float *gbar_v, float *gbar_a,
                          float *norms, float *loss, const t2va_block_grads *grads, void *workspace,
                          size_t workspace_bytes, t2va_stream stream);

/* ------------------------------------------------------------------------ */
/* Joint DMD term and the stage-3 objective                                  */
/* ------------------------------------------------------------------------ */

typedef struct {
  int B;        /* samples, 1..T2VA_MAX_BATCH */
  int Nv, Na;   /* video and audio tokens per sample (>= 1) */
  int Nt;       /* text positions per sample (>= 0) */
  int Cv, Ca;   /* latent channels, multiples of 64 */
  int d, H;     /* block width and heads; d = H*dh with dh in {64, 128} */
  int in_dtype; /* dtype of x0, eps and text: T2VA_DTYPE_BF16 or T2VA_DTYPE_FP32 */
  int weight_dtype; /* dtype of all weights (fp32 is rounded to bf16 in the workspace) */
  double cfg_v, cfg_a; /* guidance scales of the teacher prediction per modality
                          (finite; 1 for both skips the unconditional pass) */
  double eps_dmd;      /* > 0, added to the residual scale */
  double w_v, w_a;     /* modality weights of the joint loss */
  int param;           /* T2VA_PARAM_X0 or T2VA_PARAM_RF, as in t2va_scm_desc */
  int precision;       /* T2VA_PREC_BF16 or T2VA_PREC_SPLIT, as in t2va_scm_desc */
} t2va_dmd_desc;

/* Exact workspace size in bytes for t2va_dmd_target (0 if the descriptor is invalid). */
size_t t2va_dmd_workspace_bytes(const t2va_dmd_desc *desc);

/*
 * t2va_dmd_target - the joint DMD term (deep read, section 4):
 *   z_t^m   = cos t x0^m + sin t eps^m        (x0 = the student's paired sample)
 *   x0_T^m  = u^m + s_m (c^m - u^m)           guided teacher prediction: c = G_T(z_t, t, text),
 *                                             u = G_T(z_t, t, no text) (every text key masked),
 *                                             s_v = cfg_v, s_a = cfg_a
 *   x0_F^m  = G_F(z_t, t, text)               the fake-score block
 *   g^m     = x0_F^m - x0_T^m
 *   c^m     = (1/(Nm*Cm)) sum_i |x0_i^m - x0_T,i^m|          residual scale
 *   gbar^m  = g^m/(c^m + eps_dmd),  Delta^m = x0^m - sg(x0^m - gbar^m) = gbar^m (value)
 *   loss_b  = w_v sum_i (Delta_i^v)^2 + w_a sum_i (Delta_i^a)^2   (summed, not averaged)
 * With desc->param == T2VA_PARAM_RF all three passes go through the TrigFlow
 * wrapper and are converted to x0 before the guidance and the differences.
 * The unconditional pass shares the conditional pass's Q, K and V (in this
 * one-block model the video and audio rows do not depend on the text); only
 * its attention runs again over the video and audio keys.
 *
 * Inputs (device):
 *   x0_v, eps_v [B, Nv, Cv] in_dtype     x0_a, eps_a [B, Na, Ca] in_dtype
 *   text        [B, Nt, d]  in_dtype     text_mask   uint8 [B, Nt], nonzero = valid
 *   t_host      host double [B], each finite with 0 < t < pi/2
 *   teacher, fake: block weights as for t2va_scm_target
 * Outputs (device, fp32):
 *   delta_v [B, Nv, Cv], delta_a [B, Na, Ca]    required (Delta = gbar in value)
 *   scales  [B, 2]  (c^v, c^a)                   nullable
 *   loss    [B]                                  required
 * workspace: at least t2va_dmd_workspace_bytes(desc) bytes, 256-byte aligned.
 * Errors: as t2va_scm_target, plus T2VA_INVALID_ARG for non-finite guidance
 * scales or eps_dmd <= 0.
 */
t2va_status t2va_dmd_target(const t2va_dmd_desc *desc, const t2va_block_weights *teacher,
                            const t2va_block_weights *fake, const void *x0_v, const void *x0_a,
                            const void *eps_v, const void *eps_a, const void *text,
                            const uint8_t *text_mask, const double *t_host, float *delta_v,
                            float *delta_a, float *scales, float *loss, void *workspace,
                            size_t workspace_bytes, t2va_stream stream);

/*
 * t2va_stage3_mix - out[b] = lam_scm * loss_scm[b] + lam_dmd * loss_dmd[b]
 * (deep read, section 4.1), fp32 device arrays of B elements (in place on
 * either input is allowed).  B in 1..T2VA_MAX_BATCH, lam finite.
 */
t2va_status t2va_stage3_mix(int B, double lam_scm, double lam_dmd, const float *loss_scm,
                            const float *loss_dmd, float *out, t2va_stream stream);

/* ------------------------------------------------------------------------ */
/* Phase timing (instrumentation for benchmarks)                             */
/* ------------------------------------------------------------------------ */
#define T2VA_PHASE_TOTAL 0        /* whole t2va_scm_target / _dmd_target call */
#define T2VA_PHASE_TEACHER_ATTN 1 /* forward-only attention (teacher, fake)   */
#define T2VA_PHASE_STUDENT_ATTN 2 /* student attention forward + JVP       */
#define T2VA_PHASE_GEMM 3         /* all projection GEMMs                  */
#define T2VA_PHASE_OTHER 4        /* embedding, compaction, elementwise    */
#define T2VA_PHASE_BWD_ATTN 5     /* attention backward (t2va_scm_grad)    */
#define T2VA_NUM_PHASES 6

/*
 * t2va_profile_enable - with max_calls > 0, the next up to max_calls calls of
 * t2va_scm_target or t2va_dmd_target record HIP events around each phase on their stream (the
 * events are created here, outside the timed calls); with 0, recording stops
 * and the events are destroyed.  Not thread-safe: enable, run, read from one
 * thread.
 */
t2va_status t2va_profile_enable(int max_calls);

/*
 * t2va_profile_set_phases - which phases the calls record: bit p of
 * phase_mask for phase T2VA_PHASE_p (all phases until this is called).  A
 * phase left out issues no events, so a timed loop carries only the events
 * it reads.  T2VA_PHASE_OTHER (total minus the timed parts) is reported only
 * when the total and every part are recorded, else 0.  Returns
 * T2VA_INVALID_ARG while recorded events are unread.
 */
t2va_status t2va_profile_set_phases(unsigned phase_mask);

/*
 * t2va_profile_read - waits for the recorded events, writes per-phase sums of
 * milliseconds over the recorded calls into ms_out[T2VA_NUM_PHASES], the
 * number of recorded calls into *n_calls, and starts a new recording window.
 */
t2va_status t2va_profile_read(double *ms_out, int *n_calls);

#ifdef __cplusplus
}
#endif

#endif /* T2VA_H */
