// Host driver for the sanitizer build of the C ABI's validation paths: every
// entry point is called with arguments that must be rejected before anything
// reaches the GPU (and the workspace-size queries with valid and invalid
// descriptors), and each status and message is checked.  Built and run by
// tests/test_host_sanitizers.py with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code; it needs no GPU, since no call
// here gets past validation.
#include "t2va.h"

#include <math.h>
#include <stdio.h>
#include <string.h>

static int failures = 0;

#define EXPECT(cond, what)                                                         \
  do {                                                                             \
    if (!(cond)) {                                                                 \
      fprintf(stderr, "FAILED: %s (%s:%d) last_error='%s'\n", what, __FILE__, __LINE__, \
              t2va_last_error());                                                  \
      ++failures;                                                                  \
    }                                                                              \
  } while (0)

static void *fake(int i) { return (void *)(uintptr_t)(0x10000 * (uintptr_t)i); }

static t2va_scm_desc scm(int B, int Nv, int Na, int Nt, int d, int H) {
  t2va_scm_desc s;
  memset(&s, 0, sizeof(s));
  s.B = B; s.Nv = Nv; s.Na = Na; s.Nt = Nt; s.Cv = 128; s.Ca = 64; s.d = d; s.H = H;
  s.in_dtype = T2VA_DTYPE_BF16; s.weight_dtype = T2VA_DTYPE_BF16;
  s.beta = 1.0; s.gamma = 1.0; s.eps_scm = 1e-6; s.w_v = 1.0; s.w_a = 1.0;
  s.param = T2VA_PARAM_X0; s.precision = T2VA_PREC_BF16;
  return s;
}

int main() {
  EXPECT(t2va_abi_version() == T2VA_ABI_VERSION, "abi version");

  // ---- workspace sizes: every descriptor field's range ----
  t2va_scm_desc d = scm(1, 28672, 256, 256, 2048, 16);
  const size_t n_bf16 = t2va_scm_workspace_bytes(&d);
  EXPECT(n_bf16 > 0 && n_bf16 % 256 == 0, "high-res workspace");
  d.precision = T2VA_PREC_SPLIT;
  EXPECT(t2va_scm_workspace_bytes(&d) > n_bf16, "split workspace larger");
  EXPECT(t2va_scm_grad_workspace_bytes(&d) == 0 && strstr(t2va_last_error(), "precision"), "grad rejects split");
  d.precision = 7;
  EXPECT(t2va_scm_workspace_bytes(&d) == 0, "unknown precision");
  d = scm(1, 28672, 256, 256, 2048, 16);
  const struct { int B, Nv, Na, Nt, Cv, Ca, d, H; } bad[] = {
      {0, 8, 8, 0, 128, 64, 256, 2}, {65, 8, 8, 0, 128, 64, 256, 2}, {1, 0, 8, 0, 128, 64, 256, 2},
      {1, 8, 0, 0, 128, 64, 256, 2}, {1, 8, 8, -1, 128, 64, 256, 2}, {1, 8, 8, 0, 100, 64, 256, 2},
      {1, 8, 8, 0, 128, 32, 256, 2}, {1, 8, 8, 0, 128, 64, 256, 3}, {1, 8, 8, 0, 128, 64, 256, 8},
      {1, 8, 8, 0, 128, 64, 0, 2}, {1, 400000, 8, 0, 128, 64, 2048, 16}};
  for (const auto &b : bad) {
    t2va_scm_desc x = scm(b.B, b.Nv, b.Na, b.Nt, b.d, b.H);
    x.Cv = b.Cv; x.Ca = b.Ca;
    EXPECT(t2va_scm_workspace_bytes(&x) == 0 && t2va_last_error()[0] != 0, "invalid shape rejected");
  }
  t2va_scm_desc g = scm(1, 64, 16, 8, 256, 4);
  g.gamma = 1.5;
  EXPECT(t2va_scm_workspace_bytes(&g) == 0 && strstr(t2va_last_error(), "gamma"), "gamma range");
  g.gamma = 0.5; g.eps_scm = 0.0;
  EXPECT(t2va_scm_workspace_bytes(&g) == 0, "eps_scm > 0");
  g.eps_scm = NAN;
  EXPECT(t2va_scm_workspace_bytes(&g) == 0, "eps_scm finite");
  g.eps_scm = 1e-6; g.beta = INFINITY;
  EXPECT(t2va_scm_workspace_bytes(&g) == 0, "beta finite");
  g.beta = 1.0; g.param = 5;
  EXPECT(t2va_scm_workspace_bytes(&g) == 0, "param");
  g.param = T2VA_PARAM_RF; g.in_dtype = 9;
  EXPECT(t2va_scm_workspace_bytes(&g) == 0, "dtype");
  EXPECT(t2va_scm_workspace_bytes(nullptr) == 0, "NULL desc");

  // ---- t2va_scm_target: rejected before launch ----
  t2va_scm_desc tiny = scm(1, 64, 16, 8, 256, 4);
  const size_t ws = t2va_scm_workspace_bytes(&tiny);
  t2va_block_weights w;
  w.w_in_v = fake(1); w.w_in_a = fake(2); w.w_t = fake(3); w.w_qkv = fake(4); w.w_out_v = fake(5); w.w_out_a = fake(6);
  double t_ok[1] = {0.5}, t_zero[1] = {0.0}, t_half_pi[1] = {M_PI / 2}, t_nan[1] = {NAN};
  float *o[8];
  for (int i = 0; i < 8; ++i) o[i] = (float *)fake(20 + i);
  auto call = [&](const t2va_scm_desc *ds, const t2va_block_weights *tw, const double *t, void *wsp, size_t nb,
                  float *loss) {
    return t2va_scm_target(ds, tw, &w, fake(10), fake(11), fake(12), fake(13), fake(14), (const uint8_t *)fake(15), t,
                           o[0], o[1], o[2], o[3], o[4], o[5], o[6], loss, wsp, nb, nullptr);
  };
  EXPECT(call(&tiny, &w, t_zero, fake(100), ws, o[7]) == T2VA_INVALID_ARG, "t = 0");
  EXPECT(call(&tiny, &w, t_half_pi, fake(100), ws, o[7]) == T2VA_INVALID_ARG, "t = pi/2");
  EXPECT(call(&tiny, &w, t_nan, fake(100), ws, o[7]) == T2VA_INVALID_ARG, "t NaN");
  EXPECT(call(&tiny, &w, nullptr, fake(100), ws, o[7]) == T2VA_INVALID_ARG, "t NULL");
  EXPECT(call(&tiny, &w, t_ok, fake(100), ws - 1, o[7]) == T2VA_WORKSPACE_TOO_SMALL, "workspace size");
  EXPECT(call(&tiny, &w, t_ok, (void *)0x10010, ws, o[7]) == T2VA_INVALID_ARG, "workspace alignment");
  EXPECT(call(&tiny, &w, t_ok, nullptr, ws, o[7]) == T2VA_INVALID_ARG, "workspace NULL");
  EXPECT(call(&tiny, &w, t_ok, fake(100), ws, nullptr) == T2VA_INVALID_ARG, "loss required");
  EXPECT(call(nullptr, &w, t_ok, fake(100), ws, o[7]) == T2VA_INVALID_ARG, "desc NULL");
  t2va_block_weights w2 = w;
  w2.w_qkv = (void *)0x40008;
  EXPECT(call(&tiny, &w2, t_ok, fake(100), ws, o[7]) == T2VA_INVALID_ARG, "weight alignment");
  w2.w_qkv = nullptr;
  EXPECT(call(&tiny, &w2, t_ok, fake(100), ws, o[7]) == T2VA_INVALID_ARG, "weight NULL");
  EXPECT(call(&tiny, nullptr, t_ok, fake(100), ws, o[7]) == T2VA_INVALID_ARG, "weights NULL");

  // ---- the allocation-free variant: oversized shapes and bad arguments ----
  t2va_scm_desc big = scm(1, 6144, 256, 256, 2048, 16);
  EXPECT(t2va_scm_target_noalloc(&big, &w, &w, fake(10), fake(11), fake(12), fake(13), fake(14),
                                 (const uint8_t *)fake(15), t_ok, o[0], o[1], o[2], o[3], o[4], o[5], o[6], o[7],
                                 nullptr) == T2VA_WORKSPACE_TOO_SMALL,
         "noalloc oversized");
  EXPECT(t2va_scm_target_noalloc(&tiny, &w, &w, fake(10), fake(11), fake(12), fake(13), fake(14),
                                 (const uint8_t *)fake(15), t_zero, o[0], o[1], o[2], o[3], o[4], o[5], o[6], o[7],
                                 nullptr) == T2VA_INVALID_ARG,
         "noalloc t = 0");

  // ---- t2va_scm_grad ----
  t2va_block_grads gr;
  gr.w_in_v = o[0]; gr.w_in_a = o[1]; gr.w_t = o[2]; gr.w_qkv = o[3]; gr.w_out_v = o[4]; gr.w_out_a = nullptr;
  const size_t gws = t2va_scm_grad_workspace_bytes(&tiny);
  EXPECT(gws > ws, "grad workspace");
  EXPECT(t2va_scm_grad(&tiny, &w, &w, fake(10), fake(11), fake(12), fake(13), fake(14), (const uint8_t *)fake(15), t_ok,
                       o[2], o[3], o[6], o[7], &gr, fake(100), gws, nullptr) == T2VA_INVALID_ARG,
         "grad NULL gradient");
  EXPECT(t2va_scm_grad(&tiny, &w, &w, fake(10), fake(11), fake(12), fake(13), fake(14), (const uint8_t *)fake(15), t_ok,
                       o[2], o[3], o[6], o[7], nullptr, fake(100), gws, nullptr) == T2VA_INVALID_ARG,
         "grad NULL grads");

  // ---- attention entry points ----
  t2va_attn_desc a;
  memset(&a, 0, sizeof(a));
  a.B = 1; a.H = 2; a.dh = 128; a.Nq = 10; a.Nk = 20;
  a.q_batch_stride = a.k_batch_stride = 20 * 256;
  a.q_row_stride = a.k_row_stride = a.o_row_stride = 256;
  a.o_batch_stride = 10 * 256;
  a.vt_row_stride = 64; a.vt_head_stride = 64 * 128; a.vt_batch_stride = 2 * 64 * 128;
  a.out_dtype = T2VA_DTYPE_FP32;
  auto attn = [&](const t2va_attn_desc *ad, void *qd) {
    return t2va_joint_attn_fwd_jvp(ad, fake(1), fake(2), fake(3), qd, nullptr, nullptr, (const int32_t *)fake(7),
                                   fake(8), nullptr, nullptr, nullptr);
  };
  EXPECT(attn(&a, fake(4)) == T2VA_INVALID_ARG, "tangent without has_tangent");
  a.has_tangent = 1;
  EXPECT(attn(&a, nullptr) == T2VA_INVALID_ARG, "has_tangent without tangents");
  a.has_tangent = 0; a.dh = 96;
  EXPECT(attn(&a, nullptr) == T2VA_UNSUPPORTED_SHAPE, "dh");
  a.dh = 128; a.vt_row_stride = 24;
  EXPECT(attn(&a, nullptr) == T2VA_INVALID_ARG, "vt_row_stride");
  a.vt_row_stride = 64; a.q_row_stride = 250;
  EXPECT(attn(&a, nullptr) == T2VA_INVALID_ARG, "stride multiple of 8");
  a.q_row_stride = 256; a.scale = -1.f;
  EXPECT(attn(&a, nullptr) == T2VA_INVALID_ARG, "negative scale");
  a.scale = 0.f;
  EXPECT(attn(nullptr, nullptr) == T2VA_INVALID_ARG, "attention desc NULL");
  EXPECT(t2va_joint_attn_fwd_jvp_split(&a, fake(1), nullptr, fake(2), fake(5), fake(3), nullptr, nullptr, nullptr,
                                       (const int32_t *)fake(7), fake(8), nullptr, nullptr, nullptr) == T2VA_INVALID_ARG,
         "split needs q_lo");
  // one 128-key stage past the last key must fit 32-bit offsets
  t2va_attn_desc big_k = a;
  big_k.H = 1; big_k.k_row_stride = 3 * 2048; big_k.k_batch_stride = 0;
  big_k.Nk = (int)((2147483648LL / (big_k.k_row_stride * 2)) - 127);
  big_k.vt_row_stride = (big_k.Nk + 63) / 64 * 64;
  big_k.vt_head_stride = 128 * big_k.vt_row_stride; big_k.vt_batch_stride = big_k.vt_head_stride;
  EXPECT(attn(&big_k, nullptr) == T2VA_UNSUPPORTED_SHAPE, "32-bit key offsets");

  // ---- DMD term ----
  t2va_dmd_desc dd;
  memset(&dd, 0, sizeof(dd));
  dd.B = 1; dd.Nv = 64; dd.Na = 16; dd.Nt = 8; dd.Cv = 128; dd.Ca = 64; dd.d = 256; dd.H = 4;
  dd.cfg_v = 3.0; dd.cfg_a = 5.0; dd.eps_dmd = 1e-6; dd.w_v = dd.w_a = 1.0;
  const size_t dws = t2va_dmd_workspace_bytes(&dd);
  EXPECT(dws > 0, "dmd workspace");
  dd.cfg_a = NAN;
  EXPECT(t2va_dmd_workspace_bytes(&dd) == 0, "guidance finite");
  dd.cfg_a = 5.0; dd.eps_dmd = -1.0;
  EXPECT(t2va_dmd_workspace_bytes(&dd) == 0, "eps_dmd");
  dd.eps_dmd = 1e-6;
  EXPECT(t2va_dmd_target(&dd, &w, &w, fake(10), fake(11), fake(12), fake(13), fake(14), (const uint8_t *)fake(15),
                         t_ok, o[0], o[1], o[2], o[3], fake(100), dws - 256, nullptr) == T2VA_WORKSPACE_TOO_SMALL,
         "dmd workspace size");
  EXPECT(t2va_dmd_target(&dd, &w, nullptr, fake(10), fake(11), fake(12), fake(13), fake(14), (const uint8_t *)fake(15),
                         t_ok, o[0], o[1], o[2], o[3], fake(100), dws, nullptr) == T2VA_INVALID_ARG,
         "dmd fake weights NULL");

  // ---- elementwise and mix ----
  double t2[2] = {0.3, 2.0};
  EXPECT(t2va_trigflow_field(T2VA_NOISE, 2, 16, 0, 0, 1, t2, fake(1), fake(2), fake(3), nullptr) == T2VA_INVALID_ARG,
         "trigflow t range");
  t2[1] = 0.4;
  EXPECT(t2va_trigflow_field(5, 2, 16, 0, 0, 1, t2, fake(1), fake(2), fake(3), nullptr) == T2VA_INVALID_ARG, "mode");
  EXPECT(t2va_trigflow_field(T2VA_NOISE, 2, 0, 0, 0, 1, t2, nullptr, nullptr, nullptr, nullptr) == T2VA_OK,
         "zero elements");
  EXPECT(t2va_stage3_mix(0, 1.0, 1.0, (float *)fake(1), (float *)fake(2), (float *)fake(3), nullptr) ==
             T2VA_UNSUPPORTED_SHAPE,
         "mix B");
  EXPECT(t2va_stage3_mix(2, NAN, 1.0, (float *)fake(1), (float *)fake(2), (float *)fake(3), nullptr) == T2VA_INVALID_ARG,
         "mix lam");

  // ---- profiling controls (no events are created for 0 calls) ----
  EXPECT(t2va_profile_enable(-1) == T2VA_INVALID_ARG, "profile count");
  EXPECT(t2va_profile_enable(0) == T2VA_OK, "profile off");
  EXPECT(t2va_profile_read(nullptr, nullptr) == T2VA_INVALID_ARG, "profile read NULL");

  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("abi checks ok\n");
  return 0;
}
