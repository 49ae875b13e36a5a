// C ABI of libhol.so (include/hol.h, include/hol_ops.h): argument checking, exception firewall and
// dispatch into the streaming engine and the kernel launchers. No exception crosses the ABI.
#include <immintrin.h>
#include <string.h>

#include <new>
#include <string>

#include "../../include/hol.h"
#include "../../include/hol_ops.h"
#include "engine.h"
#include "host_math.h"
#include "kernels.h"

namespace hol {
const char* last_error_cstr();
}

using namespace hol;

#define GUARD_BEGIN try {
#define GUARD_END                                   \
  }                                                 \
  catch (const std::bad_alloc&) {                   \
    set_error("host allocation failed");            \
    return HOL_ENOMEM_HOST;                         \
  }                                                 \
  catch (const std::exception& e) {                 \
    set_error(std::string("internal error: ") + e.what()); \
    return HOL_EINVAL;                              \
  }

static hol_status einval(const char* fn, const char* why) {
  set_error(std::string(fn) + ": " + why);
  return HOL_EINVAL;
}

static const TensorDesc* tensor_at(const hol_model* m, int32_t i) {
  if (!m || i < 0 || i >= (int32_t)m->tensors.size()) return nullptr;
  return &m->tensors[(size_t)i];
}

extern "C" {

hol_status hol_create(const hol_config* cfg, hol_model** out) {
  GUARD_BEGIN
  if (out) *out = nullptr;
  return engine_create(cfg, out);
  GUARD_END
}

void hol_destroy(hol_model* m) {
  try {
    engine_destroy(m);
  } catch (...) {
  }
}

hol_status hol_num_tensors(const hol_model* m, int32_t* n) {
  if (!m || !n) return einval("hol_num_tensors", "null argument");
  *n = (int32_t)m->tensors.size();
  return HOL_OK;
}

hol_status hol_tensor_info(const hol_model* m, int32_t i, char* name, size_t cap, int64_t shape[4], int32_t* ndim,
                           int32_t* trainable) {
  const TensorDesc* t = tensor_at(m, i);
  if (!t) return einval("hol_tensor_info", "bad model or index");
  if (name && cap) {
    strncpy(name, t->name.c_str(), cap - 1);
    name[cap - 1] = 0;
  }
  if (shape)
    for (int k = 0; k < 4; ++k) shape[k] = k < t->ndim ? t->shape[k] : 0;
  if (ndim) *ndim = t->ndim;
  if (trainable) *trainable = t->trainable ? 1 : 0;
  return HOL_OK;
}

hol_status hol_set_tensor(hol_model* m, int32_t i, const float* src, int64_t numel) {
  GUARD_BEGIN
  const TensorDesc* t = tensor_at(m, i);
  if (!t || !src) return einval("hol_set_tensor", "bad model, index or pointer");
  if (numel != t->numel) return einval("hol_set_tensor", "numel mismatch");
  if (t->flat < 0) {  // frozen tensor without an fp32 copy: straight into the image
    write_image_tensor(m, *t, src);
    return HOL_OK;
  }
  float* dst = m->master + t->flat;
  parallel_for(numel, 1 << 18, [&](int64_t lo, int64_t hi) { memcpy(dst + lo, src + lo, (size_t)(hi - lo) * 4); });
  refresh_image_tensor(m, *t);
  return HOL_OK;
  GUARD_END
}

hol_status hol_get_tensor(const hol_model* m, int32_t i, float* dst, int64_t numel) {
  GUARD_BEGIN
  const TensorDesc* t = tensor_at(m, i);
  if (!t || !dst) return einval("hol_get_tensor", "bad model, index or pointer");
  if (numel != t->numel) return einval("hol_get_tensor", "numel mismatch");
  if (t->flat < 0) {
    read_image_tensor(m, *t, dst);
    return HOL_OK;
  }
  const float* src = m->master + t->flat;
  parallel_for(numel, 1 << 18, [&](int64_t lo, int64_t hi) { memcpy(dst + lo, src + lo, (size_t)(hi - lo) * 4); });
  return HOL_OK;
  GUARD_END
}

hol_status hol_get_grad(const hol_model* m, int32_t i, float* dst, int64_t numel) {
  GUARD_BEGIN
  const TensorDesc* t = tensor_at(m, i);
  if (!t || !dst) return einval("hol_get_grad", "bad model, index or pointer");
  if (numel != t->numel) return einval("hol_get_grad", "numel mismatch");
  if (!t->trainable) return einval("hol_get_grad", "tensor is frozen");
  if (m->grads_stale && t->flat >= m->layer_flat0) {  // consumed by a fused step: logically zero
    parallel_for(numel, 1 << 18, [&](int64_t lo, int64_t hi) { memset(dst + lo, 0, (size_t)(hi - lo) * 4); });
    return HOL_OK;
  }
  const float* src = m->grad + t->flat;
  parallel_for(numel, 1 << 18, [&](int64_t lo, int64_t hi) { memcpy(dst + lo, src + lo, (size_t)(hi - lo) * 4); });
  return HOL_OK;
  GUARD_END
}

hol_status hol_get_adam_state(const hol_model* m, int32_t i, float* mom1, float* mom2, int64_t numel, int64_t* step) {
  const TensorDesc* t = tensor_at(m, i);
  if (!t) return einval("hol_get_adam_state", "bad model or index");
  if (numel != t->numel) return einval("hol_get_adam_state", "numel mismatch");
  if (!t->trainable) return einval("hol_get_adam_state", "tensor is frozen");
  if (mom1) memcpy(mom1, m->mom1 + t->flat, (size_t)numel * 4);
  if (mom2) memcpy(mom2, m->mom2 + t->flat, (size_t)numel * 4);
  if (step) *step = m->step_t;
  return HOL_OK;
}

hol_status hol_set_adam_state(hol_model* m, int32_t i, const float* mom1, const float* mom2, int64_t numel,
                              int64_t step) {
  const TensorDesc* t = tensor_at(m, i);
  if (!t) return einval("hol_set_adam_state", "bad model or index");
  if (numel != t->numel || step < 0) return einval("hol_set_adam_state", "numel or step invalid");
  if (!t->trainable) return einval("hol_set_adam_state", "tensor is frozen");
  if (mom1) memcpy(m->mom1 + t->flat, mom1, (size_t)numel * 4);
  if (mom2) memcpy(m->mom2 + t->flat, mom2, (size_t)numel * 4);
  m->step_t = step;
  return HOL_OK;
}

hol_status hol_get_routing(const hol_model* m, int32_t layer, int32_t* ids, int64_t n) {
  GUARD_BEGIN
  if (!m || !ids) return einval("hol_get_routing", "null argument");
  return engine_get_routing(m, layer, ids, n);
  GUARD_END
}

hol_status hol_set_ckpt_every_k(hol_model* m, int32_t k) {
  if (!m) return einval("hol_set_ckpt_every_k", "null model");
  return engine_set_k(m, k);
}

hol_status hol_set_kernel_timing(hol_model* m, int32_t on) {
  GUARD_BEGIN
  if (!m) return einval("hol_set_kernel_timing", "null model");
  return engine_set_kernel_timing(m, on != 0);
  GUARD_END
}

hol_status hol_zero_grad(hol_model* m) {
  GUARD_BEGIN
  if (!m) return einval("hol_zero_grad", "null model");
  return engine_zero_grad(m);
  GUARD_END
}

hol_status hol_forward_backward(hol_model* m, const hol_batch* batch, hol_loss loss, double* loss_sum_out) {
  GUARD_BEGIN
  if (!m) return einval("hol_forward_backward", "null model");
  return engine_forward_backward(m, batch, loss, loss_sum_out);
  GUARD_END
}

hol_status hol_forward_backward_step(hol_model* m, const hol_batch* batch, hol_loss loss, double* loss_sum_out) {
  GUARD_BEGIN
  if (!m) return einval("hol_forward_backward_step", "null model");
  return engine_forward_backward(m, batch, loss, loss_sum_out, FB_FUSED);
  GUARD_END
}

hol_status hol_forward_backward_async(hol_model* m, const hol_batch* batch, hol_loss loss, double* loss_sum_out) {
  GUARD_BEGIN
  if (!m) return einval("hol_forward_backward_async", "null model");
  return engine_forward_backward(m, batch, loss, loss_sum_out, FB_ASYNC);
  GUARD_END
}

hol_status hol_step(hol_model* m) {
  GUARD_BEGIN
  if (!m) return einval("hol_step", "null model");
  return engine_step(m);
  GUARD_END
}

hol_status hol_last_stats(const hol_model* m, char* json, size_t cap) {
  GUARD_BEGIN
  if (!m || !json || !cap) return einval("hol_last_stats", "null argument");
  const std::string s = stats_json(m);
  if (s.size() + 1 > cap)
    return einval("hol_last_stats", ("buffer too small: needs " + std::to_string(s.size() + 1) + " bytes").c_str());
  memcpy(json, s.c_str(), s.size() + 1);
  return HOL_OK;
  GUARD_END
}

hol_status hol_partition(const int64_t* t_f, const int64_t* t_b, const int64_t* m_f, const int64_t* m_b, int32_t L,
                         int64_t mem_cap, int32_t n_gpus, int32_t n_micro, int32_t* f_bounds, int32_t* n_f,
                         int32_t* b_bounds, int32_t* n_b, int64_t* t_max, int64_t* J_out) {
  GUARD_BEGIN
  if (!t_f || !t_b || !m_f || !m_b || !f_bounds || !n_f || !b_bounds || !n_b || !t_max)
    return einval("hol_partition", "null argument");
  if (L <= 0 || n_gpus <= 0 || n_micro <= 0 || mem_cap < 0) return einval("hol_partition", "bad sizes");
  for (int i = 0; i < L; ++i)
    if (t_f[i] < 0 || t_b[i] < 0 || m_f[i] < 0 || m_b[i] < 0) return einval("hol_partition", "negative cost");
  __int128 J = 0;
  int nf = 0, nb = 0;
  if (!partition_stages(t_f, t_b, m_f, m_b, L, mem_cap, n_gpus, n_micro, f_bounds, &nf, b_bounds, &nb, t_max, &J))
    return einval("hol_partition", "a layer exceeds the memory cap");
  *n_f = nf;
  *n_b = nb;
  if (J_out) *J_out = J > (__int128)INT64_MAX ? INT64_MAX : (int64_t)J;
  return HOL_OK;
  GUARD_END
}

hol_status hol_host_adam(float* theta, const float* grad, float* mom1, float* mom2, int64_t n, int64_t step_t,
                         float lr, float beta1, float beta2, float eps) {
  GUARD_BEGIN
  if (!theta || !grad || !mom1 || !mom2 || n < 0 || step_t < 1) return einval("hol_host_adam", "bad argument");
  const AdamConsts k = adam_consts(step_t, lr, beta1, beta2, eps);
  parallel_for(n, 1 << 16, [&](int64_t lo, int64_t hi) {
    adam_range(theta + lo, grad + lo, mom1 + lo, mom2 + lo, hi - lo, k);
  });
  return HOL_OK;
  GUARD_END
}

hol_status hol_host_bf16_round(const float* src, uint16_t* dst, int64_t n) {
  GUARD_BEGIN
  if (!src || !dst || n < 0) return einval("hol_host_bf16_round", "bad argument");
  parallel_for(n, 1 << 16, [&](int64_t lo, int64_t hi) {
    f32_to_bf16_range_stream(src + lo, dst + lo, hi - lo);
    _mm_sfence();
  });
  return HOL_OK;
  GUARD_END
}

const char* hol_last_error(void) { return last_error_cstr(); }
const char* hol_version(void) { return "hol 0.1 (gfx950)"; }

// ------------------------------------------------------------------------------------------
// op-level entry points
// ------------------------------------------------------------------------------------------
static hol_status launched(int e, const char* fn) {
  if (e == 0) return HOL_OK;
  set_error(std::string(fn) + ": " + hipGetErrorString((hipError_t)e));
  return e == (int)hipErrorInvalidValue ? HOL_EINVAL : HOL_EDEVICE;
}

hol_status hol_op_gemm(int32_t M, int32_t N, int32_t K, const void* A, int64_t lda, int32_t a_km, const void* B,
                       int64_t ldb, int32_t b_kn, void* C, int64_t ldc, const float* R, int64_t ldr, hol_dtype ab,
                       hol_dtype c, int32_t epi, float alpha, void* stream) {
  if (epi < 0 || epi > 2) return einval("hol_op_gemm", "bad epilogue");
  Gemm g;
  g.M = M; g.N = N; g.K = K;
  g.A = A; g.lda = lda; g.a_km = a_km != 0;
  g.B = B; g.ldb = ldb; g.b_kn = b_kn != 0;
  g.C = C; g.ldc = ldc; g.R = R; g.ldr = ldr;
  g.ab = ab == HOL_BF16 ? DT_BF16 : DT_F32;
  g.c = c == HOL_BF16 ? DT_BF16 : DT_F32;
  g.epi = epi; g.alpha = alpha;
  return launched(launch_gemm(g, (hipStream_t)stream), "hol_op_gemm");
}

int64_t hol_op_gemm_workspace_floats(void) { return GEMM_SPLIT_WS_FLOATS; }

hol_status hol_op_gemm_ws(int32_t M, int32_t N, int32_t K, const void* A, int64_t lda, int32_t a_km, const void* B,
                          int64_t ldb, int32_t b_kn, void* C, int64_t ldc, const float* R, int64_t ldr, hol_dtype ab,
                          hol_dtype c, int32_t epi, float alpha, float* workspace, int64_t workspace_floats,
                          void* stream) {
  if (epi < 0 || epi > 2) return einval("hol_op_gemm_ws", "bad epilogue");
  if (workspace_floats < 0 || (workspace_floats > 0 && !workspace)) return einval("hol_op_gemm_ws", "bad workspace");
  Gemm g;
  g.M = M; g.N = N; g.K = K;
  g.A = A; g.lda = lda; g.a_km = a_km != 0;
  g.B = B; g.ldb = ldb; g.b_kn = b_kn != 0;
  g.C = C; g.ldc = ldc; g.R = R; g.ldr = ldr;
  g.ab = ab == HOL_BF16 ? DT_BF16 : DT_F32;
  g.c = c == HOL_BF16 ? DT_BF16 : DT_F32;
  g.epi = epi; g.alpha = alpha;
  g.ws = workspace; g.ws_floats = workspace_floats;
  return launched(launch_gemm(g, (hipStream_t)stream), "hol_op_gemm_ws");
}

hol_status hol_op_gemm_rope(int32_t M, int32_t N, int32_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                            void* C, int64_t ldc, int32_t n_rot, int32_t S, const float* cos_t, const float* sin_t,
                            void* stream) {
  if (M < 0 || N < 0 || K < 0 || S <= 0) return einval("hol_op_gemm_rope", "bad size");
  Gemm g;
  g.M = M; g.N = N; g.K = K;
  g.A = A; g.lda = lda;
  g.B = B; g.ldb = ldb;
  g.C = C; g.ldc = ldc;
  g.ab = g.c = DT_BF16;
  if (M > 0 && N > 0 && !gemm_rope_supported(g, n_rot, cos_t, sin_t))
    return einval("hol_op_gemm_rope", "unsupported shape, stride or alignment");
  return launched(launch_gemm_rope(g, n_rot, S, cos_t, sin_t, (hipStream_t)stream), "hol_op_gemm_rope");
}

hol_status hol_op_gemm_swiglu(int32_t M, int32_t N, int32_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                              void* gu, int64_t ldgu, void* a, int64_t ld_a, hol_dtype t, void* stream) {
  if (M < 0 || N < 0 || K < 0) return einval("hol_op_gemm_swiglu", "negative size");
  if (N % 2) return einval("hol_op_gemm_swiglu", "N (gate and up columns) must be even");
  Gemm g;
  g.M = M; g.N = N; g.K = K;
  g.A = A; g.lda = lda;
  g.B = B; g.ldb = ldb;
  g.C = gu; g.ldc = ldgu;
  g.ab = g.c = t == HOL_BF16 ? DT_BF16 : DT_F32;
  return launched(launch_gemm_swiglu(g, a, ld_a, (hipStream_t)stream), "hol_op_gemm_swiglu");
}

hol_status hol_op_rmsnorm_fwd(const float* x, const float* gamma, float eps, void* y, hol_dtype yt, float* rstd,
                              int32_t T, int32_t H, void* stream) {
  return launched(launch_rmsnorm_fwd(x, gamma, eps, y, yt == HOL_BF16 ? DT_BF16 : DT_F32, rstd, T, H,
                                     (hipStream_t)stream), "hol_op_rmsnorm_fwd");
}

int64_t hol_op_rmsnorm_bwd_workspace(int32_t T, int32_t H) { return (int64_t)rmsnorm_bwd_blocks(T) * H; }

hol_status hol_op_rmsnorm_bwd(const float* dy, const float* x, const float* gamma, const float* rstd, float* dx,
                              int32_t accumulate, float* dgamma, float* workspace, int32_t T, int32_t H, void* stream) {
  return launched(launch_rmsnorm_bwd(dy, x, gamma, rstd, dx, accumulate != 0, dgamma, workspace, T, H,
                                     (hipStream_t)stream), "hol_op_rmsnorm_bwd");
}

hol_status hol_op_rope(void* x, hol_dtype t, int64_t ld, int32_t T, int32_t heads, int32_t d, int32_t S,
                       const float* cos_t, const float* sin_t, int32_t inverse, void* stream) {
  if (d % 2) return einval("hol_op_rope", "odd head width");
  return launched(launch_rope(x, t == HOL_BF16 ? DT_BF16 : DT_F32, ld, T, heads, d, S, cos_t, sin_t, inverse != 0,
                              (hipStream_t)stream), "hol_op_rope");
}

hol_status hol_op_rope_qkv(const float* in, int64_t ldi, void* out, int64_t ldo, int32_t T, int32_t nq,
                           int32_t nkv, int32_t d, int32_t S, const float* cos_t, const float* sin_t,
                           void* stream) {
  if (d % 2 || d <= 0 || nq < 0 || nkv < 0 || S <= 0) return einval("hol_op_rope_qkv", "bad head shape");
  if (ldi < (int64_t)(nq + 2 * nkv) * d || ldo < (int64_t)(nq + 2 * nkv) * d)
    return einval("hol_op_rope_qkv", "row stride below the projection width");
  return launched(launch_rope_qkv(in, ldi, out, ldo, T, nq, nkv, d, S, cos_t, sin_t, (hipStream_t)stream),
                  "hol_op_rope_qkv");
}

hol_status hol_op_swiglu_fwd(const void* gu, void* a, hol_dtype t, int32_t T, int32_t F, void* stream) {
  return launched(launch_swiglu_fwd(gu, a, t == HOL_BF16 ? DT_BF16 : DT_F32, T, F, (hipStream_t)stream),
                  "hol_op_swiglu_fwd");
}

hol_status hol_op_swiglu_bwd(const void* da, const void* gu, void* dgu, hol_dtype t, int32_t T, int32_t F,
                             void* stream) {
  return launched(launch_swiglu_bwd(da, gu, dgu, t == HOL_BF16 ? DT_BF16 : DT_F32, T, F, (hipStream_t)stream),
                  "hol_op_swiglu_bwd");
}

hol_status hol_op_swiglu_bwd_t(const void* da, const void* gu, void* dgu, void* dgut, int64_t ldt, int32_t T,
                               int32_t F, void* stream) {
  if (T < 0 || F < 0) return einval("hol_op_swiglu_bwd_t", "negative size");
  return launched(launch_swiglu_bwd_tr(da, gu, dgu, dgut, ldt, T, F, (hipStream_t)stream), "hol_op_swiglu_bwd_t");
}

hol_status hol_op_transpose_bf16(const void* in, int64_t ldi, void* out, int64_t ldo, int32_t R, int32_t C,
                                 void* stream) {
  if (R < 0 || C < 0) return einval("hol_op_transpose_bf16", "negative size");
  return launched(launch_transpose_bf16(in, ldi, out, ldo, R, C, (hipStream_t)stream), "hol_op_transpose_bf16");
}

static Attn attn_args(int32_t n_seq, int32_t S, int32_t nq, int32_t nkv, int32_t d, hol_dtype t, const void* q,
                      int64_t ldq, const void* k, int64_t ldk, const void* v, int64_t ldv) {
  Attn a;
  a.n_seq = n_seq; a.S = S; a.nq = nq; a.nkv = nkv; a.d = d;
  a.t = t == HOL_BF16 ? DT_BF16 : DT_F32;
  a.q = q; a.ldq = ldq; a.k = k; a.ldk = ldk; a.v = v; a.ldv = ldv;
  return a;
}

hol_status hol_op_attention_fwd(int32_t n_seq, int32_t S, int32_t nq, int32_t nkv, int32_t d, hol_dtype t,
                                const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v, int64_t ldv,
                                void* o, int64_t ldo, float* lse, void* stream) {
  Attn a = attn_args(n_seq, S, nq, nkv, d, t, q, ldq, k, ldk, v, ldv);
  a.o = o; a.ldo = ldo; a.lse = lse;
  return launched(launch_attn_fwd(a, (hipStream_t)stream), "hol_op_attention_fwd");
}

hol_status hol_op_attention_bwd(int32_t n_seq, int32_t S, int32_t nq, int32_t nkv, int32_t d, hol_dtype t,
                                const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v, int64_t ldv,
                                const void* o, int64_t ldo, const float* lse, const void* dO, int64_t lddo, void* dq,
                                int64_t lddq, void* dk, int64_t lddk, void* dv, int64_t lddv, float* delta,
                                void* stream) {
  Attn a = attn_args(n_seq, S, nq, nkv, d, t, q, ldq, k, ldk, v, ldv);
  a.o = (void*)o; a.ldo = ldo; a.lse = (float*)lse;
  a.dO = dO; a.lddo = lddo;
  a.dq = dq; a.lddq = lddq; a.dk = dk; a.lddk = lddk; a.dv = dv; a.lddv = lddv;
  a.delta = delta;
  return launched(launch_attn_bwd(a, (hipStream_t)stream), "hol_op_attention_bwd");
}

hol_status hol_op_attention_bwd_rope(int32_t n_seq, int32_t S, int32_t nq, int32_t nkv, int32_t d, hol_dtype t,
                                     const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v,
                                     int64_t ldv, const void* o, int64_t ldo, const float* lse, const void* dO,
                                     int64_t lddo, void* dq, int64_t lddq, void* dk, int64_t lddk, void* dv,
                                     int64_t lddv, float* delta, const float* cos_t, const float* sin_t, void* stream) {
  if (!cos_t || !sin_t) return einval("hol_op_attention_bwd_rope", "null RoPE table");
  if (d % 2) return einval("hol_op_attention_bwd_rope", "odd head width");
  Attn a = attn_args(n_seq, S, nq, nkv, d, t, q, ldq, k, ldk, v, ldv);
  a.o = (void*)o; a.ldo = ldo; a.lse = (float*)lse;
  a.dO = dO; a.lddo = lddo;
  a.dq = dq; a.lddq = lddq; a.dk = dk; a.lddk = lddk; a.dv = dv; a.lddv = lddv;
  a.delta = delta;
  a.rope_cos = cos_t; a.rope_sin = sin_t;
  return launched(launch_attn_bwd(a, (hipStream_t)stream), "hol_op_attention_bwd_rope");
}

hol_status hol_op_attention_bwd_noalloc(int32_t n_seq, int32_t S, int32_t nq, int32_t nkv, int32_t d, hol_dtype t,
                                        const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v,
                                        int64_t ldv, const void* o, int64_t ldo, const float* lse, const void* dO,
                                        int64_t lddo, void* dq, int64_t lddq, void* dk, int64_t lddk, void* dv,
                                        int64_t lddv, void* stream) {
  if ((int64_t)n_seq * nq * S > ATTN_SCRATCH_FLOATS) {
    const std::string why = "n_seq * n_q_heads * S = " + std::to_string((int64_t)n_seq * nq * S) +
                            " exceeds the static scratch of " + std::to_string(ATTN_SCRATCH_FLOATS) + " row sums";
    return einval("hol_op_attention_bwd_noalloc", why.c_str());
  }
  Attn a = attn_args(n_seq, S, nq, nkv, d, t, q, ldq, k, ldk, v, ldv);
  a.o = (void*)o; a.ldo = ldo; a.lse = (float*)lse;
  a.dO = dO; a.lddo = lddo;
  a.dq = dq; a.lddq = lddq; a.dk = dk; a.lddk = lddk; a.dv = dv; a.lddv = lddv;
  return launched(launch_attn_bwd_noalloc(a, (hipStream_t)stream), "hol_op_attention_bwd_noalloc");
}

hol_status hol_op_cross_entropy(const float* logits, int64_t ld, const int32_t* labels, const float* w,
                                float* row_loss, void* dlogits, hol_dtype dt, int64_t ldd, int32_t Tc, int32_t V,
                                void* stream) {
  return launched(launch_ce_fwd_bwd(logits, ld, labels, w, row_loss, dlogits, dt == HOL_BF16 ? DT_BF16 : DT_F32,
                                    ldd, Tc, V, (hipStream_t)stream), "hol_op_cross_entropy");
}

hol_status hol_op_sync(void* stream) {
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) {
    set_error(std::string("hol_op_sync: ") + hipGetErrorString(e));
    return HOL_EDEVICE;
  }
  return HOL_OK;
}

}  // extern "C"
