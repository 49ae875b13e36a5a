/* hol_ops.h - the kernels of the weight-free decoder-layer template, one entry point each.
 *
 * MegaTrain summary page, 核心方法: the GPU keeps a pool of stateless layer templates, each
 * wrapping the kernels of the Attention and MLP blocks and holding no weight pointers; streamed
 * weights are bound to it per layer. These entry points expose those kernels individually (the
 * same launchers hol_forward_backward uses) so each can be checked in isolation.
 *
 * Every data pointer is a DEVICE pointer owned by the caller. `stream` is a hipStream_t (NULL for
 * the default stream). Calls are asynchronous on that stream and return HOL_OK when the launch
 * was accepted, HOL_EINVAL for unsupported shapes/alignments, HOL_EDEVICE for launch failures.
 * Layouts are row-major; dtype 0 = fp32, 1 = bf16 (hol_dtype).
 */
#ifndef HOL_OPS_H
#define HOL_OPS_H

#include <stdint.h>

#include "hol.h"

#ifdef __cplusplus
extern "C" {
#endif

/* C[M,N] op= alpha * sum_k A(m,k) B(k,n), fp32 accumulation.
 *   A(m,k) = a_km ? A[k*lda+m] : A[m*lda+k];   B(k,n) = b_kn ? B[k*ldb+n] : B[n*ldb+k]
 * epi 0: C = alpha*AB (C fp32 or bf16); 1: C += alpha*AB (C fp32); 2: C = R + alpha*AB (C, R fp32).
 * bf16 operands need K, lda, ldb multiples of 8 and 16-byte aligned A, B. */
hol_status hol_op_gemm(int32_t M, int32_t N, int32_t K, const void* A, int64_t lda, int32_t a_km,
                       const void* B, int64_t ldb, int32_t b_kn, void* C, int64_t ldc,
                       const float* R, int64_t ldr, hol_dtype ab, hol_dtype c, int32_t epi,
                       float alpha, void* stream);

/* hol_op_gemm with an fp32 device workspace of workspace_floats floats (at most
 * hol_op_gemm_workspace_floats() are used; 0 / NULL: exactly hol_op_gemm). With it, a bf16
 * product in the NT layout, or with both operands K-major (a_km = b_kn = 1: the weight-gradient
 * layout), with an fp32 store (EPI_STORE) whose 256 x 256 tiles leave the last round of the
 * persistent grid at most half full (every XCD with R >= 1 full rounds and r <= half a round of
 * tiles left) cuts those r tiles along K into 2 or 4 parts, runs the parts in the last round and
 * adds them in part order in a second kernel: the weight-gradient products dW = dY^T X of the
 * q/k/v and down projections at the LLaMA-8B shape (MegaTrain summary page, 核心方法: the
 * per-layer backward). The result is deterministic and within fp32 accumulation error of the
 * unsplit product, not bit for bit equal to it. The caller owns the workspace; calls that share
 * one must not overlap. */
int64_t hol_op_gemm_workspace_floats(void);
hol_status hol_op_gemm_ws(int32_t M, int32_t N, int32_t K, const void* A, int64_t lda, int32_t a_km,
                          const void* B, int64_t ldb, int32_t b_kn, void* C, int64_t ldc,
                          const float* R, int64_t ldr, hol_dtype ab, hol_dtype c, int32_t epi,
                          float alpha, float* workspace, int64_t workspace_floats, void* stream);

/* q/k/v projection with RoPE in the product's epilogue (MegaTrain summary page, 核心方法: the
 * attention block of the layer template): C [M, N] (bf16, row stride ldc) = A B^T with A [M, K]
 * and B [N, K] bf16 (NT, row strides lda, ldb), where the columns form heads of 128 and the first
 * n_rot columns (the q and k heads) are rotated by RoPE at position row mod S with fp32 tables
 * cos_t / sin_t [S, 64] as for hol_op_rope; every value is rounded to bf16 once. Bit for bit the
 * fp32 product of hol_op_gemm followed by hol_op_rope_qkv. K % 64 == 0, N % 128 == 0,
 * n_rot % 128 == 0, n_rot <= N, lda and ldb multiples of 8 with 16-byte aligned A, B and tables,
 * ldc % 4 == 0 and 8-byte aligned C, S > 0; else HOL_EINVAL. */
hol_status hol_op_gemm_rope(int32_t M, int32_t N, int32_t K, const void* A, int64_t lda, const void* B,
                            int64_t ldb, void* C, int64_t ldc, int32_t n_rot, int32_t S,
                            const float* cos_t, const float* sin_t, void* stream);

/* Gate/up projection with the SwiGLU activation (MegaTrain summary page, 核心方法: the MLP block
 * of the layer template, here with the activation fused into the product's epilogue):
 * gu [M, N] = A B^T with A [M, K] (row stride lda) and B = [W_gate; W_up] [N, K] (ldb), so gate
 * in columns [0, N/2) and up in [N/2, N) of gu (row stride ldgu), and a [M, N/2] (row stride ld_a)
 * = silu(gate) * up of the values as stored in gu. Every array is of dtype t. The result is bit
 * for bit that of hol_op_gemm (EPI_STORE, alpha 1) followed by hol_op_swiglu_fwd. One kernel when
 * t is bf16, K % 64 == 0, (N/2) % 32 == 0, lda and ldb multiples of 8 with 16-byte aligned A, B,
 * ldgu and ld_a multiples of 4 with 8-byte aligned gu, a; otherwise the two kernels, which need
 * ldgu == N and ld_a == N/2 (else HOL_EINVAL). Odd N: HOL_EINVAL. */
hol_status hol_op_gemm_swiglu(int32_t M, int32_t N, int32_t K, const void* A, int64_t lda, const void* B,
                              int64_t ldb, void* gu, int64_t ldgu, void* a, int64_t ld_a, hol_dtype t,
                              void* stream);

/* RMSNorm: y = x * rstd * gamma, rstd = 1/sqrt(mean(x^2) + eps); x fp32 [T,H], y [T,H] of
 * dtype yt, rstd fp32 [T]. H % 4 == 0. */
hol_status hol_op_rmsnorm_fwd(const float* x, const float* gamma, float eps, void* y, hol_dtype yt,
                              float* rstd, int32_t T, int32_t H, void* stream);
/* Backward: dx (fp32 [T,H]) = dx_in_place_if(accumulate) + d RMSNorm; dgamma (fp32 [H]) +=.
 * H must be a multiple of 4 and at most 4096, else HOL_EINVAL.
 * workspace: fp32 buffer of hol_op_rmsnorm_bwd_workspace(T, H) floats. */
int64_t hol_op_rmsnorm_bwd_workspace(int32_t T, int32_t H);
hol_status hol_op_rmsnorm_bwd(const float* dy, const float* x, const float* gamma, const float* rstd,
                              float* dx, int32_t accumulate, float* dgamma, float* workspace,
                              int32_t T, int32_t H, void* stream);

/* RoPE in place on `heads` heads of width d (row stride ld elements), position = t % S, with
 * fp32 tables cos/sin [S, d/2]. inverse != 0 rotates by the negative angle (the backward). */
hol_status hol_op_rope(void* x, hol_dtype t, int64_t ld, int32_t T, int32_t heads, int32_t d,
                       int32_t S, const float* cos_t, const float* sin_t, int32_t inverse,
                       void* stream);

/* RoPE of the fused q | k | v projection output (the bf16 forward, MegaTrain summary page, the
 * Attention block of the layer template): in is fp32 [T, (nq + 2 nkv) d] at row stride ldi;
 * out (bf16, row stride ldo) receives q and k rotated at position t % S and v unchanged, each
 * value rounded to bf16 once. d even; tables as for hol_op_rope. */
hol_status hol_op_rope_qkv(const float* in, int64_t ldi, void* out, int64_t ldo, int32_t T, int32_t nq,
                           int32_t nkv, int32_t d, int32_t S, const float* cos_t, const float* sin_t,
                           void* stream);

/* SwiGLU: gu = [g | u] ([T, 2F]); a = silu(g) u ([T, F]). Backward: dgu = [dg | du]. */
hol_status hol_op_swiglu_fwd(const void* gu, void* a, hol_dtype t, int32_t T, int32_t F, void* stream);
hol_status hol_op_swiglu_bwd(const void* da, const void* gu, void* dgu, hol_dtype t, int32_t T,
                             int32_t F, void* stream);
/* bf16 SwiGLU backward that also writes its result transposed: dgu [T, 2F] exactly as
 * hol_op_swiglu_bwd writes it, and dgut [2F, T] (row stride ldt >= T) for the weight-gradient
 * product dW_gate|up = dgu^T n2. F % 64 == 0, T % 8 == 0, ldt % 8 == 0 and 16-byte aligned
 * pointers, else HOL_EINVAL. */
hol_status hol_op_swiglu_bwd_t(const void* da, const void* gu, void* dgu, void* dgut, int64_t ldt,
                               int32_t T, int32_t F, void* stream);

/* bf16 transpose out[c][r] = in[r][c] of an R x C matrix at row strides ldi, ldo (elements,
 * multiples of 8; 16-byte aligned pointers, else HOL_EINVAL). The backward uses it to present
 * every product to the GEMM as A row-major by K and B row-major by K. */
hol_status hol_op_transpose_bf16(const void* in, int64_t ldi, void* out, int64_t ldo, int32_t R,
                                 int32_t C, void* stream);

/* Causal GQA attention over n_seq sequences of length S (token-major rows, T = n_seq*S).
 * q [T, nq*d] at row stride ldq, k/v [T, nkv*d] at ldk/ldv, o [T, nq*d] at ldo, lse fp32
 * [n_seq, nq, S]. Scale 1/sqrt(d). */
hol_status hol_op_attention_fwd(int32_t n_seq, int32_t S, int32_t nq, int32_t nkv, int32_t d,
                                hol_dtype t, const void* q, int64_t ldq, const void* k, int64_t ldk,
                                const void* v, int64_t ldv, void* o, int64_t ldo, float* lse,
                                void* stream);
/* Backward: dq/dk/dv written (not accumulated). delta: fp32 scratch [n_seq, nq, S]. */
hol_status hol_op_attention_bwd(int32_t n_seq, int32_t S, int32_t nq, int32_t nkv, int32_t d,
                                hol_dtype t, const void* q, int64_t ldq, const void* k, int64_t ldk,
                                const void* v, int64_t ldv, const void* o, int64_t ldo,
                                const float* lse, const void* dO, int64_t lddo, void* dq,
                                int64_t lddq, void* dk, int64_t lddk, void* dv, int64_t lddv,
                                float* delta, void* stream);

/* The backward followed by the RoPE backward of dq and dk (MegaTrain summary page, 核心方法: the
 * attention block of the layer template; q and k entered attention rotated by RoPE at position
 * t mod S): dq and dk are rotated back by the negative angle, with fp32 tables cos_t / sin_t
 * [S, d/2] as for hol_op_rope. Head width 128 (bf16) applies the rotation in the kernels' own
 * epilogues before the single rounding of dq and dk; other shapes run hol_op_rope(inverse) after
 * the backward. NULL tables or odd d: HOL_EINVAL. Other arguments as hol_op_attention_bwd. */
hol_status hol_op_attention_bwd_rope(int32_t n_seq, int32_t S, int32_t nq, int32_t nkv, int32_t d,
                                     hol_dtype t, const void* q, int64_t ldq, const void* k,
                                     int64_t ldk, const void* v, int64_t ldv, const void* o,
                                     int64_t ldo, const float* lse, const void* dO, int64_t lddo,
                                     void* dq, int64_t lddq, void* dk, int64_t lddk, void* dv,
                                     int64_t lddv, float* delta, const float* cos_t,
                                     const float* sin_t, void* stream);

/* hol_op_attention_bwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels and results,
 * with no delta argument. The row sums live in a static device array of the library, 16 MiB on
 * each GPU it runs on (4,194,304 floats, held until the process ends); its address is looked up
 * once per device on the first call with that device current. `stream` must belong to the current
 * device. Nothing is allocated or freed. n_seq * nq * S above 4,194,304 returns HOL_EINVAL with
 * the limit in hol_last_error() and launches nothing. Every call on one GPU shares that array and
 * leaves its last row sums there (each call writes every row sum it reads, so nothing needs
 * clearing); calls that overlap on one GPU (different streams or threads) race on it and must be
 * serialised by the caller. */
hol_status hol_op_attention_bwd_noalloc(int32_t n_seq, int32_t S, int32_t nq, int32_t nkv, int32_t d,
                                        hol_dtype t, const void* q, int64_t ldq, const void* k,
                                        int64_t ldk, const void* v, int64_t ldv, const void* o,
                                        int64_t ldo, const float* lse, const void* dO, int64_t lddo,
                                        void* dq, int64_t lddq, void* dk, int64_t lddk, void* dv,
                                        int64_t lddv, void* stream);

/* Cross entropy rows (loss anchor): logits fp32 [Tc, V] (row stride ld); labels int32 [Tc]
 * (-1 ignored); w fp32 [Tc] per-row weight. row_loss[t] = w[t] (logsumexp - z[label]);
 * dlogits [Tc, V] (dtype dt, row stride ldd) = w[t] (softmax - onehot). */
hol_status hol_op_cross_entropy(const float* logits, int64_t ld, const int32_t* labels, const float* w,
                                float* row_loss, void* dlogits, hol_dtype dt, int64_t ldd, int32_t Tc,
                                int32_t V, void* stream);

/* Blocks until all work on `stream` is done; HOL_EDEVICE with the HIP error text on failure. */
hol_status hol_op_sync(void* stream);

#ifdef __cplusplus
}
#endif
#endif /* HOL_OPS_H */
