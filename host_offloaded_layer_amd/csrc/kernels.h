// Host-callable launchers of the HIP kernels that make up the weight-free decoder-layer template
// (MegaTrain summary page, 核心方法: a stateless template pool of Attention and MLP kernels bound
// to whatever weights were streamed in). Every pointer is a device pointer; every launcher is
// asynchronous on `stream` and returns 0 or a hipError_t code.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace hol {

enum DType : int { DT_F32 = 0, DT_BF16 = 1 };

// GEMM epilogues
enum Epi : int {
  EPI_STORE = 0,   // C = alpha * A.B
  EPI_ACCUM = 1,   // C += alpha * A.B          (C fp32)
  EPI_RESID = 2,   // C = R + alpha * A.B       (C, R fp32; R may alias C)
};

// C[M,N] (op) sum_k A(m,k) B(k,n)
//   A(m,k) = a_km ? A[k*lda + m] : A[m*lda + k]
//   B(k,n) = b_kn ? B[k*ldb + n] : B[n*ldb + k]
// Forward y = x W^T: a_km = 0, b_kn = 0. dX = dY W: a_km = 0, b_kn = 1. dW += dY^T X: a_km = 1, b_kn = 1.
// `batch` > 1 repeats the product with element strides sA, sB, sC (and sR).
struct Gemm {
  int M = 0, N = 0, K = 0;
  const void* A = nullptr; int64_t lda = 0; bool a_km = false;
  const void* B = nullptr; int64_t ldb = 0; bool b_kn = false;
  void* C = nullptr; int64_t ldc = 0;
  const float* R = nullptr; int64_t ldr = 0;
  DType ab = DT_F32, c = DT_F32;
  int epi = EPI_STORE;
  float alpha = 1.f;
  int batch = 1; int64_t sA = 0, sB = 0, sC = 0, sR = 0;
  int bt = -1;             // dtype of B when it differs from ab (fp32 adapter factors); -1: ab
  bool any_align = false;  // bf16 operands that miss the MFMA alignment take the tiled kernel
  // grouped product (launch_gemm_grouped): `grp` is a device table from launch_gemm_group_table
  // over `ngroups` groups; group e owns rows [grp[e], grp[e+1]) of A, C and R and uses B + e * sB.
  // M bounds the total rows; grp_max_rt bounds the total 256-row tiles (sizes the grid).
  const int32_t* grp = nullptr;
  int ngroups = 0, grp_max_rt = 0;
  // second output of launch_gemm_swiglu (set by it)
  void* C2 = nullptr;
  int64_t ldc2 = 0;
  // optional fp32 workspace of ws_floats floats (GEMM_SPLIT_WS_FLOATS suffice): with it an fp32
  // store whose tiles leave the last round of the persistent grid part-empty splits those tiles
  // along K and adds the parts in a fixed order (results deterministic, not bitwise those of the
  // unsplit product). spl_full / spl_f are set by the launcher.
  float* ws = nullptr;
  int64_t ws_floats = 0;
  int spl_full = 0, spl_f = 1;
  // launch_gemm_rope: RoPE tables [rope_S][64] and the number of rotated columns (set by it)
  const float* rope_cos = nullptr;
  const float* rope_sin = nullptr;
  int rope_S = 0, rope_nr = 0;
};
constexpr int64_t GEMM_SPLIT_WS_FLOATS = (int64_t)256 * 256 * 256;  // 256 tile parts (64 MiB)
int launch_gemm(const Gemm& g, hipStream_t s);
// Gate/up product with the SwiGLU activation: g is the plain product gu [M, N] = x [gate; up]^T
// (EPI_STORE, no batch; gate in columns [0, N/2), up in [N/2, N)); also writes a [M, N/2] (row
// stride ld_a) = swiglu(gate, up) of the values as stored in gu. Bit for bit the result of
// launch_gemm(g) then launch_swiglu_fwd. One kernel (SwiGLU in the epilogue) when the operands
// are bf16 and NT with K % 64 == 0, N/2 % 32 == 0, 16-byte aligned A and B, ldc and ld_a
// multiples of 4 and 8-byte aligned outputs; otherwise the two launches, which need ldc = N and
// ld_a = N/2.
int launch_gemm_swiglu(const Gemm& g, void* a, int64_t ld_a, hipStream_t s);
// The q/k/v product with RoPE in its epilogue: g is the plain product C [M, N] = x Wqkv^T with a
// bf16 store (EPI_STORE, no batch), columns in heads of 128; the first nrot columns (the q and k
// heads) leave rotated at position row mod S (tables [S][64]), each value rounded to bf16 once:
// bit for bit launch_gemm into fp32 followed by launch_rope_qkv. Needs bf16 NT operands with
// K % 64 == 0, 16-byte aligned A and B with lda, ldb multiples of 8, N % 128 == 0, nrot % 128 == 0,
// ldc % 4 == 0, 8-byte aligned C and 16-byte aligned tables (gemm_rope_supported), else
// hipErrorInvalidValue.
bool gemm_rope_supported(const Gemm& g, int nrot, const float* cos_t, const float* sin_t);
int launch_gemm_rope(const Gemm& g, int nrot, int S, const float* cos_t, const float* sin_t, hipStream_t s);
// out[u][:] = sum over i in [seg[u], seg[u+1]) of dh[order[i]][:], in order of i from zero (fp32)
int launch_embed_row_sums(const float* dh, const int32_t* order, const int32_t* seg, int nrows, int H, float* out,
                          hipStream_t s);
// Row tile of the grouped product.
constexpr int GEMM_GROUP_BM = 256;
// Grouped bf16 NT product (K % 64 == 0, 16-byte aligned operands and leading dimensions).
int launch_gemm_grouped(const Gemm& g, hipStream_t s);
// tab[0..G]: exclusive prefix of counts (tab[G] = all rows); tab[G+1+e]: exclusive prefix of
// ceil(counts / GEMM_GROUP_BM) (tab[2G+1] = all row tiles). G <= 512.
int launch_gemm_group_table(const int32_t* counts, int G, int32_t* tab, hipStream_t s);

// RMSNorm forward: y = x * rstd * gamma, rstd = 1/sqrt(mean(x^2)+eps). x fp32 [T,H].
int launch_rmsnorm_fwd(const float* x, const float* gamma, float eps, void* y, DType yt,
                       float* rstd, int T, int H, hipStream_t s);
// RMSNorm backward. dx_out = (accumulate ? dx_out : 0) + dx; dgamma_acc += sum_t dy*x*rstd.
// `partial` is scratch of nb*H floats, nb = rmsnorm_bwd_blocks(T). dx_bf16 (optional, 8-byte
// aligned, [T,H]) also receives dx_out rounded to bf16 (what launch_cast_f32 would make of it).
int rmsnorm_bwd_blocks(int T);
int launch_rmsnorm_bwd(const float* dy, const float* x, const float* gamma, const float* rstd,
                       float* dx_out, bool accumulate, float* dgamma_acc, float* partial,
                       int T, int H, hipStream_t s, void* dx_bf16 = nullptr);

// RoPE (rotate-half) on `heads` heads of width d at row stride ld (elements); position = t % S.
// inverse = rotation by the negative angle (the backward).
int launch_rope(void* x, DType xt, int64_t ld, int T, int heads, int d, int S, const float* cos_t,
                const float* sin_t, bool inverse, hipStream_t s);

// RoPE of q and k fused with the fp32 -> bf16 cast of the whole q/k/v projection output (in fp32
// [T, (nq + 2 nkv) d], out bf16 with the same layout): one rounding per element.
int launch_rope_qkv(const float* in, int64_t ldi, void* out, int64_t ldo, int T, int nq, int nkv, int d, int S,
                    const float* cos_t, const float* sin_t, hipStream_t s);

// SwiGLU: gu holds [g | u] row-wise ([T, 2F], g first); a = silu(g) * u.
int launch_swiglu_fwd(const void* gu, void* a, DType t, int T, int F, hipStream_t s);
// dgu = [dg | du] from da.
int launch_swiglu_bwd(const void* da, const void* gu, void* dgu, DType t, int T, int F, hipStream_t s);
// bf16 SwiGLU backward writing dgu [T][2F] (as launch_swiglu_bwd) and its transpose dgut [2F][T]
// (row stride ldt); F % 64 == 0, T % 8 == 0, 16-byte aligned pointers, else hipErrorInvalidValue.
int launch_swiglu_bwd_tr(const void* da, const void* gu, void* dgu, void* dgut, int64_t ldt, int T, int F,
                         hipStream_t s);

// out[c][r] = in[r][c] for an R x C bf16 matrix (row strides ldi, ldo; multiples of 8, 16-byte
// aligned pointers).
int launch_transpose_bf16(const void* in, int64_t ldi, void* out, int64_t ldo, int R, int C, hipStream_t s);

// Elementwise helpers
int launch_cast_f32(const float* x, void* y, DType yt, int64_t n, hipStream_t s);
int launch_fill_f32(float* x, float v, int64_t n, hipStream_t s);
int launch_scale_f32(const float* x, float a, float* y, int64_t n, hipStream_t s);

// Causal GQA attention for `n_seq` sequences of length S. q/k/v/o are rows of a token-major
// activation ([T, *] with row strides ldq, ldk, ldv, ldo). lse fp32 [n_seq, nq, S].
struct Attn {
  int n_seq = 0, S = 0, nq = 0, nkv = 0, d = 0;
  DType t = DT_F32;
  const void* q = nullptr; const void* k = nullptr; const void* v = nullptr;
  int64_t ldq = 0, ldk = 0, ldv = 0;
  void* o = nullptr; int64_t ldo = 0;
  float* lse = nullptr;
  // backward
  const void* dO = nullptr; int64_t lddo = 0;
  void* dq = nullptr; void* dk = nullptr; void* dv = nullptr;
  int64_t lddq = 0, lddk = 0, lddv = 0;
  float* delta = nullptr;    // scratch fp32 [n_seq, nq, S]
  // backward, optional: RoPE tables (fp32 [S, d/2], position = token index within its sequence);
  // when set, dq and dk leave rotated back by the RoPE inverse (the RoPE backward applied)
  const float* rope_cos = nullptr;
  const float* rope_sin = nullptr;
};
int launch_attn_fwd(const Attn& a, hipStream_t s);
int launch_attn_bwd(const Attn& a, hipStream_t s);
// The same backward with the row sums delta in the library's static device scratch (a.delta is
// ignored): nothing is allocated. n_seq * nq * S must not exceed ATTN_SCRATCH_FLOATS.
constexpr int64_t ATTN_SCRATCH_FLOATS = (int64_t)4 << 20;
int launch_attn_bwd_noalloc(Attn a, hipStream_t s);

// Next-token cross entropy over one chunk of rows. logits fp32 [Tc, V]; labels int32 (-1 =
// ignore); w fp32 per-row weight (1/count of the row's micro-batch, 0 if ignored).
// row_loss[t] = w[t] * (lse - z[label]); dlogits = w[t] * (softmax - onehot) in type dt.
int launch_ce_fwd_bwd(const float* logits, int64_t ld, const int32_t* labels, const float* w,
                      float* row_loss, void* dlogits, DType dt, int64_t ldd, int Tc, int V,
                      hipStream_t s);
// Mixture-of-experts routing and permutation (k_moe.hip). logits / probs fp32 [T, E]; ids int32
// and w fp32 [T, k]; counts int32 [E]; offsets int32 [E + 1]; perm_slot and slot_pos
// int32 [T k]. E <= 512, k <= 16.
int launch_fill_i32(int32_t* x, int32_t v, int64_t n, hipStream_t s);
int launch_moe_route(const float* logits, int T, int E, int k, float* probs, int32_t* ids, float* w,
                     int32_t* counts, hipStream_t s);
// Stable permutation (rows of an expert in slot order); scratch holds moe_permute_scratch(T, E, k)
// int32.
int64_t moe_permute_scratch(int T, int E, int k);
int launch_moe_permute(const int32_t* ids, int T, int E, int k, const int32_t* counts, int32_t* offsets,
                       int32_t* scratch, int32_t* perm_slot, int32_t* slot_pos, hipStream_t s);
// Xp[p] = X[perm_slot[p] / k] for rows of H elements of type t
int launch_moe_gather(const void* X, DType t, const int32_t* perm_slot, int k, int64_t n_rows, int H, void* Xp,
                      hipStream_t s);
// hout[t] = h1[t] + sum_i w[t, i] Yp[slot_pos[t k + i]]   (fp32)
int launch_moe_combine(const float* h1, const float* Yp, const float* w, const int32_t* slot_pos, int T, int k, int H,
                       float* hout, hipStream_t s);
// dw[t, i] = <dh[t], Yp[p_i]>; dYp[p_i] = w[t, i] dh[t] (type t)
int launch_moe_combine_bwd(const float* dh, const float* Yp, const float* w, const int32_t* slot_pos, int T, int k,
                           int H, float* dw, void* dYp, DType t, hipStream_t s);
// dn[t] = sum_i dXp[slot_pos[t k + i]]   (fp32, overwrites dn)
int launch_moe_unpermute(const float* dXp, const int32_t* slot_pos, int T, int k, int H, float* dn, hipStream_t s);
// d loss / d router logits from d loss / d w (type t output)
int launch_moe_router_bwd(const float* probs, const int32_t* ids, const float* w, const float* dw, int T, int E, int k,
                          void* dlogits, DType t, hipStream_t s);

// Sum of squares: row_loss[t] = sum_j h^2, dh = 2h.
int launch_sumsq(const float* h, float* row_loss, float* dh, int T, int H, hipStream_t s);

}  // namespace hol
