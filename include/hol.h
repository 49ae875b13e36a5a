/* hol.h - layer-streamed training with host-resident model state on one AMD MI355X (gfx950).
 *
 * The GPU holds no persistent model state (RoundPipe popular article §二, the computation-dispatch
 * paradigm; MegaTrain summary page, 研究动机 and 核心方法: host memory owns parameters, optimiser
 * state and accumulated gradients, device memory holds only a template pool). One call of
 * hol_forward_backward streams every decoder layer's weights host->HBM into a ring of device
 * slots (2 to 8, `weight_slots`; the pages' double buffer is the 2-slot case), binds them to a
 * weight-free layer template, runs the forward pass keeping a checkpoint every K
 * layers, then runs the loss anchor and a block-wise backward (recompute each block from its
 * checkpoint, then backward layer by layer), streaming each layer's gradient back to the host
 * (MegaTrain summary page, 方法步骤详情 phases 1-3). hol_step runs Adam on the host (phase 4).
 *
 * The two training calls follow the RoundPipe user guide (核心概念): forward_backward(input,
 * label, loss_fn) returns the SUM of the micro-batch losses and accumulates gradients
 * (输入分割与 microbatch 执行), and step() runs the optimiser then zero_grad().
 *
 * Conventions
 *  - Every pointer argument is a HOST pointer owned by the caller, read or written only during
 *    the call (the library copies what it keeps). Device memory is private to the library.
 *  - Calls are synchronous. A model is not re-entrant; distinct models are independent.
 *  - All functions return hol_status. On error, hol_last_error() returns a message
 *    (thread-local, valid until the next call on the same thread).
 *  - HOL_EINVAL is returned before any work is done and leaves the model untouched.
 *  - A device failure inside forward_backward or step returns HOL_EDEVICE and poisons the model:
 *    further forward_backward / step return HOL_ESTATE until hol_zero_grad() is called.
 *  - Allocation failures (HOL_ENOMEM_HOST / HOL_ENOMEM_DEVICE) come from hol_create only: all
 *    host and device memory is planned and allocated there.
 */
#ifndef HOL_H
#define HOL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HOL_OK = 0,
  HOL_EINVAL = -1,        /* bad argument, shape or state; nothing was done */
  HOL_ENOMEM_HOST = -2,   /* host (pageable or pinned) allocation failed in hol_create */
  HOL_ENOMEM_DEVICE = -3, /* HBM allocation failed in hol_create */
  HOL_EDEVICE = -4,       /* HIP runtime or kernel failure; the model is poisoned */
  HOL_ESTATE = -5,        /* model poisoned by an earlier device error */
  HOL_EUNSUPPORTED = -6   /* configuration this build does not implement */
} hol_status;

typedef enum { HOL_F32 = 0, HOL_BF16 = 1 } hol_dtype;   /* compute dtype; masters/Adam are fp32 */
typedef enum { HOL_LOSS_NEXT_TOKEN_CE = 0, HOL_LOSS_SUM_SQUARES = 1 } hol_loss;

typedef struct hol_model hol_model; /* opaque, library-owned */

/* Model and run configuration. Layer math (not fixed by the pages; the plain reading):
 * pre-norm decoder layer = RMSNorm -> q,k,v projections -> RoPE (rotate-half, theta_j =
 * rope_base^(-2j/head_dim)) -> causal grouped-query attention (q head h uses kv head
 * h / (n_q_heads / n_kv_heads)) -> output projection + residual -> RMSNorm -> SwiGLU MLP
 * (silu(x W_gate^T) * (x W_up^T)) W_down^T + residual. Weights are [out, in] (y = x W^T). */
typedef struct {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn;
  int32_t vocab;              /* > 0: token input with untied embedding and LM head;
                                 0: hidden-state input, no embedding, no head */
  int32_t n_experts, top_k, expert_ffn; /* n_experts == 0: dense SwiGLU MLP of width ffn.
                                 n_experts in [1, 512]: mixture-of-experts MLP instead (ffn
                                 unused): router logits n W_r^T (W_r [n_experts, hidden]),
                                 softmax, the top_k (<= 16) largest probabilities with ties to the
                                 lower expert index, weights renormalised over the kept experts,
                                 no capacity limit; each kept expert is a SwiGLU of width
                                 expert_ffn; outputs summed with those weights */
  int32_t lora_rank;          /* 0: full fine-tune. 1..64: every base tensor is frozen and a
                                 LoRA adapter y += lora_scale (x A^T) B^T (A [r, in], B [out, r],
                                 fp32) on the q, k, v and output projections is trained */
  float lora_scale;
  float rope_base, rms_eps;   /* e.g. 10000, 1e-5 */
  int32_t ckpt_every_k;       /* keep h_0, h_K, h_2K, ... in HBM (MegaTrain: checkpoint every K) */
  hol_dtype compute_dtype;    /* HOL_F32 or HOL_BF16 (bf16 operands, fp32 accumulation) */
  float lr, beta1, beta2, adam_eps, weight_decay; /* weight_decay must be 0 */
  int32_t device;             /* HIP device ordinal */
  int32_t max_tokens;         /* largest batch*seq passed to forward_backward (sizes the HBM plan) */
  int32_t max_seq;            /* longest sequence (sizes the RoPE table) */
  int32_t weight_slots;       /* HBM slots of the weight ring, 2..8; 0: min(8, max(4, K + 2)) for
                               * K = ckpt_every_k. Two is the pages' double buffer; with K or more
                               * a block's layers stay resident from its recompute through its
                               * backward, and further slots let the transfer stream run ahead
                               * where the compute is the longer of the two. Results do not
                               * depend on it. */
  int32_t grad_buffers;       /* HBM layer-gradient buffers awaiting the device->host copy, 2..4;
                               * 0: 4. Results do not depend on it. */
  int32_t async_optimizer;    /* 1: also allocate a second pinned low-precision image, which
                               * hol_forward_backward_async needs; 0: none (that call returns
                               * HOL_EINVAL). */
  uint64_t pinned_budget_bytes; /* Host memory the low-precision image may pin (MegaTrain summary
                               * page, 技术新颖性: pinned segments reused across layers instead of
                               * pinning the whole model). 0, or at least the image size (twice it
                               * with async_optimizer): the whole image is pinned and every weight
                               * copy is one DMA from its final place. Smaller: the image stays in
                               * pageable memory and every weight copy is staged by the host through
                               * a ring of R = min(8, budget / S) pinned segments of S bytes (S =
                               * one layer's block rounded up to 4 KiB; the LM-head block goes in
                               * pieces of S), a segment being reused once the DMA that read it is
                               * done; budget < 2 S is HOL_EINVAL, and so is the ring together with
                               * async_optimizer. Results do not depend on it. The fp32 gradient
                               * block and the small staging buffers are always pinned; a host that
                               * cannot pin what is asked gets HOL_ENOMEM_HOST from hol_create. */
} hol_config;

/* One forward_backward input. tokens: int32 [batch*seq] (vocab > 0); labels: int32
 * [batch*seq] or NULL for next-token labels (last position of every sequence ignored); a label
 * of -1 is ignored. hidden_in: fp32 [batch*seq*hidden] when vocab == 0. The batch is split into
 * n_micro contiguous groups of batch/n_micro sequences (RoundPipe user guide, 输入分割与
 * microbatch 执行); batch % n_micro != 0 is HOL_EINVAL. */
typedef struct {
  const int32_t* tokens;
  const int32_t* labels;
  const float* hidden_in;
  int32_t batch, seq, n_micro;
} hol_batch;

/* Creates a model: plans and allocates all host state (fp32 masters, Adam m/v, pinned fp32
 * gradients, layer-contiguous low-precision image with 4 KiB-aligned sub-tensors, pinned or
 * behind the pinned ring of pinned_budget_bytes) and all
 * device memory (the ring of weight slots, head buffer, checkpoint store, block activation
 * store, gradient buffers). Weights start at zero; load them with hol_set_tensor. */
hol_status hol_create(const hol_config* cfg, hol_model** out);
void hol_destroy(hol_model* m);

/* Tensor directory: index i in [0, n). name is NUL-terminated (truncated to cap). shape[0..ndim-1].
 * trainable == 0 for frozen tensors. */
hol_status hol_num_tensors(const hol_model* m, int32_t* n);
hol_status hol_tensor_info(const hol_model* m, int32_t i, char* name, size_t cap, int64_t shape[4],
                           int32_t* ndim, int32_t* trainable);
/* fp32 master <- src (numel floats, row-major) and refresh of the low-precision image. A frozen
 * tensor other than the embedding keeps no fp32 master: set writes its image (rounded to the
 * compute dtype) and get returns the image's values. */
hol_status hol_set_tensor(hol_model* m, int32_t i, const float* src, int64_t numel);
hol_status hol_get_tensor(const hol_model* m, int32_t i, float* dst, int64_t numel);
/* Accumulated gradient of a trainable tensor (zeros after hol_step / hol_zero_grad). */
hol_status hol_get_grad(const hol_model* m, int32_t i, float* dst, int64_t numel);
/* Adam moments and the step counter (number of hol_step calls so far) of a trainable tensor;
 * set restores them. HOL_EINVAL for a frozen tensor. */
hol_status hol_get_adam_state(const hol_model* m, int32_t i, float* mom1, float* mom2, int64_t numel,
                              int64_t* step);
hol_status hol_set_adam_state(hol_model* m, int32_t i, const float* mom1, const float* mom2,
                              int64_t numel, int64_t step);

/* Mixture-of-experts routing of the last forward_backward: the top_k expert ids chosen for each
 * token of layer `layer` in slot order (ids[t * top_k + i]; t over batch*seq tokens, n =
 * batch*seq*top_k). HOL_EINVAL for a dense model, a bad layer or n, or before any call. */
hol_status hol_get_routing(const hol_model* m, int32_t layer, int32_t* ids, int64_t n);

/* Checkpoint interval for later forward_backward calls: 1 <= k <= cfg.ckpt_every_k (the
 * activation store is planned for cfg.ckpt_every_k layers, the checkpoint store for k = 1).
 * Results do not depend on k (the recompute repeats the forward bit for bit). */
hol_status hol_set_ckpt_every_k(hol_model* m, int32_t k);

/* Zeroes accumulated gradients and clears the poisoned state. */
hol_status hol_zero_grad(hol_model* m);

/* One streamed forward + backward over all micro-batches (MegaTrain summary page, 方法步骤详情
 * phases 1-3). *loss_sum_out = sum over micro-batches of the micro-batch loss: the mean
 * next-token cross entropy over the micro-batch's labelled positions, or the plain sum of squares
 * of the last hidden state. Gradients are ADDED to the host accumulators. Returns after every
 * gradient is in host memory. */
hol_status hol_forward_backward(hol_model* m, const hol_batch* batch, hol_loss loss,
                                double* loss_sum_out);

/* Host Adam over every trainable tensor, step counter += 1, refresh of the low-precision image,
 * then zero_grad (MegaTrain summary page, 方法步骤详情 phase 4; RoundPipe user guide, 核心概念). */
hol_status hol_step(hol_model* m);

/* on != 0: every kernel launch of later forward_backward calls is bracketed by HIP events on the
 * compute stream and hol_last_stats reports, per kernel class (gemm, attn_fwd, attn_bwd, rmsnorm,
 * rope, swiglu, ce, other), the launch count, summed duration, algorithmic FLOPs and bytes. */
hol_status hol_set_kernel_timing(hol_model* m, int32_t on);

/* forward_backward followed by step, with the same result bit for bit: when no gradient is
 * accumulated from earlier calls, each layer's host optimiser update (and the refresh of its
 * low-precision copy) starts as soon as that layer's gradient is in host memory, so the optimiser
 * runs under the remaining backward pass; otherwise the two calls run one after the other. A device
 * error inside the call may leave the step applied to some tensors only (the model is poisoned). */
hol_status hol_forward_backward_step(hol_model* m, const hol_batch* batch, hol_loss loss,
                                     double* loss_sum_out);

/* Staleness-1 asynchronous optimiser (RoundPipe paper summary, 异步优化器 and 方法步骤详情 step 6):
 * the host optimiser step of one call's gradients runs while the next call computes, and that call
 * does not wait for it. One call does three things:
 *   1. a streamed forward + backward of `batch` at the parameters as they stand when the call
 *      starts (what hol_get_tensor returns then);
 *   2. meanwhile, if gradients are accumulated (from the previous async call, or from
 *      hol_forward_backward calls since the last step or zero_grad), hol_step's update with them,
 *      on host threads (Adam, step counter + 1, refresh of the low-precision copy);
 *   3. on return this call's gradients are the accumulated gradients (hol_get_grad reads them).
 * So with theta_0 the starting parameters and g_t the gradient of the t-th call in a row,
 * g_t = grad L_t(theta_{t-2}) (theta_{-1} = theta_0) and theta_t = Adam(theta_{t-1}, g_t), applied
 * by call t + 1, or by hol_step at the end. Apart from the parameters the gradient is taken at,
 * this is hol_forward_backward followed by hol_step, bit for bit. The first call in a row (nothing
 * accumulated) applies no update. Needs cfg.async_optimizer = 1 (HOL_EINVAL otherwise): the update
 * refreshes the second image while the GPU streams from the first. The gradient block is shared:
 * each unit's new gradient copy (LM head, then layers from the last, then the embedding rows) is
 * issued only once the update has read that unit's old gradient. Every other call keeps its
 * meaning. A device error poisons the model as in hol_forward_backward; the overlapped update has
 * then still been applied whole. */
hol_status hol_forward_backward_async(hol_model* m, const hol_batch* batch, hol_loss loss,
                                      double* loss_sum_out);

/* Timing and traffic of the last forward_backward / step as a JSON object (NUL-terminated).
 * Fields: fb_ms, step_ms, h2d_bytes, d2h_bytes, h2d_busy_ms, d2h_busy_ms, compute_busy_ms,
 * n_weight_streams, h2d_span_bytes (the bytes of the weight copies h2d_busy_ms times: h2d_bytes
 * also counts h0 and the copies a fused step sends ahead for the next call, which have no span),
 * per-kernel-class compute ms, and for hol_forward_backward_step the host
 * timeline (gpu_done_ms, scatter_done_ms, worker_busy_ms, units = [unit, start, end] of each
 * optimiser unit in ms from the call's start); for hol_forward_backward_async worker_busy_ms is the
 * overlapped step's time and async_wait_ms the time gradient copies waited for it. HOL_EINVAL, with nothing written, when the
 * object does not fit in cap bytes. */
hol_status hol_last_stats(const hol_model* m, char* json, size_t cap);

/* Stage partition (host only). RoundPipe popular article §六 and paper summary (方法步骤详情,
 * step 2): contiguous stages with a bound t_max on every stage's time and a memory cap; forward
 * and backward partitioned separately (backward filled from the last layer). Objective (reading):
 * minimise J = (n_micro*(S_f+S_b) + n_gpus*(n_gpus-1)) * t_max over candidate t_max values (every
 * contiguous sum of t_f and of t_b), ties to the smaller t_max; for each candidate the greedy
 * pass packs the longest stages allowed. Inputs int64 [L]; outputs: f_bounds[0..*n_f) = first
 * layer of each forward stage (ascending), b_bounds[0..*n_b) = highest layer of each backward
 * stage (descending from L-1); both arrays need L entries. *J_out may be NULL. Returns HOL_EINVAL
 * when some layer exceeds mem_cap or on bad sizes. Exact (integer) result. */
hol_status hol_partition(const int64_t* t_f, const int64_t* t_b, const int64_t* m_f,
                         const int64_t* m_b, int32_t L, int64_t mem_cap, int32_t n_gpus,
                         int32_t n_micro, int32_t* f_bounds, int32_t* n_f, int32_t* b_bounds,
                         int32_t* n_b, int64_t* t_max, int64_t* J_out);

/* The host optimiser step on one fp32 tensor (what hol_step runs per tensor), exposed for
 * testing: theta, grad, mom1, mom2 are host arrays of n floats; step_t >= 1. The arithmetic order
 * is fixed (bias corrections 1 - beta^t in fp64 rounded to fp32 once; no fused multiply-add):
 * m = b1 m + (1-b1) g; v = b2 v + (1-b2) g^2; theta -= (lr m/bc1) / (sqrt(v/bc2) + eps). */
hol_status hol_host_adam(float* theta, const float* grad, float* mom1, float* mom2, int64_t n,
                         int64_t step_t, float lr, float beta1, float beta2, float eps);
/* fp32 -> bf16 round-to-nearest-even (the low-precision refresh), host only. */
hol_status hol_host_bf16_round(const float* src, uint16_t* dst, int64_t n);

const char* hol_last_error(void);
const char* hol_version(void);

#ifdef __cplusplus
}
#endif
#endif /* HOL_H */
