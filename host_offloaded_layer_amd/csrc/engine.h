// The streamed trainer behind the C ABI: host state, HBM plan, streams/events and the
// phase 1-3 schedule of MegaTrain's streaming training step.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <array>
#include <atomic>
#include <condition_variable>
#include <map>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "../../include/hol.h"
#include "kernels.h"

namespace hol {

struct TensorDesc {
  std::string name;
  int ndim = 0;
  int64_t shape[4] = {0, 0, 0, 0};
  int64_t numel = 0;
  bool trainable = true;
  int64_t flat = 0;      // offset (floats) in the flat host arrays (master / grad / m / v); -1 for a
                         // frozen tensor whose only copy is its image (frozen base under LoRA)
  int block = 0;         // image block: layer index, or -1 for the head block, -2 none (embed)
  int64_t img = -1;      // byte offset inside that image block
  bool img_f32 = false;  // kept fp32 in the image (norm gains)
};

// Saved intermediates of one layer (row-major, T tokens).
struct Act {
  float* hin = nullptr;  // layer input (fp32 [T,H]); for the first layer of a block: a checkpoint
  float* r1 = nullptr;   // rstd of the attention norm [T]
  void* n1 = nullptr;    // normed input [T,H]
  void* qkv = nullptr;   // [T, QKV] (q, k after RoPE)
  void* o = nullptr;     // attention output [T, nq*d]
  float* lse = nullptr;  // [n_seq, nq, S]
  float* h1 = nullptr;   // residual after attention (fp32 [T,H])
  float* r2 = nullptr;   // rstd of the MLP norm [T]
  void* n2 = nullptr;    // [T,H]
  void* gu = nullptr;    // [T, 2F] (gate | up)
  void* a = nullptr;     // silu(gate)*up [T, F]
  // mixture of experts (T k routed rows)
  float* probs = nullptr;       // router softmax fp32 [T, E]
  int32_t* ids = nullptr;       // [T, k] expert of each slot
  float* w = nullptr;           // [T, k] renormalised routing weight
  int32_t* slot_pos = nullptr;  // [T k] routed row of each slot
  int32_t* perm_slot = nullptr; // [T k] slot of each routed row
  void* gup = nullptr;          // [T k, 2 Fe] expert gate | up outputs
  float* yp = nullptr;          // [T k, H] expert outputs (fp32)
  int32_t* mtab = nullptr;      // [2 E + 2] expert row offsets and 256-row tile offsets
};

enum OpKind { OP_FWD = 0, OP_RECOMP = 1, OP_BWD = 2, OP_HEAD = 3 };
struct Op {
  OpKind kind;
  int layer;  // 0-based
  int block;  // checkpoint block of the layer
  int pos;    // position inside the block
};

enum KClass { KC_GEMM = 0, KC_ATTN_FWD, KC_ATTN_BWD, KC_RMSNORM, KC_ROPE, KC_SWIGLU, KC_CE, KC_TRANSPOSE, KC_OTHER, KC_N };
struct KStat {
  int launches = 0;
  double ms = 0, flops = 0, bytes = 0;
};

struct Stats {
  double fb_ms = 0, step_ms = 0, h2d_bytes = 0, d2h_bytes = 0, h2d_busy_ms = 0, d2h_busy_ms = 0,
         h2d_span_bytes = 0,  // bytes of the weight copies h2d_busy_ms times (the call's own layer and head copies)
         compute_busy_ms = 0, fwd_ms = 0, recomp_ms = 0, bwd_ms = 0, head_ms = 0, host_embed_ms = 0;
  // host timeline of a fused call (ms from the call's start): GPU work drained, embedding
  // scatter-add done; per optimiser unit: gradient arrived on the host, Adam done
  double gpu_done_ms = 0, scatter_done_ms = 0, worker_busy_ms = 0;
  // staleness-1 call: time the issuing thread waited for the overlapped step to read old gradients
  double async_wait_ms = 0;
  // device timeline (ms after the first weight copy starts): first compute op starts, last ends
  double first_compute_ms = 0, last_compute_end_ms = 0;
  std::vector<std::array<double, 3>> units;  // {unit, arrived, done}
  std::vector<std::array<double, 3>> waits;  // staleness-1 call: {unit, wait start, wait end}
  // device spans of the call: {class (0 h2d, 1 d2h, 2 fwd, 3 recompute, 4 bwd, 5 head), start, end}
  // in ms after the first weight copy starts
  std::vector<std::array<float, 3>> timeline;
  int n_weight_streams = 0;
  int tokens = 0;
  // pinned ring: bytes staged through it and host time spent copying into its segments
  double staged_bytes = 0, staging_ms = 0;
  KStat k[KC_N];
  std::map<std::array<int, 3>, KStat> gemm_shapes;  // per (M, N, K) of the GEMM launches
};

}  // namespace hol

struct hol_model {
  hol_config cfg{};
  // derived shape
  int L = 0, H = 0, nq = 0, nkv = 0, d = 0, F = 0, V = 0, QKV = 0, nqd = 0;
  int NE = 0, topk = 0, Fe = 0;  // experts (NE == 0: dense MLP), experts per token, expert FFN width
  int R = 0;                     // LoRA rank (0: full fine-tune)
  bool base_trainable = true;    // false under LoRA: every base tensor is frozen
  bool head_trainable = false, embed_trainable = false;
  int E = 4;  // bytes per compute element
  hol::DType dt = hol::DT_F32;
  int Tmax = 0, Smax = 0, K = 1, Kmax = 1, nblocks = 0, n_ckpt = 0;
  std::vector<hol::TensorDesc> tensors;

  // host state (flat arrays; per layer contiguous in device grad-block order)
  int64_t n_flat = 0, layer_flat0 = 0, layer_flat_n = 0, head_flat0 = 0, head_flat_n = 0, embed_flat0 = -1;
  float* master = nullptr;   // fp32 masters
  float* grad = nullptr;     // fp32 accumulated gradients (pinned)
  float* mom1 = nullptr;
  float* mom2 = nullptr;
  uint8_t* image = nullptr;  // low-precision copy, layer-contiguous, 4 KiB aligned (pinned, or
                             // pageable under a pinned budget smaller than the image)
  // Pinned ring (a pinned budget below the image size): nring pinned segments of ring_seg bytes
  // through which every image-to-HBM copy is staged; segment s is reused once the DMA that last
  // read it (ring_ev[s]) is done. Guarded by h2d_mu, like every weight copy.
  int nring = 0, ring_next = 0;
  int64_t ring_seg = 0;
  uint8_t* ring[8] = {};
  hipEvent_t ring_ev[8] = {};
  std::vector<void*> host_allocs;  // pageable images (freed at destroy)
  // staleness-1 asynchronous optimiser (allocated only when configured): the second image takes
  // the step's refreshed copy while the GPU streams from the first
  uint8_t* image_alt = nullptr;
  int64_t layer_img_bytes = 0, head_img_bytes = 0, image_bytes = 0;
  // layer image offsets (bytes); MoE: router [E, H], expert gates [E, Fe, H], ups [E, Fe, H],
  // downs [E, H, Fe]; LoRA factors fp32: A [r, in], B [out, r] for q, k, v, o
  int64_t o_wqkv = 0, o_wo = 0, o_wgu = 0, o_wd = 0, o_g1 = 0, o_g2 = 0;
  int64_t o_router = 0, o_egate = 0, o_eup = 0, o_edown = 0, o_lA[4] = {}, o_lB[4] = {};
  int64_t o_gf = 0, o_wout = 0;                                           // head image offsets
  // layer gradient block offsets (floats); -1 when the tensor is frozen
  int64_t g_wqkv = -1, g_wo = -1, g_wgu = -1, g_wd = -1, g_g1 = -1, g_g2 = -1;
  int64_t g_router = -1, g_egate = -1, g_eup = -1, g_edown = -1, g_lA[4] = {-1, -1, -1, -1}, g_lB[4] = {-1, -1, -1, -1};
  int64_t wT_bytes = 0;  // bytes of the layer image the bf16 backward transposes
  // bf16 MoE with 64-aligned widths: one grouped launch per expert product; the backward's data
  // gradients read the experts transposed, stacked: gate and up [H, E Fe], down [Fe, E H]
  bool moe_grp = false;
  int64_t t_egate = 0, t_eup = 0, t_edown = 0;  // byte offsets of those in wT

  // pinned host staging
  float* h_stage = nullptr;      // [Tmax, H] embedding rows up / first-layer gradient down
  float* grad_stage = nullptr;   // layer grad block (accumulate mode)
  float* head_stage = nullptr;   // head grad (accumulate mode)
  float* loss_stage = nullptr;   // [Tmax]
  int32_t* lab_stage = nullptr;  // [Tmax]
  float* w_stage = nullptr;      // [Tmax]
  int32_t* ord_stage = nullptr;  // [2 Tmax + 1] positions by token id, then each token's first index

  // device
  hipStream_t sc = nullptr, sh2d = nullptr, sd2h = nullptr;
  static constexpr int MAX_SLOTS = 8, MAX_GBUF = 4;
  int nslots = 2, ngbuf = 2;
  uint8_t* slot[MAX_SLOTS] = {};
  int slot_layer[MAX_SLOTS] = {};
  hipEvent_t ev_ready[MAX_SLOTS] = {}, ev_free[MAX_SLOTS] = {}, ev_gdone[MAX_GBUF] = {}, ev_gfree[MAX_GBUF] = {},
             ev_head = nullptr, ev_h0 = nullptr;
  uint8_t* head_dev = nullptr;
  float* gdev[MAX_GBUF] = {};
  int32_t *ord_dev = nullptr, *seg_dev = nullptr;  // the same on the device
  float* erows = nullptr;                          // [Tmax, H] embedding-row gradients
  float* head_gdev = nullptr;
  float* ckpt = nullptr;
  uint8_t* act_mem = nullptr;
  int64_t act_stride = 0;
  int64_t ao_hin = 0, ao_r1 = 0, ao_n1 = 0, ao_qkv = 0, ao_o = 0, ao_lse = 0, ao_h1 = 0, ao_r2 = 0, ao_n2 = 0,
          ao_gu = 0, ao_a = 0, ao_probs = 0, ao_ids = 0, ao_w = 0, ao_slot = 0, ao_perm = 0, ao_gup = 0, ao_yp = 0,
          ao_mtab = 0;
  // mixture of experts: per activation-store position, the host copy of the expert row counts
  // (read only where per-expert launches need them: fp32 compute, expert weight gradients)
  std::vector<std::vector<int32_t>> act_counts;
  float* mlogits = nullptr;                       // router logits fp32 [T, E]
  int32_t *mcounts = nullptr, *moffsets = nullptr, *mperm = nullptr;
  int32_t* counts_stage = nullptr;                // pinned [E]
  void *xp = nullptr, *ap = nullptr, *dyp = nullptr, *dap = nullptr, *dgup = nullptr, *dlogr = nullptr;
  float *dxp = nullptr, *dwr = nullptr;
  int32_t* route_rec = nullptr;                   // [L, T k] expert ids of the last forward pass
  int last_T = 0;
  // LoRA scratch: x A^T and dy B, fp32 [T, r]
  float *lu = nullptr, *lg = nullptr;
  float* hbuf[2] = {nullptr, nullptr};
  float* dh = nullptr;
  float* dn = nullptr;
  void* dhb = nullptr;
  bool dhb_current = false;  // dhb holds dh rounded to bf16 (kept by the writers of dh)
  void* dqkv = nullptr;
  void* dO = nullptr;
  void* da = nullptr;
  void* dgu = nullptr;
  float* delta = nullptr;
  float* partial = nullptr;
  void* zbuf = nullptr;
  float* rz = nullptr;
  float* logits = nullptr;
  void* dlogits = nullptr;
  int Tc = 0;
  int32_t* labels_dev = nullptr;
  float* w_dev = nullptr;
  float* rowloss_dev = nullptr;
  float* cos_dev = nullptr;
  float* sin_dev = nullptr;
  // bf16 path: every backward product runs as C = A B^T with both operands K-contiguous, so the
  // layer's weights, the upstream gradients and the saved activations are transposed first
  void* wT = nullptr;     // transposed weights of the resident layer (layer image size)
  void* yT = nullptr;     // transposed upstream gradient (largest: [2F, T] or the head's [V, Tc])
  void* xT = nullptr;     // transposed activation (largest: [F, T])
  void* woutT = nullptr;  // transposed LM head [H, V]
  float* qkvf = nullptr;  // fp32 q/k/v projection output before RoPE and the single bf16 rounding
  float* gemm_ws = nullptr;  // GEMM split-tail workspace (GEMM_SPLIT_WS_FLOATS floats)
  std::vector<void*> dev_allocs;
  std::vector<void*> pinned_allocs;
  std::vector<hipEvent_t> tev;  // timing events
  int tev_used = 0;
  bool ktiming = false;                 // per-kernel-launch events
  std::vector<hipEvent_t> kev;          // pool for per-kernel events
  struct KRec { int cls; int ev; double flops, bytes; int gm, gn, gk; };  // gm/gn/gk: GEMM shape (0 otherwise)
  std::vector<KRec> krec;

  int64_t step_t = 0;
  bool poisoned = false;
  bool grads_zero = true;
  // after a fused forward_backward + step the layer and head gradient blocks hold the consumed
  // gradients instead of zeros (the next call's copies overwrite them whole); they read as zero
  // and are cleared before anything accumulates into them. The embedding block is always zeroed.
  bool grads_stale = false;
  hol::Stats stats;

  // The next call's LM-head weights: the fused step's worker queues their copy into head_dev on the
  // weight stream as soon as the head's update is done (it runs in the backward, where the link
  // has slack, instead of behind the last forward layer). They are used while the head's image
  // has not been written since (head_img_ver counts those writes) and the image buffer is the same.
  // held around each sequence of calls that queue one copy on the weight stream (the worker's head
  // copy must not fall between a layer copy and the event that marks that layer ready)
  std::mutex h2d_mu;
  hipEvent_t ev_head_done = nullptr, ev_head_pf = nullptr;  // head op done with head_dev / copy done
  bool head_pf = false;  // a copy was issued (it may still be in flight)
  std::atomic<uint64_t> head_img_ver{0};
  // The next call's first layers. The backward ends with the first block's layers, and their
  // updates are the fused step's last units (layer 0's in pieces). Once a layer's update is done
  // the worker queues its new image into the slot that layer occupied, on the weight stream, when
  // no copy of this call can reuse that slot (every op left uses another layer that is resident).
  // The next call keeps such a slot bound while that layer's image has not been written since
  // (lpf_img_ver) and the image buffer is the same.
  static constexpr int NPF = 4;
  std::atomic<uint64_t> lpf_img_ver[NPF]{};
  uint64_t lpf_ver[NPF] = {};
  const uint8_t* lpf_src[NPF] = {};
  int lpf_slot[NPF] = {-1, -1, -1, -1};  // slot of the copy in flight or landed (-1: none)
  int lpf_next[NPF] = {-1, -1, -1, -1};  // this call: the layer's slot, once its backward is queued
  int n_tail_expect = 0;         // this call: N_TAIL pieces of a last layer copied that way, else 0
  hipEvent_t ev_lpf_done[NPF] = {};  // the layer's backward done with its slot
  uint64_t head_pf_ver = 0;
  const uint8_t* head_pf_src = nullptr;

  // optimiser units: 0 = embedding, 1 + l = layer l, L + 1 = final norm and LM head
  std::vector<std::vector<int>> unit_tensors;
  // fused forward_backward + step: per-unit gradient-arrival events and the host worker
  std::vector<hipEvent_t> ev_unit;     // recorded on the d2h stream after a unit's gradient copy
  std::mutex fmu;
  std::condition_variable fcv;
  std::vector<int> unit_queue;         // units whose gradient copy has been enqueued, in order
  // a layer that is not copied in pieces (below: MoE, adapters, fp32) copies its gradient whole,
  // except the last one of a fused call, in N_TAIL pieces each handed to the worker on its own
  // (queue code TAIL_CODE + piece), so its Adam overlaps the rest of the copy
  static constexpr int N_TAIL = 4, TAIL_CODE = 1 << 20;
  hipEvent_t ev_tail[N_TAIL] = {};
  int tail_unit = -1;
  int64_t tail_lo[N_TAIL] = {}, tail_hi[N_TAIL] = {};  // piece ranges inside the layer block
  int n_tail = 0;
  // dense bf16 layers with trainable weights: the gradient goes down in three pieces, each as soon
  // as it is final: w_down (its product is the MLP backward's first), then w_gate | w_up (the MLP
  // backward's last), then the rest once the layer's backward is done. The backward records
  // ev_wd_final and ev_mlp_final on the compute stream when pieces_armed. In a fused call every
  // piece is also its own optimiser job (queue code PIECE_CODE + index into pjobs), so the Adam of
  // a layer's MLP weights runs while its attention backward computes.
  hipEvent_t ev_wd_final = nullptr, ev_mlp_final = nullptr;
  bool pieces_armed = false;
  std::vector<hipEvent_t> ev_piece;  // 3 per layer, recorded on the d2h stream after each piece
  struct PieceJob {
    int unit;
    int64_t lo, hi;  // flat parameter range
    hipEvent_t ev;
    bool last;  // the unit's last job
  };
  static constexpr int PIECE_CODE = 1 << 21;
  std::vector<PieceJob> pjobs;  // this call's piece jobs (only the main thread appends, before the push)
  std::vector<int32_t> emb_touched, emb_untouched;  // embedding rows the call's tokens use / do not
  bool fused_abort = false;
  double fused_overlap_ms = 0, fused_tail_ms = 0;
};

namespace hol {
hol_status engine_create(const hol_config* cfg, hol_model** out);
void engine_destroy(hol_model* m);
// mode: FB_PLAIN (gradients accumulated), FB_FUSED (forward_backward then step, the step
// overlapped where nothing was accumulated before), FB_ASYNC (the accumulated gradient's step runs
// on the host while this call computes at the parameters from before it)
enum FbMode { FB_PLAIN = 0, FB_FUSED = 1, FB_ASYNC = 2 };
hol_status engine_forward_backward(hol_model* m, const hol_batch* b, hol_loss loss, double* out,
                                  FbMode mode = FB_PLAIN);
hol_status engine_step(hol_model* m);
hol_status engine_zero_grad(hol_model* m);
hol_status engine_set_k(hol_model* m, int k);
hol_status engine_set_kernel_timing(hol_model* m, bool on);
void refresh_image_tensor(hol_model* m, const TensorDesc& t);
void write_image_tensor(hol_model* m, const TensorDesc& t, const float* src);
void read_image_tensor(const hol_model* m, const TensorDesc& t, float* dst);
hol_status engine_get_routing(const hol_model* m, int layer, int32_t* ids, int64_t n);
std::string stats_json(const hol_model* m);
void set_error(const std::string& s);
}  // namespace hol
