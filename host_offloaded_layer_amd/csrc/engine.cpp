// Streaming engine of the layer-streamed trainer (MegaTrain summary page, 核心方法 and 方法步骤详情).
//
// Host memory owns every persistent tensor: fp32 masters, Adam moments, fp32 accumulated
// gradients and a low-precision, layer-contiguous image whose sub-tensors are 4 KiB aligned so a
// layer travels as one DMA burst (技术新颖性: layer-contiguous memory tiling). The GPU holds only
// the template pool's working memory: two weight slots (the GPU-domain double buffer), a head
// buffer, the checkpoint store (h every K layers), the activation store of one block, and two
// gradient buffers.
//
// Three HIP streams (核心方法: compute, weight-transfer and gradient-transfer streams) are ordered
// by events only (技术新颖性: weight-ready, backward-done and buffer-free events instead of host
// barriers); nothing is captured into a graph, every StreamIn-Bind-Compute-Offload step is issued
// explicitly:
//   * h2d stream: wait buffer_free[slot] -> copy layer image into slot -> record weight_ready[slot]
//   * compute   : wait weight_ready[slot] -> layer kernels -> record buffer_free[slot]
//   * backward  : wait grad_free[g] -> layer backward into grad buffer g -> record backward_done[g]
//   * d2h stream: wait backward_done[g] -> copy grad buffer to host -> record grad_free[g]
//
// Schedule of one forward_backward (phases 1-3 of the training step; block loop reading: block b
// covers layers bK+1 .. min((b+1)K, L), checkpoints are h_0, h_K, h_2K, ... and h_L):
//   FWD 1..L, HEAD (loss anchor), then for b = last .. 0: RECOMP layers of b in forward order,
//   BWD layers of b in reverse order. A layer still resident in a slot is not streamed again, and
//   the last block is not recomputed: its forward writes the activation store directly.
// Every micro-batch of the call is resident at once and processed by each resident layer
// (layer-major order): GEMMs run over all T = batch*seq tokens, attention per sequence; the loss
// weights each token by 1/(labelled tokens of its micro-batch), which makes the returned value the
// sum of the micro-batch mean losses and the gradient the sum of the micro-batch gradients.
#include "engine.h"

#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <chrono>
#include <immintrin.h>
#include <sstream>

#include "host_math.h"

namespace hol {

static thread_local std::string g_err;
void set_error(const std::string& s) { g_err = s; }
const char* last_error_cstr() { return g_err.c_str(); }

#define HCHECK(expr)                                                                      \
  do {                                                                                    \
    hipError_t e__ = (expr);                                                              \
    if (e__ != hipSuccess) {                                                              \
      set_error(std::string(#expr) + ": " + hipGetErrorString(e__) + " (" __FILE__ ":" + \
                std::to_string(__LINE__) + ")");                                          \
      return HOL_EDEVICE;                                                                 \
    }                                                                                     \
  } while (0)

#define KCHECK(expr)                                                                           \
  do {                                                                                         \
    int e__ = (expr);                                                                          \
    if (e__ != 0) {                                                                            \
      set_error(std::string(#expr) + ": " + hipGetErrorString((hipError_t)e__) + " (" __FILE__ \
                ":" + std::to_string(__LINE__) + ")");                                         \
      return HOL_EDEVICE;                                                                      \
    }                                                                                          \
  } while (0)

static int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

static double now_ms() {
  return std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now().time_since_epoch()).count();
}

// ------------------------------------------------------------------------------------------
// create / destroy
// ------------------------------------------------------------------------------------------
static hol_status validate_config(const hol_config& c) {
  auto bad = [](const std::string& s) {
    set_error("hol_create: " + s);
    return HOL_EINVAL;
  };
  if (c.n_layers <= 0 || c.hidden <= 0 || c.n_q_heads <= 0 || c.n_kv_heads <= 0 || c.head_dim <= 0)
    return bad("non-positive shape");
  if (c.n_q_heads % c.n_kv_heads) return bad("n_q_heads must be a multiple of n_kv_heads");
  if (c.head_dim % 2 || c.head_dim > 128) return bad("head_dim must be even and <= 128");
  if (c.hidden % 8 || c.hidden > 4096) return bad("hidden must be a multiple of 8 and <= 4096");
  if (c.n_experts < 0 || c.lora_rank < 0) return bad("n_experts / lora_rank must be >= 0");
  if (c.n_experts > 0) {
    if (c.n_experts > 512) return bad("n_experts must be <= 512");
    if (c.top_k < 1 || c.top_k > c.n_experts || c.top_k > 16) return bad("top_k must be in [1, min(n_experts, 16)]");
    if (c.expert_ffn <= 0) return bad("expert_ffn must be positive");
  } else if (c.ffn <= 0) {
    return bad("ffn must be positive");
  }
  if (c.lora_rank > 64) return bad("lora_rank must be <= 64");
  if (c.vocab < 0) return bad("vocab must be >= 0");
  // bf16 operands go through the MFMA GEMM, whose rows are moved in 16-byte pieces
  if (c.compute_dtype == HOL_BF16 && (c.vocab % 8 || c.head_dim % 8 ||
                                      (c.n_experts > 0 ? c.expert_ffn % 8 : c.ffn % 8)))
    return bad("bf16 compute needs ffn (expert_ffn), vocab and head_dim multiples of 8");
  if (c.ckpt_every_k <= 0) return bad("ckpt_every_k must be >= 1");
  if (c.compute_dtype != HOL_F32 && c.compute_dtype != HOL_BF16) return bad("compute_dtype");
  if (c.weight_decay != 0.f) return bad("weight_decay must be 0");
  if (c.max_tokens <= 0 || c.max_seq <= 0 || c.max_seq > c.max_tokens) return bad("max_tokens / max_seq");
  if (!(c.rms_eps > 0) || !(c.rope_base > 0)) return bad("rms_eps / rope_base");
  if (c.weight_slots != 0 && (c.weight_slots < 2 || c.weight_slots > 8)) return bad("weight_slots must be 0 or 2..8");
  if (c.grad_buffers != 0 && (c.grad_buffers < 2 || c.grad_buffers > 4)) return bad("grad_buffers must be 0 or 2..4");
  if (c.async_optimizer != 0 && c.async_optimizer != 1) return bad("async_optimizer must be 0 or 1");
  return HOL_OK;
}

static void add_tensor(hol_model* m, const std::string& name, std::initializer_list<int64_t> shape, bool tr,
                       int64_t flat, int block, int64_t img, bool f32) {
  TensorDesc t;
  t.name = name;
  t.ndim = (int)shape.size();
  int i = 0;
  t.numel = 1;
  for (int64_t s : shape) {
    t.shape[i++] = s;
    t.numel *= s;
  }
  t.trainable = tr;
  t.flat = flat;
  t.block = block;
  t.img = img;
  t.img_f32 = f32;
  m->tensors.push_back(t);
}

// Row length (elements) of the transposed token-major operands in yT / xT ([*, t]): t rounded up
// to 8, plus 64. With rows of exactly 2t bytes (32 KB at t = 16384) every row of a 256-row stage
// load starts at the same offset modulo the memory interleave, and the gate/up and down weight
// gradients ran 9 % and 4 % slower than with 128 bytes of padding (3250 → 2958 and 1612 →
// 1546 µs alone at the LLaMA-8B shape; the products are the same bit for bit).
static inline int64_t tpad(int64_t t) { return (t + 7) / 8 * 8 + 64; }

static void* dev_alloc(hol_model* m, int64_t bytes, hol_status* st) {
  void* p = nullptr;
  if (bytes <= 0) bytes = 256;
  if (hipMalloc(&p, (size_t)bytes) != hipSuccess) {
    *st = HOL_ENOMEM_DEVICE;
    set_error("hipMalloc of " + std::to_string(bytes) + " bytes failed");
    return nullptr;
  }
  m->dev_allocs.push_back(p);
  return p;
}

static void* pinned_alloc(hol_model* m, int64_t bytes, hol_status* st) {
  void* p = nullptr;
  if (bytes <= 0) bytes = 256;
  if (hipHostMalloc(&p, (size_t)bytes, hipHostMallocDefault) != hipSuccess) {
    *st = HOL_ENOMEM_HOST;
    set_error("hipHostMalloc of " + std::to_string(bytes) + " bytes failed");
    return nullptr;
  }
  m->pinned_allocs.push_back(p);
  return p;
}

static float* host_alloc_f32(int64_t n) {
  void* p = nullptr;
  if (posix_memalign(&p, 4096, (size_t)std::max<int64_t>(n, 1) * 4) != 0) return nullptr;
  return (float*)p;
}

// zero-fill with the host pool (first touch spreads pages over the pool's threads)
static void parallel_zero(void* p, int64_t bytes) {
  parallel_for(bytes, 1 << 22, [&](int64_t lo, int64_t hi) { memset((uint8_t*)p + lo, 0, (size_t)(hi - lo)); });
}

hol_status engine_create(const hol_config* cfg, hol_model** out) {
  if (!cfg || !out) {
    set_error("hol_create: null argument");
    return HOL_EINVAL;
  }
  hol_status st = validate_config(*cfg);
  if (st != HOL_OK) return st;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) {
    set_error("hol_create: no HIP device available");
    return HOL_EDEVICE;
  }
  if (cfg->device < 0 || cfg->device >= ndev) {
    set_error("hol_create: bad device ordinal");
    return HOL_EINVAL;
  }
  HCHECK(hipSetDevice(cfg->device));

  hol_model* m = new hol_model();
  m->cfg = *cfg;
  const hol_config& c = m->cfg;
  m->L = c.n_layers;
  m->H = c.hidden;
  m->nq = c.n_q_heads;
  m->nkv = c.n_kv_heads;
  m->d = c.head_dim;
  m->F = c.n_experts > 0 ? 0 : c.ffn;  // a mixture-of-experts layer has no dense MLP
  m->V = c.vocab;
  m->nqd = m->nq * m->d;
  m->QKV = (m->nq + 2 * m->nkv) * m->d;
  m->dt = c.compute_dtype == HOL_BF16 ? DT_BF16 : DT_F32;
  m->E = c.compute_dtype == HOL_BF16 ? 2 : 4;
  m->Tmax = c.max_tokens;
  m->Smax = c.max_seq;
  m->K = c.ckpt_every_k;
  m->Kmax = m->K;
  m->nblocks = (m->L + m->K - 1) / m->K;
  m->n_ckpt = m->L + 1;  // enough for any k <= Kmax, down to k = 1
  const int64_t H = m->H, L = m->L, F = m->F, V = m->V, QKV = m->QKV, nqd = m->nqd, E = m->E;

  m->NE = c.n_experts;
  m->topk = c.n_experts > 0 ? c.top_k : 0;
  m->Fe = c.n_experts > 0 ? c.expert_ffn : 0;
  m->R = c.lora_rank;
  m->base_trainable = m->R == 0;
  m->embed_trainable = V > 0 && m->base_trainable;
  m->head_trainable = V > 0 && m->base_trainable;
  const int64_t F_ = m->F, NE = m->NE, Fe = m->Fe, R = m->R, kvd = (int64_t)m->nkv * m->d;

  // ---- image layout of one layer block (each sub-tensor 4 KiB aligned)
  int64_t o = 0;
  m->o_wqkv = o; o = align_up(o + QKV * H * E, 4096);
  m->o_wo = o;   o = align_up(o + H * nqd * E, 4096);
  m->wT_bytes = o;
  if (NE > 0) {
    m->o_router = o; o = align_up(o + NE * H * E, 4096);
    m->o_egate = o;  o = align_up(o + NE * Fe * H * E, 4096);
    m->o_eup = o;    o = align_up(o + NE * Fe * H * E, 4096);
    m->o_edown = o;  o = align_up(o + NE * H * Fe * E, 4096);
  } else {
    m->o_wgu = o;  o = align_up(o + 2 * F_ * H * E, 4096);
    m->o_wd = o;   o = align_up(o + H * F_ * E, 4096);
    m->wT_bytes = o;
  }
  m->moe_grp = NE > 0 && m->dt == DT_BF16 && H % 64 == 0 && Fe % 64 == 0;
  if (m->moe_grp) {
    int64_t t = m->wT_bytes;
    m->t_egate = t; t = align_up(t + NE * Fe * H * E, 4096);
    m->t_eup = t;   t = align_up(t + NE * Fe * H * E, 4096);
    m->t_edown = t; t = align_up(t + NE * H * Fe * E, 4096);
    m->wT_bytes = t;
  }
  m->o_g1 = o;   o = align_up(o + H * 4, 4096);
  m->o_g2 = o;   o = align_up(o + H * 4, 4096);
  // LoRA factors (fp32): q, k, v on the attention-norm output, o on the attention output
  const int64_t l_in[4] = {H, H, H, nqd}, l_out[4] = {nqd, kvd, kvd, H};
  for (int j = 0; j < 4 && R > 0; ++j) {
    m->o_lA[j] = o; o = align_up(o + R * l_in[j] * 4, 4096);
    m->o_lB[j] = o; o = align_up(o + l_out[j] * R * 4, 4096);
  }
  m->layer_img_bytes = o;
  o = 0;
  if (V > 0) {
    m->o_gf = o;   o = align_up(o + H * 4, 4096);
    m->o_wout = o; o = align_up(o + V * H * E, 4096);
  }
  m->head_img_bytes = o;
  m->image_bytes = L * m->layer_img_bytes + m->head_img_bytes;

  // ---- layer gradient block (= the flat host order of the layer's trainable tensors)
  int64_t g = 0;
  if (m->base_trainable) {
    m->g_wqkv = g; g += QKV * H;
    m->g_wo = g;   g += H * nqd;
    if (NE > 0) {
      m->g_router = g; g += NE * H;
      m->g_egate = g;  g += NE * Fe * H;
      m->g_eup = g;    g += NE * Fe * H;
      m->g_edown = g;  g += NE * H * Fe;
    } else {
      m->g_wgu = g; g += 2 * F_ * H;
      m->g_wd = g;  g += H * F_;
    }
    m->g_g1 = g; g += H;
    m->g_g2 = g; g += H;
  }
  for (int j = 0; j < 4 && R > 0; ++j) {
    m->g_lA[j] = g; g += R * l_in[j];
    m->g_lB[j] = g; g += l_out[j] * R;
  }
  m->layer_flat_n = g;

  // ---- flat host layout: [embed] [layer 0 .. L-1] [final_norm, lm_head (when trainable)]
  int64_t flat = 0;
  if (V > 0) {  // the embedding lives only on the host: it always has an fp32 copy
    m->embed_flat0 = 0;
    flat = V * H;
  }
  m->layer_flat0 = flat;
  flat += L * m->layer_flat_n;
  m->head_flat0 = flat;
  m->head_flat_n = m->head_trainable ? H + V * H : 0;
  flat += m->head_flat_n;
  m->n_flat = flat;

  // ---- tensor directory (canonical order)
  const bool bt = m->base_trainable;
  auto gofs = [&](int64_t f0, int64_t go) -> int64_t { return go < 0 ? -1 : f0 + go; };
  if (V > 0) add_tensor(m, "embed", {V, H}, m->embed_trainable, 0, -2, -1, false);
  for (int l = 0; l < L; ++l) {
    const int64_t f0 = m->layer_flat0 + l * m->layer_flat_n;
    const std::string p = "layers." + std::to_string(l) + ".";
    add_tensor(m, p + "attn_norm", {H}, bt, gofs(f0, m->g_g1), l, m->o_g1, true);
    add_tensor(m, p + "wq", {nqd, H}, bt, gofs(f0, m->g_wqkv), l, m->o_wqkv, false);
    add_tensor(m, p + "wk", {kvd, H}, bt, bt ? f0 + m->g_wqkv + nqd * H : -1, l, m->o_wqkv + nqd * H * E, false);
    add_tensor(m, p + "wv", {kvd, H}, bt, bt ? f0 + m->g_wqkv + (nqd + kvd) * H : -1, l,
               m->o_wqkv + (nqd + kvd) * H * E, false);
    add_tensor(m, p + "wo", {H, nqd}, bt, gofs(f0, m->g_wo), l, m->o_wo, false);
    add_tensor(m, p + "mlp_norm", {H}, bt, gofs(f0, m->g_g2), l, m->o_g2, true);
    if (NE > 0) {
      add_tensor(m, p + "router", {NE, H}, bt, gofs(f0, m->g_router), l, m->o_router, false);
      add_tensor(m, p + "experts.w_gate", {NE, Fe, H}, bt, gofs(f0, m->g_egate), l, m->o_egate, false);
      add_tensor(m, p + "experts.w_up", {NE, Fe, H}, bt, gofs(f0, m->g_eup), l, m->o_eup, false);
      add_tensor(m, p + "experts.w_down", {NE, H, Fe}, bt, gofs(f0, m->g_edown), l, m->o_edown, false);
    } else {
      add_tensor(m, p + "w_gate", {F_, H}, bt, gofs(f0, m->g_wgu), l, m->o_wgu, false);
      add_tensor(m, p + "w_up", {F_, H}, bt, bt ? f0 + m->g_wgu + F_ * H : -1, l, m->o_wgu + F_ * H * E, false);
      add_tensor(m, p + "w_down", {H, F_}, bt, gofs(f0, m->g_wd), l, m->o_wd, false);
    }
    static const char* lname[4] = {"q", "k", "v", "o"};
    for (int j = 0; j < 4 && R > 0; ++j) {
      add_tensor(m, p + "lora." + lname[j] + ".A", {R, l_in[j]}, true, f0 + m->g_lA[j], l, m->o_lA[j], true);
      add_tensor(m, p + "lora." + lname[j] + ".B", {l_out[j], R}, true, f0 + m->g_lB[j], l, m->o_lB[j], true);
    }
  }
  if (V > 0) {
    const bool ht = m->head_trainable;
    add_tensor(m, "final_norm", {H}, ht, ht ? m->head_flat0 : -1, -1, m->o_gf, true);
    add_tensor(m, "lm_head", {V, H}, ht, ht ? m->head_flat0 + H : -1, -1, m->o_wout, false);
  }

  // ---- host allocations
  m->master = host_alloc_f32(m->n_flat);
  m->mom1 = host_alloc_f32(m->n_flat);
  m->mom2 = host_alloc_f32(m->n_flat);
  if (!m->master || !m->mom1 || !m->mom2) {
    set_error("hol_create: host allocation of fp32 state failed");
    engine_destroy(m);
    return HOL_ENOMEM_HOST;
  }
  parallel_zero(m->master, m->n_flat * 4);
  parallel_zero(m->mom1, m->n_flat * 4);
  parallel_zero(m->mom2, m->n_flat * 4);
  st = HOL_OK;
  m->grad = (float*)pinned_alloc(m, m->n_flat * 4, &st);
  // the image: pinned whole, or pageable behind a ring of pinned segments when the pinned budget
  // is smaller than the image(s)
  const uint64_t img_total = (uint64_t)m->image_bytes * (c.async_optimizer ? 2u : 1u);
  if (c.pinned_budget_bytes == 0 || c.pinned_budget_bytes >= img_total) {
    m->image = (uint8_t*)pinned_alloc(m, m->image_bytes, &st);
  } else {
    m->ring_seg = align_up(m->layer_img_bytes, 4096);
    const uint64_t r = c.pinned_budget_bytes / (uint64_t)m->ring_seg;
    if (r < 2 || c.async_optimizer) {
      set_error(r < 2 ? "hol_create: pinned_budget_bytes " + std::to_string(c.pinned_budget_bytes) +
                            " is below the image (" + std::to_string(img_total) + " bytes) and below two ring segments of " +
                            std::to_string(m->ring_seg) + " bytes"
                      : std::string("hol_create: the pinned ring (pinned_budget_bytes below the image size) does not "
                                    "serve async_optimizer"));
      engine_destroy(m);
      return HOL_EINVAL;
    }
    m->nring = (int)std::min<uint64_t>(8, r);
    for (int i = 0; i < m->nring; ++i) m->ring[i] = (uint8_t*)pinned_alloc(m, m->ring_seg, &st);
    void* p = nullptr;
    if (posix_memalign(&p, 4096, (size_t)m->image_bytes) != 0) {
      set_error("hol_create: pageable allocation of the " + std::to_string(m->image_bytes) + "-byte image failed");
      engine_destroy(m);
      return HOL_ENOMEM_HOST;
    }
    m->host_allocs.push_back(p);
    m->image = (uint8_t*)p;
  }
  const int64_t T = m->Tmax;
  m->h_stage = (float*)pinned_alloc(m, T * H * 4, &st);
  m->grad_stage = (float*)pinned_alloc(m, m->layer_flat_n * 4, &st);
  m->head_stage = (float*)pinned_alloc(m, std::max<int64_t>(m->head_flat_n, 1) * 4, &st);
  m->loss_stage = (float*)pinned_alloc(m, T * 4, &st);
  m->lab_stage = (int32_t*)pinned_alloc(m, T * 4, &st);
  m->w_stage = (float*)pinned_alloc(m, T * 4, &st);
  if (m->embed_trainable) m->ord_stage = (int32_t*)pinned_alloc(m, (2 * T + 1) * 4, &st);
  if (m->NE > 0) m->counts_stage = (int32_t*)pinned_alloc(m, (int64_t)m->NE * 4, &st);
  if (c.async_optimizer) m->image_alt = (uint8_t*)pinned_alloc(m, m->image_bytes, &st);
  if (st != HOL_OK) {
    engine_destroy(m);
    return st;
  }
  parallel_zero(m->grad, m->n_flat * 4);
  parallel_zero(m->image, m->image_bytes);
  if (m->image_alt) parallel_zero(m->image_alt, m->image_bytes);

  // ---- device plan
  auto D = [&](int64_t bytes) { return dev_alloc(m, align_up(bytes, 256), &st); };
  // default ring: the K layers of a block stay resident from the recompute through the block's
  // backward, and two more slots take the next block's layers while that backward computes
  m->nslots = c.weight_slots ? c.weight_slots : std::min(8, std::max(4, c.ckpt_every_k + 2));
  m->ngbuf = c.grad_buffers ? c.grad_buffers : 4;
  for (int i = 0; i < m->nslots; ++i) m->slot[i] = (uint8_t*)D(m->layer_img_bytes);
  if (m->dt == DT_BF16) m->gemm_ws = (float*)D(GEMM_SPLIT_WS_FLOATS * 4);
  if (V > 0) m->head_dev = (uint8_t*)D(m->head_img_bytes);
  for (int i = 0; i < m->ngbuf; ++i) m->gdev[i] = (float*)D(m->layer_flat_n * 4);
  if (m->embed_trainable) {
    m->ord_dev = (int32_t*)D(T * 4);
    m->seg_dev = (int32_t*)D((T + 1) * 4);
    m->erows = (float*)D(T * H * 4);
  }
  if (V > 0) m->head_gdev = (float*)D(m->head_flat_n * 4);
  m->ckpt = (float*)D((int64_t)m->n_ckpt * T * H * 4);
  // activation block: K layers
  int64_t a = 0;
  auto A = [&](int64_t bytes) {
    const int64_t off = a;
    a = align_up(a + bytes, 256);
    return off;
  };
  m->ao_hin = A(T * H * 4);
  m->ao_r1 = A(T * 4);
  m->ao_n1 = A(T * H * E);
  m->ao_qkv = A(T * QKV * E);
  m->ao_o = A(T * nqd * E);
  m->ao_lse = A(T * m->nq * 4);
  m->ao_h1 = A(T * H * 4);
  m->ao_r2 = A(T * 4);
  m->ao_n2 = A(T * H * E);
  m->ao_gu = A(T * 2 * F * E);
  m->ao_a = A(T * F * E);
  const int64_t Tk = T * m->topk;
  if (NE > 0) {
    m->ao_probs = A(T * NE * 4);
    m->ao_ids = A(Tk * 4);
    m->ao_w = A(Tk * 4);
    m->ao_slot = A(Tk * 4);
    m->ao_perm = A(Tk * 4);
    m->ao_gup = A(Tk * 2 * Fe * E);
    m->ao_yp = A(Tk * H * 4);
    m->ao_mtab = A((2 * NE + 2) * 4);
  }
  m->act_stride = a;
  m->act_counts.assign(m->Kmax, std::vector<int32_t>(std::max<int64_t>(NE, 1), 0));
  m->act_mem = (uint8_t*)D((int64_t)m->Kmax * m->act_stride);
  m->hbuf[0] = (float*)D(T * H * 4);
  m->hbuf[1] = (float*)D(T * H * 4);
  m->dh = (float*)D(T * H * 4);
  m->dn = (float*)D(T * H * 4);
  m->dhb = D(T * H * E);
  m->dqkv = D(T * QKV * E);
  m->dO = D(T * nqd * E);
  m->da = D(T * F * E);
  m->dgu = D(T * 2 * F * E);
  m->delta = (float*)D(T * m->nq * 4);
  m->partial = (float*)D((int64_t)rmsnorm_bwd_blocks((int)T) * H * 4);
  m->labels_dev = (int32_t*)D(T * 4);
  m->w_dev = (float*)D(T * 4);
  m->rowloss_dev = (float*)D(T * 4);
  if (V > 0) {
    m->zbuf = D(T * H * E);
    m->rz = (float*)D(T * 4);
    // logits chunk: up to 4 GiB of fp32 logits, rows a multiple of 256
    int64_t tc = std::max<int64_t>(256, ((int64_t)1 << 30) / V / 256 * 256);
    tc = std::min<int64_t>(tc, align_up(T, 256));
    m->Tc = (int)tc;
    m->logits = (float*)D(tc * V * 4);
    m->dlogits = D(tc * V * E);
  }
  if (NE > 0) {
    m->mlogits = (float*)D(T * NE * 4);
    m->mcounts = (int32_t*)D((NE + 1) * 4);
    m->moffsets = (int32_t*)D((NE + 1) * 4);
    m->mperm = (int32_t*)D(moe_permute_scratch((int)T, (int)NE, m->topk) * 4);  // permutation scratch
    m->xp = D(Tk * H * E);
    m->ap = D(Tk * Fe * E);
    m->dyp = D(Tk * H * E);
    m->dap = D(Tk * Fe * E);
    m->dgup = D(Tk * 2 * Fe * E);
    m->dxp = (float*)D(Tk * H * 4);
    m->dwr = (float*)D(Tk * 4);
    m->dlogr = D(T * NE * E);
    m->route_rec = (int32_t*)D(L * Tk * 4);
  }
  if (m->R > 0) {
    m->lu = (float*)D(T * m->R * 4);
    m->lg = (float*)D(T * m->R * 4);
  }
  if (m->dt == DT_BF16) {
    m->wT = D(m->wT_bytes);
    const int64_t Tc64 = V > 0 ? m->Tc : 0;
    // transposed operands of the weight-gradient products run in the GEMM's NT layout (dgu^T is
    // written by the SwiGLU backward)
    const int64_t Tp = tpad(T), Tcp = tpad(Tc64);  // (padded rows)
    m->yT = D(std::max<int64_t>(Tp * std::max<int64_t>(2 * F, std::max<int64_t>(QKV, H)), Tcp * V) * 2);
    m->xT = D(std::max<int64_t>(Tp * std::max<int64_t>(F, std::max<int64_t>(nqd, H)), Tcp * H) * 2);
    if (V > 0) m->woutT = D(V * H * 2);
    m->qkvf = (float*)D(T * std::max<int64_t>(QKV, H) * 4);  // also the fp32 dO under LoRA
  }
  const int half = m->d / 2;
  m->cos_dev = (float*)D((int64_t)m->Smax * half * 4);
  m->sin_dev = (float*)D((int64_t)m->Smax * half * 4);
  if (st != HOL_OK) {
    engine_destroy(m);
    return st;
  }
  // RoPE tables: angle p * base^(-2j/d) in fp64, cos/sin rounded to fp32
  {
    std::vector<float> cs((size_t)m->Smax * half), sn((size_t)m->Smax * half);
    for (int p = 0; p < m->Smax; ++p)
      for (int j = 0; j < half; ++j) {
        const double th = pow((double)c.rope_base, -2.0 * j / m->d);
        const double ang = (double)p * th;
        cs[(size_t)p * half + j] = (float)cos(ang);
        sn[(size_t)p * half + j] = (float)sin(ang);
      }
    HCHECK(hipMemcpy(m->cos_dev, cs.data(), cs.size() * 4, hipMemcpyHostToDevice));
    HCHECK(hipMemcpy(m->sin_dev, sn.data(), sn.size() * 4, hipMemcpyHostToDevice));
  }
  HCHECK(hipStreamCreateWithFlags(&m->sc, hipStreamNonBlocking));
  HCHECK(hipStreamCreateWithFlags(&m->sh2d, hipStreamNonBlocking));
  HCHECK(hipStreamCreateWithFlags(&m->sd2h, hipStreamNonBlocking));
  for (int i = 0; i < m->nslots; ++i) {
    HCHECK(hipEventCreateWithFlags(&m->ev_ready[i], hipEventDisableTiming));
    HCHECK(hipEventCreateWithFlags(&m->ev_free[i], hipEventDisableTiming));
  }
  for (int i = 0; i < m->ngbuf; ++i) {
    HCHECK(hipEventCreateWithFlags(&m->ev_gdone[i], hipEventDisableTiming));
    HCHECK(hipEventCreateWithFlags(&m->ev_gfree[i], hipEventDisableTiming));
  }
  HCHECK(hipEventCreateWithFlags(&m->ev_head, hipEventDisableTiming));
  HCHECK(hipEventCreateWithFlags(&m->ev_head_done, hipEventDisableTiming));
  HCHECK(hipEventCreateWithFlags(&m->ev_head_pf, hipEventDisableTiming));
  for (int p = 0; p < hol_model::NPF; ++p) HCHECK(hipEventCreateWithFlags(&m->ev_lpf_done[p], hipEventDisableTiming));
  HCHECK(hipEventCreateWithFlags(&m->ev_h0, hipEventDisableTiming));
  for (auto& e : m->ev_tail) HCHECK(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  HCHECK(hipEventCreateWithFlags(&m->ev_wd_final, hipEventDisableTiming));
  HCHECK(hipEventCreateWithFlags(&m->ev_mlp_final, hipEventDisableTiming));
  m->ev_piece.resize(3 * (size_t)m->L);
  for (auto& e : m->ev_piece) HCHECK(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  for (int i = 0; i < m->nring; ++i) HCHECK(hipEventCreateWithFlags(&m->ring_ev[i], hipEventDisableTiming));
  m->unit_tensors.assign(m->L + 2, {});
  for (int i = 0; i < (int)m->tensors.size(); ++i) {
    const TensorDesc& t = m->tensors[i];
    const int u = t.block == -2 ? 0 : (t.block == -1 ? m->L + 1 : 1 + t.block);
    if (t.trainable) m->unit_tensors[u].push_back(i);
  }
  m->ev_unit.resize(m->L + 2);
  for (auto& e : m->ev_unit) HCHECK(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  // timing events: two per compute op, weight stream and gradient copy (at most ~14 L + 8)
  const int nt = 20 * m->L + 64;
  m->tev.resize(nt);
  for (int i = 0; i < nt; ++i) HCHECK(hipEventCreate(&m->tev[i]));
  *out = m;
  return HOL_OK;
}

void engine_destroy(hol_model* m) {
  if (!m) return;
  if (m->sc) hipStreamSynchronize(m->sc);
  if (m->sh2d) hipStreamSynchronize(m->sh2d);
  if (m->sd2h) hipStreamSynchronize(m->sd2h);
  for (int i = 0; i < hol_model::MAX_SLOTS; ++i) {
    if (m->ev_ready[i]) hipEventDestroy(m->ev_ready[i]);
    if (m->ev_free[i]) hipEventDestroy(m->ev_free[i]);
  }
  for (int i = 0; i < hol_model::MAX_GBUF; ++i) {
    if (m->ev_gdone[i]) hipEventDestroy(m->ev_gdone[i]);
    if (m->ev_gfree[i]) hipEventDestroy(m->ev_gfree[i]);
  }
  if (m->ev_head) hipEventDestroy(m->ev_head);
  if (m->ev_head_done) hipEventDestroy(m->ev_head_done);
  if (m->ev_head_pf) hipEventDestroy(m->ev_head_pf);
  for (int p = 0; p < hol_model::NPF; ++p)
    if (m->ev_lpf_done[p]) hipEventDestroy(m->ev_lpf_done[p]);
  if (m->ev_h0) hipEventDestroy(m->ev_h0);
  for (auto e : m->ev_tail)
    if (e) hipEventDestroy(e);
  if (m->ev_wd_final) hipEventDestroy(m->ev_wd_final);
  if (m->ev_mlp_final) hipEventDestroy(m->ev_mlp_final);
  for (auto e : m->ev_piece)
    if (e) hipEventDestroy(e);
  for (auto e : m->tev)
    if (e) hipEventDestroy(e);
  for (auto e : m->kev)
    if (e) hipEventDestroy(e);
  for (auto e : m->ev_unit)
    if (e) hipEventDestroy(e);
  if (m->sc) hipStreamDestroy(m->sc);
  if (m->sh2d) hipStreamDestroy(m->sh2d);
  if (m->sd2h) hipStreamDestroy(m->sd2h);
  for (void* p : m->dev_allocs) hipFree(p);
  for (void* p : m->pinned_allocs) hipHostFree(p);
  for (void* p : m->host_allocs) free(p);
  for (auto e : m->ring_ev)
    if (e) hipEventDestroy(e);
  free(m->master);
  free(m->mom1);
  free(m->mom2);
  delete m;
}

// ------------------------------------------------------------------------------------------
// image refresh (master -> low-precision copy)
// ------------------------------------------------------------------------------------------
// block of the image at `base` (m->image unless given)
static uint8_t* image_block(hol_model* m, int block, uint8_t* base = nullptr) {
  if (!base) base = m->image;
  return block >= 0 ? base + (int64_t)block * m->layer_img_bytes : base + (int64_t)m->L * m->layer_img_bytes;
}

// Queues the copy of `bytes` of the image at src into device memory at dst on the weight stream
// s (the caller holds h2d_mu). Pinned image: one DMA. Pinned ring: piece by piece, each piece
// copied by the host pool into the next ring segment once the DMA that last read that segment is
// done (its event; that DMA depends only on work queued before it), then one DMA from the segment.
static hipError_t image_h2d(hol_model* m, void* dst, const uint8_t* src, int64_t bytes, hipStream_t s) {
  if (m->nring == 0) return hipMemcpyAsync(dst, src, (size_t)bytes, hipMemcpyHostToDevice, s);
  for (int64_t off = 0; off < bytes; off += m->ring_seg) {
    const int64_t n = std::min<int64_t>(m->ring_seg, bytes - off);
    const int r = m->ring_next;
    m->ring_next = (r + 1) % m->nring;
    hipError_t e = hipEventSynchronize(m->ring_ev[r]);
    if (e != hipSuccess) return e;
    const double t0 = now_ms();
    uint8_t* seg = m->ring[r];
    const uint8_t* from = src + off;
    parallel_for(n, 1 << 22, [&](int64_t lo, int64_t hi) { memcpy(seg + lo, from + lo, (size_t)(hi - lo)); });
    m->stats.staging_ms += now_ms() - t0;
    m->stats.staged_bytes += (double)n;
    e = hipMemcpyAsync((uint8_t*)dst + off, seg, (size_t)n, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return e;
    e = hipEventRecord(m->ring_ev[r], s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

void refresh_image_tensor(hol_model* m, const TensorDesc& t) {
  if (t.flat >= 0) write_image_tensor(m, t, m->master + t.flat);
}

// Tensor values as the image holds them (fp32, or bf16 widened); for frozen tensors this is the
// only copy.
void read_image_tensor(const hol_model* m, const TensorDesc& t, float* dst) {
  const uint8_t* src = (t.block == -1 ? m->image + (int64_t)m->L * m->layer_img_bytes
                                      : m->image + (int64_t)t.block * m->layer_img_bytes) + t.img;
  if (t.img_f32 || m->dt == DT_F32) {
    parallel_for(t.numel, 1 << 18, [&](int64_t lo, int64_t hi) { memcpy(dst + lo, (const float*)src + lo, (hi - lo) * 4); });
  } else {
    parallel_for(t.numel, 1 << 18, [&](int64_t lo, int64_t hi) {
      const uint16_t* b = (const uint16_t*)src;
      for (int64_t i = lo; i < hi; ++i) {
        const uint32_t u = (uint32_t)b[i] << 16;
        memcpy(dst + i, &u, 4);
      }
    });
  }
}

// (into both images when the model has two: a frozen tensor's only copy must be in each)
void write_image_tensor(hol_model* m, const TensorDesc& t, const float* src) {
  if (t.block == -2 || t.img < 0) return;
  if (t.block == -1) m->head_img_ver++;
  if (t.block >= 0 && t.block < hol_model::NPF) m->lpf_img_ver[t.block]++;
  for (uint8_t* base : {m->image, m->image_alt}) {
    if (!base) continue;
    uint8_t* dst = image_block(m, t.block, base) + t.img;
    if (t.img_f32 || m->dt == DT_F32) {
      parallel_for(t.numel, 1 << 18, [&](int64_t lo, int64_t hi) { memcpy((float*)dst + lo, src + lo, (hi - lo) * 4); });
    } else {
      parallel_for(t.numel, 1 << 18,
                   [&](int64_t lo, int64_t hi) { f32_to_bf16_range(src + lo, (uint16_t*)dst + lo, hi - lo); });
    }
  }
}

// ------------------------------------------------------------------------------------------
// layer template: bind weights (slot pointers) and run kernels
// ------------------------------------------------------------------------------------------
struct W {
  const void *wqkv, *wo, *wgu, *wd;
  const float *g1, *g2;
  const void *router, *egate, *eup, *edown;  // mixture of experts
  const float *lA[4], *lB[4];                 // LoRA factors of q, k, v, o
};
static W bind(const hol_model* m, const uint8_t* slot) {
  W w{};
  w.wqkv = slot + m->o_wqkv;
  w.wo = slot + m->o_wo;
  w.wgu = slot + m->o_wgu;
  w.wd = slot + m->o_wd;
  w.g1 = (const float*)(slot + m->o_g1);
  w.g2 = (const float*)(slot + m->o_g2);
  w.router = slot + m->o_router;
  w.egate = slot + m->o_egate;
  w.eup = slot + m->o_eup;
  w.edown = slot + m->o_edown;
  for (int j = 0; j < 4; ++j) {
    w.lA[j] = (const float*)(slot + m->o_lA[j]);
    w.lB[j] = (const float*)(slot + m->o_lB[j]);
  }
  return w;
}

static Act act_at(const hol_model* m, int j) {
  uint8_t* b = m->act_mem + (int64_t)j * m->act_stride;
  Act a;
  a.hin = (float*)(b + m->ao_hin);
  a.r1 = (float*)(b + m->ao_r1);
  a.n1 = b + m->ao_n1;
  a.qkv = b + m->ao_qkv;
  a.o = b + m->ao_o;
  a.lse = (float*)(b + m->ao_lse);
  a.h1 = (float*)(b + m->ao_h1);
  a.r2 = (float*)(b + m->ao_r2);
  a.n2 = b + m->ao_n2;
  a.gu = b + m->ao_gu;
  a.a = b + m->ao_a;
  a.probs = (float*)(b + m->ao_probs);
  a.ids = (int32_t*)(b + m->ao_ids);
  a.w = (float*)(b + m->ao_w);
  a.slot_pos = (int32_t*)(b + m->ao_slot);
  a.perm_slot = (int32_t*)(b + m->ao_perm);
  a.gup = b + m->ao_gup;
  a.yp = (float*)(b + m->ao_yp);
  a.mtab = (int32_t*)(b + m->ao_mtab);
  return a;
}

// Runs `launch` on the compute stream; with kernel timing on, brackets it with events and
// records its class and algorithmic work.
template <typename F>
static int timed_shape(hol_model* m, int cls, double flops, double bytes, int gm, int gn, int gk, F&& launch) {
  if (!m->ktiming || (size_t)m->krec.size() * 2 + 2 > m->kev.size()) return launch();
  const int e = (int)m->krec.size() * 2;
  hipError_t r = hipEventRecord(m->kev[e], m->sc);
  if (r != hipSuccess) return (int)r;
  const int rc = launch();
  if (rc) return rc;
  r = hipEventRecord(m->kev[e + 1], m->sc);
  if (r != hipSuccess) return (int)r;
  m->krec.push_back({cls, e, flops, bytes, gm, gn, gk});
  return 0;
}

template <typename F>
static int timed(hol_model* m, int cls, double flops, double bytes, F&& launch) {
  return timed_shape(m, cls, flops, bytes, 0, 0, 0, launch);
}

static int run_gemm(hol_model* m, const Gemm& g) {
  const double E = (g.ab == DT_BF16) ? 2 : 4, Ec = (g.c == DT_BF16) ? 2 : 4;
  const double bytes = E * ((double)g.M * g.K + (double)g.N * g.K) + Ec * (double)g.M * g.N * (g.epi == EPI_STORE ? 1 : 2);
  return timed_shape(m, KC_GEMM, 2.0 * g.M * g.N * g.K * g.batch, bytes, g.M, g.N, g.K,
                     [&] { return launch_gemm(g, m->sc); });
}

// A weight-gradient product dW = dY^T X (K = tokens) of the dense bf16 backward: given the split
// workspace, a product whose tiles leave the last round of the grid part-empty splits those
// tiles along K (deterministic). Only these: a split changes the rounding with the token count,
// and every product over model dimensions must give each token's row the same bits whatever the
// batch it is in.
static int run_gemm_dw(hol_model* m, const Gemm& g0) {
  Gemm g = g0;
  g.ws = m->gemm_ws;
  g.ws_floats = m->gemm_ws ? GEMM_SPLIT_WS_FLOATS : 0;
  return run_gemm(m, g);
}

// the gate/up product with SwiGLU (launch_gemm_swiglu); a: [M, N/2] at row stride ld_a
static int run_gemm_swiglu(hol_model* m, const Gemm& g, void* a, int64_t ld_a) {
  const double E = (g.ab == DT_BF16) ? 2 : 4, Ec = (g.c == DT_BF16) ? 2 : 4;
  const double bytes = E * ((double)g.M * g.K + (double)g.N * g.K) + Ec * 1.5 * (double)g.M * g.N;
  return timed_shape(m, KC_GEMM, 2.0 * g.M * g.N * g.K, bytes, g.M, g.N, g.K,
                     [&] { return launch_gemm_swiglu(g, a, ld_a, m->sc); });
}

#define KT(cls, flops, bytes, expr) KCHECK(timed(m, cls, (double)(flops), (double)(bytes), [&] { return (expr); }))
#define STEP_OK(expr)               \
  do {                              \
    hol_status st__ = (expr);       \
    if (st__ != HOL_OK) return st__; \
  } while (0)

static Gemm gemm(int M, int N, int K, const void* A, int64_t lda, bool a_km, const void* B, int64_t ldb, bool b_kn,
                 void* C, int64_t ldc, DType ab, DType c, int epi, const float* R = nullptr, int64_t ldr = 0) {
  Gemm g;
  g.M = M; g.N = N; g.K = K;
  g.A = A; g.lda = lda; g.a_km = a_km;
  g.B = B; g.ldb = ldb; g.b_kn = b_kn;
  g.C = C; g.ldc = ldc; g.ab = ab; g.c = c; g.epi = epi; g.R = R; g.ldr = ldr;
  return g;
}

// Operands of different types (fp32 adapter factors against activations of the compute type).
static Gemm mixed(int M, int N, int K, const void* A, int64_t lda, bool a_km, DType at, const void* B, int64_t ldb,
                  bool b_kn, DType bt, void* C, int64_t ldc, int epi, float alpha) {
  Gemm g = gemm(M, N, K, A, lda, a_km, B, ldb, b_kn, C, ldc, at, DT_F32, epi);
  g.bt = bt;
  g.alpha = alpha;
  return g;
}

// LoRA branch of one projection (reading: y += s (x A^T) B^T, A [r, in], B [out, r], fp32):
// y is fp32 [T, out] at row stride ldy, x the projection's input in the compute type.
static hol_status lora_fwd(hol_model* m, const void* x, int64_t ldx, int in, int out, const float* A, const float* B,
                           float* y, int64_t ldy, int T) {
  const int r = m->R;
  KCHECK(run_gemm(m, mixed(T, r, in, x, ldx, false, m->dt, A, in, false, DT_F32, m->lu, r, EPI_STORE, 1.f)));
  KCHECK(run_gemm(m, mixed(T, out, r, m->lu, r, false, DT_F32, B, r, false, DT_F32, y, ldy, EPI_ACCUM,
                           m->cfg.lora_scale)));
  return HOL_OK;
}

// Its backward: u = x A^T, g = dy B; gB = s dy^T u, gA = s g^T x (stored), dx (fp32) += s g A.
static hol_status lora_bwd(hol_model* m, const void* dy, int64_t lddy, const void* x, int64_t ldx, int in, int out,
                           const float* A, const float* B, float* gA, float* gB, float* dx, int64_t lddx, int T) {
  const int r = m->R;
  const float sc = m->cfg.lora_scale;
  const DType dt = m->dt;
  KCHECK(run_gemm(m, mixed(T, r, in, x, ldx, false, dt, A, in, false, DT_F32, m->lu, r, EPI_STORE, 1.f)));
  KCHECK(run_gemm(m, mixed(out, r, T, dy, lddy, true, dt, m->lu, r, true, DT_F32, gB, r, EPI_STORE, sc)));
  KCHECK(run_gemm(m, mixed(T, r, out, dy, lddy, false, dt, B, r, true, DT_F32, m->lg, r, EPI_STORE, 1.f)));
  KCHECK(run_gemm(m, mixed(r, in, T, m->lg, r, true, DT_F32, x, ldx, true, dt, gA, in, EPI_STORE, sc)));
  KCHECK(run_gemm(m, mixed(T, in, r, m->lg, r, false, DT_F32, A, in, true, DT_F32, dx, lddx, EPI_ACCUM, sc)));
  return HOL_OK;
}

// One product over every expert's rows (grouped launch): C[rows of e] = A[rows of e] B_e^T with
// B_e = B + e sB elements; the group table of the activation-store position gives the rows.
static Gemm grouped(const hol_model* m, const Act& A, int64_t rows, int N, int K, const void* a, int64_t lda,
                    const void* b, int64_t ldb, int64_t sB, void* c, int64_t ldc, DType ct, int epi) {
  Gemm g = gemm((int)rows, N, K, a, lda, false, b, ldb, false, c, ldc, DT_BF16, ct, epi);
  g.grp = A.mtab;
  g.ngroups = m->NE;
  g.sB = sB;
  g.grp_max_rt = (int)((rows + (int64_t)m->NE * (GEMM_GROUP_BM - 1)) / GEMM_GROUP_BM);
  return g;
}

static int run_grouped(hol_model* m, const Gemm& g) {
  const double bytes = 2.0 * ((double)g.M * g.K + (double)g.ngroups * g.N * g.K) +
                       (g.c == DT_BF16 ? 2.0 : 4.0) * (double)g.M * g.N * (g.epi == EPI_STORE ? 1 : 2);
  return timed(m, KC_GEMM, 2.0 * g.M * g.N * g.K, bytes, [&] { return launch_gemm_grouped(g, m->sc); });
}

// Mixture-of-experts MLP: hout = h1 + sum_i w_i SwiGLU_{e_i}(n2). Routing, the permutation, the
// group table and the expert outputs go to the activation store. The expert products are grouped
// launches (bf16, 64-aligned widths) that read the row counts on the device; otherwise the host
// reads the counts into act_counts[pos] and launches one pair of products per expert, as it also
// does for the expert weight gradients.
static hol_status moe_forward(hol_model* m, const W& w, const Act& A, int T, float* hout, int pos) {
  const int H = m->H, NE = m->NE, k = m->topk, Fe = m->Fe;
  const DType dt = m->dt;
  const int64_t E = m->E, Tk = (int64_t)T * k;
  hipStream_t s = m->sc;
  KCHECK(run_gemm(m, gemm(T, NE, H, A.n2, H, false, w.router, H, false, m->mlogits, NE, dt, DT_F32, EPI_STORE)));
  KT(KC_OTHER, 0, (double)T * NE * 8, launch_moe_route(m->mlogits, T, NE, k, A.probs, A.ids, A.w, m->mcounts, s));
  KT(KC_OTHER, 0, (double)Tk * 16, launch_moe_permute(A.ids, T, NE, k, m->mcounts, m->moffsets, m->mperm,
                                                      A.perm_slot, A.slot_pos, s));
  if (m->moe_grp) KT(KC_OTHER, 0, (double)NE * 12, launch_gemm_group_table(m->mcounts, NE, A.mtab, s));
  if (!m->moe_grp || m->base_trainable) {
    HCHECK(hipMemcpyAsync(m->counts_stage, m->mcounts, (size_t)NE * 4, hipMemcpyDeviceToHost, s));
    HCHECK(hipStreamSynchronize(s));
    memcpy(m->act_counts[pos].data(), m->counts_stage, (size_t)NE * 4);
  }
  const std::vector<int32_t>& cnt = m->act_counts[pos];
  KT(KC_OTHER, 0, 2.0 * Tk * H * E, launch_moe_gather(A.n2, dt, A.perm_slot, k, Tk, H, m->xp, s));
  if (m->moe_grp) {
    KCHECK(run_grouped(m, grouped(m, A, Tk, Fe, H, m->xp, H, w.egate, H, (int64_t)Fe * H, A.gup, 2 * Fe, dt, EPI_STORE)));
    KCHECK(run_grouped(m, grouped(m, A, Tk, Fe, H, m->xp, H, w.eup, H, (int64_t)Fe * H, (uint8_t*)A.gup + Fe * E, 2 * Fe,
                                  dt, EPI_STORE)));
    KT(KC_SWIGLU, 0, 3.0 * Tk * Fe * E, launch_swiglu_fwd(A.gup, m->ap, dt, (int)Tk, Fe, s));
    KCHECK(run_grouped(m, grouped(m, A, Tk, H, Fe, m->ap, Fe, w.edown, Fe, (int64_t)H * Fe, A.yp, H, DT_F32, EPI_STORE)));
      if (hout)
      KT(KC_OTHER, 0, (double)T * H * 8 + (double)Tk * H * 4, launch_moe_combine(A.h1, A.yp, A.w, A.slot_pos, T, k, H, hout, s));
    return HOL_OK;
  }
  int64_t off = 0;
  for (int e = 0; e < NE; ++e) {
    const int me = cnt[e];
    if (me > 0) {
      const uint8_t* X = (const uint8_t*)m->xp + off * H * E;
      uint8_t* GU = (uint8_t*)A.gup + off * 2 * Fe * E;
      const int64_t wo = (int64_t)e * Fe * H * E;
      KCHECK(run_gemm(m, gemm(me, Fe, H, X, H, false, (const uint8_t*)w.egate + wo, H, false, GU, 2 * Fe, dt, dt, EPI_STORE)));
      KCHECK(run_gemm(m, gemm(me, Fe, H, X, H, false, (const uint8_t*)w.eup + wo, H, false, GU + Fe * E, 2 * Fe, dt, dt,
                              EPI_STORE)));
    }
    off += me;
  }
  KT(KC_SWIGLU, 0, 3.0 * Tk * Fe * E, launch_swiglu_fwd(A.gup, m->ap, dt, (int)Tk, Fe, s));
  off = 0;
  for (int e = 0; e < NE; ++e) {
    const int me = cnt[e];
    if (me > 0)
      KCHECK(run_gemm(m, gemm(me, H, Fe, (const uint8_t*)m->ap + off * Fe * E, Fe, false,
                              (const uint8_t*)w.edown + (int64_t)e * H * Fe * E, Fe, false, A.yp + off * H, H, dt, DT_F32,
                              EPI_STORE)));
    off += me;
  }
  if (hout)
    KT(KC_OTHER, 0, (double)T * H * 8 + (double)Tk * H * 4, launch_moe_combine(A.h1, A.yp, A.w, A.slot_pos, T, k, H, hout, s));
  return HOL_OK;
}

// Backward of moe_forward: m->dh holds d loss / d hout; writes dn = d loss / d n2 (fp32, stored)
// and, when the MoE weights train, their gradients into the layer block G.
static hol_status moe_backward(hol_model* m, const W& w, const Act& A, int T, float* G, int pos) {
  const int H = m->H, NE = m->NE, k = m->topk, Fe = m->Fe;
  const DType dt = m->dt;
  const int64_t E = m->E, Tk = (int64_t)T * k;
  hipStream_t s = m->sc;
  const std::vector<int32_t>& cnt = m->act_counts[pos];
  const bool tr_w = m->base_trainable, grp = m->moe_grp;
  const uint8_t* wt = (const uint8_t*)m->wT;
  KT(KC_OTHER, 0, (double)Tk * H * (4 + 4 + E), launch_moe_combine_bwd(m->dh, A.yp, A.w, A.slot_pos, T, k, H, m->dwr, m->dyp, dt, s));
  if (tr_w) KT(KC_SWIGLU, 0, 3.0 * Tk * Fe * E, launch_swiglu_fwd(A.gup, m->ap, dt, (int)Tk, Fe, s));
  // dA = dY W_down,e: B_e = (W_down,e)^T, columns e H .. e H + H - 1 of the stacked transpose
  if (grp)
    KCHECK(run_grouped(m, grouped(m, A, Tk, Fe, H, m->dyp, H, wt + m->t_edown, (int64_t)NE * H, H, m->dap, Fe, dt, EPI_STORE)));
  int64_t off = 0;
  for (int e = 0; e < NE; ++e) {
    const int me = grp && !tr_w ? 0 : cnt[e];
    const uint8_t* dY = (const uint8_t*)m->dyp + off * H * E;
    const uint8_t* Wd = (const uint8_t*)w.edown + (int64_t)e * H * Fe * E;
    if (me > 0 && !grp)
      KCHECK(run_gemm(m, gemm(me, Fe, H, dY, H, false, Wd, Fe, true, (uint8_t*)m->dap + off * Fe * E, Fe, dt, dt, EPI_STORE)));
    if (tr_w) {
      float* gWd = G + m->g_edown + (int64_t)e * H * Fe;
      if (me > 0) {
        Gemm g = gemm(H, Fe, me, dY, H, true, (const uint8_t*)m->ap + off * Fe * E, Fe, true, gWd, Fe, dt, DT_F32, EPI_STORE);
        g.any_align = true;
        KCHECK(run_gemm(m, g));
      } else {
        KCHECK(launch_fill_f32(gWd, 0.f, (int64_t)H * Fe, s));
      }
    }
    off += me;
  }
  KT(KC_SWIGLU, 0, 5.0 * Tk * Fe * E, launch_swiglu_bwd(m->dap, A.gup, m->dgup, dt, (int)Tk, Fe, s));
  if (tr_w) KT(KC_OTHER, 0, 2.0 * Tk * H * E, launch_moe_gather(A.n2, dt, A.perm_slot, k, Tk, H, m->xp, s));
  // dX = dG W_gate,e + dU W_up,e: B_e = (W_gate,e)^T, columns e Fe .. e Fe + Fe - 1 of [H, E Fe]
  if (grp) {
    KCHECK(run_grouped(m, grouped(m, A, Tk, H, Fe, m->dgup, 2 * Fe, wt + m->t_egate, (int64_t)NE * Fe, Fe, m->dxp, H,
                                  DT_F32, EPI_STORE)));
    KCHECK(run_grouped(m, grouped(m, A, Tk, H, Fe, (const uint8_t*)m->dgup + Fe * E, 2 * Fe, wt + m->t_eup, (int64_t)NE * Fe,
                                  Fe, m->dxp, H, DT_F32, EPI_ACCUM)));
  }
  off = 0;
  for (int e = 0; e < NE; ++e) {
    const int me = grp && !tr_w ? 0 : cnt[e];
    const uint8_t* dGU = (const uint8_t*)m->dgup + off * 2 * Fe * E;
    const int64_t wo = (int64_t)e * Fe * H * E;
    if (me > 0 && !grp) {
      KCHECK(run_gemm(m, gemm(me, H, Fe, dGU, 2 * Fe, false, (const uint8_t*)w.egate + wo, H, true, m->dxp + off * H, H, dt,
                              DT_F32, EPI_STORE)));
      KCHECK(run_gemm(m, gemm(me, H, Fe, dGU + Fe * E, 2 * Fe, false, (const uint8_t*)w.eup + wo, H, true, m->dxp + off * H,
                              H, dt, DT_F32, EPI_ACCUM)));
    }
    if (tr_w) {
      float* gG = G + m->g_egate + (int64_t)e * Fe * H;
      float* gU = G + m->g_eup + (int64_t)e * Fe * H;
      if (me > 0) {
        const uint8_t* X = (const uint8_t*)m->xp + off * H * E;
        Gemm g1 = gemm(Fe, H, me, dGU, 2 * Fe, true, X, H, true, gG, H, dt, DT_F32, EPI_STORE);
        Gemm g2 = gemm(Fe, H, me, dGU + Fe * E, 2 * Fe, true, X, H, true, gU, H, dt, DT_F32, EPI_STORE);
        g1.any_align = g2.any_align = true;
        KCHECK(run_gemm(m, g1));
        KCHECK(run_gemm(m, g2));
      } else {
        KCHECK(launch_fill_f32(gG, 0.f, (int64_t)Fe * H, s));
        KCHECK(launch_fill_f32(gU, 0.f, (int64_t)Fe * H, s));
      }
    }
    off += me;
  }
  KT(KC_OTHER, 0, (double)Tk * H * 4 + (double)T * H * 4, launch_moe_unpermute(m->dxp, A.slot_pos, T, k, H, m->dn, s));
  // router: dn += dlogits W_r, dW_r = dlogits^T n2
  KT(KC_OTHER, 0, (double)T * NE * 8, launch_moe_router_bwd(A.probs, A.ids, A.w, m->dwr, T, NE, k, m->dlogr, dt, s));
  {
    Gemm g = gemm(T, H, NE, m->dlogr, NE, false, w.router, H, true, m->dn, H, dt, DT_F32, EPI_ACCUM);
    g.any_align = true;
    KCHECK(run_gemm(m, g));
  }
  if (tr_w) {
    Gemm g = gemm(NE, H, T, m->dlogr, NE, true, A.n2, H, true, G + m->g_router, H, dt, DT_F32, EPI_STORE);
    g.any_align = true;
    KCHECK(run_gemm(m, g));
  }
  return HOL_OK;
}

static hol_status layer_forward(hol_model* m, const W& w, const float* hin, float* hout, const Act& A, int T,
                                int n_seq, int S, int pos) {
  const int H = m->H, QKV = m->QKV, nqd = m->nqd, F = m->F, d = m->d, kvd = m->nkv * m->d;
  const DType dt = m->dt;
  const int64_t E = m->E;
  hipStream_t s = m->sc;
  KT(KC_RMSNORM, 0, (double)T * H * (4 + E), launch_rmsnorm_fwd(hin, w.g1, m->cfg.rms_eps, A.n1, dt, A.r1, T, H, s));
  // q/k/v projection and RoPE. bf16 without adapters: one product with RoPE in its epilogue, each
  // value rounded once. Otherwise an fp32 product (to which the adapters add), then RoPE with the
  // single bf16 rounding.
  const int nrot = (m->nq + m->nkv) * d;
  const Gemm gq = gemm(T, QKV, H, A.n1, H, false, w.wqkv, H, false, A.qkv, QKV, dt, dt, EPI_STORE);
  if (dt == DT_BF16 && m->R == 0 && d == 128 && gemm_rope_supported(gq, nrot, m->cos_dev, m->sin_dev)) {
    KCHECK(timed_shape(m, KC_GEMM, 2.0 * T * QKV * H, 2.0 * ((double)T * H + (double)QKV * H + (double)T * QKV), T, QKV,
                       H, [&] { return launch_gemm_rope(gq, nrot, S, m->cos_dev, m->sin_dev, s); }));
  } else {
    // fp32 q | k | v projection output (the bf16 path rounds once, after RoPE)
    float* qkv32 = dt == DT_BF16 ? m->qkvf : (float*)A.qkv;
    KCHECK(run_gemm(m, gemm(T, QKV, H, A.n1, H, false, w.wqkv, H, false, qkv32, QKV, dt, DT_F32, EPI_STORE)));
    if (m->R > 0) {
      const int c0[3] = {0, nqd, nqd + kvd}, outd[3] = {nqd, kvd, kvd};
      for (int j = 0; j < 3; ++j)
        STEP_OK(lora_fwd(m, A.n1, H, H, outd[j], w.lA[j], w.lB[j], qkv32 + c0[j], QKV, T));
    }
    if (dt == DT_BF16) {
      KT(KC_ROPE, 0, (double)T * QKV * (4 + E), launch_rope_qkv(m->qkvf, QKV, A.qkv, QKV, T, m->nq, m->nkv, d, S,
                                                                m->cos_dev, m->sin_dev, s));
    } else {
      KT(KC_ROPE, 0, 2.0 * T * nqd * E, launch_rope(A.qkv, dt, QKV, T, m->nq, d, S, m->cos_dev, m->sin_dev, false, s));
      KT(KC_ROPE, 0, 2.0 * T * m->nkv * d * E, launch_rope((uint8_t*)A.qkv + (int64_t)nqd * E, dt, QKV, T, m->nkv, d, S, m->cos_dev, m->sin_dev, false, s));
    }
  }
  Attn at;
  at.n_seq = n_seq; at.S = S; at.nq = m->nq; at.nkv = m->nkv; at.d = d; at.t = dt;
  at.q = A.qkv; at.k = (uint8_t*)A.qkv + (int64_t)nqd * E; at.v = (uint8_t*)A.qkv + (int64_t)(nqd + m->nkv * d) * E;
  at.ldq = at.ldk = at.ldv = QKV;
  at.o = A.o; at.ldo = nqd; at.lse = A.lse;
  KT(KC_ATTN_FWD, 2.0 * d * m->nq * (double)S * (S + 1) * n_seq, (double)T * (QKV + nqd) * E, launch_attn_fwd(at, s));
  KCHECK(run_gemm(m, gemm(T, H, nqd, A.o, nqd, false, w.wo, nqd, false, A.h1, H, dt, DT_F32, EPI_RESID, hin, H)));
  if (m->R > 0) STEP_OK(lora_fwd(m, A.o, nqd, nqd, H, w.lA[3], w.lB[3], A.h1, H, T));
  KT(KC_RMSNORM, 0, (double)T * H * (4 + E), launch_rmsnorm_fwd(A.h1, w.g2, m->cfg.rms_eps, A.n2, dt, A.r2, T, H, s));
  if (m->NE > 0) return moe_forward(m, w, A, T, hout, pos);
  // gate/up product with SwiGLU in its epilogue (one kernel for bf16 with F % 32 == 0; else the
  // product and the element-wise kernel, timed together as one GEMM record)
  KCHECK(run_gemm_swiglu(m, gemm(T, 2 * F, H, A.n2, H, false, w.wgu, H, false, A.gu, 2 * F, dt, dt, EPI_STORE), A.a, F));
  if (hout)  // (null: the output is not needed, see the recompute)
    KCHECK(run_gemm(m, gemm(T, H, F, A.a, F, false, w.wd, F, false, hout, H, dt, DT_F32, EPI_RESID, A.h1, H)));
  return HOL_OK;
}

// out[c][r] = in[r][c] (bf16)
static int tr(hol_model* m, const void* in, int64_t ldi, void* out, int64_t ldo, int R, int C) {
  return timed(m, KC_TRANSPOSE, 0, 4.0 * R * C, [&] { return launch_transpose_bf16(in, ldi, out, ldo, R, C, m->sc); });
}

// C[M,N] = A[M,K] B[N,K]^T with both operands K-contiguous (the fast NT kernel)
static Gemm nt(int M, int N, int K, const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
               DType c, int epi = EPI_STORE) {
  Gemm g;
  g.M = M; g.N = N; g.K = K;
  g.A = A; g.lda = lda; g.B = B; g.ldb = ldb;
  g.C = C; g.ldc = ldc; g.ab = DT_BF16; g.c = c; g.epi = epi;
  return g;
}

// Whether a weight gradient Y^T X of token-major bf16 activations Y [T, M], X [T, N] can run in
// the GEMM's TN layout, reading both as stored (K = T a multiple of 64, 16-byte rows and bases,
// byte offsets within 32 bits).
static bool dw_tn_ok(int M, int N, int T, const void* Y, int64_t ldy, const void* X, int64_t ldx) {
  return T % 64 == 0 && M % 8 == 0 && N % 8 == 0 && ldy % 8 == 0 && ldx % 8 == 0 &&
         (((uintptr_t)Y | (uintptr_t)X) % 16) == 0 && (uint64_t)T * ldy * 2 < (1ull << 32) &&
         (uint64_t)T * ldx * 2 < (1ull << 32);
}

// G [M, N] (fp32, row stride ldg) = Y^T X: the TN layout when asked for (tn) and dw_tn_ok, else
// both operands transposed into yT / xT for the NT layout (the same products, bit for bit, and
// the same split tail). The TN layout reads each fragment with two transposing LDS reads instead
// of one, and runs 7-24 % slower than NT on the LLaMA-8B weight-gradient shapes; it pays where
// the two transposes cost more than that (the o and q/k/v products: 2 x 134 MB and 201 + 134 MB
// transposed for 0.5-0.7 ms products), not for w_down, w_gate|w_up or the LM head.
static int dw_bf16(hol_model* m, int M, int N, int T, const void* Y, int64_t ldy, const void* X, int64_t ldx, float* G,
                   int64_t ldg, bool tn) {
  if (tn && dw_tn_ok(M, N, T, Y, ldy, X, ldx))
    return run_gemm_dw(m, gemm(M, N, T, Y, ldy, true, X, ldx, true, G, ldg, DT_BF16, DT_F32, EPI_STORE));
  const int64_t lt = tpad(T);
  int e = tr(m, Y, ldy, m->yT, lt, T, M);
  if (!e) e = tr(m, X, ldx, m->xT, lt, T, N);
  if (!e) e = run_gemm_dw(m, nt(M, N, T, m->yT, lt, m->xT, lt, G, ldg, DT_F32));
  return e;
}

// Transposes the resident layer's weights into m->wT (same sub-tensor offsets as the slot):
// Wqkv^T [H, QKV], Wo^T [nqd, H], and for a dense MLP Wgu^T [H, 2F], Wd^T [F, H].
static hol_status transpose_layer_weights(hol_model* m, const W& w) {
  const int H = m->H, QKV = m->QKV, nqd = m->nqd, F = m->F;
  uint8_t* t = (uint8_t*)m->wT;
  KCHECK(tr(m, w.wqkv, H, t + m->o_wqkv, QKV, QKV, H));
  KCHECK(tr(m, w.wo, nqd, t + m->o_wo, H, H, nqd));
  if (m->moe_grp) {
    const int NE = m->NE, Fe = m->Fe;
    KCHECK(tr(m, w.egate, H, t + m->t_egate, NE * Fe, NE * Fe, H));  // [E Fe, H] -> [H, E Fe]
    KCHECK(tr(m, w.eup, H, t + m->t_eup, NE * Fe, NE * Fe, H));
    KCHECK(tr(m, w.edown, Fe, t + m->t_edown, NE * H, NE * H, Fe));  // [E H, Fe] -> [Fe, E H]
  }
  if (m->NE > 0) return HOL_OK;
  KCHECK(tr(m, w.wgu, H, t + m->o_wgu, 2 * F, 2 * F, H));
  KCHECK(tr(m, w.wd, F, t + m->o_wd, H, H, F));
  return HOL_OK;
}

// bf16 backward: identical dataflow to layer_backward, every dense product as NT. Frozen base
// weights (LoRA) get no gradient products; the adapters' products run in fp32.
static hol_status layer_backward_bf16(hol_model* m, const W& w, const Act& A, const float* hin, float* G, int T,
                                      int n_seq, int S, int pos) {
  const int H = m->H, QKV = m->QKV, nqd = m->nqd, F = m->F, d = m->d, kvd = m->nkv * m->d;
  const DType dt = DT_BF16;
  const int64_t E = 2;
  const bool tw = m->base_trainable;
  hipStream_t s = m->sc;
  const uint8_t* wt = (const uint8_t*)m->wT;
  const void* WqkvT = wt + m->o_wqkv;  // [H, QKV]
  const void* WoT = wt + m->o_wo;      // [nqd, H]
  const void* WguT = wt + m->o_wgu;    // [H, 2F]
  const void* WdT = wt + m->o_wd;      // [F, H]
  STEP_OK(transpose_layer_weights(m, w));
  if (m->NE > 0) {
    STEP_OK(moe_backward(m, w, A, T, G, pos));
  } else {
    // MLP: da = dh Wd, dWd = dh^T a (dhb is normally written with dh by the RMSNorm backward
    // above this layer)
    if (!m->dhb_current)
      KT(KC_OTHER, 0, (double)T * H * (4 + E), launch_cast_f32(m->dh, m->dhb, dt, (int64_t)T * H, s));
    m->dhb_current = true;
    KCHECK(run_gemm(m, nt(T, F, H, m->dhb, H, WdT, H, m->da, F, dt)));
    if (tw) {
      KCHECK(dw_bf16(m, H, F, T, m->dhb, H, A.a, F, G + m->g_wd, F, false));  // dWd = dh^T a
      if (m->pieces_armed) HCHECK(hipEventRecord(m->ev_wd_final, s));  // w_down final
    }
    // (with weight gradients the SwiGLU backward also writes dgu^T for the dWgu product)
    const bool dgu_t = tw && F % 64 == 0;
    if (dgu_t)
      KT(KC_SWIGLU, 0, 7.0 * T * F * E, launch_swiglu_bwd_tr(m->da, A.gu, m->dgu, m->yT, tpad(T), T, F, s));
    else
      KT(KC_SWIGLU, 0, 5.0 * T * F * E, launch_swiglu_bwd(m->da, A.gu, m->dgu, dt, T, F, s));
    // dn2 = dgu Wgu, dWgu = dgu^T n2
    KCHECK(run_gemm(m, nt(T, H, 2 * F, m->dgu, 2 * F, WguT, 2 * F, m->dn, H, DT_F32)));
    if (tw) {
      if (!dgu_t) KCHECK(tr(m, m->dgu, 2 * F, m->yT, tpad(T), T, 2 * F));
      KCHECK(tr(m, A.n2, H, m->xT, tpad(T), T, H));
      KCHECK(run_gemm_dw(m, nt(2 * F, H, T, m->yT, tpad(T), m->xT, tpad(T), G + m->g_wgu, H, DT_F32)));
    }
    if (m->pieces_armed) HCHECK(hipEventRecord(m->ev_mlp_final, s));  // w_gate, w_up final
  }
  if (tw) KCHECK(launch_fill_f32(G + m->g_g1, 0.f, 2 * (int64_t)H, s));
  // (the RMSNorm backward also writes dh rounded to bf16 into dhb)
  KT(KC_RMSNORM, 0, (16.0 + E) * T * H, launch_rmsnorm_bwd(m->dn, A.h1, w.g2, A.r2, m->dh, true,
                                                             tw ? G + m->g_g2 : nullptr, m->partial, T, H, s, m->dhb));
  // attention output projection: dO = dh1 Wo (+ LoRA), dWo = dh1^T o
  if (m->R > 0) {
    float* dO32 = m->qkvf;  // fp32 [T, nqd]
    KCHECK(run_gemm(m, nt(T, nqd, H, m->dhb, H, WoT, H, dO32, nqd, DT_F32)));
    STEP_OK(lora_bwd(m, m->dhb, H, A.o, nqd, nqd, H, w.lA[3], w.lB[3], G + m->g_lA[3], G + m->g_lB[3], dO32, nqd, T));
    KT(KC_OTHER, 0, (double)T * nqd * (4 + E), launch_cast_f32(dO32, m->dO, dt, (int64_t)T * nqd, s));
  } else {
    KCHECK(run_gemm(m, nt(T, nqd, H, m->dhb, H, WoT, H, m->dO, nqd, dt)));
  }
  if (tw) KCHECK(dw_bf16(m, H, nqd, T, m->dhb, H, A.o, nqd, G + m->g_wo, nqd, true));  // dWo = dh1^T o
  Attn at;
  at.n_seq = n_seq; at.S = S; at.nq = m->nq; at.nkv = m->nkv; at.d = d; at.t = dt;
  at.q = A.qkv; at.k = (uint8_t*)A.qkv + (int64_t)nqd * E; at.v = (uint8_t*)A.qkv + (int64_t)(nqd + m->nkv * d) * E;
  at.ldq = at.ldk = at.ldv = QKV;
  at.o = A.o; at.ldo = nqd; at.lse = A.lse;
  at.dO = m->dO; at.lddo = nqd;
  at.dq = m->dqkv; at.dk = (uint8_t*)m->dqkv + (int64_t)nqd * E; at.dv = (uint8_t*)m->dqkv + (int64_t)(nqd + m->nkv * d) * E;
  at.lddq = at.lddk = at.lddv = QKV;
  at.delta = m->delta;
  at.rope_cos = m->cos_dev;  // dq and dk leave with the RoPE backward applied
  at.rope_sin = m->sin_dev;
  KT(KC_ATTN_BWD, 5.0 * d * m->nq * (double)S * (S + 1) * n_seq, (double)T * (2 * QKV + 3 * nqd) * E, launch_attn_bwd(at, s));
  // q/k/v projections: dn1 = dqkv Wqkv (+ LoRA), dWqkv = dqkv^T n1
  KCHECK(run_gemm(m, nt(T, H, QKV, m->dqkv, QKV, WqkvT, QKV, m->dn, H, DT_F32)));
  if (m->R > 0) {
    const int c0[3] = {0, nqd, nqd + kvd}, outd[3] = {nqd, kvd, kvd};
    for (int j = 0; j < 3; ++j)
      STEP_OK(lora_bwd(m, (const uint8_t*)m->dqkv + (int64_t)c0[j] * E, QKV, A.n1, H, H, outd[j], w.lA[j], w.lB[j],
                       G + m->g_lA[j], G + m->g_lB[j], m->dn, H, T));
  }
  if (tw) KCHECK(dw_bf16(m, QKV, H, T, m->dqkv, QKV, A.n1, H, G + m->g_wqkv, H, true));  // dWqkv = dqkv^T n1
  KT(KC_RMSNORM, 0, (16.0 + E) * T * H, launch_rmsnorm_bwd(m->dn, hin, w.g1, A.r1, m->dh, true,
                                                             tw ? G + m->g_g1 : nullptr, m->partial, T, H, s, m->dhb));
  m->dhb_current = true;
  return HOL_OK;
}

// dh (fp32 [T,H]) holds d loss / d h_out on entry and d loss / d h_in on exit; G is the layer's
// gradient block (fully overwritten).
static hol_status layer_backward(hol_model* m, const W& w, const Act& A, const float* hin, float* G, int T, int n_seq,
                                 int S, int pos) {
  if (m->dt == DT_BF16) return layer_backward_bf16(m, w, A, hin, G, T, n_seq, S, pos);
  const int H = m->H, QKV = m->QKV, nqd = m->nqd, F = m->F, d = m->d, kvd = m->nkv * m->d;
  const DType dt = m->dt;
  const int64_t E = m->E;
  const bool tw = m->base_trainable;
  hipStream_t s = m->sc;
  // MLP
  if (m->NE > 0) {
    STEP_OK(moe_backward(m, w, A, T, G, pos));
  } else {
    KT(KC_OTHER, 0, (double)T * H * (4 + E), launch_cast_f32(m->dh, m->dhb, dt, (int64_t)T * H, s));
    KCHECK(run_gemm(m, gemm(T, F, H, m->dhb, H, false, w.wd, F, true, m->da, F, dt, dt, EPI_STORE)));
    if (tw) KCHECK(run_gemm(m, gemm(H, F, T, m->dhb, H, true, A.a, F, true, G + m->g_wd, F, dt, DT_F32, EPI_STORE)));
    KT(KC_SWIGLU, 0, 5.0 * T * F * E, launch_swiglu_bwd(m->da, A.gu, m->dgu, dt, T, F, s));
    KCHECK(run_gemm(m, gemm(T, H, 2 * F, m->dgu, 2 * F, false, w.wgu, H, true, m->dn, H, dt, DT_F32, EPI_STORE)));
    if (tw) KCHECK(run_gemm(m, gemm(2 * F, H, T, m->dgu, 2 * F, true, A.n2, H, true, G + m->g_wgu, H, dt, DT_F32, EPI_STORE)));
  }
  if (tw) KCHECK(launch_fill_f32(G + m->g_g1, 0.f, 2 * (int64_t)H, s));
  KT(KC_RMSNORM, 0, 16.0 * T * H, launch_rmsnorm_bwd(m->dn, A.h1, w.g2, A.r2, m->dh, true, tw ? G + m->g_g2 : nullptr,
                                                      m->partial, T, H, s));
  // attention
  KT(KC_OTHER, 0, (double)T * H * (4 + E), launch_cast_f32(m->dh, m->dhb, dt, (int64_t)T * H, s));
  KCHECK(run_gemm(m, gemm(T, nqd, H, m->dhb, H, false, w.wo, nqd, true, m->dO, nqd, dt, dt, EPI_STORE)));
  if (m->R > 0)
    STEP_OK(lora_bwd(m, m->dhb, H, A.o, nqd, nqd, H, w.lA[3], w.lB[3], G + m->g_lA[3], G + m->g_lB[3], (float*)m->dO,
                     nqd, T));
  if (tw) KCHECK(run_gemm(m, gemm(H, nqd, T, m->dhb, H, true, A.o, nqd, true, G + m->g_wo, nqd, dt, DT_F32, EPI_STORE)));
  Attn at;
  at.n_seq = n_seq; at.S = S; at.nq = m->nq; at.nkv = m->nkv; at.d = d; at.t = dt;
  at.q = A.qkv; at.k = (uint8_t*)A.qkv + (int64_t)nqd * E; at.v = (uint8_t*)A.qkv + (int64_t)(nqd + m->nkv * d) * E;
  at.ldq = at.ldk = at.ldv = QKV;
  at.o = A.o; at.ldo = nqd; at.lse = A.lse;
  at.dO = m->dO; at.lddo = nqd;
  at.dq = m->dqkv; at.dk = (uint8_t*)m->dqkv + (int64_t)nqd * E; at.dv = (uint8_t*)m->dqkv + (int64_t)(nqd + m->nkv * d) * E;
  at.lddq = at.lddk = at.lddv = QKV;
  at.delta = m->delta;
  KT(KC_ATTN_BWD, 5.0 * d * m->nq * (double)S * (S + 1) * n_seq, (double)T * (2 * QKV + 3 * nqd) * E, launch_attn_bwd(at, s));
  KT(KC_ROPE, 0, 2.0 * T * nqd * E, launch_rope(m->dqkv, dt, QKV, T, m->nq, d, S, m->cos_dev, m->sin_dev, true, s));
  KT(KC_ROPE, 0, 2.0 * T * m->nkv * d * E, launch_rope((uint8_t*)m->dqkv + (int64_t)nqd * E, dt, QKV, T, m->nkv, d, S, m->cos_dev, m->sin_dev, true, s));
  KCHECK(run_gemm(m, gemm(T, H, QKV, m->dqkv, QKV, false, w.wqkv, H, true, m->dn, H, dt, DT_F32, EPI_STORE)));
  if (m->R > 0) {
    const int c0[3] = {0, nqd, nqd + kvd}, outd[3] = {nqd, kvd, kvd};
    for (int j = 0; j < 3; ++j)
      STEP_OK(lora_bwd(m, (const uint8_t*)m->dqkv + (int64_t)c0[j] * E, QKV, A.n1, H, H, outd[j], w.lA[j], w.lB[j],
                       G + m->g_lA[j], G + m->g_lB[j], m->dn, H, T));
  }
  if (tw) KCHECK(run_gemm(m, gemm(QKV, H, T, m->dqkv, QKV, true, A.n1, H, true, G + m->g_wqkv, H, dt, DT_F32, EPI_STORE)));
  KT(KC_RMSNORM, 0, 16.0 * T * H, launch_rmsnorm_bwd(m->dn, hin, w.g1, A.r1, m->dh, true, tw ? G + m->g_g1 : nullptr,
                                                      m->partial, T, H, s));
  return HOL_OK;
}

// Loss anchor (phase 2): loss rows, head gradient into head_gdev, d loss / d h_L into m->dh.
static hol_status head_forward_backward(hol_model* m, const float* hL, int T, hol_loss loss) {
  hipStream_t s = m->sc;
  const int H = m->H;
  if (loss == HOL_LOSS_SUM_SQUARES) {
    KT(KC_OTHER, 0, 8.0 * T * H, launch_sumsq(hL, m->rowloss_dev, m->dh, T, H, s));
    m->dhb_current = false;
    return HOL_OK;
  }
  const int V = m->V;
  const DType dt = m->dt;
  const int64_t E = m->E;
  const float* gf = (const float*)(m->head_dev + m->o_gf);
  const void* wout = m->head_dev + m->o_wout;
  KT(KC_RMSNORM, 0, (double)T * H * (4 + E), launch_rmsnorm_fwd(hL, gf, m->cfg.rms_eps, m->zbuf, dt, m->rz, T, H, s));
  const bool ht = m->head_trainable;  // frozen under LoRA: no W_out / final-norm gradient
  float* gW = ht ? m->head_gdev + H : nullptr;
  if (dt == DT_BF16) KCHECK(tr(m, wout, H, m->woutT, V, V, H));  // W_out^T [H, V]
  for (int r0 = 0; r0 < T; r0 += m->Tc) {
    const int tc = std::min(m->Tc, T - r0);
    const void* zc = (const uint8_t*)m->zbuf + (int64_t)r0 * H * E;
    KCHECK(run_gemm(m, gemm(tc, V, H, zc, H, false, wout, H, false, m->logits, V, dt, DT_F32, EPI_STORE)));
    if (dt == DT_BF16) {
      KT(KC_CE, 0, (double)tc * V * (4 + E), launch_ce_fwd_bwd(m->logits, V, m->labels_dev + r0, m->w_dev + r0,
                                                               m->rowloss_dev + r0, m->dlogits, dt, V, tc, V, s));
      KCHECK(run_gemm(m, nt(tc, H, V, m->dlogits, V, m->woutT, V, m->dn + (int64_t)r0 * H, H, DT_F32)));
      if (!ht) continue;
      KCHECK(tr(m, m->dlogits, V, m->yT, tpad(tc), tc, V));   // dlogits^T [V, tc]
      KCHECK(tr(m, zc, H, m->xT, tpad(tc), tc, H));           // z^T [H, tc]
      KCHECK(run_gemm(m, nt(V, H, tc, m->yT, tpad(tc), m->xT, tpad(tc), gW, H, DT_F32, r0 == 0 ? EPI_STORE : EPI_ACCUM)));
      continue;
    }
    KT(KC_CE, 0, (double)tc * V * (4 + E), launch_ce_fwd_bwd(m->logits, V, m->labels_dev + r0, m->w_dev + r0,
                                                             m->rowloss_dev + r0, m->dlogits, dt, V, tc, V, s));
    KCHECK(run_gemm(m, gemm(tc, H, V, m->dlogits, V, false, wout, H, true, m->dn + (int64_t)r0 * H, H, dt, DT_F32,
                            EPI_STORE)));
    if (ht)
      KCHECK(run_gemm(m, gemm(V, H, tc, m->dlogits, V, true, zc, H, true, gW, H, dt, DT_F32,
                              r0 == 0 ? EPI_STORE : EPI_ACCUM)));
  }
  if (ht) KCHECK(launch_fill_f32(m->head_gdev, 0.f, H, s));
  void* dhb = dt == DT_BF16 ? m->dhb : nullptr;  // (bf16: the layer below reads dh rounded)
  KT(KC_RMSNORM, 0, (12.0 + (dhb ? 2 : 0)) * T * H,
     launch_rmsnorm_bwd(m->dn, hL, gf, m->rz, m->dh, false, ht ? m->head_gdev : nullptr, m->partial, T, H, s, dhb));
  m->dhb_current = dhb != nullptr;
  return HOL_OK;
}

// ------------------------------------------------------------------------------------------
// forward_backward
// ------------------------------------------------------------------------------------------
struct AccumJob {
  float* dst;
  const float* src;
  int64_t n;
};
static void host_accumulate(void* p) {
  AccumJob* j = (AccumJob*)p;
  parallel_for(j->n, 1 << 16, [&](int64_t lo, int64_t hi) {
    for (int64_t i = lo; i < hi; ++i) j->dst[i] += j->src[i];
  });
}

static void adam_unit(hol_model* m, int u, const AdamConsts& k, int64_t lo = -1, int64_t hi = -1, bool zero = true,
                      float* gbase = nullptr, uint8_t* ibase = nullptr);
static void adam_embed_rows(hol_model* m, const std::vector<int32_t>& rows, const AdamConsts& k, bool zero = true,
                            const float* gsrc = nullptr);

// Waits for an event by polling it. A blocking wait (hipEventSynchronize) on an event still
// pending when it was called returned ≈8 ms after the copy it marks had finished, which the
// optimiser thread paid at the first unit of every block.
static hipError_t wait_event(hipEvent_t ev) {
  for (;;) {
    const hipError_t e = hipEventQuery(ev);
    if (e != hipErrorNotReady) return e;
    std::this_thread::sleep_for(std::chrono::microseconds(50));
  }
}

// Host worker of the fused forward_backward + step: runs the optimiser on each unit as soon as
// that unit's gradient copy (enqueued by the main thread, in backward order) has completed.
struct FusedWorker {
  hol_model* m;
  std::thread th;
  bool running = false;
  bool failed = false;
  bool prefetched = false;  // the next call's head weights were sent
  int lpf_sent = 0;         // first layers of the next call sent
  int tail_done = 0;        // optimiser pieces of the last layer done
  double busy_ms = 0;
  double t_call = 0;
  void start(const AdamConsts& kc, double t_start) {
    t_call = t_start;
    {
      std::lock_guard<std::mutex> g(m->fmu);
      m->unit_queue.clear();
      m->pjobs.clear();
      m->fused_abort = false;
    }
    running = true;
    th = std::thread([this, kc] {
      (void)hipSetDevice(m->cfg.device);
      size_t next = 0;
      for (;;) {
        int u;
        hol_model::PieceJob job{};
        {
          std::unique_lock<std::mutex> lk(m->fmu);
          m->fcv.wait(lk, [&] { return m->fused_abort || next < m->unit_queue.size(); });
          if (m->fused_abort) return;
          u = m->unit_queue[next++];
          if (u >= hol_model::PIECE_CODE) job = m->pjobs[u - hol_model::PIECE_CODE];
        }
        if (u < 0) return;  // every unit handed over
        const bool pjob = u >= hol_model::PIECE_CODE;
        const bool piece = !pjob && u >= hol_model::TAIL_CODE;
        // unit L + 2: embedding rows no token of this call touches (their gradient is zero and
        // known from the start)
        hipEvent_t ev = pjob    ? job.ev
                        : piece ? m->ev_tail[u - hol_model::TAIL_CODE]
                                : (u != m->L + 2 ? m->ev_unit[u] : nullptr);
        if (ev && wait_event(ev) != hipSuccess) {
          failed = true;
          return;
        }
        const double t0 = now_ms();
        if (pjob) {
          adam_unit(m, job.unit, kc, job.lo, job.hi, false);
          const int l = job.unit - 1;  // the layer's last piece: the next call's copy of it may go up
          if (job.last && l < hol_model::NPF && m->lpf_next[l] >= 0 && !prefetch_layer(l)) {
            failed = true;
            return;
          }
        } else if (piece) {
          const int c = u - hol_model::TAIL_CODE;
          const int64_t f0 = m->layer_flat0 + (int64_t)(m->tail_unit - 1) * m->layer_flat_n;
          adam_unit(m, m->tail_unit, kc, f0 + m->tail_lo[c], f0 + m->tail_hi[c], false);
          if (++tail_done == m->n_tail_expect && m->tail_unit == 1 && m->lpf_next[0] >= 0 && !prefetch_layer(0)) {
            failed = true;
            return;
          }
        } else if (u == m->L + 2) {
          adam_embed_rows(m, m->emb_untouched, kc, false);  // their gradient is zero already
        } else {
          adam_unit(m, u, kc, -1, -1, u == 0);  // layer and head blocks: overwritten by the next copies
          if (u == m->L + 1 && !prefetch_head()) {
            failed = true;
            return;
          }
          if (u >= 2 && u <= hol_model::NPF && m->lpf_next[u - 1] >= 0 && !prefetch_layer(u - 1)) {
            failed = true;
            return;
          }
        }
        const double t1 = now_ms();
        busy_ms += t1 - t0;
        m->stats.units.push_back({(double)u, t0 - t_call, t1 - t_call});
      }
    });
  }
  // the next call's head weights (final now) go up on the weight stream once this call's head op
  // is done with head_dev. By then the backward's layer copies are mostly queued, so the copy
  // runs late in the backward, where the link has slack. No stream of its own: the runtime maps
  // streams onto a few hardware queues, and a further stream sharing one with the weight or
  // gradient stream has stalled the device for a second and more behind its wait and copy.
  bool prefetch_head() {
    const uint8_t* src = image_block(m, -1);
    std::lock_guard<std::mutex> g(m->h2d_mu);
    if (hipStreamWaitEvent(m->sh2d, m->ev_head_done, 0) != hipSuccess ||
        image_h2d(m, m->head_dev, src, m->head_img_bytes, m->sh2d) != hipSuccess ||
        hipEventRecord(m->ev_head_pf, m->sh2d) != hipSuccess)
      return false;
    m->head_pf_ver = m->head_img_ver;
    m->head_pf_src = src;
    m->head_pf = true;
    prefetched = true;
    return true;
  }
  // one of the next call's first layers (its image final now) into the slot it occupied, once
  // this call's backward of it is done with that slot; on the weight stream like every slot copy
  bool prefetch_layer(int p) {
    const uint8_t* src = image_block(m, p);
    const int s = m->lpf_next[p];
    std::lock_guard<std::mutex> g(m->h2d_mu);
    if (hipStreamWaitEvent(m->sh2d, m->ev_lpf_done[p], 0) != hipSuccess ||
        image_h2d(m, m->slot[s], src, m->layer_img_bytes, m->sh2d) != hipSuccess ||
        hipEventRecord(m->ev_ready[s], m->sh2d) != hipSuccess)
      return false;
    m->lpf_ver[p] = m->lpf_img_ver[p];
    m->lpf_src[p] = src;
    m->lpf_slot[p] = s;
    ++lpf_sent;
    return true;
  }
  void push(int u) {
    {
      std::lock_guard<std::mutex> g(m->fmu);
      m->unit_queue.push_back(u);
    }
    m->fcv.notify_one();
  }
  void push_job(const hol_model::PieceJob& j) {
    {
      std::lock_guard<std::mutex> g(m->fmu);
      m->pjobs.push_back(j);
      m->unit_queue.push_back(hol_model::PIECE_CODE + (int)m->pjobs.size() - 1);
    }
    m->fcv.notify_one();
  }
  // waits for every handed-over unit (finish) or stops after the current one (abort)
  void stop(bool abort) {
    if (!running) return;
    if (abort) {
      std::lock_guard<std::mutex> g(m->fmu);
      m->fused_abort = true;
    } else {
      push(-1);
    }
    m->fcv.notify_one();
    th.join();
    running = false;
  }
  ~FusedWorker() { stop(true); }
};

// Host step of a staleness-1 call. Once the first layer's inputs are gathered, Adam runs over
// every unit on a thread of its own with the accumulated gradient, refreshing the second image
// while the GPU streams from the first, in the order the call's gradient copies land (LM head,
// layers from the last, embedding). The gradient block is shared: a unit's new gradient copy runs
// only after the step has read the old one. That wait sits on the gradient-transfer stream (a host
// function that returns once the unit is done, gate()), so the issuing thread never blocks and the
// whole call is queued up front. The step clears what the copies do not overwrite (the embedding
// rows, which the call adds into, and a head the call does not write). finish() waits for the
// thread and makes its image the streamed one.
struct AsyncStep {
  hol_model* m;
  std::thread th;
  bool started = false;
  double busy_ms = 0;
  std::mutex mu;
  std::condition_variable cv;
  std::vector<char> done;  // per unit: old gradient consumed
  double wait_ms = 0;      // time the transfer stream spent waiting for it
  double t_call = 0;
  std::vector<std::array<double, 3>> units, waits;  // {unit, start, end} in ms from the call's start
  void start(const AdamConsts& kc, bool zero_head, double t_start) {
    t_call = t_start;
    const int n = (int)m->unit_tensors.size();  // 0 embedding, 1 + l layer l, L + 1 head
    done.assign(n, 0);
    gates.resize(n);
    for (int u = 0; u < n; ++u) gates[u] = {this, u};
    started = true;
    uint8_t* img = m->image_alt;
    th = std::thread([this, kc, zero_head, n, img] {
      const double t0 = now_ms();
      for (int u = n - 1; u >= 0; --u) {
        const double a = now_ms();
        adam_unit(m, u, kc, -1, -1, u == 0 || (u == n - 1 && zero_head), m->grad, img);
        units.push_back({(double)u, a - t_call, now_ms() - t_call});
        {
          std::lock_guard<std::mutex> g(mu);
          done[u] = 1;
        }
        cv.notify_all();
      }
      busy_ms = now_ms() - t0;
    });
  }
  void wait_unit(int u) {
    if (!started) return;
    const double t0 = now_ms();
    std::unique_lock<std::mutex> lk(mu);
    cv.wait(lk, [&] { return done[u] != 0; });
    const double t1 = now_ms();
    wait_ms += t1 - t0;
    waits.push_back({(double)u, t0 - t_call, t1 - t_call});
  }
  // the stream's later work waits until unit u is done (the host function returns only then; it
  // depends on host work alone, so it always returns)
  struct Gate {
    AsyncStep* a;
    int u;
  };
  std::vector<Gate> gates;
  static void gate_fn(void* p) {
    Gate* g = (Gate*)p;
    g->a->wait_unit(g->u);
  }
  hipError_t gate(int u, hipStream_t s) {
    if (!started) return hipSuccess;
    return hipLaunchHostFunc(s, gate_fn, &gates[u]);
  }
  void finish() {
    if (!started) return;
    th.join();
    started = false;
    std::swap(m->image, m->image_alt);
    m->step_t += 1;
  }
  ~AsyncStep() {
    if (started) (void)hipStreamSynchronize(m->sd2h);  // no gate left waiting on this object
    finish();
  }
};

hol_status engine_forward_backward(hol_model* m, const hol_batch* b, hol_loss loss, double* out, FbMode mode) {
  const double t_start = now_ms();
  const bool fuse_step = mode == FB_FUSED, async = mode == FB_ASYNC;
  // ---- validation (nothing touched before this passes)
  auto bad = [](const std::string& s) {
    set_error("hol_forward_backward: " + s);
    return HOL_EINVAL;
  };
  if (!b || !out) return bad("null argument");
  if (async && !m->image_alt) return bad("the asynchronous optimiser needs a model created with async_optimizer = 1");
  if (m->poisoned) {
    set_error("hol_forward_backward: model poisoned by an earlier device error; call hol_zero_grad");
    return HOL_ESTATE;
  }
  const int B = b->batch, S = b->seq, M = b->n_micro;
  if (B <= 0 || S <= 0 || M <= 0) return bad("batch, seq and n_micro must be positive");
  if (B % M) return bad("batch must be a multiple of n_micro");
  const int64_t T64 = (int64_t)B * S;
  if (T64 > m->Tmax) return bad("batch*seq exceeds max_tokens");
  if (S > m->Smax) return bad("seq exceeds max_seq");
  if (m->dt == DT_BF16 && T64 % 8) return bad("bf16 compute needs batch*seq to be a multiple of 8");
  const int T = (int)T64, H = m->H;
  if (loss == HOL_LOSS_NEXT_TOKEN_CE) {
    if (m->V <= 0) return bad("cross entropy needs vocab > 0");
    if (!b->tokens) return bad("tokens required");
    for (int64_t i = 0; i < T64; ++i)
      if (b->tokens[i] < 0 || b->tokens[i] >= m->V) return bad("token id out of range");
    if (b->labels)
      for (int64_t i = 0; i < T64; ++i)
        if (b->labels[i] < -1 || b->labels[i] >= m->V) return bad("label out of range");
  } else if (loss == HOL_LOSS_SUM_SQUARES) {
    if (m->V > 0) {
      if (!b->tokens) return bad("tokens required");
      for (int64_t i = 0; i < T64; ++i)
        if (b->tokens[i] < 0 || b->tokens[i] >= m->V) return bad("token id out of range");
    } else if (!b->hidden_in) {
      return bad("hidden_in required when vocab == 0");
    }
  } else {
    return bad("unknown loss");
  }
  m->stats = Stats();
  m->stats.tokens = T;
  AsyncStep astep{m};
  const bool apply_prev = async && !m->grads_zero;  // an accumulated gradient to step with
  const int L = m->L, K = m->K;
  const int64_t E = m->E;
  // ---- labels and per-token weights (1/labelled count of the token's micro-batch)
  if (loss == HOL_LOSS_NEXT_TOKEN_CE) {
    const int per = B / M;
    for (int mb = 0; mb < M; ++mb) {
      int64_t cnt = 0;
      const int64_t t0 = (int64_t)mb * per * S, t1 = t0 + (int64_t)per * S;
      for (int64_t t = t0; t < t1; ++t) {
        int32_t y;
        if (b->labels) y = b->labels[t];
        else y = ((t % S) == S - 1) ? -1 : b->tokens[t + 1];
        m->lab_stage[t] = y;
        if (y >= 0) ++cnt;
      }
      const float w = cnt ? (float)(1.0 / (double)cnt) : 0.f;
      for (int64_t t = t0; t < t1; ++t) m->w_stage[t] = m->lab_stage[t] >= 0 ? w : 0.f;
    }
  }
  // ---- h_0: embedding rows gathered on the host from the fp32 masters, or the given hidden states
  // (run while the first layer's weights stream in)
  auto gather_h0 = [&]() {
    const double te = now_ms();
    if (m->V > 0) {
      const float* emb = m->master + m->embed_flat0;
      parallel_for(T64, 256, [&](int64_t lo, int64_t hi) {
        for (int64_t t = lo; t < hi; ++t) memcpy(m->h_stage + t * H, emb + (int64_t)b->tokens[t] * H, (size_t)H * 4);
      });
    } else {
      parallel_for(T64 * H, 1 << 20,
                   [&](int64_t lo, int64_t hi) { memcpy(m->h_stage + lo, b->hidden_in + lo, (size_t)(hi - lo) * 4); });
    }
    m->stats.host_embed_ms = now_ms() - te;
  };

  hol_status st = HOL_OK;
  auto fail = [&](hol_status s) {
    m->poisoned = true;
    hipDeviceSynchronize();
    return s;
  };
  // (the FusedWorker destructor stops the worker on every early return)
#define STEP(expr)                    \
  do {                                \
    hol_status s__ = (expr);          \
    if (s__ != HOL_OK) return fail(s__); \
  } while (0)
#define HSTEP(expr)                                                                        \
  do {                                                                                     \
    hipError_t e__ = (expr);                                                               \
    if (e__ != hipSuccess) {                                                               \
      set_error(std::string(#expr) + ": " + hipGetErrorString(e__) + " (" __FILE__ ":" + \
                std::to_string(__LINE__) + ")");                                           \
      return fail(HOL_EDEVICE);                                                            \
    }                                                                                      \
  } while (0)

  HSTEP(hipSetDevice(m->cfg.device));
  hipStream_t sc = m->sc, sh = m->sh2d, sd = m->sd2h;
  // initial event states: every buffer free; a slot holding one of the first layers as sent by
  // the previous fused step stays bound to it while that image is unwritten since (its ready event
  // is that copy's), else it is free (a new copy into it queues behind that one)
  for (int i = 0; i < m->nslots; ++i) {
    HSTEP(hipEventRecord(m->ev_free[i], sc));
    m->slot_layer[i] = -1;
  }
  for (int p = 0; p < hol_model::NPF && p < L; ++p) {
    const int ps = m->lpf_slot[p];
    if (ps >= 0 && m->lpf_ver[p] == m->lpf_img_ver[p] && m->lpf_src[p] == image_block(m, p)) m->slot_layer[ps] = p;
    m->lpf_slot[p] = -1;
    m->lpf_next[p] = -1;
  }
  m->n_tail_expect = 0;
  for (int i = 0; i < m->ngbuf; ++i) HSTEP(hipEventRecord(m->ev_gfree[i], sd));
  m->tev_used = 0;
  m->krec.clear();
  auto tev = [&]() -> hipEvent_t { return m->tev[std::min<int>(m->tev_used++, (int)m->tev.size() - 1)]; };
  struct Span { hipEvent_t a, b; int cls; };
  std::vector<Span> spans;  // cls: 0 h2d, 1 d2h, 2 fwd, 3 recomp, 4 bwd, 5 head

  if (loss == HOL_LOSS_NEXT_TOKEN_CE) {
    HSTEP(hipMemcpyAsync(m->labels_dev, m->lab_stage, T64 * 4, hipMemcpyHostToDevice, sc));
    HSTEP(hipMemcpyAsync(m->w_dev, m->w_stage, T64 * 4, hipMemcpyHostToDevice, sc));
  }
  // ---- op list
  std::vector<Op> ops;
  for (int l = 0; l < L; ++l) ops.push_back({OP_FWD, l, l / K, l % K});
  ops.push_back({OP_HEAD, -1, -1, 0});
  for (int bl = m->nblocks - 1; bl >= 0; --bl) {
    const int l0 = bl * K, l1 = std::min(L, (bl + 1) * K);
    // the last block's forward already stored its activations: no recompute for it
    if (bl < m->nblocks - 1)
      for (int l = l0; l < l1; ++l) ops.push_back({OP_RECOMP, l, bl, l - l0});
    for (int l = l1 - 1; l >= l0; --l) ops.push_back({OP_BWD, l, bl, l - l0});
  }
  auto ckpt_of = [&](int idx) { return m->ckpt + (int64_t)idx * T64 * H; };  // idx: block, or nblocks for h_L
  // direct: the copies overwrite the gradient blocks (nothing accumulated, or the accumulated
  // gradient is consumed by this call's overlapped step before each copy)
  const bool direct = m->grads_zero || apply_prev;
  // fused optimiser: only when this call's gradients are the whole gradient (nothing accumulated)
  const bool fused = fuse_step && m->grads_zero;
  // a stale head block that this call does not overwrite is cleared now (the layer blocks are
  // overwritten whole by their copies; an overlapped step clears it after reading it)
  const bool head_written = m->V > 0 && loss == HOL_LOSS_NEXT_TOKEN_CE && m->head_trainable;
  if (m->grads_stale && !head_written && m->head_flat_n > 0) parallel_zero(m->grad + m->head_flat0, m->head_flat_n * 4);
  const hol_config& cf = m->cfg;
  const AdamConsts kc = adam_consts(m->step_t + 1, cf.lr, cf.beta1, cf.beta2, cf.adam_eps);
  FusedWorker worker{m};
  if (fused) worker.start(kc, t_start);

  // ---- weight streaming: the layer of each op sits in one of the nslots HBM slots. After binding
  // op j, the transfer stream fills slots with the layers of the next nslots - 1 ops; a slot is
  // reused only when no op from j up to the one being loaded needs its layer, and among those the
  // one whose layer is needed furthest ahead (or never) goes first.
  const int NS = m->nslots;
  auto slot_of = [&](int layer) -> int {
    for (int s = 0; s < NS; ++s)
      if (m->slot_layer[s] == layer) return s;
    return -1;
  };
  auto next_use = [&](int layer, size_t from) -> size_t {
    for (size_t i = from; i < ops.size(); ++i)
      if (ops[i].kind != OP_HEAD && ops[i].layer == layer) return i;
    return ops.size();
  };
  // makes op k's layer resident while op j is the current op; *placed = false when no slot can
  // be reused yet
  auto ensure = [&](size_t j, size_t k, bool* placed = nullptr) -> hol_status {
    const int layer = ops[k].layer;
    if (placed) *placed = true;
    if (slot_of(layer) >= 0) return HOL_OK;
    int best = -1;
    size_t best_use = 0;
    for (int s = 0; s < NS; ++s) {
      const size_t u = m->slot_layer[s] < 0 ? ops.size() + 1 : next_use(m->slot_layer[s], j);
      if (u <= k) continue;
      if (best < 0 || u > best_use) {
        best = s;
        best_use = u;
      }
    }
    if (best < 0) {
      if (placed) *placed = false;
      return HOL_OK;
    }
    std::lock_guard<std::mutex> g(m->h2d_mu);
    HCHECK(hipStreamWaitEvent(sh, m->ev_free[best], 0));
    hipEvent_t a = tev(), e = tev();
    HCHECK(hipEventRecord(a, sh));
    HCHECK(image_h2d(m, m->slot[best], image_block(m, layer), m->layer_img_bytes, sh));
    HCHECK(hipEventRecord(e, sh));
    spans.push_back({a, e, 0});
    HCHECK(hipEventRecord(m->ev_ready[best], sh));
    m->slot_layer[best] = layer;
    m->stats.h2d_bytes += (double)m->layer_img_bytes;
    m->stats.h2d_span_bytes += (double)m->layer_img_bytes;
    m->stats.n_weight_streams++;
    return HOL_OK;
  };
  bool head_loaded = false;
  auto load_head = [&]() -> hol_status {
    if (head_loaded || m->V <= 0 || loss != HOL_LOSS_NEXT_TOKEN_CE) return HOL_OK;
    std::lock_guard<std::mutex> g(m->h2d_mu);
    if (m->head_pf) {
      // the previous call's copy of these weights stands (or a stale one may still be landing)
      HCHECK(hipStreamWaitEvent(sh, m->ev_head_pf, 0));
      m->head_pf = false;
      if (m->head_pf_ver == m->head_img_ver && m->head_pf_src == image_block(m, -1)) {
        HCHECK(hipEventRecord(m->ev_head, sh));
        head_loaded = true;
        return HOL_OK;
      }
    }
    hipEvent_t a = tev(), e = tev();
    HCHECK(hipEventRecord(a, sh));
    HCHECK(image_h2d(m, m->head_dev, image_block(m, -1), m->head_img_bytes, sh));
    HCHECK(hipEventRecord(e, sh));
    spans.push_back({a, e, 0});
    HCHECK(hipEventRecord(m->ev_head, sh));
    m->stats.h2d_bytes += (double)m->head_img_bytes;
    m->stats.h2d_span_bytes += (double)m->head_img_bytes;
    head_loaded = true;
    return HOL_OK;
  };

  STEP(ensure(0, 0));
  gather_h0();
  // the embedding rows are read: the step may now change the masters
  if (apply_prev) astep.start(adam_consts(m->step_t + 1, cf.lr, cf.beta1, cf.beta2, cf.adam_eps), !head_written, t_start);
  HSTEP(hipMemcpyAsync(m->ckpt, m->h_stage, T64 * H * 4, hipMemcpyHostToDevice, sc));
  m->stats.h2d_bytes += (double)T64 * H * 4;
  // further weight copies start after h0 is up: the first layer needs both
  HSTEP(hipEventRecord(m->ev_h0, sc));
  HSTEP(hipStreamWaitEvent(sh, m->ev_h0, 0));
  // embedding rows by token: occurrences of each token id in order of position (the scatter-add of
  // the first-layer gradient sums them in that order), and the rows no token touches
  std::vector<int32_t> tok_order;
  if (m->embed_trainable) {
    tok_order.resize(T64);
    for (int64_t t = 0; t < T64; ++t) tok_order[t] = (int32_t)t;
    std::stable_sort(tok_order.begin(), tok_order.end(),
                     [&](int32_t x, int32_t y) { return b->tokens[x] < b->tokens[y]; });
    m->emb_touched.clear();
    int32_t* seg = m->ord_stage + T64;
    for (int64_t i = 0; i < T64; ++i) {
      m->ord_stage[i] = tok_order[i];
      if (i == 0 || b->tokens[tok_order[i]] != b->tokens[tok_order[i - 1]]) {
        seg[m->emb_touched.size()] = (int32_t)i;
        m->emb_touched.push_back(b->tokens[tok_order[i]]);
      }
    }
    seg[m->emb_touched.size()] = (int32_t)T64;
    HSTEP(hipMemcpyAsync(m->ord_dev, m->ord_stage, T64 * 4, hipMemcpyHostToDevice, sc));
    HSTEP(hipMemcpyAsync(m->seg_dev, seg, (m->emb_touched.size() + 1) * 4, hipMemcpyHostToDevice, sc));
    if (fused) {
      m->emb_untouched.clear();
      size_t q = 0;
      for (int32_t r = 0; r < m->V; ++r) {
        if (q < m->emb_touched.size() && m->emb_touched[q] == r) ++q;
        else m->emb_untouched.push_back(r);
      }
      worker.push(m->L + 2);  // their Adam overlaps the forward
    }
  }
  int gi = 0;  // grad buffer ping-pong
  for (size_t j = 0; j < ops.size(); ++j) {
    const Op& op = ops[j];
    // bind
    if (op.kind != OP_HEAD && slot_of(op.layer) < 0) STEP(ensure(j, j));
    // prefetch the layers of the next ops (overlaps this op's compute); the head's weights go up
    // when the window reaches the head
    auto prefetch = [&]() -> hol_status {
      int ahead = 0;
      for (size_t k = j + 1; k < ops.size() && ahead < NS - 1; ++k) {
        if (ops[k].kind == OP_HEAD) {
          const hol_status r = load_head();
          if (r != HOL_OK) return r;
          continue;
        }
        ++ahead;
        bool placed = true;
        const hol_status r = ensure(j, k, &placed);
        if (r != HOL_OK) return r;
        if (!placed) break;
      }
      return HOL_OK;
    };
    hipEvent_t ta = tev(), tb = tev();
    if (op.kind == OP_HEAD) {
      STEP(load_head());
      if (m->V > 0 && loss == HOL_LOSS_NEXT_TOKEN_CE) HSTEP(hipStreamWaitEvent(sc, m->ev_head, 0));
      HSTEP(hipEventRecord(ta, sc));
      STEP(head_forward_backward(m, ckpt_of(m->nblocks), T, loss));
      HSTEP(hipEventRecord(m->ev_head_done, sc));  // head_dev free for the next call's weights
      HSTEP(hipEventRecord(tb, sc));
      spans.push_back({ta, tb, 5});
      if (m->V > 0 && loss == HOL_LOSS_NEXT_TOKEN_CE && m->head_trainable) {
        // head gradient to the host (gradient-transfer stream)
        HSTEP(hipEventRecord(m->ev_gdone[0], sc));
        HSTEP(astep.gate(m->L + 1, sd));
        HSTEP(hipStreamWaitEvent(sd, m->ev_gdone[0], 0));
        float* dst = direct ? m->grad + m->head_flat0 : m->head_stage;
        hipEvent_t a = tev(), e = tev();
        HSTEP(hipEventRecord(a, sd));
        HSTEP(hipMemcpyAsync(dst, m->head_gdev, m->head_flat_n * 4, hipMemcpyDeviceToHost, sd));
        HSTEP(hipEventRecord(e, sd));
        spans.push_back({a, e, 1});
        m->stats.d2h_bytes += (double)m->head_flat_n * 4;
        if (!direct) {
          static thread_local AccumJob job;
          job = {m->grad + m->head_flat0, m->head_stage, m->head_flat_n};
          HSTEP(hipLaunchHostFunc(sd, host_accumulate, &job));
        }
        if (fused) {
          HSTEP(hipEventRecord(m->ev_unit[m->L + 1], sd));
          worker.push(m->L + 1);
        }
      }
      STEP(prefetch());
      continue;
    }
    const int s = slot_of(op.layer);
    const W w = bind(m, m->slot[s]);
    HSTEP(hipStreamWaitEvent(sc, m->ev_ready[s], 0));
    // the next layer's weights go to the other slot while this op computes (issued first: a
    // mixture-of-experts layer waits on the host for its routing counts mid-op)
    STEP(prefetch());
    const int n_seq = B;
    if (op.kind == OP_FWD) {
      // h_in: checkpoint of the block for the block's first layer, else the previous output
      const int l = op.layer;
      const int lb0 = (m->nblocks - 1) * K;  // first layer of the last block
      const float* hin = (l == 0) ? ckpt_of(0) : ((l % K == 0) ? ckpt_of(l / K) : m->hbuf[(l - 1) & 1]);
      float* hout;
      if (l + 1 == L) hout = ckpt_of(m->nblocks);
      else if ((l + 1) % K == 0) hout = ckpt_of((l + 1) / K);
      else hout = m->hbuf[l & 1];
      // The last block keeps its forward activations in the store, where the backward reads them
      // (the recompute of that block would reproduce them bit for bit).
      Act A = act_at(m, 0);
      int pos = 0;
      if (l >= lb0) {
        pos = l - lb0;
        A = act_at(m, pos);
        if (l > lb0) hin = A.hin;
        if (l + 1 < L) hout = act_at(m, pos + 1).hin;
      }
      HSTEP(hipEventRecord(ta, sc));
      STEP(layer_forward(m, w, hin, hout, A, T, n_seq, S, pos));
      if (m->NE > 0)  // routing of this forward pass, kept for hol_get_routing
        HSTEP(hipMemcpyAsync(m->route_rec + (int64_t)l * T * m->topk, A.ids, (size_t)T * m->topk * 4,
                             hipMemcpyDeviceToDevice, sc));
      HSTEP(hipEventRecord(tb, sc));
      spans.push_back({ta, tb, 2});
    } else if (op.kind == OP_RECOMP) {
      const int l1 = std::min(L, (op.block + 1) * K);
      const Act A = act_at(m, op.pos);
      const float* hin = op.pos == 0 ? ckpt_of(op.block) : A.hin;
      // the block's last layer: its output (the next block's checkpoint, already stored) is not
      // needed, and its backward reads only the stored intermediates, so the product that would
      // form it is skipped
      float* hout = (op.layer + 1 < l1) ? act_at(m, op.pos + 1).hin : nullptr;
      HSTEP(hipEventRecord(ta, sc));
      STEP(layer_forward(m, w, hin, hout, A, T, n_seq, S, op.pos));
      HSTEP(hipEventRecord(tb, sc));
      spans.push_back({ta, tb, 3});
    } else {  // OP_BWD
      const Act A = act_at(m, op.pos);
      const float* hin = op.pos == 0 ? ckpt_of(op.block) : A.hin;
      const bool tail = fused && j + 1 == ops.size();
      // dense bf16 layer with trainable weights, gradient block [wqkv | wo | w_gate w_up | w_down |
      // attn_norm | mlp_norm ...]: copied in three pieces, each as soon as it is final
      const bool pieces = direct && m->dt == DT_BF16 && m->NE == 0 && m->base_trainable;
      HSTEP(hipStreamWaitEvent(sc, m->ev_gfree[gi], 0));
      HSTEP(hipEventRecord(ta, sc));
      m->pieces_armed = pieces;
      const hol_status bst = layer_backward(m, w, A, hin, m->gdev[gi], T, n_seq, S, op.pos);
      m->pieces_armed = false;
      STEP(bst);
      HSTEP(hipEventRecord(tb, sc));
      spans.push_back({ta, tb, 4});
      HSTEP(hipEventRecord(m->ev_gdone[gi], sc));
      // one of the first layers: its slot takes the next call's copy once this backward is done,
      // when no copy of this call can reuse it, i.e. every op left uses another layer that is
      // resident (always for the call's last op)
      if (fused && op.layer < hol_model::NPF) {
        bool rest_resident = true;
        for (size_t k = j + 1; rest_resident && k < ops.size(); ++k)
          if (ops[k].kind != OP_HEAD && (ops[k].layer == op.layer || slot_of(ops[k].layer) < 0)) rest_resident = false;
        if (rest_resident) {
          HSTEP(hipEventRecord(m->ev_lpf_done[op.layer], sc));
          m->lpf_next[op.layer] = s;
        }
      }
      // gradient offload on the gradient-transfer stream
      float* lg = m->grad + m->layer_flat0 + (int64_t)op.layer * m->layer_flat_n;
      HSTEP(astep.gate(1 + op.layer, sd));
      hipEvent_t a = tev(), e = tev();
      HSTEP(hipEventRecord(a, sd));
      const int64_t n = m->layer_flat_n;
      hipEvent_t* pe = pieces ? &m->ev_piece[3 * (size_t)op.layer] : nullptr;
      if (pieces) {
        const float* gd = m->gdev[gi];
        auto copy = [&](int64_t lo, int64_t hi) {
          return hipMemcpyAsync(lg + lo, gd + lo, (size_t)(hi - lo) * 4, hipMemcpyDeviceToHost, sd);
        };
        HSTEP(hipStreamWaitEvent(sd, m->ev_wd_final, 0));
        HSTEP(copy(m->g_wd, m->g_g1));
        HSTEP(hipEventRecord(pe[0], sd));
        HSTEP(hipStreamWaitEvent(sd, m->ev_mlp_final, 0));
        HSTEP(copy(m->g_wgu, m->g_wd));
        HSTEP(hipEventRecord(pe[1], sd));
        HSTEP(hipStreamWaitEvent(sd, m->ev_gdone[gi], 0));
        HSTEP(copy(0, m->g_wgu));
        HSTEP(copy(m->g_g1, n));
        HSTEP(hipEventRecord(pe[2], sd));
      } else if (tail) {
        // the call's last gradient: in pieces, each handed to the optimiser as it lands
        m->tail_unit = 1 + op.layer;
        m->n_tail = 0;
        m->n_tail_expect = hol_model::N_TAIL;
        HSTEP(hipStreamWaitEvent(sd, m->ev_gdone[gi], 0));
        for (int c = 0; c < hol_model::N_TAIL; ++c) {
          const int64_t lo = n * c / hol_model::N_TAIL, hi = n * (c + 1) / hol_model::N_TAIL;
          m->tail_lo[c] = lo;
          m->tail_hi[c] = hi;
          m->n_tail++;
          HSTEP(hipMemcpyAsync(lg + lo, m->gdev[gi] + lo, (size_t)(hi - lo) * 4, hipMemcpyDeviceToHost, sd));
          HSTEP(hipEventRecord(m->ev_tail[c], sd));
          worker.push(hol_model::TAIL_CODE + c);
        }
      } else {
        HSTEP(hipStreamWaitEvent(sd, m->ev_gdone[gi], 0));
        HSTEP(hipMemcpyAsync(direct ? lg : m->grad_stage, m->gdev[gi], n * 4, hipMemcpyDeviceToHost, sd));
      }
      HSTEP(hipEventRecord(e, sd));
      spans.push_back({a, e, 1});
      if (!direct) {
        static thread_local std::vector<AccumJob> jobs;
        jobs.resize(L);
        jobs[op.layer] = {lg, m->grad_stage, m->layer_flat_n};
        HSTEP(hipLaunchHostFunc(sd, host_accumulate, &jobs[op.layer]));
      }
      HSTEP(hipEventRecord(m->ev_gfree[gi], sd));
      if (fused && pieces) {  // the pieces' optimiser jobs, in the order they land
        const int u = 1 + op.layer;
        const int64_t f0 = m->layer_flat0 + (int64_t)op.layer * n;
        worker.push_job({u, f0 + m->g_wd, f0 + m->g_g1, pe[0], false});
        worker.push_job({u, f0 + m->g_wgu, f0 + m->g_wd, pe[1], false});
        worker.push_job({u, f0, f0 + m->g_wgu, pe[2], false});
        worker.push_job({u, f0 + m->g_g1, f0 + n, pe[2], true});
      } else if (fused && !tail) {
        HSTEP(hipEventRecord(m->ev_unit[1 + op.layer], sd));
        worker.push(1 + op.layer);
      }
      m->stats.d2h_bytes += (double)m->layer_flat_n * 4;
      gi = (gi + 1) % m->ngbuf;
    }
    HSTEP(hipEventRecord(m->ev_free[s], sc));
  }
  // ---- first-layer gradient (embedding rows) and loss rows back to the host
  m->last_T = T;
  // (the gradient of each touched embedding row, summed on the device in position order)
  const int64_t n_rows = m->embed_trainable ? (int64_t)m->emb_touched.size() : 0;
  if (m->embed_trainable) {
    HSTEP((hipError_t)launch_embed_row_sums(m->dh, m->ord_dev, m->seg_dev, (int)n_rows, H, m->erows, sc));
    HSTEP(hipMemcpyAsync(m->h_stage, m->erows, n_rows * H * 4, hipMemcpyDeviceToHost, sc));
    m->stats.d2h_bytes += (double)n_rows * H * 4;
  }
  HSTEP(hipMemcpyAsync(m->loss_stage, m->rowloss_dev, T64 * 4, hipMemcpyDeviceToHost, sc));
  // the code below needs only the compute stream's copies; the last gradient copy may still run
  HSTEP(hipStreamSynchronize(sc));
  HSTEP(hipStreamSynchronize(sh));
  HSTEP(hipGetLastError());
  // embedding gradient rows: the fused step reads them from the staging buffer in its Adam (the
  // embedding's gradient block stays zero); otherwise they are added into that block
  if (m->embed_trainable && !fused) {
    astep.wait_unit(0);
    float* gE = m->grad + m->embed_flat0;
    parallel_for(n_rows, 8, [&](int64_t lo, int64_t hi) {
      for (int64_t u = lo; u < hi; ++u) {
        float* dst = gE + (int64_t)m->emb_touched[u] * H;
        const float* src = m->h_stage + u * H;
        for (int64_t c = 0; c < H; ++c) dst[c] += src[c];
      }
    });
  }
  double total = 0.0;
  for (int64_t t = 0; t < T64; ++t) total += (double)m->loss_stage[t];
  *out = total;
  m->grads_zero = false;
  m->grads_stale = false;
  m->stats.scatter_done_ms = now_ms() - t_start;
  HSTEP(hipStreamSynchronize(sd));
  m->stats.gpu_done_ms = now_ms() - t_start;
  if (apply_prev) {
    const double tw = now_ms();
    astep.finish();
    m->stats.worker_busy_ms = astep.busy_ms;
    m->stats.async_wait_ms = astep.wait_ms;
    m->stats.units = astep.units;
    m->stats.waits = astep.waits;
    m->stats.step_ms = now_ms() - tw;  // update time not hidden under the GPU work
  }
  if (fused) {
    const double t_gpu_done = now_ms();
    worker.stop(false);
    m->stats.worker_busy_ms = worker.busy_ms;
    if (worker.prefetched) m->stats.h2d_bytes += (double)m->head_img_bytes;  // the next call's head weights
    m->stats.h2d_bytes += (double)worker.lpf_sent * m->layer_img_bytes;  // and first layers
    m->stats.n_weight_streams += worker.lpf_sent;
    if (worker.failed) {
      set_error("hol_forward_backward_step: gradient copy failed; the step may be partially applied");
      return fail(HOL_EDEVICE);
    }
    // the touched embedding rows: their gradients arrived with the last copies
    adam_embed_rows(m, m->emb_touched, kc, false, m->h_stage);
    m->step_t += 1;
    m->grads_zero = true;
    m->grads_stale = true;
    m->stats.step_ms = now_ms() - t_gpu_done;  // optimiser time not hidden under the GPU work
    m->fused_overlap_ms = worker.busy_ms;
  } else if (fuse_step) {
    m->stats.fb_ms = now_ms() - t_start;
    return engine_step(m);
  }
  // ---- stats
  {
    // device timeline from the first weight copy: when compute starts and ends
    int f = -1, l = -1;
    for (int i = 0; i < (int)spans.size(); ++i)
      if (spans[i].cls >= 2) {
        if (f < 0) f = i;
        l = i;
      }
    float a = 0.f, b2 = 0.f;
    if (!spans.empty() && f >= 0 && hipEventElapsedTime(&a, spans[0].a, spans[f].a) == hipSuccess &&
        hipEventElapsedTime(&b2, spans[0].a, spans[l].b) == hipSuccess) {
      m->stats.first_compute_ms = a;
      m->stats.last_compute_end_ms = b2;
    }
  }
  m->stats.timeline.clear();
  for (auto& sp : spans) {
    float ms = 0.f, t0 = 0.f;
    if (hipEventElapsedTime(&ms, sp.a, sp.b) != hipSuccess) continue;
    if (hipEventElapsedTime(&t0, spans[0].a, sp.a) == hipSuccess) m->stats.timeline.push_back({(float)sp.cls, t0, t0 + ms});
    switch (sp.cls) {
      case 0: m->stats.h2d_busy_ms += ms; break;
      case 1: m->stats.d2h_busy_ms += ms; break;
      case 2: m->stats.fwd_ms += ms; m->stats.compute_busy_ms += ms; break;
      case 3: m->stats.recomp_ms += ms; m->stats.compute_busy_ms += ms; break;
      case 4: m->stats.bwd_ms += ms; m->stats.compute_busy_ms += ms; break;
      case 5: m->stats.head_ms += ms; m->stats.compute_busy_ms += ms; break;
    }
  }
  for (const auto& r : m->krec) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, m->kev[r.ev], m->kev[r.ev + 1]) != hipSuccess) continue;
    KStat& k = m->stats.k[r.cls];
    k.launches++;
    k.ms += ms;
    k.flops += r.flops;
    k.bytes += r.bytes;
    if (r.cls == KC_GEMM) {
      KStat& gs = m->stats.gemm_shapes[{r.gm, r.gn, r.gk}];
      gs.launches++;
      gs.ms += ms;
      gs.flops += r.flops;
      gs.bytes += r.bytes;
    }
  }
  m->krec.clear();
  m->stats.fb_ms = now_ms() - t_start;
  (void)E;
  (void)st;
#undef STEP
#undef HSTEP
  return HOL_OK;
}

// ------------------------------------------------------------------------------------------
// step: host Adam, refresh of the low-precision image, zero_grad
// ------------------------------------------------------------------------------------------
// Adam (and the image refresh) on the trainable tensors of unit u, restricted to the flat
// parameter range [lo, hi) when lo >= 0 (the same per-element arithmetic either way); with zero
// the gradients read are cleared. gbase / ibase: the gradient block read and the image written
// (m->grad and m->image unless given).
static void adam_unit(hol_model* m, int u, const AdamConsts& k, int64_t lo, int64_t hi, bool zero, float* gbase,
                      uint8_t* ibase) {
  if (!gbase) gbase = m->grad;
  for (int ti : m->unit_tensors[u]) {
    const TensorDesc& t = m->tensors[ti];
    if (!t.trainable) continue;
    const int64_t a0 = lo < 0 ? 0 : std::max<int64_t>(0, lo - t.flat);
    const int64_t a1 = lo < 0 ? t.numel : std::min<int64_t>(t.numel, hi - t.flat);
    if (a1 <= a0) continue;
    float* th = m->master + t.flat + a0;
    float* g = gbase + t.flat + a0;
    float* m1 = m->mom1 + t.flat + a0;
    float* m2 = m->mom2 + t.flat + a0;
    const bool to_bf16 = !(t.img_f32 || m->dt == DT_F32) && t.img >= 0 && t.block != -2;
    uint8_t* dst = (t.block == -2 || t.img < 0) ? nullptr
                                                : image_block(m, t.block, ibase) + t.img + a0 * (to_bf16 ? 2 : 4);
    parallel_for(a1 - a0, 1 << 16, [&](int64_t lo, int64_t hi) {
      // chunked so the refreshed values are still in cache when converted
      for (int64_t a = lo; a < hi; a += 4096) {
        const int64_t n = std::min<int64_t>(4096, hi - a);
        adam_range(th + a, g + a, m1 + a, m2 + a, n, k);
        if (dst) {
          if (to_bf16) f32_to_bf16_range_stream(th + a, (uint16_t*)dst + a, n);
          else memcpy((float*)dst + a, th + a, (size_t)n * 4);
        }
        if (zero) memset(g + a, 0, (size_t)n * 4);
      }
      _mm_sfence();  // the image's non-temporal stores are visible before the unit counts as done
    });
  }
  if (u == m->L + 1) m->head_img_ver++;  // the head's image changed
  if (u >= 1 && u <= hol_model::NPF) m->lpf_img_ver[u - 1]++;  // one of the first layers''
}

// Adam on the given rows of the embedding (and zeroing of their gradients): the same per-element
// arithmetic as adam_unit, split by rows.
// (gsrc: the gradient of rows[q] at gsrc + q H instead of in the gradient block)
static void adam_embed_rows(hol_model* m, const std::vector<int32_t>& rows, const AdamConsts& k, bool zero,
                            const float* gsrc) {
  if (!m->embed_trainable || rows.empty()) return;
  const int64_t H = m->H, f0 = m->embed_flat0;
  parallel_for((int64_t)rows.size(), 16, [&](int64_t lo, int64_t hi) {
    for (int64_t q = lo; q < hi; ++q) {
      const int64_t o = f0 + (int64_t)rows[q] * H;
      adam_range(m->master + o, gsrc ? gsrc + q * H : m->grad + o, m->mom1 + o, m->mom2 + o, H, k);
      if (zero) memset(m->grad + o, 0, (size_t)H * 4);
    }
  });
}

// Clears the layer and head gradient blocks a fused step left holding consumed gradients.
static void clear_stale_grads(hol_model* m) {
  if (!m->grads_stale) return;
  const int64_t n = m->n_flat - m->layer_flat0;
  parallel_zero(m->grad + m->layer_flat0, n * 4);
  m->grads_stale = false;
}

hol_status engine_step(hol_model* m) {
  if (m->poisoned) {
    set_error("hol_step: model poisoned by an earlier device error; call hol_zero_grad");
    return HOL_ESTATE;
  }
  const double t0 = now_ms();
  clear_stale_grads(m);  // logically zero
  const hol_config& c = m->cfg;
  const AdamConsts k = adam_consts(m->step_t + 1, c.lr, c.beta1, c.beta2, c.adam_eps);
  for (int u = 0; u < (int)m->unit_tensors.size(); ++u) adam_unit(m, u, k);
  m->step_t += 1;
  // every trainable gradient was zeroed by its unit; frozen tensors never hold gradients
  m->grads_zero = true;
  m->stats.step_ms = now_ms() - t0;
  return HOL_OK;
}

hol_status engine_get_routing(const hol_model* m, int layer, int32_t* ids, int64_t n) {
  if (m->NE <= 0) {
    set_error("hol_get_routing: the model has no mixture-of-experts layers");
    return HOL_EINVAL;
  }
  if (layer < 0 || layer >= m->L || m->last_T <= 0 || n != (int64_t)m->last_T * m->topk) {
    set_error("hol_get_routing: bad layer or n, or no forward_backward yet");
    return HOL_EINVAL;
  }
  HCHECK(hipSetDevice(m->cfg.device));
  HCHECK(hipMemcpy(ids, m->route_rec + (int64_t)layer * m->last_T * m->topk, (size_t)n * 4, hipMemcpyDeviceToHost));
  return HOL_OK;
}

hol_status engine_set_k(hol_model* m, int k) {
  if (k < 1 || k > m->Kmax) {
    set_error("hol_set_ckpt_every_k: k must be in [1, ckpt_every_k given at create]");
    return HOL_EINVAL;
  }
  m->K = k;
  m->nblocks = (m->L + k - 1) / k;
  return HOL_OK;
}

hol_status engine_set_kernel_timing(hol_model* m, bool on) {
  if (on && m->kev.empty()) {
    m->kev.resize(16384);
    for (auto& e : m->kev) HCHECK(hipEventCreate(&e));
  }
  m->ktiming = on;
  return HOL_OK;
}

hol_status engine_zero_grad(hol_model* m) {
  if (m->sc) hipStreamSynchronize(m->sc);
  if (m->sh2d) hipStreamSynchronize(m->sh2d);
  if (m->sd2h) hipStreamSynchronize(m->sd2h);
  parallel_zero(m->grad, m->n_flat * 4);
  m->grads_zero = true;
  m->grads_stale = false;
  m->poisoned = false;
  return HOL_OK;
}

std::string stats_json(const hol_model* m) {
  const Stats& s = m->stats;
  std::ostringstream o;
  o.precision(6);
  o << std::fixed;
  o << "{\"tokens\":" << s.tokens << ",\"fb_ms\":" << s.fb_ms << ",\"step_ms\":" << s.step_ms
    << ",\"h2d_bytes\":" << s.h2d_bytes << ",\"d2h_bytes\":" << s.d2h_bytes << ",\"h2d_busy_ms\":" << s.h2d_busy_ms
    << ",\"h2d_span_bytes\":" << s.h2d_span_bytes
    << ",\"d2h_busy_ms\":" << s.d2h_busy_ms << ",\"compute_busy_ms\":" << s.compute_busy_ms
    << ",\"fwd_ms\":" << s.fwd_ms << ",\"recomp_ms\":" << s.recomp_ms << ",\"bwd_ms\":" << s.bwd_ms
    << ",\"head_ms\":" << s.head_ms << ",\"host_embed_ms\":" << s.host_embed_ms
    << ",\"n_weight_streams\":" << s.n_weight_streams << ",\"layer_image_bytes\":" << m->layer_img_bytes
    << ",\"head_image_bytes\":" << m->head_img_bytes << ",\"host_threads\":" << pool_threads()
    << ",\"ring_segments\":" << m->nring << ",\"ring_segment_bytes\":" << m->ring_seg
    << ",\"staged_bytes\":" << s.staged_bytes << ",\"staging_ms\":" << s.staging_ms
    << ",\"gpu_done_ms\":" << s.gpu_done_ms << ",\"scatter_done_ms\":" << s.scatter_done_ms
    << ",\"worker_busy_ms\":" << s.worker_busy_ms << ",\"async_wait_ms\":" << s.async_wait_ms
    << ",\"first_compute_ms\":" << s.first_compute_ms
    << ",\"last_compute_end_ms\":" << s.last_compute_end_ms << ",\"units\":[";
  for (size_t i = 0; i < s.units.size(); ++i)
    o << (i ? "," : "") << "[" << (int)s.units[i][0] << "," << s.units[i][1] << "," << s.units[i][2] << "]";
  o << "],\"async_waits\":[";
  for (size_t i = 0; i < s.waits.size(); ++i)
    o << (i ? "," : "") << "[" << (int)s.waits[i][0] << "," << s.waits[i][1] << "," << s.waits[i][2] << "]";
  o << "],\"timeline\":[";
  for (size_t i = 0; i < s.timeline.size(); ++i)
    o << (i ? "," : "") << "[" << (int)s.timeline[i][0] << "," << s.timeline[i][1] << "," << s.timeline[i][2] << "]";
  o << "]";
  static const char* names[KC_N] = {"gemm", "attn_fwd", "attn_bwd", "rmsnorm", "rope", "swiglu", "ce", "transpose", "other"};
  o << ",\"kernels\":{";
  for (int c = 0; c < KC_N; ++c) {
    if (c) o << ",";
    o << "\"" << names[c] << "\":{\"launches\":" << s.k[c].launches << ",\"ms\":" << s.k[c].ms
      << ",\"flops\":" << s.k[c].flops << ",\"bytes\":" << s.k[c].bytes << "}";
  }
  o << "},\"gemm_shapes\":[";
  bool first = true;
  for (const auto& kv : s.gemm_shapes) {
    o << (first ? "" : ",") << "[" << kv.first[0] << "," << kv.first[1] << "," << kv.first[2] << ","
      << kv.second.launches << "," << kv.second.ms << "," << kv.second.flops << "]";
    first = false;
  }
  o << "]}";
  return o.str();
}

}  // namespace hol
