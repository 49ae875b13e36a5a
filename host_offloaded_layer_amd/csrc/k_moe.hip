// Mixture-of-experts MLP kernels of the decoder-layer template: router softmax with top-k
// selection, token permutation into expert-contiguous rows, the weighted combine, and their
// backward (routing weights, un-permutation, router softmax Jacobian).
//
// Reading of the routing (the pages name a mixture-of-experts model but not its router): softmax
// over the E router logits, the k largest probabilities (ties to the lower expert index), the
// kept probabilities renormalised to sum to one, no capacity limit and no token dropping.
//
// Layout: logits / probs fp32 [T, E]; ids int32 and w fp32 [T, k] (slot i of token t at t*k+i).
// A routed row p in [0, T*k) belongs to expert e when offsets[e] <= p < offsets[e+1];
// perm_slot[p] = t*k+i names the slot it came from and slot_pos[t*k+i] = p is the inverse. The
// rows of an expert keep the order of their slots, so the permutation (and every sum over an
// expert's rows) is the same on every call and in the recompute.
#include "device_common.h"
#include "kernels.h"

namespace hol {

constexpr int MOE_MAX_E = 512;   // experts per lane register budget: 8 x 64 lanes
constexpr int MOE_MAX_K = 16;

__global__ void fill_i32_k(int32_t* x, int32_t v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) x[i] = v;
}

// One wavefront per token. Lane l owns experts l, l+64, ... (at most 8).
__global__ __launch_bounds__(256) void moe_route_k(const float* __restrict__ logits, int T, int E, int k,
                                                   float* __restrict__ probs, int32_t* __restrict__ ids,
                                                   float* __restrict__ w, int32_t* __restrict__ counts) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  const float* lr = logits + (int64_t)t * E;
  float p[8];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int e = lane + 64 * j;
    p[j] = e < E ? lr[e] : -INFINITY;
    mx = fmaxf(mx, p[j]);
  }
  mx = wave_max(mx);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int e = lane + 64 * j;
    p[j] = e < E ? expf(p[j] - mx) : 0.f;
    s += p[j];
  }
  s = wave_sum(s);
  float* pr = probs + (int64_t)t * E;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int e = lane + 64 * j;
    if (e < E) {
      p[j] = p[j] / s;
      pr[e] = p[j];
      if (!(p[j] >= 0.f)) p[j] = 0.f;   // NaN (non-finite logits): still selectable, so every id is valid
    } else {
      p[j] = -1.f;   // never selected: every valid candidate is >= 0
    }
  }
  // k rounds of (max probability, lowest index) over the experts not yet taken; the butterfly
  // leaves the same winner in every lane, and lane r keeps the winner of round r
  int my_e = 0;
  float my_p = 0.f, ks = 0.f;
  for (int r = 0; r < k; ++r) {
    float bv = -2.f;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = lane + 64 * j;
      if (p[j] > bv) { bv = p[j]; bi = e; }   // ascending e within the lane: strict > keeps the lower index
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (lane == r) { my_e = bi; my_p = bv; }
    ks += bv;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (lane + 64 * j == bi) p[j] = -1.f;
  }
  if (lane < k) {
    ids[(int64_t)t * k + lane] = my_e;
    w[(int64_t)t * k + lane] = my_p / ks;
    atomicAdd(&counts[my_e], 1);
  }
}

// offsets[e] = sum_{e' < e} counts[e'], offsets[E] = total. One thread.
__global__ void moe_offsets_k(const int32_t* __restrict__ counts, int E, int32_t* __restrict__ offsets) {
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  int32_t acc = 0;
  for (int e = 0; e < E; ++e) {
    offsets[e] = acc;
    acc += counts[e];
  }
  offsets[E] = acc;
}

// Stable permutation: inside an expert, routed rows keep the order of their slots (t k + i), so
// every sum over an expert's rows (its weight gradients) is taken in one fixed order.
// Pass 1: per chunk of MOE_CH slots, how many go to each expert (cc [n_chunks, E]).
constexpr int MOE_CH = 256;
__global__ __launch_bounds__(256) void moe_chunk_count_k(const int32_t* __restrict__ ids, int64_t n, int E,
                                                         int32_t* __restrict__ cc) {
  __shared__ int32_t hist[MOE_MAX_E];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int64_t q = (int64_t)blockIdx.x * MOE_CH + threadIdx.x;
  if (threadIdx.x < MOE_CH && q < n) atomicAdd(&hist[ids[q]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) cc[(int64_t)blockIdx.x * E + e] = hist[e];
}
// Pass 2: first position of each (chunk, expert): co[c][e] = offsets[e] + sum_{c' < c} cc[c'][e].
__global__ void moe_chunk_offsets_k(const int32_t* __restrict__ cc, int nch, int E, const int32_t* __restrict__ offsets,
                                    int32_t* __restrict__ co) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  int32_t acc = offsets[e];
  for (int c = 0; c < nch; ++c) {
    co[(int64_t)c * E + e] = acc;
    acc += cc[(int64_t)c * E + e];
  }
}
// Pass 3: one thread per chunk walks its slots in order.
__global__ __launch_bounds__(64) void moe_chunk_scatter_k(const int32_t* __restrict__ ids, int64_t n, int E,
                                                          const int32_t* __restrict__ co, int32_t* __restrict__ perm_slot,
                                                          int32_t* __restrict__ slot_pos) {
  __shared__ int32_t cur[MOE_MAX_E];
  for (int e = threadIdx.x; e < E; e += blockDim.x) cur[e] = co[(int64_t)blockIdx.x * E + e];
  __syncthreads();
  if (threadIdx.x != 0) return;
  const int64_t q0 = (int64_t)blockIdx.x * MOE_CH, q1 = q0 + MOE_CH < n ? q0 + MOE_CH : n;
  for (int64_t q = q0; q < q1; ++q) {
    const int p = cur[ids[q]]++;
    perm_slot[p] = (int32_t)q;
    slot_pos[q] = p;
  }
}

// Xp[p, :] = X[perm_slot[p] / k, :]; rows of H elements (H * sizeof(T) a multiple of 16 bytes).
template <typename T>
__global__ __launch_bounds__(256) void moe_gather_k(const T* __restrict__ X, const int32_t* __restrict__ perm_slot,
                                                    int k, int64_t n_rows, int H, T* __restrict__ Xp) {
  const int64_t p = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (p >= n_rows) return;
  const int64_t t = perm_slot[p] / k;
  const uint4* src = (const uint4*)(X + t * H);
  uint4* dst = (uint4*)(Xp + p * H);
  const int nv = H * (int)sizeof(T) / 16;
  for (int j = lane; j < nv; j += 64) dst[j] = src[j];
}

// hout[t, :] = h1[t, :] + sum_i w[t, i] Yp[slot_pos[t k + i], :]   (fp32; one block per token)
__global__ __launch_bounds__(256) void moe_combine_k(const float* __restrict__ h1, const float* __restrict__ Yp,
                                                     const float* __restrict__ w, const int32_t* __restrict__ slot_pos,
                                                     int k, int H, float* __restrict__ hout) {
  const int64_t t = blockIdx.x;
  __shared__ int32_t pos[MOE_MAX_K];
  __shared__ float wt[MOE_MAX_K];
  if (threadIdx.x < k) {
    pos[threadIdx.x] = slot_pos[t * k + threadIdx.x];
    wt[threadIdx.x] = w[t * k + threadIdx.x];
  }
  __syncthreads();
  for (int j = threadIdx.x; j < H; j += blockDim.x) {
    float acc = 0.f;
    for (int i = 0; i < k; ++i) acc += wt[i] * Yp[(int64_t)pos[i] * H + j];
    hout[t * H + j] = h1[t * H + j] + acc;
  }
}

// Backward of the combine for one token: dw[t, i] = <dh[t], Yp[p_i]>, dYp[p_i] = w[t, i] dh[t].
template <typename T>
__global__ __launch_bounds__(256) void moe_combine_bwd_k(const float* __restrict__ dh, const float* __restrict__ Yp,
                                                         const float* __restrict__ w,
                                                         const int32_t* __restrict__ slot_pos, int k, int H,
                                                         float* __restrict__ dw, T* __restrict__ dYp) {
  const int64_t t = blockIdx.x;
  __shared__ float red[16];
  const float* g = dh + t * H;
  for (int i = 0; i < k; ++i) {
    const int64_t p = slot_pos[t * k + i];
    const float wi = w[t * k + i];
    float acc = 0.f;
    for (int j = threadIdx.x; j < H; j += blockDim.x) {
      const float gj = g[j];
      acc += gj * Yp[p * H + j];
      dYp[p * H + j] = from_f<T>(wi * gj);
    }
    acc = block_sum(acc, red);
    if (threadIdx.x == 0) dw[t * k + i] = acc;
  }
}

// dn[t, :] = sum_i dXp[slot_pos[t k + i], :]   (fp32; one block per token)
__global__ __launch_bounds__(256) void moe_unpermute_k(const float* __restrict__ dXp, const int32_t* __restrict__ slot_pos,
                                                       int k, int H, float* __restrict__ dn) {
  const int64_t t = blockIdx.x;
  __shared__ int32_t pos[MOE_MAX_K];
  if (threadIdx.x < k) pos[threadIdx.x] = slot_pos[t * k + threadIdx.x];
  __syncthreads();
  for (int j = threadIdx.x; j < H; j += blockDim.x) {
    float acc = 0.f;
    for (int i = 0; i < k; ++i) acc += dXp[(int64_t)pos[i] * H + j];
    dn[t * H + j] = acc;
  }
}

// Router backward for one token (one wavefront): renormalisation w_i = p_i / s (s = sum of the
// kept p) gives dp_i = (dw_i - sum_j dw_j w_j) / s on the kept experts and 0 elsewhere; the
// softmax Jacobian gives dlogits_e = p_e (dp_e - sum_j dp_j p_j).
template <typename T>
__global__ __launch_bounds__(256) void moe_router_bwd_k(const float* __restrict__ probs, const int32_t* __restrict__ ids,
                                                        const float* __restrict__ w, const float* __restrict__ dw,
                                                        int T_, int E, int k, T* __restrict__ dlogits) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T_) return;
  const float* pr = probs + (int64_t)t * E;
  float ssum = 0.f, sdw = 0.f;
  for (int i = 0; i < k; ++i) {
    ssum += pr[ids[(int64_t)t * k + i]];
    sdw += dw[(int64_t)t * k + i] * w[(int64_t)t * k + i];
  }
  // sum_j dp_j p_j over the kept experts
  float sdp = 0.f;
  for (int i = 0; i < k; ++i) {
    const float dpi = (dw[(int64_t)t * k + i] - sdw) / ssum;
    sdp += dpi * pr[ids[(int64_t)t * k + i]];
  }
  for (int e = lane; e < E; e += 64) {
    float dp = 0.f;
    for (int i = 0; i < k; ++i)
      if (ids[(int64_t)t * k + i] == e) dp = (dw[(int64_t)t * k + i] - sdw) / ssum;
    dlogits[(int64_t)t * E + e] = from_f<T>(pr[e] * (dp - sdp));
  }
}

// ------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------
int launch_fill_i32(int32_t* x, int32_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(fill_i32_k, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, v, n);
  return (int)hipGetLastError();
}

int launch_moe_route(const float* logits, int T, int E, int k, float* probs, int32_t* ids, float* w,
                     int32_t* counts, hipStream_t s) {
  if (T <= 0) return 0;
  if (E < 1 || E > MOE_MAX_E || k < 1 || k > E || k > MOE_MAX_K) return (int)hipErrorInvalidValue;
  int rc = launch_fill_i32(counts, 0, E, s);
  if (rc) return rc;
  hipLaunchKernelGGL(moe_route_k, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, probs, ids, w, counts);
  return (int)hipGetLastError();
}

int64_t moe_permute_scratch(int T, int E, int k) {
  const int64_t n = (int64_t)T * k;
  return 2 * ((n + MOE_CH - 1) / MOE_CH) * E;
}

int launch_moe_permute(const int32_t* ids, int T, int E, int k, const int32_t* counts, int32_t* offsets,
                       int32_t* scratch, int32_t* perm_slot, int32_t* slot_pos, hipStream_t s) {
  if (T <= 0) return 0;
  if (E < 1 || E > MOE_MAX_E) return (int)hipErrorInvalidValue;
  const int64_t n = (int64_t)T * k;
  const int nch = (int)((n + MOE_CH - 1) / MOE_CH);
  int32_t* cc = scratch;
  int32_t* co = scratch + (int64_t)nch * E;
  hipLaunchKernelGGL(moe_offsets_k, dim3(1), dim3(64), 0, s, counts, E, offsets);
  hipLaunchKernelGGL(moe_chunk_count_k, dim3(nch), dim3(256), 0, s, ids, n, E, cc);
  hipLaunchKernelGGL(moe_chunk_offsets_k, dim3((E + 255) / 256), dim3(256), 0, s, cc, nch, E, offsets, co);
  hipLaunchKernelGGL(moe_chunk_scatter_k, dim3(nch), dim3(64), 0, s, ids, n, E, co, perm_slot, slot_pos);
  return (int)hipGetLastError();
}

int launch_moe_gather(const void* X, DType t, const int32_t* perm_slot, int k, int64_t n_rows, int H, void* Xp,
                      hipStream_t s) {
  if (n_rows <= 0) return 0;
  if ((H * (t == DT_BF16 ? 2 : 4)) % 16 || ((uintptr_t)X | (uintptr_t)Xp) % 16) return (int)hipErrorInvalidValue;
  dim3 grid((unsigned)((n_rows + 3) / 4));
  if (t == DT_BF16)
    hipLaunchKernelGGL(moe_gather_k<bf16>, grid, dim3(256), 0, s, (const bf16*)X, perm_slot, k, n_rows, H, (bf16*)Xp);
  else
    hipLaunchKernelGGL(moe_gather_k<float>, grid, dim3(256), 0, s, (const float*)X, perm_slot, k, n_rows, H, (float*)Xp);
  return (int)hipGetLastError();
}

int launch_moe_combine(const float* h1, const float* Yp, const float* w, const int32_t* slot_pos, int T, int k, int H,
                       float* hout, hipStream_t s) {
  if (T <= 0) return 0;
  if (k > MOE_MAX_K) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(moe_combine_k, dim3(T), dim3(256), 0, s, h1, Yp, w, slot_pos, k, H, hout);
  return (int)hipGetLastError();
}

int launch_moe_combine_bwd(const float* dh, const float* Yp, const float* w, const int32_t* slot_pos, int T, int k,
                           int H, float* dw, void* dYp, DType t, hipStream_t s) {
  if (T <= 0) return 0;
  if (k > MOE_MAX_K) return (int)hipErrorInvalidValue;
  if (t == DT_BF16)
    hipLaunchKernelGGL(moe_combine_bwd_k<bf16>, dim3(T), dim3(256), 0, s, dh, Yp, w, slot_pos, k, H, dw, (bf16*)dYp);
  else
    hipLaunchKernelGGL(moe_combine_bwd_k<float>, dim3(T), dim3(256), 0, s, dh, Yp, w, slot_pos, k, H, dw, (float*)dYp);
  return (int)hipGetLastError();
}

int launch_moe_unpermute(const float* dXp, const int32_t* slot_pos, int T, int k, int H, float* dn, hipStream_t s) {
  if (T <= 0) return 0;
  if (k > MOE_MAX_K) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(moe_unpermute_k, dim3(T), dim3(256), 0, s, dXp, slot_pos, k, H, dn);
  return (int)hipGetLastError();
}

int launch_moe_router_bwd(const float* probs, const int32_t* ids, const float* w, const float* dw, int T, int E, int k,
                          void* dlogits, DType t, hipStream_t s) {
  if (T <= 0) return 0;
  dim3 grid((T + 3) / 4);
  if (t == DT_BF16)
    hipLaunchKernelGGL(moe_router_bwd_k<bf16>, grid, dim3(256), 0, s, probs, ids, w, dw, T, E, k, (bf16*)dlogits);
  else
    hipLaunchKernelGGL(moe_router_bwd_k<float>, grid, dim3(256), 0, s, probs, ids, w, dw, T, E, k, (float*)dlogits);
  return (int)hipGetLastError();
}

}  // namespace hol
