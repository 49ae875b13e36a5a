// Causal grouped-query attention of the decoder-layer template, forward and backward, tiled so
// the S x S score matrix is never materialised (MegaTrain summary page, 核心方法: the Attention
// block kernels of the layer template). Deterministic: dK/dV are owned by key-tile blocks that
// loop over the query tiles and over every q head of the kv group; dQ is owned by query-tile
// blocks; nothing is accumulated with atomics, so a recompute reproduces results bit for bit.
//
// This file holds the plain LDS-tiled version (fp32 arithmetic on fp32 or bf16 storage): tiles
// of 64 queries x 64 keys, 4 threads per row. It serves the fp32 path and head widths the matrix-
// core kernels (k_attn_mfma.hip: bf16, head width 64 or 128) do not take.
#include <mutex>

#include "device_common.h"
#include "kernels.h"

namespace hol {

constexpr int AT_B = 64;  // queries / keys per tile

__device__ __forceinline__ int64_t tok(int seq, int S, int i) { return (int64_t)seq * S + i; }

template <typename T>
__device__ __forceinline__ void load_tile(float* dst, int pitch, const T* src, int64_t ld, int64_t row0,
                                          int nrows, int d) {
  for (int e = threadIdx.x; e < AT_B * d; e += blockDim.x) {
    const int r = e / d, c = e % d;
    dst[r * pitch + c] = r < nrows ? to_f(src[(row0 + r) * ld + c]) : 0.f;
  }
}

// ---------------------------------------------------------------- forward
template <typename T>
__global__ __launch_bounds__(256) void attn_fwd_tiled(Attn a) {
  extern __shared__ float sm[];
  const int d = a.d, pitch = d + 1;
  float* Qs = sm;
  float* Ks = Qs + AT_B * pitch;
  float* Vs = Ks + AT_B * pitch;
  float* Ps = Vs + AT_B * pitch;  // [64][65]
  const int qt = blockIdx.x, h = blockIdx.y, seq = blockIdx.z;
  const int kvh = h / (a.nq / a.nkv);
  const int S = a.S;
  const int q0 = qt * AT_B;
  const int nqr = min(AT_B, S - q0);
  const float scale = 1.0f / sqrtf((float)d);
  const T* Q = (const T*)a.q + (int64_t)h * d;
  const T* K = (const T*)a.k + (int64_t)kvh * d;
  const T* V = (const T*)a.v + (int64_t)kvh * d;
  load_tile<T>(Qs, pitch, Q, a.ldq, tok(seq, S, q0), nqr, d);
  const int r = threadIdx.x >> 2, c = threadIdx.x & 3;
  const int qi = q0 + r;
  float m = -INFINITY, l = 0.f;
  float o[32];
  const int ne = (d + 3) / 4;
#pragma unroll
  for (int e = 0; e < 32; ++e) o[e] = 0.f;
  const int last_kt = (q0 + nqr - 1) / AT_B;
  for (int kt = 0; kt <= last_kt; ++kt) {
    const int k0 = kt * AT_B;
    const int nkr = min(AT_B, S - k0);
    __syncthreads();
    load_tile<T>(Ks, pitch, K, a.ldk, tok(seq, S, k0), nkr, d);
    load_tile<T>(Vs, pitch, V, a.ldv, tok(seq, S, k0), nkr, d);
    __syncthreads();
    float s[16];
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = c + 4 * i;
      const int kj = k0 + j;
      float acc = 0.f;
      for (int dd = 0; dd < d; ++dd) acc += Qs[r * pitch + dd] * Ks[j * pitch + dd];
      s[i] = (j < nkr && kj <= qi) ? acc * scale : -INFINITY;
      mt = fmaxf(mt, s[i]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 1, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 2, 64));
    const float mn = fmaxf(m, mt);
    const float corr = (m == -INFINITY) ? 0.f : __expf(m - mn);
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = (s[i] == -INFINITY) ? 0.f : __expf(s[i] - mn);
      ls += p;
      Ps[r * 65 + c + 4 * i] = p;
    }
    ls += __shfl_xor(ls, 1, 64);
    ls += __shfl_xor(ls, 2, 64);
    l = l * corr + ls;
    m = mn;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      if (e < ne) {
        const int dd = c + 4 * e;
        float acc = o[e] * corr;
        if (dd < d)
          for (int j = 0; j < AT_B; ++j) acc += Ps[r * 65 + j] * Vs[j * pitch + dd];
        o[e] = acc;
      }
    }
  }
  if (r < nqr) {
    T* O = (T*)a.o + tok(seq, S, qi) * a.ldo + (int64_t)h * d;
    const float inv = 1.f / l;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int dd = c + 4 * e;
      if (e < ne && dd < d) O[dd] = from_f<T>(o[e] * inv);
    }
    if (c == 0) a.lse[((int64_t)seq * a.nq + h) * S + qi] = m + __logf(l);
  }
}

// ---------------------------------------------------------------- backward
// delta[seq, h, i] = sum_d dO * O
template <typename T>
__global__ __launch_bounds__(256) void attn_delta_k(Attn a) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // over n_seq*S*nq
  const int lane = threadIdx.x & 63;
  const int64_t total = (int64_t)a.n_seq * a.S * a.nq;
  if (row >= total) return;
  const int h = (int)(row % a.nq);
  const int64_t t = row / a.nq;
  const T* o = (const T*)a.o + t * a.ldo + (int64_t)h * a.d;
  const T* g = (const T*)a.dO + t * a.lddo + (int64_t)h * a.d;
  float s = 0.f;
  for (int j = lane; j < a.d; j += 64) s += to_f(o[j]) * to_f(g[j]);
  s = wave_sum(s);
  const int seq = (int)(t / a.S), i = (int)(t % a.S);
  if (lane == 0) a.delta[((int64_t)seq * a.nq + h) * a.S + i] = s;
}

// dK, dV for one key tile of one kv head
template <typename T>
__global__ __launch_bounds__(256) void attn_dkdv_tiled(Attn a) {
  extern __shared__ float sm[];
  const int d = a.d, pitch = d + 1;
  float* Ks = sm;
  float* Vs = Ks + AT_B * pitch;
  float* Qs = Vs + AT_B * pitch;
  float* Gs = Qs + AT_B * pitch;  // dO tile
  float* Ps = Gs + AT_B * pitch;  // [key][query] 64 x 65
  const int kt = blockIdx.x, kvh = blockIdx.y, seq = blockIdx.z;
  const int group = a.nq / a.nkv;
  const int S = a.S, k0 = kt * AT_B, nkr = min(AT_B, S - k0);
  const float scale = 1.0f / sqrtf((float)d);
  load_tile<T>(Ks, pitch, (const T*)a.k + (int64_t)kvh * d, a.ldk, tok(seq, S, k0), nkr, d);
  load_tile<T>(Vs, pitch, (const T*)a.v + (int64_t)kvh * d, a.ldv, tok(seq, S, k0), nkr, d);
  const int j = threadIdx.x >> 2, c = threadIdx.x & 3;  // this thread's key row
  const int ne = (d + 3) / 4;
  float dk[32], dv[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) { dk[e] = 0.f; dv[e] = 0.f; }
  const int nqt = (S + AT_B - 1) / AT_B;
  for (int hh = 0; hh < group; ++hh) {
    const int h = kvh * group + hh;
    const float* lse = a.lse + ((int64_t)seq * a.nq + h) * S;
    const float* dl = a.delta + ((int64_t)seq * a.nq + h) * S;
    for (int qt = kt; qt < nqt; ++qt) {
      const int q0 = qt * AT_B, nqr = min(AT_B, S - q0);
      __syncthreads();
      load_tile<T>(Qs, pitch, (const T*)a.q + (int64_t)h * d, a.ldq, tok(seq, S, q0), nqr, d);
      load_tile<T>(Gs, pitch, (const T*)a.dO + (int64_t)h * d, a.lddo, tok(seq, S, q0), nqr, d);
      __syncthreads();
      // p[key j][query i] for queries i = c + 4 m
      float p[16];
#pragma unroll
      for (int mm = 0; mm < 16; ++mm) {
        const int i = c + 4 * mm;
        float acc = 0.f;
        for (int dd = 0; dd < d; ++dd) acc += Qs[i * pitch + dd] * Ks[j * pitch + dd];
        const bool ok = i < nqr && j < nkr && (k0 + j) <= (q0 + i);
        p[mm] = ok ? __expf(acc * scale - lse[q0 + i]) : 0.f;
        Ps[j * 65 + i] = p[mm];
      }
      __syncthreads();
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int dd = c + 4 * e;
        if (e < ne && dd < d) {
          float acc = dv[e];
          for (int i = 0; i < AT_B; ++i) acc += Ps[j * 65 + i] * Gs[i * pitch + dd];
          dv[e] = acc;
        }
      }
      // dS = P (dP - delta) * scale, dP[i][j] = dO_i . V_j
      float ds[16];
#pragma unroll
      for (int mm = 0; mm < 16; ++mm) {
        const int i = c + 4 * mm;
        float acc = 0.f;
        for (int dd = 0; dd < d; ++dd) acc += Gs[i * pitch + dd] * Vs[j * pitch + dd];
        ds[mm] = (i < nqr) ? p[mm] * (acc - dl[q0 + i]) * scale : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int mm = 0; mm < 16; ++mm) Ps[j * 65 + c + 4 * mm] = ds[mm];
      __syncthreads();
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int dd = c + 4 * e;
        if (e < ne && dd < d) {
          float acc = dk[e];
          for (int i = 0; i < AT_B; ++i) acc += Ps[j * 65 + i] * Qs[i * pitch + dd];
          dk[e] = acc;
        }
      }
    }
  }
  if (j < nkr) {
    T* DK = (T*)a.dk + tok(seq, S, k0 + j) * a.lddk + (int64_t)kvh * d;
    T* DV = (T*)a.dv + tok(seq, S, k0 + j) * a.lddv + (int64_t)kvh * d;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int dd = c + 4 * e;
      if (e < ne && dd < d) { DK[dd] = from_f<T>(dk[e]); DV[dd] = from_f<T>(dv[e]); }
    }
  }
}

// dQ for one query tile of one q head
template <typename T>
__global__ __launch_bounds__(256) void attn_dq_tiled(Attn a) {
  extern __shared__ float sm[];
  const int d = a.d, pitch = d + 1;
  float* Qs = sm;
  float* Gs = Qs + AT_B * pitch;
  float* Ks = Gs + AT_B * pitch;
  float* Vs = Ks + AT_B * pitch;
  float* Ps = Vs + AT_B * pitch;  // dS [query][key]
  const int qt = blockIdx.x, h = blockIdx.y, seq = blockIdx.z;
  const int kvh = h / (a.nq / a.nkv);
  const int S = a.S, q0 = qt * AT_B, nqr = min(AT_B, S - q0);
  const float scale = 1.0f / sqrtf((float)d);
  load_tile<T>(Qs, pitch, (const T*)a.q + (int64_t)h * d, a.ldq, tok(seq, S, q0), nqr, d);
  load_tile<T>(Gs, pitch, (const T*)a.dO + (int64_t)h * d, a.lddo, tok(seq, S, q0), nqr, d);
  const int i = threadIdx.x >> 2, c = threadIdx.x & 3;
  const int ne = (d + 3) / 4;
  const bool rv = i < nqr;
  const float lse_i = rv ? a.lse[((int64_t)seq * a.nq + h) * S + q0 + i] : 0.f;
  const float dl_i = rv ? a.delta[((int64_t)seq * a.nq + h) * S + q0 + i] : 0.f;
  float dq[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) dq[e] = 0.f;
  for (int kt = 0; kt <= qt; ++kt) {
    const int k0 = kt * AT_B, nkr = min(AT_B, S - k0);
    __syncthreads();
    load_tile<T>(Ks, pitch, (const T*)a.k + (int64_t)kvh * d, a.ldk, tok(seq, S, k0), nkr, d);
    load_tile<T>(Vs, pitch, (const T*)a.v + (int64_t)kvh * d, a.ldv, tok(seq, S, k0), nkr, d);
    __syncthreads();
#pragma unroll
    for (int mm = 0; mm < 16; ++mm) {
      const int j = c + 4 * mm;
      float s = 0.f, dp = 0.f;
      for (int dd = 0; dd < d; ++dd) {
        s += Qs[i * pitch + dd] * Ks[j * pitch + dd];
        dp += Gs[i * pitch + dd] * Vs[j * pitch + dd];
      }
      const bool ok = rv && j < nkr && (k0 + j) <= (q0 + i);
      const float p = ok ? __expf(s * scale - lse_i) : 0.f;
      Ps[i * 65 + j] = p * (dp - dl_i) * scale;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int dd = c + 4 * e;
      if (e < ne && dd < d) {
        float acc = dq[e];
        for (int j = 0; j < AT_B; ++j) acc += Ps[i * 65 + j] * Ks[j * pitch + dd];
        dq[e] = acc;
      }
    }
  }
  if (rv) {
    T* DQ = (T*)a.dq + tok(seq, S, q0 + i) * a.lddq + (int64_t)h * d;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int dd = c + 4 * e;
      if (e < ne && dd < d) DQ[dd] = from_f<T>(dq[e]);
    }
  }
}

bool attn_mfma_supported(const Attn& a);
bool attn_mfma_bwd_supported(const Attn& a);
int launch_attn_fwd_mfma(const Attn& a, hipStream_t s);
int launch_attn_bwd_mfma(const Attn& a, hipStream_t s);

static size_t tiled_smem(int d) { return (size_t)(4 * AT_B * (d + 1) + AT_B * 65) * sizeof(float); }

template <typename K>
static void allow_smem(K kern, size_t bytes) {
  (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

int launch_attn_fwd(const Attn& a, hipStream_t s) {
  if (a.n_seq <= 0 || a.S <= 0) return 0;
  if (a.d > 128 || a.nkv <= 0 || a.nq % a.nkv) return (int)hipErrorInvalidValue;
  if (attn_mfma_supported(a)) return launch_attn_fwd_mfma(a, s);
  const size_t sm = tiled_smem(a.d) - AT_B * (a.d + 1) * sizeof(float);
  dim3 grid((a.S + AT_B - 1) / AT_B, a.nq, a.n_seq);
  if (a.t == DT_BF16) {
    allow_smem(attn_fwd_tiled<bf16>, sm);
    hipLaunchKernelGGL(attn_fwd_tiled<bf16>, grid, dim3(256), sm, s, a);
  } else {
    allow_smem(attn_fwd_tiled<float>, sm);
    hipLaunchKernelGGL(attn_fwd_tiled<float>, grid, dim3(256), sm, s, a);
  }
  return (int)hipGetLastError();
}

// The RoPE backward of dq and dk for the kernels that do not apply it in their epilogue.
static int attn_rope_back(const Attn& a, hipStream_t s) {
  if (!a.rope_cos) return 0;
  const int T = a.n_seq * a.S;
  int e = launch_rope(a.dq, a.t, a.lddq, T, a.nq, a.d, a.S, a.rope_cos, a.rope_sin, true, s);
  if (e) return e;
  return launch_rope(a.dk, a.t, a.lddk, T, a.nkv, a.d, a.S, a.rope_cos, a.rope_sin, true, s);
}

int launch_attn_bwd(const Attn& a, hipStream_t s) {
  if (a.n_seq <= 0 || a.S <= 0) return 0;
  if (a.d > 128 || a.nkv <= 0 || a.nq % a.nkv) return (int)hipErrorInvalidValue;
  if (a.rope_cos && a.d % 2) return (int)hipErrorInvalidValue;
  if (attn_mfma_bwd_supported(a)) {
    const int e = launch_attn_bwd_mfma(a, s);  // (head width 128: the RoPE backward is in its epilogues)
    if (e || a.d == 128) return e;
    return attn_rope_back(a, s);
  }
  const size_t sm = tiled_smem(a.d);
  const int64_t rows = (int64_t)a.n_seq * a.S * a.nq;
  const int nt = (a.S + AT_B - 1) / AT_B;
  if (a.t == DT_BF16) {
    hipLaunchKernelGGL(attn_delta_k<bf16>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
    allow_smem(attn_dkdv_tiled<bf16>, sm);
    allow_smem(attn_dq_tiled<bf16>, sm);
    hipLaunchKernelGGL(attn_dkdv_tiled<bf16>, dim3(nt, a.nkv, a.n_seq), dim3(256), sm, s, a);
    hipLaunchKernelGGL(attn_dq_tiled<bf16>, dim3(nt, a.nq, a.n_seq), dim3(256), sm, s, a);
  } else {
    hipLaunchKernelGGL(attn_delta_k<float>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
    allow_smem(attn_dkdv_tiled<float>, sm);
    allow_smem(attn_dq_tiled<float>, sm);
    hipLaunchKernelGGL(attn_dkdv_tiled<float>, dim3(nt, a.nkv, a.n_seq), dim3(256), sm, s, a);
    hipLaunchKernelGGL(attn_dq_tiled<float>, dim3(nt, a.nq, a.n_seq), dim3(256), sm, s, a);
  }
  const int e = (int)hipGetLastError();
  if (e) return e;
  return attn_rope_back(a, s);
}


// ---------------------------------------------------------------- allocation-free backward
// The row sums delta of the backward live in this file-scope device array (16 MiB on every GPU the
// library runs on, held until the process ends) instead of a caller's workspace. Host code never
// passes the array's name to a kernel: each device's address of it is looked up once, with that
// device current, and kept.
static __device__ __align__(256) float scratch[ATTN_SCRATCH_FLOATS];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_dev[kMaxDevices] = {};
}  // namespace

static int scratch_address(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    g_scratch_dev[dev] = (float*)p;
  }
  *out = g_scratch_dev[dev];
  return 0;
}

int launch_attn_bwd_noalloc(Attn a, hipStream_t s) {
  if ((int64_t)a.n_seq * a.nq * a.S > ATTN_SCRATCH_FLOATS) return (int)hipErrorInvalidValue;
  float* p = nullptr;
  const int e = scratch_address(&p);
  if (e) return e;
  a.delta = p;  // every row sum is written by the delta kernel before the gradient kernels read it
  return launch_attn_bwd(a, s);
}

}  // namespace hol
