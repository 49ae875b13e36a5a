// Row-wise and elementwise kernels of the decoder-layer template: RMSNorm forward/backward, RoPE,
// SwiGLU, casts, the next-token cross entropy of the loss anchor and the sum-of-squares loss.
// All are HBM-bound: one wavefront per row, 16-byte vector accesses, wavefront reductions, and
// deterministic two-stage reductions (no atomics) for the RMSNorm gain gradient.
#include "device_common.h"
#include "kernels.h"

#include <initializer_list>

namespace hol {

// ------------------------------------------------------------------------------------------
// RMSNorm
// ------------------------------------------------------------------------------------------
template <typename TO>
__device__ __forceinline__ void store4(TO* p, float4 v);
template <>
__device__ __forceinline__ void store4<float>(float* p, float4 v) { *(float4*)p = v; }
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, float4 v) {
  bf16x4 b = {(bf16)v.x, (bf16)v.y, (bf16)v.z, (bf16)v.w};
  *(bf16x4*)p = b;
}

// One wavefront per row; H % 4 == 0. For H <= 256 NV the row stays in registers between the
// sum of squares and the scaling, so x is read from HBM once; wider rows take two passes.
template <typename TO, int NV>
__global__ __launch_bounds__(256) void rmsnorm_fwd_k(const float* __restrict__ x, const float* __restrict__ g,
                                                     float eps, TO* __restrict__ y, float* __restrict__ rstd,
                                                     int T, int H) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= T) return;
  const float* xr = x + (int64_t)row * H;
  TO* yr = y + (int64_t)row * H;
  float ss = 0.f;
  if constexpr (NV > 0) {
    float4 xv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int j = lane * 4 + i * 256;
      xv[i] = j < H ? *(const float4*)(xr + j) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) ss += xv[i].x * xv[i].x + xv[i].y * xv[i].y + xv[i].z * xv[i].z + xv[i].w * xv[i].w;
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)H + eps);
    if (lane == 0) rstd[row] = r;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int j = lane * 4 + i * 256;
      if (j < H) {
        const float4 gg = *(const float4*)(g + j);
        store4<TO>(yr + j, make_float4(xv[i].x * r * gg.x, xv[i].y * r * gg.y, xv[i].z * r * gg.z, xv[i].w * r * gg.w));
      }
    }
  } else {
    for (int j = lane * 4; j < H; j += 256) {
      float4 v = *(const float4*)(xr + j);
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)H + eps);
    if (lane == 0) rstd[row] = r;
    for (int j = lane * 4; j < H; j += 256) {
      float4 v = *(const float4*)(xr + j);
      float4 gg = *(const float4*)(g + j);
      store4<TO>(yr + j, make_float4(v.x * r * gg.x, v.y * r * gg.y, v.z * r * gg.z, v.w * r * gg.w));
    }
  }
}

template <typename TO>
static void rmsnorm_fwd_dispatch(dim3 grid, hipStream_t s, const float* x, const float* gamma, float eps, TO* y,
                                 float* rstd, int T, int H) {
  const int nv = (H + 255) / 256;
#define RMSF(NV) hipLaunchKernelGGL((rmsnorm_fwd_k<TO, NV>), grid, dim3(256), 0, s, x, gamma, eps, y, rstd, T, H)
  if (nv <= 1) RMSF(1);
  else if (nv <= 2) RMSF(2);
  else if (nv <= 4) RMSF(4);
  else if (nv <= 8) RMSF(8);
  else if (nv <= 16) RMSF(16);
  else RMSF(0);
#undef RMSF
}

int launch_rmsnorm_fwd(const float* x, const float* gamma, float eps, void* y, DType yt, float* rstd,
                       int T, int H, hipStream_t s) {
  if (T <= 0) return 0;
  if (H % 4) return (int)hipErrorInvalidValue;
  dim3 grid((T + 3) / 4);
  if (yt == DT_BF16) rmsnorm_fwd_dispatch<bf16>(grid, s, x, gamma, eps, (bf16*)y, rstd, T, H);
  else rmsnorm_fwd_dispatch<float>(grid, s, x, gamma, eps, (float*)y, rstd, T, H);
  return (int)hipGetLastError();
}

constexpr int RMS_BWD_BLOCKS = 1024;
int rmsnorm_bwd_blocks(int T) { return T < RMS_BWD_BLOCKS * 4 ? (T + 3) / 4 : RMS_BWD_BLOCKS; }

// Wide rows (H >= 1024): one block of 256 threads per row, 4 NV columns a thread (columns
// 4 t + 1024 i), so a thread holds few registers and many waves share a CU; the row's dot
// product is a block reduction through a double-buffered 4-float LDS array (one barrier a row).
// A thread owns the same columns on every row, so its gain-gradient sums need no reduction.
template <int NV>
__global__ __launch_bounds__(256) void rmsnorm_bwd_row_k(const float* __restrict__ dy, const float* __restrict__ x,
                                                         const float* __restrict__ g, const float* __restrict__ rstd,
                                                         float* __restrict__ dx, int accumulate,
                                                         float* __restrict__ partial, int T, int H,
                                                         bf16* __restrict__ dxb) {
  __shared__ float red[2][4];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  float4 dg[NV], gv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j = tid * 4 + i * 1024;
    dg[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    gv[i] = j < H ? *(const float4*)(g + j) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  int par = 0;
  for (int row = blockIdx.x; row < T; row += gridDim.x, par ^= 1) {
    const float r = rstd[row];
    const float* xr = x + (int64_t)row * H;
    const float* dyr = dy + (int64_t)row * H;
    float* dxr = dx + (int64_t)row * H;
    float4 xv[NV], dv[NV], pv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int j = tid * 4 + i * 1024;
      const bool in = j < H;
      xv[i] = in ? *(const float4*)(xr + j) : make_float4(0.f, 0.f, 0.f, 0.f);
      dv[i] = in ? *(const float4*)(dyr + j) : make_float4(0.f, 0.f, 0.f, 0.f);
      pv[i] = in && accumulate ? *(const float4*)(dxr + j) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      dg[i].x += dv[i].x * xv[i].x * r; dg[i].y += dv[i].y * xv[i].y * r;
      dg[i].z += dv[i].z * xv[i].z * r; dg[i].w += dv[i].w * xv[i].w * r;
      dv[i].x *= gv[i].x; dv[i].y *= gv[i].y; dv[i].z *= gv[i].z; dv[i].w *= gv[i].w;
      dot += (dv[i].x * xv[i].x + dv[i].y * xv[i].y + dv[i].z * xv[i].z + dv[i].w * xv[i].w) * r;
    }
    dot = wave_sum(dot);
    if (lane == 0) red[par][w] = dot;
    __syncthreads();
    dot = ((red[par][0] + red[par][1]) + (red[par][2] + red[par][3])) / (float)H;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int j = tid * 4 + i * 1024;
      if (j < H) {
        float4 o;
        o.x = r * (dv[i].x - xv[i].x * r * dot) + pv[i].x; o.y = r * (dv[i].y - xv[i].y * r * dot) + pv[i].y;
        o.z = r * (dv[i].z - xv[i].z * r * dot) + pv[i].z; o.w = r * (dv[i].w - xv[i].w * r * dot) + pv[i].w;
        *(float4*)(dxr + j) = o;
        if (dxb) {
          const bf16x4 ob = {(bf16)o.x, (bf16)o.y, (bf16)o.z, (bf16)o.w};
          *(bf16x4*)(dxb + (int64_t)row * H + j) = ob;
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j = tid * 4 + i * 1024;
    if (j < H) *(float4*)(partial + (int64_t)blockIdx.x * H + j) = dg[i];
  }
}

// Each block handles rows blockIdx.x*4 + wave, stepping by gridDim.x*4; NV = float4s per lane.
template <int NV>
__global__ __launch_bounds__(256) void rmsnorm_bwd_k(const float* __restrict__ dy, const float* __restrict__ x,
                                                     const float* __restrict__ g, const float* __restrict__ rstd,
                                                     float* __restrict__ dx, int accumulate,
                                                     float* __restrict__ partial, int T, int H,
                                                     bf16* __restrict__ dxb) {
  __shared__ float red[4][NV * 256];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float4 dg[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) dg[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int row = blockIdx.x * 4 + w; row < T; row += gridDim.x * 4) {
    const float r = rstd[row];
    const float* xr = x + (int64_t)row * H;
    const float* dyr = dy + (int64_t)row * H;
    float* dxr = dx + (int64_t)row * H;
    float4 xv[NV], dv[NV];
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int j = lane * 4 + i * 256;
      if (j < H) {
        xv[i] = *(const float4*)(xr + j);
        dv[i] = *(const float4*)(dyr + j);
        const float4 gg = *(const float4*)(g + j);
        // xhat = x r ; dxhat = dy g ; accumulate dg += dy xhat and dot += dxhat xhat
        dg[i].x += dv[i].x * xv[i].x * r; dg[i].y += dv[i].y * xv[i].y * r;
        dg[i].z += dv[i].z * xv[i].z * r; dg[i].w += dv[i].w * xv[i].w * r;
        dv[i].x *= gg.x; dv[i].y *= gg.y; dv[i].z *= gg.z; dv[i].w *= gg.w;
        dot += (dv[i].x * xv[i].x + dv[i].y * xv[i].y + dv[i].z * xv[i].z + dv[i].w * xv[i].w) * r;
      }
    }
    dot = wave_sum(dot) / (float)H;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int j = lane * 4 + i * 256;
      if (j < H) {
        float4 o;
        o.x = r * (dv[i].x - xv[i].x * r * dot); o.y = r * (dv[i].y - xv[i].y * r * dot);
        o.z = r * (dv[i].z - xv[i].z * r * dot); o.w = r * (dv[i].w - xv[i].w * r * dot);
        if (accumulate) {
          const float4 p = *(const float4*)(dxr + j);
          o.x += p.x; o.y += p.y; o.z += p.z; o.w += p.w;
        }
        *(float4*)(dxr + j) = o;
        if (dxb) {
          const bf16x4 ob = {(bf16)o.x, (bf16)o.y, (bf16)o.z, (bf16)o.w};
          *(bf16x4*)(dxb + (int64_t)row * H + j) = ob;
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) *(float4*)&red[w][lane * 4 + i * 256] = dg[i];
  __syncthreads();
  for (int j = threadIdx.x; j < H; j += 256)
    partial[(int64_t)blockIdx.x * H + j] = (red[0][j] + red[1][j]) + (red[2][j] + red[3][j]);
}

// out[j] += sum_b partial[b][j]: a block of 16 waves owns 64 columns (one per lane); wave w sums
// rows w, w + 16, ..., then the 16 wave sums are added in a fixed order. The loads of 8 rows go
// out before their adds (same order of additions, same bits): with one load in flight per wave
// the 16 MB of partial sums at the LLaMA-8B shape (1024 x 4096) took ≈17 µs, with 8 ≈5.5 µs.
__global__ __launch_bounds__(1024) void reduce_cols_add_k(const float* __restrict__ partial, int nb, int H,
                                                          float* __restrict__ out) {
  __shared__ float red[16][64];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = blockIdx.x * 64 + lane;
  float s = 0.f;
  if (j < H) {
    int b = w;
    for (; b + 16 * 7 < nb; b += 16 * 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = partial[(int64_t)(b + 16 * u) * H + j];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; b < nb; b += 16) s += partial[(int64_t)b * H + j];
  }
  red[w][lane] = s;
  __syncthreads();
  if (w == 0 && j < H) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) t += red[i][lane];
    out[j] += t;
  }
}

int launch_rmsnorm_bwd(const float* dy, const float* x, const float* gamma, const float* rstd, float* dx_out,
                       bool accumulate, float* dgamma_acc, float* partial, int T, int H, hipStream_t s,
                       void* dx_bf16) {
  if (T <= 0) return 0;
  if (H % 4 || H > 4096) return (int)hipErrorInvalidValue;
  if ((uintptr_t)dx_bf16 % 8) return (int)hipErrorInvalidValue;
  bf16* dxb = (bf16*)dx_bf16;
  const int nb = rmsnorm_bwd_blocks(T);
  if (H >= 1024) {
#define RR(NVV)                                                                                       \
  hipLaunchKernelGGL(rmsnorm_bwd_row_k<NVV>, dim3(nb), dim3(256), 0, s, dy, x, gamma, rstd, dx_out, \
                     (int)accumulate, partial, T, H, dxb)
    if (H <= 2048) RR(2);
    else RR(4);
#undef RR
    if (dgamma_acc) hipLaunchKernelGGL(reduce_cols_add_k, dim3((H + 63) / 64), dim3(1024), 0, s, partial, nb, H, dgamma_acc);
    return (int)hipGetLastError();
  }
  const int nv = (H + 255) / 256;
#define RB(NVV)                                                                                   \
  hipLaunchKernelGGL(rmsnorm_bwd_k<NVV>, dim3(nb), dim3(256), 0, s, dy, x, gamma, rstd, dx_out, \
                     (int)accumulate, partial, T, H, dxb)
  if (nv <= 1) RB(1);
  else if (nv <= 2) RB(2);
  else if (nv <= 4) RB(4);
  else if (nv <= 8) RB(8);
  else RB(16);
#undef RB
  if (dgamma_acc) hipLaunchKernelGGL(reduce_cols_add_k, dim3((H + 63) / 64), dim3(1024), 0, s, partial, nb, H, dgamma_acc);
  return (int)hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// RoPE (rotate-half). One thread per rotated pair.
// ------------------------------------------------------------------------------------------
template <typename T>
__global__ void rope_k(T* __restrict__ x, int64_t ld, int Tn, int heads, int d, int S,
                       const float* __restrict__ cs, const float* __restrict__ sn, float sgn) {
  const int half = d >> 1;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)Tn * heads * half;
  if (i >= total) return;
  const int j = (int)(i % half);
  const int64_t th = i / half;
  const int h = (int)(th % heads);
  const int64_t t = th / heads;
  const int p = (int)(t % S);
  T* row = x + t * ld + (int64_t)h * d;
  const float c = cs[(int64_t)p * half + j], s_ = sgn * sn[(int64_t)p * half + j];
  const float a = to_f(row[j]), b = to_f(row[j + half]);
  row[j] = from_f<T>(a * c - b * s_);
  row[j + half] = from_f<T>(b * c + a * s_);
}

int launch_rope(void* x, DType xt, int64_t ld, int T, int heads, int d, int S, const float* cos_t,
                const float* sin_t, bool inverse, hipStream_t s) {
  const int64_t total = (int64_t)T * heads * (d / 2);
  if (total <= 0) return 0;
  const float sgn = inverse ? -1.f : 1.f;
  dim3 grid((unsigned)((total + 255) / 256));
  if (xt == DT_BF16) hipLaunchKernelGGL(rope_k<bf16>, grid, dim3(256), 0, s, (bf16*)x, ld, T, heads, d, S, cos_t, sin_t, sgn);
  else hipLaunchKernelGGL(rope_k<float>, grid, dim3(256), 0, s, (float*)x, ld, T, heads, d, S, cos_t, sin_t, sgn);
  return (int)hipGetLastError();
}

// RoPE fused with the cast of the projection output: in = fp32 [T, QKV] rows (q heads, k heads,
// v heads), out = bf16 rows with q and k rotated; one rounding per element. One thread per pair.
// (rot_pair, one rotated pair, lives in device_common.h: the q/k/v GEMM epilogue shares it)

__global__ void rope_qkv_k(const float* __restrict__ in, int64_t ldi, bf16* __restrict__ out, int64_t ldo, int Tn,
                           int nq, int nkv, int d, int S, const float* __restrict__ cs, const float* __restrict__ sn) {
  const int half = d >> 1;
  const int heads = nq + 2 * nkv;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)Tn * heads * half;
  if (i >= total) return;
  const int j = (int)(i % half);
  const int64_t th = i / half;
  const int h = (int)(th % heads);
  const int64_t t = th / heads;
  const float* r = in + t * ldi + (int64_t)h * d;
  bf16* o = out + t * ldo + (int64_t)h * d;
  const float a = r[j], b = r[j + half];
  if (h < nq + nkv) {
    const int p = (int)(t % S);
    float x, y;
    rot_pair(a, b, cs[(int64_t)p * half + j], sn[(int64_t)p * half + j], x, y);
    o[j] = (bf16)x;
    o[j + half] = (bf16)y;
  } else {
    o[j] = (bf16)a;
    o[j + half] = (bf16)b;
  }
}

// Four consecutive pairs per thread (16-byte fp32 loads, 8-byte bf16 stores); the same rounding
// as the one-pair kernel. Needs half % 4 == 0, 16-byte aligned input rows, 8-byte aligned output
// rows and fewer than 2^31 units.
__global__ __launch_bounds__(256) void rope_qkv4_k(const float* __restrict__ in, int64_t ldi, bf16* __restrict__ out,
                                                   int64_t ldo, uint32_t units, uint32_t h4, uint32_t heads, int nrot,
                                                   int d, int S, const float* __restrict__ cs,
                                                   const float* __restrict__ sn) {
  const uint32_t u = blockIdx.x * 256u + threadIdx.x;
  if (u >= units) return;
  const int half = d >> 1;
  const uint32_t th = u / h4, j = (u - th * h4) * 4;
  const uint32_t t = th / heads, h = th - t * heads;
  const float* r = in + (int64_t)t * ldi + (int64_t)h * d;
  bf16* o = out + (int64_t)t * ldo + (int64_t)h * d;
  const float4 a = *(const float4*)(r + j), b = *(const float4*)(r + j + half);
  bf16x4 x, y;
  if ((int)h < nrot) {
    const int64_t pc = (int64_t)(t % (uint32_t)S) * half + j;
    const float4 c = *(const float4*)(cs + pc), s_ = *(const float4*)(sn + pc);
    float xx, yy;
    rot_pair(a.x, b.x, c.x, s_.x, xx, yy); x[0] = (bf16)xx; y[0] = (bf16)yy;
    rot_pair(a.y, b.y, c.y, s_.y, xx, yy); x[1] = (bf16)xx; y[1] = (bf16)yy;
    rot_pair(a.z, b.z, c.z, s_.z, xx, yy); x[2] = (bf16)xx; y[2] = (bf16)yy;
    rot_pair(a.w, b.w, c.w, s_.w, xx, yy); x[3] = (bf16)xx; y[3] = (bf16)yy;
  } else {
    x[0] = (bf16)a.x; x[1] = (bf16)a.y; x[2] = (bf16)a.z; x[3] = (bf16)a.w;
    y[0] = (bf16)b.x; y[1] = (bf16)b.y; y[2] = (bf16)b.z; y[3] = (bf16)b.w;
  }
  *(bf16x4*)(o + j) = x;
  *(bf16x4*)(o + j + half) = y;
}

int launch_rope_qkv(const float* in, int64_t ldi, void* out, int64_t ldo, int T, int nq, int nkv, int d, int S,
                    const float* cos_t, const float* sin_t, hipStream_t s) {
  const int64_t total = (int64_t)T * (nq + 2 * nkv) * (d / 2);
  if (total <= 0) return 0;
  const int half = d / 2;
  if (half % 4 == 0 && ldi % 4 == 0 && ldo % 4 == 0 && (uintptr_t)in % 16 == 0 && (uintptr_t)out % 8 == 0 &&
      (uintptr_t)cos_t % 16 == 0 && (uintptr_t)sin_t % 16 == 0 && total / 4 < (int64_t(1) << 31)) {
    const uint32_t units = (uint32_t)(total / 4);
    hipLaunchKernelGGL(rope_qkv4_k, dim3((units + 255) / 256), dim3(256), 0, s, in, ldi, (bf16*)out, ldo, units,
                       (uint32_t)(half / 4), (uint32_t)(nq + 2 * nkv), nq + nkv, d, S, cos_t, sin_t);
    return (int)hipGetLastError();
  }
  hipLaunchKernelGGL(rope_qkv_k, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, in, ldi, (bf16*)out, ldo, T,
                     nq, nkv, d, S, cos_t, sin_t);
  return (int)hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// SwiGLU
// ------------------------------------------------------------------------------------------
// (sigm, swiglu_f and swiglu_b live in device_common.h: the gate/up GEMM epilogue shares them)

template <typename T>
__global__ void swiglu_fwd_k(const T* __restrict__ gu, T* __restrict__ a, int Tn, int F) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)Tn * F) return;
  const int64_t t = i / F;
  const int f = (int)(i % F);
  const float g = to_f(gu[t * 2 * F + f]), u = to_f(gu[t * 2 * F + F + f]);
  a[i] = from_f<T>(swiglu_f(g, u));
}

template <typename T>
__global__ void swiglu_bwd_k(const T* __restrict__ da, const T* __restrict__ gu, T* __restrict__ dgu, int Tn, int F) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)Tn * F) return;
  const int64_t t = i / F;
  const int f = (int)(i % F);
  const float g = to_f(gu[t * 2 * F + f]), u = to_f(gu[t * 2 * F + F + f]);
  float dg, du;
  swiglu_b(to_f(da[i]), g, u, dg, du);
  dgu[t * 2 * F + f] = from_f<T>(dg);
  dgu[t * 2 * F + F + f] = from_f<T>(du);
}

// Eight consecutive elements per thread (16-byte bf16 / 2 x 16-byte fp32 accesses). Each element
// goes through the same uncontracted expressions as in the one-element kernels above, so both give
// identical bits; these are taken when F % 8 == 0, the pointers are 16-byte aligned and T * F / 8 < 2^31.
__device__ __forceinline__ void ld8(const bf16* p, float* v) {
  const bf16x8 x = *(const bf16x8*)p;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (float)x[j];
}
__device__ __forceinline__ void ld8(const float* p, float* v) {
  const float4 x = *(const float4*)p, y = *(const float4*)(p + 4);
  v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w; v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
}
__device__ __forceinline__ void st8(bf16* p, const float* v) {
  bf16x8 x;
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = (bf16)v[j];
  *(bf16x8*)p = x;
}
__device__ __forceinline__ void st8(float* p, const float* v) {
  *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
  *(float4*)(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

template <typename T>
__global__ __launch_bounds__(256) void swiglu_fwd8_k(const T* __restrict__ gu, T* __restrict__ a, uint32_t units,
                                                     uint32_t nv) {
  const uint32_t u = blockIdx.x * 256u + threadIdx.x;
  if (u >= units) return;
  const uint32_t t = u / nv, c = u - t * nv;
  const T* gr = gu + (int64_t)t * 16 * nv + c * 8;
  float g[8], up[8], o[8];
  ld8(gr, g);
  ld8(gr + 8 * nv, up);
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = swiglu_f(g[j], up[j]);
  st8(a + (int64_t)u * 8, o);
}

template <typename T>
__global__ __launch_bounds__(256) void swiglu_bwd8_k(const T* __restrict__ da, const T* __restrict__ gu,
                                                     T* __restrict__ dgu, uint32_t units, uint32_t nv) {
  const uint32_t u = blockIdx.x * 256u + threadIdx.x;
  if (u >= units) return;
  const uint32_t t = u / nv, c = u - t * nv;
  const int64_t base = (int64_t)t * 16 * nv + c * 8;
  float g[8], up[8], d[8], dg[8], du[8];
  ld8(gu + base, g);
  ld8(gu + base + 8 * nv, up);
  ld8(da + (int64_t)u * 8, d);
#pragma unroll
  for (int j = 0; j < 8; ++j) swiglu_b(d[j], g[j], up[j], dg[j], du[j]);
  st8(dgu + base, dg);
  st8(dgu + base + 8 * nv, du);
}

static bool vec8_ok(int64_t units, std::initializer_list<const void*> ptrs) {
  if (units >= (int64_t(1) << 31)) return false;
  for (const void* p : ptrs)
    if ((uintptr_t)p & 15) return false;
  return true;
}

int launch_swiglu_fwd(const void* gu, void* a, DType t, int T, int F, hipStream_t s) {
  const int64_t n = (int64_t)T * F;
  if (n <= 0) return 0;
  if (F % 8 == 0 && vec8_ok(n / 8, {gu, a})) {
    const uint32_t units = (uint32_t)(n / 8), nv = (uint32_t)(F / 8);
    dim3 grid((units + 255) / 256);
    if (t == DT_BF16) hipLaunchKernelGGL(swiglu_fwd8_k<bf16>, grid, dim3(256), 0, s, (const bf16*)gu, (bf16*)a, units, nv);
    else hipLaunchKernelGGL(swiglu_fwd8_k<float>, grid, dim3(256), 0, s, (const float*)gu, (float*)a, units, nv);
    return (int)hipGetLastError();
  }
  dim3 grid((unsigned)((n + 255) / 256));
  if (t == DT_BF16) hipLaunchKernelGGL(swiglu_fwd_k<bf16>, grid, dim3(256), 0, s, (const bf16*)gu, (bf16*)a, T, F);
  else hipLaunchKernelGGL(swiglu_fwd_k<float>, grid, dim3(256), 0, s, (const float*)gu, (float*)a, T, F);
  return (int)hipGetLastError();
}

int launch_swiglu_bwd(const void* da, const void* gu, void* dgu, DType t, int T, int F, hipStream_t s) {
  const int64_t n = (int64_t)T * F;
  if (n <= 0) return 0;
  if (F % 8 == 0 && vec8_ok(n / 8, {da, gu, dgu})) {
    const uint32_t units = (uint32_t)(n / 8), nv = (uint32_t)(F / 8);
    dim3 grid((units + 255) / 256);
    if (t == DT_BF16)
      hipLaunchKernelGGL(swiglu_bwd8_k<bf16>, grid, dim3(256), 0, s, (const bf16*)da, (const bf16*)gu, (bf16*)dgu, units, nv);
    else
      hipLaunchKernelGGL(swiglu_bwd8_k<float>, grid, dim3(256), 0, s, (const float*)da, (const float*)gu, (float*)dgu, units, nv);
    return (int)hipGetLastError();
  }
  dim3 grid((unsigned)((n + 255) / 256));
  if (t == DT_BF16) hipLaunchKernelGGL(swiglu_bwd_k<bf16>, grid, dim3(256), 0, s, (const bf16*)da, (const bf16*)gu, (bf16*)dgu, T, F);
  else hipLaunchKernelGGL(swiglu_bwd_k<float>, grid, dim3(256), 0, s, (const float*)da, (const float*)gu, (float*)dgu, T, F);
  return (int)hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// bf16 transpose out[c][r] = in[r][c] through a 128 x 128 LDS tile: coalesced 16-byte loads of
// input rows, 8 x 8 register transposes of LDS blocks, coalesced 16-byte stores of output rows.
// LDS chunk c of tile row r is stored at chunk c ^ ((r / 8) % 16).
// ------------------------------------------------------------------------------------------
typedef uint32_t tu32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void tr8x8(const tu32x4 in[8], tu32x4 out[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int w = c >> 1;
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int p = 0; p < 4; ++p) out[c][p] = __builtin_amdgcn_perm(in[2 * p + 1][w], in[2 * p][w], sel);
  }
}

__device__ __forceinline__ tu32x4 load8_bf16_tail(const uint16_t* row, int gc, int C) {
  uint16_t e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) e[j] = gc + j < C ? row[gc + j] : (uint16_t)0;
  return tu32x4{e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16), e[4] | ((uint32_t)e[5] << 16),
                e[6] | ((uint32_t)e[7] << 16)};
}

// Interior tiles take a branch-free path whose eight 16-byte loads are all in flight before the
// first LDS write; edge tiles take a guarded path.
__global__ __launch_bounds__(256) void transpose_bf16_k(const uint16_t* __restrict__ in, int64_t ldi,
                                                        uint16_t* __restrict__ out, int64_t ldo, int R, int C) {
  __shared__ tu32x4 tile[128 * 16];
  const int r0 = blockIdx.y * 128, c0 = blockIdx.x * 128;
  const int t = threadIdx.x;
  const bool full = r0 + 128 <= R && c0 + 128 <= C;
  // phase 1: rows r0 + t/16 + 16 k, chunk t % 16
  const int ch = t % 16;
  tu32x4 v[8];
  if (full) {
    const uint16_t* src = in + (int64_t)(r0 + t / 16) * ldi + c0 + ch * 8;
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = *(const tu32x4*)(src + (int64_t)(16 * k) * ldi);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int gr = r0 + t / 16 + 16 * k, gc = c0 + ch * 8;
      v[k] = tu32x4{0u, 0u, 0u, 0u};
      if (gr < R) {
        const uint16_t* row = in + (int64_t)gr * ldi;
        v[k] = gc + 8 <= C ? *(const tu32x4*)(row + gc) : load8_bf16_tail(row, gc, C);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int r = t / 16 + 16 * k;
    tile[r * 16 + (ch ^ ((r >> 3) & 15))] = v[k];
  }
  __syncthreads();
  // phase 2: thread owns the 8x8 block (row block rb = t % 16, column chunk cb = t / 16)
  const int rb = t % 16, cb = t / 16;
  tu32x4 in8[8], o8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = rb * 8 + i;
    in8[i] = tile[r * 16 + (cb ^ ((r >> 3) & 15))];
  }
  tr8x8(in8, o8);
  const int orr = r0 + rb * 8;      // output column
  if (full) {
    uint16_t* dst = out + (int64_t)(c0 + cb * 8) * ldo + orr;
#pragma unroll
    for (int j = 0; j < 8; ++j) *(tu32x4*)(dst + (int64_t)j * ldo) = o8[j];
    return;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int oc = c0 + cb * 8 + j;   // output row
    if (oc >= C) continue;
    if (orr + 8 <= R) {
      *(tu32x4*)(out + (int64_t)oc * ldo + orr) = o8[j];
    } else {
      const uint16_t* e = (const uint16_t*)&o8[j];
      for (int q = 0; q < 8 && orr + q < R; ++q) out[(int64_t)oc * ldo + orr + q] = e[q];
    }
  }
}

int launch_transpose_bf16(const void* in, int64_t ldi, void* out, int64_t ldo, int R, int C, hipStream_t s) {
  if (R <= 0 || C <= 0) return 0;
  if (ldi % 8 || ldo % 8 || ((uintptr_t)in | (uintptr_t)out) % 16) return (int)hipErrorInvalidValue;
  dim3 grid((C + 127) / 128, (R + 127) / 128);
  hipLaunchKernelGGL(transpose_bf16_k, grid, dim3(256), 0, s, (const uint16_t*)in, ldi, (uint16_t*)out, ldo, R, C);
  return (int)hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// SwiGLU backward that also writes its result transposed (bf16): dgu [T][2F] as launch_swiglu_bwd
// writes it (bit for bit), and dguT [2F][T] for the weight-gradient product, so the gradient is
// not read back for a separate transpose. A block takes 128 tokens x 64 features: phase 1 reads
// da, gate and up for its rows (a thread: 8 features of 4 rows), computes the gate and up
// gradients, stores the dgu rows and parks both 128 x 64 halves in one 128 x 128 LDS tile (gate
// gradients in columns 0..63, up gradients in 64..127); phase 2 is the transpose kernel's
// 8 x 8-block pass, writing output rows f0 + c (gate) and F + f0 + c - 64 (up).
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void swiglu_bwd_tr_k(const bf16* __restrict__ da, const bf16* __restrict__ gu,
                                                       bf16* __restrict__ dgu, bf16* __restrict__ dgut, int64_t ldt,
                                                       int T, int F) {
  __shared__ tu32x4 tile[128 * 16];
  const int t0 = blockIdx.y * 128, f0 = blockIdx.x * 64;
  const int t = threadIdx.x;
  const int cf = t & 7;  // features f0 + 8 cf .. + 7
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = (t >> 3) + 32 * k, row = t0 + r;
    float dg[8], du[8];
    if (row < T) {
      const bf16* gr = gu + (int64_t)row * 2 * F + f0 + 8 * cf;
      float g[8], up[8], d[8];
      ld8(gr, g);
      ld8(gr + F, up);
      ld8(da + (int64_t)row * F + f0 + 8 * cf, d);
#pragma unroll
      for (int j = 0; j < 8; ++j) swiglu_b(d[j], g[j], up[j], dg[j], du[j]);
      bf16* dr = dgu + (int64_t)row * 2 * F + f0 + 8 * cf;
      st8(dr, dg);
      st8(dr + F, du);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) dg[j] = du[j] = 0.f;
    }
    bf16x8 xg, xu;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      xg[j] = (bf16)dg[j];
      xu[j] = (bf16)du[j];
    }
    tile[r * 16 + (cf ^ ((r >> 3) & 15))] = __builtin_bit_cast(tu32x4, xg);
    tile[r * 16 + ((8 + cf) ^ ((r >> 3) & 15))] = __builtin_bit_cast(tu32x4, xu);
  }
  __syncthreads();
  // phase 2: thread owns the 8x8 block of token rows rb * 8.., tile columns cb * 8..
  const int rb = t % 16, cb = t / 16;
  tu32x4 in8[8], o8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = rb * 8 + i;
    in8[i] = tile[r * 16 + (cb ^ ((r >> 3) & 15))];
  }
  tr8x8(in8, o8);
  const int tok = t0 + rb * 8;                                   // first output column
  const int64_t orow = cb < 8 ? f0 + cb * 8 : (int64_t)F + f0 + (cb - 8) * 8;  // first output row
  uint16_t* dst = (uint16_t*)dgut + orow * ldt + tok;
  if (tok + 8 <= T) {
#pragma unroll
    for (int j = 0; j < 8; ++j) *(tu32x4*)(dst + (int64_t)j * ldt) = o8[j];
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint16_t* e = (const uint16_t*)&o8[j];
      for (int q = 0; q < 8 && tok + q < T; ++q) dst[(int64_t)j * ldt + q] = e[q];
    }
  }
}

int launch_swiglu_bwd_tr(const void* da, const void* gu, void* dgu, void* dgut, int64_t ldt, int T, int F,
                         hipStream_t s) {
  if (T <= 0 || F <= 0) return 0;
  if (F % 64 || T % 8 || ldt % 8 || ldt < T ||
      (((uintptr_t)da | (uintptr_t)gu | (uintptr_t)dgu | (uintptr_t)dgut) % 16))
    return (int)hipErrorInvalidValue;
  dim3 grid(F / 64, (T + 127) / 128);
  hipLaunchKernelGGL(swiglu_bwd_tr_k, grid, dim3(256), 0, s, (const bf16*)da, (const bf16*)gu, (bf16*)dgu,
                     (bf16*)dgut, ldt, T, F);
  return (int)hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Embedding-row gradient: out[u] = sum of dh[order[i]] over i in [seg[u], seg[u+1]), added in
// order of i from zero (the occurrences of one token in position order). One block per row.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void embed_row_sums_k(const float* __restrict__ dh, const int32_t* __restrict__ order,
                                                        const int32_t* __restrict__ seg, int H, float* __restrict__ out) {
  const int u = blockIdx.x;
  const int i0 = seg[u], i1 = seg[u + 1];
  for (int c = threadIdx.x * 4; c < H; c += 1024) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i = i0; i < i1; ++i) {
      const float4 x = *(const float4*)(dh + (int64_t)order[i] * H + c);
      acc.x += x.x;
      acc.y += x.y;
      acc.z += x.z;
      acc.w += x.w;
    }
    *(float4*)(out + (int64_t)u * H + c) = acc;
  }
}

int launch_embed_row_sums(const float* dh, const int32_t* order, const int32_t* seg, int nrows, int H, float* out,
                          hipStream_t s) {
  if (nrows <= 0) return 0;
  if (H % 4) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(embed_row_sums_k, dim3(nrows), dim3(256), 0, s, dh, order, seg, H, out);
  return (int)hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// casts and fills
// ------------------------------------------------------------------------------------------
template <typename T>
__global__ void cast_k(const float* __restrict__ x, T* __restrict__ y, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = from_f<T>(x[i]);
}
template <typename T>
__global__ __launch_bounds__(256) void cast8_k(const float* __restrict__ x, T* __restrict__ y, uint32_t units) {
  const uint32_t u = blockIdx.x * 256u + threadIdx.x;
  if (u >= units) return;
  float v[8];
  ld8(x + (int64_t)u * 8, v);
  st8(y + (int64_t)u * 8, v);
}
__global__ void fill_k(float* x, float v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) x[i] = v;
}
__global__ void scale_k(const float* x, float a, float* y, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = a * x[i];
}

int launch_cast_f32(const float* x, void* y, DType yt, int64_t n, hipStream_t s) {
  if (n <= 0) return 0;
  if (n % 8 == 0 && vec8_ok(n / 8, {x, y})) {
    const uint32_t units = (uint32_t)(n / 8);
    dim3 grid((units + 255) / 256);
    if (yt == DT_BF16) hipLaunchKernelGGL(cast8_k<bf16>, grid, dim3(256), 0, s, x, (bf16*)y, units);
    else hipLaunchKernelGGL(cast8_k<float>, grid, dim3(256), 0, s, x, (float*)y, units);
    return (int)hipGetLastError();
  }
  dim3 grid((unsigned)((n + 255) / 256));
  if (yt == DT_BF16) hipLaunchKernelGGL(cast_k<bf16>, grid, dim3(256), 0, s, x, (bf16*)y, n);
  else hipLaunchKernelGGL(cast_k<float>, grid, dim3(256), 0, s, x, (float*)y, n);
  return (int)hipGetLastError();
}
int launch_fill_f32(float* x, float v, int64_t n, hipStream_t s) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(fill_k, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, v, n);
  return (int)hipGetLastError();
}
int launch_scale_f32(const float* x, float a, float* y, int64_t n, hipStream_t s) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(scale_k, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, a, y, n);
  return (int)hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// cross entropy over rows of fp32 logits (loss anchor). One 256-thread block per row:
// online (max, sum-exp) in one pass, then the weighted softmax-minus-onehot gradient.
// ------------------------------------------------------------------------------------------
template <typename TD>
__global__ __launch_bounds__(256) void ce_k(const float* __restrict__ z, int64_t ld, const int32_t* __restrict__ lab,
                                            const float* __restrict__ wt, float* __restrict__ row_loss,
                                            TD* __restrict__ dz, int64_t ldd, int V) {
  __shared__ float red[16];
  const int row = blockIdx.x;
  const float* zr = z + (int64_t)row * ld;
  float m = -INFINITY, s = 0.f;
  for (int j = threadIdx.x; j < V; j += 256) {
    const float v = zr[j];
    if (v > m) { s = s * __expf(m - v) + 1.f; m = v; }
    else s += __expf(v - m);
  }
  // combine (m, s) across the block
  const float M = block_max(m, red);
  s = (m == -INFINITY) ? 0.f : s * __expf(m - M);
  const float S = block_sum(s, red);
  const float lse = M + __logf(S);
  const int y = lab[row];
  const float w = wt[row];
  if (threadIdx.x == 0) row_loss[row] = (y >= 0) ? w * (lse - zr[y]) : 0.f;
  TD* dr = dz + (int64_t)row * ldd;
  for (int j = threadIdx.x; j < V; j += 256) {
    float p = __expf(zr[j] - lse);
    if (j == y) p -= 1.f;
    dr[j] = from_f<TD>(y >= 0 ? w * p : 0.f);
  }
}

// The same with 8 logits per thread and step (two 16-byte loads; one 16-byte store of bf16 or two
// of fp32): V, ld and ldd multiples of 8 and 16-byte aligned rows. The running maximum moves at
// most once per 8 values, and the exponentials are taken against the maximum of the 8.
template <typename TD>
__global__ __launch_bounds__(256) void ce8_k(const float* __restrict__ z, int64_t ld, const int32_t* __restrict__ lab,
                                             const float* __restrict__ wt, float* __restrict__ row_loss,
                                             TD* __restrict__ dz, int64_t ldd, int V) {
  __shared__ float red[16];
  const int row = blockIdx.x;
  const float* zr = z + (int64_t)row * ld;
  const int n8 = V >> 3;
  float m = -INFINITY, s = 0.f;
  for (int j = threadIdx.x; j < n8; j += 256) {
    float v[8];
    ld8(zr + 8 * (int64_t)j, v);
    float mx = v[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, v[e]);
    if (mx > m) {
      s *= __expf(m - mx);
      m = mx;
    }
    float t = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) t += __expf(v[e] - m);
    s += t;
  }
  const float M = block_max(m, red);
  s = (m == -INFINITY) ? 0.f : s * __expf(m - M);
  const float S = block_sum(s, red);
  const float lse = M + __logf(S);
  const int y = lab[row];
  const float w = wt[row];
  if (threadIdx.x == 0) row_loss[row] = (y >= 0) ? w * (lse - zr[y]) : 0.f;
  TD* dr = dz + (int64_t)row * ldd;
  const float wy = y >= 0 ? w : 0.f;
  for (int j = threadIdx.x; j < n8; j += 256) {
    float v[8];
    ld8(zr + 8 * (int64_t)j, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float p = __expf(v[e] - lse);
      if (8 * j + e == y) p -= 1.f;
      v[e] = wy * p;
    }
    st8(dr + 8 * (int64_t)j, v);
  }
}

int launch_ce_fwd_bwd(const float* logits, int64_t ld, const int32_t* labels, const float* w, float* row_loss,
                      void* dlogits, DType dt, int64_t ldd, int Tc, int V, hipStream_t s) {
  if (Tc <= 0) return 0;
  const bool v8 = V % 8 == 0 && ld % 8 == 0 && ldd % 8 == 0 && (uintptr_t)logits % 16 == 0 && (uintptr_t)dlogits % 16 == 0;
  if (v8 && dt == DT_BF16) hipLaunchKernelGGL(ce8_k<bf16>, dim3(Tc), dim3(256), 0, s, logits, ld, labels, w, row_loss, (bf16*)dlogits, ldd, V);
  else if (v8) hipLaunchKernelGGL(ce8_k<float>, dim3(Tc), dim3(256), 0, s, logits, ld, labels, w, row_loss, (float*)dlogits, ldd, V);
  else if (dt == DT_BF16) hipLaunchKernelGGL(ce_k<bf16>, dim3(Tc), dim3(256), 0, s, logits, ld, labels, w, row_loss, (bf16*)dlogits, ldd, V);
  else hipLaunchKernelGGL(ce_k<float>, dim3(Tc), dim3(256), 0, s, logits, ld, labels, w, row_loss, (float*)dlogits, ldd, V);
  return (int)hipGetLastError();
}

__global__ __launch_bounds__(256) void sumsq_k(const float* __restrict__ h, float* __restrict__ row_loss,
                                               float* __restrict__ dh, int T, int H) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= T) return;
  const float* hr = h + (int64_t)row * H;
  float* dr = dh + (int64_t)row * H;
  float ss = 0.f;
  for (int j = lane; j < H; j += 64) {
    const float v = hr[j];
    ss += v * v;
    dr[j] = 2.f * v;
  }
  ss = wave_sum(ss);
  if (lane == 0) row_loss[row] = ss;
}

int launch_sumsq(const float* h, float* row_loss, float* dh, int T, int H, hipStream_t s) {
  if (T <= 0) return 0;
  hipLaunchKernelGGL(sumsq_k, dim3((T + 3) / 4), dim3(256), 0, s, h, row_loss, dh, T, H);
  return (int)hipGetLastError();
}

}  // namespace hol
