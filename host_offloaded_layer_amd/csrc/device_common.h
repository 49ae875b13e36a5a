// Device-side helpers shared by the HIP kernels of the layer template (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }

// 64-lane wavefront reductions (DPP/permute via __shfl_xor)
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Block-wide sum for blockDim.x a multiple of 64 (<= 1024). `red` must hold 16 floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, nw = blockDim.x >> 6;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, nw = blockDim.x >> 6;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float t = -INFINITY;
  for (int i = 0; i < nw; ++i) t = fmaxf(t, red[i]);
  return t;
}

// SwiGLU element operations. Contraction is off so that every kernel that calls them (the
// element-wise kernels and the fused gate/up GEMM epilogue) rounds the same way. The logistic
// function takes the hardware reciprocal (v_rcp_f32, 1 ulp) rather than a correctly rounded
// division: a third of the instructions, which matters in the GEMM epilogue, and an error far
// below the bf16 rounding of every value it feeds (1 / inf = 0 and 1 / 1 = 1 at the extremes).
__device__ __forceinline__ float sigm(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }
__device__ __forceinline__ float swiglu_f(float g, float u) {
#pragma clang fp contract(off)
  return g * sigm(g) * u;
}
__device__ __forceinline__ void swiglu_b(float d, float g, float u, float& dg, float& du) {
#pragma clang fp contract(off)
  const float sg = sigm(g);
  dg = d * u * sg * (1.f + g * (1.f - sg));
  du = d * g * sg;
}

// One RoPE-rotated pair (x, y) = (a c - b s, b c + a s). Contraction off so that every kernel that
// calls it (the element-wise RoPE kernels and the q/k/v GEMM epilogue) rounds the same way.
__device__ __forceinline__ void rot_pair(float a, float b, float c, float s, float& x, float& y) {
#pragma clang fp contract(off)
  x = a * c - b * s;
  y = b * c + a * s;
}
