// Host-side numerics of the streamed trainer: a small thread pool, the fp32 Adam step, the bf16
// refresh of the low-precision copy and the stage partitioner.
#pragma once
#include <stdint.h>

#include <functional>

namespace hol {

// Runs fn(begin, end) over [0, n) split into roughly equal chunks on the pool's threads.
void parallel_for(int64_t n, int64_t min_chunk, const std::function<void(int64_t, int64_t)>& fn);
int pool_threads();

struct AdamConsts {
  float b1, b2, omb1, omb2, bc1, bc2, lr, eps;
};
AdamConsts adam_consts(int64_t t, float lr, float b1, float b2, float eps);
// In place on [0, n): fixed op order, no fused multiply-add (compiled with -ffp-contract=off).
void adam_range(float* theta, const float* g, float* m, float* v, int64_t n, const AdamConsts& c);

uint16_t f32_to_bf16(float x);
void f32_to_bf16_range(const float* src, uint16_t* dst, int64_t n);
// the same values; non-temporal stores (the caller issues a store fence before others read dst)
void f32_to_bf16_range_stream(const float* src, uint16_t* dst, int64_t n);

// Stage partition; returns false when some layer alone exceeds the memory cap.
bool partition_stages(const int64_t* t_f, const int64_t* t_b, const int64_t* m_f, const int64_t* m_b,
                      int L, int64_t cap, int n_gpus, int n_micro, int* f_bounds, int* n_f,
                      int* b_bounds, int* n_b, int64_t* t_max, __int128* J);

}  // namespace hol
