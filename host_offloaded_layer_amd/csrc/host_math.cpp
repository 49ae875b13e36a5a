// Host-side numerics: thread pool, fp32 Adam (MegaTrain summary page, 方法步骤详情 phase 4:
// the optimiser update runs on the CPU), bf16 refresh of the low-precision copy (RoundPipe
// popular article §五: compute copy / low-precision host copy / high-precision optimiser copy)
// and the stage partitioner (RoundPipe popular article §六, paper summary 方法步骤详情 step 2).
//
// Built with -ffp-contract=off: the Adam arithmetic must not be fused so its results are
// reproducible bit for bit.
#include "host_math.h"

#include <immintrin.h>

#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <condition_variable>
#include <mutex>
#include <thread>
#include <vector>

namespace hol {

// ------------------------------------------------------------------------------------------
// thread pool
// ------------------------------------------------------------------------------------------
namespace {
class Pool {
 public:
  Pool() {
    int n = (int)std::thread::hardware_concurrency();
    const char* e = getenv("HOL_HOST_THREADS");
    if (!e) e = getenv("OMP_NUM_THREADS");
    if (e && atoi(e) > 0) n = atoi(e);
    n = std::max(1, std::min(n, 64));
    nthreads_ = n;
    for (int i = 1; i < n; ++i) workers_.emplace_back([this, i] { loop(i); });
  }
  ~Pool() {
    {
      std::lock_guard<std::mutex> g(mu_);
      stop_ = true;
      ++gen_;
    }
    cv_.notify_all();
    for (auto& t : workers_) t.join();
  }
  int size() const { return nthreads_; }

  // Dynamic schedule: about 8 chunks per thread (none below min_chunk) handed out through an
  // atomic counter, so a thread that loses its core for a while (other busy threads in the
  // process) only takes fewer chunks instead of holding every other thread up.
  void run(int64_t n, int64_t min_chunk, const std::function<void(int64_t, int64_t)>& fn) {
    if (n <= 0) return;
    const int64_t chunk = std::max<int64_t>(std::max<int64_t>(1, min_chunk), n / ((int64_t)nthreads_ * 8));
    const int64_t nchunks = (n + chunk - 1) / chunk;
    if (nchunks <= 1 || nthreads_ <= 1) {
      fn(0, n);
      return;
    }
    std::lock_guard<std::mutex> serial(run_mu_);
    {
      std::lock_guard<std::mutex> g(mu_);
      fn_ = &fn;
      n_ = n;
      chunk_ = chunk;
      nchunks_ = nchunks;
      next_.store(0, std::memory_order_relaxed);
      helpers_ = (int)std::min<int64_t>(nthreads_ - 1, nchunks - 1);
      pending_ = helpers_;
      ++gen_;
    }
    cv_.notify_all();
    work();
    std::unique_lock<std::mutex> lk(mu_);
    done_cv_.wait(lk, [this] { return pending_ == 0; });
    fn_ = nullptr;
  }

 private:
  void work() {
    for (;;) {
      const int64_t c = next_.fetch_add(1, std::memory_order_relaxed);
      if (c >= nchunks_) return;
      const int64_t lo = c * chunk_, hi = std::min(n_, lo + chunk_);
      (*fn_)(lo, hi);
    }
  }
  void loop(int id) {
    uint64_t seen = 0;
    for (;;) {
      std::unique_lock<std::mutex> lk(mu_);
      cv_.wait(lk, [&] { return gen_ != seen; });
      seen = gen_;
      if (stop_) return;
      if (id > helpers_ || fn_ == nullptr) continue;
      lk.unlock();
      work();
      lk.lock();
      if (--pending_ == 0) done_cv_.notify_one();
    }
  }
  int nthreads_ = 1;
  std::vector<std::thread> workers_;
  std::mutex mu_, run_mu_;
  std::condition_variable cv_, done_cv_;
  const std::function<void(int64_t, int64_t)>* fn_ = nullptr;
  int64_t n_ = 0, chunk_ = 1, nchunks_ = 0;
  std::atomic<int64_t> next_{0};
  int helpers_ = 0, pending_ = 0;
  uint64_t gen_ = 0;
  bool stop_ = false;
};

// Never destroyed: worker threads stay parked until the process exits.
Pool& pool() {
  static Pool* p = new Pool();
  return *p;
}
}  // namespace

void parallel_for(int64_t n, int64_t min_chunk, const std::function<void(int64_t, int64_t)>& fn) {
  pool().run(n, min_chunk, fn);
}
int pool_threads() { return pool().size(); }

// ------------------------------------------------------------------------------------------
// Adam
// ------------------------------------------------------------------------------------------
AdamConsts adam_consts(int64_t t, float lr, float b1, float b2, float eps) {
  AdamConsts c;
  c.b1 = b1;
  c.b2 = b2;
  c.omb1 = (float)(1.0 - (double)b1);
  c.omb2 = (float)(1.0 - (double)b2);
  c.bc1 = (float)(1.0 - pow((double)b1, (double)t));
  c.bc2 = (float)(1.0 - pow((double)b2, (double)t));
  c.lr = lr;
  c.eps = eps;
  return c;
}

static inline __attribute__((always_inline)) void adam_body(float* __restrict theta, const float* __restrict g,
                                                            float* __restrict m, float* __restrict v, int64_t n,
                                                            const AdamConsts& c) {
  const float b1 = c.b1, b2 = c.b2, omb1 = c.omb1, omb2 = c.omb2, bc1 = c.bc1, bc2 = c.bc2,
              lr = c.lr, eps = c.eps;
  for (int64_t i = 0; i < n; ++i) {
    const float gi = g[i];
    const float mi = b1 * m[i] + omb1 * gi;
    const float vi = b2 * v[i] + omb2 * (gi * gi);
    m[i] = mi;
    v[i] = vi;
    const float mhat = mi / bc1;
    const float vhat = vi / bc2;
    theta[i] = theta[i] - (lr * mhat) / (sqrtf(vhat) + eps);
  }
}

// The same loop vectorised 16 wide where the host has AVX-512 (the element operations are the
// same IEEE operations in the same order, so the results are identical bit for bit; about 5-8 %
// faster per layer on the Zen 5 hosts here, where the update is mostly bound by memory).
__attribute__((target("avx512f,avx512dq,avx512bw,avx512vl"))) static void adam_range_avx512(
    float* __restrict theta, const float* __restrict g, float* __restrict m, float* __restrict v, int64_t n,
    const AdamConsts& c) {
  adam_body(theta, g, m, v, n, c);
}

void adam_range(float* __restrict theta, const float* __restrict g, float* __restrict m,
                float* __restrict v, int64_t n, const AdamConsts& c) {
  static const bool avx512 = __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512dq") &&
                             __builtin_cpu_supports("avx512bw") && __builtin_cpu_supports("avx512vl");
  if (avx512) adam_range_avx512(theta, g, m, v, n, c);
  else adam_body(theta, g, m, v, n, c);
}

uint16_t f32_to_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// The same rounding, 16 values a step, stored with non-temporal stores when the destination is
// 32-byte aligned (the low-precision image is read next by the device copy, not by this core).
void f32_to_bf16_range_stream(const float* __restrict src, uint16_t* __restrict dst, int64_t n) {
  int64_t i = 0;
  if (((uintptr_t)dst & 31) == 0) {
    const __m256i lsb1 = _mm256_set1_epi32(1), bias = _mm256_set1_epi32(0x7fff), absm = _mm256_set1_epi32(0x7fffffff),
                  inf = _mm256_set1_epi32(0x7f800000), q = _mm256_set1_epi32(0x40);
    for (; i + 16 <= n; i += 16) {
      __m256i h[2];
      for (int k = 0; k < 2; ++k) {
        const __m256i u = _mm256_loadu_si256((const __m256i*)(src + i + 8 * k));
        const __m256i r = _mm256_srli_epi32(
            _mm256_add_epi32(_mm256_add_epi32(u, bias), _mm256_and_si256(_mm256_srli_epi32(u, 16), lsb1)), 16);
        const __m256i nan = _mm256_cmpgt_epi32(_mm256_and_si256(u, absm), inf);
        const __m256i qn = _mm256_or_si256(_mm256_srli_epi32(u, 16), q);
        h[k] = _mm256_blendv_epi8(r, qn, nan);
      }
      // pack the two 8 x 32-bit halves to 16 x 16-bit in order (packus works per 128-bit lane)
      const __m256i p = _mm256_permute4x64_epi64(_mm256_packus_epi32(h[0], h[1]), 0xD8);
      _mm256_stream_si256((__m256i*)(dst + i), p);
    }
  }
  f32_to_bf16_range(src + i, dst + i, n - i);
}

void f32_to_bf16_range(const float* __restrict src, uint16_t* __restrict dst, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u;
    memcpy(&u, src + i, 4);
    const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    dst[i] = ((u & 0x7fffffffu) > 0x7f800000u) ? (uint16_t)((u >> 16) | 0x40) : (uint16_t)r;
  }
}

// ------------------------------------------------------------------------------------------
// stage partition
// ------------------------------------------------------------------------------------------
namespace {
// Greedy pass over costs given in pass order; returns the stage count (0 if infeasible) and
// writes stage start offsets (in pass order) to `starts`.
int greedy(const int64_t* t, const int64_t* m, int L, int64_t tmax, int64_t cap, int* starts) {
  int S = 0;
  int64_t st = 0, sm = 0;
  for (int i = 0; i < L; ++i) {
    if (t[i] > tmax || m[i] > cap) return 0;
    if (i == 0 || st + t[i] > tmax || sm + m[i] > cap) {
      if (starts) starts[S] = i;
      ++S;
      st = 0;
      sm = 0;
    }
    st += t[i];
    sm += m[i];
  }
  return S;
}
}  // namespace

bool partition_stages(const int64_t* t_f, const int64_t* t_b, const int64_t* m_f, const int64_t* m_b, int L,
                      int64_t cap, int n_gpus, int n_micro, int* f_bounds, int* n_f, int* b_bounds, int* n_b,
                      int64_t* t_max, __int128* J_out) {
  for (int i = 0; i < L; ++i)
    if (m_f[i] > cap || m_b[i] > cap) return false;
  std::vector<int64_t> tb(t_b, t_b + L), mb(m_b, m_b + L);
  std::reverse(tb.begin(), tb.end());
  std::reverse(mb.begin(), mb.end());
  // candidate thresholds: every contiguous sum of either pass's costs
  std::vector<int64_t> cand;
  cand.reserve((size_t)L * (L + 1));
  for (int i = 0; i < L; ++i) {
    int64_t sf = 0, sb = 0;
    for (int j = i; j < L; ++j) {
      sf += t_f[j];
      sb += t_b[j];
      cand.push_back(sf);
      cand.push_back(sb);
    }
  }
  std::sort(cand.begin(), cand.end());
  cand.erase(std::unique(cand.begin(), cand.end()), cand.end());
  const __int128 warm = (__int128)n_gpus * (n_gpus - 1);
  bool found = false;
  __int128 bestJ = 0;
  int64_t bestT = 0;
  for (int64_t t : cand) {  // ascending: the first minimum is the one with the smallest t
    const int sf = greedy(t_f, m_f, L, t, cap, nullptr);
    if (!sf) continue;
    const int sb = greedy(tb.data(), mb.data(), L, t, cap, nullptr);
    if (!sb) continue;
    const __int128 J = ((__int128)n_micro * (sf + sb) + warm) * (__int128)t;
    if (!found || J < bestJ) {
      found = true;
      bestJ = J;
      bestT = t;
    }
  }
  if (!found) return false;
  std::vector<int> st(L);
  *n_f = greedy(t_f, m_f, L, bestT, cap, f_bounds);
  *n_b = greedy(tb.data(), mb.data(), L, bestT, cap, st.data());
  for (int s = 0; s < *n_b; ++s) b_bounds[s] = L - 1 - st[s];
  *t_max = bestT;
  if (J_out) *J_out = bestJ;
  return true;
}

}  // namespace hol
