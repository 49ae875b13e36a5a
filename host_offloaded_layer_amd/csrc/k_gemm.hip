// GEMMs of the decoder-layer template: the q/k/v, output, gate/up and down projections, the LM
// head, and their backward products (dX = dY W, dW += dY^T X). MegaTrain summary page, 核心方法:
// each template encapsulates the kernels of the Attention and MLP blocks and holds no weights;
// the weight operand is whichever streamed slot the engine binds.
//
// Two kernels:
//  * gemm_mfma  - bf16 operands, fp32 accumulation on CDNA4 matrix cores
//                 (v_mfma_f32_32x32x16_bf16). 256x128x64 block tile, 4 waves of 128x64,
//                 LDS double buffer with padded K-contiguous rows. Operands stored MN-contiguous
//                 (the backward layouts) are transposed 8x8 in registers on their way into LDS,
//                 so every MFMA fragment is one 16-byte LDS read.
//  * gemm_tiled - plain LDS-tiled FMA kernel for fp32 operands (the fp32 path).
#include "device_common.h"
#include "kernels.h"

namespace hol {

// ------------------------------------------------------------------------------------------
// generic fp32 / mixed tiled GEMM
// ------------------------------------------------------------------------------------------
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void gemm_tiled(Gemm g) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  const int z = blockIdx.z;
  const TI* A = (const TI*)g.A + z * g.sA;
  const TI* B = (const TI*)g.B + z * g.sB;
  const int M = g.M, N = g.N, K = g.K;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int e = t; e < 1024; e += 256) {
      int mm, kk;
      if (g.a_km) { kk = e >> 6; mm = e & 63; } else { mm = e >> 4; kk = e & 15; }
      const int m = m0 + mm, k = k0 + kk;
      float v = 0.f;
      if (m < M && k < K) v = to_f(A[g.a_km ? (int64_t)k * g.lda + m : (int64_t)m * g.lda + k]);
      As[kk][mm] = v;
    }
    for (int e = t; e < 1024; e += 256) {
      int nn, kk;
      if (g.b_kn) { kk = e >> 6; nn = e & 63; } else { nn = e >> 4; kk = e & 15; }
      const int n = n0 + nn, k = k0 + kk;
      float v = 0.f;
      if (n < N && k < K) v = to_f(B[g.b_kn ? (int64_t)k * g.ldb + n : (int64_t)n * g.ldb + k]);
      Bs[kk][nn] = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  TO* C = (TO*)g.C + z * g.sC;
  const float* R = g.R ? g.R + z * g.sR : nullptr;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      float v = g.alpha * acc[i][j];
      TO* c = C + (int64_t)m * g.ldc + n;
      if (g.epi == EPI_ACCUM) v += to_f(*c);
      else if (g.epi == EPI_RESID) v += R[(int64_t)m * g.ldr + n];
      *c = from_f<TO>(v);
    }
  }
}

// ------------------------------------------------------------------------------------------
// bf16 MFMA GEMM
// ------------------------------------------------------------------------------------------
constexpr int MF_BM = 256, MF_BN = 128, MF_BK = 64;
constexpr int MF_P = MF_BK + 8;                 // LDS row pitch (bf16): 144 B, conflict-free b128 reads
constexpr int MF_STAGE = (MF_BM + MF_BN) * MF_P; // bf16 elements per LDS stage

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 8x8 transpose of 16-bit values: in[r] holds row r (8 values as 4 dwords); out[c] holds column c.
__device__ __forceinline__ void transpose8x8(const u32x4 in[8], u32x4 out[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int w = c >> 1;
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;  // high or low halves
#pragma unroll
    for (int p = 0; p < 4; ++p)
      out[c][p] = __builtin_amdgcn_perm(in[2 * p + 1][w], in[2 * p][w], sel);
  }
}

// Loads of one operand tile (`ROWS` MN-rows x 64 k) into registers.
// K-contiguous source: thread owns chunk (t & 7) of rows (t >> 3) + 32 i.
// MN-contiguous source: thread owns 8x8 block(s) and transposes them.
template <int ROWS, bool KM>
struct TileLoader {
  static constexpr int NREG = KM ? ((ROWS / 8) * (MF_BK / 8) + 255) / 256 * 8 : ROWS * 8 / 256;
  u32x4 r[NREG];

  __device__ __forceinline__ void load(const bf16* __restrict__ P, int64_t ld, int mn0, int MN, int k0,
                                       int K) {
    const int t = threadIdx.x;
    if constexpr (!KM) {
      const int c = t & 7;
      const int k = k0 + c * 8;
#pragma unroll
      for (int i = 0; i < NREG; ++i) {
        int row = mn0 + (t >> 3) + 32 * i;
        row = row < MN ? row : MN - 1;
        if (k < K) r[i] = *(const u32x4*)(P + (int64_t)row * ld + k);
        else r[i] = u32x4{0u, 0u, 0u, 0u};
      }
    } else {
      constexpr int NB = (ROWS / 8) * (MF_BK / 8);
#pragma unroll
      for (int bi = 0; bi < NREG / 8; ++bi) {
        const int b = t + 256 * bi;
        u32x4 in[8];
        if (b < NB) {
          const int mb = b % (ROWS / 8), kb = b / (ROWS / 8);
          const int m = mn0 + mb * 8;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int k = k0 + kb * 8 + i;
            if (k < K && m + 8 <= MN) {
              in[i] = *(const u32x4*)(P + (int64_t)k * ld + m);
            } else {
              uint16_t e[8];
#pragma unroll
              for (int j = 0; j < 8; ++j)
                e[j] = (k < K && m + j < MN) ? ((const uint16_t*)P)[(int64_t)k * ld + m + j] : (uint16_t)0;
              in[i] = u32x4{e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16),
                            e[4] | ((uint32_t)e[5] << 16), e[6] | ((uint32_t)e[7] << 16)};
            }
          }
          transpose8x8(in, &r[bi * 8]);
        }
      }
    }
  }

  __device__ __forceinline__ void store(bf16* lds) const {
    const int t = threadIdx.x;
    if constexpr (!KM) {
      const int c = t & 7;
#pragma unroll
      for (int i = 0; i < NREG; ++i) *(u32x4*)(lds + ((t >> 3) + 32 * i) * MF_P + c * 8) = r[i];
    } else {
      constexpr int NB = (ROWS / 8) * (MF_BK / 8);
#pragma unroll
      for (int bi = 0; bi < NREG / 8; ++bi) {
        const int b = t + 256 * bi;
        if (b < NB) {
          const int mb = b % (ROWS / 8), kb = b / (ROWS / 8);
#pragma unroll
          for (int j = 0; j < 8; ++j) *(u32x4*)(lds + (mb * 8 + j) * MF_P + kb * 8) = r[bi * 8 + j];
        }
      }
    }
  }
};

template <bool A_KM, bool B_KN, int EPI, typename TO>
__global__ __launch_bounds__(256, 1) void gemm_mfma(Gemm g) {
  __shared__ bf16 lds[2 * MF_STAGE];
  const int M = g.M, N = g.N, K = g.K;
  const int z = blockIdx.y;
  const bf16* __restrict__ A = (const bf16*)g.A + z * g.sA;
  const bf16* __restrict__ B = (const bf16*)g.B + z * g.sB;

  // tile order: contiguous tile ranges per XCD (blocks are dealt round-robin over 8 XCDs),
  // then groups of 8 tile-rows so neighbouring blocks share A rows and B columns in L2
  const int tiles_m = (M + MF_BM - 1) / MF_BM, tiles_n = (N + MF_BN - 1) / MF_BN;
  const int ntiles = tiles_m * tiles_n;
  int pid = blockIdx.x;
  if ((ntiles & 7) == 0) pid = (pid & 7) * (ntiles >> 3) + (pid >> 3);
  const int GM = 8;
  const int group = GM * tiles_n;
  const int first_m = (pid / group) * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int tm = first_m + (pid % group) % gsz;
  const int tn = (pid % group) / gsz;
  const int m0 = tm * MF_BM, n0 = tn * MF_BN;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  TileLoader<MF_BM, A_KM> la;
  TileLoader<MF_BN, B_KN> lb;
  const int nk = (K + MF_BK - 1) / MF_BK;
  la.load(A, g.lda, m0, M, 0, K);
  lb.load(B, g.ldb, n0, N, 0, K);
  la.store(lds);
  lb.store(lds + MF_BM * MF_P);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      la.load(A, g.lda, m0, M, (kt + 1) * MF_BK, K);
      lb.load(B, g.ldb, n0, N, (kt + 1) * MF_BK, K);
    }
    const bf16* As = lds + cur * MF_STAGE;
    const bf16* Bs = As + MF_BM * MF_P;
#pragma unroll
    for (int kk = 0; kk < MF_BK / 16; ++kk) {
      bf16x8 a[4], b[2];
      const int kc = kk * 16 + (lane >> 5) * 8;
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *(const bf16x8*)(As + (wm * 128 + i * 32 + (lane & 31)) * MF_P + kc);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = *(const bf16x8*)(Bs + (wn * 64 + j * 32 + (lane & 31)) * MF_P + kc);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      bf16* nx = lds + (cur ^ 1) * MF_STAGE;
      la.store(nx);
      lb.store(nx + MF_BM * MF_P);
    }
    __syncthreads();
  }

  // epilogue: lane holds column (lane & 31) and rows 8*(r/4) + 4*(lane/32) + r%4 of each 32x32 block
  TO* C = (TO*)g.C + z * g.sC;
  const float* R = g.R ? g.R + z * g.sR : nullptr;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= M) continue;
        float v = g.alpha * acc[i][j][r];
        TO* c = C + (int64_t)row * g.ldc + col;
        if constexpr (EPI == EPI_ACCUM) v += to_f(*c);
        if constexpr (EPI == EPI_RESID) v += R[(int64_t)row * g.ldr + col];
        *c = from_f<TO>(v);
      }
    }
}

template <bool AK, bool BK_, int EPI, typename TO>
static int launch_mfma_t(const Gemm& g, hipStream_t s) {
  const int tiles = ((g.M + MF_BM - 1) / MF_BM) * ((g.N + MF_BN - 1) / MF_BN);
  hipLaunchKernelGGL((gemm_mfma<AK, BK_, EPI, TO>), dim3(tiles, g.batch), dim3(256), 0, s, g);
  return (int)hipGetLastError();
}

template <bool AK, bool BK_>
static int launch_mfma_l(const Gemm& g, hipStream_t s) {
  if (g.epi == EPI_STORE) {
    return g.c == DT_BF16 ? launch_mfma_t<AK, BK_, EPI_STORE, bf16>(g, s)
                          : launch_mfma_t<AK, BK_, EPI_STORE, float>(g, s);
  }
  if (g.c != DT_F32) return (int)hipErrorInvalidValue;
  if (g.epi == EPI_ACCUM) return launch_mfma_t<AK, BK_, EPI_ACCUM, float>(g, s);
  return launch_mfma_t<AK, BK_, EPI_RESID, float>(g, s);
}

int launch_gemm(const Gemm& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return 0;
  if (g.K <= 0) return (int)hipErrorInvalidValue;
  if (g.epi != EPI_STORE && g.c != DT_F32) return (int)hipErrorInvalidValue;
  if (g.epi == EPI_RESID && !g.R) return (int)hipErrorInvalidValue;
  if (g.ab == DT_BF16) {
    // MFMA path: 16-byte rows need K, leading dimensions and base pointers 8-element aligned
    const bool aligned = (g.K % 8 == 0) && (g.lda % 8 == 0) && (g.ldb % 8 == 0) &&
                         (((uintptr_t)g.A | (uintptr_t)g.B) % 16 == 0) &&
                         (g.batch == 1 || (g.sA % 8 == 0 && g.sB % 8 == 0));
    if (!aligned) return (int)hipErrorInvalidValue;
    if (!g.a_km && !g.b_kn) return launch_mfma_l<false, false>(g, s);
    if (!g.a_km && g.b_kn) return launch_mfma_l<false, true>(g, s);
    if (g.a_km && g.b_kn) return launch_mfma_l<true, true>(g, s);
    return launch_mfma_l<true, false>(g, s);
  }
  dim3 grid((g.N + 63) / 64, (g.M + 63) / 64, g.batch);
  if (g.c == DT_BF16) hipLaunchKernelGGL((gemm_tiled<float, bf16>), grid, dim3(256), 0, s, g);
  else hipLaunchKernelGGL((gemm_tiled<float, float>), grid, dim3(256), 0, s, g);
  return (int)hipGetLastError();
}

}  // namespace hol
