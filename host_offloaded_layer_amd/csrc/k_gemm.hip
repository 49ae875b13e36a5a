// GEMMs of the decoder-layer template: the q/k/v, output, gate/up and down projections, the LM
// head, and their backward products (dX = dY W, dW += dY^T X). MegaTrain summary page, 核心方法:
// each template encapsulates the kernels of the Attention and MLP blocks and holds no weights;
// the weight operand is whichever streamed slot the engine binds.
//
// Two kernels:
//  * gemm_mfma  - bf16 operands, fp32 accumulation on CDNA4 matrix cores
//                 (v_mfma_f32_32x32x16_bf16). 256x128x64 block tile, 4 waves of 128x64,
//                 LDS double buffer with XOR-swizzled K-contiguous rows. Operands stored MN-contiguous
//                 (the backward layouts) are transposed 8x8 in registers on their way into LDS,
//                 so every MFMA fragment is one 16-byte LDS read.
//  * gemm_tiled - plain LDS-tiled FMA kernel for fp32 operands (the fp32 path).
#include "device_common.h"
#include "kernels.h"

namespace hol {

// ------------------------------------------------------------------------------------------
// generic fp32 / mixed tiled GEMM
// ------------------------------------------------------------------------------------------
template <typename TA, typename TB, typename TO>
__global__ __launch_bounds__(256) void gemm_tiled(Gemm g) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  const int z = blockIdx.z;
  const TA* A = (const TA*)g.A + z * g.sA;
  const TB* B = (const TB*)g.B + z * g.sB;
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
constexpr int MF_P = MF_BK;                      // LDS row pitch (bf16): 128 B = 8 chunks of 16 B
constexpr int MF_STAGE = (MF_BM + MF_BN) * MF_P; // bf16 elements per LDS stage

// LDS swizzle: logical 16-byte chunk c of tile row r lives at physical chunk c ^ sw(r). Eight
// consecutive rows (an MFMA fragment read) and rows eight apart (a transposed 8x8 store) both map
// one chunk onto eight different bank groups.
__device__ __forceinline__ int sw(int r) { return (r & 7) ^ ((r >> 3) & 7); }
__device__ __forceinline__ int lds_off(int r, int c) { return r * MF_P + ((c ^ sw(r)) << 3); }

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
      for (int i = 0; i < NREG; ++i) *(u32x4*)(lds + lds_off((t >> 3) + 32 * i, c)) = r[i];
    } else {
      constexpr int NB = (ROWS / 8) * (MF_BK / 8);
#pragma unroll
      for (int bi = 0; bi < NREG / 8; ++bi) {
        const int b = t + 256 * bi;
        if (b < NB) {
          const int mb = b % (ROWS / 8), kb = b / (ROWS / 8);
#pragma unroll
          for (int j = 0; j < 8; ++j) *(u32x4*)(lds + lds_off(mb * 8 + j, kb)) = r[bi * 8 + j];
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
      const int kc = kk * 2 + (lane >> 5);  // logical chunk
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *(const bf16x8*)(As + lds_off(wm * 128 + i * 32 + (lane & 31), kc));
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = *(const bf16x8*)(Bs + lds_off(wn * 64 + j * 32 + (lane & 31), kc));
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


// ------------------------------------------------------------------------------------------
// bf16 MFMA GEMM, both operands K-contiguous (the forward products y = x W^T, and any product
// whose operands were laid out K-contiguous): 256x256 block tile, 4 waves of 128x128 (fp32
// accumulators in AGPRs), BK = 32, a 4-stage LDS ring filled by global_load_lds_dwordx4 (each
// lane's 16 bytes land at LDS base + 16 * lane, no register staging), loads issued 4 tiles ahead.
// Tile rows are 64 bytes (4 chunks of 16 B); two consecutive tile rows share one 128-byte LDS row
// (chunks 0-3: even row, 4-7: odd row) and the 8 chunks of LDS row R are XOR-swizzled with
// (R & 7) ^ ((R >> 3) & 7), so any 8 consecutive lanes of a fragment read hit 8 distinct 16-byte
// bank groups. Requires K % 32 == 0.
// ------------------------------------------------------------------------------------------
constexpr int N2_BM = 256, N2_BN = 256, N2_BK = 32, N2_ST = 4;
constexpr int N2_TILE = (N2_BM + N2_BN) * N2_BK;  // bf16 elements per stage

__device__ __forceinline__ int n2_sw(int R) { return (R & 7) ^ ((R >> 3) & 7); }
// element offset of logical chunk c (0..3) of tile row r
__device__ __forceinline__ int n2_off(int r, int c) { return (r >> 1) * 64 + ((((r & 1) << 2) | c) ^ n2_sw(r >> 1)) * 8; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) const void* gbl_ptr_t;

// Issue this wave's share of one stage (NW waves): LDS rows [8 q, 8 q + 8) (tile rows
// [16 q, 16 q + 16)) of the A tile for q = wave + NW i, and the same of the B tile. Lane i fills
// LDS row 8 q + i / 8 at physical chunk i % 8, so it fetches the logical (row, chunk) stored there.
template <int NW>
__device__ __forceinline__ void n2_issue(bf16* stage, const bf16* __restrict__ A, int64_t lda, int m0, int M,
                                         const bf16* __restrict__ B, int64_t ldb, int n0, int N, int k0) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 16 / NW; ++i) {
    const int R = (w + NW * i) * 8 + (lane >> 3);  // LDS row
    const int lc = (lane & 7) ^ n2_sw(R);          // logical 8-chunk index: (odd row?) * 4 + chunk
    const int r = 2 * R + (lc >> 2);               // tile row
    const int c = lc & 3;
    int gr = m0 + r;
    gr = gr < M ? gr : M - 1;
    const bf16* src = A + (int64_t)gr * lda + k0 + c * 8;
    __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)(stage + (w + NW * i) * 16 * N2_BK), 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 16 / NW; ++i) {
    const int R = (w + NW * i) * 8 + (lane >> 3);
    const int lc = (lane & 7) ^ n2_sw(R);
    const int r = 2 * R + (lc >> 2);
    const int c = lc & 3;
    int gr = n0 + r;
    gr = gr < N ? gr : N - 1;
    const bf16* src = B + (int64_t)gr * ldb + k0 + c * 8;
    __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)(stage + N2_BM * N2_BK + (w + NW * i) * 16 * N2_BK),
                                     16, 0, 0);
  }
}

// NW = 4: waves in a 2 x 2 grid, 128 x 128 each (one wave per SIMD, 256 accumulators a lane).
// NW = 8: waves in a 2 x 4 grid, 128 x 64 each (two waves per SIMD, one's MFMAs cover the other's
// waits).
template <int EPI, typename TO, int NW>
__global__ __launch_bounds__(64 * NW, 1) void gemm_nt2(Gemm g) {
  constexpr int WJ = NW == 4 ? 4 : 2;           // 32-column blocks per wave
  constexpr int LOADS = 2 * 16 / NW;            // loads per wave per stage
  __shared__ __attribute__((aligned(1024))) bf16 lds[N2_ST * N2_TILE];
  const int M = g.M, N = g.N, K = g.K;
  const int z = blockIdx.y;
  const bf16* __restrict__ A = (const bf16*)g.A + z * g.sA;
  const bf16* __restrict__ B = (const bf16*)g.B + z * g.sB;
  const int tiles_m = (M + N2_BM - 1) / N2_BM, tiles_n = (N + N2_BN - 1) / N2_BN;
  const int ntiles = tiles_m * tiles_n;
  int pid = blockIdx.x;
  if ((ntiles & 7) == 0) pid = (pid & 7) * (ntiles >> 3) + (pid >> 3);
  const int GM = 4;
  const int group = GM * tiles_n;
  const int first_m = (pid / group) * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int tm = first_m + (pid % group) % gsz;
  const int tn = (pid % group) / gsz;
  const int m0 = tm * N2_BM, n0 = tn * N2_BN;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w / (NW / 2), wn = w % (NW / 2);
  f32x16 acc[4][WJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < WJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = K / N2_BK;
  // prologue fills the whole ring: stages 0 .. N2_ST-1; iteration kt refills the slot of stage kt
  // with stage kt + N2_ST once stage kt is in registers
#pragma unroll
  for (int s = 0; s < N2_ST; ++s)
    if (s < nk) n2_issue<NW>(lds + s * N2_TILE, A, g.lda, m0, M, B, g.ldb, n0, N, s * N2_BK);

  // Fragments: F0 = k-step 0 of the current stage, F1 = k-step 1. Each k-step's 16 MFMAs run
  // while the next k-step's 8 fragments are being read from LDS.
  bf16x8 a0[4], b0[WJ], a1[4], b1[WJ];
  auto frags = [&](const bf16* st, int kk, bf16x8* a, bf16x8* b) {
    const bf16* As = st;
    const bf16* Bs = st + N2_BM * N2_BK;
    const int c = kk * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *(const bf16x8*)(As + n2_off(wm * 128 + i * 32 + (lane & 31), c));
#pragma unroll
    for (int j = 0; j < WJ; ++j) b[j] = *(const bf16x8*)(Bs + n2_off(wn * 32 * WJ + j * 32 + (lane & 31), c));
  };
  // C^T blocks (B fragment as the MFMA's A operand): a lane then holds one row of C and, per
  // accumulator quad, 4 consecutive columns, so the epilogue moves 16-byte pieces
  auto mma = [&](const bf16x8* a, const bf16x8* b) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < WJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
  };
  // Stage t is ready for everyone once this wave's loads of it are done (at most `later` later
  // stages of 8 loads each may still be in flight) and every wave has passed the barrier; the
  // barrier also certifies that nobody still reads the slot the next issue overwrites.
  // (__syncthreads would drain every prefetched stage: it waits for all outstanding loads.)
  // When stage t is awaited, stages up to t + 2 have been issued (t + 3 for t = 0, right after
  // the prologue).
  auto stage_ready = [&](int t) {
    const int later = min(t == 0 ? N2_ST - 1 : N2_ST - 2, nk - 1 - t);
    if constexpr (LOADS == 8) {
      if (later >= 3) asm volatile("s_waitcnt vmcnt(24)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else if (later == 2) asm volatile("s_waitcnt vmcnt(16)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else if (later == 1) asm volatile("s_waitcnt vmcnt(8)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    } else {
      static_assert(LOADS == 4, "4 or 8 loads per wave per stage");
      if (later >= 3) asm volatile("s_waitcnt vmcnt(12)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else if (later == 2) asm volatile("s_waitcnt vmcnt(8)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else if (later == 1) asm volatile("s_waitcnt vmcnt(4)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
  };
  stage_ready(0);
  frags(lds, 0, a0, b0);
  for (int kt = 0; kt < nk; ++kt) {
    const bf16* st = lds + (kt % N2_ST) * N2_TILE;
    frags(st, 1, a1, b1);
    mma(a0, b0);
    if (kt + 1 < nk) {
      stage_ready(kt + 1);  // stage kt is fully in registers now: its slot can be refilled
      if (kt + N2_ST < nk)
        n2_issue<NW>(lds + (kt % N2_ST) * N2_TILE, A, g.lda, m0, M, B, g.ldb, n0, N, (kt + N2_ST) * N2_BK);
      frags(lds + ((kt + 1) % N2_ST) * N2_TILE, 0, a0, b0);
    }
    mma(a1, b1);
  }

  // epilogue: acc[i][j][4 q + e] is C[row][col + e], row = m0 + 128 wm + 32 i + lane % 32,
  // col = n0 + 32 WJ wn + 32 j + 8 q + 4 (lane / 32)
  TO* C = (TO*)g.C + z * g.sC;
  const float* R = g.R ? g.R + z * g.sR : nullptr;
  constexpr int VB = 4 * (int)sizeof(TO);  // bytes of 4 outputs
  const bool vec = g.ldc % 4 == 0 && (uintptr_t)C % VB == 0 &&
                   (EPI != EPI_RESID || (g.ldr % 4 == 0 && (uintptr_t)R % 16 == 0));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + wm * 128 + i * 32 + (lane & 31);
    if (row >= M) continue;
    TO* crow = C + (int64_t)row * g.ldc;
    const float* rrow = EPI == EPI_RESID ? R + (int64_t)row * g.ldr : nullptr;
#pragma unroll
    for (int j = 0; j < WJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = n0 + wn * 32 * WJ + j * 32 + 8 * q + 4 * (lane >> 5);
        if (col >= N) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = g.alpha * acc[i][j][4 * q + e];
        if (vec && col + 4 <= N) {
          if constexpr (EPI == EPI_RESID) {
            const float4 rv = *(const float4*)(rrow + col);
            v[0] += rv.x; v[1] += rv.y; v[2] += rv.z; v[3] += rv.w;
          }
          if constexpr (sizeof(TO) == 4) {
            if constexpr (EPI == EPI_ACCUM) {
              const float4 cv = *(const float4*)(crow + col);
              v[0] += cv.x; v[1] += cv.y; v[2] += cv.z; v[3] += cv.w;
            }
            *(float4*)(crow + col) = make_float4(v[0], v[1], v[2], v[3]);
          } else {
            bf16x4 o = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
            *(bf16x4*)(crow + col) = o;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (col + e >= N) break;
            float x = v[e];
            if constexpr (EPI == EPI_ACCUM) x += to_f(crow[col + e]);
            if constexpr (EPI == EPI_RESID) x += rrow[col + e];
            crow[col + e] = from_f<TO>(x);
          }
        }
      }
  }
}

// ------------------------------------------------------------------------------------------
// NT3: the same 256 x 256 block and 8-wave grid with 64-deep stages in a 2-slot ring, so one block
// barrier covers twice the MFMA work. A tile row (64 bf16) is one 128-byte LDS row; physical
// 16-byte chunk = logical chunk ^ ((row / 2) % 8) (16 consecutive rows read conflict-free).
// Ungrouped launches are persistent: one block per CU walks several tiles, and the first two
// stages of its next tile are in flight while it stores the current one (a block that stored and
// exited would leave its CU idle through the next block's first loads).
// ------------------------------------------------------------------------------------------
constexpr int N3_BK = 64;
constexpr int N3_TILE = (N2_BM + N2_BN) * N3_BK;  // bf16 elements per stage

__device__ __forceinline__ int n3_off(int r, int c) { return r * N3_BK + ((c ^ ((r >> 1) & 7)) << 3); }

// Pair modes of the NT3 product: the B rows are read in an order that puts both members of every
// pair an epilogue combines into the same wave (its two 32-column blocks).
constexpr int PM_NONE = 0, PM_SWIGLU = 1, PM_ROPE = 2;
// Row of B that feeds output column v. PM_NONE: v. PM_SWIGLU (the gate/up product, B = [W_gate;
// W_up] with F = pp rows each, F % 32 == 0): the columns of each 64-wide block c are the gate rows
// 32 c .. 32 c + 31 followed by the up rows F + 32 c .. F + 32 c + 31. PM_ROPE (the q/k/v product,
// heads of 128 columns, the first pp columns rotated): inside a rotated head, block c (0 or 1)
// holds rows 32 c .. 32 c + 31 of the head and then their rotation partners 64 + 32 c ..; the
// columns past pp keep their order.
template <int PM>
__device__ __forceinline__ int n3_brow(int v, int pp) {
  if constexpr (PM == PM_SWIGLU) return ((v >> 6) << 5) + (v & 31) + ((v & 32) ? pp : 0);
  else if constexpr (PM == PM_ROPE) return v < pp ? (v & ~127) + (((v >> 6) & 1) << 5) + (v & 31) + ((v & 32) ? 64 : 0) : v;
  else return v;
}

// this wave's 64 / NW loads of one stage: LDS rows [8 q, 8 q + 8) for q = wave + NW i of A, then
// of B
template <int NW, int PM = PM_NONE>
__device__ __forceinline__ void n3_issue(bf16* stage, const bf16* __restrict__ A, int64_t lda, int m0, int M,
                                         const bf16* __restrict__ B, int64_t ldb, int n0, int N, int k0, int pp) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 32 / NW; ++i) {
    const int R = (w + NW * i) * 8 + (lane >> 3);
    const int lc = (lane & 7) ^ ((R >> 1) & 7);
    int gr = m0 + R;
    gr = gr < M ? gr : M - 1;
    __builtin_amdgcn_global_load_lds((gbl_ptr_t)(A + (int64_t)gr * lda + k0 + lc * 8),
                                     (lds_ptr_t)(stage + (w + NW * i) * 8 * N3_BK), 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 32 / NW; ++i) {
    const int R = (w + NW * i) * 8 + (lane >> 3);
    const int lc = (lane & 7) ^ ((R >> 1) & 7);
    int gr = n0 + R;
    gr = n3_brow<PM>(gr < N ? gr : N - 1, pp);
    __builtin_amdgcn_global_load_lds((gbl_ptr_t)(B + (int64_t)gr * ldb + k0 + lc * 8),
                                     (lds_ptr_t)(stage + N2_BM * N3_BK + (w + NW * i) * 8 * N3_BK), 16, 0, 0);
  }
}

// NW = 8: 2 x 4 waves of 128 x 64 (two per SIMD); NW = 4: 2 x 2 waves of 128 x 128 (one per SIMD,
// a third fewer LDS fragment reads per MFMA).
// The same loads through buffer resources: a lane's byte offset into A (B) is fixed for the whole
// tile (rows clamped as above), the stage's k offset is a scalar, so no per-load address arithmetic.
template <int NW, int PM = PM_NONE>
struct N3Buf {
  uint32_t va[32 / NW], vb[32 / NW];
  __device__ __forceinline__ void init(int64_t lda, int m0, int M, int64_t ldb, int n0, int N, int pp) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < 32 / NW; ++i) {
      const int R = (w + NW * i) * 8 + (lane >> 3);
      const int lc = (lane & 7) ^ ((R >> 1) & 7);
      va[i] = (uint32_t)(min(m0 + R, M - 1) * lda * 2 + lc * 16);
      vb[i] = (uint32_t)(n3_brow<PM>(min(n0 + R, N - 1), pp) * ldb * 2 + lc * 16);
    }
  }
  __device__ __forceinline__ void issue(bf16* stage, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, int k0) const {
    // wave-uniform, so the LDS destinations are scalar arithmetic
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int i = 0; i < 32 / NW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(stage + (w + NW * i) * 8 * N3_BK), 16, va[i], k0 * 2, 0, 0);
#pragma unroll
    for (int i = 0; i < 32 / NW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(stage + N2_BM * N3_BK + (w + NW * i) * 8 * N3_BK), 16,
                                               vb[i], k0 * 2, 0, 0);
  }
};

// Whether every byte of A and B lies within an unsigned 32-bit offset of its base (the buffer path).
static bool n3_buffer_ok(const Gemm& g) {
  const uint64_t ea = (uint64_t)g.M * (uint64_t)g.lda * 2, eb = (uint64_t)g.N * (uint64_t)g.ldb * 2;
  return g.batch == 1 && ea < (1ull << 32) && eb < (1ull << 32);
}

// ------------------------------------------------------------------------------------------
// TN layout of the NT3 kernel: C = Aᵀ B with both operands stored K-major (A [K][M], B [K][N], row
// strides lda, ldb), the layout of the weight-gradient products dW = dYᵀ X over saved activations,
// read as stored (no transposes). Same block, waves, ring, persistence and split tail. A stage holds 64 k-rows
// of 256 values (512 B) per operand, 16-byte chunk c of row k at physical chunk c ^ 4 (k mod 4).
// An MFMA fragment (8 consecutive k of one m) is two ds_read_b64_tr_b16: within each 16-lane
// group, lane 16 g + 4 a + b receives element b of the 8-byte pieces addressed by lanes
// 16 g + a + 4 j (j = 0..3), so lane 16 g + a + 4 j addresses row k0 + j, columns
// m0 + 16 (g mod 2) + 4 a .. + 3, and lane l ends with m = m0 + l mod 32, k = k0 + 0..3. The
// swizzle keeps each half-wave's 4 rows x 64 bytes on distinct banks.
// ------------------------------------------------------------------------------------------
typedef short tr4_t __attribute__((ext_vector_type(4)));

typedef short tr8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ tr4_t tr_read(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) tr4_t*)p);
}

// fragment of 8 consecutive k: rows k0 .. k0 + 3 at p, k0 + 4 .. k0 + 7 four rows further
__device__ __forceinline__ bf16x8 tr_frag(const bf16* p) {
  const tr4_t lo = tr_read(p), hi = tr_read(p + 4 * 256);
  const tr8_t x = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, x);
}

// element offset, inside one operand's stage region, of this lane's transposed-read piece for
// the 32-wide block at column c0, k-row offset 0 (add 256 k for row k)
__device__ __forceinline__ int t3_frag_off(int c0, int lane) {
  const int g = lane >> 4, a = lane & 3, j = (lane >> 2) & 3;
  const int col = c0 + 16 * (g & 1) + 4 * a;
  const int pc = (col >> 3) ^ (4 * j);
  return (8 * (g >> 1) + j) * 256 + pc * 8 + (col & 4);
}

// Stage loads: instruction q = w + NW i fills stage rows 2 q, 2 q + 1 (1 KB) of an operand;
// lane: row 2 q + lane / 32, physical chunk lane % 32 = logical chunk (lane % 32) ^ 4 (row % 4).
// Columns past M (N) are clamped (their products land in rows that are not stored).
template <int NW>
struct T3Buf {
  uint32_t va[32 / NW], vb[32 / NW];
  __device__ __forceinline__ void init(int64_t lda, int m0, int M, int64_t ldb, int n0, int N) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < 32 / NW; ++i) {
      const int r = 2 * (w + NW * i) + (lane >> 5);
      const int c = (lane & 31) ^ (4 * (r & 3));
      va[i] = (uint32_t)(((int64_t)r * lda + min(m0 + 8 * c, M - 8)) * 2);
      vb[i] = (uint32_t)(((int64_t)r * ldb + min(n0 + 8 * c, N - 8)) * 2);
    }
  }
  __device__ __forceinline__ void issue(bf16* stage, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, uint32_t sa,
                                        uint32_t sb) const {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // scalar LDS destinations
#pragma unroll
    for (int i = 0; i < 32 / NW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(stage + (w + NW * i) * 512), 16, va[i], (int)sa, 0, 0);
#pragma unroll
    for (int i = 0; i < 32 / NW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(stage + 64 * 256 + (w + NW * i) * 512), 16, vb[i],
                                               (int)sb, 0, 0);
  }
};

// Whether every byte of A and B lies within an unsigned 32-bit offset of its base.
static bool t3_buffer_ok(const Gemm& g) {
  const uint64_t ea = (uint64_t)g.K * (uint64_t)g.lda * 2, eb = (uint64_t)g.K * (uint64_t)g.ldb * 2;
  return g.batch == 1 && ea < (1ull << 32) && eb < (1ull << 32);
}


// GRP: one launch over groups of rows (the experts of a mixture-of-experts layer). The table gives
// each group's first row and first row tile; the grid is an upper bound, the real tile count is
// read from the table, dealt in 8 equal contiguous ranges (one per XCD) with the surplus blocks
// leaving at once, and a block finds its group by binary search over the row-tile offsets.
// Epilogue of the 256 x 256 tiles: acc[i][j][4 q + e] is C[row][col + e], row = m0 + 128 wm +
// 32 i + lane % 32, col = n0 + 32 WJ wn + 32 j + 8 q + 4 (lane / 32) (Cᵀ blocks, so a lane holds
// 4 consecutive columns of one row per quad).
template <int EPI, typename TO, int WJ>
__device__ __forceinline__ void n3_store(const Gemm& g, const f32x16 (&acc)[4][WJ], TO* C, const float* R, int M,
                                         int N, int m0, int n0, int wm, int wn, int lane) {
  constexpr int VB = 4 * (int)sizeof(TO);
  const bool vec = g.ldc % 4 == 0 && (uintptr_t)C % VB == 0 &&
                   (EPI != EPI_RESID || (g.ldr % 4 == 0 && (uintptr_t)R % 16 == 0));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + wm * 128 + i * 32 + (lane & 31);
    if (row >= M) continue;
    TO* crow = C + (int64_t)row * g.ldc;
    const float* rrow = EPI == EPI_RESID ? R + (int64_t)row * g.ldr : nullptr;
#pragma unroll
    for (int j = 0; j < WJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = n0 + wn * 32 * WJ + j * 32 + 8 * q + 4 * (lane >> 5);
        if (col >= N) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = g.alpha * acc[i][j][4 * q + e];
        if (vec && col + 4 <= N) {
          if constexpr (EPI == EPI_RESID) {
            const float4 rv = *(const float4*)(rrow + col);
            v[0] += rv.x; v[1] += rv.y; v[2] += rv.z; v[3] += rv.w;
          }
          if constexpr (sizeof(TO) == 4) {
            if constexpr (EPI == EPI_ACCUM) {
              const float4 cv = *(const float4*)(crow + col);
              v[0] += cv.x; v[1] += cv.y; v[2] += cv.z; v[3] += cv.w;
            }
            *(float4*)(crow + col) = make_float4(v[0], v[1], v[2], v[3]);
          } else {
            bf16x4 o = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
            *(bf16x4*)(crow + col) = o;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (col + e >= N) break;
            float x = v[e];
            if constexpr (EPI == EPI_ACCUM) x += to_f(crow[col + e]);
            if constexpr (EPI == EPI_RESID) x += rrow[col + e];
            crow[col + e] = from_f<TO>(x);
          }
        }
      }
  }
}

// Whether a tile's epilogue is guaranteed to issue one vector store (and, for the accumulate and
// residual epilogues, one vector load) per quad of every wave: a full tile with the vector path.
template <int EPI, typename TO>
__device__ __forceinline__ bool n3_full_tile(const Gemm& g, const TO* C, const float* R, int M, int N, int m0, int n0) {
  constexpr int VB = 4 * (int)sizeof(TO);
  return m0 + N2_BM <= M && n0 + N2_BN <= N && g.ldc % 4 == 0 && (uintptr_t)C % VB == 0 &&
         (EPI != EPI_RESID || (g.ldr % 4 == 0 && (uintptr_t)R % 16 == 0));
}

// SwiGLU epilogue (B rows interleaved by n3_brow<true>): block j = 0 of a wave holds the gate and
// j = 1 the up value of feature f = (n0 + 64 wn) / 2 + 8 q + 4 (lane / 32) + e. C receives gate |
// up rounded to bf16, exactly as the plain product stores them, and C2 (row stride ldc2) the
// SwiGLU of the rounded pair. Vector stores only: F % 32 == 0, ldc and ldc2 multiples of 4 and
// 8-byte aligned C, C2 (checked by the launcher). 48 stores per wave for a full tile.
__device__ __forceinline__ void n3_store_swiglu(const Gemm& g, const f32x16 (&acc)[4][2], bf16* C, int M, int N,
                                                int m0, int n0, int wm, int wn, int lane) {
  const int F = N >> 1;
  bf16* C2 = (bf16*)g.C2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + wm * 128 + i * 32 + (lane & 31);
    if (row >= M) continue;
    bf16* crow = C + (int64_t)row * g.ldc;
    bf16* arow = C2 + (int64_t)row * g.ldc2;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int f = (n0 >> 1) + wn * 32 + 8 * q + 4 * (lane >> 5);
      if (f >= F) continue;
      bf16x4 gb, ub, ab;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gb[e] = (bf16)(g.alpha * acc[i][0][4 * q + e]);
        ub[e] = (bf16)(g.alpha * acc[i][1][4 * q + e]);
        ab[e] = (bf16)swiglu_f((float)gb[e], (float)ub[e]);
      }
      *(bf16x4*)(crow + f) = gb;
      *(bf16x4*)(crow + F + f) = ub;
      *(bf16x4*)(arow + f) = ab;
    }
  }
}

// Tile origin of tile q in the grouped order: groups of 4 row tiles, column-major inside a group
// (the 32 tiles an XCD runs at once share A and B panels in its L2).
__device__ __forceinline__ void n3_origin(int q, int tiles_m, int tiles_n, int& m0, int& n0) {
  const int GM = 4;
  const int group = GM * tiles_n;
  const int first_m = (q / group) * GM;
  const int gsz = min(tiles_m - first_m, GM);
  m0 = (first_m + (q % group) % gsz) * N2_BM;
  n0 = ((q % group) / gsz) * N2_BN;
}

// SPL (split tail, fp32 store only): an XCD's tiles that do not fill a last round of its blocks
// are each cut along K into g.spl_f equal parts. A block's work items are then its whole tiles
// (g.spl_full per XCD, the full rounds) followed by at most one part, whose raw sums go to the
// workspace (one 256 x 256 fp32 slot per part: slot x r f + q f + part for the XCD's q-th split
// tile); gemm_split_reduce_k adds the parts in order and applies alpha.
// RoPE epilogue (B rows read by n3_brow<PM_ROPE>): in a rotated head, block j = 0 of a wave holds
// column jj = 32 c + 8 q + 4 (lane / 32) + e of the head (c = the wave's 64-column block within
// the head) and block j = 1 its partner jj + 64; they are rotated with the table row of the
// token's position (row mod S, tables [S][64]) exactly as the element-wise RoPE does on the fp32
// product, and rounded to bf16 once. Columns past the rotated ones (v) are stored as they are.
// 32 vector stores a wave for a full tile (and the table loads before them).
__device__ __forceinline__ void n3_store_rope(const Gemm& g, const f32x16 (&acc)[4][2], bf16* C, int M, int N,
                                              int m0, int n0, int wm, int wn, int lane) {
  const int cb = n0 + wn * 64;  // this wave's first (virtual) column
  if (cb >= N) return;
  const bool rot = cb < g.rope_nr;
  const int hb = cb & ~127, c = (cb >> 6) & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + wm * 128 + i * 32 + (lane & 31);
    if (row >= M) continue;
    bf16* crow = C + (int64_t)row * g.ldc;
    const int pos = row % g.rope_S;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int jj = 32 * c + 8 * q + 4 * (lane >> 5);
      bf16x4 x, y;
      if (rot) {
        const float4 c4 = *(const float4*)(g.rope_cos + (int64_t)pos * 64 + jj);
        const float4 s4 = *(const float4*)(g.rope_sin + (int64_t)pos * 64 + jj);
        const float cv[4] = {c4.x, c4.y, c4.z, c4.w}, sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float xx, yy;
          rot_pair(g.alpha * acc[i][0][4 * q + e], g.alpha * acc[i][1][4 * q + e], cv[e], sv[e], xx, yy);
          x[e] = (bf16)xx;
          y[e] = (bf16)yy;
        }
        *(bf16x4*)(crow + hb + jj) = x;
        *(bf16x4*)(crow + hb + 64 + jj) = y;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = (bf16)(g.alpha * acc[i][0][4 * q + e]);
          y[e] = (bf16)(g.alpha * acc[i][1][4 * q + e]);
        }
        *(bf16x4*)(crow + cb + 8 * q + 4 * (lane >> 5)) = x;
        *(bf16x4*)(crow + cb + 32 + 8 * q + 4 * (lane >> 5)) = y;
      }
    }
  }
}

// Instruction order of one k-step: the first six of its 8 MFMAs each followed by one of the 6
// fragment reads of the next k-step, the last two MFMAs alone. Left to itself the compiler moved each read down
// next to the MFMA that consumes it, so a wave waited for LDS before most of its MFMAs; with the
// reads spread over the step they have ≈6 MFMAs to land (2.5–3 % over the decoder shapes,
// bitwise the same products). Off for the global_load_lds path (operands past 4 GiB), where the
// longer-lived fragments would push more registers to scratch.
// (RD: LDS reads per fragment, 2 in the TN layout)
template <bool ON, int RD = 1>
__device__ __forceinline__ void n3_interleave() {
  if constexpr (ON) {
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);  // one fragment's LDS reads
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  }
}

// TN: both operands K-major (the TN layout above); buffer path only, no groups, no pair modes.
template <int EPI, typename TO, int NW, bool BUF, bool GRP, int PM = PM_NONE, bool SPL = false, bool TN = false>
__global__ __launch_bounds__(64 * NW, 1) void gemm_nt3(Gemm g) {
  constexpr int WJ = NW == 4 ? 4 : 2;  // 32-column blocks per wave
  static_assert(NW == 8, "the epilogue count below assumes 8 waves");
  __shared__ __attribute__((aligned(1024))) bf16 lds[2 * N3_TILE];
  int M = g.M;
  const int N = g.N, K = g.K;
  const int z = blockIdx.y;
  const bf16* __restrict__ A = (const bf16*)g.A + z * g.sA;
  const bf16* __restrict__ B = (const bf16*)g.B + z * g.sB;
  TO* C = (TO*)g.C + z * g.sC;
  const float* R = g.R ? g.R + z * g.sR : nullptr;
  const int tiles_n = (N + N2_BN - 1) / N2_BN;
  int m0, n0;
  // tile sequence: grouped, one tile; otherwise the tiles are dealt in 8 contiguous ranges, one
  // per XCD (workgroup i runs on XCD i % 8), and the XCD's blocks take its tiles in turn, so the
  // 32 tiles in flight on one XCD share A and B panels in its L2
  int p = 0, p_end = 1, p_step = 1;
  const int tiles_m = (M + N2_BM - 1) / N2_BM;
  auto origin = [&](int q) { n3_origin(q, tiles_m, tiles_n, m0, n0); };
  // K range of the current work item, and its workspace slot (-1: a whole tile, stored normally)
  int kbeg = 0, kend = K, slot = -1;
  int xstart = 0;  // SPL: first tile of this XCD's range
  auto item = [&](int i) {
    if constexpr (SPL) {
      if (i < g.spl_full) {
        origin(xstart + i);
        kbeg = 0;
        kend = K;
        slot = -1;
      } else {
        const int j = i - g.spl_full, kp = K / g.spl_f;
        origin(xstart + g.spl_full + j / g.spl_f);
        kbeg = (j % g.spl_f) * kp;
        kend = kbeg + kp;
        slot = (blockIdx.x & 7) * (p_end - g.spl_full) + j;
      }
    } else {
      origin(i);
    }
  };
  if constexpr (GRP) {
    const int G = g.ngroups;
    const int32_t* roff = g.grp;
    const int32_t* toff = g.grp + G + 1;
    const int total = toff[G] * tiles_n;
    const int per = (total + 7) >> 3;
    const int i = blockIdx.x >> 3;
    if (i >= per) return;
    const int lp = (blockIdx.x & 7) * per + i;
    if (lp >= total) return;
    const int rt = lp / tiles_n, tn = lp - rt * tiles_n;
    int lo = 0, hi = G;  // toff[lo] <= rt < toff[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (toff[mid] <= rt) lo = mid;
      else hi = mid;
    }
    const int r0 = roff[lo];
    M = roff[lo + 1] - r0;
    A += (int64_t)r0 * g.lda;
    B = (const bf16*)g.B + (int64_t)lo * g.sB;
    C += (int64_t)r0 * g.ldc;
    if (R) R += (int64_t)r0 * g.ldr;
    m0 = (rt - toff[lo]) * N2_BM;
    n0 = tn * N2_BN;
  } else {
    const int ntiles = tiles_m * tiles_n;
    const int x = blockIdx.x & 7;
    p_step = gridDim.x >> 3;
    if constexpr (SPL) {  // items, not tiles (ntiles % 8 == 0: every XCD has ntiles / 8 tiles)
      xstart = (ntiles >> 3) * x;
      p = blockIdx.x >> 3;
      p_end = g.spl_full + ((ntiles >> 3) - g.spl_full) * g.spl_f;
    } else {
      p = (int)((int64_t)ntiles * x / 8) + (blockIdx.x >> 3);
      p_end = (int)((int64_t)ntiles * (x + 1) / 8);
    }
    if (p >= p_end) return;
    item(p);
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w / (NW / 2), wn = w % (NW / 2);
  f32x16 acc[4][WJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < WJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  static_assert(PM == PM_NONE || (EPI == EPI_STORE && sizeof(TO) == 2 && !GRP && WJ == 2), "pair modes: bf16 store, one group");
  static_assert(!SPL || (EPI == EPI_STORE && sizeof(TO) == 4 && !GRP && PM == PM_NONE), "split tail: fp32 store, one group");
  static_assert(!TN || (BUF && !GRP && PM == PM_NONE), "TN layout: buffer path, one group, no pair mode");
  constexpr bool SW = PM == PM_SWIGLU;
  const int pp = PM == PM_SWIGLU ? N >> 1 : (PM == PM_ROPE ? g.rope_nr : 0);
  int nk = (kend - kbeg) / N3_BK;
  N3Buf<NW, PM> nb;
  T3Buf<NW> tb;
  const int64_t ea = TN ? (int64_t)K * g.lda * 2 : (int64_t)M * g.lda * 2;
  const int64_t eb = TN ? (int64_t)K * g.ldb * 2 : (int64_t)N * g.ldb * 2;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, (int)(uint32_t)ea, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void*)B, (short)0, (int)(uint32_t)eb, 0x00020000);
  auto issue = [&](bf16* stage, int k0) {  // k0 relative to the item's first k
    if constexpr (TN) tb.issue(stage, ra, rb, (uint32_t)((kbeg + k0) * g.lda * 2), (uint32_t)((kbeg + k0) * g.ldb * 2));
    else if constexpr (BUF) nb.issue(stage, ra, rb, kbeg + k0);
    else n3_issue<NW, PM>(stage, A, g.lda, m0, M, B, g.ldb, n0, N, kbeg + k0, pp);
  };
  auto start_tile = [&]() {
    if constexpr (TN) tb.init(g.lda, m0, M, g.ldb, n0, N);
    else if constexpr (BUF) nb.init(g.lda, m0, M, g.ldb, n0, N, pp);
    issue(lds, 0);
    if (nk > 1) issue(lds + N3_TILE, N3_BK);
  };
  // TN: this lane's transposed-read offsets inside a stage (A region, then B at 64 x 256)
  int fa[4], fb[WJ];
  if constexpr (TN) {
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = t3_frag_off(wm * 128 + i * 32, lane);
#pragma unroll
    for (int j = 0; j < WJ; ++j) fb[j] = 64 * 256 + t3_frag_off(wn * 32 * WJ + j * 32, lane);
  }
  bf16x8 a0[4], b0[WJ], a1[4], b1[WJ];
  auto frags = [&](const bf16* st, int kk, bf16x8* a, bf16x8* b) {
    if constexpr (TN) {
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = tr_frag(st + fa[i] + kk * 16 * 256);
#pragma unroll
      for (int j = 0; j < WJ; ++j) b[j] = tr_frag(st + fb[j] + kk * 16 * 256);
    } else {
      const bf16* Bs = st + N2_BM * N3_BK;
      const int c = kk * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *(const bf16x8*)(st + n3_off(wm * 128 + i * 32 + (lane & 31), c));
#pragma unroll
      for (int j = 0; j < WJ; ++j) b[j] = *(const bf16x8*)(Bs + n3_off(wn * 32 * WJ + j * 32 + (lane & 31), c));
    }
  };
  auto mma = [&](const bf16x8* a, const bf16x8* b) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < WJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
  };
  start_tile();
  // memory operations the previous tile's epilogue issued after this tile's first two stages, at
  // least (vmcnt counts loads and stores together, in issue order): 0 for the first tile
  int after = 0;
  for (;;) {
    // stage 0 ready (stage 1's loads and the previous epilogue may still be in flight)
    // (the epilogue issues 32 memory operations per wave, 48 with SwiGLU)
    if (nk > 1) {
      if (after && SW) asm volatile("s_waitcnt vmcnt(56)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else if (after) asm volatile("s_waitcnt vmcnt(40)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(8)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    } else {
      if (after && SW) asm volatile("s_waitcnt vmcnt(48)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else if (after) asm volatile("s_waitcnt vmcnt(32)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    frags(lds, 0, a0, b0);
    for (int kt = 0; kt + 1 < nk; ++kt) {
      const bf16* st = lds + (kt & 1) * N3_TILE;
      frags(st, 1, a1, b1);
      mma(a0, b0);
      n3_interleave<BUF, TN ? 2 : 1>();
      frags(st, 2, a0, b0);
      mma(a1, b1);
      n3_interleave<BUF, TN ? 2 : 1>();
      frags(st, 3, a1, b1);
      mma(a0, b0);
      n3_interleave<BUF, TN ? 2 : 1>();
      // stage kt + 1 is the only load in flight (for the first stage of a tile, behind it at
      // most the previous epilogue's memory operations); once every wave has also finished
      // reading this slot, it takes stage kt + 2
      if (kt == 0 && after && SW) asm volatile("s_waitcnt vmcnt(48)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else if (kt == 0 && after) asm volatile("s_waitcnt vmcnt(32)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (kt + 2 < nk) issue(lds + (kt & 1) * N3_TILE, (kt + 2) * N3_BK);
      frags(lds + ((kt + 1) & 1) * N3_TILE, 0, a0, b0);
      mma(a1, b1);
      n3_interleave<BUF, TN ? 2 : 1>();
    }
    {  // the tile's last stage
      const bf16* st = lds + ((nk - 1) & 1) * N3_TILE;
      frags(st, 1, a1, b1);
      mma(a0, b0);
      n3_interleave<BUF, TN ? 2 : 1>();
      frags(st, 2, a0, b0);
      mma(a1, b1);
      n3_interleave<BUF, TN ? 2 : 1>();
      frags(st, 3, a1, b1);
      mma(a0, b0);
      n3_interleave<BUF, TN ? 2 : 1>();
      mma(a1, b1);
    }
    // next tile: its first two stages go up before this tile's results go out
    const int cm0 = m0, cn0 = n0, cslot = slot;
    p += p_step;
    const bool next = !GRP && p < p_end;
    if (next) {
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // every wave done with both slots
      item(p);
      nk = (kend - kbeg) / N3_BK;
      start_tile();
      asm volatile("" ::: "memory");
    }
    if constexpr (SW) {
      after = cm0 + N2_BM <= M && cn0 + N2_BN <= N ? 1 : 0;
      n3_store_swiglu(g, acc, C, M, N, cm0, cn0, wm, wn, lane);
    } else if constexpr (PM == PM_ROPE) {
      after = cm0 + N2_BM <= M && cn0 + N2_BN <= N ? 1 : 0;  // (32 stores a wave; the table loads only add)
      n3_store_rope(g, acc, C, M, N, cm0, cn0, wm, wn, lane);
    } else if (SPL && cslot >= 0) {  // a part of a split tile: raw sums, whole 256 x 256 slot
      Gemm gw = g;
      gw.ldc = N2_BN;
      gw.alpha = 1.f;
      after = 1;  // 32 vector stores a wave, as a whole fp32 tile
      n3_store<EPI_STORE, TO, WJ>(gw, acc, (TO*)(g.ws + (int64_t)cslot * (N2_BM * N2_BN)), nullptr, N2_BM, N2_BN, 0, 0,
                                  wm, wn, lane);
    } else {
      after = n3_full_tile<EPI, TO>(g, C, R, M, N, cm0, cn0) ? 1 : 0;
      n3_store<EPI, TO, WJ>(g, acc, C, R, M, N, cm0, cn0, wm, wn, lane);
    }
    if (!next) break;
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < WJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  }
}

constexpr int NT3_WAVES = 8;
// (explicit instantiations: the host pass does not always emit the launch stubs of the
// buffer-path instantiations on its own)
#define HOL_NT3_INST(GRP)                                                           \
  template __global__ void gemm_nt3<EPI_STORE, float, NT3_WAVES, true, GRP>(Gemm);  \
  template __global__ void gemm_nt3<EPI_STORE, bf16, NT3_WAVES, true, GRP>(Gemm);   \
  template __global__ void gemm_nt3<EPI_ACCUM, float, NT3_WAVES, true, GRP>(Gemm);  \
  template __global__ void gemm_nt3<EPI_RESID, float, NT3_WAVES, true, GRP>(Gemm);  \
  template __global__ void gemm_nt3<EPI_STORE, float, NT3_WAVES, false, GRP>(Gemm); \
  template __global__ void gemm_nt3<EPI_STORE, bf16, NT3_WAVES, false, GRP>(Gemm);  \
  template __global__ void gemm_nt3<EPI_ACCUM, float, NT3_WAVES, false, GRP>(Gemm); \
  template __global__ void gemm_nt3<EPI_RESID, float, NT3_WAVES, false, GRP>(Gemm);
HOL_NT3_INST(false)
HOL_NT3_INST(true)
#undef HOL_NT3_INST
template __global__ void gemm_nt3<EPI_STORE, bf16, NT3_WAVES, true, false, PM_SWIGLU>(Gemm);
template __global__ void gemm_nt3<EPI_STORE, bf16, NT3_WAVES, false, false, PM_SWIGLU>(Gemm);
template __global__ void gemm_nt3<EPI_STORE, bf16, NT3_WAVES, true, false, PM_ROPE>(Gemm);
template __global__ void gemm_nt3<EPI_STORE, bf16, NT3_WAVES, false, false, PM_ROPE>(Gemm);
template __global__ void gemm_nt3<EPI_STORE, float, NT3_WAVES, true, false, PM_NONE, true>(Gemm);
template __global__ void gemm_nt3<EPI_STORE, float, NT3_WAVES, true, false, PM_NONE, false, true>(Gemm);
template __global__ void gemm_nt3<EPI_STORE, bf16, NT3_WAVES, true, false, PM_NONE, false, true>(Gemm);
template __global__ void gemm_nt3<EPI_ACCUM, float, NT3_WAVES, true, false, PM_NONE, false, true>(Gemm);
template __global__ void gemm_nt3<EPI_RESID, float, NT3_WAVES, true, false, PM_NONE, false, true>(Gemm);
template __global__ void gemm_nt3<EPI_STORE, float, NT3_WAVES, true, false, PM_NONE, true, true>(Gemm);

// Sum of the parts of the split tiles (gemm_nt3 with SPL): one block per split tile; thread t
// owns columns 4 (t mod 64) .. + 3 of rows t / 64 + 4 i. Parts are added in order 0, 1, ... so the
// result does not depend on which part finished first.
__global__ __launch_bounds__(256) void gemm_split_reduce_k(Gemm g) {
  const int tiles_m = (g.M + N2_BM - 1) / N2_BM, tiles_n = (g.N + N2_BN - 1) / N2_BN;
  const int n_x = tiles_m * tiles_n / 8, r = n_x - g.spl_full;  // split tiles per XCD range
  const int x = blockIdx.x / r, q = blockIdx.x % r;
  int m0, n0;
  n3_origin(n_x * x + g.spl_full + q, tiles_m, tiles_n, m0, n0);
  const float* part = g.ws + (int64_t)(x * r + q) * g.spl_f * (N2_BM * N2_BN);
  float* C = (float*)g.C;
  const int c = 4 * (threadIdx.x & 63);
  const int col = n0 + c;
  const bool vec = g.ldc % 4 == 0 && ((uintptr_t)C & 15) == 0 && col + 4 <= g.N;
  for (int rr = threadIdx.x >> 6; rr < N2_BM; rr += 4) {
    const int row = m0 + rr;
    if (row >= g.M || col >= g.N) continue;
    float4 v = *(const float4*)(part + rr * N2_BN + c);
    for (int f = 1; f < g.spl_f; ++f) {
      const float4 u = *(const float4*)(part + (int64_t)f * (N2_BM * N2_BN) + rr * N2_BN + c);
      v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
    }
    v.x *= g.alpha; v.y *= g.alpha; v.z *= g.alpha; v.w *= g.alpha;
    float* crow = C + (int64_t)row * g.ldc;
    if (vec) {
      *(float4*)(crow + col) = v;
    } else {
      const float e[4] = {v.x, v.y, v.z, v.w};
      for (int k = 0; k < 4 && col + k < g.N; ++k) crow[col + k] = e[k];
    }
  }
}

// persistent grid of the ungrouped GEMM: one block per CU (a block fills a CU's LDS), in whole
// XCD rounds of 8
static int n3_persistent_grid(int ntiles) {
  static int ncu = 0;
  if (!ncu) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    ncu = n;
  }
  const int g = ntiles < ncu ? ntiles : ncu;
  return (g + 7) / 8 * 8;
}

// Split-tail plan for an fp32-store product: with every XCD range holding n tiles for its c
// blocks, n = R c + r with R >= 1 and 0 < r <= c / 2, the r tail tiles are cut into f = 2 or 4 K
// parts (r f <= c, K % 64 f == 0), so the last round runs r f part tiles instead of r whole
// ones. Returns false when the plan does not apply.
static bool n3_split_plan(const Gemm& g, int grid, Gemm& out) {
  if (!g.ws || g.batch != 1 || g.epi != EPI_STORE || g.c != DT_F32 || !(g.a_km ? t3_buffer_ok(g) : n3_buffer_ok(g)))
    return false;
  const int ntiles = ((g.M + N2_BM - 1) / N2_BM) * ((g.N + N2_BN - 1) / N2_BN);
  if (ntiles % 8 || grid % 8) return false;
  const int c = grid / 8, n = ntiles / 8, R = n / c, r = n % c;
  if (R < 1 || r == 0 || 2 * r > c) return false;
  int f = 4 * r <= c ? 4 : 2;
  while (f > 1 && g.K % (N3_BK * f)) f /= 2;
  if (f < 2 || (int64_t)8 * r * f * N2_BM * N2_BN > g.ws_floats) return false;
  out = g;
  out.spl_full = R * c;
  out.spl_f = f;
  return true;
}

// TN: both operands K-major (checked by the caller: buffer path, M and N multiples of 8)
template <int EPI, typename TO, bool GRP, bool TN = false>
static int launch_nt3_t(const Gemm& g, hipStream_t s) {
  const int tn = (g.N + N2_BN - 1) / N2_BN;
  // grouped: an upper bound of the tile count rounded up to the 8 XCD ranges
  const int tiles = GRP ? (int)((((int64_t)g.grp_max_rt * tn) + 7) / 8 * 8) : n3_persistent_grid(((g.M + N2_BM - 1) / N2_BM) * tn);
  if (tiles <= 0) return 0;
  if constexpr (EPI == EPI_STORE && sizeof(TO) == 4 && !GRP) {
    Gemm gs;
    if (n3_split_plan(g, tiles, gs)) {
      hipLaunchKernelGGL((gemm_nt3<EPI_STORE, float, NT3_WAVES, true, false, PM_NONE, true, TN>), dim3(tiles),
                         dim3(64 * NT3_WAVES), 0, s, gs);
      const int nsplit = (((g.M + N2_BM - 1) / N2_BM) * tn / 8 - gs.spl_full) * 8;
      hipLaunchKernelGGL(gemm_split_reduce_k, dim3(nsplit), dim3(256), 0, s, gs);
      return (int)hipGetLastError();
    }
  }
  if constexpr (TN)
    hipLaunchKernelGGL((gemm_nt3<EPI, TO, NT3_WAVES, true, false, PM_NONE, false, true>), dim3(tiles), dim3(64 * NT3_WAVES),
                       0, s, g);
  else if (n3_buffer_ok(g))
    hipLaunchKernelGGL((gemm_nt3<EPI, TO, NT3_WAVES, true, GRP>), dim3(tiles, g.batch), dim3(64 * NT3_WAVES), 0, s, g);
  else
    hipLaunchKernelGGL((gemm_nt3<EPI, TO, NT3_WAVES, false, GRP>), dim3(tiles, g.batch), dim3(64 * NT3_WAVES), 0, s, g);
  return (int)hipGetLastError();
}

template <bool GRP, bool TN = false>
static int launch_nt3(const Gemm& g, hipStream_t s) {
  if (g.epi == EPI_STORE)
    return g.c == DT_BF16 ? launch_nt3_t<EPI_STORE, bf16, GRP, TN>(g, s) : launch_nt3_t<EPI_STORE, float, GRP, TN>(g, s);
  if (g.epi == EPI_ACCUM) return launch_nt3_t<EPI_ACCUM, float, GRP, TN>(g, s);
  return launch_nt3_t<EPI_RESID, float, GRP, TN>(g, s);
}

int launch_gemm_grouped(const Gemm& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.grp_max_rt <= 0) return 0;
  if (!g.grp || g.ngroups <= 0 || g.batch != 1 || g.ab != DT_BF16 || (g.bt >= 0 && g.bt != DT_BF16) || g.a_km ||
      g.b_kn || g.K <= 0 || g.K % N3_BK != 0 || g.lda % 8 || g.ldb % 8 || g.sB % 8 ||
      (((uintptr_t)g.A | (uintptr_t)g.B) % 16))
    return (int)hipErrorInvalidValue;
  if (g.epi != EPI_STORE && g.c != DT_F32) return (int)hipErrorInvalidValue;
  if (g.epi == EPI_RESID && !g.R) return (int)hipErrorInvalidValue;
  return launch_nt3<true>(g, s);
}

// Exclusive prefix sums of the group sizes and of their 256-row tile counts (one block).
__global__ __launch_bounds__(512) void gemm_group_table_k(const int32_t* __restrict__ counts, int G,
                                                          int32_t* __restrict__ tab) {
  __shared__ int32_t sr[512], st[512];
  const int t = threadIdx.x;
  const int c = t < G ? counts[t] : 0;
  sr[t] = c;
  st[t] = (c + GEMM_GROUP_BM - 1) / GEMM_GROUP_BM;
  __syncthreads();
  for (int o = 1; o < 512; o <<= 1) {
    const int a = t >= o ? sr[t - o] : 0, b = t >= o ? st[t - o] : 0;
    __syncthreads();
    sr[t] += a;
    st[t] += b;
    __syncthreads();
  }
  if (t < G) {
    tab[t + 1] = sr[t];
    tab[G + 2 + t] = st[t];
  }
  if (t == 0) {
    tab[0] = 0;
    tab[G + 1] = 0;
  }
}

int launch_gemm_group_table(const int32_t* counts, int G, int32_t* tab, hipStream_t s) {
  if (G <= 0 || G > 512) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_group_table_k, dim3(1), dim3(512), 0, s, counts, G, tab);
  return (int)hipGetLastError();
}

constexpr int NT2_WAVES = 8;
template <int EPI, typename TO>
static int launch_nt2_t(const Gemm& g, hipStream_t s) {
  const int tiles = ((g.M + N2_BM - 1) / N2_BM) * ((g.N + N2_BN - 1) / N2_BN);
  hipLaunchKernelGGL((gemm_nt2<EPI, TO, NT2_WAVES>), dim3(tiles, g.batch), dim3(64 * NT2_WAVES), 0, s, g);
  return (int)hipGetLastError();
}

static int launch_nt2(const Gemm& g, hipStream_t s) {
  if (g.epi == EPI_STORE) return g.c == DT_BF16 ? launch_nt2_t<EPI_STORE, bf16>(g, s) : launch_nt2_t<EPI_STORE, float>(g, s);
  if (g.epi == EPI_ACCUM) return launch_nt2_t<EPI_ACCUM, float>(g, s);
  return launch_nt2_t<EPI_RESID, float>(g, s);
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

int launch_gemm_swiglu(const Gemm& g0, void* a, int64_t ld_a, hipStream_t s) {
  if (g0.M <= 0 || g0.N <= 0) return 0;
  if (g0.N % 2 || g0.epi != EPI_STORE || g0.batch != 1 || !a) return (int)hipErrorInvalidValue;
  Gemm g = g0;
  g.C2 = a;
  g.ldc2 = ld_a;
  const int F = g.N / 2;
  const DType tb = g.bt < 0 ? g.ab : (DType)g.bt;
  const bool fused = g.ab == DT_BF16 && tb == DT_BF16 && g.c == DT_BF16 && !g.a_km && !g.b_kn && g.K > 0 &&
                     g.K % N3_BK == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0 &&
                     (((uintptr_t)g.A | (uintptr_t)g.B) % 16 == 0) && F % 32 == 0 && g.ldc % 4 == 0 &&
                     ld_a % 4 == 0 && (((uintptr_t)g.C | (uintptr_t)a) % 8 == 0);
  if (fused) {
    const int tiles = n3_persistent_grid(((g.M + N2_BM - 1) / N2_BM) * ((g.N + N2_BN - 1) / N2_BN));
    if (n3_buffer_ok(g))
      hipLaunchKernelGGL((gemm_nt3<EPI_STORE, bf16, NT3_WAVES, true, false, PM_SWIGLU>), dim3(tiles), dim3(64 * NT3_WAVES), 0,
                         s, g);
    else
      hipLaunchKernelGGL((gemm_nt3<EPI_STORE, bf16, NT3_WAVES, false, false, PM_SWIGLU>), dim3(tiles), dim3(64 * NT3_WAVES),
                         0, s, g);
    return (int)hipGetLastError();
  }
  // otherwise the plain product and the element-wise kernel, which needs the packed layouts
  if (g.ldc != g.N || ld_a != F) return (int)hipErrorInvalidValue;
  const int e = launch_gemm(g0, s);
  if (e) return e;
  return launch_swiglu_fwd(g.C, a, g.c, g.M, F, s);
}

bool gemm_rope_supported(const Gemm& g, int nrot, const float* cos_t, const float* sin_t) {
  const DType tb = g.bt < 0 ? g.ab : (DType)g.bt;
  return g.ab == DT_BF16 && tb == DT_BF16 && g.c == DT_BF16 && g.epi == EPI_STORE && g.batch == 1 && !g.a_km &&
         !g.b_kn && g.K > 0 && g.K % N3_BK == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0 &&
         (((uintptr_t)g.A | (uintptr_t)g.B) % 16 == 0) && g.N % 128 == 0 && nrot >= 0 && nrot % 128 == 0 &&
         nrot <= g.N && g.ldc % 4 == 0 && (uintptr_t)g.C % 8 == 0 && cos_t && sin_t &&
         (((uintptr_t)cos_t | (uintptr_t)sin_t) % 16 == 0);
}

int launch_gemm_rope(const Gemm& g0, int nrot, int S, const float* cos_t, const float* sin_t, hipStream_t s) {
  if (g0.M <= 0 || g0.N <= 0) return 0;
  if (S <= 0 || !gemm_rope_supported(g0, nrot, cos_t, sin_t)) return (int)hipErrorInvalidValue;
  Gemm g = g0;
  g.rope_cos = cos_t;
  g.rope_sin = sin_t;
  g.rope_S = S;
  g.rope_nr = nrot;
  const int tiles = n3_persistent_grid(((g.M + N2_BM - 1) / N2_BM) * ((g.N + N2_BN - 1) / N2_BN));
  if (n3_buffer_ok(g))
    hipLaunchKernelGGL((gemm_nt3<EPI_STORE, bf16, NT3_WAVES, true, false, PM_ROPE>), dim3(tiles), dim3(64 * NT3_WAVES), 0,
                       s, g);
  else
    hipLaunchKernelGGL((gemm_nt3<EPI_STORE, bf16, NT3_WAVES, false, false, PM_ROPE>), dim3(tiles), dim3(64 * NT3_WAVES),
                       0, s, g);
  return (int)hipGetLastError();
}

int launch_gemm(const Gemm& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return 0;
  if (g.K <= 0) return (int)hipErrorInvalidValue;
  if (g.epi != EPI_STORE && g.c != DT_F32) return (int)hipErrorInvalidValue;
  if (g.epi == EPI_RESID && !g.R) return (int)hipErrorInvalidValue;
  const DType tb = g.bt < 0 ? g.ab : (DType)g.bt;
  dim3 grid((g.N + 63) / 64, (g.M + 63) / 64, g.batch);
  if (g.ab == DT_BF16 && tb == DT_BF16) {
    // MFMA path: 16-byte rows need K, leading dimensions and base pointers 8-element aligned
    const bool aligned = (g.K % 8 == 0) && (g.lda % 8 == 0) && (g.ldb % 8 == 0) &&
                         (((uintptr_t)g.A | (uintptr_t)g.B) % 16 == 0) &&
                         (g.batch == 1 || (g.sA % 8 == 0 && g.sB % 8 == 0));
    if (aligned) {
      if (!g.a_km && !g.b_kn && g.K % N3_BK == 0) return launch_nt3<false>(g, s);
      if (!g.a_km && !g.b_kn && g.K % N2_BK == 0) return launch_nt2(g, s);
      if (!g.a_km && !g.b_kn) return launch_mfma_l<false, false>(g, s);
      if (!g.a_km && g.b_kn) return launch_mfma_l<false, true>(g, s);
      if (g.a_km && g.b_kn && g.K % N3_BK == 0 && g.M % 8 == 0 && g.N % 8 == 0 && t3_buffer_ok(g))
        return launch_nt3<false, true>(g, s);
      if (g.a_km && g.b_kn) return launch_mfma_l<true, true>(g, s);
      return launch_mfma_l<true, false>(g, s);
    }
    if (!g.any_align) return (int)hipErrorInvalidValue;
    if (g.c == DT_BF16) hipLaunchKernelGGL((gemm_tiled<bf16, bf16, bf16>), grid, dim3(256), 0, s, g);
    else hipLaunchKernelGGL((gemm_tiled<bf16, bf16, float>), grid, dim3(256), 0, s, g);
    return (int)hipGetLastError();
  }
  // fp32 and mixed operands (fp32 adapter factors against bf16 activations)
#define GT(TA, TB)                                                                           \
  do {                                                                                       \
    if (g.c == DT_BF16) hipLaunchKernelGGL((gemm_tiled<TA, TB, bf16>), grid, dim3(256), 0, s, g); \
    else hipLaunchKernelGGL((gemm_tiled<TA, TB, float>), grid, dim3(256), 0, s, g);          \
  } while (0)
  if (g.ab == DT_F32 && tb == DT_F32) GT(float, float);
  else if (g.ab == DT_BF16) GT(bf16, float);
  else GT(float, bf16);
#undef GT
  return (int)hipGetLastError();
}

}  // namespace hol
