// Causal grouped-query attention on CDNA4 matrix cores (bf16 operands, fp32 accumulation and
// softmax), head width 64 or 128: the Attention block of the weight-free layer template
// (MegaTrain summary page, 核心方法). Forward keeps the log-sum-exp per query; backward recomputes
// P from it. Deterministic: the dK/dV kernel owns a key tile and loops over the queries and every q
// head of its kv group; the dQ kernel owns a query tile and loops over the keys; no atomics.
//
// MFMA v_mfma_f32_32x32x16_bf16 lane layout (lane l, h = l / 32):
//   A[i][k]: i = l % 32, k = 8h .. 8h+7           B[k][j]: j = l % 32, k = 8h .. 8h+7
//   D[i][j]: j = l % 32, i = 8 (r / 4) + 4h + r % 4 for accumulator element r = 0..15
// A score product computed so that the contraction index of the NEXT product lies along i gives
// every lane exactly the B fragment of that next product for k-step ks (16 rows):
//   rows 16 ks + 4h + {0,1,2,3}  and  16 ks + 8 + 4h + {0,1,2,3}  = accumulator elements
//   4 (2 ks') + {0..3} and 4 (2 ks' + 1) + {0..3} of 32-row block ks / 2 (ks' = ks % 2).
// The matching A fragment is read from a transposed LDS tile with two 8-byte reads at those rows.
#include "device_common.h"
#include "kernels.h"

namespace hol {

namespace fa {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void zero(f32x16& x) {
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = 0.f;
}

// Online softmax of the forward: the reference m that the probabilities 2^(s - m) are taken
// against is raised only when a tile's maximum exceeds it by more than RESCALE_SLACK (log2 units).
// The probabilities then stay below 2^8, far inside fp32 and without effect on the relative
// precision of their bf16 rounding, the final o / l and lse = m + log l are unchanged up to
// rounding, and the rescale of the output accumulators (64 products a lane) runs in a few tiles
// of a row instead of in most.
constexpr float RESCALE_SLACK = 8.f;

// B fragment of k-step ks' (0 or 1) inside a 32-row accumulator block
__device__ __forceinline__ bf16x8 acc_frag(const f32x16& acc, int ksp) {
  bf16x8 b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    b[i] = (bf16)acc[8 * ksp + i];
    b[4 + i] = (bf16)acc[8 * ksp + 4 + i];
  }
  return b;
}

// A fragment from a transposed LDS tile Xt[row][col] (pitch P): row = r, cols 16 ks + 4h + 0..3 and +8
__device__ __forceinline__ bf16x8 tfrag(const bf16* Xt, int P, int row, int ks, int h) {
  const bf16* p = Xt + row * P + 16 * ks + 4 * h;
  const u32x2 lo = *(const u32x2*)p;
  const u32x2 hi = *(const u32x2*)(p + 8);
  u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ void transpose8x8(const u32x4 in[8], u32x4 out[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int w = c >> 1;
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int p = 0; p < 4; ++p) out[c][p] = __builtin_amdgcn_perm(in[2 * p + 1][w], in[2 * p][w], sel);
  }
}

// rows [row0, row0 + R) of a token-major matrix (row stride ld, D columns starting at col0) into
// LDS row-major with pitch P; rows >= nvalid are clamped to the last valid row. NT threads.
template <int R, int D, int NT = 256>
__device__ __forceinline__ void load_rows(bf16* dst, int P, const bf16* src, int64_t ld, int64_t row0, int nvalid) {
  constexpr int CH = R * D / 8;
  for (int c = threadIdx.x; c < CH; c += NT) {
    const int r = c / (D / 8), k = (c % (D / 8)) * 8;
    const int rr = r < nvalid ? r : nvalid - 1;
    *(u32x4*)(dst + r * P + k) = *(const u32x4*)(src + (row0 + rr) * ld + k);
  }
}

// the same rows transposed: dst[d][r] with pitch P (P a multiple of 4 elements)
template <int R, int D>
__device__ __forceinline__ void load_rows_t(bf16* dst, int P, const bf16* src, int64_t ld, int64_t row0, int nvalid) {
  constexpr int NB = (R / 8) * (D / 8);
  for (int b = threadIdx.x; b < NB; b += 256) {
    const int rb = b % (R / 8), db = b / (R / 8);
    u32x4 in[8], out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = rb * 8 + i;
      const int rr = r < nvalid ? r : nvalid - 1;
      in[i] = *(const u32x4*)(src + (row0 + rr) * ld + db * 8);
    }
    transpose8x8(in, out);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      bf16* q = dst + (db * 8 + c) * P + rb * 8;
      *(u32x2*)q = u32x2{out[c][0], out[c][1]};
      *(u32x2*)(q + 4) = u32x2{out[c][2], out[c][3]};
    }
  }
}

// 4 consecutive fp32 values -> 4 bf16 (8-byte store)
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
  bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
  *(bf16x4*)p = v;
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }  // v_exp_f32; ex2(-inf) = 0

// The RoPE backward of one row of a head-width-128 gradient held as v[db][4 g + e] = column
// 32 db + 8 g + 4 hh + e: pairs (j, j + 64) for j < 64 (blocks db and db + 2, same lane) are
// rotated by minus the angle of position p (tables [S][64]), in fp32 before the single rounding.
__device__ __forceinline__ void rope_back_row(float (&v)[4][16], const float* cs, const float* sn, int p, int hh) {
#pragma clang fp contract(off)
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int j = db * 32 + 8 * g + 4 * hh;
      const float4 c4 = *(const float4*)(cs + (int64_t)p * 64 + j);
      const float4 s4 = *(const float4*)(sn + (int64_t)p * 64 + j);
      const float c[4] = {c4.x, c4.y, c4.z, c4.w}, sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = v[db][4 * g + e], b = v[db + 2][4 * g + e], s_ = -sv[e];
        v[db][4 * g + e] = a * c[e] - b * s_;
        v[db + 2][4 * g + e] = b * c[e] + a * s_;
      }
    }
}

// Reductions over the two halves of a wave (lanes l and l ^ 32), by v_permlane32_swap: swapping
// the upper half of one copy of x with the lower half of another leaves x[l % 32] in the first and
// x[32 + l % 32] in the second, in both halves, so both halves get the same result bit for bit.
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Block order: `per` units for each (sequence, kv head) pair, unit 0 of a pair the longest.
// Workgroups go to the 8 XCDs in turn (workgroup i to XCD i % 8), so that the blocks an XCD runs
// at once stream the tiles of one pair through its L2:
//   pairs a multiple of 8: each XCD takes a contiguous range of whole pairs;
//   pairs dividing 8 (r = 8 / pairs XCDs a pair): XCD x serves pair x / r, units x % r + r j;
//   otherwise: plain order.
// Returns false for the surplus blocks of the second case (the grid is rounded up to 8 r units).
__host__ __device__ __forceinline__ unsigned pair_grid(int per, int npairs) {
  if (npairs % 8 != 0 && 8 % npairs == 0) {
    const int r = 8 / npairs;
    return 8u * (unsigned)((per + r - 1) / r);
  }
  return (unsigned)(per * npairs);
}
__device__ __forceinline__ bool pair_unit(int per, int npairs, int& pair, int& unit) {
  const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
  if ((npairs & 7) == 0) {
    const int u = x * ((per * npairs) >> 3) + j;
    pair = u / per;
    unit = u - pair * per;
    return true;
  }
  if (8 % npairs == 0) {
    const int r = 8 / npairs;
    pair = x / r;
    unit = x % r + r * j;
    return unit < per;
  }
  pair = blockIdx.x / per;
  unit = blockIdx.x - pair * per;
  return true;
}

// Register-staged tiles: a thread's share of the next tile is fetched into registers while the
// current tile is computed on, then written to LDS after the next barrier.
// Natural layout, 16-byte chunks: chunk c = tid + NT i is row c / (D/8), columns (c % (D/8)) * 8
// (NT threads in the block).
template <int R, int D, int NT = 256>
struct NatTile {
  static constexpr int N = R * D / 8 / NT;
  static_assert(R * D / 8 % NT == 0, "tile must split into whole chunks per thread");
  u32x4 v[N];
  __device__ __forceinline__ void load(const bf16* src, int64_t ld, int64_t row0, int nvalid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = threadIdx.x + NT * i;
      const int r = c / (D / 8), k = (c % (D / 8)) * 8;
      const int rr = r < nvalid ? r : nvalid - 1;
      v[i] = *(const u32x4*)(src + (row0 + rr) * ld + k);
    }
  }
  __device__ __forceinline__ void store(bf16* dst, int P) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = threadIdx.x + NT * i;
      *(u32x4*)(dst + (c / (D / 8)) * P + (c % (D / 8)) * 8) = v[i];
    }
  }
};

// Per-thread offsets of a NatTile's chunks from the tile's first row, for one row stride: a whole
// tile then loads with one address add per chunk; a ragged last tile takes NatTile::load, which
// clamps rows.
template <int R, int D, int NT = 256>
struct NatOff {
  int64_t off[NatTile<R, D, NT>::N];
  __device__ __forceinline__ void init(int64_t ld) {
#pragma unroll
    for (int i = 0; i < NatTile<R, D, NT>::N; ++i) {
      const int c = threadIdx.x + NT * i;
      off[i] = (int64_t)(c / (D / 8)) * ld + (c % (D / 8)) * 8;
    }
  }
  __device__ __forceinline__ void load(NatTile<R, D, NT>& t, const bf16* row0) const {
#pragma unroll
    for (int i = 0; i < NatTile<R, D, NT>::N; ++i) t.v[i] = *(const u32x4*)(row0 + off[i]);
  }
};

// Transposed layout dst[d][r]: 8 x 8 blocks b = t + NT j (t in [0, NT)), rows 8 (b % (R/8)) + 0..7,
// columns 8 (b / (R/8)) + 0..7; a thread with t outside [0, NT) holds nothing.
template <int R, int D, int NT>
struct TrTile {
  static constexpr int NB = (R / 8) * (D / 8);
  static constexpr int N = (NB + NT - 1) / NT;
  u32x4 v[N][8];
  __device__ __forceinline__ void load(int t, const bf16* src, int64_t ld, int64_t row0, int nvalid) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int b = t + NT * j;
      if (t < 0 || t >= NT || b >= NB) continue;
      const int rb = b % (R / 8), db = b / (R / 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = rb * 8 + i;
        const int rr = r < nvalid ? r : nvalid - 1;
        v[j][i] = *(const u32x4*)(src + (row0 + rr) * ld + db * 8);
      }
    }
  }
  __device__ __forceinline__ void store(int t, bf16* dst, int P) const {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int b = t + NT * j;
      if (t < 0 || t >= NT || b >= NB) continue;
      const int rb = b % (R / 8), db = b / (R / 8);
      u32x4 out[8];
      transpose8x8(v[j], out);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        bf16* q = dst + (db * 8 + c) * P + rb * 8;
        *(u32x2*)q = u32x2{out[c][0], out[c][1]};
        *(u32x2*)(q + 4) = u32x2{out[c][2], out[c][3]};
      }
    }
  }
};

// dst[d][r] (pitch TP) = src[r][d] (pitch SP) for an R x D tile already in LDS; 8 x 8 blocks with
// the column block varying fastest across lanes (conflict-free 16-byte reads of source rows).
template <int R, int D>
__device__ __forceinline__ void lds_transpose(const bf16* src, int SP, bf16* dst, int TP) {
  constexpr int NB = (R / 8) * (D / 8);
  for (int b = threadIdx.x; b < NB; b += 256) {
    const int db = b % (D / 8), rb = b / (D / 8);
    u32x4 in[8], out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) in[i] = *(const u32x4*)(src + (rb * 8 + i) * SP + db * 8);
    transpose8x8(in, out);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      bf16* q = dst + (db * 8 + c) * TP + rb * 8;
      *(u32x2*)q = u32x2{out[c][0], out[c][1]};
      *(u32x2*)(q + 4) = u32x2{out[c][2], out[c][3]};
    }
  }
}

}  // namespace fa

using namespace fa;

// ------------------------------------------------------------------------------------------
// forward: block = 4 waves x 32 queries; key tiles of 64
// ------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_mfma(Attn a) {
  constexpr int BQ = 128, BK = 64, KP = D + 8, VP = BK + 12;
  __shared__ bf16 Ks[BK * KP];
  __shared__ bf16 Vt[D * VP];
  const int S = a.S;
  const int nqt = (S + BQ - 1) / BQ;
  const int group = a.nq / a.nkv;
  int pair, unit;
  if (!pair_unit(group * nqt, a.nkv * a.n_seq, pair, unit)) return;
  const int qt = nqt - 1 - unit / group;  // longest (latest) query tiles first, the group's heads together
  const int kvh = pair % a.nkv, seq = pair / a.nkv;
  const int h = kvh * group + unit % group;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, hh = lane >> 5, lq = lane & 31;
  const int q0 = qt * BQ;
  const int qi = q0 + 32 * w + lq;  // this lane's query (column of every accumulator)
  const int64_t base = (int64_t)seq * S;
  const bf16* Q = (const bf16*)a.q + (int64_t)h * D;
  const bf16* K = (const bf16*)a.k + (int64_t)kvh * D;
  const bf16* V = (const bf16*)a.v + (int64_t)kvh * D;

  bf16x8 qf[D / 16];
  {
    const bf16* qp = Q + (base + min(qi, S - 1)) * a.ldq;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = *(const bf16x8*)(qp + 16 * kk + 8 * hh);
  }
  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) zero(o[i]);
  const float sl2 = LOG2E / sqrtf((float)D);
  float m = -INFINITY, l = 0.f;
  const int qmax = min(q0 + BQ, S) - 1;
  const int nkt = qmax / BK + 1;
  const int wave_qmax = min(q0 + 32 * w + 31, S - 1);

  NatTile<BK, D> kreg;
  TrTile<BK, D, 256> vreg;
  kreg.load(K, a.ldk, base, min(BK, S));
  vreg.load(threadIdx.x, V, a.ldv, base, min(BK, S));
  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * BK;
    __syncthreads();
    kreg.store(Ks, KP);
    vreg.store(threadIdx.x, Vt, VP);
    __syncthreads();
    if (kt + 1 < nkt) {  // next tile in flight while this one is computed on
      kreg.load(K, a.ldk, base + k0 + BK, min(BK, S - k0 - BK));
      vreg.load(threadIdx.x, V, a.ldv, base + k0 + BK, min(BK, S - k0 - BK));
    }
    if (k0 > wave_qmax) continue;  // every key of this tile is in this wave's future
    f32x16 s[2];
    zero(s[0]);
    zero(s[1]);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = *(const bf16x8*)(Ks + (kb * 32 + lq) * KP + 16 * kk + 8 * hh);
        s[kb] = mfma(kf, qf[kk], s[kb]);
      }
    }
    // s[kb][r] = score(key k0 + 32 kb + 8 (r/4) + 4 hh + r%4, query qi)
    const bool diag = (k0 + BK - 1 > q0 + 32 * w) || (k0 + BK > S);
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = s[kb][r] * sl2;
        if (diag) {
          const int kj = k0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (kj > qi || kj >= S) v = -INFINITY;
        }
        s[kb][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (mx > m + RESCALE_SLACK) {  // the reference moves (m = -inf before the first tile: corr = 0)
      const float corr = ex2(m - mx);
      l *= corr;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= corr;
      m = mx;
    }
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = ex2(s[kb][r] - m);
        s[kb][r] = p;
        ls += p;
      }
    ls += __shfl_xor(ls, 32, 64);
    l += ls;
    // O^T[d][q] += V^T[d][key] P^T[key][q]
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const bf16x8 pb = acc_frag(s[ks >> 1], ks & 1);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] = mfma(tfrag(Vt, VP, db * 32 + lq, ks, hh), pb, o[db]);
    }
  }
  if (qi < S) {
    const float inv = 1.f / l;
    bf16* op = (bf16*)a.o + (base + qi) * a.ldo + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4(op + db * 32 + 8 * g + 4 * hh, o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
               o[db][4 * g + 3] * inv);
    if (hh == 0) a.lse[((int64_t)seq * a.nq + h) * S + qi] = (m + __log2f(l)) * LN2;
  }
}

// ------------------------------------------------------------------------------------------
// backward, dK/dV: block = 4 waves x 32 keys (128 keys) of one kv head; loops over the q heads
// of the group and over query tiles of 64 from the diagonal to the end.
// ------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 1) void attn_dkdv_mfma(Attn a) {
  constexpr int BKV = 128, BQ = 64, KP = D + 8, TP = BQ + 12;
  __shared__ bf16 Qs[BQ * KP];
  __shared__ bf16 Gs[BQ * KP];  // dO
  __shared__ bf16 Qt[D * TP];
  __shared__ bf16 Gt[D * TP];
  __shared__ float lse2[BQ], dlt[BQ];
  __shared__ bf16 Kb[BKV * KP];  // the block's keys and values (fragments read per use, which
  __shared__ bf16 Vb[BKV * KP];  // leaves the registers to the accumulators and the prefetch)
  const int S = a.S;
  const int nkt = (S + BKV - 1) / BKV;
  int pair, kt;  // early keys see the most queries: key tile 0 of a pair first
  if (!pair_unit(nkt, a.nkv * a.n_seq, pair, kt)) return;
  const int kvh = pair % a.nkv, seq = pair / a.nkv;
  const int group = a.nq / a.nkv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, hh = lane >> 5, lq = lane & 31;
  const int k0 = kt * BKV;
  const int kj = k0 + 32 * w + lq;  // this lane's key (column of the S / dP accumulators)
  const int64_t base = (int64_t)seq * S;
  const float sl2 = LOG2E / sqrtf((float)D);
  const float scale = 1.f / sqrtf((float)D);

  // (visible to every wave after the first iteration's barrier)
  load_rows<BKV, D>(Kb, KP, (const bf16*)a.k + (int64_t)kvh * D, a.ldk, base + k0, min(BKV, S - k0));
  load_rows<BKV, D>(Vb, KP, (const bf16*)a.v + (int64_t)kvh * D, a.ldv, base + k0, min(BKV, S - k0));
  const bf16* kfp = Kb + (32 * w + lq) * KP + 8 * hh;
  const bf16* vfp = Vb + (32 * w + lq) * KP + 8 * hh;
  f32x16 dv[D / 32], dk[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    zero(dv[i]);
    zero(dk[i]);
  }
  const int wave_kmin = k0 + 32 * w;
  const int nqt = (S + BQ - 1) / BQ;
  const int qt0 = k0 / BQ, nper = nqt - qt0, nit = group * nper;
  // iteration it: query tile nqt - 1 - it / group (from the last down to the diagonal), q head
  // kvh * group + it % group; every key tile of a pair walks the query tiles in the same order
  NatTile<BQ, D> qreg, greg;
  float lse_r = 0.f, dl_r = 0.f;
  auto fetch = [&](int it) {
    const int h = kvh * group + it % group, q0 = (nqt - 1 - it / group) * BQ, nq = min(BQ, S - q0);
    const bf16* Q = (const bf16*)a.q + (int64_t)h * D;
    const bf16* G = (const bf16*)a.dO + (int64_t)h * D;
    qreg.load(Q, a.ldq, base + q0, nq);
    greg.load(G, a.lddo, base + q0, nq);
    if (threadIdx.x < BQ) {
      const int qq = q0 + threadIdx.x;
      const int64_t hrow = ((int64_t)seq * a.nq + h) * S;
      lse_r = qq < S ? a.lse[hrow + qq] * LOG2E : 0.f;
      dl_r = qq < S ? a.delta[hrow + qq] : 0.f;
    }
  };
  fetch(0);
  for (int it = 0; it < nit; ++it) {
    const int q0 = (nqt - 1 - it / group) * BQ;
    {
      __syncthreads();
      qreg.store(Qs, KP);
      greg.store(Gs, KP);
      if (threadIdx.x < BQ) {
        lse2[threadIdx.x] = lse_r;
        dlt[threadIdx.x] = dl_r;
      }
      __syncthreads();
      lds_transpose<BQ, D>(Qs, KP, Qt, TP);
      lds_transpose<BQ, D>(Gs, KP, Gt, TP);
      if (it + 1 < nit) fetch(it + 1);  // next tile in flight while this one is computed on
      __syncthreads();
      if (q0 + BQ - 1 < wave_kmin) continue;  // all queries before this wave's keys
      // two 32-query halves in turn: S[q][key] and dP[q][key], then their dV / dK products
      // (element r of a half qb: query q0 + 32 qb + 8 (r/4) + 4 hh + r%4, key kj)
      const bool full = q0 >= wave_kmin + 31 && q0 + BQ <= S && kj < S;  // no masking in this tile
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x16 s, dp;
        zero(s);
        zero(dp);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          s = mfma(*(const bf16x8*)(Qs + (qb * 32 + lq) * KP + 16 * kk + 8 * hh), *(const bf16x8*)(kfp + 16 * kk), s);
          dp = mfma(*(const bf16x8*)(Gs + (qb * 32 + lq) * KP + 16 * kk + 8 * hh), *(const bf16x8*)(vfp + 16 * kk), dp);
        }
        if (full) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qloc = 32 * qb + 8 * (r >> 2) + 4 * hh + (r & 3);
            const float p = ex2(fmaf(s[r], sl2, -lse2[qloc]));
            s[r] = p;
            dp[r] = p * (dp[r] - dlt[qloc]);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qloc = 32 * qb + 8 * (r >> 2) + 4 * hh + (r & 3);
            const int qq = q0 + qloc;
            const bool ok = qq < S && kj <= qq && kj < S;
            const float p = ok ? ex2(fmaf(s[r], sl2, -lse2[qloc])) : 0.f;
            s[r] = p;
            dp[r] = p * (dp[r] - dlt[qloc]);
          }
        }
        // dV^T[d][key] += dO^T[d][q] P[q][key];  dK^T[d][key] += Q^T[d][q] dS[q][key]
#pragma unroll
        for (int ksp = 0; ksp < 2; ++ksp) {
          const int ks = 2 * qb + ksp;
          const bf16x8 pb = acc_frag(s, ksp);
          const bf16x8 sb = acc_frag(dp, ksp);
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            dv[db] = mfma(tfrag(Gt, TP, db * 32 + lq, ks, hh), pb, dv[db]);
            dk[db] = mfma(tfrag(Qt, TP, db * 32 + lq, ks, hh), sb, dk[db]);
          }
        }
      }
    }
  }
  if (kj < S) {
    bf16* dkp = (bf16*)a.dk + (base + kj) * a.lddk + (int64_t)kvh * D;
    bf16* dvp = (bf16*)a.dv + (base + kj) * a.lddv + (int64_t)kvh * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = db * 32 + 8 * g + 4 * hh;
        store4(dkp + dd, dk[db][4 * g] * scale, dk[db][4 * g + 1] * scale, dk[db][4 * g + 2] * scale,
               dk[db][4 * g + 3] * scale);
        store4(dvp + dd, dv[db][4 * g], dv[db][4 * g + 1], dv[db][4 * g + 2], dv[db][4 * g + 3]);
      }
  }
}

// ------------------------------------------------------------------------------------------
// dK/dV for head width 128 without transposed copies: the query-side tiles (Q, dO) stay in their
// natural [q][d] layout, double-buffered in LDS (one block barrier per iteration), and the dV / dK
// products read them transposed with ds_read_b64_tr_b16: within each 16-lane group, lane
// 16 g + 4 a + b receives element b of the 8-byte pieces addressed by lanes 16 g + a + 4 j
// (j = 0..3). Lane 16 g + a + 4 j therefore addresses row (query) q0 + 4 (g / 2) + j, columns
// (d) d0 + 16 (g mod 2) + 4 a .. + 3, and a second read 8 rows further completes the fragment in
// the query order of acc_frag. Tile rows are 256 B; 16-byte chunk c of row r sits at c ^ sw(r),
// sw(r) = 4 (r mod 4) + (r / 4) mod 4, which keeps both the score products' row reads (16 rows at
// one chunk) and the transposed reads (4 rows over 4 chunks) on distinct banks.
// ------------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* fa_lptr;
typedef __attribute__((address_space(1))) const void* fa_gptr;
__device__ __forceinline__ int qsw(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }
__device__ __forceinline__ int qoff(int r, int c) { return r * 128 + (((c >> 3) ^ qsw(r)) << 3) + (c & 7); }

typedef short trv4 __attribute__((ext_vector_type(4)));
typedef short trv8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ bf16x8 tr_pair(const bf16* lo, const bf16* hi) {
  const trv4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) trv4*)lo);
  const trv4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) trv4*)hi);
  const trv8 v = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// 8 waves, two per SIMD: waves w and w + 4 own the same 32 keys and take the two 32-query halves
// of every query tile; the second wave's dV / dK partial sums go through LDS to the first at the
// end (one fixed order, so the result is deterministic).
__global__ __launch_bounds__(512, 1) void attn_dkdv_tr128(Attn a) {
  constexpr int D = 128, BKV = 128, BQ = 64, KP = D + 8, QT = BQ * D, NT = 512;
  __shared__ __attribute__((aligned(16))) bf16 Qs[2 * QT];
  __shared__ __attribute__((aligned(16))) bf16 Gs[2 * QT];  // dO
  __shared__ float lse2[2][BQ], dlt[2][BQ];
  __shared__ __attribute__((aligned(16))) bf16 Kb[BKV * KP];
  __shared__ __attribute__((aligned(16))) bf16 Vb[BKV * KP];
  const int S = a.S;
  const int nkt = (S + BKV - 1) / BKV;
  int pair, kt;  // early keys see the most queries: key tile 0 of a pair first
  if (!pair_unit(nkt, a.nkv * a.n_seq, pair, kt)) return;
  const int kvh = pair % a.nkv, seq = pair / a.nkv;
  const int group = a.nq / a.nkv;
  const int lane = threadIdx.x & 63, hh = lane >> 5, lq = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: tile tests are scalar branches
  const int kw = w & 3, qb = w >> 2;  // key group of 32, query half of each tile
  const int k0 = kt * BKV;
  const int kj = k0 + 32 * kw + lq;  // this lane's key (column of the S / dP accumulators)
  const int64_t base = (int64_t)seq * S;
  const float sl2 = LOG2E / sqrtf((float)D);
  const float scale = 1.f / sqrtf((float)D);

  load_rows<BKV, D, NT>(Kb, KP, (const bf16*)a.k + (int64_t)kvh * D, a.ldk, base + k0, min(BKV, S - k0));
  load_rows<BKV, D, NT>(Vb, KP, (const bf16*)a.v + (int64_t)kvh * D, a.ldv, base + k0, min(BKV, S - k0));
  const bf16* kfp = Kb + (32 * kw + lq) * KP + 8 * hh;
  const bf16* vfp = Vb + (32 * kw + lq) * KP + 8 * hh;
  // transposed-read offsets: [half][d block] for k-step 0 (add 16 rows per k-step)
  int toff[2][D / 32];
  {
    const int g = lane >> 4, aa = lane & 3, j = (lane >> 2) & 3;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) toff[hf][db] = qoff(8 * hf + 4 * (g >> 1) + j, db * 32 + 16 * (g & 1) + 4 * aa);
  }
  f32x16 dv[D / 32], dk[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    zero(dv[i]);
    zero(dk[i]);
  }
  const int wave_kmin = k0 + 32 * kw;
  const int nqt = (S + BQ - 1) / BQ;
  const int qt0 = k0 / BQ, nper = nqt - qt0, nit = group * nper;
  // iteration it: query tile nqt - 1 - it / group (from the last down to the diagonal), q head
  // kvh * group + it % group; every key tile of a pair walks the query tiles in the same order
  NatTile<BQ, D, NT> qreg, greg;
  NatOff<BQ, D, NT> qoffs, goffs;
  qoffs.init(a.ldq);
  goffs.init(a.lddo);
  float lse_r = 0.f, dl_r = 0.f;
  auto fetch = [&](int it) {
    const int h = kvh * group + it % group, q0 = (nqt - 1 - it / group) * BQ, nq = min(BQ, S - q0);
    const bf16* Q = (const bf16*)a.q + (int64_t)h * D;
    const bf16* G = (const bf16*)a.dO + (int64_t)h * D;
    if (nq == BQ) {
      qoffs.load(qreg, Q + (base + q0) * a.ldq);
      goffs.load(greg, G + (base + q0) * a.lddo);
    } else {
      qreg.load(Q, a.ldq, base + q0, nq);
      greg.load(G, a.lddo, base + q0, nq);
    }
    if (threadIdx.x < BQ) {
      const int qq = q0 + threadIdx.x;
      const int64_t hrow = ((int64_t)seq * a.nq + h) * S;
      lse_r = qq < S ? a.lse[hrow + qq] * LOG2E : 0.f;
      dl_r = qq < S ? a.delta[hrow + qq] : 0.f;
    }
  };
  // a thread's share of the fetched tile into buffer b (chunk c = tid + NT i: row c / 16,
  // logical chunk c % 16)
  auto put = [&](int b) {
#pragma unroll
    for (int i = 0; i < NatTile<BQ, D, NT>::N; ++i) {
      const int c = threadIdx.x + NT * i, r = c >> 4, ch = c & 15;
      const int o = b * QT + r * 128 + ((ch ^ qsw(r)) << 3);
      *(u32x4*)(Qs + o) = qreg.v[i];
      *(u32x4*)(Gs + o) = greg.v[i];
    }
    if (threadIdx.x < BQ) {
      lse2[b][threadIdx.x] = lse_r;
      dlt[b][threadIdx.x] = dl_r;
    }
  };
  fetch(0);
  put(0);
  if (nit > 1) fetch(1);
  __syncthreads();
  for (int it = 0; it < nit; ++it) {
    const int cur = it & 1;
    const int q0 = (nqt - 1 - it / group) * BQ, qh0 = q0 + 32 * qb;  // this wave's first query
    const bf16* Qc = Qs + cur * QT;
    const bf16* Gc = Gs + cur * QT;
    if (qh0 + 31 >= wave_kmin) {  // else every query of the half is before this wave's keys
      // S[q][key] and dP[q][key] for the half, then its dV / dK products (element r: query
      // qh0 + 8 (r/4) + 4 hh + r%4, key kj)
      const bool full = qh0 >= wave_kmin + 31 && qh0 + 32 <= S && wave_kmin + 32 <= S;  // no masking here (wave-uniform)
      f32x16 s, dp;
      zero(s);
      zero(dp);
      const int qr = qb * 32 + lq;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const int o = qoff(qr, 16 * kk + 8 * hh);
        s = mfma(*(const bf16x8*)(Qc + o), *(const bf16x8*)(kfp + 16 * kk), s);
        dp = mfma(*(const bf16x8*)(Gc + o), *(const bf16x8*)(vfp + 16 * kk), dp);
      }
      if (full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qloc = 32 * qb + 8 * (r >> 2) + 4 * hh + (r & 3);
          const float p = ex2(fmaf(s[r], sl2, -lse2[cur][qloc]));
          s[r] = p;
          dp[r] = p * (dp[r] - dlt[cur][qloc]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qloc = 32 * qb + 8 * (r >> 2) + 4 * hh + (r & 3);
          const int qq = q0 + qloc;
          const bool ok = qq < S && kj <= qq && kj < S;
          const float p = ok ? ex2(fmaf(s[r], sl2, -lse2[cur][qloc])) : 0.f;
          s[r] = p;
          dp[r] = p * (dp[r] - dlt[cur][qloc]);
        }
      }
      // dV^T[d][key] += dO^T[d][q] P[q][key];  dK^T[d][key] += Q^T[d][q] dS[q][key]
#pragma unroll
      for (int ksp = 0; ksp < 2; ++ksp) {
        const int ks = 2 * qb + ksp;
        const bf16x8 pb = acc_frag(s, ksp);
        const bf16x8 sb = acc_frag(dp, ksp);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          dv[db] = mfma(tr_pair(Gc + ks * 16 * 128 + toff[0][db], Gc + ks * 16 * 128 + toff[1][db]), pb, dv[db]);
          dk[db] = mfma(tr_pair(Qc + ks * 16 * 128 + toff[0][db], Qc + ks * 16 * 128 + toff[1][db]), sb, dk[db]);
        }
      }
    }
    if (it + 1 < nit) {
      put(cur ^ 1);  // tile it + 1 (its loads were issued an iteration ago); every wave finished
                     // reading that buffer before the previous barrier
      if (it + 2 < nit) fetch(it + 2);
    }
    __syncthreads();
  }
  // the second-half waves hand their sums to the first-half waves: float4 j4 of accumulator
  // half hf goes to ((kw * 8 + j4) * 64 + lane) of a 32 KB region (the tile buffers are free
  // after the last barrier): dv[0..1] -> Qs, dv[2..3] -> Gs, dk[0..1] -> Kb, dk[2..3] -> Vb
  f32x4* red[4] = {(f32x4*)Qs, (f32x4*)Gs, (f32x4*)Kb, (f32x4*)Vb};
  if (qb == 1) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j4 = (db & 1) * 4 + g;
        red[db >> 1][(kw * 8 + j4) * 64 + lane] = f32x4{dv[db][4 * g], dv[db][4 * g + 1], dv[db][4 * g + 2], dv[db][4 * g + 3]};
        red[2 + (db >> 1)][(kw * 8 + j4) * 64 + lane] =
            f32x4{dk[db][4 * g], dk[db][4 * g + 1], dk[db][4 * g + 2], dk[db][4 * g + 3]};
      }
  }
  __syncthreads();
  if (qb == 0 && kj < S) {
    bf16* dkp = (bf16*)a.dk + (base + kj) * a.lddk + (int64_t)kvh * D;
    bf16* dvp = (bf16*)a.dv + (base + kj) * a.lddv + (int64_t)kvh * D;
    float kv[D / 32][16];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = db * 32 + 8 * g + 4 * hh, j4 = (db & 1) * 4 + g;
        const f32x4 pv = red[db >> 1][(kw * 8 + j4) * 64 + lane];
        const f32x4 pk = red[2 + (db >> 1)][(kw * 8 + j4) * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) kv[db][4 * g + e] = (dk[db][4 * g + e] + pk[e]) * scale;
        store4(dvp + dd, dv[db][4 * g] + pv[0], dv[db][4 * g + 1] + pv[1], dv[db][4 * g + 2] + pv[2],
               dv[db][4 * g + 3] + pv[3]);
      }
    if (a.rope_cos) rope_back_row(kv, a.rope_cos, a.rope_sin, kj, hh);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4(dkp + db * 32 + 8 * g + 4 * hh, kv[db][4 * g], kv[db][4 * g + 1], kv[db][4 * g + 2], kv[db][4 * g + 3]);
  }
}

// ------------------------------------------------------------------------------------------
// backward, dQ: block = 4 waves x 32 queries of one q head; key tiles of 64 up to the diagonal
// ------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 1) void attn_dq_mfma(Attn a) {
  constexpr int BQ = 128, BK = 64, KP = D + 8, TP = BK + 12;
  __shared__ bf16 Ks[BK * KP];
  __shared__ bf16 Vs[BK * KP];
  __shared__ bf16 Kt[D * TP];
  const int S = a.S;
  const int nqt = (S + BQ - 1) / BQ;
  const int group = a.nq / a.nkv;
  int pair, unit;
  if (!pair_unit(group * nqt, a.nkv * a.n_seq, pair, unit)) return;
  const int qt = nqt - 1 - unit / group;  // longest first, the group's heads together
  const int kvh = pair % a.nkv, seq = pair / a.nkv;
  const int h = kvh * group + unit % group;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, hh = lane >> 5, lq = lane & 31;
  const int q0 = qt * BQ;
  const int qi = q0 + 32 * w + lq;
  const int64_t base = (int64_t)seq * S;
  const float sl2 = LOG2E / sqrtf((float)D);
  const float scale = 1.f / sqrtf((float)D);
  const bf16* K = (const bf16*)a.k + (int64_t)kvh * D;
  const bf16* V = (const bf16*)a.v + (int64_t)kvh * D;

  bf16x8 qf[D / 16], gf[D / 16];
  {
    const int64_t row = base + min(qi, S - 1);
    const bf16* qp = (const bf16*)a.q + row * a.ldq + (int64_t)h * D;
    const bf16* gp = (const bf16*)a.dO + row * a.lddo + (int64_t)h * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      qf[kk] = *(const bf16x8*)(qp + 16 * kk + 8 * hh);
      gf[kk] = *(const bf16x8*)(gp + 16 * kk + 8 * hh);
    }
  }
  const bool qv = qi < S;
  const float lse_q = qv ? a.lse[((int64_t)seq * a.nq + h) * S + qi] * LOG2E : 0.f;
  const float dl_q = qv ? a.delta[((int64_t)seq * a.nq + h) * S + qi] : 0.f;
  f32x16 dq[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) zero(dq[i]);
  const int qmax = min(q0 + BQ, S) - 1;
  const int nkt = qmax / BK + 1;
  const int wave_qmax = min(q0 + 32 * w + 31, S - 1);
  NatTile<BK, D> kreg, vreg;
  kreg.load(K, a.ldk, base, min(BK, S));
  vreg.load(V, a.ldv, base, min(BK, S));
  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * BK;
    __syncthreads();
    kreg.store(Ks, KP);
    vreg.store(Vs, KP);
    __syncthreads();
    lds_transpose<BK, D>(Ks, KP, Kt, TP);
    if (kt + 1 < nkt) {  // next tile in flight while this one is computed on
      const int n1 = min(BK, S - k0 - BK);
      kreg.load(K, a.ldk, base + k0 + BK, n1);
      vreg.load(V, a.ldv, base + k0 + BK, n1);
    }
    __syncthreads();
    if (k0 > wave_qmax) continue;
    f32x16 s[2], dp[2];
    zero(s[0]); zero(s[1]); zero(dp[0]); zero(dp[1]);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = mfma(*(const bf16x8*)(Ks + (kb * 32 + lq) * KP + 16 * kk + 8 * hh), qf[kk], s[kb]);
        dp[kb] = mfma(*(const bf16x8*)(Vs + (kb * 32 + lq) * KP + 16 * kk + 8 * hh), gf[kk], dp[kb]);
      }
    // element r of block kb: key k0 + 32 kb + 8 (r/4) + 4 hh + r%4, query qi
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = k0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
        const bool ok = qv && kk <= qi && kk < S;
        const float p = ok ? ex2(s[kb][r] * sl2 - lse_q) : 0.f;
        dp[kb][r] = p * (dp[kb][r] - dl_q);
      }
    // dQ^T[d][q] += K^T[d][key] dS^T[key][q]
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const bf16x8 sb = acc_frag(dp[ks >> 1], ks & 1);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) dq[db] = mfma(tfrag(Kt, TP, db * 32 + lq, ks, hh), sb, dq[db]);
    }
  }
  if (qv) {
    bf16* dqp = (bf16*)a.dq + (base + qi) * a.lddq + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4(dqp + db * 32 + 8 * g + 4 * hh, dq[db][4 * g] * scale, dq[db][4 * g + 1] * scale,
               dq[db][4 * g + 2] * scale, dq[db][4 * g + 3] * scale);
  }
}

// dQ for head width 128 without the transposed key copy: K and V tiles stay natural in a
// double-buffered, swizzled LDS pair (the layout of the dK/dV kernel above, one block barrier per
// key tile) and the dQ product reads K transposed with ds_read_b64_tr_b16.
// 8 waves, two per SIMD: waves w and w + 4 hold the same 32 queries and take the two 32-key halves
// of every key tile; the second wave's dQ partial sum goes through LDS to the first at the end.
__global__ __launch_bounds__(512, 1) void attn_dq_tr128(Attn a) {
  constexpr int D = 128, BQ = 128, BK = 64, KT = BK * D, NT = 512;
  __shared__ __attribute__((aligned(16))) bf16 Ks[2 * KT];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2 * KT];
  const int S = a.S;
  const int nqt = (S + BQ - 1) / BQ;
  const int group = a.nq / a.nkv;
  int pair, unit;
  if (!pair_unit(group * nqt, a.nkv * a.n_seq, pair, unit)) return;
  const int qt = nqt - 1 - unit / group;  // longest first, the group's heads together
  const int kvh = pair % a.nkv, seq = pair / a.nkv;
  const int h = kvh * group + unit % group;
  const int lane = threadIdx.x & 63, hh = lane >> 5, lq = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: tile tests are scalar branches
  const int qw = w & 3, kb = w >> 2;  // query group of 32, key half of each tile
  const int q0 = qt * BQ;
  const int qi = q0 + 32 * qw + lq;
  const int64_t base = (int64_t)seq * S;
  const float sl2 = LOG2E / sqrtf((float)D);
  const float scale = 1.f / sqrtf((float)D);
  const bf16* K = (const bf16*)a.k + (int64_t)kvh * D;
  const bf16* V = (const bf16*)a.v + (int64_t)kvh * D;

  bf16x8 qf[D / 16], gf[D / 16];
  {
    const int64_t row = base + min(qi, S - 1);
    const bf16* qp = (const bf16*)a.q + row * a.ldq + (int64_t)h * D;
    const bf16* gp = (const bf16*)a.dO + row * a.lddo + (int64_t)h * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      qf[kk] = *(const bf16x8*)(qp + 16 * kk + 8 * hh);
      gf[kk] = *(const bf16x8*)(gp + 16 * kk + 8 * hh);
    }
  }
  const bool qv = qi < S;
  const float lse_q = qv ? a.lse[((int64_t)seq * a.nq + h) * S + qi] * LOG2E : 0.f;
  const float dl_q = qv ? a.delta[((int64_t)seq * a.nq + h) * S + qi] : 0.f;
  int toff[2][D / 32];
  {
    const int g = lane >> 4, aa = lane & 3, j = (lane >> 2) & 3;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) toff[hf][db] = qoff(8 * hf + 4 * (g >> 1) + j, db * 32 + 16 * (g & 1) + 4 * aa);
  }
  f32x16 dq[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) zero(dq[i]);
  const int qmax = min(q0 + BQ, S) - 1;
  const int nkt = qmax / BK + 1;
  const int wave_qmax = min(q0 + 32 * qw + 31, S - 1);
  NatTile<BK, D, NT> kreg, vreg;
  NatOff<BK, D, NT> koffs, voffs;
  koffs.init(a.ldk);
  voffs.init(a.ldv);
  auto fetch = [&](int kt) {
    const int k0 = kt * BK;
    if (k0 + BK <= S) {
      koffs.load(kreg, K + (base + k0) * a.ldk);
      voffs.load(vreg, V + (base + k0) * a.ldv);
    } else {
      kreg.load(K, a.ldk, base + k0, S - k0);
      vreg.load(V, a.ldv, base + k0, S - k0);
    }
  };
  auto put = [&](int b) {
#pragma unroll
    for (int i = 0; i < NatTile<BK, D, NT>::N; ++i) {
      const int c = threadIdx.x + NT * i, r = c >> 4, ch = c & 15;
      const int o = b * KT + r * 128 + ((ch ^ qsw(r)) << 3);
      *(u32x4*)(Ks + o) = kreg.v[i];
      *(u32x4*)(Vs + o) = vreg.v[i];
    }
  };
  fetch(0);
  put(0);
  if (nkt > 1) fetch(1);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * BK, cur = kt & 1, kh0 = k0 + 32 * kb;  // this wave's first key
    const bf16* Kc = Ks + cur * KT;
    const bf16* Vc = Vs + cur * KT;
    if (kh0 <= wave_qmax) {  // else every key of the half is after this wave's queries
      f32x16 s, dp;
      zero(s);
      zero(dp);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const int o = qoff(kb * 32 + lq, 16 * kk + 8 * hh);
        s = mfma(*(const bf16x8*)(Kc + o), qf[kk], s);
        dp = mfma(*(const bf16x8*)(Vc + o), gf[kk], dp);
      }
      // element r: key kh0 + 8 (r/4) + 4 hh + r%4, query qi; P as the dK/dV kernel forms it
      if (kh0 + 31 <= q0 + 32 * qw && q0 + 32 * qw + 31 < S) {  // every key at or before every query (wave-uniform)
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = ex2(fmaf(s[r], sl2, -lse_q)) * (dp[r] - dl_q);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = kh0 + 8 * (r >> 2) + 4 * hh + (r & 3);
          const bool ok = qv && kk <= qi && kk < S;
          const float p = ok ? ex2(fmaf(s[r], sl2, -lse_q)) : 0.f;
          dp[r] = p * (dp[r] - dl_q);
        }
      }
      // dQ^T[d][q] += K^T[d][key] dS^T[key][q]
#pragma unroll
      for (int ksp = 0; ksp < 2; ++ksp) {
        const int ks = 2 * kb + ksp;
        const bf16x8 sb = acc_frag(dp, ksp);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          dq[db] = mfma(tr_pair(Kc + ks * 16 * 128 + toff[0][db], Kc + ks * 16 * 128 + toff[1][db]), sb, dq[db]);
      }
    }
    if (kt + 1 < nkt) {
      put(cur ^ 1);  // every wave finished reading that buffer before the previous barrier
      if (kt + 2 < nkt) fetch(kt + 2);
    }
    __syncthreads();
  }
  // the second-half waves hand their sums to the first-half waves: float4 j4 of accumulator
  // half hf goes to ((qw * 8 + j4) * 64 + lane) of a 32 KB region (the tile buffers are free
  // after the last barrier): dq[0..1] -> Ks, dq[2..3] -> Vs
  f32x4* red[2] = {(f32x4*)Ks, (f32x4*)Vs};
  if (kb == 1) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        red[db >> 1][(qw * 8 + (db & 1) * 4 + g) * 64 + lane] =
            f32x4{dq[db][4 * g], dq[db][4 * g + 1], dq[db][4 * g + 2], dq[db][4 * g + 3]};
  }
  __syncthreads();
  if (kb == 0 && qv) {
    bf16* dqp = (bf16*)a.dq + (base + qi) * a.lddq + (int64_t)h * D;
    float qv4[D / 32][16];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 pq = red[db >> 1][(qw * 8 + (db & 1) * 4 + g) * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) qv4[db][4 * g + e] = (dq[db][4 * g + e] + pq[e]) * scale;
      }
    if (a.rope_cos) rope_back_row(qv4, a.rope_cos, a.rope_sin, qi, hh);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4(dqp + db * 32 + 8 * g + 4 * hh, qv4[db][4 * g], qv4[db][4 * g + 1], qv4[db][4 * g + 2], qv4[db][4 * g + 3]);
  }
}

// Forward for head width 128 in the same layout: K and V tiles of 64 keys natural, swizzled and
// double-buffered in LDS (one block barrier per tile); the P V product reads V transposed with
// ds_read_b64_tr_b16.
__global__ __launch_bounds__(256, 2) void attn_fwd_tr128(Attn a) {
  constexpr int D = 128, BQ = 128, BK = 64, KT = BK * D;
  __shared__ __attribute__((aligned(1024))) bf16 Ks[2 * KT];
  __shared__ __attribute__((aligned(1024))) bf16 Vs[2 * KT];
  const int S = a.S;
  const int nqt = (S + BQ - 1) / BQ;
  const int group = a.nq / a.nkv;
  int pair, unit;
  if (!pair_unit(group * nqt, a.nkv * a.n_seq, pair, unit)) return;
  const int qt = nqt - 1 - unit / group;  // longest (latest) query tiles first, the group's heads together
  const int kvh = pair % a.nkv, seq = pair / a.nkv;
  const int h = kvh * group + unit % group;
  const int lane = threadIdx.x & 63, hh = lane >> 5, lq = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: the mask test below is a scalar branch
  const int q0 = qt * BQ;
  const int qi = q0 + 32 * w + lq;  // this lane's query (column of every accumulator)
  const int64_t base = (int64_t)seq * S;
  const bf16* Q = (const bf16*)a.q + (int64_t)h * D;
  const bf16* K = (const bf16*)a.k + (int64_t)kvh * D;
  const bf16* V = (const bf16*)a.v + (int64_t)kvh * D;

  bf16x8 qf[D / 16];
  {
    const bf16* qp = Q + (base + min(qi, S - 1)) * a.ldq;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = *(const bf16x8*)(qp + 16 * kk + 8 * hh);
  }
  int toff[2][D / 32];
  {
    const int g = lane >> 4, aa = lane & 3, j = (lane >> 2) & 3;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) toff[hf][db] = qoff(8 * hf + 4 * (g >> 1) + j, db * 32 + 16 * (g & 1) + 4 * aa);
  }
  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) zero(o[i]);
  const float sl2 = LOG2E / sqrtf((float)D);
  float m = -INFINITY, l = 0.f;
  const int qmax = min(q0 + BQ, S) - 1;
  const int nkt = qmax / BK + 1;
  const int wave_qmax = min(q0 + 32 * w + 31, S - 1);

  // Tiles go straight into LDS (no register staging): instruction i of wave w fills rows
  // 4 (w + 4 i) .. + 3 of a 64-row tile (1 KB); lane l takes row 4 (w + 4 i) + l / 16, physical
  // 16-byte chunk l % 16, i.e. logical chunk (l % 16) ^ qsw(row); rows past S are clamped.
  auto load_tile = [&](bf16* dst, const bf16* src, int64_t ld, int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * (w + 4 * i) + (lane >> 4);
      const int c = (lane & 15) ^ qsw(r);
      const int rr = min(r, S - 1 - k0);
      __builtin_amdgcn_global_load_lds((fa_gptr)(src + (base + k0 + rr) * ld + c * 8), (fa_lptr)(dst + 4 * (w + 4 * i) * 128),
                                       16, 0, 0);
    }
  };
  // the unscaled scores of a tile: s[kb][r] = score(key k0 + 32 kb + 8 (r/4) + 4 hh + r%4, query qi)
  auto scores = [&](f32x16* s, const bf16* Kc) {
    zero(s[0]);
    zero(s[1]);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = *(const bf16x8*)(Kc + qoff(kb * 32 + lq, 16 * kk + 8 * hh));
        s[kb] = mfma(kf, qf[kk], s[kb]);
      }
  };
  // Software pipeline: iteration kt computes the scores of tile kt + 1 among the exponentials of
  // tile kt, so the matrix unit works beside the vector unit (+5-8 % at 4K-16K tokens, the same
  // bits). K buffer kt % 2 takes tile kt + 2 once every wave has the scores of tile kt; V buffer
  // (kt + 1) % 2 takes tile kt + 1 once every wave is past the products of tile kt - 1; both are
  // issued at the start of iteration kt, so each tile has one iteration to land.
  auto step = [&](int kt, f32x16* sc, f32x16* sn) {
    const int k0 = kt * BK, cur = kt & 1;
    // K of tile kt + 1 and V of tile kt landed; every wave is done with iteration kt - 1
    asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (kt + 2 < nkt) load_tile(Ks + cur * KT, K, a.ldk, kt + 2);
    if (kt + 1 < nkt) load_tile(Vs + (cur ^ 1) * KT, V, a.ldv, kt + 1);
    if (k0 > wave_qmax) return;  // every key of this tile is in this wave's future
    f32x16* s = sc;
    const bool diag = (k0 + BK - 1 > q0 + 32 * w) || (k0 + BK > S);  // wave-uniform
    if (diag) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kj = k0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
          s[kb][r] = (kj > qi || kj >= S) ? -INFINITY : s[kb][r];
        }
    }
    // the maximum of the unscaled scores (scaling by sl2 > 0 keeps the order), over both halves
    // of the wave, which hold the same query
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = xhalf_max(mx);
    const float tm = mx * sl2;
    if (tm > m + RESCALE_SLACK) {  // the reference moves (m = -inf before the first tile: corr = 0)
      const float corr = ex2(m - tm);
      l *= corr;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= corr;
      m = tm;
    }
    // the scores of tile kt + 1, in the same block as the exponentials below so that they can
    // interleave (also when that tile is past this wave's queries or past the sequence: then its
    // buffer holds stale keys and the scores are never read)
    scores(sn, Ks + (cur ^ 1) * KT);
    // p = 2^(s sl2 - m); four partial row sums
    float ls4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = ex2(fmaf(s[kb][r], sl2, -m));
        s[kb][r] = p;
        ls4[r & 3] += p;
      }
    float ls = (ls4[0] + ls4[1]) + (ls4[2] + ls4[3]);
    ls = xhalf_sum(ls);
    l += ls;
    // O^T[d][q] += V^T[d][key] P^T[key][q]
    const bf16* Vc = Vs + cur * KT;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const bf16x8 pb = acc_frag(s[ks >> 1], ks & 1);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        o[db] = mfma(tr_pair(Vc + ks * 16 * 128 + toff[0][db], Vc + ks * 16 * 128 + toff[1][db]), pb, o[db]);
    }
  };
  load_tile(Ks, K, a.ldk, 0);
  if (nkt > 1) load_tile(Ks + KT, K, a.ldk, 1);
  load_tile(Vs, V, a.ldv, 0);
  if (nkt > 1) asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");  // K of tile 0
  else asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
  f32x16 sa[2], sb[2];
  scores(sa, Ks);  // every wave sees tile 0
  for (int kt = 0; kt < nkt; kt += 2) {  // two iterations a trip, the score sets swapped
    step(kt, sa, sb);
    if (kt + 1 < nkt) step(kt + 1, sb, sa);
  }
  if (qi < S) {
    const float inv = 1.f / l;
    bf16* op = (bf16*)a.o + (base + qi) * a.ldo + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4(op + db * 32 + 8 * g + 4 * hh, o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
               o[db][4 * g + 3] * inv);
    if (hh == 0) a.lse[((int64_t)seq * a.nq + h) * S + qi] = (m + __log2f(l)) * LN2;
  }
}

// delta[seq, h, i] = sum_d dO * O  (one wavefront per (token, head))
__global__ __launch_bounds__(256) void attn_delta_bf16(Attn a) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t total = (int64_t)a.n_seq * a.S * a.nq;
  if (row >= total) return;
  const int h = (int)(row % a.nq);
  const int64_t t = row / a.nq;
  const bf16* o = (const bf16*)a.o + t * a.ldo + (int64_t)h * a.d;
  const bf16* g = (const bf16*)a.dO + t * a.lddo + (int64_t)h * a.d;
  float s = 0.f;
  for (int j = lane * 2; j < a.d; j += 128) s += (float)o[j] * (float)g[j] + (float)o[j + 1] * (float)g[j + 1];
  s = wave_sum(s);
  const int seq = (int)(t / a.S), i = (int)(t % a.S);
  if (lane == 0) a.delta[((int64_t)seq * a.nq + h) * a.S + i] = s;
}

bool attn_mfma_supported(const Attn& a) {
  const bool aligned = ((a.ldq | a.ldk | a.ldv | a.ldo) % 8 == 0) &&
                       ((((uintptr_t)a.q) | ((uintptr_t)a.k) | ((uintptr_t)a.v) | ((uintptr_t)a.o)) % 16 == 0);
  return a.t == DT_BF16 && (a.d == 64 || a.d == 128) && aligned;
}

bool attn_mfma_bwd_supported(const Attn& a) {
  const bool aligned = ((a.lddo | a.lddq | a.lddk | a.lddv) % 8 == 0) &&
                       ((((uintptr_t)a.dO) | ((uintptr_t)a.dq) | ((uintptr_t)a.dk) | ((uintptr_t)a.dv)) % 16 == 0);
  return attn_mfma_supported(a) && aligned;
}

int launch_attn_fwd_mfma(const Attn& a, hipStream_t s) {
  dim3 grid(pair_grid(((a.S + 127) / 128) * (a.nq / a.nkv), a.nkv * a.n_seq));
  if (a.d == 128) hipLaunchKernelGGL(attn_fwd_tr128, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(attn_fwd_mfma<64>, grid, dim3(256), 0, s, a);
  return (int)hipGetLastError();
}

int launch_attn_bwd_mfma(const Attn& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.n_seq * a.S * a.nq;
  hipLaunchKernelGGL(attn_delta_bf16, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
  dim3 gk(pair_grid((a.S + 127) / 128, a.nkv * a.n_seq)),
      gq(pair_grid(((a.S + 127) / 128) * (a.nq / a.nkv), a.nkv * a.n_seq));
  if (a.d == 128) {
    hipLaunchKernelGGL(attn_dkdv_tr128, gk, dim3(512), 0, s, a);
    hipLaunchKernelGGL(attn_dq_tr128, gq, dim3(512), 0, s, a);
  } else {
    hipLaunchKernelGGL(attn_dkdv_mfma<64>, gk, dim3(256), 0, s, a);
    hipLaunchKernelGGL(attn_dq_mfma<64>, gq, dim3(256), 0, s, a);
  }
  return (int)hipGetLastError();
}

}  // namespace hol
