// Projected value norms on gfx950 (CriticalKV composite, LaProx score).
//
// CriticalKV notes, "损失函数 / 训练策略": the only new runtime quantity is the
// L1 norm of every row of V W^O; "两阶段贪心选择算法": the composite score of an
// entry is (A + eps) * ||(V W^O)_t||_1.  Under GQA the composite of a KV head is
// the mean over its query heads i of (A_i[t] + eps) * ||(V_g W^O_i)[t]||_1.
// LaProx page, Section 4.1, Algorithm 1: p[t] = ||A[:, t]||_2 * ||H[t, :]||_2
// with H = V W_O; the group takes the mean over its query heads of
// sqrt(sum_r A_i[r, t]^2) * ||(V_g W^O_i)[t]||_2 (L2 = true).
//
// For one KV head g and 256 keys, a workgroup forms V_g[t, :] W^O_i (K = d = 128,
// N = hidden) for every query head i of the group on 16x16x32 bf16 MFMA tiles,
// and folds every product element into |.| row sums as soon as it leaves the
// accumulator: the [keys x hidden] product is never written.  W^O is read in
// the nn.Linear layout [hidden, hq*d], so a 64-column tile of W^O_i is 64
// contiguous 256-byte rows.  Each tile is loaded into registers two tiles
// ahead of its multiply and written to one of two LDS slots, 16-byte chunk ch
// of row r at position ch ^ (r & 15), so the 16 rows of one B-operand read fall
// in 16 different bank groups.  One barrier per tile, and loads stay in flight
// across it.
#include "common.hpp"
#include "kernels.hpp"

namespace adakv {
namespace {

constexpr int D = 128;
constexpr int KEYS = 256;          // keys per workgroup (64 per wave)
constexpr int NT = 64;             // hidden columns per tile
constexpr int ROWB = D * 2;        // bytes per W^O tile row
constexpr int SLOT = NT * ROWB;    // 16 KB per tile
constexpr int CPT = SLOT / 16 / 256;   // 16-byte chunks per thread per tile
constexpr int KSTEPS = D / 32;
constexpr int MAXG = 8;

// Workgroup barrier for LDS only: global loads issued before it stay in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <bool L2>
__global__ __launch_bounds__(256, 2) void vwo_norm_kernel(const uint16_t* __restrict__ v,
                                                          const uint16_t* __restrict__ w_o,
                                                          const float* __restrict__ head_scores,
                                                          float* __restrict__ comp, int inst0, int hq, int hkv, int G,
                                                          int n, int p, int hidden, float eps) {
  __shared__ __align__(16) char wt[2][SLOT];
  __shared__ float ahs[MAXG][KEYS];     // (A_i + eps) of the workgroup's keys
  const int g = blockIdx.y, il = blockIdx.z, inst = inst0 + il;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int gq = lane >> 4, c = lane & 15;
  const int kwg = blockIdx.x * KEYS;
  const int key0 = kwg + 64 * wv;
  const uint16_t* vb = v + ((size_t)inst * hkv + g) * (size_t)n * D;
  const size_t wrow = (size_t)hq * D;
  const int ntiles = hidden / NT;
  const int total = G * ntiles;        // (head, tile) pairs in order

  // this thread's chunks of a tile: row r = idx / 16, chunk idx % 16
  auto load_tile = [&](u32x4 (&reg)[CPT], int T) {
    const uint16_t* wb = w_o + (size_t)(g * G + T / ntiles) * D + (size_t)((T % ntiles) * NT) * wrow;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = threadIdx.x + 256 * i;
      reg[i] = ld16(wb + (size_t)(idx >> 4) * wrow + (idx & 15) * 8);
    }
  };
  auto store_tile = [&](const u32x4 (&reg)[CPT], char* slot) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = threadIdx.x + 256 * i, r = idx >> 4, ch = idx & 15;
      st16(slot + r * ROWB + ((ch ^ (r & 15)) * 16), reg[i]);
    }
  };

  u32x4 ra[CPT], rb[CPT];
  load_tile(ra, 0);
  if (total > 1) load_tile(rb, 1);
  for (int idx = threadIdx.x; idx < G * KEYS; idx += 256) {
    const int h = idx / KEYS, t = kwg + idx % KEYS;
    float a = 0.f;
    if (t < p) {
      const float hsv = head_scores[((size_t)il * hq + g * G + h) * p + t];
      a = L2 ? sqrtf(hsv) : hsv + eps;
    }
    ahs[h][idx % KEYS] = a;
  }
  // A operands: 4 M-blocks of 16 keys, held for the whole workgroup.
  bf16x8 aop[4][KSTEPS];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    int t = key0 + 16 * mb + c;
    t = (t < p) ? t : 0;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) aop[mb][ks] = Mma<uint16_t>::load(vb + (size_t)t * D + ks * 32 + 8 * gq);
  }
  store_tile(ra, wt[0]);
  if (total > 2) load_tile(ra, 2);
  __syncthreads();     // ahs and tile 0 in LDS

  float cacc[4][4], rsum[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) { cacc[mb][j] = 0.f; rsum[mb][j] = 0.f; }

  // Tile T is in slot T % 2; the registers of tile T+1 are `nxt` (written to the
  // other slot after the multiply), and `nxt` then takes tile T+3.
  auto step = [&](int T, u32x4 (&nxt)[CPT]) {
    const char* slot = wt[T & 1];
    // one 16-column block at a time: its |.| sums overlap the next block's MFMAs
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int r = 16 * nb + c;
      f32x4 acc[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb] = zero4();
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const bf16x8 bop = *reinterpret_cast<const bf16x8*>(slot + r * ROWB + (((ks * 4 + gq) ^ c) * 16));
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) acc[mb] = Mma<uint16_t>::mma(aop[mb][ks], bop, acc[mb]);
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) rsum[mb][j] = L2 ? fmaf(acc[mb][j], acc[mb][j], rsum[mb][j]) : rsum[mb][j] + fabsf(acc[mb][j]);
    }
    if ((T + 1) % ntiles == 0) {
      // head done: rsum[mb][j] is this lane's part of key key0 + 16mb + 4gq + j
      const int h = T / ntiles;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float x = rsum[mb][j];
          x += shfl_xor(x, 8);
          x += shfl_xor(x, 4);
          x += shfl_xor(x, 2);
          x += shfl_xor(x, 1);
          if (L2) x = sqrtf(x);
          cacc[mb][j] += ahs[h][64 * wv + 16 * mb + 4 * gq + j] * x;
          rsum[mb][j] = 0.f;
        }
    }
    if (T + 1 < total) store_tile(nxt, wt[(T + 1) & 1]);
    lds_barrier();     // tile T+1 in LDS; slot T & 1 free
    if (T + 3 < total) load_tile(nxt, T + 3);
  };
  for (int T = 0; T < total; T += 2) {
    step(T, rb);
    if (T + 1 < total) step(T + 1, ra);
  }
  const float invG = 1.0f / (float)G;
  if (c == 0) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = key0 + 16 * mb + 4 * gq + j;
        if (t < p) comp[((size_t)inst * hkv + g) * p + t] = cacc[mb][j] * invG;
      }
  }
}

}  // namespace

hipError_t launch_vwo(const Geo& g, int inst0, int ni, const void* v, const void* w_o, const float* head_scores,
                      float* score2, hipStream_t st) {
  if (g.dtype != ADAKV_BF16 || g.d != D || g.hidden % NT != 0 || g.G > MAXG) return hipErrorInvalidValue;
  dim3 grid((g.p + KEYS - 1) / KEYS, g.hkv, ni);
  if (g.scorer == ADAKV_SCORE_LAPROX)
    vwo_norm_kernel<true><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(w_o),
                                                head_scores, score2, inst0, g.hq, g.hkv, g.G, g.n, g.p, g.hidden, g.eps);
  else
    vwo_norm_kernel<false><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(w_o),
                                                 head_scores, score2, inst0, g.hq, g.hkv, g.G, g.n, g.p, g.hidden, g.eps);
  return hipGetLastError();
}

}  // namespace adakv
