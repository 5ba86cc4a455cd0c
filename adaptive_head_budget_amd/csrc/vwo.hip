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
// For the L2 norm a wide projection need not be formed at all:
// ||v W^O_i||_2^2 = v M_i v^T with M_i = W^O_i W^O_i^T, the d x d Gram
// matrix.  gram_kernel forms the Gram matrices on MFMA (fp32 partial sums over
// slices of the hidden dimension), gram_planes_kernel adds the slices in fp64
// and writes M_i as two bf16 planes (M = hi + lo to ~2^-17 relative), and the
// norm kernel forms u = v M_i from the two planes (2*d columns instead of D),
// places v itself in the same accumulator layout with one MFMA against an
// identity operand, and folds u . v.  The form only depends on M + M^T, so the
// planes hold M' with M'[c][e] = 2 M[c][e] where e lies in an earlier 32-block
// than c, M[c][e] in the same block and 0 in a later one: output columns of
// block t contract over k-steps 0..t only (10 of 16 steps per head).
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
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace adakv {
namespace {

constexpr int D = 128;
constexpr int KEYS = 256;          // keys per workgroup (64 per wave)
constexpr int TROWS_W = 64;        // W^O rows per tile (all planes)
constexpr int ROWB = D * 2;        // bytes per W^O tile row
constexpr int SLOT = TROWS_W * ROWB;   // 16 KB per tile
constexpr int CPT = SLOT / 16 / 256;   // 16-byte chunks per thread per tile
constexpr int KSTEPS = D / 32;
constexpr int MAXG = 8;

// Workgroup barrier for LDS only: global loads issued before it stay in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// MODE 0 (CriticalKV) and 1 (LaProx): w_o is the projection itself ([hidden,
// hq*d]), a tile holds 64 output columns, folded as |x| or x^2.  MODE 2
// (LaProx, wide projection): w_o holds the two bf16 planes of the Gram
// matrices one after the other ([2*d, hq*d]); a tile holds 32 columns of both
// planes, their products are summed into u = v M, and u . v is folded, v
// taken into the accumulator layout by one MFMA against an identity operand.
enum { VWO_L1 = 0, VWO_L2 = 1, VWO_GRAM = 2 };
template <int MODE>
__global__ __launch_bounds__(256, 2) void vwo_norm_kernel(const uint16_t* __restrict__ v,
                                                          const uint16_t* __restrict__ w_o,
                                                          const float* __restrict__ head_scores,
                                                          float* __restrict__ comp, int inst0, int hq, int hkv, int G,
                                                          int n, int p, int hidden, float eps) {
  __shared__ __align__(16) char wt[2][SLOT];
  __shared__ float ahs[MAXG][KEYS];     // (A_i + eps) of the workgroup's keys
  // Workgroups are dealt round-robin to the 8 XCDs (workgroup b to XCD b % 8),
  // and each XCD has its own L2.  Work item (key block, head) is therefore
  // chosen so that XCD x takes a contiguous run of the (head, key block) order:
  // the CUs of one XCD stream the same head's W^O tiles through their shared
  // L2 instead of every XCD streaming every head's.  One instance per launch
  // plane (blockIdx.z); a grid whose size is not a multiple of 8 keeps the
  // plain order.
  int kb = blockIdx.x, g = blockIdx.y;
  {
    const int nkb = gridDim.x, items = gridDim.x * gridDim.y;
    if (items % 8 == 0) {
      const int b = blockIdx.y * nkb + blockIdx.x;
      const int w = (b % 8) * (items / 8) + b / 8;
      g = w / nkb;
      kb = w % nkb;
    }
  }
  const int il = blockIdx.z, inst = inst0 + il;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int gq = lane >> 4, c = lane & 15;
  const int kwg = kb * KEYS;
  const int key0 = kwg + 64 * wv;
  const uint16_t* vb = v + ((size_t)inst * hkv + g) * (size_t)n * D;
  constexpr int NPLANE = (MODE == VWO_GRAM) ? 2 : 1;
  constexpr int NT = TROWS_W / NPLANE;   // output columns per tile
  const size_t wrow = (size_t)hq * D;
  const int ntiles = hidden / NT;      // hidden = output columns (one plane)
  const int total = G * ntiles;        // (head, tile) pairs in order

  // this thread's chunks of a tile: row r = idx / 16, chunk idx % 16; row r is
  // plane r / NT, column (T % ntiles) * NT + r % NT of that plane
  auto load_tile = [&](u32x4 (&reg)[CPT], int T) {
    const uint16_t* wb = w_o + (size_t)(g * G + T / ntiles) * D + (size_t)((T % ntiles) * NT) * wrow;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = threadIdx.x + 256 * i, r = idx >> 4;
      const size_t row = (size_t)(r / NT) * hidden + (r % NT);
      // MODE 2: tile T reads k-steps 0..T % 4 only (chunks 4 ks .. 4 ks + 3)
      if (MODE != VWO_GRAM || ((idx & 15) >> 2) <= (T % ntiles)) reg[i] = ld16(wb + row * wrow + (idx & 15) * 8);
      else reg[i] = u32x4{0u, 0u, 0u, 0u};   // never read back
    }
  };
  auto store_tile = [&](const u32x4 (&reg)[CPT], char* slot) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = threadIdx.x + 256 * i, r = idx >> 4, ch = idx & 15;
      st16(slot + r * ROWB + ((ch ^ (r & 15)) * 16), reg[i]);
    }
  };

  // Every prologue load is issued before the first wait: the A operands (4
  // M-blocks of 16 keys, held for the whole workgroup), tiles 0 and 1, and the
  // head scores of the workgroup's keys (thread = key).
  static_assert(KEYS == 256, "one key per thread in the prologue");
  bf16x8 aop[4][KSTEPS];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    int t = key0 + 16 * mb + c;
    t = (t < p) ? t : 0;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) aop[mb][ks] = Mma<uint16_t>::load(vb + (size_t)t * D + ks * 32 + 8 * gq);
  }
  u32x4 ra[CPT], rb[CPT];
  load_tile(ra, 0);
  if (total > 1) load_tile(rb, 1);
  const int tk = kwg + (int)threadIdx.x;
  float hsv[MAXG];
#pragma unroll
  for (int h = 0; h < MAXG; ++h)
    hsv[h] = (h < G && tk < p) ? head_scores[((size_t)il * hq + g * G + h) * p + tk] : 0.f;
#pragma unroll
  for (int h = 0; h < MAXG; ++h)
    if (h < G) ahs[h][threadIdx.x] = (tk < p) ? ((MODE != VWO_L1) ? sqrtf(hsv[h]) : hsv[h] + eps) : 0.f;
  store_tile(ra, wt[0]);
  if (total > 2) load_tile(ra, 2);
  __syncthreads();     // ahs and tile 0 in LDS

  float cacc[4][4], rsum[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) { cacc[mb][j] = 0.f; rsum[mb][j] = 0.f; }

  // MODE 2: identity operands of the two 16-column blocks of a tile.  Block nb
  // of a tile covers columns 32 * (T % 4) + 16 nb + c, which lie in k-step
  // T % 4; within it lane (gq, c) holds k = 8 gq .. 8 gq + 7, so its one is at
  // position 16 nb + c - 8 gq when that lies in [0, 8).
  bf16x8 bid[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int tpos = 16 * nb + c - 8 * gq;
    u32x4 idw = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      idw[q] = ((tpos == 2 * q) ? 0x3F80u : 0u) | ((tpos == 2 * q + 1) ? 0x3F800000u : 0u);
    bid[nb] = __builtin_bit_cast(bf16x8, idw);
  }

  // Tile T is in slot T % 2; the registers of tile T+1 are `nxt` (written to the
  // other slot after the multiply), and `nxt` then takes tile T+3.  KSID: the
  // k-step of a MODE 2 tile's columns (T % 4), fixed at compile time.
  auto step = [&](int T, u32x4 (&nxt)[CPT], auto ksid_tag) {
    constexpr int KSID = decltype(ksid_tag)::value;
    const char* slot = wt[T & 1];
    // one 16-column block at a time: its |.| sums overlap the next block's MFMAs
#pragma unroll
    for (int nb = 0; nb < NT / 16; ++nb) {
      f32x4 acc[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb] = zero4();
#pragma unroll
      for (int pl = 0; pl < NPLANE; ++pl) {
        const int r = pl * NT + 16 * nb + c;
#pragma unroll
        for (int ks = 0; ks < (MODE == VWO_GRAM ? KSID + 1 : KSTEPS); ++ks) {
          const bf16x8 bop = *reinterpret_cast<const bf16x8*>(slot + r * ROWB + (((ks * 4 + gq) ^ c) * 16));
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) acc[mb] = Mma<uint16_t>::mma(aop[mb][ks], bop, acc[mb]);
        }
      }
      if (MODE == VWO_GRAM) {
        // v at the tile's columns in the accumulator layout:
        // D[m][n] = sum_k v[m][k] [k == column n], one MFMA per M-block
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const f32x4 vv = Mma<uint16_t>::mma(aop[mb][KSID], bid[nb], zero4());
#pragma unroll
          for (int j = 0; j < 4; ++j) rsum[mb][j] = fmaf(acc[mb][j], vv[j], rsum[mb][j]);
        }
      } else {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            rsum[mb][j] = (MODE == VWO_L2) ? fmaf(acc[mb][j], acc[mb][j], rsum[mb][j]) : rsum[mb][j] + fabsf(acc[mb][j]);
      }
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
          if (MODE != VWO_L1) x = sqrtf(fmaxf(x, 0.f));
          cacc[mb][j] += ahs[h][64 * wv + 16 * mb + 4 * gq + j] * x;
          rsum[mb][j] = 0.f;
        }
    }
    if (T + 1 < total) store_tile(nxt, wt[(T + 1) & 1]);
    lds_barrier();     // tile T+1 in LDS; slot T & 1 free
    if (T + 3 < total) load_tile(nxt, T + 3);
  };
  using K0 = std::integral_constant<int, 0>;
  if (MODE == VWO_GRAM) {
    // four tiles per head (ntiles == 4): the k-step of tile T is T % 4
    for (int T = 0; T < total; T += 4) {
      step(T, rb, K0{});
      step(T + 1, ra, std::integral_constant<int, 1>{});
      step(T + 2, rb, std::integral_constant<int, 2>{});
      step(T + 3, ra, std::integral_constant<int, 3>{});
    }
  } else {
    for (int T = 0; T < total; T += 2) {
      step(T, rb, K0{});
      if (T + 1 < total) step(T + 1, ra, K0{});
    }
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

// Gram partials: part[i][s] = sum over hidden rows c of slice s of
// x_c x_c^T, x_c = w_o[c, i*d .. i*d + d) (row c of the nn.Linear weight
// restricted to head i), as fp32 on 16x16x32 bf16 MFMA.  Slices are staged
// through LDS transposed ([e][c], 32 rows of c per step) so both operands
// read 8 consecutive c per lane; 16-byte chunk ch of row e sits at position
// ch ^ ((e >> 4) & 3), so one transposed store instruction (rows 8k + q of 16
// chunks k) touches 8 bank groups instead of 1, and the 16 rows of one operand
// read keep one swizzle (reads stay conflict-free with the 80-byte pitch).
// Wave w computes output row blocks 2w, 2w+1.  The loads of GDEPTH steps are in flight at once (one workgroup per CU, so
// the slice streams at the rate of many outstanding loads, not of one
// round trip per step), and the barrier leaves them in flight.
constexpr int GSTEP = 32;                  // hidden rows per step
constexpr int GDEPTH = 4;                  // steps of loads in flight
__global__ __launch_bounds__(256) void gram_kernel(const uint16_t* __restrict__ w_o, float* __restrict__ part,
                                                   int hq, int hidden, int nslice) {
  __shared__ __align__(16) uint16_t t[2][D][GSTEP + 8];   // padded rows
  const int i = blockIdx.x, sl = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int gq = lane >> 4, c = lane & 15;
  const size_t wrow = (size_t)hq * D;
  const int per = hidden / nslice;
  const int c0 = sl * per;
  f32x4 acc[2][8];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = zero4();
  // each thread moves 2 chunks of 8 columns per step: rows c (32) x 16 chunks
  auto load = [&](u32x4 (&r)[2], int step) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = threadIdx.x + 256 * q, rr = idx >> 4, ch = idx & 15;
      r[q] = ld16(w_o + (size_t)(c0 + step * GSTEP + rr) * wrow + (size_t)i * D + ch * 8);
    }
  };
  auto store = [&](const u32x4 (&r)[2], int buf) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = threadIdx.x + 256 * q, rr = idx >> 4, ch = idx & 15;
      const int col = (((rr >> 3) ^ ((ch >> 1) & 3)) << 3) + (rr & 7);   // rows ch*8.. share e >> 4 = ch >> 1
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        t[buf][ch * 8 + 2 * j][col] = (uint16_t)(r[q][j] & 0xffffu);
        t[buf][ch * 8 + 2 * j + 1][col] = (uint16_t)(r[q][j] >> 16);
      }
    }
  };
  const int nsteps = per / GSTEP;
  // rg[j] holds the loads of steps j, j + GDEPTH, j + 2 GDEPTH, ... in turn
  u32x4 rg[GDEPTH][2];
#pragma unroll
  for (int j = 0; j < GDEPTH; ++j)
    if (j < nsteps) load(rg[j], j);
  store(rg[0], 0);
  if (GDEPTH < nsteps) load(rg[0], GDEPTH);
  lds_barrier();
  for (int s0 = 0; s0 < nsteps; s0 += GDEPTH) {
#pragma unroll
    for (int k = 0; k < GDEPTH; ++k) {
      const int s = s0 + k;
      if (s < nsteps) {
        // step s + 1 into the other buffer (its readers, step s - 1, are past
        // the last barrier), then its registers take step s + 1 + GDEPTH
        if (s + 1 < nsteps) {
          store(rg[(k + 1) % GDEPTH], (s + 1) & 1);
          if (s + 1 + GDEPTH < nsteps) load(rg[(k + 1) % GDEPTH], s + 1 + GDEPTH);
        }
        const int buf = s & 1;
        bf16x8 aop[2], bop[8];
#pragma unroll
        for (int a = 0; a < 2; ++a)
          aop[a] = *reinterpret_cast<const bf16x8*>(&t[buf][16 * (2 * wv + a) + c][8 * (gq ^ ((2 * wv + a) & 3))]);
#pragma unroll
        for (int b = 0; b < 8; ++b) bop[b] = *reinterpret_cast<const bf16x8*>(&t[buf][16 * b + c][8 * (gq ^ (b & 3))]);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 8; ++b) acc[a][b] = Mma<uint16_t>::mma(aop[a], bop[b], acc[a][b]);
        lds_barrier();
      }
    }
  }
  float* out = part + ((size_t)i * nslice + sl) * D * D;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) out[(size_t)(16 * (2 * wv + a) + 4 * gq + j) * D + 16 * b + c] = acc[a][b][j];
}

// bf16 bit pattern of x, round to nearest even (x finite)
__device__ __forceinline__ uint16_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// M_i = sum of the slice partials in fp64 (fixed order); M'_i (M_i doubled
// where e lies in an earlier 32-block than c, zero in a later one: the same
// v M' v^T) written as two bf16 planes in the layout of a projection:
// fac[p*d + c][i*d + e] = plane p of M'_i[c][e]; scaling by 2 is exact in
// both planes.
__global__ __launch_bounds__(256) void gram_planes_kernel(const float* __restrict__ part, int hq, int nslice,
                                                          uint16_t* __restrict__ fac) {
  const int i = blockIdx.y;
  const int idx = blockIdx.x * 256 + (int)threadIdx.x;   // c * D + e, grid covers D * D exactly
  const int c = idx / D, e = idx % D;
  const float* pi = part + (size_t)i * nslice * D * D;
  float v[8];
#pragma unroll
  for (int sl = 0; sl < 8; ++sl) v[sl] = (sl < nslice) ? pi[(size_t)sl * D * D + idx] : 0.f;
  double m = 0.0;
#pragma unroll
  for (int sl = 0; sl < 8; ++sl) m += (double)v[sl];
  if ((e >> 5) < (c >> 5)) m *= 2.0;
  else if ((e >> 5) > (c >> 5)) m = 0.0;
  const uint16_t hi = bf16_rne((float)m);
  const uint16_t lo = bf16_rne((float)(m - (double)__uint_as_float((uint32_t)hi << 16)));
  const size_t wrow = (size_t)hq * D;
  fac[(size_t)c * wrow + (size_t)i * D + e] = hi;
  fac[(size_t)(D + c) * wrow + (size_t)i * D + e] = lo;
}

}  // namespace

size_t factor_ws_bytes(const Geo& g) {
  if (!use_factor(g)) return 0;
  return align_up((size_t)g.hq * factor_slices(g) * D * D * sizeof(float), 256) +
         align_up((size_t)2 * D * g.hq * D * sizeof(uint16_t), 256);
}

hipError_t launch_factor(const Geo& g, const void* w_o, char* ws, hipStream_t st) {
  float* part = reinterpret_cast<float*>(ws);
  uint16_t* fac = reinterpret_cast<uint16_t*>(ws + align_up((size_t)g.hq * factor_slices(g) * D * D * sizeof(float), 256));
  const int ns = factor_slices(g);
  gram_kernel<<<dim3(g.hq, ns), 256, 0, st>>>(static_cast<const uint16_t*>(w_o), part, g.hq, g.hidden, ns);
  gram_planes_kernel<<<dim3(D * D / 256, g.hq), 256, 0, st>>>(part, g.hq, ns, fac);
  return hipGetLastError();
}

hipError_t launch_vwo(const Geo& g, int inst0, int ni, const void* v, const void* w_o, const float* head_scores,
                      float* score2, bool factor, hipStream_t st) {
  if (g.dtype != ADAKV_BF16 || g.d != D || g.hidden % TROWS_W != 0 || g.G > MAXG) return hipErrorInvalidValue;
  dim3 grid((g.p + KEYS - 1) / KEYS, g.hkv, ni);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  const uint16_t* ww = static_cast<const uint16_t*>(w_o);
  if (g.scorer == ADAKV_SCORE_LAPROX && factor)
    vwo_norm_kernel<VWO_GRAM><<<grid, 256, 0, st>>>(vv, ww, head_scores, score2, inst0, g.hq, g.hkv, g.G, g.n, g.p, D,
                                                    g.eps);
  else if (g.scorer == ADAKV_SCORE_LAPROX)
    vwo_norm_kernel<VWO_L2><<<grid, 256, 0, st>>>(vv, ww, head_scores, score2, inst0, g.hq, g.hkv, g.G, g.n, g.p,
                                                  g.hidden, g.eps);
  else
    vwo_norm_kernel<VWO_L1><<<grid, 256, 0, st>>>(vv, ww, head_scores, score2, inst0, g.hq, g.hkv, g.G, g.n, g.p,
                                                  g.hidden, g.eps);
  return hipGetLastError();
}

}  // namespace adakv
