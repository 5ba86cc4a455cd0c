// Observation-window scoring on gfx950.
//
// Pass 1: per window row, the softmax normaliser over the row's key domain, as
// (reference, sum of exp) partials over key chunks.  Pass 2: the pooled,
// normalised weights reduced to one score per key.  Both passes form Q_win K^T
// with 16x16x32 MFMA tiles, keys on the M side and window rows on the N side,
// the A rows permuted so that every lane ends up with consecutive keys of one
// window row (the max pooling is a register-local sliding maximum) and row sums
// over a lane group done with DPP lane moves on the vector unit.  Two layouts:
//  * register-K (kr_stats_kernel, kr_emit_kernel; bf16, d = 128, w <= 32):
//    the window queries of the KV head's G query heads stay in LDS, and every
//    wave streams its own 64-key blocks of K straight into its A-operand
//    registers, so no K tile is staged through LDS and no barrier follows the
//    prologue; a wave covers all G*w rows of its keys, so its row sums need one
//    lane butterfly per block.  LAVa's pass 2 on this layout (kr_lava_kernel)
//    swaps the MFMA operands so a lane holds four rows of one key, writes the
//    unpooled group maxima, and lava_pool_kernel pools them (LAVa pools the
//    final vector, so no pooling halo is computed);
//  * LDS-tiled (score_stats_kernel, score_emit_kernel; every other geometry,
//    CriticalKV's emit pass, LAVa's for one instance, small calls): 128-key K
//    tiles staged through LDS, each wave one query head with its rows'
//    operands in registers.
//
// Definitions followed:
//  * Ada-KV notes, Algorithm 2 ("Ada-KV Integration") steps 2-4: softmax of the
//    window queries against the cache outside the window, max pooling of every
//    row, mean over the rows; GQA groups average their query heads ("与分组查询
//    注意力（GQA）的兼容性").  Logits carry the 1/sqrt(d_h) of the Ada-KV paper,
//    Section 3.1, footnote 5.
//  * LAVa notes, Definition 1, "适配GQA架构" and "实验环境": causal window rows,
//    row weights summed, group maximum, times max_k ||V[k]||_1 / w, max pooled.
//  * CriticalKV notes, "作为通用插件融入现有驱逐流水线": the per-query-head Ada-KV
//    score is kept for the composite score.
//  * LaProx page, Section 4.1, Algorithm 1: every window row softmaxed over all
//    n keys (no mask, as printed); per head and prefix key the sum over the rows
//    of the squared weights, whose square root is ||A[:, t]||_2 (the value
//    factor ||(V W_O)[t, :]||_2 and the product come from the V W^O kernel).
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace adakv {
namespace {

constexpr int TILE = 128;          // keys per tile (8 M-blocks of 16)
constexpr int HALO = 4;            // extra keys on each side of an emit tile
constexpr int TROWS = TILE + 2 * HALO;

template <typename T, int D>
struct Lay {
  static constexpr int ROWB = D * (int)sizeof(T);
  static constexpr int STRIDE = ROWB;                // LDS row pitch (chunks swizzled, no padding)
  static constexpr int RP = ROWB >= 256 ? 1 : 256 / ROWB;   // rows per 256 bytes
  static constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
  static constexpr int EPC = 16 / (int)sizeof(T);    // elements per chunk
  static constexpr int KSTEPS = D / Mma<T>::KSTEP;
};

// LDS row of key offset koff in [0, TILE).  M-row m of M-block mb holds key
// 32*(m/4) + 4*mb + (m%4) (so every lane of the MFMA result owns 32
// consecutive keys); it is stored at LDS row 16*mb + m, so the lanes of one
// A-operand read touch 16 consecutive rows (no bank conflicts with the odd
// 16-byte row pitch).  Halo keys take rows TILE .. TILE+7.
__device__ __forceinline__ int tile_row(int koff) {
  if (koff < 0) return TILE + (koff + HALO);
  if (koff >= TILE) return TILE + HALO + (koff - TILE);
  return (((koff >> 2) & 7) << 4) | ((koff >> 5) << 2) | (koff & 3);
}

// LDS row read by lane m (= lane % 16) of M-block mb.  The halo block
// (mb == 8) holds keys -4..-1 in lane group 0 and TILE..TILE+3 in lane group 3
// (groups 1, 2 read duplicates).
__device__ __forceinline__ int a_row(int mb, int m) {
  if (mb < 8) return 16 * mb + m;
  return ((m >> 2) == 3) ? TILE + HALO + (m & 3) : TILE + (m & 3);
}

// 16-byte chunk ch of LDS row R is stored at position ch ^ swz(R): the 16 rows
// of one MFMA operand read (same logical chunk) fall in 16 distinct bank groups.
template <typename T, int D>
__device__ __forceinline__ int swz(int R) {
  using L = Lay<T, D>;
  return (R / L::RP) & (L::CPR - 1);
}

// Address of the A operand of M-block mb, k-step ks for lane (m = c, group gq).
template <typename T, int D>
__device__ __forceinline__ const T* a_ptr(const char* lds, int mb, int ks, int c, int gq) {
  using L = Lay<T, D>;
  using M = Mma<T>;
  const int R = a_row(mb, c);
  const int eb = (ks * M::KSTEP + M::KPL * gq) * (int)sizeof(T);   // byte offset in the row
  return reinterpret_cast<const T*>(lds + R * L::STRIDE + (((eb >> 4) ^ swz<T, D>(R)) << 4) + (eb & 15));
}

// K tile staging in two halves so the global loads of tile t+1 are in
// flight while tile t is multiplied: load() fills registers, store() moves
// them to LDS.  K is streamed (the second pass re-reads it from HBM), so the
// loads are nontemporal.  Keys [k0 + KLO, k0 + KHI) of one head; keys outside [0, n)
// become zero rows.  The per-thread chunk -> (source offset, LDS row) map is
// the same for every tile and is computed once.  Needs >= 256 threads.
template <typename T, int D, int KLO, int KHI>
struct TileRegs {
  using L = Lay<T, D>;
  static constexpr int CHUNKS = (KHI - KLO) * L::CPR;
  static constexpr int PER = (CHUNKS + 255) / 256;
  u32x4 r[PER];
  int src[PER];   // element offset from row k0 (key offset * D + chunk column)
  int dst[PER];   // LDS byte offset, -1 when this thread has no chunk
  int kof[PER];   // key offset of the chunk
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = threadIdx.x + i * (int)blockDim.x;
      const int koff = KLO + idx / L::CPR, ch = idx % L::CPR;
      kof[i] = koff;
      src[i] = koff * D + ch * L::EPC;
      const int R = (idx < CHUNKS) ? tile_row(koff) : 0;
      dst[i] = (idx < CHUNKS) ? R * L::STRIDE + ((ch ^ swz<T, D>(R)) * 16) : -1;
    }
  }
  __device__ __forceinline__ void load(const T* kb, int n, int k0) {
    const T* base = kb + (ptrdiff_t)k0 * D;
    if (k0 + KLO >= 0 && k0 + KHI <= n) {
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (dst[i] >= 0) r[i] = ld16_nt(base + src[i]);
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int key = k0 + kof[i];
        u32x4 v = {0u, 0u, 0u, 0u};
        if (dst[i] >= 0 && key >= 0 && key < n) v = ld16_nt(base + src[i]);
        r[i] = v;
      }
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (dst[i] >= 0) st16(lds + dst[i], r[i]);
  }
};

// Row statistics live in the base-2 domain: m is the row maximum times
// log2(e)/sqrt(d) (one rounding), and every weight is exp2(fma(z, c2, -m)).
// Both passes use the same rounded m, so its rounding error is a common
// factor of a row's weights and its sum and cancels in the normalised weight.
__device__ __forceinline__ void merge_ml(float& m, float& l, float m2, float l2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  l = l * fast_exp2(m - M) + l2 * fast_exp2(m2 - M);
  m = M;
}

// The partial row statistics of a launch merged once per window row: part
// holds nsub (max, sum) pairs per row, [instance][KV head][partial][G*w];
// merged gets one per row, [instance][KV head][G*w], formed in partial order.
// Calls that split a head over many chunks (one long instance) run it before
// pass 2, whose every workgroup would otherwise merge all nsub pairs of its
// rows in its prologue.
constexpr int MERGE_MIN = 64;   // partials per row above which the merge runs on its own
// One wave per row: lane L merges partials L, L+64, ... in order, then a
// butterfly over the 64 lanes (a fixed order, the same on every run).
__global__ __launch_bounds__(256) void merge_part_kernel(const float2* __restrict__ part, float2* __restrict__ merged,
                                                         int rows, int Gw, int nsub) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= rows) return;                          // uniform across the wave
  const int head = t / Gw, j = t - head * Gw;
  const float2* pr = part + (size_t)head * nsub * Gw + j;
  float m = -INFINITY, l = 0.f;
  for (int c0 = lane; c0 < nsub; c0 += 4 * WAVE) {
    float2 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + u * WAVE;
      v[u] = c < nsub ? pr[(size_t)c * Gw] : make_float2(-INFINITY, 0.f);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) merge_ml(m, l, v[u].x, v[u].y);
  }
#pragma unroll
  for (int mask = 1; mask < WAVE; mask <<= 1) {
    const float om = shfl_xor(m, mask), ol = shfl_xor(l, mask);
    merge_ml(m, l, om, ol);
  }
  if (lane == 0) merged[t] = make_float2(m, l);
}

// Sum 32 per-lane values across the 16 lanes of a lane group (lanes sharing
// lane/16); afterwards lane c of the group holds the totals of entries 2c, 2c+1.
// A butterfly of four DPP involutions (mirror, half mirror, quad ^2, quad ^1):
// at each step a lane keeps the half of its entries selected by one bit of c
// and adds its partner's copy of that half.
template <int CTRL, int HALF>
__device__ __forceinline__ void rs_step(const float* in, float* out, bool upper) {
#pragma unroll
  for (int i = 0; i < HALF; ++i) {
    const float send = upper ? in[i] : in[i + HALF];
    const float keep = upper ? in[i + HALF] : in[i];
    out[i] = keep + dpp<CTRL>(send);
  }
}
__device__ __forceinline__ void reduce_scatter16(float (&x)[32], int c, float& o0, float& o1) {
  float y[16], z[8], u[4], t[2];
  rs_step<DPP_MIRROR, 16>(x, y, (c >> 3) & 1);
  rs_step<DPP_HALF_MIRROR, 8>(y, z, (c >> 2) & 1);
  rs_step<DPP_XOR2, 4>(z, u, (c >> 1) & 1);
  rs_step<DPP_XOR1, 2>(u, t, c & 1);
  o0 = t[0];
  o1 = t[1];
}

__device__ __forceinline__ float allsum16(float x) {
  x += dpp<DPP_MIRROR>(x);
  x += dpp<DPP_HALF_MIRROR>(x);
  x += dpp<DPP_XOR2>(x);
  x += dpp<DPP_XOR1>(x);
  return x;
}

// Logits of M-block mb for the NB window-row blocks: Q_win K^T with the head
// dimension split into parts accumulated separately and added at the end.
// The matrix units round their running sum every few products; with one
// accumulator, the error of a logit of magnitude ~600 (a head with temperature
// 0.1) reaches ~1e-4, which moves a softmax weight by ~1e-5 relative.  Two
// half-length sums halve the magnitude the rounding works at.  fp32 inputs run
// 4-product steps (16 of them for d = 64), so they take four quarter-length
// sums, added pairwise.
template <typename T, int D, int NB>
__device__ __forceinline__ void logits_block(const char* lds, int mb, int c, int gq,
                                             const typename Mma<T>::op_t (&qop)[NB][Lay<T, D>::KSTEPS],
                                             f32x4 (&out)[NB]) {
  using L = Lay<T, D>;
  using M = Mma<T>;
  constexpr int NPART = (sizeof(T) == 4 && L::KSTEPS >= 4) ? 4 : 2;
  constexpr int PER = L::KSTEPS / NPART;
  f32x4 part[NPART][NB];
#pragma unroll
  for (int i = 0; i < NPART; ++i)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) part[i][nb] = zero4();
#pragma unroll
  for (int ks = 0; ks < L::KSTEPS; ++ks) {
    const typename M::op_t a = M::load(a_ptr<T, D>(lds, mb, ks, c, gq));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) part[ks / PER][nb] = M::mma(a, qop[nb][ks], part[ks / PER][nb]);
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (NPART == 4) out[nb][j] = (part[0][nb][j] + part[1][nb][j]) + (part[2][nb][j] + part[3][nb][j]);
      else out[nb][j] = part[0][nb][j] + part[1][nb][j];
    }
}

// ---------------------------------------------------------------- pass 1
// Workgroup = max(G, 4) waves; wave h < G owns query head g*G + h (its w window
// rows on the N side, NB blocks of 16); the others only help load K.
template <typename T, int D, int NB, bool CAUSAL>
__global__ __launch_bounds__(512) void score_stats_kernel(
    const T* __restrict__ q, const T* __restrict__ k, float2* __restrict__ part, int inst0, int hq,
    int hkv, int G, int n, int w, int p, int kend, int nchunk, int keys_per_wg, float c2) {
  using L = Lay<T, D>;
  using M = Mma<T>;
  extern __shared__ __align__(16) char lds[];
  const int chunk = blockIdx.x, g = blockIdx.y, il = blockIdx.z, inst = inst0 + il;
  const int lane = threadIdx.x & 63, h = threadIdx.x >> 6;
  const int gq = lane >> 4, c = lane & 15;
  const bool active = h < G;
  const T* kb = k + ((size_t)inst * hkv + g) * (size_t)n * D;
  const T* qb = q + ((size_t)inst * hq + (size_t)g * G + (active ? h : 0)) * (size_t)w * D;

  typename M::op_t qop[NB][L::KSTEPS];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int r = 16 * nb + c;
#pragma unroll
    for (int ks = 0; ks < L::KSTEPS; ++ks)
      qop[nb][ks] = (active && r < w) ? M::load(qb + (size_t)r * D + ks * M::KSTEP + M::KPL * gq) : M::zero();
  }
  float rm[NB], rl[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) { rm[nb] = -INFINITY; rl[nb] = 0.f; }

  const int kbeg = chunk * keys_per_wg;
  const int kfin = min(kbeg + keys_per_wg, kend);
  TileRegs<T, D, 0, TILE> tr;
  tr.init();
  tr.load(kb, n, kbeg);
  for (int k0 = kbeg; k0 < kfin; k0 += TILE) {
    __syncthreads();
    tr.store(lds);
    __syncthreads();
    if (k0 + TILE < kfin) tr.load(kb, n, k0 + TILE);     // next tile in flight
    if (!active) continue;
    f32x4 acc[8][NB];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) logits_block<T, D, NB>(lds, mb, c, gq, qop, acc[mb]);
    // every key of the tile inside every row's domain: no per-key test (and a
    // finite row maximum); one copy of the fold per value of the test
    const bool full = k0 + TILE - 1 <= (CAUSAL ? min(kend - 1, p) : kend - 1);
    auto fold = [&](auto full_tag) {
      constexpr bool FULL = decltype(full_tag)::value;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int r = 16 * nb + c;
        const int lim = CAUSAL ? min(kend - 1, p + r) : kend - 1;   // last key of this row's domain
        float lm = -INFINITY;
        if (FULL) {
#pragma unroll
          for (int mb = 0; mb < 8; ++mb)
            lm = fmax3(lm, fmax3(acc[mb][nb][0], acc[mb][nb][1], acc[mb][nb][2]), acc[mb][nb][3]);
        } else {
#pragma unroll
          for (int mb = 0; mb < 8; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (k0 + 32 * gq + 4 * mb + j <= lim) lm = fmaxf(lm, acc[mb][nb][j]);
        }
        if (FULL || lm != -INFINITY) {
          const float lmc = lm * c2;
          float ls = 0.f;
          if (FULL) {
#pragma unroll
            for (int mb = 0; mb < 8; ++mb)
#pragma unroll
              for (int j = 0; j < 4; ++j) ls += fast_exp2(fmaf(acc[mb][nb][j], c2, -lmc));
          } else {
#pragma unroll
            for (int mb = 0; mb < 8; ++mb)
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const float e = fast_exp2(fmaf(acc[mb][nb][j], c2, -lmc));
                ls += (k0 + 32 * gq + 4 * mb + j <= lim) ? e : 0.f;
              }
          }
          merge_ml(rm[nb], rl[nb], lmc, ls);
        }
      }
    };
    if (full) fold(std::true_type{});
    else fold(std::false_type{});
  }
  if (!active) return;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int mask = 16; mask <= 32; mask <<= 1) {
      const float om = shfl_xor(rm[nb], mask), ol = shfl_xor(rl[nb], mask);
      merge_ml(rm[nb], rl[nb], om, ol);
    }
    const int r = 16 * nb + c;
    if (gq == 0 && r < w)
      part[(((size_t)il * hkv + g) * nchunk + chunk) * (size_t)(G * w) + h * w + r] = make_float2(rm[nb], rl[nb]);
  }
}

// ---------------------------------------------------------------- register-K path
// bf16 keys, d = 128, G query heads of w <= 32 rows per KV head.  The window
// queries of the workgroup's KV head sit in LDS for its whole life (the B
// operand, read 16 bytes per lane per k-step); every wave streams its own
// 64-key blocks of K from global memory straight into the A-operand registers.
// No K tile goes through LDS and no barrier follows the prologue, so the
// waves of a CU drift apart and hide each other's load latency.  The MFMA
// inputs and their order (two half-length accumulations of the head
// dimension, added at the end) are those of logits_block, so the logits are
// bit-identical to the LDS-tiled kernels'.
constexpr int KB = 64;          // keys per block: 4 M-blocks
constexpr int KR_WAVES = 4;     // waves per workgroup
constexpr int KR_QROWB = 256;   // bytes per query row in LDS (d = 128 bf16)

// M-row m of M-block mb holds block key 16*(m/4) + 4*mb + (m%4): lane group gq
// of the result owns the 16 consecutive keys 16*gq .. 16*gq + 15.
__device__ __forceinline__ int kr_key(int mb, int m) { return 16 * (m >> 2) + 4 * mb + (m & 3); }

// LDS row R = 16*nb + c (nb over the G heads' NBW blocks of 16 window rows,
// rows past w zero); 16-byte chunk ch of row R at position ch ^ (R % 16), so
// the 16 rows of one B-operand read fall in 16 distinct bank groups.
template <int G, int NBW>
__device__ __forceinline__ void kr_stage_q(char* lds, const uint16_t* q, int inst, int hq, int g, int w) {
  constexpr int ROWS = G * NBW * 16;
  for (int idx = threadIdx.x; idx < ROWS * 16; idx += blockDim.x) {
    const int R = idx >> 4, ch = idx & 15;
    const int h = R / (NBW * 16), r = R % (NBW * 16);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < w) v = ld16(q + (((size_t)inst * hq + (size_t)g * G + h) * w + r) * 128 + ch * 8);
    st16(lds + R * KR_QROWB + ((ch ^ (R & 15)) << 4), v);
  }
}

// Per-lane byte offsets of the B operand of k-step ks (window-row block 0);
// block nb adds the constant 4096*nb.
__device__ __forceinline__ int kr_qoff(int ks, int c, int gq) { return c * KR_QROWB + (((4 * ks + gq) ^ c) << 4); }

// A operands of M-blocks [0, NMB) of the block starting at key kb0: [mb][ks],
// lane (c, gq) holds elements 32*ks + 8*gq .. +8 of key row kb0 + key(mb, c)
// (koff[mb] = byte offset of that row relative to kb0, plus 16*gq).  Buffer
// loads whose whole offset is per lane, so the hardware range check covers it:
// rows outside the head's n keys (past the end, or before key 0: the offset
// wraps to a huge value) read as zeros, masked by the caller.
template <int NMB>
__device__ __forceinline__ void kr_load(bf16x8 (&kf)[NMB][4], __amdgpu_buffer_rsrc_t rs, const int (&koff)[NMB], int kb0) {
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    const int off = koff[mb] + kb0 * KR_QROWB;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      kf[mb][ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 64 * ks, 0, 0));
  }
}

// Logits of M-block mb against the window-row block whose operands are qo.
template <int NMB>
__device__ __forceinline__ f32x4 kr_logits(const bf16x8 (&kf)[NMB][4], int mb, const bf16x8 (&qo)[4]) {
  f32x4 p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[mb][0], qo[0], zero4(), 0, 0, 0);
  f32x4 p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[mb][2], qo[2], zero4(), 0, 0, 0);
  p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[mb][1], qo[1], p0, 0, 0, 0);
  p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[mb][3], qo[3], p1, 0, 0, 0);
  f32x4 z;
#pragma unroll
  for (int j = 0; j < 4; ++j) z[j] = p0[j] + p1[j];
  return z;
}

// Pass 1 on the register-K path: the workgroup covers keys [chunk*kpw,
// +kpw) of one KV head, wave v its blocks v, v+4, ... (kpw a multiple of
// 4*KB).  Per window row each lane sums exp2(z*c2 - m) over its keys against a
// reference m fixed at its first block (the largest scaled logit there), so a
// block costs one FMA, one exp and one add per logit and no maximum.  Only
// when a block's sum leaves the safe range (a logit more than 2^6 above the
// reference, or the first block, whose reference is still -inf) does the lane
// take the maximum of the block, raise m and rescale its sum.  Every wave
// writes its own partial per row: sub-chunk chunk*4 + wave.
template <int G, int NBW, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void kr_stats_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                      float2* __restrict__ part, int inst0, int hq, int hkv, int n,
                                                      int w, int p, int kend, int nsub, int kpw, float c2) {
  constexpr int NBT = G * NBW;
  extern __shared__ __align__(16) char lds[];
  const int chunk = blockIdx.x, g = blockIdx.y, il = blockIdx.z, inst = inst0 + il;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: block offsets stay scalar
  const int gq = lane >> 4, c = lane & 15;
  kr_stage_q<G, NBW>(lds, q, inst, hq, g, w);
  __syncthreads();
  const uint16_t* kh = k + ((size_t)inst * hkv + g) * (size_t)n * 128;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kh), 0, n * KR_QROWB, 0x00020000);
  int koff[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) koff[mb] = kr_key(mb, c) * KR_QROWB + 16 * gq;
  int qoff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qoff[ks] = kr_qoff(ks, c, gq);

  float rm[NBT], rl[NBT];
#pragma unroll
  for (int nb = 0; nb < NBT; ++nb) { rm[nb] = -INFINITY; rl[nb] = 0.f; }
  const int c0 = chunk * kpw, c1 = min(c0 + kpw, kend);
  const int full_end = CAUSAL ? min(kend - 1, p) : kend - 1;   // last key inside every row's domain
  auto block = [&](const bf16x8 (&kf)[4][4], int b0) {
    const int kl = b0 + 16 * gq;   // first key of this lane's 16
    auto fold = [&](auto full_tag) {
      constexpr bool FULL = decltype(full_tag)::value;
#pragma unroll
      for (int nb = 0; nb < NBT; ++nb) {
        bf16x8 qo[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qo[ks] = *reinterpret_cast<const bf16x8*>(lds + qoff[ks] + 4096 * nb);
        f32x4 z[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) z[mb] = kr_logits(kf, mb, qo);
        const int r = (nb % NBW) * 16 + c;
        const int lim = CAUSAL ? min(kend - 1, p + r) : kend - 1;
        auto sum = [&](float mref) {
          float ls = 0.f;
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float e = fast_exp2(fmaf(z[mb][j], c2, -mref));
              if (FULL) ls += e;
              else ls += (kl + 4 * mb + j <= lim) ? e : 0.f;
            }
          return ls;
        };
        float ls = sum(rm[nb]);
        // first block, a much larger logit, or (invalid input) NaN; taken by the
        // whole wave (a lane whose reference stands recomputes the same sum)
        if (__builtin_amdgcn_ballot_w64(!(ls < 0x1p64f)) != 0) {
          float lm = -INFINITY;
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (FULL || kl + 4 * mb + j <= lim) lm = fmaxf(lm, z[mb][j]);
          const float lmc = lm * c2;
          if (lmc > rm[nb]) {
            rl[nb] *= fast_exp2(rm[nb] - lmc);   // exp2(-inf) = 0 at the first block
            rm[nb] = lmc;
          }
          ls = (lm == -INFINITY) ? 0.f : sum(rm[nb]);
        }
        rl[nb] += ls;
      }
    };
    if (b0 + KB - 1 <= full_end) fold(std::true_type{});
    else fold(std::false_type{});
  };
  // Two register sets: the next block's loads are in flight while a block is
  // folded.  The loads are unconditional (past the wave's last block they
  // re-read its current block, an L2 hit) so the waits stay exact.
  int b0 = c0 + wv * KB;
  if (b0 < c1) {
    bf16x8 ka[4][4], kb[4][4];
    kr_load(ka, rs, koff, b0);
    while (true) {
      int b1 = b0 + KR_WAVES * KB;
      bool more = b1 < c1;
      kr_load(kb, rs, koff, more ? b1 : b0);
      block(ka, b0);
      if (!more) break;
      b0 = b1;
      b1 = b0 + KR_WAVES * KB;
      more = b1 < c1;
      kr_load(ka, rs, koff, more ? b1 : b0);
      block(kb, b0);
      if (!more) break;
      b0 = b1;
    }
  }
  const int Gw = G * w;
#pragma unroll
  for (int nb = 0; nb < NBT; ++nb) {
#pragma unroll
    for (int mask = 16; mask <= 32; mask <<= 1) {
      const float om = shfl_xor(rm[nb], mask), ol = shfl_xor(rl[nb], mask);
      merge_ml(rm[nb], rl[nb], om, ol);
    }
    const int h = nb / NBW, r = (nb % NBW) * 16 + c;
    if (gq == 0 && r < w)
      part[(((size_t)il * hkv + g) * nsub + (size_t)chunk * KR_WAVES + wv) * (size_t)Gw + h * w + r] =
          make_float2(rm[nb], rl[nb]);
  }
}

// Sum 16 per-lane values over the 16 lanes of each lane group; afterwards lane
// c holds the total of entry c.  The butterfly of reduce_scatter16, one step
// shorter.
__device__ __forceinline__ float reduce16(const float (&x)[16], int c) {
  float z[8], u[4], t[2], o[1];
  rs_step<DPP_MIRROR, 8>(x, z, (c >> 3) & 1);
  rs_step<DPP_HALF_MIRROR, 4>(z, u, (c >> 2) & 1);
  rs_step<DPP_XOR2, 2>(u, t, (c >> 1) & 1);
  rs_step<DPP_XOR1, 1>(t, o, c & 1);
  return o[0];
}

// Pass 2 on the register-K path, SnapKV / Ada-KV scores of prefix keys (no
// per-head output).  The workgroup covers keys [chunk*kpw, +kpw) of one KV
// head, wave v its 64-key blocks v, v+4, ...  For every window-row block the
// lane holds the logits of its 16 consecutive keys (M-blocks 0-3); a fifth
// M-block gives the pooling halo of the block's two ends (keys b0-4 .. b0-1
// and b0+64 .. b0+67), and every lane group takes its 3 + 3 neighbours from
// the adjacent groups by lane moves.  The max pooling runs on the logits (exp is
// increasing), then the normalised weight exp2(z*c2 - m)*(1/l) is added per
// key over all G*w rows of the KV head inside the lane; one butterfly over
// the 16 lanes of a group per block finishes the sum, which is the mean over
// rows and query heads once divided by G*w.
template <int G, int NBW, int POOL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void kr_emit_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float2* __restrict__ part,
    const float* __restrict__ row_lse, float* __restrict__ score, int inst0, int hq, int hkv, int n, int w, int p,
    int nsub, int kpw, float c2) {
  constexpr int NBT = G * NBW, RHO = (POOL - 1) / 2;
  constexpr int NMB = RHO > 0 ? 5 : 4;
  constexpr int NX = 16 + 2 * RHO;
  extern __shared__ __align__(16) char lds[];
  const int chunk = blockIdx.x, g = blockIdx.y, il = blockIdx.z, inst = inst0 + il;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gq = lane >> 4, c = lane & 15;
  kr_stage_q<G, NBW>(lds, q, inst, hq, g, w);
  const int Gw = G * w;

  // Row statistics of rows (nb, c), wave v taking blocks nb = v, v+4, ...:
  // the pass-1 partials merged, lane group gq folding partials gq, gq+4, ...
  // in order, then the four groups combined (the same order in every
  // workgroup of the head).  With row_lse given, its value times log2 e split
  // in float64 into hi (the reference) + lo (the factor exp2(-lo)).  Padding
  // rows (r >= w, zero queries) get weight 0.  Kept in LDS after the queries:
  // (reference, 1/sum) per row.
  float2* rstat = reinterpret_cast<float2*>(lds + NBT * 4096);
  for (int nb = wv; nb < NBT; nb += KR_WAVES) {
    const int h = nb / NBW, r = (nb % NBW) * 16 + c;
    const bool ok = r < w;
    float mc = 0.f, il_row = 0.f;
    if (row_lse != nullptr) {
      if (ok) {
        const double x = (double)row_lse[((size_t)inst * hq + (size_t)g * G + h) * w + r] * 1.4426950408889634;
        const float hi = (float)x;
        mc = hi;
        il_row = fast_exp2(-(float)(x - (double)hi));
      }
    } else {
      float m = -INFINITY, l = 0.f;
      if (ok) {
        const float2* pr = part + ((size_t)il * hkv + g) * nsub * (size_t)Gw + h * w + r;
        for (int ch0 = gq; ch0 < nsub; ch0 += 32) {
          float2 v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int ch = ch0 + 4 * u;
            v[u] = ch < nsub ? pr[(size_t)ch * Gw] : make_float2(-INFINITY, 0.f);
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) merge_ml(m, l, v[u].x, v[u].y);
        }
      }
#pragma unroll
      for (int mask = 16; mask <= 32; mask <<= 1) {
        const float om = shfl_xor(m, mask), ol = shfl_xor(l, mask);
        merge_ml(m, l, om, ol);
      }
      mc = ok ? m : 0.f;
      il_row = ok ? 1.0f / l : 0.f;
    }
    if (gq == 0) rstat[nb * 16 + c] = make_float2(mc, il_row);
  }
  __syncthreads();

  const uint16_t* kh = k + ((size_t)inst * hkv + g) * (size_t)n * 128;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kh), 0, n * KR_QROWB, 0x00020000);
  int koff[NMB];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) koff[mb] = kr_key(mb, c) * KR_QROWB + 16 * gq;
  // halo block: M-rows 12-15 (lane group 3 of the result) hold keys b0-4 ..
  // b0-1, the others b0+64 .. b0+67 (used by lane group 0)
  if (NMB == 5) koff[NMB - 1] = (((c >> 2) == 3) ? -4 + (c & 3) : 64 + (c & 3)) * KR_QROWB + 16 * gq;
  int qoff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qoff[ks] = kr_qoff(ks, c, gq);
  const float inv_gw = 1.0f / (float)Gw;
  const int c0 = chunk * kpw, c1 = min(c0 + kpw, p);
  float* out = score + ((size_t)inst * hkv + g) * (size_t)p;

  auto block = [&](const bf16x8 (&kf)[NMB][4], int b0) {
    const int kl = b0 + 16 * gq;   // first key of this lane's 16
    float ks[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) ks[i] = 0.f;
    auto logits = [&](int nb, f32x4 (&z)[NMB]) {
      bf16x8 qo[4];
#pragma unroll
      for (int ks2 = 0; ks2 < 4; ++ks2) qo[ks2] = *reinterpret_cast<const bf16x8*>(lds + qoff[ks2] + 4096 * nb);
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) z[mb] = kr_logits<NMB>(kf, mb, qo);
    };
    auto fold = [&](auto interior_tag) {
      constexpr bool INTERIOR = decltype(interior_tag)::value;
      // software pipeline over the window-row blocks: the MFMAs of block
      // nb + 1 are issued between the vector instructions of block nb (the
      // matrix unit runs while vector instructions issue)
      f32x4 zc[NMB];
      logits(0, zc);
#pragma unroll
      for (int nb = 0; nb < NBT; ++nb) {
        __builtin_amdgcn_sched_barrier(0);
        f32x4 zn[NMB];
        if (nb + 1 < NBT) logits(nb + 1, zn);
        const float2 st = rstat[nb * 16 + c];
        const f32x4 (&z)[NMB] = zc;
        // x[t] <-> key kl - RHO + t; keys outside the prefix -> -inf
        float x[NX];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int j = 0; j < 4; ++j) x[RHO + 4 * mb + j] = z[mb][j];
#pragma unroll
        for (int j = 0; j < RHO; ++j) {
          // lane group gq reads its left halo from group gq - 1 and its right
          // halo from group gq + 1 (mod 4); groups 3 and 0 offer the halo
          // block's keys in place of their own edge keys.  (Selecting after
          // the lane moves instead made the compiler spill.)
          const float yl = (gq == 3) ? z[NMB - 1][4 - RHO + j] : z[(16 - RHO + j) >> 2][(16 - RHO + j) & 3];
          const float yr = (gq == 0) ? z[NMB - 1][j] : z[0][j];
          x[j] = shfl_lane(yl, (lane - 16) & 63);
          x[16 + RHO + j] = shfl_lane(yr, (lane + 16) & 63);
        }
        if (!INTERIOR) {
#pragma unroll
          for (int t = 0; t < NX; ++t) {
            const int key = kl - RHO + t;
            if (key < 0 || key >= p) x[t] = -INFINITY;
          }
        }
        const float mc = st.x, il_row = st.y;
        if (RHO == 3) {
          float a3[NX - 2];
#pragma unroll
          for (int t = 0; t < NX - 2; ++t) a3[t] = fmax3(x[t], x[t + 1], x[t + 2]);
#pragma unroll
          for (int kk = 0; kk < 16; ++kk)
            ks[kk] = fmaf(fast_exp2(fmaf(fmax3(a3[kk], a3[kk + 2], a3[kk + 4]), c2, -mc)), il_row, ks[kk]);
        } else {
#pragma unroll
          for (int kk = 0; kk < 16; ++kk) {
            float pooled = x[kk + RHO];
            if (RHO >= 1) pooled = fmax3(pooled, x[kk + RHO - 1], x[kk + RHO + 1]);
            if (RHO >= 2) pooled = fmax3(pooled, x[kk + RHO - 2], x[kk + RHO + 2]);
            ks[kk] = fmaf(fast_exp2(fmaf(pooled, c2, -mc)), il_row, ks[kk]);
          }
        }
        if (nb + 1 < NBT) {
#pragma unroll
          for (int i = 0; i < NMB * 4; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // six vector instructions
          }
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) zc[mb] = zn[mb];
        }
      }
    };
    if (b0 >= RHO && b0 + KB + RHO <= p) fold(std::true_type{});
    else fold(std::false_type{});
    const float tot = reduce16(ks, c);
    if (kl + c < p) out[kl + c] = tot * inv_gw;
  };
  for (int b0 = c0 + wv * KB; b0 < c1; b0 += KR_WAVES * KB) {
    bf16x8 kf[NMB][4];
    kr_load<NMB>(kf, rs, koff, b0);
    block(kf, b0);
  }
}

// Logits of key block mb against a window-row block with the MFMA operands
// swapped: lane (gq, c) gets rows 4*gq + j (j < 4) of the row block against
// block key kr_key(mb, c).  The products and their order are kr_logits'.
__device__ __forceinline__ f32x4 kr_logits_t(const bf16x8 (&kf)[4][4], int mb, const bf16x8 (&qo)[4]) {
  f32x4 p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qo[0], kf[mb][0], zero4(), 0, 0, 0);
  f32x4 p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qo[2], kf[mb][2], zero4(), 0, 0, 0);
  p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qo[1], kf[mb][1], p0, 0, 0, 0);
  p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qo[3], kf[mb][3], p1, 0, 0, 0);
  f32x4 z;
#pragma unroll
  for (int j = 0; j < 4; ++j) z[j] = p0[j] + p1[j];
  return z;
}

// Pass 2 of LAVa on the register-K path.  LAVa pools the final vector, not
// every row, so no pooling halo is computed here: the kernel writes the
// unpooled group maximum max_i S_i[t] (S_i[t] the sum of head i's causal
// weights of key t over its w rows) for keys t < ke = min(n, p + rho), and
// lava_pool_kernel pools it and applies max_k ||V[k]||_1 / w.  The workgroup
// covers keys [chunk*kpw, +kpw) of one KV head, wave v its 64-key blocks v,
// v+4, ...  With the operands swapped, a lane holds four rows of one key per
// row block, so a head's rows are summed inside the lane and then over the
// four lane groups by two lane moves; one FMA, one exp and one FMA per logit.
template <int G, int NBW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void kr_lava_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float2* __restrict__ part,
    const float* __restrict__ row_lse, float* __restrict__ smax, int inst0, int hq, int hkv, int n, int w, int p,
    int ke, int nsub, int kpw, float c2) {
  constexpr int NBT = G * NBW;
  extern __shared__ __align__(16) char lds[];
  const int chunk = blockIdx.x, g = blockIdx.y, il = blockIdx.z, inst = inst0 + il;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gq = lane >> 4, c = lane & 15;
  kr_stage_q<G, NBW>(lds, q, inst, hq, g, w);
  const int Gw = G * w;

  // Row statistics (reference, 1/sum) of rows (nb, c) in LDS after the
  // queries, merged exactly as in kr_emit_kernel.
  float2* rstat = reinterpret_cast<float2*>(lds + NBT * 4096);
  for (int nb = wv; nb < NBT; nb += KR_WAVES) {
    const int h = nb / NBW, r = (nb % NBW) * 16 + c;
    const bool ok = r < w;
    float mc = 0.f, il_row = 0.f;
    if (row_lse != nullptr) {
      if (ok) {
        const double x = (double)row_lse[((size_t)inst * hq + (size_t)g * G + h) * w + r] * 1.4426950408889634;
        const float hi = (float)x;
        mc = hi;
        il_row = fast_exp2(-(float)(x - (double)hi));
      }
    } else {
      float m = -INFINITY, l = 0.f;
      if (ok) {
        const float2* pr = part + ((size_t)il * hkv + g) * nsub * (size_t)Gw + h * w + r;
        for (int ch0 = gq; ch0 < nsub; ch0 += 32) {
          float2 v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int ch = ch0 + 4 * u;
            v[u] = ch < nsub ? pr[(size_t)ch * Gw] : make_float2(-INFINITY, 0.f);
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) merge_ml(m, l, v[u].x, v[u].y);
        }
      }
#pragma unroll
      for (int mask = 16; mask <= 32; mask <<= 1) {
        const float om = shfl_xor(m, mask), ol = shfl_xor(l, mask);
        merge_ml(m, l, om, ol);
      }
      mc = ok ? m : 0.f;
      il_row = ok ? 1.0f / l : 0.f;
    }
    if (gq == 0) rstat[nb * 16 + c] = make_float2(mc, il_row);
  }
  __syncthreads();

  const uint16_t* kh = k + ((size_t)inst * hkv + g) * (size_t)n * 128;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kh), 0, n * KR_QROWB, 0x00020000);
  int koff[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) koff[mb] = kr_key(mb, c) * KR_QROWB + 16 * gq;
  int qoff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qoff[ks] = kr_qoff(ks, c, gq);
  const int c0 = chunk * kpw, c1 = min(c0 + kpw, ke);
  float* out = smax + ((size_t)il * hkv + g) * (size_t)ke;

  auto block = [&](const bf16x8 (&kf)[4][4], int b0) {
    float acc[G][4];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[h][mb] = 0.f;
    auto logits = [&](int nb, f32x4 (&z)[4]) {
      bf16x8 qo[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qo[ks] = *reinterpret_cast<const bf16x8*>(lds + qoff[ks] + 4096 * nb);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) z[mb] = kr_logits_t(kf, mb, qo);
    };
    auto fold = [&](auto interior_tag) {
      constexpr bool INTERIOR = decltype(interior_tag)::value;
      // software pipeline over the window-row blocks: the MFMAs of block
      // nb + 1 are issued between the vector instructions of block nb
      f32x4 zc[4];
      logits(0, zc);
#pragma unroll
      for (int nb = 0; nb < NBT; ++nb) {
        __builtin_amdgcn_sched_barrier(0);
        f32x4 zn[4];
        if (nb + 1 < NBT) logits(nb + 1, zn);
        const int h = nb / NBW;
        // (reference, 1/sum) of the lane's rows 4*gq + j of block nb
        const f32x4 s01 = *reinterpret_cast<const f32x4*>(rstat + nb * 16 + 4 * gq);
        const f32x4 s23 = *reinterpret_cast<const f32x4*>(rstat + nb * 16 + 4 * gq + 2);
        const float mc[4] = {s01[0], s01[2], s23[0], s23[2]};
        const float ir[4] = {s01[1], s01[3], s23[1], s23[3]};
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int key = b0 + kr_key(mb, c);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float e = fast_exp2(fmaf(zc[mb][j], c2, -mc[j]));
            if (INTERIOR) {
              acc[h][mb] = fmaf(e, ir[j], acc[h][mb]);
            } else {
              const int r = (nb % NBW) * 16 + 4 * gq + j;
              acc[h][mb] += (key <= p + r && key < n) ? e * ir[j] : 0.f;
            }
          }
        }
        if (nb + 1 < NBT) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // four vector instructions
          }
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) zc[mb] = zn[mb];
        }
      }
    };
    // keys below p are inside every row's causal domain (and below n)
    if (b0 + KB <= p) fold(std::true_type{});
    else fold(std::false_type{});
    // each head's sum over its rows: the four lane groups hold rows 4*gq .. 4*gq+3
    // of every block; then the maximum over the group's heads
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      float m = 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float x = acc[h][mb];
        x += shfl_xor(x, 16);
        x += shfl_xor(x, 32);
        m = h == 0 ? x : fmaxf(m, x);
      }
      const int key = b0 + kr_key(mb, c);
      if (gq == 0 && key < ke) out[key] = m;
    }
  };
  for (int b0 = c0 + wv * KB; b0 < c1; b0 += KR_WAVES * KB) {
    bf16x8 kf[4][4];
    kr_load<4>(kf, rs, koff, b0);
    block(kf, b0);
  }
}

// LAVa scores from kr_lava_kernel's group maxima: score[t] = max_k ||V[k]||_1 /
// w times the maximum of smax over keys t - RHO .. t + RHO inside [0, ke), for
// t < p (every group maximum is >= 0, so keys outside the range count as 0).
// A workgroup pools LP_KEYS keys of one KV head from an LDS copy of them and
// their halo; V's norm maximum comes from vbar_kernel's block maxima.
constexpr int LP_KEYS = 2048;
template <int RHO>
__global__ __launch_bounds__(256) void lava_pool_kernel(const float* __restrict__ smax,
                                                        const float* __restrict__ vpart, int nvblk,
                                                        float* __restrict__ score, int inst0, int hkv, int p, int ke,
                                                        int w) {
  const int g = blockIdx.y, il = blockIdx.z, inst = inst0 + il;
  __shared__ float tile[LP_KEYS + 2 * RHO];
  __shared__ float vsc;
  const int t0 = blockIdx.x * LP_KEYS;
  const float* sm = smax + ((size_t)il * hkv + g) * (size_t)ke;
  for (int i = threadIdx.x; i < LP_KEYS + 2 * RHO; i += 256) {
    const int t = t0 - RHO + i;
    tile[i] = (t >= 0 && t < ke) ? sm[t] : 0.f;
  }
  if (threadIdx.x < WAVE) {
    float vb = 0.f;
    for (int b = threadIdx.x; b < nvblk; b += WAVE) vb = fmaxf(vb, vpart[((size_t)inst * hkv + g) * nvblk + b]);
#pragma unroll
    for (int mask = 1; mask < 64; mask <<= 1) vb = fmaxf(vb, shfl_xor(vb, mask));
    if (threadIdx.x == 0) vsc = vb / (float)w;
  }
  __syncthreads();
  float* out = score + ((size_t)inst * hkv + g) * p;
#pragma unroll
  for (int u = 0; u < LP_KEYS / 256; ++u) {
    const int i = u * 256 + threadIdx.x;
    if (t0 + i < p) {
      float m = tile[RHO + i];
#pragma unroll
      for (int o = 1; o <= RHO; ++o) m = fmax3(m, tile[RHO + i - o], tile[RHO + i + o]);
      out[t0 + i] = vsc * m;
    }
  }
}

// ---------------------------------------------------------------- pass 2
// EMIT_SQ: the SNAP path without pooling on squared weights, written per head
// unscaled (sum over rows of A^2).
enum { EMIT_SNAP = 0, EMIT_LAVA = 1, EMIT_SQ = 2 };

template <typename T, int D, int NB, int POOL, int KIND>
__global__ __launch_bounds__(512) void score_emit_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const float2* __restrict__ part,
    const float* __restrict__ row_lse, const float* __restrict__ vpart, int nvblk, float* __restrict__ score,
    float* __restrict__ head_scores, int inst0, int hq, int hkv, int G, int n, int w, int p, int nchunk,
    int tiles_per_wg, float c2) {
  using L = Lay<T, D>;
  using M = Mma<T>;
  constexpr int RHO = (POOL - 1) / 2;
  extern __shared__ __align__(16) char lds[];
  float* hs = reinterpret_cast<float*>(lds + TROWS * L::STRIDE);   // [G][TROWS]
  float* gmx = hs + G * TROWS;                                      // [TROWS]
  const int g = blockIdx.y, il = blockIdx.z, inst = inst0 + il;
  const int lane = threadIdx.x & 63, h = threadIdx.x >> 6;
  const int gq = lane >> 4, c = lane & 15;
  const bool active = h < G;
  const int Gw = G * w;
  const T* kb = k + ((size_t)inst * hkv + g) * (size_t)n * D;
  const T* qb = q + ((size_t)inst * hq + (size_t)g * G + (active ? h : 0)) * (size_t)w * D;

  // Row statistics: the pass-1 chunk partials of each row merged here, lane
  // group gq folding chunks gq, gq+4, ... in order, then the four groups
  // combined (the same order in every workgroup of the head).  With row_lse
  // given (natural-log log-sum-exp of the row's logits / sqrt(d) over its
  // domain) there is no pass 1: the row's weights are exp2(z*c2 - lse*log2 e),
  // lse*log2 e split in float64 into hi + lo, hi the reference and exp2(-lo)
  // the row factor, so the fp32 rounding of the product costs nothing.
  typename M::op_t qop[NB][L::KSTEPS];
  float smc[NB], sil[NB];   // scaled row max and 1 / row sum
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int r = 16 * nb + c;
    const bool ok = active && r < w;
#pragma unroll
    for (int ks = 0; ks < L::KSTEPS; ++ks)
      qop[nb][ks] = ok ? M::load(qb + (size_t)r * D + ks * M::KSTEP + M::KPL * gq) : M::zero();
    if (row_lse != nullptr) {
      smc[nb] = 0.f;                 // padding rows: q = 0, weight 0
      sil[nb] = 0.f;
      if (ok) {
        const double x = (double)row_lse[((size_t)inst * hq + (size_t)g * G + h) * w + r] * 1.4426950408889634;
        const float hi = (float)x;
        smc[nb] = hi;
        sil[nb] = fast_exp2(-(float)(x - (double)hi));
      }
      continue;
    }
    float m = -INFINITY, l = 0.f;
    if (ok) {
      // eight partials loaded before any is merged (a dependent load per
      // merge made this prologue latency-bound for small launches); the merge
      // order is unchanged
      const float2* pr = part + ((size_t)il * hkv + g) * nchunk * (size_t)Gw + h * w + r;
      for (int ch0 = gq; ch0 < nchunk; ch0 += 32) {
        float2 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int ch = ch0 + 4 * u;
          v[u] = ch < nchunk ? pr[(size_t)ch * Gw] : make_float2(-INFINITY, 0.f);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) merge_ml(m, l, v[u].x, v[u].y);
      }
    }
#pragma unroll
    for (int mask = 16; mask <= 32; mask <<= 1) {
      const float om = shfl_xor(m, mask), ol = shfl_xor(l, mask);
      merge_ml(m, l, om, ol);
    }
    smc[nb] = ok ? m : 0.f;          // padding rows: q = 0, weight 0
    sil[nb] = ok ? 1.0f / l : 0.f;
  }
  // Squared weights: (exp2(z c2 - m) s)^2 = exp2(z (2 c2) - 2 m) s^2, the
  // doubling exact, so the exponent argument is still one FMA.
  float c2e = c2;
  if (KIND == EMIT_SQ) {
    c2e = 2.0f * c2;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      smc[nb] *= 2.0f;
      sil[nb] *= sil[nb];
    }
  }
  // LAVa: max_k ||V[k]||_1 of the head from the value-norm kernel's block maxima
  float vscale = 0.f;
  if (KIND == EMIT_LAVA) {
    float vb = 0.f;
    for (int b = lane; b < nvblk; b += WAVE) vb = fmaxf(vb, vpart[((size_t)inst * hkv + g) * nvblk + b]);
#pragma unroll
    for (int mask = 1; mask < 64; mask <<= 1) vb = fmaxf(vb, shfl_xor(vb, mask));
    vscale = vb / (float)w;
  }
  const float inv_gw = 1.0f / (float)Gw, inv_w = 1.0f / (float)w;

  const int t0 = blockIdx.x * tiles_per_wg;
  TileRegs<T, D, -HALO, TILE + HALO> tr;
  tr.init();
  if (t0 * TILE < p) tr.load(kb, n, t0 * TILE);
  for (int t = 0; t < tiles_per_wg; ++t) {
    const int k0 = (t0 + t) * TILE;
    if (k0 >= p) break;
    __syncthreads();
    tr.store(lds);
    __syncthreads();
    if (t + 1 < tiles_per_wg && k0 + TILE < p) tr.load(kb, n, k0 + TILE);   // next tile in flight

    if (active) {
      const int kbase = k0 + 32 * gq;   // first key of this lane group
      if (KIND != EMIT_LAVA && RHO == 0) {
        // No pooling: each M-block is folded in as soon as its MFMAs finish.
        float ks[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) ks[i] = 0.f;
        const bool interior = k0 + TILE <= p;
        // one copy per value of the interior test (a per-logit test compiled
        // to a scalar branch per logit)
        auto fold = [&](auto interior_tag) {
          constexpr bool INTERIOR = decltype(interior_tag)::value;
#pragma unroll
          for (int mb = 0; mb < 8; ++mb) {
            f32x4 acc[NB];
            logits_block<T, D, NB>(lds, mb, c, gq, qop, acc);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const float e = fast_exp2(fmaf(acc[nb][j], c2e, -smc[nb]));
                if (INTERIOR) ks[4 * mb + j] = fmaf(e, sil[nb], ks[4 * mb + j]);
                else ks[4 * mb + j] += (kbase + 4 * mb + j < p) ? e * sil[nb] : 0.f;
              }
          }
        };
        if (interior) fold(std::true_type{});
        else fold(std::false_type{});
        float s0, s1;
        reduce_scatter16(ks, c, s0, s1);
        hs[h * TILE + 32 * gq + 2 * c] = s0;
        hs[h * TILE + 32 * gq + 2 * c + 1] = s1;
      } else if (KIND != EMIT_LAVA) {
        // the halo M-block (mb = 8) only feeds the pooling
        constexpr int NMB = RHO > 0 ? 9 : 8;
        f32x4 acc[NMB][NB];
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) logits_block<T, D, NB>(lds, mb, c, gq, qop, acc[mb]);
        const bool interior = k0 >= RHO && k0 + TILE + RHO <= p;   // all pooled keys inside the prefix
        float ks[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) ks[i] = 0.f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          // x[t] <-> key kbase - 3 + t, t in [0, 38); outside the prefix -> -inf
          float x[38];
#pragma unroll
          for (int mb = 0; mb < 8; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j) x[3 + 4 * mb + j] = acc[mb][nb][j];
          if (RHO > 0) {
#pragma unroll
            for (int j = 0; j < 3; ++j) {
              const float lft = shfl_lane(acc[7][nb][1 + j], (lane - 16) & 63);
              const float rgt = shfl_lane(acc[0][nb][j], (lane + 16) & 63);
              x[j] = (gq == 0) ? acc[NMB - 1][nb][1 + j] : lft;
              x[35 + j] = (gq == 3) ? acc[NMB - 1][nb][j] : rgt;
            }
          } else {
#pragma unroll
            for (int j = 0; j < 3; ++j) x[j] = x[35 + j] = -INFINITY;   // never read without pooling
          }
          if (!interior) {
#pragma unroll
            for (int t2 = 0; t2 < 38; ++t2) {
              const int key = kbase - 3 + t2;
              if (key < 0 || key >= p) x[t2] = -INFINITY;
            }
          }
          const float mc = smc[nb], il_row = sil[nb];
          if (RHO == 3) {
            float a3[36];
#pragma unroll
            for (int t2 = 0; t2 < 36; ++t2) a3[t2] = fmax3(x[t2], x[t2 + 1], x[t2 + 2]);
#pragma unroll
            for (int kk = 0; kk < 32; ++kk) {
              const float pooled = fmax3(a3[kk], a3[kk + 2], a3[kk + 4]);
              ks[kk] = fmaf(fast_exp2(fmaf(pooled, c2e, -mc)), il_row, ks[kk]);
            }
          } else {
#pragma unroll
            for (int kk = 0; kk < 32; ++kk) {
              float pooled = x[kk + 3];
              if (RHO >= 1) pooled = fmax3(pooled, x[kk + 2], x[kk + 4]);
              if (RHO >= 2) pooled = fmax3(pooled, x[kk + 1], x[kk + 5]);
              ks[kk] = fmaf(fast_exp2(fmaf(pooled, c2e, -mc)), il_row, ks[kk]);
            }
          }
        }
        float s0, s1;
        reduce_scatter16(ks, c, s0, s1);
        hs[h * TILE + 32 * gq + 2 * c] = s0;
        hs[h * TILE + 32 * gq + 2 * c + 1] = s1;
      } else {
        // LAVa: causal weights summed over the head's rows, before pooling.  Rows
        // are summed before pooling, so each M-block is folded in as soon as its
        // MFMAs finish (one block of accumulators live at a time).
        const bool interior = k0 >= HALO && k0 + TILE + HALO <= p;   // every key <= p <= p + r, >= 0
        float ks[32], hsum[4];
#pragma unroll
        for (int i = 0; i < 32; ++i) ks[i] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) hsum[j] = 0.f;
        const int hkey0 = (gq == 0) ? k0 - HALO : ((gq == 3) ? k0 + TILE : -1);
        // the interior test is a compile-time constant of each copy: tested
        // per logit, it compiled to a scalar branch per logit
        auto fold = [&](auto interior_tag) {
          constexpr bool INTERIOR = decltype(interior_tag)::value;
#pragma unroll
          for (int mb = 0; mb < 9; ++mb) {
            f32x4 acc[NB];
            logits_block<T, D, NB>(lds, mb, c, gq, qop, acc);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              const int r = 16 * nb + c;
              const int lim = min(n - 1, p + r);
              const float mc = smc[nb], il_row = sil[nb];
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const float e = fast_exp2(fmaf(acc[nb][j], c2, -mc));
                if (mb < 8) {
                  if (INTERIOR) ks[4 * mb + j] = fmaf(e, il_row, ks[4 * mb + j]);
                  else ks[4 * mb + j] += (kbase + 4 * mb + j <= lim) ? e * il_row : 0.f;
                } else {
                  const int key = hkey0 + j;
                  hsum[j] += (hkey0 >= 0 && key >= 0 && key <= lim) ? e * il_row : 0.f;
                }
              }
            }
          }
        };
        if (interior) fold(std::true_type{});
        else fold(std::false_type{});
        float s0, s1;
        reduce_scatter16(ks, c, s0, s1);
#pragma unroll
        for (int j = 0; j < 4; ++j) hsum[j] = allsum16(hsum[j]);
        float* hrow = hs + h * TROWS;
        hrow[HALO + 32 * gq + 2 * c] = s0;
        hrow[HALO + 32 * gq + 2 * c + 1] = s1;
        if (c == 0 && gq == 0)
          for (int j = 0; j < 4; ++j) hrow[j] = hsum[j];
        if (c == 0 && gq == 3)
          for (int j = 0; j < 4; ++j) hrow[HALO + TILE + j] = hsum[j];
      }
    }
    __syncthreads();
    if (KIND == EMIT_SQ) {
      for (int idx = threadIdx.x; idx < G * TILE; idx += blockDim.x) {
        const int hh = idx / TILE, t2 = idx % TILE, key = k0 + t2;
        if (key < p) head_scores[(((size_t)il * hq) + (size_t)g * G + hh) * p + key] = hs[hh * TILE + t2];
      }
    } else if (KIND == EMIT_SNAP) {
      for (int t2 = threadIdx.x; t2 < TILE; t2 += blockDim.x) {
        const int key = k0 + t2;
        if (key < p) {
          float sum = 0.f;
          for (int hh = 0; hh < G; ++hh) sum += hs[hh * TILE + t2];
          score[((size_t)inst * hkv + g) * p + key] = sum * inv_gw;
        }
      }
      if (head_scores != nullptr) {
        for (int idx = threadIdx.x; idx < G * TILE; idx += blockDim.x) {
          const int hh = idx / TILE, t2 = idx % TILE, key = k0 + t2;
          if (key < p)
            head_scores[(((size_t)il * hq) + (size_t)g * G + hh) * p + key] = hs[hh * TILE + t2] * inv_w;
        }
      }
    } else {
      for (int t2 = threadIdx.x; t2 < TROWS; t2 += blockDim.x) {
        float m = hs[t2];
        for (int hh = 1; hh < G; ++hh) m = fmaxf(m, hs[hh * TROWS + t2]);
        gmx[t2] = m;
      }
      __syncthreads();
      for (int t2 = threadIdx.x; t2 < TILE; t2 += blockDim.x) {
        const int key = k0 + t2;
        if (key < p) {
          float m = gmx[HALO + t2];
#pragma unroll
          for (int o = 1; o <= RHO; ++o) m = fmax3(m, gmx[HALO + t2 - o], gmx[HALO + t2 + o]);
          score[((size_t)inst * hkv + g) * p + key] = vscale * m;
        }
      }
    }
  }
}

// LAVa value-norm maximum, max_t sum_e |v[i, g, t, e]|, as one maximum per block
// of rows_per_wg rows (row sums in a fixed order; a maximum is exact and order
// independent), reduced by the consumer.  No atomics: with one per wave,
// contention on the few targets held the workgroups back and cost a fifth of
// the read bandwidth.  V is read once, so the loads are nontemporal; each lane
// keeps U of them in flight and a row's |.| sum is completed across its lanes
// with DPP moves.
template <int LPR>
__device__ __forceinline__ float rowsum_lanes(float x) {
  if (LPR >= 16) x += dpp<DPP_MIRROR>(x);
  if (LPR >= 8) x += dpp<DPP_HALF_MIRROR>(x);
  if (LPR >= 4) x += dpp<DPP_XOR2>(x);
  if (LPR >= 2) x += dpp<DPP_XOR1>(x);
  return x;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void vbar_kernel(const T* __restrict__ v, float* __restrict__ vpart,
                                                   int inst0, int hkv, int n, int rows_per_wg) {
  __shared__ float wmax[4];
  using L = Lay<T, D>;
  constexpr int LPR = L::CPR;              // lanes per row
  static_assert(LPR <= 16 && (LPR & (LPR - 1)) == 0, "a row spans at most one 16-lane DPP row");
  constexpr int RPL = WAVE / LPR;          // rows per wave load
  constexpr int U = 8;                     // loads in flight per lane
  const int g = blockIdx.y, inst = inst0 + blockIdx.z;
  const T* vb = v + ((size_t)inst * hkv + g) * (size_t)n * D;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int lr = lane / LPR, ch = lane % LPR;
  const int r0 = blockIdx.x * rows_per_wg, r1 = min(n, r0 + rows_per_wg);
  const int nwv = blockDim.x / WAVE;
  float best = 0.f;
  for (int base = r0 + wv * U * RPL; base < r1; base += nwv * U * RPL) {   // same trip count in a wave
    u32x4 x[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int r = base + i * RPL + lr;
      u32x4 z = {0u, 0u, 0u, 0u};
      x[i] = (r < r1) ? ld16_nt(vb + (size_t)r * D + ch * L::EPC) : z;
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
      float s = 0.f;
      if (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s += fabsf(bf16_bits_to_f32(x[i][e] & 0xffffu)) + fabsf(bf16_bits_to_f32(x[i][e] >> 16));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) s += fabsf(__uint_as_float(x[i][e]));
      }
      best = fmaxf(best, rowsum_lanes<LPR>(s));
    }
  }
#pragma unroll
  for (int m = LPR; m < 64; m <<= 1) best = fmaxf(best, shfl_xor(best, m));
  if (lane == 0) wmax[wv] = best;
  __syncthreads();
  if (threadIdx.x == 0)
    vpart[((size_t)inst * hkv + g) * gridDim.x + blockIdx.x] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
}

// ---------------------------------------------------------------- host side
constexpr int VBAR_ROWS = 2048;   // rows per value-norm workgroup
int vbar_blocks(const Geo& g) { return (g.n + VBAR_ROWS - 1) / VBAR_ROWS; }

constexpr int KR_MIN_KPW = 512;   // keys per register-K statistics workgroup, at least
constexpr int KR_MIN_BLOCKS = 8;  // 64-key blocks per resident workgroup below which the LDS-tiled kernels run

// The register-K kernels of a geometry, or nullptr where the LDS-tiled
// kernels serve it (fp32, d != 128, w > 32, group sizes without an instance;
// for pass 2 also LAVa, LaProx and CriticalKV, which need per-head or summed
// rows).
using KrStatsFn = void (*)(const uint16_t*, const uint16_t*, float2*, int, int, int, int, int, int, int, int, int,
                           float);
using KrEmitFn = void (*)(const uint16_t*, const uint16_t*, const float2*, const float*, float*, int, int, int, int,
                          int, int, int, int, float);
bool kr_geometry(const Geo& g) {
  if (g.dtype != ADAKV_BF16 || g.d != 128 || g.w > 32) return false;
  if ((int64_t)g.n * KR_QROWB >= ((int64_t)1 << 31)) return false;   // buffer range in 32 bits
  return g.G == 1 || g.G == 2 || g.G == 4 || g.G == 5 || (g.G == 8 && g.w <= 16);
}
template <int G>
KrStatsFn kr_stats_for(int w, bool causal) {
  if (w <= 16) return causal ? kr_stats_kernel<G, 1, true> : kr_stats_kernel<G, 1, false>;
  if constexpr (G <= 5) return causal ? kr_stats_kernel<G, 2, true> : kr_stats_kernel<G, 2, false>;
  return nullptr;
}
KrStatsFn kr_stats_pick(const Geo& g, bool causal) {
  if (!kr_geometry(g)) return nullptr;
  switch (g.G) {
    case 1: return kr_stats_for<1>(g.w, causal);
    case 2: return kr_stats_for<2>(g.w, causal);
    case 4: return kr_stats_for<4>(g.w, causal);
    case 5: return kr_stats_for<5>(g.w, causal);
    case 8: return kr_stats_for<8>(g.w, causal);
    default: return nullptr;
  }
}
template <int G, int NBW>
KrEmitFn kr_emit_for_pool(int pool) {
  switch (pool) {
    case 1: return kr_emit_kernel<G, NBW, 1>;
    case 3: return kr_emit_kernel<G, NBW, 3>;
    case 5: return kr_emit_kernel<G, NBW, 5>;
    case 7: return kr_emit_kernel<G, NBW, 7>;
    default: return nullptr;
  }
}
template <int G>
KrEmitFn kr_emit_for(int w, int pool) {
  if (w <= 16) return kr_emit_for_pool<G, 1>(pool);
  if constexpr (G <= 5) return kr_emit_for_pool<G, 2>(pool);
  return nullptr;
}
KrEmitFn kr_emit_pick(const Geo& g) {
  if (!kr_geometry(g) || g.scorer != ADAKV_SCORE_SNAPKV) return nullptr;
  switch (g.G) {
    case 1: return kr_emit_for<1>(g.w, g.pool);
    case 2: return kr_emit_for<2>(g.w, g.pool);
    case 4: return kr_emit_for<4>(g.w, g.pool);
    case 5: return kr_emit_for<5>(g.w, g.pool);
    case 8: return kr_emit_for<8>(g.w, g.pool);
    default: return nullptr;
  }
}
using KrLavaFn = void (*)(const uint16_t*, const uint16_t*, const float2*, const float*, float*, int, int, int, int,
                          int, int, int, int, int, float);
template <int G>
KrLavaFn kr_lava_for(int w) {
  if (w <= 16) return kr_lava_kernel<G, 1>;
  if constexpr (G <= 5) return kr_lava_kernel<G, 2>;
  return nullptr;
}
KrLavaFn kr_lava_pick(const Geo& g) {
  if (!kr_geometry(g) || g.scorer != ADAKV_SCORE_LAVA) return nullptr;
  switch (g.G) {
    case 1: return kr_lava_for<1>(g.w);
    case 2: return kr_lava_for<2>(g.w);
    case 4: return kr_lava_for<4>(g.w);
    case 5: return kr_lava_for<5>(g.w);
    case 8: return kr_lava_for<8>(g.w);
    default: return nullptr;
  }
}
// Keys whose LAVa group maximum the pooling of the prefix scores reads.
int lava_keys(const Geo& g) { return std::min(g.n, g.p + (g.pool - 1) / 2); }

// Resident workgroups of a register-K kernel on the device (one round of them
// covers a launch).
long kr_resident_wgs(const void* fn, size_t lds, int cus) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, KR_WAVES * WAVE, lds) != hipSuccess || per_cu < 1)
    per_cu = 2;
  return (long)per_cu * cus;
}
// Keys per workgroup for one round of `resident` workgroups over `blocks`
// 64-key blocks, a multiple of 4 blocks (one per wave) and at least min_keys.
int kr_keys_per_wg(long blocks, long resident, int min_keys) {
  const long per_wg = std::max<long>((blocks + resident - 1) / resident, min_keys / KB);
  return (int)(((per_wg + KR_WAVES - 1) / KR_WAVES) * KR_WAVES * KB);
}

struct ScorePlan {
  int ib;        // instances per batch
  int nchunk;    // stats chunks per head
  int kend;      // end of the widest row domain
  size_t off_part, off_heads, off_vbar, off_fac, off_smax, off_pmerge, total;
};

ScorePlan plan_score(const Geo& g) {
  ScorePlan P{};
  const size_t inst_k_bytes = (size_t)g.hkv * g.n * g.d * (g.dtype == ADAKV_BF16 ? 2 : 4);
  size_t ib = (size_t)(1024u << 20) / (inst_k_bytes ? inst_k_bytes : 1);   // ~1 GiB of K per launch
  if (ib < 1) ib = 1;
  if (ib > (size_t)g.I) ib = g.I;
  P.ib = (int)ib;
  const bool laprox = g.scorer == ADAKV_SCORE_LAPROX;
  P.kend = (g.scorer == ADAKV_SCORE_LAVA || laprox) ? g.n : g.p;
  // the most row partials a launch can write: one tile per chunk, or (register-K
  // path) four waves per chunk of at least KR_MIN_KPW keys
  P.nchunk = std::max((P.kend + TILE - 1) / TILE, KR_WAVES * ((P.kend + KR_MIN_KPW - 1) / KR_MIN_KPW));
  const size_t Gw = (size_t)g.G * g.w;
  size_t off = 0;
  P.off_part = off;  off = align_up(off + (size_t)P.ib * g.hkv * P.nchunk * Gw * sizeof(float2), 256);
  P.off_heads = off;
  if (g.scorer == ADAKV_SCORE_CRITICALKV || laprox)
    off = align_up(off + (size_t)P.ib * g.hq * g.p * sizeof(float), 256);
  P.off_vbar = off;
  if (g.scorer == ADAKV_SCORE_LAVA) off = align_up(off + (size_t)g.I * g.hkv * vbar_blocks(g) * sizeof(float), 256);
  P.off_fac = off;
  off = align_up(off + factor_ws_bytes(g), 256);
  P.off_smax = off;   // LAVa on the register-K path: unpooled group maxima of a batch
  if (g.scorer == ADAKV_SCORE_LAVA && kr_geometry(g))
    off = align_up(off + (size_t)P.ib * g.hkv * lava_keys(g) * sizeof(float), 256);
  P.off_pmerge = off;   // one merged (max, sum) pair per window row of a batch
  off = align_up(off + (size_t)P.ib * g.hkv * Gw * sizeof(float2), 256);
  P.total = off;
  return P;
}

template <typename T, int D, int NB>
hipError_t run_score(const Geo& g, const ScorePlan& P, const void* q, const void* k, const void* v,
                     const void* w_o, const float* row_lse, float* score, float* score2, char* ws,
                     hipStream_t st) {
  using L = Lay<T, D>;
  const float c2 = (float)(1.4426950408889634 / std::sqrt((double)g.d));
  float2* part = reinterpret_cast<float2*>(ws + P.off_part);
  const bool laprox = g.scorer == ADAKV_SCORE_LAPROX;
  float* heads = (g.scorer == ADAKV_SCORE_CRITICALKV || laprox) ? reinterpret_cast<float*>(ws + P.off_heads) : nullptr;
  float* vpart = reinterpret_cast<float*>(ws + P.off_vbar);
  const int nvblk = vbar_blocks(g);
  const T* qt = static_cast<const T*>(q);
  const T* kt = static_cast<const T*>(k);
  const bool lava = g.scorer == ADAKV_SCORE_LAVA;
  const int threads = std::max(g.G, 4) * WAVE;
  const size_t lds_stats = (size_t)TILE * L::STRIDE;
  const size_t lds_emit = (size_t)TROWS * L::STRIDE + (size_t)(g.G + 1) * TROWS * sizeof(float);
  const int ntiles = (g.p + TILE - 1) / TILE;
  const bool factor = use_factor(g);
  if (factor) {
    // Gram factors of the call's shared projection, once for all instances
    hipError_t e = launch_factor(g, w_o, ws + P.off_fac, st);
    if (e != hipSuccess) return e;
  }
  const void* vw = factor ? static_cast<const void*>(ws + P.off_fac + align_up((size_t)g.hq * factor_slices(g) * 128 * 128 * sizeof(float), 256)) : w_o;

  if (lava) {
    dim3 grid(nvblk, g.hkv, g.I);
    vbar_kernel<T, D><<<grid, 256, 0, st>>>(static_cast<const T*>(v), vpart, 0, g.hkv, g.n, VBAR_ROWS);
  }
  // about two resident workgroups per CU, each streaming many tiles
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const long target = 2L * (cus > 0 ? cus : 256);
  const int ktiles = (P.kend + TILE - 1) / TILE;
  KrStatsFn krs = nullptr;
  KrEmitFn kre = nullptr;
  KrLavaFn krl = nullptr;
  size_t kr_lds = 0, kr_lds_e = 0;
  long krs_res = 0, kre_res = 0, krl_res = 0;
  const int ke = lava_keys(g);
  if constexpr (sizeof(T) == 2 && D == 128) {
    if (kr_geometry(g) && !laprox) {
      // only where every resident workgroup gets several blocks of each pass
      const long blocks = (long)((P.kend + KB - 1) / KB) * g.hkv * P.ib;
      kr_lds = (size_t)g.G * ((g.w + 15) / 16) * 16 * KR_QROWB;   // the window queries
      kr_lds_e = kr_lds + (size_t)g.G * ((g.w + 15) / 16) * 16 * sizeof(float2);   // + row statistics
      krs = kr_stats_pick(g, lava);
      if (krs != nullptr) {
        krs_res = kr_resident_wgs(reinterpret_cast<const void*>(krs), kr_lds, cus > 0 ? cus : 256);
        if (blocks < KR_MIN_BLOCKS * krs_res) krs = nullptr;
      }
      kre = (krs != nullptr || row_lse != nullptr) ? kr_emit_pick(g) : nullptr;
      if (kre != nullptr) {
        kre_res = kr_resident_wgs(reinterpret_cast<const void*>(kre), kr_lds_e, cus > 0 ? cus : 256);
        if (blocks < KR_MIN_BLOCKS * kre_res) kre = nullptr;
      }
      // the pooling launch it adds costs a one-instance call (the online
      // prefill's) what the faster emit saves
      krl = (P.ib >= 2 && (krs != nullptr || row_lse != nullptr)) ? kr_lava_pick(g) : nullptr;
      if (krl != nullptr) {
        krl_res = kr_resident_wgs(reinterpret_cast<const void*>(krl), kr_lds_e, cus > 0 ? cus : 256);
        if ((long)((ke + KB - 1) / KB) * g.hkv * P.ib < KR_MIN_BLOCKS * krl_res) krl = nullptr;
      }
    }
  }
  for (int i0 = 0; i0 < g.I; i0 += P.ib) {
    const int ni = std::min(P.ib, g.I - i0);
    const long stiles = (long)ktiles * g.hkv * ni;
    const int spw = (int)std::min<long>(ktiles, std::max<long>(1, stiles / target));
    const int kpw = spw * TILE;
    int nchunk = (P.kend + kpw - 1) / kpw;
    dim3 g1(nchunk, g.hkv, ni);
    if (row_lse != nullptr) {
      // the caller's row statistics replace pass 1
    } else if (krs != nullptr) {
      // one round of resident workgroups, each over an equal key range of one head
      const int kpw_kr = kr_keys_per_wg((long)((P.kend + KB - 1) / KB) * g.hkv * ni, krs_res, KR_MIN_KPW);
      const int chunks = (P.kend + kpw_kr - 1) / kpw_kr;
      nchunk = chunks * KR_WAVES;
      krs<<<dim3(chunks, g.hkv, ni), KR_WAVES * WAVE, kr_lds, st>>>(reinterpret_cast<const uint16_t*>(qt),
                                                                   reinterpret_cast<const uint16_t*>(kt), part, i0,
                                                                   g.hq, g.hkv, g.n, g.w, g.p, P.kend, nchunk,
                                                                   kpw_kr, c2);
    } else if (lava)
      score_stats_kernel<T, D, NB, true><<<g1, threads, lds_stats, st>>>(qt, kt, part, i0, g.hq, g.hkv, g.G, g.n,
                                                                         g.w, g.p, P.kend, nchunk, kpw, c2);
    else
      score_stats_kernel<T, D, NB, false><<<g1, threads, lds_stats, st>>>(qt, kt, part, i0, g.hq, g.hkv, g.G, g.n,
                                                                          g.w, g.p, P.kend, nchunk, kpw, c2);
    // pass 2 reads one merged (max, sum) pair per row where a head's keys
    // were split over many chunks (a long instance alone in its batch)
    const float2* part_e = part;
    int nsub_e = nchunk;
    if (row_lse == nullptr && nchunk > MERGE_MIN) {
      float2* pm = reinterpret_cast<float2*>(ws + P.off_pmerge);
      const int Gw = g.G * g.w;
      const int rows = ni * g.hkv * Gw;
      merge_part_kernel<<<(rows + 3) / 4, 256, 0, st>>>(part, pm, rows, Gw, nchunk);
      part_e = pm;
      nsub_e = 1;
    }
    const long tiles_total = (long)ntiles * g.hkv * ni;
    int tpw = (int)std::max<long>(1, (tiles_total + target - 1) / target);
    if (tpw > ntiles) tpw = ntiles;
    dim3 g2((ntiles + tpw - 1) / tpw, g.hkv, ni);
#define EMIT(POOLV)                                                                                          \
  do {                                                                                                       \
    if (lava)                                                                                                \
      score_emit_kernel<T, D, NB, POOLV, EMIT_LAVA><<<g2, threads, lds_emit, st>>>(                          \
          qt, kt, part_e, row_lse, vpart, nvblk, score, nullptr, i0, g.hq, g.hkv, g.G, g.n, g.w, g.p, nsub_e, tpw, c2);              \
    else                                                                                                     \
      score_emit_kernel<T, D, NB, POOLV, EMIT_SNAP><<<g2, threads, lds_emit, st>>>(                          \
          qt, kt, part_e, row_lse, vpart, nvblk, score, heads, i0, g.hq, g.hkv, g.G, g.n, g.w, g.p, nsub_e, tpw, c2);              \
  } while (0)
    if (krl != nullptr) {
      float* smax = reinterpret_cast<float*>(ws + P.off_smax);
      const int kpw_l = kr_keys_per_wg((long)((ke + KB - 1) / KB) * g.hkv * ni, krl_res, KR_WAVES * KB);
      krl<<<dim3((ke + kpw_l - 1) / kpw_l, g.hkv, ni), KR_WAVES * WAVE, kr_lds_e, st>>>(
          reinterpret_cast<const uint16_t*>(qt), reinterpret_cast<const uint16_t*>(kt), part_e, row_lse, smax, i0,
          g.hq, g.hkv, g.n, g.w, g.p, ke, nsub_e, kpw_l, c2);
      const dim3 gp((g.p + LP_KEYS - 1) / LP_KEYS, g.hkv, ni);
      switch (g.pool) {
        case 1: lava_pool_kernel<0><<<gp, 256, 0, st>>>(smax, vpart, nvblk, score, i0, g.hkv, g.p, ke, g.w); break;
        case 3: lava_pool_kernel<1><<<gp, 256, 0, st>>>(smax, vpart, nvblk, score, i0, g.hkv, g.p, ke, g.w); break;
        case 5: lava_pool_kernel<2><<<gp, 256, 0, st>>>(smax, vpart, nvblk, score, i0, g.hkv, g.p, ke, g.w); break;
        default: lava_pool_kernel<3><<<gp, 256, 0, st>>>(smax, vpart, nvblk, score, i0, g.hkv, g.p, ke, g.w); break;
      }
    } else if (kre != nullptr && heads == nullptr) {
      const int kpw_e = kr_keys_per_wg((long)((g.p + KB - 1) / KB) * g.hkv * ni, kre_res, KR_WAVES * KB);
      kre<<<dim3((g.p + kpw_e - 1) / kpw_e, g.hkv, ni), KR_WAVES * WAVE, kr_lds_e, st>>>(
          reinterpret_cast<const uint16_t*>(qt), reinterpret_cast<const uint16_t*>(kt), part_e, row_lse, score, i0,
          g.hq, g.hkv, g.n, g.w, g.p, nsub_e, kpw_e, c2);
    } else if (laprox) {
      if constexpr (sizeof(T) == 2 && D == 128)   // the only LaProx geometry the ABI accepts
        score_emit_kernel<T, D, NB, 1, EMIT_SQ><<<g2, threads, lds_emit, st>>>(
            qt, kt, part_e, row_lse, vpart, nvblk, score, heads, i0, g.hq, g.hkv, g.G, g.n, g.w, g.p, nsub_e, tpw, c2);
      else
        return hipErrorInvalidValue;
    } else switch (g.pool) {
      case 1: EMIT(1); break;
      case 3: EMIT(3); break;
      case 5: EMIT(5); break;
      default: EMIT(7); break;
    }
#undef EMIT
    if (g.scorer == ADAKV_SCORE_CRITICALKV || laprox) {
      hipError_t e = launch_vwo(g, i0, ni, v, vw, heads, laprox ? score : score2, factor, st);
      if (e != hipSuccess) return e;
    }
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run_score_nb(const Geo& g, const ScorePlan& P, const void* q, const void* k, const void* v,
                        const void* w_o, const float* row_lse, float* score, float* score2, char* ws,
                        hipStream_t st) {
  if (g.w <= 16) return run_score<T, D, 1>(g, P, q, k, v, w_o, row_lse, score, score2, ws, st);
  if (g.w <= 32) return run_score<T, D, 2>(g, P, q, k, v, w_o, row_lse, score, score2, ws, st);
  return run_score<T, D, 4>(g, P, q, k, v, w_o, row_lse, score, score2, ws, st);
}

}  // namespace

size_t score_ws_bytes(const Geo& g) { return plan_score(g).total; }

hipError_t launch_score(const Geo& g, const void* q, const void* k, const void* v, const void* w_o,
                        const float* row_lse, float* score, float* score2, char* ws, hipStream_t st) {
  const ScorePlan P = plan_score(g);
  if (g.dtype == ADAKV_BF16) {
    if (g.d == 128) return run_score_nb<uint16_t, 128>(g, P, q, k, v, w_o, row_lse, score, score2, ws, st);
    if (g.d == 64) return run_score_nb<uint16_t, 64>(g, P, q, k, v, w_o, row_lse, score, score2, ws, st);
  } else {
    if (g.d == 16) return run_score_nb<float, 16>(g, P, q, k, v, w_o, row_lse, score, score2, ws, st);
    if (g.d == 64) return run_score_nb<float, 64>(g, P, q, k, v, w_o, row_lse, score, score2, ws, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace adakv
