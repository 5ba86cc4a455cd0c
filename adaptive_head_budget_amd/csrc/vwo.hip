// CriticalKV projected value norms on gfx950.
//
// CriticalKV notes, "损失函数 / 训练策略": the only new runtime quantity is the
// L1 norm of every row of V W^O; "两阶段贪心选择算法": the composite score of an
// entry is (A + eps) * ||(V W^O)_t||_1.  Under GQA the composite of a KV head is
// the mean over its query heads i of (A_i[t] + eps) * ||(V_g W^O_i)[t]||_1.
//
// For one KV head g and 256 keys, a workgroup forms V_g[t, :] W^O_i (K = d = 128,
// N = hidden) for every query head i of the group on 16x16x32 bf16 MFMA tiles,
// and folds every product element into |.| row sums as soon as it leaves the
// accumulator: the [keys x hidden] product is never written.  W^O is read in
// the nn.Linear layout [hidden, hq*d], so a 64-column tile of W^O_i is 64
// contiguous 256-byte rows, staged through LDS and shared by the 4 waves.
#include "common.hpp"
#include "kernels.hpp"

namespace adakv {
namespace {

constexpr int D = 128;
constexpr int KEYS = 256;          // keys per workgroup (64 per wave)
constexpr int NT = 64;             // hidden columns per tile
constexpr int WSTRIDE = D * 2 + 16;
constexpr int KSTEPS = D / 32;

__global__ __launch_bounds__(256) void vwo_norm_kernel(const uint16_t* __restrict__ v, const uint16_t* __restrict__ w_o,
                                                       const float* __restrict__ head_scores, float* __restrict__ comp,
                                                       int inst0, int hq, int hkv, int G, int n, int p, int hidden,
                                                       float eps) {
  __shared__ __align__(16) char wt[2][NT * WSTRIDE];
  const int g = blockIdx.y, il = blockIdx.z, inst = inst0 + il;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int gq = lane >> 4, c = lane & 15;
  const int key0 = blockIdx.x * KEYS + 64 * wv;
  const uint16_t* vb = v + ((size_t)inst * hkv + g) * (size_t)n * D;

  // A operands: 4 M-blocks of 16 keys, held for the whole workgroup.
  bf16x8 aop[4][KSTEPS];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    int t = key0 + 16 * mb + c;
    t = (t < p) ? t : 0;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) aop[mb][ks] = Mma<uint16_t>::load(vb + (size_t)t * D + ks * 32 + 8 * gq);
  }
  float cacc[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) cacc[mb][j] = 0.f;

  const int ntiles = hidden / NT;
  for (int h = 0; h < G; ++h) {
    const int i = g * G + h;
    const uint16_t* wb = w_o + (size_t)i * D;   // column block of head i, row stride hq*D
    const size_t wrow = (size_t)hq * D;
    float rsum[4][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) rsum[mb][j] = 0.f;
    // stage tile 0
    __syncthreads();
    for (int idx = threadIdx.x; idx < NT * 16; idx += 256) {
      const int r = idx >> 4, ch = idx & 15;
      st16(wt[0] + r * WSTRIDE + ch * 16, ld16(wb + (size_t)r * wrow + ch * 8));
    }
    __syncthreads();
    for (int tile = 0; tile < ntiles; ++tile) {
      const int cur = tile & 1;
      // prefetch the next tile into registers while this one is multiplied
      u32x4 pre[4];
      const bool more = tile + 1 < ntiles;
      if (more) {
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          const int idx = threadIdx.x + 256 * q2;
          const int r = idx >> 4, ch = idx & 15;
          pre[q2] = ld16(wb + (size_t)((tile + 1) * NT + r) * wrow + ch * 8);
        }
      }
      f32x4 acc[4][4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = zero4();
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const bf16x8 bop = Mma<uint16_t>::load(
              reinterpret_cast<const uint16_t*>(wt[cur] + (16 * nb + c) * WSTRIDE) + ks * 32 + 8 * gq);
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) acc[mb][nb] = Mma<uint16_t>::mma(aop[mb][ks], bop, acc[mb][nb]);
        }
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int j = 0; j < 4; ++j) rsum[mb][j] += fabsf(acc[mb][nb][j]);
      if (more) {
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          const int idx = threadIdx.x + 256 * q2;
          const int r = idx >> 4, ch = idx & 15;
          st16(wt[cur ^ 1] + r * WSTRIDE + ch * 16, pre[q2]);
        }
      }
      __syncthreads();
    }
    // rsum[mb][j]: partial over this lane's columns of key key0 + 16mb + 4gq + j
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x = rsum[mb][j];
        x += shfl_xor(x, 8);
        x += shfl_xor(x, 4);
        x += shfl_xor(x, 2);
        x += shfl_xor(x, 1);
        const int t = key0 + 16 * mb + 4 * gq + j;
        const float a = (t < p) ? head_scores[((size_t)il * hq + i) * p + t] : 0.f;
        cacc[mb][j] += (a + eps) * x;
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

}  // namespace

hipError_t launch_vwo(const Geo& g, int inst0, int ni, const void* v, const void* w_o, const float* head_scores,
                      float* score2, hipStream_t st) {
  if (g.dtype != ADAKV_BF16 || g.d != D || g.hidden % NT != 0) return hipErrorInvalidValue;
  dim3 grid((g.p + KEYS - 1) / KEYS, g.hkv, ni);
  vwo_norm_kernel<<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(w_o),
                                        head_scores, score2, inst0, g.hq, g.hkv, g.G, g.n, g.p, g.hidden, g.eps);
  return hipGetLastError();
}

}  // namespace adakv
