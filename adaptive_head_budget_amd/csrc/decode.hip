// Decode attention over the flat variable-length cache on gfx950.
//
// Ada-KV notes, "多头自注意力层的形式化描述": append the new key/value, then
// A_i = softmax(q_i K^T) (scaled by 1/sqrt(d_h), LAVa notes "解码过程的残差流视角")
// and the head output A_i V.  The varlen design follows the Ada-KV paper's
// "Variable-length Attention with Variable-sized Cache Elements": every
// segment (instance, KV head) has its own length, and the G query heads of a
// GQA group share every row read.
//
// Work is split into chunks of DECODE_ROWS rows.  A prep kernel appends the new
// rows and lays out the chunk list; the attention kernel turns one chunk into a
// partial (row max, sum, weighted value sum) per query head, with q.K^T on
// 16x16 MFMA tiles (rows on M, query heads on N) and the value sum on the
// vector units reading V with 16-byte coalesced loads; the merge kernel
// combines the partials of each head in chunk order.
#include "common.hpp"
#include "kernels.hpp"

namespace adakv {
namespace {

constexpr int PT = 1024;
constexpr int R = DECODE_ROWS;

template <typename T, int D>
__global__ __launch_bounds__(PT) void decode_prep_kernel(const T* __restrict__ k_new, const T* __restrict__ v_new,
                                                         T* __restrict__ kf, T* __restrict__ vf,
                                                         const int64_t* __restrict__ seg_start,
                                                         int32_t* __restrict__ seg_len, int S,
                                                         int32_t* __restrict__ chunk_start) {
  __shared__ int32_t wsum[PT / WAVE];
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int CPR = D / EPC;
  int running = 0;
  for (int base = 0; base < S; base += PT) {
    const int s = base + threadIdx.x;
    int nch = 0;
    if (s < S) {
      int len = seg_len[s];
      // append only inside the segment's own rows (its reserve)
      if (k_new != nullptr && seg_start[s] + len < seg_start[s + 1]) {
        const int64_t row = seg_start[s] + len;
        for (int c = 0; c < CPR; ++c) {
          st16(kf + row * D + c * EPC, ld16(k_new + (size_t)s * D + c * EPC));
          st16(vf + row * D + c * EPC, ld16(v_new + (size_t)s * D + c * EPC));
        }
        len += 1;
        seg_len[s] = len;
      }
      nch = (len + R - 1) / R;
    }
    // exclusive scan of nch
    int inc = nch;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(inc, off);
      if ((int)__lane_id() >= off) inc += y;
    }
    const int wv = threadIdx.x / WAVE;
    if ((int)__lane_id() == 63) wsum[wv] = inc;
    __syncthreads();
    int before = 0, all = 0;
    for (int i = 0; i < PT / WAVE; ++i) {
      before += (i < wv) ? wsum[i] : 0;
      all += wsum[i];
    }
    __syncthreads();
    if (s < S) chunk_start[s] = running + before + inc - nch;
    running += all;
  }
  if (threadIdx.x == 0) chunk_start[S] = running;
}

// One chunk of up to R rows of one segment.  4 waves x 64 rows.
template <typename T, int D, int GT>
__global__ __launch_bounds__(256) void decode_attn_kernel(const T* __restrict__ q, const T* __restrict__ kf,
                                                          const T* __restrict__ vf,
                                                          const int64_t* __restrict__ seg_start,
                                                          const int32_t* __restrict__ seg_len,
                                                          const int32_t* __restrict__ chunk_start, int S, int hq,
                                                          int hkv, int G, float c2, float* __restrict__ part) {
  using M = Mma<T>;
  constexpr int KSTEPS = D / M::KSTEP;
  constexpr int EPL = 16 / (int)sizeof(T);     // value elements per lane
  constexpr int LPR = D / EPL;                 // lanes per value row
  constexpr int RS = WAVE / LPR;               // row slots per wave
  constexpr int PSTR = D + 2;
  __shared__ float P[4][64][GT];
  __shared__ float Ow[4][GT][D];
  __shared__ float Mw[4][GT], Lw[4][GT];
  __shared__ int seg_sh;

  const int b = blockIdx.x;
  const int total = chunk_start[S];
  if (b >= total) return;
  if (threadIdx.x == 0) {
    int lo = 0, hi = S - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (chunk_start[mid] <= b) lo = mid;
      else hi = mid - 1;
    }
    seg_sh = lo;
  }
  __syncthreads();
  const int s = seg_sh;
  const int inst = s / hkv, g = s % hkv;
  const int len = seg_len[s];
  const int row0 = (b - chunk_start[s]) * R;
  const int64_t base_row = seg_start[s];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int gq = lane >> 4, c = lane & 15;

  // B operand: q^T, column c = query head of the group (zero beyond G).
  typename M::op_t qop[KSTEPS];
  const T* qb = q + ((size_t)inst * hq + (size_t)g * G + (c < G ? c : 0)) * D;
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) qop[ks] = (c < G) ? M::load(qb + ks * M::KSTEP + M::KPL * gq) : M::zero();

  const int wrow0 = row0 + 64 * wv;   // first row of this wave
  f32x4 acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    acc[mb] = zero4();
    int r = wrow0 + 16 * mb + c;
    r = (r < len) ? r : 0;
    const T* krow = kf + (base_row + r) * D;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) acc[mb] = M::mma(M::load(krow + ks * M::KSTEP + M::KPL * gq), qop[ks], acc[mb]);
  }
  // acc[mb][j] <-> row wrow0 + 16*mb + 4*gq + j, query head c
  float m = -INFINITY;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wrow0 + 16 * mb + 4 * gq + j;
      if (r < len) m = fmaxf(m, acc[mb][j]);
    }
  m = fmaxf(m, shfl_xor(m, 16));
  m = fmaxf(m, shfl_xor(m, 32));
  float l = 0.f;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wrow0 + 16 * mb + 4 * gq + j;
      const float e = (r < len && m != -INFINITY) ? fast_exp2((acc[mb][j] - m) * c2) : 0.f;
      l += e;
      if (c < GT) P[wv][16 * mb + 4 * gq + j][c] = e;
    }
  l += shfl_xor(l, 16);
  l += shfl_xor(l, 32);
  if (gq == 0 && c < GT) {
    Mw[wv][c] = m;
    Lw[wv][c] = l;
  }
  __syncthreads();

  // value sum: lane (row slot rs, element chunk cc)
  const int rs = lane / LPR, cc = lane % LPR;
  float o[GT][EPL];
#pragma unroll
  for (int h = 0; h < GT; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = 0.f;
#pragma unroll 4
  for (int t = 0; t < 64 / RS; ++t) {
    const int rr = t * RS + rs;
    const int r = wrow0 + rr;
    if (r < len) {
      const u32x4 raw = ld16(vf + (base_row + r) * D + cc * EPL);
      float vv[EPL];
      if (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vv[2 * e] = bf16_bits_to_f32(raw[e] & 0xffffu);
          vv[2 * e + 1] = bf16_bits_to_f32(raw[e] >> 16);
        }
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) vv[e] = __uint_as_float(raw[e]);
      }
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        const float pw = P[wv][rr][h];
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[h][e] += pw * vv[e];
      }
    }
  }
#pragma unroll
  for (int msk = LPR; msk < 64; msk <<= 1)
#pragma unroll
    for (int h = 0; h < GT; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] += shfl_xor(o[h][e], msk);
  if (rs == 0) {
#pragma unroll
    for (int h = 0; h < GT; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) Ow[wv][h][cc * EPL + e] = o[h][e];
  }
  __syncthreads();
  // combine the 4 waves in order
  for (int idx = threadIdx.x; idx < G * (D + 2); idx += blockDim.x) {
    const int h = idx / (D + 2), e = idx % (D + 2);
    float Mx = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) Mx = fmaxf(Mx, Mw[w2][h]);
    float acc2 = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
      const float sc = (Mw[w2][h] == -INFINITY) ? 0.f : fast_exp2((Mw[w2][h] - Mx) * c2);
      acc2 += sc * ((e < D) ? Ow[w2][h][e] : (e == D ? 0.f : Lw[w2][h]));
    }
    part[((size_t)b * G + h) * PSTR + e] = (e == D) ? Mx : acc2;
  }
}

template <int D>
__global__ void decode_merge_kernel(const float* __restrict__ part, const int32_t* __restrict__ chunk_start, int hq,
                                    int hkv, int G, int max_chunks, float c2, float* __restrict__ out) {
  constexpr int PSTR = D + 2;
  const int inst = blockIdx.x / hq, j = blockIdx.x % hq;
  const int g = j / G, h = j % G;
  const int s = inst * hkv + g;
  const int c0 = min(chunk_start[s], max_chunks), c1 = min(chunk_start[s + 1], max_chunks);
  float Mx = -INFINITY;
  for (int cix = c0; cix < c1; ++cix) Mx = fmaxf(Mx, part[((size_t)cix * G + h) * PSTR + D]);
  for (int e = threadIdx.x; e < D; e += blockDim.x) {
    float o = 0.f, l = 0.f;
    for (int cix = c0; cix < c1; ++cix) {
      const float* pp = part + ((size_t)cix * G + h) * PSTR;
      const float sc = fast_exp2((pp[D] - Mx) * c2);
      o += sc * pp[e];
      l += sc * pp[D + 1];
    }
    out[((size_t)inst * hq + j) * D + e] = o / l;
  }
}

template <typename T, int D, int GT>
hipError_t run_decode(const Geo& g, int64_t max_rows, const void* q, const void* k_new, const void* v_new,
                      void* k_flat, void* v_flat, const int64_t* seg_start, int32_t* seg_len, float* out, char* ws,
                      hipStream_t st) {
  const int S = g.I * g.hkv;
  int32_t* chunk_start = reinterpret_cast<int32_t*>(ws);
  float* part = reinterpret_cast<float*>(ws + align_up((size_t)(S + 1) * 4, 256));
  const float c2 = (float)(1.4426950408889634 / std::sqrt((double)g.d));
  decode_prep_kernel<T, D><<<1, PT, 0, st>>>(static_cast<const T*>(k_new), static_cast<const T*>(v_new),
                                             static_cast<T*>(k_flat), static_cast<T*>(v_flat), seg_start, seg_len, S,
                                             chunk_start);
  const int64_t max_chunks = max_rows / R + S;
  decode_attn_kernel<T, D, GT><<<(unsigned)max_chunks, 256, 0, st>>>(
      static_cast<const T*>(q), static_cast<const T*>(k_flat), static_cast<const T*>(v_flat), seg_start, seg_len,
      chunk_start, S, g.hq, g.hkv, g.G, c2, part);
  decode_merge_kernel<D><<<g.I * g.hq, D < 64 ? 64 : D, 0, st>>>(part, chunk_start, g.hq, g.hkv, g.G, (int)max_chunks,
                                                                c2, out);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run_decode_g(const Geo& g, int64_t max_rows, const void* q, const void* k_new, const void* v_new,
                        void* k_flat, void* v_flat, const int64_t* seg_start, int32_t* seg_len, float* out, char* ws,
                        hipStream_t st) {
  if (g.G <= 1) return run_decode<T, D, 1>(g, max_rows, q, k_new, v_new, k_flat, v_flat, seg_start, seg_len, out, ws, st);
  if (g.G <= 2) return run_decode<T, D, 2>(g, max_rows, q, k_new, v_new, k_flat, v_flat, seg_start, seg_len, out, ws, st);
  if (g.G <= 4) return run_decode<T, D, 4>(g, max_rows, q, k_new, v_new, k_flat, v_flat, seg_start, seg_len, out, ws, st);
  return run_decode<T, D, 8>(g, max_rows, q, k_new, v_new, k_flat, v_flat, seg_start, seg_len, out, ws, st);
}

}  // namespace

size_t decode_ws_bytes(const Geo& g, int64_t max_rows) {
  const int S = g.I * g.hkv;
  const int64_t max_chunks = max_rows / R + S;
  return align_up((size_t)(S + 1) * 4, 256) + (size_t)max_chunks * g.G * (g.d + 2) * sizeof(float);
}

hipError_t launch_decode(const Geo& g, int64_t max_rows, const void* q, const void* k_new, const void* v_new,
                         void* k_flat, void* v_flat, const int64_t* seg_start, int32_t* seg_len, float* out,
                         char* ws, hipStream_t st) {
  if (g.dtype == ADAKV_BF16) {
    if (g.d == 128) return run_decode_g<uint16_t, 128>(g, max_rows, q, k_new, v_new, k_flat, v_flat, seg_start, seg_len, out, ws, st);
    if (g.d == 64) return run_decode_g<uint16_t, 64>(g, max_rows, q, k_new, v_new, k_flat, v_flat, seg_start, seg_len, out, ws, st);
  } else {
    if (g.d == 16) return run_decode_g<float, 16>(g, max_rows, q, k_new, v_new, k_flat, v_flat, seg_start, seg_len, out, ws, st);
    if (g.d == 64) return run_decode_g<float, 64>(g, max_rows, q, k_new, v_new, k_flat, v_flat, seg_start, seg_len, out, ws, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace adakv
