// Compaction of the retained rows into the flat cache on gfx950.
//
// Ada-KV notes, Algorithm 2 steps 10-11: keep the selected prefix rows and
// append the window rows; the Ada-KV paper ("Variable-length Attention with
// Variable-sized Cache Elements") stores all heads' retained caches in one
// tensor.  Segment s = i*hkv + g occupies rows seg_start[s] .. seg_start[s+1]-1:
// B_g selected rows (ascending token order), w window rows, then `reserve`
// rows kept free for decode appends.  The copy is a pure byte move: every row
// is moved by 16-byte lanes, consecutive lanes covering consecutive bytes,
// with nontemporal loads and stores (each byte is touched once here).
#include "common.hpp"
#include "kernels.hpp"

namespace adakv {
namespace {

constexpr int LT = 1024;

// Exclusive prefix sum (int64) over the workgroup in thread order.
__device__ __forceinline__ int64_t block_excl_i64(int64_t x, int64_t* wsum, int64_t& total) {
  int64_t inc = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t y = __shfl_up(inc, off);
    if ((int)__lane_id() >= off) inc += y;
  }
  const int wv = threadIdx.x / WAVE, nw = blockDim.x / WAVE;
  if ((int)__lane_id() == 63) wsum[wv] = inc;
  __syncthreads();
  int64_t before = 0, all = 0;
  for (int i = 0; i < nw; ++i) {
    before += (i < wv) ? wsum[i] : 0;
    all += wsum[i];
  }
  __syncthreads();
  total = all;
  return before + inc - x;
}

__global__ __launch_bounds__(LT) void compact_layout_kernel(const int32_t* __restrict__ budgets, int S, int w,
                                                            int reserve, int64_t* __restrict__ seg_start,
                                                            int32_t* __restrict__ seg_len) {
  __shared__ int64_t wsum[LT / WAVE];
  int64_t running = 0;
  for (int base = 0; base < S; base += LT) {
    const int s = base + threadIdx.x;
    const int len = (s < S) ? budgets[s] + w : 0;
    int64_t tot;
    const int64_t ex = block_excl_i64((s < S) ? (int64_t)len + reserve : 0, wsum, tot);
    if (s < S) {
      seg_start[s] = running + ex;
      seg_len[s] = len;
    }
    running += tot;
  }
  if (threadIdx.x == 0) seg_start[S] = running;
}

constexpr int RPW = 64;   // retained rows per copy workgroup

template <int ROWB>
__global__ __launch_bounds__(256) void compact_copy_kernel(const char* __restrict__ k, const char* __restrict__ v,
                                                           const int32_t* __restrict__ budgets,
                                                           const int32_t* __restrict__ sel,
                                                           const int64_t* __restrict__ sel_off,
                                                           const int64_t* __restrict__ seg_start, int S, int hkv,
                                                           int n, int w, int p, int reserve, int64_t total_rows,
                                                           int64_t flat_rows, char* __restrict__ kf,
                                                           char* __restrict__ vf) {
  __shared__ int64_t src_row[RPW], dst_row[RPW];
  __shared__ int s_first;
  const int64_t r0 = (int64_t)blockIdx.x * RPW;
  // packed(s) = seg_start[s] - s * reserve: first retained row of segment s,
  // strictly increasing in s (every segment holds at least its w window rows)
  auto packed = [&](int s) { return seg_start[s] - (int64_t)s * reserve; };
  if (threadIdx.x < WAVE) {
    // segment of row r0 by a 64-way search: each round one wave probes 64
    // evenly spaced segments of the range and keeps the last one at or before r0
    const int lane = threadIdx.x;
    int lo = 0, len = S;
    while (len > 1) {
      const int step = (len + WAVE - 1) / WAVE;
      const bool ok = lane * step < len && packed(lo + lane * step) <= r0;
      const uint64_t m = __ballot(ok);   // lane 0 probes lo itself: always set
      const int j = 63 - __builtin_clzll(m);
      lo += j * step;
      len = min(step, len - j * step);
    }
    if (lane == 0) s_first = lo;
  }
  __syncthreads();
  if (threadIdx.x < RPW) {
    const int64_t r = r0 + threadIdx.x;
    int64_t src = -1, dst = -1;
    if (r < total_rows) {
      int s = s_first;
      while (s + 1 < S && packed(s + 1) <= r) ++s;
      const int inst = s / hkv, g = s % hkv;
      const int64_t packed_s = packed(s);
      const int64_t j = r - packed_s;
      const int B = budgets[s];
      int64_t tok;
      if (j < B) {
        // budgets that sum past the instance's span of sel (not an allocate
        // output) leave the rows past it unwritten instead of reading beyond
        const int s0 = inst * hkv;
        const int64_t head_off = packed_s - packed(s0) - (int64_t)g * w;
        const int64_t si = sel_off[inst] + head_off + j;
        tok = si < sel_off[inst + 1] ? sel[si] : -1;
      } else {
        tok = (int64_t)p + (j - B);
      }
      dst = seg_start[s] + j;
      // rows outside the caller's flat buffer or the source head are never touched
      if (dst < flat_rows && tok >= 0 && tok < n) src = ((int64_t)inst * hkv + g) * n + tok;
      else dst = -1;
    }
    src_row[threadIdx.x] = src;
    dst_row[threadIdx.x] = dst;
  }
  __syncthreads();
  constexpr int LPR = ROWB / 16;          // lanes per row
  constexpr int RPP = 256 / LPR;          // rows per pass
  constexpr int NP = RPW / RPP;           // rows per thread
  const int rr0 = threadIdx.x / LPR, ch = threadIdx.x % LPR;
  // all of the thread's loads are issued before its first store
  u32x4 a[NP], b[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int64_t src = src_row[rr0 + i * RPP];
    if (src >= 0) {
      a[i] = ld16_nt(k + src * ROWB + ch * 16);
      b[i] = ld16_nt(v + src * ROWB + ch * 16);
    }
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int64_t src = src_row[rr0 + i * RPP], dst = dst_row[rr0 + i * RPP];
    if (src >= 0) {
      st16_nt(kf + dst * ROWB + ch * 16, a[i]);
      st16_nt(vf + dst * ROWB + ch * 16, b[i]);
    }
  }
}

// LAVa online prefill: the flat cache of layers 0..I-1 after layer I-1's
// prefill.  Rows of the newest layer (instance I-1) come from its dense K/V;
// rows of the lower layers from the previous flat cache of layers 0..I-2
// (no reserve rows), where every kept token still is: a prefix token is
// found by binary search in the head's previous ascending selection, a window
// token at its fixed place after it.  Rows past the device total or the
// buffer, and tokens missing from the previous cache, are skipped; reads stay
// inside each layer's span of sel and sel_old and inside max_rows rows of the
// previous cache even when budgets and offsets disagree.
template <int ROWB>
__global__ __launch_bounds__(256) void online_copy_kernel(
    const char* __restrict__ k_new, const char* __restrict__ v_new, const char* __restrict__ k_old,
    const char* __restrict__ v_old, const int64_t* __restrict__ seg_start_old, const int32_t* __restrict__ sel_old,
    const int64_t* __restrict__ sel_off_old, const int32_t* __restrict__ budgets, const int32_t* __restrict__ sel,
    const int64_t* __restrict__ sel_off, const int64_t* __restrict__ seg_start, int S, int hkv, int n, int w, int p,
    int64_t flat_rows, char* __restrict__ kf, char* __restrict__ vf) {
  __shared__ const char* src_k[RPW];
  __shared__ const char* src_v[RPW];
  __shared__ int64_t dst_row[RPW];
  __shared__ int s_first;
  const int64_t r0 = (int64_t)blockIdx.x * RPW;
  const int64_t total = seg_start[S];
  if (r0 >= total) return;                     // uniform across the workgroup
  if (threadIdx.x < WAVE) {
    const int lane = threadIdx.x;
    int lo = 0, len = S;
    while (len > 1) {
      const int step = (len + WAVE - 1) / WAVE;
      const bool ok = lane * step < len && seg_start[lo + lane * step] <= r0;
      const uint64_t m = __ballot(ok);
      const int j = 63 - __builtin_clzll(m);
      lo += j * step;
      len = min(step, len - j * step);
    }
    if (lane == 0) s_first = lo;
  }
  __syncthreads();
  if (threadIdx.x < RPW) {
    const int64_t r = r0 + threadIdx.x;
    const char* sk = nullptr;
    const char* sv = nullptr;
    int64_t dst = -1;
    if (r < total && r < flat_rows) {
      int s = s_first;
      while (s + 1 < S && seg_start[s + 1] <= r) ++s;
      const int inst = s / hkv, g = s % hkv, s0 = inst * hkv;
      const int64_t j = r - seg_start[s];
      const int B = budgets[s];
      int64_t tok;
      if (j < B) {
        // never past the layer's span of sel, whatever the budgets add up to
        const int64_t si = sel_off[inst] + (seg_start[s] - seg_start[s0] - (int64_t)g * w) + j;
        tok = si < sel_off[inst + 1] ? sel[si] : -1;
      } else {
        tok = (int64_t)p + (j - B);
      }
      if (inst == S / hkv - 1) {
        if (tok >= 0 && tok < n) {
          const int64_t row = (int64_t)g * n + tok;
          sk = k_new + row * ROWB;
          sv = v_new + row * ROWB;
        }
      } else {
        const int64_t ob = seg_start_old[s];
        const int64_t bold = seg_start_old[s + 1] - ob - w;
        int64_t pos = -1;
        if (tok >= p) {
          pos = bold + (tok - p);
        } else if (tok >= 0) {
          const int64_t h0 = sel_off_old[inst] + (ob - seg_start_old[s0] - (int64_t)g * w);
          // the head's previous selection, kept inside the layer's span of sel_old
          const int64_t hn = min(bold, sel_off_old[inst + 1] - h0);
          const int32_t* hs = sel_old + h0;
          int64_t lo = 0, hi = hn;               // first index with hs[index] >= tok
          while (lo < hi) {
            const int64_t mid = (lo + hi) >> 1;
            if (hs[mid] < tok) lo = mid + 1;
            else hi = mid;
          }
          if (lo < hn && hs[lo] == tok) pos = lo;
        }
        // rows of the previous cache past the buffer (max_rows, as this one) are not read
        if (pos >= 0 && pos < bold + w && ob + pos < flat_rows) {
          sk = k_old + (ob + pos) * ROWB;
          sv = v_old + (ob + pos) * ROWB;
        }
      }
      if (sk != nullptr) dst = r;
    }
    src_k[threadIdx.x] = sk;
    src_v[threadIdx.x] = sv;
    dst_row[threadIdx.x] = dst;
  }
  __syncthreads();
  constexpr int LPR = ROWB / 16;
  constexpr int RPP = 256 / LPR;
  constexpr int NP = RPW / RPP;
  const int rr0 = threadIdx.x / LPR, ch = threadIdx.x % LPR;
  u32x4 a[NP], b[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int64_t dst = dst_row[rr0 + i * RPP];
    if (dst >= 0) {
      a[i] = ld16_nt(src_k[rr0 + i * RPP] + ch * 16);
      b[i] = ld16_nt(src_v[rr0 + i * RPP] + ch * 16);
    }
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int64_t dst = dst_row[rr0 + i * RPP];
    if (dst >= 0) {
      st16_nt(kf + dst * ROWB + ch * 16, a[i]);
      st16_nt(vf + dst * ROWB + ch * 16, b[i]);
    }
  }
}

}  // namespace

hipError_t launch_online_compact(const Geo& g, int64_t max_rows, const void* k_new, const void* v_new,
                                 const void* k_old, const void* v_old, const int64_t* seg_start_old,
                                 const int32_t* sel_old, const int64_t* sel_off_old, const int32_t* budgets,
                                 const int32_t* sel, const int64_t* sel_off, void* k_flat, void* v_flat,
                                 int64_t* seg_start, int32_t* seg_len, hipStream_t st) {
  const int S = g.I * g.hkv;
  compact_layout_kernel<<<1, LT, 0, st>>>(budgets, S, g.w, 0, seg_start, seg_len);
  const int rowb = g.d * (g.dtype == ADAKV_BF16 ? 2 : 4);
  const int64_t blocks = (max_rows + RPW - 1) / RPW;
  if (blocks == 0) return hipGetLastError();
#define OCOPY(RB)                                                                                               \
  online_copy_kernel<RB><<<(unsigned)blocks, 256, 0, st>>>(                                                       \
      static_cast<const char*>(k_new), static_cast<const char*>(v_new), static_cast<const char*>(k_old),          \
      static_cast<const char*>(v_old), seg_start_old, sel_old, sel_off_old, budgets, sel, sel_off, seg_start, S,  \
      g.hkv, g.n, g.w, g.p, max_rows, static_cast<char*>(k_flat), static_cast<char*>(v_flat))
  switch (rowb) {
    case 64: OCOPY(64); break;
    case 128: OCOPY(128); break;
    case 256: OCOPY(256); break;
    case 512: OCOPY(512); break;
    default: return hipErrorInvalidValue;
  }
#undef OCOPY
  return hipGetLastError();
}

hipError_t launch_compact(const Geo& g, int64_t retained_rows, const void* k, const void* v,
                          const int32_t* budgets, const int32_t* sel, const int64_t* sel_off, int reserve,
                          void* k_flat, void* v_flat, int64_t* seg_start, int32_t* seg_len, hipStream_t st) {
  const int S = g.I * g.hkv;
  compact_layout_kernel<<<1, LT, 0, st>>>(budgets, S, g.w, reserve, seg_start, seg_len);
  const int rowb = g.d * (g.dtype == ADAKV_BF16 ? 2 : 4);
  const int64_t blocks = (retained_rows + RPW - 1) / RPW;
  const int64_t flat_rows = retained_rows + (int64_t)S * reserve;
  if (blocks == 0) return hipGetLastError();
  const char* kc = static_cast<const char*>(k);
  const char* vc = static_cast<const char*>(v);
  char* kfc = static_cast<char*>(k_flat);
  char* vfc = static_cast<char*>(v_flat);
#define COPY(RB)                                                                                                  \
  compact_copy_kernel<RB><<<(unsigned)blocks, 256, 0, st>>>(kc, vc, budgets, sel, sel_off, seg_start, S, g.hkv, g.n, \
                                                            g.w, g.p, reserve, retained_rows, flat_rows, kfc, vfc)
  switch (rowb) {
    case 64: COPY(64); break;
    case 128: COPY(128); break;
    case 256: COPY(256); break;
    case 512: COPY(512); break;
    default: return hipErrorInvalidValue;
  }
#undef COPY
  return hipGetLastError();
}

}  // namespace adakv
