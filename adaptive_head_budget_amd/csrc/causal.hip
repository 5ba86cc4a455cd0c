// The window rows' softmax normaliser over each scorer's key domain, from the
// causal one an attention pass over the prompt leaves behind.
//
// A causal prefill ends window row r (position p + r) with L, the natural-log
// log-sum-exp of its logits z_t = q.k_t / sqrt(d) over keys 0 .. p + r: the
// domain of LAVa's window weights ([LAVa-notes] Definition 1).  The Ada-KV and
// CriticalKV weights are normalised over the prefix t < p ([AdaKV-notes]
// Algorithm 2, step 2), LaProx's over all n keys ([LaProx] Section 4.1,
// Algorithm 1).  The two differ from L only by window keys, so one read of the
// w window rows of K per head fixes L:
//   prefix: L + ln(1 - sum_{t=p}^{p+r} exp(z_t - L))
//   full:   L + ln(1 + sum_{t=p+r+1}^{n-1} exp(z_t - L)).
// All of it in float64: the products of bf16 or f32 values are exact in
// float64, the dot products run in a fixed order, so the correction adds
// nothing visible to the rounding of the float32 L it starts from.  The
// subtraction scales L's absolute error by 1 / (1 - sum); rows where the prefix
// keeps less than 2^-7 of the causal mass are flagged.
//
// Layout: one workgroup of four waves per (KV head, instance).  The logits of
// the group's G*w window rows against the head's w window keys form a small
// [G*w, w] product over d, taken on v_mfma_f64_16x16x4f64 in 16 x 16 tiles
// (operands held as loaded, converted to float64 exactly as they issue; each
// lane group of 16 takes a contiguous quarter of d, an order of the d sum as
// good as any; key tiles outside every row's domain are skipped).  Each wave
// owns row tiles; per key tile a lane holds the logits of four rows against
// one key, adds exp(z - L) where the key is in its row's domain, and the 16
// lanes of a row sum in a fixed butterfly; row sums run over key tiles in
// order.  Operands come from L2 (the window is a few KiB per head): no LDS, no
// barrier.
#include <cmath>

#include "common.hpp"
#include "kernels.hpp"

namespace adakv {
namespace {

enum { DOM_CAUSAL = 0, DOM_PREFIX = 1, DOM_FULL = 2 };

typedef double f64x4 __attribute__((ext_vector_type(4)));

// S consecutive elements at src kept as loaded (16-byte loads; zeros for
// NULL), and element i of them as float64 (exact for bf16 and f32).
template <typename T, int S>
struct Chunk {
  static constexpr int PER = 16 / sizeof(T);
  static_assert(S % PER == 0, "chunk of whole 16-byte loads");
  u32x4 raw[S / PER];
  __device__ __forceinline__ void load(const T* __restrict__ src) {
#pragma unroll
    for (int c = 0; c < S / PER; ++c) raw[c] = src != nullptr ? ld16(src + c * PER) : u32x4{0u, 0u, 0u, 0u};
  }
  __device__ __forceinline__ double at(int i) const {
    if constexpr (sizeof(T) == 2) {
      const uint32_t x = raw[i / 8][(i % 8) / 2];
      return (double)__uint_as_float((i & 1) ? (x & 0xFFFF0000u) : (x << 16));
    } else {
      return (double)__uint_as_float(raw[i / 4][i % 4]);
    }
  }
};

__device__ __forceinline__ double sum16(double x) {
  // butterfly over the 16 lanes of a row group: every lane ends with the same sum
  x += __shfl_xor(x, 1, 16);
  x += __shfl_xor(x, 2, 16);
  x += __shfl_xor(x, 4, 16);
  x += __shfl_xor(x, 8, 16);
  return x;
}

template <typename T, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void causal_lse_kernel(const T* __restrict__ q_win, const T* __restrict__ k,
                                                         const float* lse_c, float* lse_out,
                                                         int32_t* __restrict__ row_flag, int hq, int hkv, int n,
                                                         int w, int dom, double inv_sqrt_d) {
  constexpr int S = D / 4;   // MFMA steps; lane group lq holds d elements [lq*S, lq*S + S)
  const int g = blockIdx.x, inst = blockIdx.y;
  const int G = hq / hkv, rows = G * w;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int li = lane & 15, lq = lane >> 4;
  const T* kg = k + (((size_t)inst * hkv + g) * n + (size_t)(n - w)) * D;   // window keys [w][D]
  const size_t row0 = ((size_t)inst * hq + (size_t)g * G) * w;              // the group's rows [G*w]
  const T* qg = q_win + row0 * D;
  const int ntile = (rows + 15) / 16, nkt = (w + 15) / 16;
  for (int rt = wv; rt < ntile; rt += 4) {
    // this lane finishes rows rt*16 + lq + 4v, v < 4: the float64 MFMA leaves result
    // row lq + 4v, column li in register v of lane 16*lq + li
    double L[4], s[4];
    int r[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = rt * 16 + lq + 4 * v;
      L[v] = row < rows ? (double)lse_c[row0 + row] : 0.0;
      r[v] = row < rows ? row % w : -1;
      s[v] = 0.0;
    }
    if (dom != DOM_CAUSAL) {
      const int ra = rt * 16 + li;   // the A row this lane supplies
      Chunk<T, S> a;
      a.load(ra < rows ? qg + (size_t)ra * D + lq * S : nullptr);
      for (int kt = 0; kt < nkt; ++kt) {
        // key tiles that hold no key of any domain in the row tile are skipped
        bool need = false;
#pragma unroll
        for (int v = 0; v < 4; ++v)
          need |= r[v] >= 0 && (dom == DOM_PREFIX ? kt * 16 <= r[v] : kt * 16 + 15 > r[v]);
        if (!__any(need)) continue;
        const int j = kt * 16 + li;   // window key of this lane's B column and result column
        Chunk<T, S> b;
        b.load(j < w ? kg + (size_t)j * D + lq * S : nullptr);
        // operands stay as loaded and become float64 four steps at a time, next
        // to the MFMAs that take them (the empty asm keeps a's float64 form
        // from being made once for all key tiles: 2*S registers)
#pragma unroll
        for (int c = 0; c < S / Chunk<T, S>::PER; ++c) asm volatile("" : "+v"(a.raw[c]));
        f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int st0 = 0; st0 < S; st0 += 4) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int st = st0; st < st0 + 4; ++st)
            acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a.at(st), b.at(st), acc, 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const bool in = r[v] >= 0 && j < w && std::isfinite(L[v]) && (dom == DOM_PREFIX ? j <= r[v] : j > r[v]);
          const double e = in ? exp(acc[v] * inv_sqrt_d - L[v]) : 0.0;
          s[v] += sum16(e);
        }
      }
    }
    if (li == 0) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (r[v] < 0) continue;
        double out = L[v];
        int flag = 0;
        if (!std::isfinite(L[v])) {
          flag = 2;
        } else if (dom == DOM_PREFIX) {
          double keep = 1.0 - s[v];
          if (!(keep >= 0x1p-7)) flag = 1;
          if (!(keep >= 0x1p-60)) keep = 0x1p-60;   // rounding in L left no prefix mass
          out = L[v] + log(keep);
        } else if (dom == DOM_FULL) {
          out = L[v] + log1p(s[v]);
        }
        if (!std::isfinite(out)) {
          flag = 2;
          out = L[v];
        }
        const size_t row = row0 + rt * 16 + lq + 4 * v;
        lse_out[row] = (float)out;
        if (row_flag != nullptr) row_flag[row] = flag;
      }
    }
  }
}

template <typename T, int D>
hipError_t run(const Geo& g, const void* q_win, const void* k, const float* lse_c, float* lse_out,
               int32_t* row_flag, int dom, hipStream_t st) {
  causal_lse_kernel<T, D><<<dim3(g.hkv, g.I), 4 * WAVE, 0, st>>>(
      static_cast<const T*>(q_win), static_cast<const T*>(k), lse_c, lse_out, row_flag, g.hq, g.hkv, g.n, g.w, dom,
      1.0 / std::sqrt((double)g.d));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_from_causal(const Geo& g, const void* q_win, const void* k, const float* lse_c,
                                  float* lse_out, int32_t* row_flag, hipStream_t st) {
  const int dom = g.scorer == ADAKV_SCORE_LAVA     ? DOM_CAUSAL
                  : g.scorer == ADAKV_SCORE_LAPROX ? DOM_FULL
                                                   : DOM_PREFIX;
  if (g.dtype == ADAKV_BF16) {
    if (g.d == 128) return run<uint16_t, 128>(g, q_win, k, lse_c, lse_out, row_flag, dom, st);
    if (g.d == 64) return run<uint16_t, 64>(g, q_win, k, lse_c, lse_out, row_flag, dom, st);
  } else {
    if (g.d == 64) return run<float, 64>(g, q_win, k, lse_c, lse_out, row_flag, dom, st);
    if (g.d == 16) return run<float, 16>(g, q_win, k, lse_c, lse_out, row_flag, dom, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace adakv
