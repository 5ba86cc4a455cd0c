// Budget allocation and selection on gfx950.
//
// Top-k over non-negative fp32 scores is a radix select on the bit patterns,
// most significant digit first: bits [30:20], [19:9], [8:0] (bit 31 is zero for
// every non-negative score).  The select yields a threshold key T and the number
// of entries equal to T that are kept; entries equal to T are kept in index
// order, so the result is the first k of the order (-score, index) and is
// exactly reproducible.
//
// Every streaming pass is spread over the whole chip: a score row (one KV head
// of one instance) is cut into chunks of up to 4096 scores, one workgroup per
// chunk, each thread holding up to 16 consecutive scores.  A segment is the unit
// a top-k runs over: an instance (all its heads, for the layer-wide top-B) or a
// single row (a head's own top-k).  Chunks add their digit histogram into the
// segment's histogram with global atomics and end; a small kernel with one
// workgroup per segment then picks the digit and clears the histogram for the
// next pass.  No workgroup ever waits for another.
//
// The first digit pass of every selection reads every score once; a negative
// (other than -0), NaN or infinite one sets the int32 at the start of the
// workspace (cleared at the start of the call).  Such keys stay plain uint32
// patterns (negatives count as zero), so the selection stays in bounds.
//
// Definitions followed:
//  * Ada-KV notes, Algorithm 1 (concatenate the heads, top-B, count per head)
//    and Algorithm 2 steps 6-9 (window out of the budget, safeguard, per-head
//    top-k); the safeguard alpha*f + (1-alpha)*B/h is made integer exactly.
//  * LAVa notes, "动态头预算的逐层缓存驱逐" (flattened layer top-k, no safeguard)
//    and "基于不确定性的层预算分配" (entropy-proportional layer budgets).
//  * CriticalKV notes, "两阶段贪心选择算法" (top-b' by attention, then top-b''
//    of the rest by the composite score).
//  * LaProx page, Algorithm 1 (TopK(p, B_total), window tokens at infinity)
//    with the abstract's model-wide selection: one top-k over every head of
//    every instance of the call.
//  * The safeguard read as a floor (Ada-KV notes, Algorithm 2 step 8: no head
//    may get too small a budget): each head's own top floor(alpha*P/h) first,
//    then Algorithm 1 over the remaining entries of all heads.
//  * StreamingLLM (Ada-KV paper, "Baselines" / "Parameters"): sink tokens and
//    the most recent ones, the prefix share split evenly over the heads.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace adakv {
namespace {

constexpr int SB = 256;             // threads of a selection workgroup
constexpr int SW = SB / WAVE;       // waves
constexpr int TILE = SB * 4;        // scores per chunk for each unit of ntile
constexpr int MAXT = 4;             // ntile <= MAXT: up to 4 * MAXT consecutive scores per thread
constexpr int NK = 4 * MAXT;
constexpr int NBIN = 2048;          // histogram bins (11-bit digits)
constexpr uint32_t NONE = 0xFFFFFFFFu;

struct RState {                     // radix state of a segment
  uint32_t prefix;                  // digits fixed so far; after the last pass: T (NONE = take nothing)
  int32_t krem;                     // entries still to take below the prefix; at the end: ties to keep
};

// Keys of the select: the bit pattern of a non-negative float orders like its
// value.  Negative inputs (outside the scores' domain) count as zero.
__device__ __forceinline__ uint32_t sel_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u >> 31) ? 0u : u;
}

__device__ __forceinline__ int digit_shift(int ps) { return ps == 0 ? 20 : (ps == 1 ? 9 : 0); }
__device__ __forceinline__ uint32_t digit_of(uint32_t u, int ps) {
  return ps == 0 ? (u >> 20) : (ps == 1 ? ((u >> 9) & 2047u) : (u & 511u));
}
__device__ __forceinline__ bool in_prefix(uint32_t u, uint32_t prefix, int ps) {
  return ps == 0 ? true : (ps == 1 ? ((u >> 20) == (prefix >> 20)) : ((u >> 9) == (prefix >> 9)));
}
__device__ __forceinline__ int pass_bins(int ps) { return ps == 2 ? 512 : NBIN; }

// Exclusive scan over the 64 lanes of a wave (lane 0 first).
__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t x) {
  uint32_t inc = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)inc, off);
    if ((int)__lane_id() >= off) inc += y;
  }
  return inc - x;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += (uint32_t)__shfl_xor((int)x, off);
  return x;
}

// Exclusive scan over the workgroup in thread order, plus the total.  sh: SW words.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* sh, uint32_t& total) {
  const uint32_t ex = wave_excl_scan(x);
  const int wv = threadIdx.x / WAVE;
  if ((threadIdx.x & (WAVE - 1)) == WAVE - 1) sh[wv] = ex + x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < SW; ++i) {
    const uint32_t s = sh[i];
    before += (i < wv) ? s : 0u;
    all += s;
  }
  __syncthreads();
  total = all;
  return before + ex;
}

__device__ __forceinline__ uint32_t block_sum(uint32_t x, uint32_t* sh) {
  uint32_t t;
  block_excl_scan(x, sh, t);
  return t;
}

// Digit pick over nb bins (bin(b) gives the count of digit b): the digit d with
// count(> d) < krem <= count(>= d).  Returns d and count(> d) to every thread.
// sh: SW + 2 words.
template <class BinF>
__device__ void block_pick(BinF bin, int nb, uint32_t krem, uint32_t* sh, uint32_t& dig, uint32_t& above_out) {
  const int bpt = nb / SB;            // 8 or 2 bins per thread, from the top
  uint32_t c[8];
  uint32_t s = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    c[j] = (j < bpt) ? bin(nb - 1 - ((int)threadIdx.x * bpt + j)) : 0u;
    s += c[j];
  }
  if (threadIdx.x == 0) { sh[SW] = 0u; sh[SW + 1] = 0u; }
  uint32_t total;
  uint32_t above = block_excl_scan(s, sh, total);
  if (above < krem && krem <= above + s) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < bpt && above < krem && krem <= above + c[j]) {
        sh[SW] = (uint32_t)(nb - 1 - ((int)threadIdx.x * bpt + j));
        sh[SW + 1] = above;
      }
      above += c[j];
    }
  }
  __syncthreads();
  dig = sh[SW];
  above_out = sh[SW + 1];
  __syncthreads();
}

// The chunk of a workgroup: row r, scores [e_begin, e_end) of the row.
struct Chunk {
  int r, c, e_begin, e_end;
};
__device__ __forceinline__ Chunk chunk_of(int cpr, int ntile, int p) {
  Chunk k;
  k.r = blockIdx.x / cpr;
  k.c = blockIdx.x % cpr;
  k.e_begin = k.c * ntile * TILE;
  k.e_end = min(p, k.e_begin + ntile * TILE);
  return k;
}

// The thread's scores: [e0, e0 + 4*ntile) with e0 = e_begin + 4*ntile*tid, in
// index order; the first n of them lie inside the chunk.  Every load is issued
// before any is used: addresses past the chunk are clamped to its last score
// (16-byte groups for rows of a multiple of 4 scores on a 16-byte aligned base,
// single scores otherwise), so a partial chunk costs no more than a full one.
// CHECK: `bad` is nonzero when a loaded score breaks the precondition
// (negative other than -0, NaN or infinite); clamped duplicates repeat scores
// of the chunk, so they need no mask.
struct ChunkKeys {
  uint32_t k[NK];
  int e0, n;
  uint32_t bad;
};
__device__ __forceinline__ uint32_t bad_score(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u > 0x80000000u || (u & 0x7FFFFFFFu) >= 0x7F800000u) ? 1u : 0u;
}
template <bool CHECK = false>
__device__ __forceinline__ void load_chunk(const float* row, const Chunk& ch, int ntile, bool vec, ChunkKeys& K) {
  K.bad = 0u;
  const int npt = 4 * ntile;
  K.e0 = ch.e_begin + npt * (int)threadIdx.x;
  K.n = max(0, min(npt, ch.e_end - K.e0));
  if (vec) {
    f32x4 v[MAXT];
#pragma unroll
    for (int t = 0; t < MAXT; ++t)
      v[t] = *reinterpret_cast<const f32x4*>(row + min(K.e0 + 4 * (t < ntile ? t : 0), ch.e_end - 4));
#pragma unroll
    for (int t = 0; t < MAXT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        K.k[4 * t + j] = sel_key(v[t][j]);
        if (CHECK) K.bad |= bad_score(v[t][j]);
      }
    return;
  }
  float v[NK];
#pragma unroll
  for (int j = 0; j < NK; ++j) v[j] = row[min(K.e0 + (j < npt ? j : 0), ch.e_end - 1)];
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    K.k[j] = sel_key(v[j]);
    if (CHECK) K.bad |= bad_score(v[j]);
  }
}

// Member flags of the thread's scores (CriticalKV stage 1), clamped like the scores.
__device__ __forceinline__ void load_member(const uint8_t* mrow, const Chunk& ch, int ntile, bool vec,
                                            const ChunkKeys& K, uint8_t m[NK]) {
  if (vec) {
    uint32_t w[MAXT];
#pragma unroll
    for (int t = 0; t < MAXT; ++t)
      w[t] = *reinterpret_cast<const uint32_t*>(mrow + min(K.e0 + 4 * (t < ntile ? t : 0), ch.e_end - 4));
#pragma unroll
    for (int t = 0; t < MAXT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) m[4 * t + j] = (uint8_t)((w[t] >> (8 * j)) & 255u);
    return;
  }
#pragma unroll
  for (int j = 0; j < NK; ++j) m[j] = mrow[min(K.e0 + (j < 4 * ntile ? j : 0), ch.e_end - 1)];
}

// Counts the chunk's eligible digits into the LDS histogram h.  A thread's
// scores are neighbours in the row (pooled scores come in plateaus), so equal
// digits in a row of them go in with one atomic.
__device__ __forceinline__ void chunk_hist(uint32_t* h, const ChunkKeys& K, const uint8_t (&m)[NK], bool use_m,
                                           uint32_t prefix, int ps) {
  uint32_t cur = NONE, run = 0;
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    const uint32_t u = K.k[j];
    const bool el = j < K.n && (!use_m || m[j] == 0) && in_prefix(u, prefix, ps);
    const uint32_t d = el ? digit_of(u, ps) : NONE;
    if (d != cur) {
      if (cur != NONE) atomicAdd(h + cur, run);
      cur = d;
      run = 0;
    }
    ++run;
  }
  if (cur != NONE) atomicAdd(h + cur, run);
}

// Picks the digit of pass ps from the histogram hs (global, complete) and
// clears it, also for a segment with nothing left to take (a first-pass
// histogram holds counts even then).  st is the state before the pass.
__device__ __forceinline__ RState pick_and_clear(uint32_t* hs, int ps, RState st, uint32_t* sh) {
  const int nb = pass_bins(ps);
  RState out = {NONE, 0};
  if (st.krem > 0 && st.prefix != NONE) {
    uint32_t d, above;
    block_pick([&](int b) { return hs[b]; }, nb, (uint32_t)st.krem, sh, d, above);
    out.prefix = st.prefix | (d << digit_shift(ps));
    out.krem = st.krem - (int32_t)above;
  }
  for (int b = threadIdx.x; b < nb; b += SB) hs[b] = 0u;
  return out;
}

// The pick of pass ps from a complete histogram hs that stays as it is: every
// workgroup of the launch after a digit pass forms the same pick itself, so no
// launch of its own is needed for it.  st is the state before the pass.
__device__ __forceinline__ RState pick_keep(const uint32_t* __restrict__ hs, int ps, RState st, uint32_t* sh) {
  RState out = {NONE, 0};
  if (st.krem > 0 && st.prefix != NONE) {   // uniform
    uint32_t d, above;
    block_pick([&](int b) { return hs[b]; }, pass_bins(ps), (uint32_t)st.krem, sh, d, above);
    out.prefix = st.prefix | (d << digit_shift(ps));
    out.krem = st.krem - (int32_t)above;
  }
  return out;
}

// ---------------------------------------------------------------- zero fill
__global__ __launch_bounds__(SB) void sel_zero_kernel(u32x4* __restrict__ p, size_t n16) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (size_t i = (size_t)blockIdx.x * SB + threadIdx.x; i < n16; i += (size_t)gridDim.x * SB) p[i] = z;
}

// ---------------------------------------------------------------- digit histograms
// Adds the chunk's LDS histogram (nb bins) into the global one.
__device__ __forceinline__ void flush_hist(const uint32_t* h, uint32_t* hg, int nb) {
  for (int b = threadIdx.x; b < nb; b += SB) {
    const uint32_t v = h[b];
    if (v) atomicAdd(hg + b, v);
  }
}

// One digit pass over segments of seg_rows rows: the histogram of the digits
// of pass PS among the candidates that match the segment's prefix.  Pass 0
// takes k from kinit[segment] (kconst when kinit is NULL), later passes
// continue from st[segment].  With member flags (USE_M), flagged scores are not
// candidates.  The pass and the flags are compile-time: with them at run time
// the per-score loop compiles to a chain of divergent branches that costs more
// than the chunk's load.  pick_hist (later passes): st is the state before the
// previous pass, whose digit every workgroup picks from pick_hist (that pass's
// complete histograms); the segment's first chunk stores the result in st_out.
template <int PS, bool USE_M>
__global__ __launch_bounds__(SB) void radix_hist_kernel(const float* __restrict__ score,
                                                        const uint8_t* __restrict__ member, int p, int cpr,
                                                        int ntile, int vec, int seg_rows,
                                                        const int32_t* __restrict__ kinit, int kconst,
                                                        const RState* __restrict__ st, uint32_t* __restrict__ hist,
                                                        uint32_t* __restrict__ flag,
                                                        const uint32_t* __restrict__ pick_hist,
                                                        RState* __restrict__ st_out) {
  __shared__ uint32_t h[NBIN];
  __shared__ uint32_t sh[SW + 4];
  const Chunk ch = chunk_of(cpr, ntile, p);
  const int s = ch.r / seg_rows;
  ChunkKeys K;
  uint8_t m[NK];
  load_chunk<PS == 0>(score + (size_t)ch.r * p, ch, ntile, vec != 0, K);
  if (PS == 0 && K.bad) atomicOr(flag, 1u);   // precondition broken somewhere in the chunk
  if (USE_M) load_member(member + (size_t)ch.r * p, ch, ntile, vec != 0, K, m);
  RState cur;
  if (PS == 0) {
    cur.prefix = 0u;
    cur.krem = kinit ? kinit[s] : kconst;
  } else {
    cur = st[s];
    if (pick_hist != nullptr) {
      cur = pick_keep(pick_hist + (size_t)s * NBIN, PS - 1, cur, sh);
      if (threadIdx.x == 0 && ch.r % seg_rows == 0 && ch.c == 0) st_out[s] = cur;
    }
  }
  if (cur.krem <= 0 || cur.prefix == NONE) return;
  constexpr int nb = PS == 2 ? 512 : NBIN;
  bool el[NK];
  int any = 0;
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    el[j] = j < K.n && (!USE_M || m[j] == 0) && in_prefix(K.k[j], cur.prefix, PS);
    any |= el[j] ? 1 : 0;
  }
  // after the first digit most chunks hold no candidate: no histogram then
  if (PS > 0 && !__syncthreads_or(any)) return;
  for (int b = threadIdx.x; b < nb; b += SB) h[b] = 0u;
  __syncthreads();
  if (PS == 0) {
    chunk_hist(h, K, m, USE_M, 0u, 0);
  } else {
    // candidates are sparse: one masked atomic each, no run merging
#pragma unroll
    for (int j = 0; j < NK; ++j)
      if (el[j]) atomicAdd(h + digit_of(K.k[j], PS), 1u);
  }
  __syncthreads();
  flush_hist(h, hist + (size_t)s * NBIN, nb);
}

// Launches the digit pass ps (0..2) with or without member flags.
void radix_hist(int nc, hipStream_t stream, const float* score, const uint8_t* member, int p, int cpr, int ntile,
                int vec, int seg_rows, int ps, const int32_t* kinit, int kconst, const RState* st, uint32_t* hist,
                uint32_t* flag, const uint32_t* pick_hist = nullptr, RState* st_out = nullptr) {
#define RH(PSV, M)                                                                                       \
  radix_hist_kernel<PSV, M><<<nc, SB, 0, stream>>>(score, member, p, cpr, ntile, vec, seg_rows, kinit, kconst, st, hist, \
                                                   flag, pick_hist, st_out)
  if (member != nullptr) {
    if (ps == 0) RH(0, true); else if (ps == 1) RH(1, true); else RH(2, true);
  } else {
    if (ps == 0) RH(0, false); else if (ps == 1) RH(1, false); else RH(2, false);
  }
#undef RH
}

// The digit pick of pass ps for every segment, one workgroup each; pass 0
// starts from kinit[segment].
__global__ __launch_bounds__(SB) void radix_pick_kernel(uint32_t* __restrict__ hist, int ps,
                                                        const int32_t* __restrict__ kinit, int kconst,
                                                        RState* __restrict__ st) {
  __shared__ uint32_t sh[SW + 4];
  const int s = blockIdx.x;
  RState cur;
  if (ps == 0) {
    cur.prefix = 0u;
    cur.krem = kinit ? kinit[s] : kconst;
  } else {
    cur = st[s];
  }
  const RState nx = pick_and_clear(hist + (size_t)s * NBIN, ps, cur, sh);
  if (threadIdx.x == 0) st[s] = nx;
}

// ---------------------------------------------------------------- layer pass 0
// ln of a positive normal float v = 2^e m: with m_hi = 1 + k/256 (k the top 8
// bits of the mantissa) and m = m_hi (1 + d), 0 <= d < 2^-8,
// ln v = e ln 2 + ln m_hi + ln(1 + d); ln m_hi and 1/m_hi come from tables, and
// ln(1 + d) from its Taylor series up to d^7 (the rest is below 2^-56
// relative).  m - m_hi is exact; a subnormal v takes the library ln.
__device__ __forceinline__ double ln_float(uint32_t u, double v, const double* __restrict__ ltab,
                                           const double* __restrict__ itab) {
  const int ex = (int)(u >> 23);
  if (ex == 0) return log(v);
  const uint32_t mb = u & 0x7FFFFFu;
  const int k = (int)(mb >> 15);
  const double d = (double)(mb & 0x7FFFu) * 0x1p-23 * itab[k];
  const double l1p =
      d * (1.0 + d * (-0.5 + d * (1.0 / 3.0 + d * (-0.25 + d * (0.2 + d * (-1.0 / 6.0 + d * (1.0 / 7.0)))))));
  return (double)(ex - 127) * 0.69314718055994530942 + ltab[k] + l1p;
}

// First digit pass of the layer-wide top-k, kept per row (the row histograms
// also serve each head's own top-k later).  For LAVa each chunk from ent_chunk0
// on also leaves its partial sums S = sum s and Q = sum s ln s (fp64) for the
// layer entropy, at part[2 * (chunk - ent_chunk0)] (the online prefill takes
// the older layers' entropies from its cache and sums the newest layer only).
__global__ __launch_bounds__(SB) void layer_hist0_kernel(const float* __restrict__ score, int p, int cpr, int ntile,
                                                         int vec, int lava_in, int ent_chunk0,
                                                         uint32_t* __restrict__ rowhist, double* __restrict__ part,
                                                         uint32_t* __restrict__ flag) {
  const bool lava = lava_in != 0 && (int)blockIdx.x >= ent_chunk0;   // uniform over the workgroup
  __shared__ uint32_t h[NBIN];
  __shared__ double dsh[2][SW];
  __shared__ double ltab[SB], itab[SB];   // ln(1 + k/256) and 1/(1 + k/256), k < 256 (LAVa)
  static_assert(SB == 256, "one table entry per thread");
  const Chunk ch = chunk_of(cpr, ntile, p);
  ChunkKeys K;
  uint8_t m[NK];
  load_chunk<true>(score + (size_t)ch.r * p, ch, ntile, vec != 0, K);
  if (K.bad) atomicOr(flag, 1u);   // precondition broken somewhere in the chunk
  for (int b = threadIdx.x; b < NBIN; b += SB) h[b] = 0u;
  if (lava) {
    const double mh = 1.0 + (double)threadIdx.x * 0x1p-8;
    ltab[threadIdx.x] = log(mh);
    itab[threadIdx.x] = 1.0 / mh;
  }
  __syncthreads();
  chunk_hist(h, K, m, false, 0u, 0);
  if (lava) {
    double S = 0.0, Q = 0.0;
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const double v = (double)__uint_as_float(K.k[j]);
      if (j < K.n && v > 0.0) {
        S += v;
        Q += v * ln_float(K.k[j], v, ltab, itab);
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      S += __shfl_xor(S, off);
      Q += __shfl_xor(Q, off);
    }
    const int wv = threadIdx.x / WAVE;
    if ((threadIdx.x & (WAVE - 1)) == 0) { dsh[0][wv] = S; dsh[1][wv] = Q; }
  }
  __syncthreads();
  if (lava && threadIdx.x == 0) {
    double s2 = 0.0, q2 = 0.0;
    for (int i = 0; i < SW; ++i) { s2 += dsh[0][i]; q2 += dsh[1][i]; }
    part[2 * (size_t)(blockIdx.x - ent_chunk0)] = s2;
    part[2 * (size_t)(blockIdx.x - ent_chunk0) + 1] = q2;
  }
  flush_hist(h, rowhist + (size_t)ch.r * NBIN, NBIN);
}

// First digit pick of every layer-wide top-k (one workgroup per instance) from
// the sum of its rows' histograms, with k = kP, or klist[instance] for LAVa.
// The row histograms are kept.
__device__ __forceinline__ void layer_pick0_of(const uint32_t* __restrict__ h0, int hkv, int k,
                                               RState* __restrict__ out) {
  __shared__ uint32_t sh[SW + 4];
  if (k <= 0) {                                  // uniform
    if (threadIdx.x == 0) { RState none = {NONE, 0}; *out = none; }
    return;
  }
  // the instance's pass-0 histogram: its rows' histograms added bin by bin,
  // 32 independent loads in flight per thread, into LDS
  __shared__ uint32_t hsum[NBIN];
  uint32_t t[NBIN / SB];
#pragma unroll
  for (int j = 0; j < NBIN / SB; ++j) t[j] = 0u;
  for (int g0 = 0; g0 < hkv; g0 += 4) {
    uint32_t x[4][NBIN / SB];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < NBIN / SB; ++j)
        x[u][j] = (g0 + u < hkv) ? h0[(size_t)(g0 + u) * NBIN + (int)threadIdx.x + SB * j] : 0u;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < NBIN / SB; ++j) t[j] += x[u][j];
  }
#pragma unroll
  for (int j = 0; j < NBIN / SB; ++j) hsum[(int)threadIdx.x + SB * j] = t[j];
  __syncthreads();
  uint32_t d, above;
  block_pick([&](int b) { return hsum[b]; }, NBIN, (uint32_t)k, sh, d, above);
  if (threadIdx.x == 0) { RState x = {d << 20, k - (int32_t)above}; *out = x; }
}

__global__ __launch_bounds__(SB) void layer_pick0_kernel(const uint32_t* __restrict__ rowhist, int hkv, int kP,
                                                         const int64_t* __restrict__ klist, RState* __restrict__ seg) {
  const int inst = blockIdx.x;
  layer_pick0_of(rowhist + (size_t)inst * hkv * NBIN, hkv, klist ? (int)klist[inst] : kP, seg + inst);
}

// LAVa: per layer, S and Q from the chunk partials in a fixed order,
// e_l = (ln S - Q / S) / (hkv * p); then B'_l = largest remainder of
// B' * e_l / sum(e) (equal remainders: lower layer first) and sel_off = scan.
// online: the LAVa online prefill (LAVa notes, "在线预填充与层预算调整"): each
// layer's budget is capped by its budget of the previous step, read from that
// step's offsets prev_off [L] (layers 0..L-2; NULL when L == 1), and by its
// prefix hkv * p; the newest layer (L-1) only by hkv * p.
// Layers below `first` take e_l from ent (each layer's entropy as the step that
// first saw it computed it); part holds the partials of layers first..L-1, and
// their e_l are written to ent when it is given.
__global__ __launch_bounds__(SB) void lava_budget_kernel(const double* __restrict__ part, int L, int chunks_per_layer,
                                                         int hkv, int p, int64_t Bp, int online,
                                                         const int64_t* __restrict__ prev_off, int first,
                                                         double* __restrict__ ent, int64_t* __restrict__ klist,
                                                         int64_t* __restrict__ sel_off,
                                                         const uint32_t* __restrict__ pick_rowhist,
                                                         RState* __restrict__ pick_out) {
  extern __shared__ __align__(16) char smem[];
  double* rem = reinterpret_cast<double*>(smem);     // e_l first, then the remainders
  int64_t* fl = reinterpret_cast<int64_t*>(rem + L);
  __shared__ double Esh;
  __shared__ int64_t def, klast;
  // one wave per layer: lane-strided sums over the layer's chunk partials,
  // then a fixed butterfly (the same order on every run)
  {
    const int lane = threadIdx.x & (WAVE - 1), wv = threadIdx.x / WAVE;
    for (int l = wv; l < L; l += SW) {
      if (l < first) {                      // wave-uniform
        if (lane == 0) rem[l] = ent[l];
        continue;
      }
      double S = 0.0, Q = 0.0;
      const double* pl = part + 2 * (size_t)(l - first) * chunks_per_layer;
      for (int c = lane; c < chunks_per_layer; c += WAVE) { S += pl[2 * c]; Q += pl[2 * c + 1]; }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        S += __shfl_xor(S, off);
        Q += __shfl_xor(Q, off);
      }
      if (lane == 0) {
        const double e = (S > 0.0) ? (log(S) - Q / S) / ((double)hkv * (double)p) : 0.0;
        rem[l] = e;
        if (ent != nullptr) ent[l] = e;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double E = 0.0;
    for (int i = 0; i < L; ++i) E += rem[i];
    Esh = E;
  }
  __syncthreads();
  const double E = Esh;
  for (int l = threadIdx.x; l < L; l += SB) {
    // kept inside [0, B']: an entropy of exactly 0 can round to -tiny, and a NaN
    // share (an infinite score breaking the precondition) counts as 0
    const double x = fmin(fmax((E > 0.0) ? ((double)Bp * rem[l]) / E : (double)Bp / (double)L, 0.0), (double)Bp);
    const double f = floor(x);
    fl[l] = (int64_t)f;
    rem[l] = x - f;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t s = 0;
    for (int i = 0; i < L; ++i) s += fl[i];
    def = Bp - s;
  }
  __syncthreads();
  for (int l = threadIdx.x; l < L; l += SB) {
    int64_t rank = 0;
    for (int j = 0; j < L; ++j) rank += (rem[j] > rem[l] || (rem[j] == rem[l] && j < l)) ? 1 : 0;
    int64_t k = fl[l] + (rank < def ? 1 : 0);
    if (online) {
      int64_t cap = (int64_t)hkv * p;
      if (l < L - 1 && prev_off != nullptr) cap = min(cap, prev_off[l + 1] - prev_off[l]);
      k = min(k, cap);
    }
    klist[l] = k;
    if (l == L - 1) klast = k;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t s = 0;
    for (int i = 0; i < L; ++i) { sel_off[i] = s; s += klist[i]; }
    sel_off[L] = s;
  }
  // with pick_rowhist (a call that selects in the newest layer alone): that
  // layer's first digit, from its rows' pass-0 histograms
  if (pick_rowhist != nullptr) layer_pick0_of(pick_rowhist, hkv, (int)klast, pick_out);
}

// ---------------------------------------------------------------- layer counts and budgets
enum { MODE_ADA = 0, MODE_CK = 2 };   // the row budget kernel's two kinds of row

// Per row: entries above its segment's threshold T and equal to it (a segment
// is seg_rows consecutive rows: one instance, or every row of the call).  With
// member flags, flagged entries are not counted.  pick_hist: seg is the state
// before the last digit pass, whose digit every workgroup picks from pick_hist
// (the complete last-pass histograms); the segment's first chunk stores the
// final state in seg_out.  cc_out: the chunk's own two counts as well (what
// chunk_count_kernel gives for rows that keep the segment's threshold).
__global__ __launch_bounds__(SB) void layer_count_kernel(const float* __restrict__ score,
                                                         const uint8_t* __restrict__ member, int p, int cpr,
                                                         int ntile, int vec, int seg_rows,
                                                         const RState* __restrict__ seg, uint32_t* __restrict__ cnt,
                                                         const uint32_t* __restrict__ pick_hist,
                                                         RState* __restrict__ seg_out, uint32_t* __restrict__ cc_out) {
  __shared__ uint32_t sh[SW + 4];
  const Chunk ch = chunk_of(cpr, ntile, p);
  ChunkKeys K;
  uint8_t m[NK];
  load_chunk(score + (size_t)ch.r * p, ch, ntile, vec != 0, K);
  if (member) load_member(member + (size_t)ch.r * p, ch, ntile, vec != 0, K, m);
  const int sg = ch.r / seg_rows;
  RState L = seg[sg];
  if (pick_hist != nullptr) {
    L = pick_keep(pick_hist + (size_t)sg * NBIN, 2, L, sh);
    if (threadIdx.x == 0 && ch.r % seg_rows == 0 && ch.c == 0) seg_out[sg] = L;
  }
  if (L.prefix == NONE) {                      // uniform
    if (cc_out != nullptr && threadIdx.x == 0) {
      cc_out[2 * (size_t)blockIdx.x] = 0u;
      cc_out[2 * (size_t)blockIdx.x + 1] = 0u;
    }
    return;
  }
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    const bool ok = j < K.n && (member == nullptr || m[j] == 0);
    gt += (ok && K.k[j] > L.prefix) ? 1u : 0u;
    eq += (ok && K.k[j] == L.prefix) ? 1u : 0u;
  }
  const uint32_t both = block_sum(gt | (eq << 16), sh);   // at most 4096 of each
  if (threadIdx.x == 0) {
    if (both & 0xFFFFu) atomicAdd(cnt + 2 * (size_t)ch.r, both & 0xFFFFu);
    if (both >> 16) atomicAdd(cnt + 2 * (size_t)ch.r + 1, both >> 16);
    if (cc_out != nullptr) {
      cc_out[2 * (size_t)blockIdx.x] = both & 0xFFFFu;
      cc_out[2 * (size_t)blockIdx.x + 1] = both >> 16;
    }
  }
}

// One workgroup per row r (head g of instance i), Ada-KV and CriticalKV.  From
// the counts of the instance's rows: the heads' layer counts f_g (ties shared
// out in flat index order), the budget B_g by the safeguard, the row's offset
// in sel, the row's k for its own top-k (B_g, or b'_g = floor(B_g * ck_num /
// ck_den) for CriticalKV stage 1, b''_g = B_g - b'_g kept for stage 2) and the
// first digit pick of that top-k from the row's pass-0 histogram.  (LAVa rows
// keep the layer threshold: lava_emit_kernel forms their budgets.)  Every
// workgroup of an instance computes the same head values.
__global__ __launch_bounds__(SB) void row_budget_kernel(int hkv, int mode, int kP0, int alpha_num, int alpha_den,
                                                        int ck_num, int ck_den, int n_inst,
                                                        const int64_t* __restrict__ klist,
                                                        const int64_t* __restrict__ kbase,
                                                        const RState* __restrict__ seg,
                                                        const uint32_t* __restrict__ cnt,
                                                        uint32_t* __restrict__ rowhist, int32_t* __restrict__ budgets,
                                                        int64_t* __restrict__ rowbase, int32_t* __restrict__ rowk2,
                                                        RState* __restrict__ rowst, int64_t* __restrict__ sel_off) {
  __shared__ uint32_t sh[SW + 4];
  __shared__ int64_t gt_sh[256], eq_sh[256], f_sh[256], q_sh[256], r_sh[256];
  __shared__ int64_t k1_sh, def_sh;
  const int r = blockIdx.x, inst = r / hkv, g = r % hkv, r0 = inst * hkv;
  const RState L = seg[inst];
  // this instance's prefix budget and first position in sel (per-instance
  // budgets: klist / kbase; else the same P for every instance)
  const int64_t kP = klist ? klist[inst] : (int64_t)kP0;
  const int64_t kb0 = kbase ? kbase[inst] : (int64_t)inst * kP0;
  for (int j = threadIdx.x; j < hkv; j += SB) {
    gt_sh[j] = cnt[2 * (size_t)(r0 + j)];
    eq_sh[j] = cnt[2 * (size_t)(r0 + j) + 1];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int64_t quota = (L.prefix == NONE) ? 0 : L.krem;
    int64_t before = 0;
    for (int j = 0; j < hkv; ++j) {
      int64_t share = quota - before;
      share = share < 0 ? 0 : (share > eq_sh[j] ? eq_sh[j] : share);
      before += eq_sh[j];
      f_sh[j] = gt_sh[j] + share;
    }
  }
  __syncthreads();
  // Safeguard in exact integers: N_g = a*h*f_g + (b-a)*P over Den = b*h, floors
  // plus one unit to the P - sum(floor) largest remainders (lower head first).
  const int64_t a = alpha_num, b = alpha_den, h = hkv;
  for (int j = threadIdx.x; j < hkv; j += SB) {
    const int64_t num = a * h * f_sh[j] + (b - a) * kP;
    const int64_t den = b * h;
    q_sh[j] = num / den;
    r_sh[j] = num % den;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t sq = 0;
    for (int j = 0; j < hkv; ++j) sq += q_sh[j];
    def_sh = kP - sq;
  }
  __syncthreads();
  for (int j = threadIdx.x; j < hkv; j += SB) {
    int rank = 0;
    for (int i = 0; i < hkv; ++i) rank += (r_sh[i] > r_sh[j] || (r_sh[i] == r_sh[j] && i < j)) ? 1 : 0;
    f_sh[j] = q_sh[j] + (rank < def_sh ? 1 : 0);     // B_j
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t base = kb0;
    for (int j = 0; j < g; ++j) base += f_sh[j];
    const int64_t Bg = f_sh[g];
    const int64_t k1 = (mode == MODE_CK) ? (Bg * ck_num) / ck_den : Bg;
    budgets[r] = (int32_t)Bg;
    rowbase[r] = base;
    if (mode == MODE_CK) rowk2[r] = (int32_t)(Bg - k1);
    k1_sh = k1;
    if (g == 0) {
      sel_off[inst] = kb0;
      if (inst == n_inst - 1) sel_off[n_inst] = kb0 + kP;
    }
  }
  __syncthreads();
  RState init = {0u, (int32_t)k1_sh};
  const RState x = pick_and_clear(rowhist + (size_t)r * NBIN, 0, init, sh);
  if (threadIdx.x == 0) rowst[r] = x;
}

// Budgets from one threshold per segment of seg_rows rows, one workgroup per
// segment (the model-wide top-k: one segment of every row; the floor reading:
// one segment per instance, its rows' floors added).  The ties the segment's
// threshold T may still take are shared out in row order (the flat index
// order); B_r = add + above + share; the rows' offsets in sel start at
// segment * seg_stride (the floor reading: P per instance) or run on from
// zero (one segment), sel_off gets each instance's first row.  A segment's
// total is below 2^31, so 32-bit sums of counts cannot wrap.
__global__ __launch_bounds__(SB) void segment_budget_kernel(int seg_rows, int hkv, int n_inst, int add,
                                                            int64_t seg_stride, const RState* __restrict__ seg,
                                                            const uint32_t* __restrict__ cnt,
                                                            int32_t* __restrict__ budgets,
                                                            int64_t* __restrict__ rowbase, RState* __restrict__ rowst,
                                                            int64_t* __restrict__ sel_off) {
  __shared__ uint32_t sh[SW + 4];
  const RState L = seg[blockIdx.x];
  const uint32_t quota = (L.prefix == NONE) ? 0u : (uint32_t)L.krem;
  const int64_t base0 = (int64_t)blockIdx.x * seg_stride;
  const int rbeg = blockIdx.x * seg_rows;
  uint32_t eq_carry = 0, f_carry = 0;
  for (int r0 = 0; r0 < seg_rows; r0 += SB) {
    const int rl = r0 + (int)threadIdx.x;
    const int r = rbeg + rl;
    const bool in = rl < seg_rows;
    const uint32_t gt = in ? cnt[2 * (size_t)r] : 0u;
    const uint32_t eq = in ? cnt[2 * (size_t)r + 1] : 0u;
    uint32_t eq_tot, f_tot;
    const uint32_t eq_before = eq_carry + block_excl_scan(eq, sh, eq_tot);
    const uint32_t share = min(quota - min(quota, eq_before), eq);   // no subtraction under a condition
    const uint32_t f = (in ? (uint32_t)add : 0u) + gt + share;
    const uint32_t before = f_carry + block_excl_scan(f, sh, f_tot);
    if (in) {
      budgets[r] = (int32_t)f;
      rowbase[r] = base0 + (int64_t)before;
      RState x = {L.prefix, (int32_t)share};
      if (L.prefix == NONE) x.krem = 0;
      rowst[r] = x;
      if (r % hkv == 0) sel_off[r / hkv] = base0 + (int64_t)before;
    }
    eq_carry += eq_tot;
    f_carry += f_tot;
  }
  if (threadIdx.x == 0 && blockIdx.x == gridDim.x - 1) sel_off[n_inst] = base0 + (int64_t)f_carry;
}

// StreamingLLM: B_g = P / h, one more for the lowest P mod h heads; head g
// keeps its first min(sinks, B_g) prefix tokens and its last B_g - that many.
// Grid (rows, chunks of SB selections); every row's budget and sel_off
// entries come from its chunk-0 workgroup.
__global__ __launch_bounds__(SB) void streaming_kernel(int hkv, int n_inst, int p, int kP, int sinks,
                                                       int32_t* __restrict__ budgets, int32_t* __restrict__ sel,
                                                       int64_t* __restrict__ sel_off) {
  const int r = blockIdx.x, inst = r / hkv, g = r % hkv;
  const int q = kP / hkv, rem = kP % hkv;
  const int bg = q + (g < rem ? 1 : 0);
  const int64_t base = (int64_t)inst * kP + (int64_t)g * q + min(g, rem);
  const int s = min(sinks, bg);
  const int j = blockIdx.y * SB + (int)threadIdx.x;
  if (j < bg) sel[base + j] = (j < s) ? j : p - bg + j;
  if (blockIdx.y == 0 && threadIdx.x == 0) {
    budgets[r] = bg;
    if (g == 0) sel_off[inst] = (int64_t)inst * kP;
    if (r == hkv * n_inst - 1) sel_off[n_inst] = (int64_t)n_inst * kP;
  }
}

// Per-instance budgets handed over as kernel arguments (so the call stays
// free of host-to-device copies and can be captured): instances [i0, i0 + n)
// take prefix budget P[t] and first position base[t] in sel; the last chunk
// also writes the total.
constexpr int PRESET_CHUNK = 64;
struct PresetArgs {
  int64_t P[PRESET_CHUNK];
  int64_t base[PRESET_CHUNK];
  int64_t total;
  int i0, n, last;
};
__global__ void preset_budget_kernel(PresetArgs a, int64_t* __restrict__ klist, int64_t* __restrict__ kbase) {
  const int t = threadIdx.x;
  if (t < a.n) {
    klist[a.i0 + t] = a.P[t];
    kbase[a.i0 + t] = a.base[t];
  }
  if (a.last && t == 0) kbase[a.i0 + a.n] = a.total;
}

// ---------------------------------------------------------------- per-chunk counts and emission
// Class of a score against a row's (T, quota): 2 = kept (above T, or a stage-1
// member when member flags are given), 1 = tie (equal to T), 0 = dropped.
__device__ __forceinline__ int klass(uint32_t u, bool ok, bool mem, uint32_t T) {
  if (!ok) return 0;
  if (mem) return 2;
  if (T == NONE) return 0;
  return u > T ? 2 : (u == T ? 1 : 0);
}

__global__ __launch_bounds__(SB) void chunk_count_kernel(const float* __restrict__ score,
                                                         const uint8_t* __restrict__ member, int p, int cpr,
                                                         int ntile, int vec, const RState* __restrict__ rowst,
                                                         uint32_t* __restrict__ cc) {
  __shared__ uint32_t sh[SW + 4];
  const Chunk ch = chunk_of(cpr, ntile, p);
  const RState S = rowst[ch.r];
  ChunkKeys K;
  uint8_t m[NK];
  load_chunk(score + (size_t)ch.r * p, ch, ntile, vec != 0, K);
  if (member) load_member(member + (size_t)ch.r * p, ch, ntile, vec != 0, K, m);
  uint32_t n2 = 0, n1 = 0;
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    const int kc = klass(K.k[j], j < K.n, member != nullptr && m[j] != 0, S.prefix);
    n2 += kc == 2 ? 1u : 0u;
    n1 += kc == 1 ? 1u : 0u;
  }
  const uint32_t both = block_sum(n2 | (n1 << 16), sh);   // at most 4096 of each
  if (threadIdx.x == 0) {
    cc[2 * (size_t)blockIdx.x] = both & 0xFFFFu;
    cc[2 * (size_t)blockIdx.x + 1] = both >> 16;
  }
}

// Writes the kept scores of the chunk in index order: as token indices at
// sel[base + position] (TO_SEL: at most lim of them, never past sel_total), or
// as member flags.  S is the row's state (threshold, ties it keeps).  USE_M:
// flagged scores count as kept.
template <bool USE_M, bool TO_SEL>
__device__ __forceinline__ void emit_chunk(const float* __restrict__ score, const uint8_t* __restrict__ member, int p,
                                           int cpr, int ntile, int vec, const Chunk& ch, const RState S,
                                           const uint32_t* __restrict__ cc, const int64_t base, const uint32_t lim,
                                           int32_t* __restrict__ sel, int64_t sel_total,
                                           uint8_t* __restrict__ member_out) {
  __shared__ uint32_t sh[SW + 4];
  __shared__ uint32_t before_sh[2][SW];
  ChunkKeys K;
  uint8_t m[NK];
  load_chunk(score + (size_t)ch.r * p, ch, ntile, vec != 0, K);
  if (USE_M) load_member(member + (size_t)ch.r * p, ch, ntile, vec != 0, K, m);
  // Kept scores and ties of the row's earlier chunks.
  uint32_t b2 = 0, b1 = 0;
  for (int c = threadIdx.x; c < ch.c; c += SB) {
    b2 += cc[2 * ((size_t)ch.r * cpr + c)];
    b1 += cc[2 * ((size_t)ch.r * cpr + c) + 1];
  }
  b2 = wave_sum(b2);
  b1 = wave_sum(b1);
  if ((threadIdx.x & (WAVE - 1)) == 0) { before_sh[0][threadIdx.x / WAVE] = b2; before_sh[1][threadIdx.x / WAVE] = b1; }
  __syncthreads();
  uint32_t B2 = 0, B1 = 0;
#pragma unroll
  for (int i = 0; i < SW; ++i) { B2 += before_sh[0][i]; B1 += before_sh[1][i]; }
  const uint32_t quota = (S.prefix == NONE) ? 0u : (uint32_t)S.krem;
  // ties kept by earlier chunks, and what is left (no subtraction under a condition)
  const uint32_t qrem = quota - min(quota, B1);
  const uint32_t pos0 = B2 + min(quota, B1);

  int kc[NK];
  uint32_t n2 = 0, n1 = 0;
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    kc[j] = klass(K.k[j], j < K.n, USE_M && m[j] != 0, S.prefix);
    n2 += kc[j] == 2 ? 1u : 0u;
    n1 += kc[j] == 1 ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t ex = block_excl_scan(n2 | (n1 << 16), sh, tot);
  const uint32_t e2 = ex & 0xFFFFu, e1 = ex >> 16;
  uint32_t tie = e1;                                   // ties of the chunk before this thread's scores
  uint32_t loc = e2 + (e1 < qrem ? e1 : qrem);         // position in the chunk's run of kept scores
  uint8_t take[NK];
  // the chunk's kept indices occupy positions pos0 .. pos0 + cnt - 1: staged
  // in LDS in order, then written with consecutive lanes on consecutive words
  __shared__ int32_t stage[SB * NK];
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    bool tk = kc[j] == 2;
    if (kc[j] == 1) { tk = tie < qrem; ++tie; }
    take[j] = tk ? 1 : 0;
    if (TO_SEL && tk) stage[loc] = K.e0 + j;
    loc += tk ? 1u : 0u;
  }
  if (TO_SEL) {
    const uint32_t cnt = (tot & 0xFFFFu) + ((tot >> 16) < qrem ? (tot >> 16) : qrem);
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < cnt; i += SB) {
      const uint32_t pos = pos0 + i;
      if (pos < lim && base + pos < sel_total) sel[base + pos] = stage[i];
    }
  }
  if (!TO_SEL) {
    uint8_t* mo = member_out + (size_t)ch.r * p;
    if (vec && ch.e_end - ch.e_begin == ntile * TILE) {
#pragma unroll
      for (int t = 0; t < MAXT; ++t) {
        if (t < ntile) {
          const uint32_t w = (uint32_t)take[4 * t] | ((uint32_t)take[4 * t + 1] << 8) |
                             ((uint32_t)take[4 * t + 2] << 16) | ((uint32_t)take[4 * t + 3] << 24);
          *reinterpret_cast<uint32_t*>(mo + K.e0 + 4 * t) = w;
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < NK; ++j)
        if (j < K.n) mo[K.e0 + j] = take[j];
    }
  }
}

template <bool USE_M, bool TO_SEL>
__global__ __launch_bounds__(SB) void emit_kernel(const float* __restrict__ score, const uint8_t* __restrict__ member,
                                                  int p, int cpr, int ntile, int vec, const RState* __restrict__ rowst,
                                                  const uint32_t* __restrict__ cc, const int64_t* __restrict__ rowbase,
                                                  const int32_t* __restrict__ cap, int32_t* __restrict__ sel,
                                                  int64_t sel_total, uint8_t* __restrict__ member_out) {
  const Chunk ch = chunk_of(cpr, ntile, p);
  emit_chunk<USE_M, TO_SEL>(score, member, p, cpr, ntile, vec, ch, rowst[ch.r], cc, TO_SEL ? rowbase[ch.r] : 0,
                            TO_SEL ? (uint32_t)cap[ch.r] : 0u, sel, sel_total, member_out);
}

// LAVa: rows keep their layer's threshold T with a share of its ties in head
// order, so each workgroup forms its row's budget B_g = above + share and its
// offset in sel from the heads' counts itself (the chunk counts of T come
// from layer_count_kernel), then emits; the row's first chunk writes B_g.
// hkv <= 256.
__global__ __launch_bounds__(SB) void lava_emit_kernel(const float* __restrict__ score, int p, int cpr, int ntile,
                                                       int vec, int hkv, const RState* __restrict__ seg,
                                                       const uint32_t* __restrict__ cnt,
                                                       const uint32_t* __restrict__ cc,
                                                       const int64_t* __restrict__ sel_off,
                                                       int32_t* __restrict__ budgets, int32_t* __restrict__ sel,
                                                       int64_t sel_total) {
  __shared__ uint32_t gt_sh[256], eq_sh[256];
  __shared__ int64_t base_sh;
  __shared__ uint32_t f_sh, q_sh;
  const Chunk ch = chunk_of(cpr, ntile, p);
  const int inst = ch.r / hkv, g = ch.r - inst * hkv;
  const RState L = seg[inst];
  for (int j = threadIdx.x; j < hkv; j += SB) {
    gt_sh[j] = cnt[2 * ((size_t)inst * hkv + j)];
    eq_sh[j] = cnt[2 * ((size_t)inst * hkv + j) + 1];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    // ties shared out in head order, as row_budget_kernel does (a layer's
    // counts stay below 2^31)
    const int64_t quota = (L.prefix == NONE) ? 0 : L.krem;
    int64_t before = 0, base = sel_off[inst];
    for (int j = 0; j < g; ++j) {
      const int64_t share = min(max(quota - before, (int64_t)0), (int64_t)eq_sh[j]);
      base += (int64_t)gt_sh[j] + share;
      before += eq_sh[j];
    }
    const int64_t share = min(max(quota - before, (int64_t)0), (int64_t)eq_sh[g]);
    base_sh = base;
    f_sh = gt_sh[g] + (uint32_t)share;
    q_sh = (uint32_t)share;
  }
  __syncthreads();
  RState S = {L.prefix, (int32_t)q_sh};
  if (L.prefix == NONE) S.krem = 0;
  if (threadIdx.x == 0 && ch.c == 0) budgets[ch.r] = (int32_t)f_sh;
  emit_chunk<false, true>(score, nullptr, p, cpr, ntile, vec, ch, S, cc, base_sh, f_sh, sel, sel_total, nullptr);
}

// ---------------------------------------------------------------- one workgroup per instance
// Small instances (at most XMAXH KV heads and XMAXE scores): the whole Ada-KV
// allocation of an instance in one 1024-thread workgroup, histograms in LDS,
// the instance's scores re-read for each of its seven passes (they stay in
// the caches at this size): the layer-wide top-P (three digit passes), the
// heads' counts and budgets, every head's own top-B_g (three digit passes, one
// wave picking each head's digit), and the emission.  Same digits, same
// order (-score, index) and the same integer safeguard as the multi-kernel
// path, so the selection is identical; one launch instead of thirteen.
// Bigger instances stay on the chunked path: one CU adding 2^17 top digits
// (pooled scores share a few exponents) into one LDS histogram serialises on
// the atomics (measured 205 us for a 130,816-score layer, against 61 us for
// thirteen chunked launches spreading them over the chip).
constexpr int XB = 1024;
constexpr int XW = XB / WAVE;
constexpr int XMAXH = 16;
constexpr int XMAXE = 1 << 14;

__device__ __forceinline__ uint32_t xblock_excl_scan(uint32_t x, uint32_t* sh, uint32_t& total) {
  const uint32_t ex = wave_excl_scan(x);
  const int wv = threadIdx.x / WAVE;
  if ((threadIdx.x & (WAVE - 1)) == WAVE - 1) sh[wv] = ex + x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < XW; ++i) {
    const uint32_t t = sh[i];
    before += (i < wv) ? t : 0u;
    all += t;
  }
  __syncthreads();
  total = all;
  return before + ex;
}

// Digit pick by one wave over nb bins (2048 or 512) of an LDS histogram: the
// digit d with count(> d) < krem <= count(>= d), and count(> d).
__device__ __forceinline__ void wave_pick(const uint32_t* h, int nb, uint32_t krem, uint32_t& dig,
                                          uint32_t& above_out) {
  const int lane = (int)__lane_id();
  const int bpl = nb / WAVE;
  uint32_t s = 0;
  for (int j = 0; j < bpl; ++j) s += h[nb - 1 - (lane * bpl + j)];
  const uint32_t ex = wave_excl_scan(s);
  const bool mine = ex < krem && krem <= ex + s;
  const uint64_t bal = __ballot(mine);
  uint32_t d = 0, ab = 0;
  if (mine) {
    uint32_t a = ex;
    for (int j = 0; j < bpl; ++j) {
      const uint32_t c = h[nb - 1 - (lane * bpl + j)];
      if (a < krem && krem <= a + c) {
        d = (uint32_t)(nb - 1 - (lane * bpl + j));
        ab = a;
        break;
      }
      a += c;
    }
  }
  const int src = bal ? (__ffsll((unsigned long long)bal) - 1) : 0;
  dig = (uint32_t)__shfl((int)d, src);
  above_out = (uint32_t)__shfl((int)ab, src);
}

// The thread's scores: flat indices [e0, e1) of the instance (head after
// head), read four at a time; fn(e, row, key) is called in index order.
template <class F>
__device__ __forceinline__ void x_each(const float* sc, int e0, int e1, int p, bool vec, F fn) {
  int row = e0 / p, k = e0 - row * p;
  for (int e = e0; e < e1; e += 4) {
    float v[4];
    if (vec) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(sc + e);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = x[j];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = (e + j < e1) ? sc[e + j] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (e + j < e1) {
        fn(e + j, row, k, v[j]);
        if (++k == p) { k = 0; ++row; }
      }
    }
  }
}

__global__ __launch_bounds__(XB) void ada_small_kernel(const float* __restrict__ score, int hkv, int p, int kP0,
                                                       const int64_t* __restrict__ klist,
                                                       const int64_t* __restrict__ kbase, int alpha_num,
                                                       int alpha_den, int n_inst, int32_t* __restrict__ budgets,
                                                       int32_t* __restrict__ sel, int64_t* __restrict__ sel_off,
                                                       uint32_t* __restrict__ flag) {
  extern __shared__ uint32_t rowhist[];               // [hkv][NBIN]
  __shared__ uint32_t lhist[NBIN];
  __shared__ uint32_t sh[XW + 4];
  __shared__ uint32_t rgt[XMAXH], req[XMAXH], reqT[XMAXH], tiepre[XMAXH];
  __shared__ RState lst, rst[XMAXH];
  __shared__ int64_t rbase[XMAXH];
  const int inst = blockIdx.x;
  const int E = hkv * p;
  const float* sc = score + (size_t)inst * E;
  const int64_t kP = klist ? klist[inst] : (int64_t)kP0;
  const int64_t base0 = kbase ? kbase[inst] : (int64_t)inst * kP0;
  const int npt = ((E + XB - 1) / XB + 3) & ~3;
  const int e0 = min(E, (int)threadIdx.x * npt), e1 = min(E, e0 + npt);
  const bool vec = (E % 4) == 0;     // every e0 and the instance base on 16 bytes
  const int wv = threadIdx.x / WAVE;

  // pass 0: the heads' top-digit histograms (their sum is the instance's)
  for (int i = threadIdx.x; i < hkv * NBIN; i += XB) rowhist[i] = 0u;
  __syncthreads();
  {
    uint32_t bad = 0u, cur = NONE, run = 0;
    x_each(sc, e0, e1, p, vec, [&](int, int row, int, float x) {
      bad |= bad_score(x);
      const uint32_t b = (uint32_t)row * NBIN + (sel_key(x) >> 20);
      if (b != cur) {
        if (cur != NONE) atomicAdd(rowhist + cur, run);
        cur = b;
        run = 0;
      }
      ++run;
    });
    if (cur != NONE) atomicAdd(rowhist + cur, run);
    if (bad) atomicOr(flag, 1u);
  }
  __syncthreads();
  for (int b = threadIdx.x; b < NBIN; b += XB) {
    uint32_t t = 0;
    for (int g = 0; g < hkv; ++g) t += rowhist[g * NBIN + b];
    lhist[b] = t;
  }
  __syncthreads();
  if (wv == 0) {
    RState x = {NONE, 0};
    if (kP > 0) {
      uint32_t d, above;
      wave_pick(lhist, NBIN, (uint32_t)kP, d, above);
      x.prefix = d << 20;
      x.krem = (int32_t)(kP - above);
    }
    if (threadIdx.x == 0) lst = x;
  }
  __syncthreads();
  // passes 1, 2 of the instance's top-P
  for (int ps = 1; ps < 3; ++ps) {
    const RState L = lst;
    if (L.prefix == NONE) break;
    for (int b = threadIdx.x; b < NBIN; b += XB) lhist[b] = 0u;
    __syncthreads();
    x_each(sc, e0, e1, p, vec, [&](int, int, int, float x) {
      const uint32_t u = sel_key(x);
      if (in_prefix(u, L.prefix, ps)) atomicAdd(lhist + digit_of(u, ps), 1u);
    });
    __syncthreads();
    if (wv == 0) {
      uint32_t d, above;
      wave_pick(lhist, pass_bins(ps), (uint32_t)L.krem, d, above);
      if (threadIdx.x == 0) {
        RState x = {L.prefix | (d << digit_shift(ps)), L.krem - (int32_t)above};
        lst = x;
      }
    }
    __syncthreads();
  }
  // pass 3: each head's entries above the instance's threshold T and equal to it
  if (threadIdx.x < XMAXH) { rgt[threadIdx.x] = 0u; req[threadIdx.x] = 0u; }
  __syncthreads();
  const RState L = lst;
  if (L.prefix != NONE) {
    int crow = -1;
    uint32_t gt = 0, eq = 0;
    x_each(sc, e0, e1, p, vec, [&](int, int row, int, float x) {
      if (row != crow) {
        if (crow >= 0) { if (gt) atomicAdd(rgt + crow, gt); if (eq) atomicAdd(req + crow, eq); }
        crow = row;
        gt = eq = 0;
      }
      const uint32_t u = sel_key(x);
      gt += u > L.prefix ? 1u : 0u;
      eq += u == L.prefix ? 1u : 0u;
    });
    if (crow >= 0) { if (gt) atomicAdd(rgt + crow, gt); if (eq) atomicAdd(req + crow, eq); }
  }
  __syncthreads();
  // budgets: counts f_g (ties at T shared out in head order), then the
  // safeguard in exact integers (floors, one more to the largest remainders,
  // lower head first), offsets in sel; then each head's first digit
  if (threadIdx.x == 0) {
    const int64_t quota = (L.prefix == NONE) ? 0 : L.krem;
    int64_t f[XMAXH], q[XMAXH], r[XMAXH];
    int64_t before = 0, sq = 0;
    const int64_t a = alpha_num, b = alpha_den, h = hkv;
    for (int g = 0; g < hkv; ++g) {
      int64_t share = quota - before;
      share = share < 0 ? 0 : (share > (int64_t)req[g] ? (int64_t)req[g] : share);
      before += req[g];
      f[g] = (int64_t)rgt[g] + share;
      const int64_t num = a * h * f[g] + (b - a) * kP;
      q[g] = num / (b * h);
      r[g] = num % (b * h);
      sq += q[g];
    }
    const int64_t def = kP - sq;
    int64_t run = base0;
    for (int g = 0; g < hkv; ++g) {
      int rank = 0;
      for (int i = 0; i < hkv; ++i) rank += (r[i] > r[g] || (r[i] == r[g] && i < g)) ? 1 : 0;
      const int64_t Bg = q[g] + (rank < def ? 1 : 0);
      budgets[(size_t)inst * hkv + g] = (int32_t)Bg;
      rbase[g] = run;
      run += Bg;
      RState x = {0u, (int32_t)Bg};
      rst[g] = x;
    }
    sel_off[inst] = base0;
    if (inst == n_inst - 1) sel_off[n_inst] = base0 + kP;
  }
  __syncthreads();
  for (int g = wv; g < hkv; g += XW) {
    const RState x = rst[g];
    RState y = {NONE, 0};
    if (x.krem > 0) {
      uint32_t d, above;
      wave_pick(rowhist + g * NBIN, NBIN, (uint32_t)x.krem, d, above);
      y.prefix = d << 20;
      y.krem = x.krem - (int32_t)above;
    }
    if (__lane_id() == 0) rst[g] = y;
  }
  __syncthreads();
  // passes 4, 5: every head's own top-B_g
  for (int ps = 1; ps < 3; ++ps) {
    for (int i = threadIdx.x; i < hkv * NBIN; i += XB) rowhist[i] = 0u;
    __syncthreads();
    x_each(sc, e0, e1, p, vec, [&](int, int row, int, float x) {
      const RState R = rst[row];
      const uint32_t u = sel_key(x);
      if (R.prefix != NONE && in_prefix(u, R.prefix, ps)) atomicAdd(rowhist + row * NBIN + digit_of(u, ps), 1u);
    });
    __syncthreads();
    for (int g = wv; g < hkv; g += XW) {
      const RState x = rst[g];
      RState y = {NONE, 0};
      uint32_t eqT = 0u;
      if (x.prefix != NONE) {
        uint32_t d, above;
        wave_pick(rowhist + g * NBIN, pass_bins(ps), (uint32_t)x.krem, d, above);
        y.prefix = x.prefix | (d << digit_shift(ps));
        y.krem = x.krem - (int32_t)above;
        if (ps == 2) eqT = rowhist[g * NBIN + d];   // entries equal to the head's threshold
      }
      if (__lane_id() == 0) {
        rst[g] = y;
        if (ps == 2) reqT[g] = eqT;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int g = 0; g < hkv; ++g) { tiepre[g] = t; t += reqT[g]; }
  }
  __syncthreads();
  // pass 6: emission in index order.  Kept: above the head's threshold, or
  // equal to it within the first krem ties of the head (index order).  The
  // class of every score (0 dropped, 1 tie, 2 kept) is parked in LDS, two
  // bits each in words the thread owns (the head histograms are done with).
  uint32_t* cls = rowhist;
  const int cwpt = (npt + 15) / 16;
  uint32_t* mine = cls + (size_t)threadIdx.x * cwpt;
  const int cnt = e1 - e0;
  uint32_t nties = 0;
  {
    uint32_t word = 0u;
    int filled = 0, wi = 0;
    x_each(sc, e0, e1, p, vec, [&](int, int row, int, float x) {
      const RState R = rst[row];
      const uint32_t u = sel_key(x);
      uint32_t code = 0u;
      if (R.prefix != NONE) code = u > R.prefix ? 2u : (u == R.prefix ? 1u : 0u);
      nties += code == 1u ? 1u : 0u;
      word |= code << (2 * filled);
      if (++filled == 16) { mine[wi++] = word; word = 0u; filled = 0; }
    });
    if (filled) mine[wi] = word;
  }
  uint32_t tall;
  uint32_t tb = xblock_excl_scan(nties, sh, tall);
  uint32_t nkept = 0;
  {
    int row = e0 / (p > 0 ? p : 1), k = e0 - row * p;
    for (int wi = 0; wi < cwpt; ++wi) {
      const uint32_t word = mine[wi];
      uint32_t nw = 0u;
      for (int b = 0; b < 16; ++b) {
        if (wi * 16 + b >= cnt) break;
        uint32_t code = (word >> (2 * b)) & 3u;
        if (code == 1u) {
          code = (tb - tiepre[row] < (uint32_t)rst[row].krem) ? 2u : 0u;
          ++tb;
        }
        nkept += code == 2u ? 1u : 0u;
        nw |= code << (2 * b);
        if (++k == p) { k = 0; ++row; }
      }
      mine[wi] = nw;
    }
  }
  uint32_t kall;
  uint32_t pos = xblock_excl_scan(nkept, sh, kall);
  {
    int row = e0 / (p > 0 ? p : 1), k = e0 - row * p;
    for (int wi = 0; wi < cwpt; ++wi) {
      const uint32_t word = mine[wi];
      for (int b = 0; b < 16; ++b) {
        if (wi * 16 + b >= cnt) break;
        if (((word >> (2 * b)) & 3u) == 2u) {
          if (pos < (uint32_t)kP) sel[base0 + pos] = k;
          ++pos;
        }
        if (++k == p) { k = 0; ++row; }
      }
    }
  }
  (void)rbase;
}

// ---------------------------------------------------------------- one workgroup per row
// Every head's own top-B_g (Ada-KV) for rows of at most RT_MAX scores, one
// 1024-thread workgroup per row, from the state row_budget_kernel leaves
// (pass 0 picked).  Each thread holds a contiguous run of up to RT_NPT keys of
// the row in registers (NONE past the row's end: no prefix matches it):
// passes 1 and 2 add the digits of the candidates into an LDS histogram, the
// workgroup picks the digit (two bins per thread, one scan), and the kept
// indices are written in index order from the same registers (kept scores
// and ties as bit masks per thread, counts scanned over the workgroup, indices
// staged in LDS).  The same digits, picks and tie rule as the
// chunked kernels, so the selection is identical; one launch and one read of
// the scores instead of six launches and four reads.  Candidates of pass 1
// share the threshold's top digit and the lanes of a wave hold keys RT_NPT
// apart, so one LDS atomic per candidate meets little contention.
constexpr int RT_NPT = 32;                // scores per thread
constexpr int RT_MAX = XB * RT_NPT;
constexpr int RT_STAGE = 8192;            // kept indices staged per window

// Digit pick over nb bins (2048 or 512) by the whole 1024-thread workgroup:
// thread t holds bins nb-1 - (t*bpt .. t*bpt+bpt-1), counted from the top; the
// digit d with count(> d) < krem <= count(>= d), and count(> d).
__device__ __forceinline__ void xblock_pick(const uint32_t* h, int nb, uint32_t krem, uint32_t* sh, uint32_t* res,
                                            uint32_t& dig, uint32_t& above_out) {
  const int bpt = nb >= XB ? nb / XB : 1;
  const int t = threadIdx.x;
  uint32_t c0 = 0, c1 = 0;
  if (t * bpt < nb) {
    c0 = h[nb - 1 - t * bpt];
    if (bpt > 1) c1 = h[nb - 2 - t * bpt];
  }
  uint32_t total;
  const uint32_t above = xblock_excl_scan(c0 + c1, sh, total);
  if (above < krem && krem <= above + c0) {
    res[0] = (uint32_t)(nb - 1 - t * bpt);
    res[1] = above;
  } else if (bpt > 1 && above + c0 < krem && krem <= above + c0 + c1) {
    res[0] = (uint32_t)(nb - 2 - t * bpt);
    res[1] = above + c0;
  }
  __syncthreads();
  dig = res[0];
  above_out = res[1];
}

template <int PS>
__device__ __forceinline__ RState row_pass(const uint32_t (&key)[RT_NPT], RState S, uint32_t* h, uint32_t* sh,
                                           uint32_t* res) {
  for (int b = threadIdx.x; b < NBIN; b += XB) h[b] = 0u;
  __syncthreads();
  const bool live = S.krem > 0 && S.prefix != NONE;   // uniform
  if (live) {
#pragma unroll
    for (int j = 0; j < RT_NPT; ++j)
      // padding (NONE) matches no prefix of a later pass; pass 0 skips it
      if ((PS != 0 || key[j] != NONE) && in_prefix(key[j], S.prefix, PS)) atomicAdd(h + digit_of(key[j], PS), 1u);
  }
  __syncthreads();
  RState out = {NONE, 0};
  if (live) {
    uint32_t d, above;
    xblock_pick(h, pass_bins(PS), (uint32_t)S.krem, sh, res, d, above);
    out.prefix = S.prefix | (d << digit_shift(PS));
    out.krem = S.krem - (int32_t)above;
  }
  __syncthreads();   // res and h are reused
  return out;
}

__global__ __launch_bounds__(XB) void row_topk_kernel(const float* __restrict__ score, int p, int vec,
                                                      const RState* __restrict__ rowst,
                                                      const int64_t* __restrict__ rowbase,
                                                      const int32_t* __restrict__ cap, int32_t* __restrict__ sel,
                                                      int64_t sel_total) {
  __shared__ uint32_t h[NBIN];
  __shared__ uint32_t sh[XW + 4];
  __shared__ uint32_t res[2];
  __shared__ int32_t stage[RT_STAGE];
  const int r = blockIdx.x;
  const int npt = ((p + XB - 1) / XB + 3) & ~3;   // <= RT_NPT, a multiple of 4
  const int e0 = min(p, (int)threadIdx.x * npt);
  const int n = min(npt, p - e0);
  const float* row = score + (size_t)r * p;
  uint32_t key[RT_NPT];
#pragma unroll
  for (int j = 0; j < RT_NPT; j += 4) {
    if (vec) {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (j < n) v = *reinterpret_cast<const f32x4*>(row + e0 + j);   // n is a multiple of 4 here
#pragma unroll
      for (int u = 0; u < 4; ++u) key[j + u] = (j < n) ? sel_key(v[u]) : NONE;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) key[j + u] = (j + u < n) ? sel_key(row[e0 + j + u]) : NONE;
    }
  }
  RState S = rowst[r];
  S = row_pass<1>(key, S, h, sh, res);
  S = row_pass<2>(key, S, h, sh, res);
  // emission in index order: S.prefix is the threshold T, S.krem the ties
  // kept.  The thread's kept scores (above T) and ties as bit masks over its
  // RT_NPT positions; the ties it keeps are the first ones its share of the
  // quota allows.
  const uint32_t quota = (S.prefix == NONE) ? 0u : (uint32_t)S.krem;
  uint32_t m2 = 0u, m1 = 0u;
#pragma unroll
  for (int j = 0; j < RT_NPT; ++j) {
    // scheduling fences every 8 keys keep the compare masks from piling up
    // in scalar registers
    if ((j & 7) == 0) __builtin_amdgcn_sched_barrier(0);
    const int kc = klass(key[j], key[j] != NONE, false, S.prefix);
    m2 |= (kc == 2 ? 1u : 0u) << j;
    m1 |= (kc == 1 ? 1u : 0u) << j;
  }
  const uint32_t n2 = __builtin_popcount(m2), n1 = __builtin_popcount(m1);
  uint32_t tot;
  const uint32_t ex = xblock_excl_scan(n2 | (n1 << 16), sh, tot);   // p <= 2^15: no carry between halves
  const uint32_t cnt = (tot & 0xFFFFu) + ((tot >> 16) < quota ? (tot >> 16) : quota);
  // ties kept by earlier threads, then this thread's share of the rest (no
  // subtraction under a condition: with `tie0 < quota ? min(n1, quota - tie0)
  // : 0` the subtraction was hoisted out of its guard with a no-wrap flag and
  // min(tie0, quota) below folded to tie0)
  const uint32_t before = min(ex >> 16, quota);
  const uint32_t take1 = min(n1, quota - before);
  // the lowest take1 set bits of m1
  uint32_t mt = 0u, rest = m1;
  for (uint32_t i = 0; i < take1; ++i) {
    const uint32_t low = rest & (0u - rest);
    mt |= low;
    rest ^= low;
  }
  const uint32_t mk = m2 | mt;                                       // kept positions
  const uint32_t loc0 = (ex & 0xFFFFu) + before;
  const int64_t base = rowbase[r];
  const uint32_t lim = (uint32_t)cap[r];
  // kept indices staged in LDS by windows of RT_STAGE positions, copied out
  // with consecutive lanes on consecutive words
  for (uint32_t w0 = 0; w0 < cnt; w0 += RT_STAGE) {
    uint32_t rem = mk, loc = loc0;
    while (rem) {
      const int j = __builtin_ctz(rem);
      rem &= rem - 1u;
      if (loc >= w0 && loc - w0 < (uint32_t)RT_STAGE) stage[loc - w0] = e0 + j;
      ++loc;
    }
    __syncthreads();
    const uint32_t nw = min((uint32_t)RT_STAGE, cnt - w0);
    for (uint32_t i = threadIdx.x; i < nw; i += XB) {
      const uint32_t pos = w0 + i;
      if (pos < lim && base + pos < sel_total) sel[base + pos] = stage[i];
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- LAVa online: older layers
// Layer j < I-1 of an online step keeps the top klist[j] of its kept entries
// of the previous step (prev_sel from prev_off[j], heads one after another,
// head g holding prev_budgets[j*hkv + g] indices in rising order).  The
// previous step kept the first prev_off[j+1] - prev_off[j] >= klist[j] entries
// of the same order (-score, flat index) over the same scores, so its first
// klist[j] are the layer's first klist[j]: the same selection as a top-k over
// all of the layer's scores, from at most RT_MAX entries instead of hkv * p.
// The entries are already in flat-index order, so a tie goes to the earlier
// entry.  One 1024-thread workgroup per older layer: the entries' scores are
// gathered into registers (RT_NPT per thread), three digit passes into an LDS
// histogram, kept entries emitted in order, head budgets counted in LDS.  The
// host takes this route only when the previous step's older layers kept at
// most RT_MAX entries in all; indices and counts read here are clamped into
// range all the same.
constexpr int RS_MAXH = 256;              // KV heads of a layer on this route
// Each older layer is re-selected by one workgroup, so while the older layers
// keep more than this many entries each on average, the layer-wide chain over
// their full scores (spread over the chip) is the faster route.
constexpr int64_t RS_AVG_MAX = 8192;

__device__ __forceinline__ int rs_head_of(const int32_t* hstart, int hkv, int e) {
  // the last head whose first entry is at most e (hstart[0] = 0)
  int lo = 0, hi = hkv - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (hstart[mid] <= e) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(XB) void lava_reselect_kernel(const float* __restrict__ score, int hkv, int p,
                                                           const int32_t* __restrict__ prev_budgets,
                                                           const int32_t* __restrict__ prev_sel,
                                                           const int64_t* __restrict__ prev_off,
                                                           const int64_t* __restrict__ klist,
                                                           const int64_t* __restrict__ sel_off,
                                                           int32_t* __restrict__ budgets, int32_t* __restrict__ sel,
                                                           int64_t sel_total) {
  __shared__ uint32_t h[NBIN];
  __shared__ uint32_t sh[XW + 4];
  __shared__ uint32_t res[2];
  __shared__ int32_t stage[RT_STAGE];
  __shared__ int32_t hstart[RS_MAXH + 1];
  __shared__ uint32_t hcnt[RS_MAXH];
  const int lay = blockIdx.x;
  const int64_t in0 = prev_off[lay];
  const int c = (int)min(max(prev_off[lay + 1] - in0, (int64_t)0), (int64_t)RT_MAX);
  const int k = (int)min(max(klist[lay], (int64_t)0), (int64_t)c);
  // first entry of every head: the scan of the previous budgets, clamped to c
  {
    const int t = threadIdx.x;
    const uint32_t bprev = t < hkv ? (uint32_t)min(max(prev_budgets[(size_t)lay * hkv + t], 0), RT_MAX) : 0u;
    uint32_t tot;
    const uint32_t ex = xblock_excl_scan(bprev, sh, tot);
    if (t < hkv) {
      hstart[t] = (int32_t)min(ex, (uint32_t)c);
      hcnt[t] = 0u;
    }
    if (t == 0) hstart[hkv] = c;
  }
  __syncthreads();
  const int npt = ((c + XB - 1) / XB + 3) & ~3;   // <= RT_NPT
  const int e0 = min(c, (int)threadIdx.x * npt);
  const int n = min(npt, c - e0);
  const int32_t* in = prev_sel + in0;
  const float* lsc = score + (size_t)lay * hkv * p;
  int32_t ix[RT_NPT];
#pragma unroll
  for (int j = 0; j < RT_NPT; ++j) ix[j] = (j < n) ? min(max(in[e0 + j], 0), p - 1) : 0;
  uint32_t key[RT_NPT];
  {
    int hd = rs_head_of(hstart, hkv, e0);
#pragma unroll
    for (int j = 0; j < RT_NPT; ++j) {
      while (hd + 1 < hkv && hstart[hd + 1] <= e0 + j) ++hd;
      key[j] = (j < n) ? sel_key(lsc[(size_t)hd * p + ix[j]]) : NONE;
    }
  }
  RState S = {0u, k};
  S = row_pass<0>(key, S, h, sh, res);
  S = row_pass<1>(key, S, h, sh, res);
  S = row_pass<2>(key, S, h, sh, res);
  // emission in entry order, as row_topk_kernel: kept scores and ties as bit
  // masks, the thread's share of the ties, positions by a workgroup scan
  const uint32_t quota = (S.prefix == NONE) ? 0u : (uint32_t)S.krem;
  uint32_t m2 = 0u, m1 = 0u;
#pragma unroll
  for (int j = 0; j < RT_NPT; ++j) {
    if ((j & 7) == 0) __builtin_amdgcn_sched_barrier(0);
    const int kc = klass(key[j], key[j] != NONE, false, S.prefix);
    m2 |= (kc == 2 ? 1u : 0u) << j;
    m1 |= (kc == 1 ? 1u : 0u) << j;
  }
  const uint32_t n2 = __builtin_popcount(m2), n1 = __builtin_popcount(m1);
  uint32_t tot;
  const uint32_t ex = xblock_excl_scan(n2 | (n1 << 16), sh, tot);   // c <= 2^15: no carry between halves
  const uint32_t cnt = (tot & 0xFFFFu) + ((tot >> 16) < quota ? (tot >> 16) : quota);
  const uint32_t before = min(ex >> 16, quota);
  const uint32_t take1 = min(n1, quota - before);
  uint32_t mt = 0u, rest = m1;
  for (uint32_t i = 0; i < take1; ++i) {
    const uint32_t low = rest & (0u - rest);
    mt |= low;
    rest ^= low;
  }
  const uint32_t mk = m2 | mt;
  const uint32_t loc0 = (ex & 0xFFFFu) + before;
  // kept entries per head: a thread's entries are consecutive, so one LDS
  // atomic per head run
  {
    int hd = rs_head_of(hstart, hkv, e0);
    uint32_t run = 0u, rem = mk;
    while (rem) {
      const int j = __builtin_ctz(rem);
      rem &= rem - 1u;
      int h2 = hd;
      while (h2 + 1 < hkv && hstart[h2 + 1] <= e0 + j) ++h2;
      if (h2 != hd) {
        if (run) atomicAdd(hcnt + hd, run);
        run = 0u;
        hd = h2;
      }
      ++run;
    }
    if (run) atomicAdd(hcnt + hd, run);
  }
  const int64_t base = sel_off[lay];
  for (uint32_t w0 = 0; w0 < cnt; w0 += RT_STAGE) {
    uint32_t rem = mk, loc = loc0;
    while (rem) {
      const int j = __builtin_ctz(rem);
      rem &= rem - 1u;
      if (loc >= w0 && loc - w0 < (uint32_t)RT_STAGE) stage[loc - w0] = min(max(in[e0 + j], 0), p - 1);
      ++loc;
    }
    __syncthreads();
    const uint32_t nw = min((uint32_t)RT_STAGE, cnt - w0);
    for (uint32_t i = threadIdx.x; i < nw; i += XB) {
      const uint32_t pos = w0 + i;
      if (pos < (uint32_t)k && base + pos < sel_total) sel[base + pos] = stage[i];
    }
    __syncthreads();
  }
  __syncthreads();   // every head count is in (also when nothing was staged)
  if ((int)threadIdx.x < hkv) budgets[(size_t)lay * hkv + threadIdx.x] = (int32_t)hcnt[threadIdx.x];
}

// ---------------------------------------------------------------- workspace plan
struct AllocPlan {
  int R, cpr, ntile, nchunk;
  size_t off_flag, off_rowhist, off_seghist, off_seghist2, off_cnt, zero_end;
  size_t off_seg, off_seg1, off_seg2, off_row, off_row2, off_rowk2, off_rowbase, off_cc, off_member, off_part,
      off_klist, off_kbase, total;
};

AllocPlan plan_alloc(const Geo& g, const adakv_alloc& a) {
  AllocPlan P{};
  P.R = g.I * g.hkv;
  P.ntile = MAXT;
  auto chunks = [&](int nt) { return (int64_t)P.R * ((g.p + nt * TILE - 1) / (nt * TILE)); };
  while (P.ntile > 1 && chunks(P.ntile) < 2048) P.ntile /= 2;
  P.cpr = (g.p + P.ntile * TILE - 1) / (P.ntile * TILE);
  P.nchunk = P.R * P.cpr;
  size_t off = 0;
  P.off_flag = off;     off = 256;   // int32: a score broke the precondition
  P.off_rowhist = off;  off = align_up(off + (size_t)P.R * NBIN * 4, 256);
  P.off_seghist = off;  off = align_up(off + (size_t)g.I * NBIN * 4, 256);
  P.off_seghist2 = off; off = align_up(off + (size_t)g.I * NBIN * 4, 256);   // the layer-wide pass 2
  P.off_cnt = off;      off = align_up(off + (size_t)P.R * 8, 256);
  P.zero_end = off;
  P.off_seg = off;      off = align_up(off + (size_t)g.I * sizeof(RState), 256);
  P.off_seg1 = off;     off = align_up(off + (size_t)g.I * sizeof(RState), 256);
  P.off_seg2 = off;     off = align_up(off + (size_t)g.I * sizeof(RState), 256);
  P.off_row = off;      off = align_up(off + (size_t)P.R * sizeof(RState), 256);
  P.off_row2 = off;     off = align_up(off + (size_t)P.R * sizeof(RState), 256);
  P.off_rowk2 = off;    off = align_up(off + (size_t)P.R * 4, 256);
  P.off_rowbase = off;  off = align_up(off + (size_t)P.R * 8, 256);
  P.off_cc = off;       off = align_up(off + (size_t)P.nchunk * 8, 256);
  P.off_member = off;
  if (a.mode == ADAKV_ALLOC_ADA_CRITICALKV || a.mode == ADAKV_ALLOC_ADA_FLOOR)
    off = align_up(off + (size_t)P.R * g.p, 256);
  P.off_part = off;
  if (a.mode == ADAKV_ALLOC_LAVA_LAYERS) off = align_up(off + (size_t)P.nchunk * 16, 256);
  P.off_klist = off;    off = align_up(off + (size_t)g.I * 8, 256);
  P.off_kbase = off;    off = align_up(off + (size_t)(g.I + 1) * 8, 256);
  P.total = off;
  return P;
}

}  // namespace

size_t alloc_ws_bytes(const Geo& g, const adakv_alloc& a) { return plan_alloc(g, a).total; }

// Launch order (every kernel on `st`, nothing waits on the host):
//   zero histograms and counts
//   layer-wide top-k: pass-0 row histograms [LAVa: + entropy partials, layer budgets],
//     pick 0, histograms of passes 1 and 2 (the pass-2 launch picks the digit of
//     pass 1 itself), layer counts per row (picking the digit of pass 2 itself)
//   [LAVa] emission in index order; each workgroup forms its row's budget and
//     offset from the counts (rows keep the layer threshold)
//   [LAVa online, older layers re-selected] the newest layer's chain as above
//     (its first pick inside the layer-budget launch), then one workgroup per
//     older layer re-selects among its previous entries
//   per-row budgets, offsets and first pick of the head's top-k
//   [Ada-KV, rows of at most RT_MAX scores] each head's top-k and emission in
//     one launch, else (histogram, pick) for passes 1 and 2 of every head's
//     top-k, per-chunk counts, emission in index order
//   [CriticalKV] stage 1 emits member flags; stage 2 runs the head top-k again on the
//     composite score over non-members and emits the union.
//   [model-wide] one segment of all rows: (histogram, pick) x 3, counts per row,
//     budgets and offsets in one workgroup, per-chunk counts, emission.
//   [floor reading] per-row top-f0 -> member flags; per-instance top over the
//     rest; counts, budgets f0 + share, emission of both stages together.
//   [StreamingLLM] one kernel writes budgets, offsets and indices; no scores.
hipError_t launch_allocate(const Geo& g, const adakv_alloc& a, const float* score, const float* score2,
                           int32_t* budgets, int32_t* sel, int64_t* sel_off, char* ws, hipStream_t st, bool online,
                           const int64_t* prev_off, const int32_t* prev_budgets, const int32_t* prev_sel,
                           double* layer_ent) {
  const AllocPlan P = plan_alloc(g, a);
  uint32_t* flag = reinterpret_cast<uint32_t*>(ws + P.off_flag);
  uint32_t* rowhist = reinterpret_cast<uint32_t*>(ws + P.off_rowhist);
  uint32_t* seghist = reinterpret_cast<uint32_t*>(ws + P.off_seghist);
  uint32_t* seghist2 = reinterpret_cast<uint32_t*>(ws + P.off_seghist2);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(ws + P.off_cnt);
  RState* segst = reinterpret_cast<RState*>(ws + P.off_seg);
  RState* segst1 = reinterpret_cast<RState*>(ws + P.off_seg1);
  RState* segst2 = reinterpret_cast<RState*>(ws + P.off_seg2);
  RState* rowst = reinterpret_cast<RState*>(ws + P.off_row);
  RState* rowst2 = reinterpret_cast<RState*>(ws + P.off_row2);
  int32_t* rowk2 = reinterpret_cast<int32_t*>(ws + P.off_rowk2);
  int64_t* rowbase = reinterpret_cast<int64_t*>(ws + P.off_rowbase);
  uint32_t* cc = reinterpret_cast<uint32_t*>(ws + P.off_cc);
  uint8_t* member = reinterpret_cast<uint8_t*>(ws + P.off_member);
  double* part = reinterpret_cast<double*>(ws + P.off_part);
  int64_t* klist = reinterpret_cast<int64_t*>(ws + P.off_klist);
  int64_t* kbase = reinterpret_cast<int64_t*>(ws + P.off_kbase);

  const bool vec1 = (g.p % 4 == 0) && (reinterpret_cast<uintptr_t>(score) % 16 == 0);
  const bool vec2 = (g.p % 4 == 0) && (reinterpret_cast<uintptr_t>(score2) % 16 == 0);
  const int nc = P.nchunk, cpr = P.cpr, nt = P.ntile, hkv = g.hkv, R = P.R;
  const bool lava = a.mode == ADAKV_ALLOC_LAVA_LAYERS;
  const bool ck = a.mode == ADAKV_ALLOC_ADA_CRITICALKV;
  const int mode = ck ? MODE_CK : MODE_ADA;
  const bool preset = a.inst_budget != nullptr;   // per-instance budgets (Ada-KV mode only)
  const int kP = (lava || preset) ? 0 : (int)(a.budget - (int64_t)g.w * g.hkv);
  int64_t sel_total = lava ? a.budget - (int64_t)g.I * g.w * g.hkv : (int64_t)g.I * kP;

  // small instances: one workgroup per instance does the whole Ada-KV allocation
  const bool small = a.mode == ADAKV_ALLOC_ADA && hkv <= XMAXH && (int64_t)hkv * g.p <= XMAXE;
  {
    // the precondition word, and the histograms and counts the chunked path adds into
    const size_t n16 = small ? 1 : P.zero_end / 16;
    const int blocks = (int)std::min<size_t>((n16 + SB - 1) / SB, 4096);
    sel_zero_kernel<<<blocks, SB, 0, st>>>(reinterpret_cast<u32x4*>(ws), n16);
  }
  if (a.mode == ADAKV_ALLOC_STREAMING) {
    const int kP = (int)(a.budget - (int64_t)g.w * g.hkv);
    const int maxb = kP / hkv + 1;
    dim3 grid(R, (maxb + SB - 1) / SB);
    streaming_kernel<<<grid, SB, 0, st>>>(hkv, g.I, g.p, kP, a.sinks, budgets, sel, sel_off);
    return hipGetLastError();
  }
  if (a.mode == ADAKV_ALLOC_ADA_FLOOR) {
    // Stage 1: every head's own top-f0 as member flags.  Stage 2: per instance
    // one top-(P - h*f0) over the non-members, their counts, budgets f0 + share,
    // then emission of members and stage-2 entries together.
    const int kP = (int)(a.budget - (int64_t)g.w * g.hkv);
    const int f0 = (int)(((int64_t)a.alpha_num * kP) / ((int64_t)a.alpha_den * hkv));
    for (int ps = 0; ps < 3; ++ps) {
      radix_hist(nc, st, score, nullptr, g.p, cpr, nt, vec1, 1, ps, nullptr, f0, rowst, rowhist, flag);
      radix_pick_kernel<<<R, SB, 0, st>>>(rowhist, ps, nullptr, f0, rowst);
    }
    chunk_count_kernel<<<nc, SB, 0, st>>>(score, nullptr, g.p, cpr, nt, vec1, rowst, cc);
    emit_kernel<false, false><<<nc, SB, 0, st>>>(score, nullptr, g.p, cpr, nt, vec1, rowst, cc, nullptr, nullptr, nullptr, 0,
                                   member);
    const int k2 = kP - hkv * f0;
    for (int ps = 0; ps < 3; ++ps) {
      radix_hist(nc, st, score, member, g.p, cpr, nt, vec1, hkv, ps, nullptr, k2, segst, seghist, flag);
      radix_pick_kernel<<<g.I, SB, 0, st>>>(seghist, ps, nullptr, k2, segst);
    }
    layer_count_kernel<<<nc, SB, 0, st>>>(score, member, g.p, cpr, nt, vec1, hkv, segst, cnt, nullptr, nullptr,
                                          nullptr);
    segment_budget_kernel<<<g.I, SB, 0, st>>>(hkv, hkv, g.I, f0, (int64_t)kP, segst, cnt, budgets, rowbase, rowst2,
                                              sel_off);
    chunk_count_kernel<<<nc, SB, 0, st>>>(score, member, g.p, cpr, nt, vec1, rowst2, cc);
    emit_kernel<true, true><<<nc, SB, 0, st>>>(score, member, g.p, cpr, nt, vec1, rowst2, cc, rowbase, budgets, sel,
                                   (int64_t)g.I * kP, nullptr);
    return hipGetLastError();
  }
  if (a.mode == ADAKV_ALLOC_GLOBAL) {
    // One top-k over all R rows: three digit passes on a single segment, the
    // rows' counts at its threshold, their budgets and offsets, emission.
    const int Bp = (int)(a.budget - (int64_t)g.I * g.w * g.hkv);
    for (int ps = 0; ps < 3; ++ps) {
      radix_hist(nc, st, score, nullptr, g.p, cpr, nt, vec1, R, ps, nullptr, Bp, segst, seghist, flag);
      radix_pick_kernel<<<1, SB, 0, st>>>(seghist, ps, nullptr, Bp, segst);
    }
    layer_count_kernel<<<nc, SB, 0, st>>>(score, nullptr, g.p, cpr, nt, vec1, R, segst, cnt, nullptr, nullptr,
                                          nullptr);
    segment_budget_kernel<<<1, SB, 0, st>>>(R, hkv, g.I, 0, 0, segst, cnt, budgets, rowbase, rowst, sel_off);
    chunk_count_kernel<<<nc, SB, 0, st>>>(score, nullptr, g.p, cpr, nt, vec1, rowst, cc);
    emit_kernel<false, true><<<nc, SB, 0, st>>>(score, nullptr, g.p, cpr, nt, vec1, rowst, cc, rowbase, budgets, sel, (int64_t)Bp,
                                   nullptr);
    return hipGetLastError();
  }
  if (preset) {
    // the instances' prefix budgets P_i = B_i - w*hkv and their offsets in sel
    int64_t run = 0;
    for (int i0 = 0; i0 < g.I; i0 += PRESET_CHUNK) {
      PresetArgs pa{};
      pa.i0 = i0;
      pa.n = std::min(PRESET_CHUNK, g.I - i0);
      for (int t = 0; t < pa.n; ++t) {
        pa.P[t] = a.inst_budget[i0 + t] - (int64_t)g.w * g.hkv;
        pa.base[t] = run;
        run += pa.P[t];
      }
      pa.last = i0 + pa.n == g.I;
      pa.total = run;
      preset_budget_kernel<<<1, PRESET_CHUNK, 0, st>>>(pa, klist, kbase);
    }
    sel_total = run;
  }
  if (small) {
    // one workgroup per instance (the zero fill above cleared the flag)
    const int npt = (int)((((int64_t)hkv * g.p + XB - 1) / XB + 3) & ~3);
    const size_t lds = std::max((size_t)hkv * NBIN, (size_t)XB * ((npt + 15) / 16)) * sizeof(uint32_t);
    ada_small_kernel<<<g.I, XB, lds, st>>>(score, hkv, g.p, kP, preset ? klist : nullptr, preset ? kbase : nullptr,
                                          a.alpha_num, a.alpha_den, g.I, budgets, sel, sel_off, flag);
    return hipGetLastError();
  }
  // LAVa online prefill: the entropies of the older layers come from the
  // caller's cache, so only the newest layer's are summed.
  const int ent_first = (lava && online) ? g.I - 1 : 0;
  const int64_t Bp_lava = lava ? a.budget - (int64_t)g.I * g.w * g.hkv : 0;
  const size_t sm_lava = (size_t)g.I * (sizeof(double) + sizeof(int64_t));
  if (lava && online && g.I > 1 && prev_budgets != nullptr && prev_sel != nullptr && hkv <= RS_MAXH &&
      a.budget - (int64_t)(g.I - 1) * g.w * hkv <= RT_MAX &&
      a.budget - (int64_t)(g.I - 1) * g.w * hkv <= RS_AVG_MAX * (g.I - 1)) {
    // Incremental step: the older layers kept at most RT_MAX entries in all at
    // the previous step (at most RS_AVG_MAX each on average), and their new
    // selections lie inside those.  The
    // newest layer runs the layer-wide chain on its own rows (same chunking
    // as the whole call, so its entropy sums are the ones the full route
    // forms); every older layer is re-selected from its previous entries.
    const int nc1 = hkv * cpr;
    const size_t lay = (size_t)(g.I - 1) * hkv;
    const float* s1 = score + lay * g.p;
    layer_hist0_kernel<<<nc1, SB, 0, st>>>(s1, g.p, cpr, nt, vec1, 1, 0, rowhist, part, flag);
    lava_budget_kernel<<<1, SB, sm_lava, st>>>(part, g.I, hkv * cpr, hkv, g.p, Bp_lava, 1, prev_off, ent_first,
                                               layer_ent, klist, sel_off, rowhist, segst);
    radix_hist(nc1, st, s1, nullptr, g.p, cpr, nt, vec1, hkv, 1, nullptr, 0, segst, seghist, flag);
    radix_hist(nc1, st, s1, nullptr, g.p, cpr, nt, vec1, hkv, 2, nullptr, 0, segst, seghist2, flag, seghist, segst1);
    layer_count_kernel<<<nc1, SB, 0, st>>>(s1, nullptr, g.p, cpr, nt, vec1, hkv, segst1, cnt, seghist2, segst2, cc);
    lava_emit_kernel<<<nc1, SB, 0, st>>>(s1, g.p, cpr, nt, vec1, hkv, segst2, cnt, cc, sel_off + (g.I - 1),
                                         budgets + lay, sel, sel_total);
    lava_reselect_kernel<<<g.I - 1, XB, 0, st>>>(score, hkv, g.p, prev_budgets, prev_sel, prev_off, klist, sel_off,
                                                 budgets, sel, sel_total);
    return hipGetLastError();
  }
  // Layer-wide top-k.
  layer_hist0_kernel<<<nc, SB, 0, st>>>(score, g.p, cpr, nt, vec1, lava ? 1 : 0, ent_first * hkv * cpr, rowhist,
                                        part, flag);
  if (lava)
    lava_budget_kernel<<<1, SB, sm_lava, st>>>(part, g.I, hkv * cpr, hkv, g.p, Bp_lava, online ? 1 : 0, prev_off,
                                               ent_first, online ? layer_ent : nullptr, klist, sel_off, nullptr,
                                               nullptr);
  layer_pick0_kernel<<<g.I, SB, 0, st>>>(rowhist, hkv, kP, (lava || preset) ? klist : nullptr, segst);
  // passes 1 and 2; the digits of passes 1 and 2 are picked by the launch after each
  radix_hist(nc, st, score, nullptr, g.p, cpr, nt, vec1, hkv, 1, nullptr, 0, segst, seghist, flag);
  radix_hist(nc, st, score, nullptr, g.p, cpr, nt, vec1, hkv, 2, nullptr, 0, segst, seghist2, flag, seghist, segst1);
  // Head budgets (LAVa: the emission forms them from the counts itself).
  layer_count_kernel<<<nc, SB, 0, st>>>(score, nullptr, g.p, cpr, nt, vec1, hkv, segst1, cnt, seghist2, segst2,
                                        lava ? cc : nullptr);
  if (lava) {
    lava_emit_kernel<<<nc, SB, 0, st>>>(score, g.p, cpr, nt, vec1, hkv, segst2, cnt, cc, sel_off, budgets, sel,
                                        sel_total);
    return hipGetLastError();
  }
  row_budget_kernel<<<R, SB, 0, st>>>(hkv, mode, kP, a.alpha_num, a.alpha_den, a.ck_num, a.ck_den, g.I,
                                      preset ? klist : nullptr, preset ? kbase : nullptr, segst2, cnt, rowhist,
                                      budgets, rowbase, rowk2, rowst, sel_off);
  if (!ck && g.p <= RT_MAX) {
    // every head's own top-k and the emission, one workgroup per row: one
    // launch and one read of the scores instead of six and four
    row_topk_kernel<<<R, XB, 0, st>>>(score, g.p, vec1 ? 1 : 0, rowst, rowbase, budgets, sel, sel_total);
    return hipGetLastError();
  }
  // Every head's own top-k.
  for (int ps = 1; ps < 3; ++ps) {
    radix_hist(nc, st, score, nullptr, g.p, cpr, nt, vec1, 1, ps, nullptr, 0, rowst, rowhist, flag);
    radix_pick_kernel<<<R, SB, 0, st>>>(rowhist, ps, nullptr, 0, rowst);
  }
  chunk_count_kernel<<<nc, SB, 0, st>>>(score, nullptr, g.p, cpr, nt, vec1, rowst, cc);
  if (!ck) {
    emit_kernel<false, true><<<nc, SB, 0, st>>>(score, nullptr, g.p, cpr, nt, vec1, rowst, cc, rowbase, budgets, sel, sel_total,
                                   nullptr);
    return hipGetLastError();
  }
  // CriticalKV: stage-1 members, then stage 2 on the composite score over the rest.
  emit_kernel<false, false><<<nc, SB, 0, st>>>(score, nullptr, g.p, cpr, nt, vec1, rowst, cc, nullptr, nullptr, nullptr, 0,
                                 member);
  for (int ps = 0; ps < 3; ++ps) {
    radix_hist(nc, st, score2, member, g.p, cpr, nt, vec2, 1, ps, rowk2, 0, rowst2, rowhist, flag);
    radix_pick_kernel<<<R, SB, 0, st>>>(rowhist, ps, rowk2, 0, rowst2);
  }
  chunk_count_kernel<<<nc, SB, 0, st>>>(score2, member, g.p, cpr, nt, vec2, rowst2, cc);
  emit_kernel<true, true><<<nc, SB, 0, st>>>(score2, member, g.p, cpr, nt, vec2, rowst2, cc, rowbase, budgets, sel, sel_total,
                                 nullptr);
  return hipGetLastError();
}

}  // namespace adakv
