// Budget allocation and selection on gfx950.
//
// Top-k over non-negative fp32 scores is a radix select on the bit patterns
// (4 passes of 8 bits, most significant first): it yields a threshold key T and
// the number of entries equal to T that are kept.  Entries equal to T are kept
// in index order, so the result is the first k of the order (-score, index)
// and is exactly reproducible.  One workgroup of 1024 threads owns one segment
// (an instance for the layer-wide top-B, a head for the per-head top-k).
//
// Definitions followed:
//  * Ada-KV notes, Algorithm 1 (concatenate the heads, top-B, count per head)
//    and Algorithm 2 steps 6-9 (window out of the budget, safeguard, per-head
//    top-k); the safeguard alpha*f + (1-alpha)*B/h is made integer exactly.
//  * LAVa notes, "动态头预算的逐层缓存驱逐" (flattened layer top-k, no safeguard)
//    and "基于不确定性的层预算分配" (entropy-proportional layer budgets).
//  * CriticalKV notes, "两阶段贪心选择算法" (top-b' by attention, then top-b''
//    of the rest by the composite score).
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace adakv {
namespace {

constexpr int ST = 1024;        // threads of a selection workgroup
constexpr int NW = ST / WAVE;   // waves
constexpr uint32_t NONE = 0xFFFFFFFFu;

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = (int)__lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Adds one to arr[key] for every lane with key != NONE.  The most common keys
// of the wave are added with one atomic each.
__device__ __forceinline__ void wave_count(uint32_t* arr, uint32_t key) {
#pragma unroll
  for (int round = 0; round < 2; ++round) {
    const uint64_t act = __ballot(key != NONE);
    if (act == 0) return;
    const int leader = __ffsll((unsigned long long)act) - 1;
    const uint32_t lk = (uint32_t)__shfl((int)key, leader);
    const uint64_t same = __ballot(key == lk);
    if ((int)__lane_id() == leader) atomicAdd(arr + lk, (uint32_t)__popcll(same));
    if (key == lk) key = NONE;
  }
  if (key != NONE) atomicAdd(arr + key, 1u);
}

struct SelShared {
  uint32_t hist[NW][256];
  uint32_t tot[256];
  uint32_t misc[8];
  uint32_t wsum[NW];
  uint32_t wsum2[NW];
};

// Exclusive count of `pred` over the workgroup in thread order, plus the total.
__device__ __forceinline__ uint32_t block_excl(SelShared& sh, bool pred, uint32_t& total) {
  const uint64_t b = __ballot(pred);
  const int wv = threadIdx.x / WAVE;
  if (__lane_id() == 0) sh.wsum[wv] = (uint32_t)__popcll(b);
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t s = sh.wsum[i];
    before += (i < wv) ? s : 0u;
    all += s;
  }
  __syncthreads();
  total = all;
  return before + (uint32_t)__popcll(b & lanemask_lt());
}

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

// Radix select of the `kth` largest keys among entries for which keep(idx)
// holds.  Returns threshold T and quota (entries == T to take, in index order).
template <class KeyF, class KeepF>
__device__ void radix_select(SelShared& sh, int L, int kth, KeyF key, KeepF keep, uint32_t& T, int& quota) {
  if (kth <= 0) {
    T = NONE;
    quota = 0;
    return;
  }
  uint32_t prefix = 0, mask = 0;
  int krem = kth;
  const int wv = threadIdx.x / WAVE;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = threadIdx.x; i < NW * 256; i += ST) (&sh.hist[0][0])[i] = 0u;
    __syncthreads();
    for (int base = 0; base < L; base += ST) {
      const int idx = base + threadIdx.x;
      uint32_t d = NONE;
      if (idx < L && keep(idx)) {
        const uint32_t u = key(idx);
        if ((u & mask) == prefix) d = (u >> shift) & 255u;
      }
      wave_count(sh.hist[wv], d);
    }
    __syncthreads();
    if (threadIdx.x < 256) {
      uint32_t t = 0;
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) t += sh.hist[w2][threadIdx.x];
      sh.tot[threadIdx.x] = t;
    }
    __syncthreads();
    if (threadIdx.x < WAVE) {
      const int lane = threadIdx.x;
      uint32_t c4[4], s = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) { c4[q] = sh.tot[255 - 4 * lane - q]; s += c4[q]; }
      uint32_t above = wave_excl_scan(s);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (above < (uint32_t)krem && (uint32_t)krem <= above + c4[q]) {
          sh.misc[0] = 255u - 4u * lane - q;
          sh.misc[1] = above;
        }
        above += c4[q];
      }
    }
    __syncthreads();
    const uint32_t b = sh.misc[0], above = sh.misc[1];
    prefix |= b << shift;
    mask |= 255u << shift;
    krem -= (int)above;
    __syncthreads();
  }
  T = prefix;
  quota = krem;
}

// Writes the indices selected by (key > T) or (key == T and tie rank < quota),
// ascending, to out[].  Optionally only among entries with keep(idx).
template <class KeyF, class KeepF>
__device__ void emit_ordered(SelShared& sh, int L, KeyF key, KeepF keep, uint32_t T, int quota, int32_t* out,
                             int cap) {
  uint32_t ties = 0, sel = 0;
  for (int base = 0; base < L; base += ST) {
    const int idx = base + threadIdx.x;
    const bool ok = idx < L && keep(idx);
    const uint32_t u = ok ? key(idx) : 0u;
    const bool eq = ok && T != NONE && u == T;
    const bool gt = ok && T != NONE && u > T;
    uint32_t teq;
    const uint32_t rank = ties + block_excl(sh, eq, teq);
    const bool take = gt || (eq && rank < (uint32_t)quota);
    uint32_t tsel;
    const uint32_t pos = sel + block_excl(sh, take, tsel);
    if (take && pos < (uint32_t)cap) out[pos] = idx;
    ties += teq;
    sel += tsel;
  }
}

// ---------------------------------------------------------------- layer-wide top-B
// mode ADA / CK: k = P (host), budgets by safeguard.  LAVA: k from klist, budgets = counts,
// and every head's share of the threshold ties is stored for the emission.
__global__ __launch_bounds__(ST) void select_layer_kernel(const float* __restrict__ score, int hkv, int p, int P,
                                                          const int64_t* __restrict__ klist, int alpha_num,
                                                          int alpha_den, int lava, int32_t* __restrict__ budgets,
                                                          uint32_t* __restrict__ hthr, int32_t* __restrict__ hquota,
                                                          int64_t* __restrict__ sel_off, int n_inst) {
  __shared__ SelShared sh;
  __shared__ uint32_t cnt_gt[256], cnt_eq[256];
  __shared__ int64_t qv[256], rv[256];
  __shared__ int64_t sums[2];
  const int inst = blockIdx.x;
  const float* x = score + (size_t)inst * hkv * p;
  const int L = hkv * p;
  const int k = lava ? (int)klist[inst] : P;
  auto key = [&](int i) { return score_key(x[i]); };
  auto all = [](int) { return true; };
  uint32_t T;
  int quota;
  radix_select(sh, L, k, key, all, T, quota);

  for (int i = threadIdx.x; i < hkv; i += ST) { cnt_gt[i] = 0u; cnt_eq[i] = 0u; }
  __syncthreads();
  const int wv = threadIdx.x / WAVE;
  (void)wv;
  for (int base = 0; base < L; base += ST) {
    const int idx = base + threadIdx.x;
    uint32_t hg = NONE, he = NONE;
    if (idx < L && T != NONE) {
      const uint32_t u = key(idx);
      const uint32_t hd = (uint32_t)(idx / p);
      if (u > T) hg = hd;
      else if (u == T) he = hd;
    }
    wave_count(cnt_gt, hg);
    wave_count(cnt_eq, he);
  }
  __syncthreads();
  if (threadIdx.x < hkv) {
    const int g = threadIdx.x;
    int64_t before = 0;
    for (int j = 0; j < g; ++j) before += cnt_eq[j];
    int64_t share = (int64_t)quota - before;
    share = share < 0 ? 0 : (share > (int64_t)cnt_eq[g] ? (int64_t)cnt_eq[g] : share);
    const int64_t f = (int64_t)cnt_gt[g] + share;
    const size_t s = (size_t)inst * hkv + g;
    if (lava) {
      budgets[s] = (int32_t)f;
      hthr[s] = T;
      hquota[s] = (int32_t)share;
    } else {
      const int64_t a = alpha_num, b = alpha_den, h = hkv;
      const int64_t num = a * h * f + (b - a) * (int64_t)k;
      const int64_t den = b * h;
      qv[g] = num / den;
      rv[g] = num % den;
    }
  }
  __syncthreads();
  if (!lava) {
    if (threadIdx.x == 0) {
      int64_t sq = 0;
      for (int j = 0; j < hkv; ++j) sq += qv[j];
      sums[0] = (int64_t)k - sq;
    }
    __syncthreads();
    if (threadIdx.x < hkv) {
      const int g = threadIdx.x;
      int rank = 0;
      for (int j = 0; j < hkv; ++j) rank += (rv[j] > rv[g] || (rv[j] == rv[g] && j < g)) ? 1 : 0;
      budgets[(size_t)inst * hkv + g] = (int32_t)(qv[g] + (rank < sums[0] ? 1 : 0));
    }
    if (threadIdx.x == 0) {
      sel_off[inst] = (int64_t)inst * k;
      if (inst == n_inst - 1) sel_off[n_inst] = (int64_t)n_inst * k;
    }
  }
}

// ---------------------------------------------------------------- per-head selection
enum { HEAD_ADA = 0, HEAD_LAVA = 1, HEAD_CK = 2 };

__global__ __launch_bounds__(ST) void select_head_kernel(const float* __restrict__ score,
                                                         const float* __restrict__ score2, int hkv, int p,
                                                         int mode, int ck_num, int ck_den,
                                                         const int32_t* __restrict__ budgets,
                                                         const uint32_t* __restrict__ hthr,
                                                         const int32_t* __restrict__ hquota,
                                                         const int64_t* __restrict__ sel_off,
                                                         int32_t* __restrict__ sel) {
  __shared__ SelShared sh;
  extern __shared__ uint32_t member[];   // CriticalKV stage-1 membership bits, (p + 31) / 32 words
  const int s = blockIdx.x, inst = s / hkv, g = s % hkv;
  const float* x = score + (size_t)s * p;
  const int B = budgets[s];
  int64_t base = sel_off[inst];
  for (int j = 0; j < g; ++j) base += budgets[(size_t)inst * hkv + j];
  int32_t* out = sel + base;
  auto keyA = [&](int i) { return score_key(x[i]); };
  auto all = [](int) { return true; };
  if (mode == HEAD_LAVA) {
    emit_ordered(sh, p, keyA, all, hthr[s], hquota[s], out, B);
    return;
  }
  if (mode == HEAD_ADA) {
    uint32_t T;
    int q;
    radix_select(sh, p, B, keyA, all, T, q);
    emit_ordered(sh, p, keyA, all, T, q, out, B);
    return;
  }
  // CriticalKV two-stage.
  const int b1 = (int)(((int64_t)B * ck_num) / ck_den);
  const int b2 = B - b1;
  uint32_t* mem = member;
  uint32_t T1;
  int q1;
  radix_select(sh, p, b1, keyA, all, T1, q1);
  {
    uint32_t ties = 0;
    for (int base2 = 0; base2 < p; base2 += ST) {
      const int idx = base2 + threadIdx.x;
      const bool ok = idx < p;
      const uint32_t u = ok ? keyA(idx) : 0u;
      const bool eq = ok && T1 != NONE && u == T1;
      const bool gt = ok && T1 != NONE && u > T1;
      uint32_t teq;
      const uint32_t rank = ties + block_excl(sh, eq, teq);
      const bool in1 = gt || (eq && rank < (uint32_t)q1);
      const uint64_t bits = __ballot(in1);
      if (__lane_id() == 0) {
        const int wi = (base2 + (threadIdx.x & ~63)) / 32;
        if (wi * 32 < p) mem[wi] = (uint32_t)bits;
        if ((wi + 1) * 32 < p) mem[wi + 1] = (uint32_t)(bits >> 32);
      }
      ties += teq;
    }
  }
  __syncthreads();
  const float* y = score2 + (size_t)s * p;
  auto keyB = [&](int i) { return score_key(y[i]); };
  auto notin1 = [&](int i) { return ((mem[i >> 5] >> (i & 31)) & 1u) == 0u; };
  uint32_t T2;
  int q2;
  radix_select(sh, p, b2, keyB, notin1, T2, q2);
  uint32_t ties2 = 0, sel_n = 0;
  for (int base2 = 0; base2 < p; base2 += ST) {
    const int idx = base2 + threadIdx.x;
    const bool ok = idx < p;
    const bool in1 = ok && !notin1(idx);
    const uint32_t u = ok ? keyB(idx) : 0u;
    const bool eq2 = ok && !in1 && T2 != NONE && u == T2;
    const bool gt2 = ok && !in1 && T2 != NONE && u > T2;
    uint32_t teq;
    const uint32_t rank = ties2 + block_excl(sh, eq2, teq);
    const bool take = in1 || gt2 || (eq2 && rank < (uint32_t)q2);
    uint32_t tsel;
    const uint32_t pos = sel_n + block_excl(sh, take, tsel);
    if (take && pos < (uint32_t)B) out[pos] = idx;
    ties2 += teq;
    sel_n += tsel;
  }
}

// ---------------------------------------------------------------- LAVa layer budgets
// Per layer: S = sum s, Q = sum s ln s in fp64; e_l = (ln S - Q / S) / (hkv * p).
__global__ __launch_bounds__(ST) void lava_entropy_kernel(const float* __restrict__ score, int hkv, int p,
                                                          double* __restrict__ ent) {
  __shared__ double red[2][NW];
  const int l = blockIdx.x;
  const float* x = score + (size_t)l * hkv * p;
  const int L = hkv * p;
  double S = 0.0, Q = 0.0;
  for (int i = threadIdx.x; i < L; i += ST) {
    const double v = (double)x[i];
    S += v;
    Q += (v > 0.0) ? v * log(v) : 0.0;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    S += __shfl_xor(S, off);
    Q += __shfl_xor(Q, off);
  }
  const int wv = threadIdx.x / WAVE;
  if (__lane_id() == 0) { red[0][wv] = S; red[1][wv] = Q; }
  __syncthreads();
  if (threadIdx.x == 0) {
    double s2 = 0.0, q2 = 0.0;
    for (int i = 0; i < NW; ++i) { s2 += red[0][i]; q2 += red[1][i]; }
    ent[l] = (s2 > 0.0) ? (log(s2) - q2 / s2) / (double)L : 0.0;
  }
}

// One workgroup: B'_l = largest remainder of B' * e_l / sum(e), sel_off = scan.
__global__ __launch_bounds__(ST) void lava_budget_kernel(const double* __restrict__ ent, int L, int64_t Bp,
                                                         int64_t* __restrict__ klist, int64_t* __restrict__ sel_off) {
  extern __shared__ __align__(16) char smem[];
  double* rem = reinterpret_cast<double*>(smem);
  int64_t* fl = reinterpret_cast<int64_t*>(rem + L);
  __shared__ double Esh;
  __shared__ int64_t def;
  if (threadIdx.x == 0) {
    double E = 0.0;
    for (int i = 0; i < L; ++i) E += ent[i];
    Esh = E;
  }
  __syncthreads();
  const double E = Esh;
  for (int l = threadIdx.x; l < L; l += ST) {
    const double x = (E > 0.0) ? ((double)Bp * ent[l]) / E : (double)Bp / (double)L;
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
  for (int l = threadIdx.x; l < L; l += ST) {
    int64_t rank = 0;
    for (int j = 0; j < L; ++j) rank += (rem[j] > rem[l] || (rem[j] == rem[l] && j < l)) ? 1 : 0;
    klist[l] = fl[l] + (rank < def ? 1 : 0);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t s = 0;
    for (int i = 0; i < L; ++i) { sel_off[i] = s; s += klist[i]; }
    sel_off[L] = s;
  }
}

struct AllocPlan {
  size_t off_thr, off_quota, off_ent, off_k, total;
};

AllocPlan plan_alloc(const Geo& g) {
  AllocPlan P{};
  const size_t S = (size_t)g.I * g.hkv;
  size_t off = 0;
  P.off_thr = off;    off = align_up(off + S * 4, 256);
  P.off_quota = off;  off = align_up(off + S * 4, 256);
  P.off_ent = off;    off = align_up(off + (size_t)g.I * 8, 256);
  P.off_k = off;      off = align_up(off + (size_t)g.I * 8, 256);
  P.total = off;
  return P;
}

}  // namespace

size_t alloc_ws_bytes(const Geo& g, const adakv_alloc&) { return plan_alloc(g).total; }

hipError_t launch_allocate(const Geo& g, const adakv_alloc& a, const float* score, const float* score2,
                           int32_t* budgets, int32_t* sel, int64_t* sel_off, char* ws, hipStream_t st) {
  const AllocPlan P = plan_alloc(g);
  uint32_t* hthr = reinterpret_cast<uint32_t*>(ws + P.off_thr);
  int32_t* hquota = reinterpret_cast<int32_t*>(ws + P.off_quota);
  double* ent = reinterpret_cast<double*>(ws + P.off_ent);
  int64_t* klist = reinterpret_cast<int64_t*>(ws + P.off_k);
  const int S = g.I * g.hkv;
  if (a.mode == ADAKV_ALLOC_LAVA_LAYERS) {
    const int64_t Bp = a.budget - (int64_t)g.I * g.w * g.hkv;
    lava_entropy_kernel<<<g.I, ST, 0, st>>>(score, g.hkv, g.p, ent);
    const size_t sm = (size_t)g.I * (sizeof(double) + sizeof(int64_t));
    lava_budget_kernel<<<1, ST, sm, st>>>(ent, g.I, Bp, klist, sel_off);
    select_layer_kernel<<<g.I, ST, 0, st>>>(score, g.hkv, g.p, 0, klist, 0, 1, 1, budgets, hthr, hquota, sel_off,
                                            g.I);
    select_head_kernel<<<S, ST, 0, st>>>(score, nullptr, g.hkv, g.p, HEAD_LAVA, 0, 1, budgets, hthr, hquota,
                                         sel_off, sel);
    return hipGetLastError();
  }
  const int P0 = (int)(a.budget - (int64_t)g.w * g.hkv);
  select_layer_kernel<<<g.I, ST, 0, st>>>(score, g.hkv, g.p, P0, nullptr, a.alpha_num, a.alpha_den, 0, budgets,
                                          hthr, hquota, sel_off, g.I);
  const int mode = (a.mode == ADAKV_ALLOC_ADA_CRITICALKV) ? HEAD_CK : HEAD_ADA;
  const size_t lds = (mode == HEAD_CK) ? (size_t)((g.p + 31) / 32) * 4 : 0;
  select_head_kernel<<<S, ST, lds, st>>>(score, score2, g.hkv, g.p, mode, a.ck_num, a.ck_den, budgets, hthr, hquota,
                                         sel_off, sel);
  return hipGetLastError();
}

}  // namespace adakv
