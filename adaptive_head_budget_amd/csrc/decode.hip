// Decode attention over the flat variable-length cache on gfx950.
//
// Ada-KV notes, "多头自注意力层的形式化描述": the new key/value is appended to
// the cache, then A_i = softmax(q_i K^T) (scaled by 1/sqrt(d_h), LAVa notes
// "解码过程的残差流视角") and the head output A_i V.  The varlen design follows
// the Ada-KV paper's "Variable-length Attention with Variable-sized Cache
// Elements": every segment (instance, KV head) has its own length, and the G
// query heads of a GQA group share every row read.
//
// One workgroup streams one segment (or one of `nsplit` row ranges of it when
// segments are too few to fill the chip).  Each of its 4 waves takes 32 rows of
// every 128-row chunk: keys go straight to LDS with coalesced direct loads,
// q.K^T runs on 16x16 MFMA tiles (rows on M, query heads on N), an online
// softmax per wave, and the value sum on the vector units with 16-byte
// coalesced V loads.  Waves only touch their own LDS, so they never wait for
// each other inside the chunk loop.  The new row of an append is read straight from
// k_new/v_new and also stored into the segment's reserved rows for later steps;
// seg_len is never modified (a call attends over seg_len + step (+1) rows), so
// a decode call carries no state from the previous one.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace adakv {
namespace {

constexpr int WR = 32;          // rows per wave per chunk
constexpr int CH = 4 * WR;      // rows per chunk (4 waves)

// Keys reach LDS with 16-byte direct-to-LDS loads: lane l of a load writes
// LDS bytes [16*l, 16*l + 16) of the instruction's 1 KB block (4 rows), so
// 16 lanes move one full 256-byte row and every load is coalesced.  Lane
// (row r, slot cs) fetches 16-byte chunk cs ^ (r & 15) of the row; an MFMA
// read of chunk ch of row r then uses slot ch ^ (r & 15), and the 16 rows of
// one read land in 16 different bank groups.
template <typename T, int D, int GT>
__global__ __launch_bounds__(256, 4) void decode_kernel(const T* __restrict__ q, const T* __restrict__ k_new,
                                                     const T* __restrict__ v_new, T* __restrict__ kf,
                                                     T* __restrict__ vf, const int64_t* __restrict__ seg_start,
                                                     const int32_t* __restrict__ seg_len, int hq, int hkv, int G,
                                                     int nsplit, int extra, int append, float c2,
                                                     float* __restrict__ out, float* __restrict__ part) {
  using M = Mma<T>;
  constexpr int KSTEPS = D / M::KSTEP;
  constexpr int ROWB = D * (int)sizeof(T);     // bytes per row
  constexpr int CPR = ROWB / 16;               // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;                // rows per direct load
  constexpr int EPL = 16 / (int)sizeof(T);     // value elements per lane
  constexpr int LPR = D / EPL;                 // lanes per value row
  constexpr int RS = WAVE / LPR;               // row slots per wave
  constexpr int RPL = WR / RS;                 // value rows per lane per chunk
  constexpr int MB = WR / 16;                  // M-blocks per wave
  // A wave's key slot also holds its partial output once its rows are done.
  static_assert(GT * D * sizeof(float) <= WR * ROWB, "partial output must fit a key slot");
  __shared__ __align__(16) char kbuf[4][WR * ROWB];
  __shared__ float P[4][WR][GT];
  __shared__ float Sc[4][GT];
  __shared__ float Mw[4][GT], Lw[4][GT];

  // Workgroups are dealt round-robin to the 8 XCDs and then to an XCD's CUs, so
  // with segment = block index every CU would hold segments of one KV head.  The
  // [8][S/8] -> [S/8][8] transpose gives the workgroups sharing a CU different
  // heads, whose unequal Ada-KV budgets then even out (split launches, with
  // few segments, keep the identity).
  int bx = blockIdx.x;
  if (nsplit == 1 && gridDim.x % 8 == 0) {
    const int Q = gridDim.x / 8;
    bx = (bx % Q) * 8 + bx / Q;
  }
  const int s = bx / nsplit, split = bx % nsplit;
  const int inst = s / hkv, g = s % hkv;
  const int64_t base = seg_start[s];
  const int cap = (int)(seg_start[s + 1] - base);
  const int len0 = seg_len[s];
  int len = len0 + extra;
  const bool do_append = append && (len0 + extra - 1) < cap;
  if (len > cap) len = cap;                      // never read past the segment's rows
  const int newrow = do_append ? len0 + extra - 1 : -1;
  const int nch = (len + CH - 1) / CH;
  const int cps = (nch + nsplit - 1) / nsplit;
  const int r_begin = split * cps * CH;
  const int r_end = min(len, r_begin + cps * CH);

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int gq = lane >> 4, c = lane & 15;
  const int rs = lane / LPR, cc = lane % LPR;
  const T* knew_s = k_new + (size_t)s * D;
  const T* vnew_s = v_new + (size_t)s * D;
  char* kb = kbuf[wv];

  if (do_append && split == 0 && threadIdx.x < CPR) {
    st16(kf + (base + newrow) * D + threadIdx.x * EPL, ld16(knew_s + threadIdx.x * EPL));
    st16(vf + (base + newrow) * D + threadIdx.x * EPL, ld16(vnew_s + threadIdx.x * EPL));
  }

  // B operand: q^T, column c = query head of the group (zero beyond G).
  typename M::op_t qop[KSTEPS];
  const T* qb = q + ((size_t)inst * hq + (size_t)g * G + (c < G ? c : 0)) * D;
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) qop[ks] = (c < G) ? M::load(qb + ks * M::KSTEP + M::KPL * gq) : M::zero();

  // this lane's part of every direct key load: row lr of each 4-row block, chunk slot cs
  const int lr = lane / CPR, cs = lane % CPR;
  float m_run = -INFINITY, l_run = 0.f;   // per query head c (same in the 4 lane groups)
  float o[GT][EPL];
#pragma unroll
  for (int h = 0; h < GT; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = 0.f;

  for (int c0 = r_begin; c0 < r_end; c0 += CH) {
    const int wrow0 = c0 + WR * wv;
    // keys: direct to LDS, rows wrow0 .. wrow0 + WR - 1
#pragma unroll
    for (int i = 0; i < WR / RPI; ++i) {
      const int rr = i * RPI + lr;
      const int r = wrow0 + rr;
      const T* src = (r == newrow) ? knew_s : kf + (base + (r < r_end ? r : r_begin)) * D;
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src + ((cs ^ (rr & 15)) % CPR) * EPL),
                                       static_cast<void*>(&kbuf[wv][i * 1024]), 16, 0, 0);
    }
    // values: registers
    u32x4 vraw[RPL];
#pragma unroll
    for (int t = 0; t < RPL; ++t) {
      const int r = wrow0 + t * RS + rs;
      const T* src = (r == newrow) ? vnew_s : vf + (base + (r < r_end ? r : r_begin)) * D;
      vraw[t] = ld16_nt(src + cc * EPL);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");     // keys in LDS, values in registers
    f32x4 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      acc[mb] = zero4();
      const int rr = 16 * mb + c;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const int ch = (ks * M::KSTEP + M::KPL * gq) / EPL;     // 16-byte chunk of this operand
        const T* ap = reinterpret_cast<const T*>(kb + rr * ROWB + (((ch ^ (rr & 15)) % CPR) * 16)) +
                      (ks * M::KSTEP + M::KPL * gq) % EPL;
        acc[mb] = M::mma(M::load(ap), qop[ks], acc[mb]);
      }
    }
    // acc[mb][j] <-> row wrow0 + 16*mb + 4*gq + j, query head c
    float mc = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (wrow0 + 16 * mb + 4 * gq + j < r_end) mc = fmaxf(mc, acc[mb][j]);
    mc = fmaxf(mc, shfl_xor(mc, 16));
    mc = fmaxf(mc, shfl_xor(mc, 32));
    const float m_new = fmaxf(m_run, mc);
    const float sc_run = (m_run == -INFINITY) ? 0.f : fast_exp2((m_run - m_new) * c2);
    const float mnc = m_new * c2;
    float lc = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rr = 16 * mb + 4 * gq + j;
        const float e = (wrow0 + rr < r_end) ? fast_exp2(fmaf(acc[mb][j], c2, -mnc)) : 0.f;
        lc += e;
        if (c < GT) P[wv][rr][c] = e;
      }
    lc += shfl_xor(lc, 16);
    lc += shfl_xor(lc, 32);
    l_run = l_run * sc_run + lc;
    m_run = m_new;
    if (gq == 0 && c < GT) Sc[wv][c] = sc_run;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's P / Sc writes are visible to its lanes
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      const float sh = Sc[wv][h];
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] *= sh;
    }
#pragma unroll
    for (int t = 0; t < RPL; ++t) {
      const int rr = t * RS + rs;
      float vv[EPL];
      if (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < EPL / 2; ++e) {
          vv[2 * e] = bf16_bits_to_f32(vraw[t][e] & 0xffffu);
          vv[2 * e + 1] = bf16_bits_to_f32(vraw[t][e] >> 16);
        }
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) vv[e] = __uint_as_float(vraw[t][e]);
      }
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        const float pw = P[wv][rr][h];   // 0 for rows past the end
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[h][e] += pw * vv[e];
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // LDS reads done before the next chunk overwrites kbuf / P
  }
  // sum the row slots of each wave, then combine the waves in order
#pragma unroll
  for (int msk = LPR; msk < 64; msk <<= 1)
#pragma unroll
    for (int h = 0; h < GT; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] += shfl_xor(o[h][e], msk);
  float* ow = reinterpret_cast<float*>(kbuf[wv]);   // [GT][D]; only this wave used this slot
  if (rs == 0) {
#pragma unroll
    for (int h = 0; h < GT; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) ow[h * D + cc * EPL + e] = o[h][e];
  }
  if (gq == 0 && c < GT) {
    Mw[wv][c] = m_run;
    Lw[wv][c] = l_run;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * (D + 2); idx += blockDim.x) {
    const int h = idx / (D + 2), e = idx % (D + 2);
    float Mx = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) Mx = fmaxf(Mx, Mw[w2][h]);
    float acc2 = 0.f, l2 = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
      const float sc = (Mw[w2][h] == -INFINITY) ? 0.f : fast_exp2((Mw[w2][h] - Mx) * c2);
      l2 += sc * Lw[w2][h];
      if (e < D) acc2 += sc * reinterpret_cast<const float*>(kbuf[w2])[h * D + e];
    }
    if (nsplit == 1) {
      if (e < D) out[((size_t)inst * hq + (size_t)g * G + h) * D + e] = acc2 / l2;
    } else {
      part[((size_t)bx * G + h) * (D + 2) + e] = (e < D) ? acc2 : (e == D ? Mx : l2);
    }
  }
}

template <int D>
__global__ void decode_merge_kernel(const float* __restrict__ part, int hq, int hkv, int G, int nsplit, float c2,
                                    float* __restrict__ out) {
  const int inst = blockIdx.x / hq, jq = blockIdx.x % hq;
  const int g = jq / G, h = jq % G;
  const int s = inst * hkv + g;
  float Mx = -INFINITY;
  for (int sp = 0; sp < nsplit; ++sp) Mx = fmaxf(Mx, part[(((size_t)s * nsplit + sp) * G + h) * (D + 2) + D]);
  for (int e = threadIdx.x; e < D; e += blockDim.x) {
    float o = 0.f, l = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) {
      const float* pp = part + (((size_t)s * nsplit + sp) * G + h) * (D + 2);
      const float sc = (pp[D] == -INFINITY) ? 0.f : fast_exp2((pp[D] - Mx) * c2);
      o += sc * pp[e];
      l += sc * pp[D + 1];
    }
    out[((size_t)inst * hq + jq) * D + e] = o / l;
  }
}

// Splits per segment: one workgroup per segment when there are enough
// segments to fill the chip, else enough splits of >= 2 chunks each.
int choose_splits(const Geo& g, int64_t max_rows) {
  const int S = g.I * g.hkv;
  if (S >= 512) return 1;
  const int64_t avg = max_rows / S;
  int want = (1024 + S - 1) / S;
  const int64_t lim = avg / (2 * CH);
  if (want > lim) want = (int)lim;
  return want < 1 ? 1 : want;
}

template <typename T, int D, int GT>
hipError_t run_decode(const Geo& g, int64_t max_rows, int extra, const void* q, const void* k_new, const void* v_new,
                      void* k_flat, void* v_flat, const int64_t* seg_start, const int32_t* seg_len, float* out,
                      char* ws, hipStream_t st) {
  const int S = g.I * g.hkv;
  const int nsplit = choose_splits(g, max_rows);
  const float c2 = (float)(1.4426950408889634 / std::sqrt((double)g.d));
  float* part = reinterpret_cast<float*>(ws);
  const int append = k_new != nullptr;
  decode_kernel<T, D, GT><<<(unsigned)(S * nsplit), 256, 0, st>>>(
      static_cast<const T*>(q), static_cast<const T*>(k_new), static_cast<const T*>(v_new), static_cast<T*>(k_flat),
      static_cast<T*>(v_flat), seg_start, seg_len, g.hq, g.hkv, g.G, nsplit, extra, append, c2, out, part);
  if (nsplit > 1)
    decode_merge_kernel<D><<<g.I * g.hq, D < 64 ? 64 : D, 0, st>>>(part, g.hq, g.hkv, g.G, nsplit, c2, out);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run_decode_g(const Geo& g, int64_t max_rows, int extra, const void* q, const void* k_new,
                        const void* v_new, void* k_flat, void* v_flat, const int64_t* seg_start,
                        const int32_t* seg_len, float* out, char* ws, hipStream_t st) {
#define RUN(GTV) run_decode<T, D, GTV>(g, max_rows, extra, q, k_new, v_new, k_flat, v_flat, seg_start, seg_len, out, ws, st)
  if (g.G <= 1) return RUN(1);
  if (g.G <= 2) return RUN(2);
  if (g.G <= 4) return RUN(4);
  return RUN(8);
#undef RUN
}

// Split partials of adakv_decode_attn_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends.  Host code reaches it only
// through the address hipGetSymbolAddress returns for the current device (the
// array's name is a host-side stand-in, not a device address).
constexpr size_t kDecodeScratchBytes = (size_t)8 << 20;
__device__ __align__(256) char scratch[kDecodeScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

}  // namespace

size_t decode_scratch_capacity() { return kDecodeScratchBytes; }

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    scratch_ptr[dev] = p;
  }
  *ptr = scratch_ptr[dev];
  return hipSuccess;
}

size_t decode_ws_bytes(const Geo& g, int64_t max_rows) {
  const int S = g.I * g.hkv;
  return (size_t)S * choose_splits(g, max_rows) * g.G * (g.d + 2) * sizeof(float);
}

hipError_t launch_decode(const Geo& g, int64_t max_rows, int extra, const void* q, const void* k_new,
                         const void* v_new, void* k_flat, void* v_flat, const int64_t* seg_start,
                         const int32_t* seg_len, float* out, char* ws, hipStream_t st) {
  if (g.dtype == ADAKV_BF16) {
    if (g.d == 128) return run_decode_g<uint16_t, 128>(g, max_rows, extra, q, k_new, v_new, k_flat, v_flat, seg_start, seg_len, out, ws, st);
    if (g.d == 64) return run_decode_g<uint16_t, 64>(g, max_rows, extra, q, k_new, v_new, k_flat, v_flat, seg_start, seg_len, out, ws, st);
  } else {
    if (g.d == 16) return run_decode_g<float, 16>(g, max_rows, extra, q, k_new, v_new, k_flat, v_flat, seg_start, seg_len, out, ws, st);
    if (g.d == 64) return run_decode_g<float, 64>(g, max_rows, extra, q, k_new, v_new, k_flat, v_flat, seg_start, seg_len, out, ws, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace adakv
