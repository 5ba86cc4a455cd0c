// Internal launch interface between the C ABI (abi.hip) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "adakv.h"

namespace adakv {

// Validated geometry of a call.
struct Geo {
  int I, hq, hkv, G, d, n, w, p, pool, dtype, scorer, hidden;
  float eps;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---- scoring (score.hip, vwo.hip)
size_t score_ws_bytes(const Geo& g);
// row_lse: NULL (two passes over K) or the caller's per-row log-sum-exp [I, hq, w]
hipError_t launch_score(const Geo& g, const void* q, const void* k, const void* v, const void* w_o,
                        const float* row_lse, float* score, float* score2, char* ws, hipStream_t st);
// factor: w_o holds the two bf16 planes of the Gram factors written by
// launch_factor (LaProx with a wide projection) instead of the projection.
hipError_t launch_vwo(const Geo& g, int inst0, int ni, const void* v, const void* w_o,
                      const float* head_scores, float* score2, bool factor, hipStream_t st);
// LaProx: the L2 value norms through the d x d Gram factor when the projection
// is at least four times as wide as the head (hidden >= 4 d).
inline bool use_factor(const Geo& g) { return g.scorer == ADAKV_SCORE_LAPROX && g.hidden >= 4 * g.d; }
// slices of the hidden dimension summed separately for the Gram matrices
inline int factor_slices(const Geo& g) {
  for (int s = 8; s > 1; s >>= 1)
    if (g.hidden % (32 * s) == 0) return s;
  return 1;
}
size_t factor_ws_bytes(const Geo& g);
hipError_t launch_factor(const Geo& g, const void* w_o, char* ws, hipStream_t st);
// Window-row log-sum-exp of the scorer's key domain from the causal one (causal.hip).
hipError_t launch_lse_from_causal(const Geo& g, const void* q_win, const void* k, const float* lse_c,
                                  float* lse_out, int32_t* row_flag, hipStream_t st);

// ---- allocation (select.hip)
size_t alloc_ws_bytes(const Geo& g, const adakv_alloc& a);
// LAVa online prefill only (online = true, a LAVA_LAYERS call whose layer
// budgets are capped by the previous step's), else unused:
//   prev_off       the previous step's sel_off (NULL at the first step)
//   layer_ent      [I] each layer's entropy: 0..I-2 read, I-1 written
//   prev_budgets, prev_sel  the previous step's outputs; with them the older
//                  layers are re-selected from their previous entries
hipError_t launch_allocate(const Geo& g, const adakv_alloc& a, const float* score, const float* score2,
                           int32_t* budgets, int32_t* sel, int64_t* sel_off, char* ws, hipStream_t st,
                           bool online = false, const int64_t* prev_off = nullptr,
                           const int32_t* prev_budgets = nullptr, const int32_t* prev_sel = nullptr,
                           double* layer_ent = nullptr);

// ---- compaction (compact.hip)
hipError_t launch_compact(const Geo& g, int64_t retained_rows, const void* k, const void* v,
                          const int32_t* budgets, const int32_t* sel, const int64_t* sel_off, int reserve,
                          void* k_flat, void* v_flat, int64_t* seg_start, int32_t* seg_len, hipStream_t st);

// LAVa online prefill: flat cache of layers 0..I-1 from the newest layer's
// dense K/V and the previous flat cache of layers 0..I-2 (no reserve rows).
hipError_t launch_online_compact(const Geo& g, int64_t max_rows, const void* k_new, const void* v_new,
                                 const void* k_old, const void* v_old, const int64_t* seg_start_old,
                                 const int32_t* sel_old, const int64_t* sel_off_old, const int32_t* budgets,
                                 const int32_t* sel, const int64_t* sel_off, void* k_flat, void* v_flat,
                                 int64_t* seg_start, int32_t* seg_len, hipStream_t st);

// ---- decode (decode.hip)
size_t decode_ws_bytes(const Geo& g, int64_t max_rows);
// The allocation-free decode's scratch: the calling device's copy of a fixed
// file-scope array (its address is looked up once per device).
size_t decode_scratch_capacity();
hipError_t decode_scratch(void** ptr);
// extra = appends made before this call + 1 if this call appends
hipError_t launch_decode(const Geo& g, int64_t max_rows, int extra, const void* q, const void* k_new,
                         const void* v_new, void* k_flat, void* v_flat, const int64_t* seg_start,
                         const int32_t* seg_len, float* out, char* ws, hipStream_t st);

}  // namespace adakv
