// C ABI of libadakv: argument checks on the host, then launches on the caller's
// stream.  Nothing here allocates device memory or waits for the device.
#include <cmath>
#include <cstdint>

#include "kernels.hpp"

using namespace adakv;

namespace {

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks common to every call; fills g.
adakv_status check_shape(const adakv_shape* s, Geo& g) {
  if (s == nullptr) return ADAKV_EINVAL;
  if (s->n_inst < 1 || s->hq < 1 || s->hkv < 1 || s->d < 1 || s->w < 1 || s->n <= s->w) return ADAKV_EINVAL;
  if (s->hq % s->hkv != 0) return ADAKV_EINVAL;
  if (s->pool < 1 || s->pool % 2 == 0) return ADAKV_EINVAL;
  if (s->dtype != ADAKV_BF16 && s->dtype != ADAKV_F32) return ADAKV_EINVAL;
  if (s->scorer < ADAKV_SCORE_SNAPKV || s->scorer > ADAKV_SCORE_LAPROX) return ADAKV_EINVAL;
  // sizes that keep every index in 32 bits per segment and 64 bits overall
  if ((int64_t)s->hkv * (s->n - s->w) > (int64_t)1 << 30) return ADAKV_EUNSUPPORTED;
  if (s->hkv > 256) return ADAKV_EUNSUPPORTED;
  g.I = s->n_inst;
  g.hq = s->hq;
  g.hkv = s->hkv;
  g.G = s->hq / s->hkv;
  g.d = s->d;
  g.n = s->n;
  g.w = s->w;
  g.p = s->n - s->w;
  g.pool = s->pool;
  g.dtype = s->dtype;
  g.scorer = s->scorer;
  g.hidden = s->hidden;
  g.eps = s->eps;
  const bool dok = (s->dtype == ADAKV_BF16) ? (s->d == 64 || s->d == 128) : (s->d == 16 || s->d == 64);
  if (!dok) return ADAKV_EUNSUPPORTED;
  return ADAKV_OK;
}

adakv_status check_alloc(const adakv_alloc* a, const Geo& g) {
  if (a == nullptr) return ADAKV_EINVAL;
  if (a->mode < ADAKV_ALLOC_ADA || a->mode > ADAKV_ALLOC_STREAMING) return ADAKV_EINVAL;
  if (a->mode == ADAKV_ALLOC_LAVA_LAYERS) {
    const int64_t bp = a->budget - (int64_t)g.I * g.w * g.hkv;
    if (bp < 0 || bp > (int64_t)g.hkv * g.p) return ADAKV_EINVAL;
  } else if (a->mode == ADAKV_ALLOC_GLOBAL) {
    const int64_t bp = a->budget - (int64_t)g.I * g.w * g.hkv;
    if (bp < 0 || bp > (int64_t)g.I * g.hkv * g.p) return ADAKV_EINVAL;
    // one radix select over every score of the call: 32-bit counts
    if ((int64_t)g.I * g.hkv * g.p > (int64_t)INT32_MAX) return ADAKV_EUNSUPPORTED;
  } else {
    if (a->alpha_den <= 0 || a->alpha_num < 0 || a->alpha_num > a->alpha_den) return ADAKV_EINVAL;
    if (a->inst_budget == nullptr && (a->budget < (int64_t)g.w * g.hkv || a->budget > (int64_t)g.n * g.hkv))
      return ADAKV_EINVAL;
    // the safeguard numerator a*h*f + (b-a)*P stays far inside int64
    if ((int64_t)a->alpha_den > ((int64_t)1 << 20)) return ADAKV_EUNSUPPORTED;
  }
  if (a->inst_budget != nullptr) {
    // per-instance budgets (preset layer budgets): Ada-KV allocation only
    if (a->mode != ADAKV_ALLOC_ADA) return ADAKV_EUNSUPPORTED;
    for (int i = 0; i < g.I; ++i)
      if (a->inst_budget[i] < (int64_t)g.w * g.hkv || a->inst_budget[i] > (int64_t)g.n * g.hkv) return ADAKV_EINVAL;
  }
  if (a->mode == ADAKV_ALLOC_STREAMING && a->sinks < 0) return ADAKV_EINVAL;
  if (a->mode == ADAKV_ALLOC_ADA_CRITICALKV) {
    if (a->ck_den <= 0 || a->ck_num < 0 || a->ck_num > a->ck_den) return ADAKV_EINVAL;
    if ((int64_t)a->ck_den > ((int64_t)1 << 20)) return ADAKV_EUNSUPPORTED;
  }
  return ADAKV_OK;
}

// Rows the selection keeps over all instances (window rows excluded).
int64_t selected_rows(const adakv_alloc& a, const Geo& g) {
  if (a.mode == ADAKV_ALLOC_LAVA_LAYERS || a.mode == ADAKV_ALLOC_GLOBAL) return a.budget - (int64_t)g.I * g.w * g.hkv;
  if (a.inst_budget != nullptr) {
    int64_t s = 0;
    for (int i = 0; i < g.I; ++i) s += a.inst_budget[i] - (int64_t)g.w * g.hkv;
    return s;
  }
  return (int64_t)g.I * (a.budget - (int64_t)g.w * g.hkv);
}

adakv_status hip_status(hipError_t e) { return e == hipSuccess ? ADAKV_OK : ADAKV_EHIP; }

}  // namespace

extern "C" {

int32_t adakv_version(void) { return 100; }

const char* adakv_strerror(adakv_status s) {
  switch (s) {
    case ADAKV_OK: return "ok";
    case ADAKV_EINVAL: return "invalid argument";
    case ADAKV_EUNSUPPORTED: return "unsupported shape or type";
    case ADAKV_ECAPACITY: return "append beyond the reserved rows";
    case ADAKV_EWORKSPACE: return "workspace too small";
    case ADAKV_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

size_t adakv_workspace_bytes(const adakv_shape* shape, const adakv_alloc* alloc, int32_t reserve) {
  Geo g{};
  if (check_shape(shape, g) != ADAKV_OK) return 0;
  size_t need = score_ws_bytes(g);
  if (alloc != nullptr) {
    if (check_alloc(alloc, g) != ADAKV_OK || reserve < 0) return 0;
    const size_t a = alloc_ws_bytes(g, *alloc);
    need = a > need ? a : need;
    const int64_t rows = selected_rows(*alloc, g) + (int64_t)g.I * g.hkv * ((int64_t)g.w + reserve);
    const size_t d = decode_ws_bytes(g, rows);
    need = d > need ? d : need;
  }
  return need < 256 ? 256 : need;
}

namespace {
adakv_status score_call(const adakv_shape* shape, const void* q_win, const void* k, const void* v, const void* w_o,
                        const float* row_lse, float* score, float* score2, void* ws, size_t ws_bytes, void* stream) {
  Geo g{};
  adakv_status st = check_shape(shape, g);
  if (st != ADAKV_OK) return st;
  if (!aligned16(q_win) || !aligned16(k) || !aligned16(score) || !aligned16(ws)) return ADAKV_EINVAL;
  if (g.w > 64 || g.pool > 7 || g.G > 8) return ADAKV_EUNSUPPORTED;
  if (g.scorer == ADAKV_SCORE_LAVA && !aligned16(v)) return ADAKV_EINVAL;
  if (g.scorer == ADAKV_SCORE_CRITICALKV) {
    if (!aligned16(v) || !aligned16(w_o) || !aligned16(score2)) return ADAKV_EINVAL;
    if (g.hidden < 1 || !(g.eps >= 0.f) || !std::isfinite(g.eps)) return ADAKV_EINVAL;
    if (g.dtype != ADAKV_BF16 || g.d != 128 || g.hidden % 64 != 0) return ADAKV_EUNSUPPORTED;
  }
  if (g.scorer == ADAKV_SCORE_LAPROX) {
    if (!aligned16(v) || !aligned16(w_o) || g.hidden < 1 || g.pool != 1) return ADAKV_EINVAL;
    if (g.dtype != ADAKV_BF16 || g.d != 128 || g.hidden % 64 != 0) return ADAKV_EUNSUPPORTED;
  }
  if (ws_bytes < score_ws_bytes(g)) return ADAKV_EWORKSPACE;
  return hip_status(launch_score(g, q_win, k, v, w_o, row_lse, score, score2, static_cast<char*>(ws),
                                 static_cast<hipStream_t>(stream)));
}
}  // namespace

adakv_status adakv_score(const adakv_shape* shape, const void* q_win, const void* k, const void* v, const void* w_o,
                         float* score, float* score2, void* ws, size_t ws_bytes, void* stream) {
  return score_call(shape, q_win, k, v, w_o, nullptr, score, score2, ws, ws_bytes, stream);
}

adakv_status adakv_score_lse(const adakv_shape* shape, const void* q_win, const void* k, const void* v,
                             const void* w_o, const float* row_lse, float* score, float* score2, void* ws,
                             size_t ws_bytes, void* stream) {
  if (!aligned16(row_lse)) return ADAKV_EINVAL;
  return score_call(shape, q_win, k, v, w_o, row_lse, score, score2, ws, ws_bytes, stream);
}

adakv_status adakv_lse_from_causal(const adakv_shape* shape, const void* q_win, const void* k,
                                   const float* lse_causal, float* lse_out, int32_t* row_flag, void* stream) {
  Geo g{};
  adakv_status st = check_shape(shape, g);
  if (st != ADAKV_OK) return st;
  if (!aligned16(q_win) || !aligned16(k) || !aligned16(lse_causal) || !aligned16(lse_out)) return ADAKV_EINVAL;
  if (row_flag != nullptr && !aligned16(row_flag)) return ADAKV_EINVAL;
  if (g.w > 64 || g.G > 8) return ADAKV_EUNSUPPORTED;
  return hip_status(launch_lse_from_causal(g, q_win, k, lse_causal, lse_out, row_flag,
                                           static_cast<hipStream_t>(stream)));
}

adakv_status adakv_allocate(const adakv_shape* shape, const adakv_alloc* alloc, const float* score,
                            const float* score2, int32_t* budgets, int32_t* sel, int64_t* sel_off, void* ws,
                            size_t ws_bytes, void* stream) {
  Geo g{};
  adakv_status st = check_shape(shape, g);
  if (st != ADAKV_OK) return st;
  st = check_alloc(alloc, g);
  if (st != ADAKV_OK) return st;
  if (!aligned16(budgets) || !aligned16(sel_off) || !aligned16(ws)) return ADAKV_EINVAL;
  if (alloc->mode != ADAKV_ALLOC_STREAMING && !aligned16(score)) return ADAKV_EINVAL;
  if (selected_rows(*alloc, g) > 0 && !aligned16(sel)) return ADAKV_EINVAL;
  if (alloc->mode == ADAKV_ALLOC_ADA_CRITICALKV && !aligned16(score2)) return ADAKV_EINVAL;
  if (alloc->mode == ADAKV_ALLOC_LAVA_LAYERS && g.I > 4096) return ADAKV_EUNSUPPORTED;
  if (alloc->mode == ADAKV_ALLOC_GLOBAL && (int64_t)g.I * g.hkv > ((int64_t)1 << 20)) return ADAKV_EUNSUPPORTED;
  if (ws_bytes < alloc_ws_bytes(g, *alloc)) return ADAKV_EWORKSPACE;
  return hip_status(launch_allocate(g, *alloc, score, score2, budgets, sel, sel_off, static_cast<char*>(ws),
                                    static_cast<hipStream_t>(stream)));
}

adakv_status adakv_lava_online_allocate(const adakv_shape* shape, int64_t total_budget, const float* score,
                                        const int64_t* prev_sel_off, const int32_t* prev_budgets,
                                        const int32_t* prev_sel, double* layer_ent, int32_t* budgets, int32_t* sel,
                                        int64_t* sel_off, void* ws, size_t ws_bytes, void* stream) {
  Geo g{};
  adakv_status st = check_shape(shape, g);
  if (st != ADAKV_OK) return st;
  const int64_t bp = total_budget - (int64_t)g.I * g.w * g.hkv;
  if (bp < 0) return ADAKV_EINVAL;
  if (!aligned16(score) || !aligned16(budgets) || !aligned16(sel_off) || !aligned16(ws)) return ADAKV_EINVAL;
  if (bp > 0 && !aligned16(sel)) return ADAKV_EINVAL;
  if (g.I > 1 && !aligned16(prev_sel_off)) return ADAKV_EINVAL;
  if (layer_ent == nullptr || reinterpret_cast<uintptr_t>(layer_ent) % alignof(double) != 0) return ADAKV_EINVAL;
  if ((prev_budgets == nullptr) != (prev_sel == nullptr)) return ADAKV_EINVAL;
  if (g.I > 1 && prev_sel != nullptr && (!aligned16(prev_budgets) || !aligned16(prev_sel))) return ADAKV_EINVAL;
  if (g.I > 4096) return ADAKV_EUNSUPPORTED;
  if (bp > (int64_t)INT32_MAX) return ADAKV_EUNSUPPORTED;
  adakv_alloc a{};
  a.mode = ADAKV_ALLOC_LAVA_LAYERS;
  a.alpha_den = 1;
  a.ck_den = 1;
  a.budget = total_budget;
  if (ws_bytes < alloc_ws_bytes(g, a)) return ADAKV_EWORKSPACE;
  return hip_status(launch_allocate(g, a, score, nullptr, budgets, sel, sel_off, static_cast<char*>(ws),
                                   static_cast<hipStream_t>(stream), true, g.I > 1 ? prev_sel_off : nullptr,
                                   g.I > 1 ? prev_budgets : nullptr, g.I > 1 ? prev_sel : nullptr, layer_ent));
}

adakv_status adakv_lava_online_compact(const adakv_shape* shape, const void* k_new, const void* v_new,
                                       const void* k_old, const void* v_old, const int64_t* seg_start_old,
                                       const int32_t* sel_old, const int64_t* sel_off_old, const int32_t* budgets,
                                       const int32_t* sel, const int64_t* sel_off, int64_t max_rows, void* k_flat,
                                       void* v_flat, int64_t* seg_start, int32_t* seg_len, void* stream) {
  Geo g{};
  adakv_status st = check_shape(shape, g);
  if (st != ADAKV_OK) return st;
  if (max_rows < 0) return ADAKV_EINVAL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(budgets) || !aligned16(sel_off) ||
      !aligned16(seg_start) || !aligned16(seg_len))
    return ADAKV_EINVAL;
  if (max_rows > 0 && (!aligned16(k_flat) || !aligned16(v_flat) || !aligned16(sel))) return ADAKV_EINVAL;
  if (g.I > 1 && (!aligned16(k_old) || !aligned16(v_old) || !aligned16(seg_start_old) || !aligned16(sel_old) ||
                  !aligned16(sel_off_old)))
    return ADAKV_EINVAL;
  return hip_status(launch_online_compact(g, max_rows, k_new, v_new, k_old, v_old, seg_start_old, sel_old,
                                          sel_off_old, budgets, sel, sel_off, k_flat, v_flat, seg_start, seg_len,
                                          static_cast<hipStream_t>(stream)));
}

adakv_status adakv_compact(const adakv_shape* shape, const adakv_alloc* alloc, const void* k, const void* v,
                           const int32_t* budgets, const int32_t* sel, const int64_t* sel_off, int32_t reserve,
                           void* k_flat, void* v_flat, int64_t* seg_start, int32_t* seg_len, void* stream) {
  Geo g{};
  adakv_status st = check_shape(shape, g);
  if (st != ADAKV_OK) return st;
  st = check_alloc(alloc, g);
  if (st != ADAKV_OK) return st;
  if (reserve < 0) return ADAKV_EINVAL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(budgets) || !aligned16(sel_off) || !aligned16(k_flat) ||
      !aligned16(v_flat) || !aligned16(seg_start) || !aligned16(seg_len))
    return ADAKV_EINVAL;
  const int64_t selected = selected_rows(*alloc, g);
  if (selected > 0 && !aligned16(sel)) return ADAKV_EINVAL;
  const int64_t retained = selected + (int64_t)g.I * g.hkv * g.w;
  return hip_status(launch_compact(g, retained, k, v, budgets, sel, sel_off, reserve, k_flat, v_flat, seg_start,
                                   seg_len, static_cast<hipStream_t>(stream)));
}

namespace {
// Argument checks shared by both decode entry points; fills g and the row count.
adakv_status check_decode(const adakv_shape* shape, const adakv_alloc* alloc, const void* q, const void* k_new,
                          const void* v_new, void* k_flat, void* v_flat, const int64_t* seg_start,
                          const int32_t* seg_len, int32_t reserve, int32_t step, float* out, Geo& g, int64_t& rows) {
  adakv_status st = check_shape(shape, g);
  if (st != ADAKV_OK) return st;
  st = check_alloc(alloc, g);
  if (st != ADAKV_OK) return st;
  if (reserve < 0 || step < 0) return ADAKV_EINVAL;
  if ((k_new == nullptr) != (v_new == nullptr)) return ADAKV_EINVAL;
  if (!aligned16(q) || !aligned16(k_flat) || !aligned16(v_flat) || !aligned16(seg_start) || !aligned16(seg_len) ||
      !aligned16(out))
    return ADAKV_EINVAL;
  if (k_new != nullptr && (!aligned16(k_new) || !aligned16(v_new))) return ADAKV_EINVAL;
  if (g.G > 8) return ADAKV_EUNSUPPORTED;
  const bool append = k_new != nullptr;
  if (append && step >= reserve) return ADAKV_ECAPACITY;
  if (!append && step > reserve) return ADAKV_EINVAL;
  rows = selected_rows(*alloc, g) + (int64_t)g.I * g.hkv * ((int64_t)g.w + step + (append ? 1 : 0));
  return ADAKV_OK;
}
}  // namespace

adakv_status adakv_decode_attn_noalloc(const adakv_shape* shape, const adakv_alloc* alloc, const void* q,
                                       const void* k_new, const void* v_new, void* k_flat, void* v_flat,
                                       const int64_t* seg_start, const int32_t* seg_len, int32_t reserve,
                                       int32_t step, float* out, void* stream) {
  Geo g{};
  int64_t rows = 0;
  adakv_status st = check_decode(shape, alloc, q, k_new, v_new, k_flat, v_flat, seg_start, seg_len, reserve, step,
                                 out, g, rows);
  if (st != ADAKV_OK) return st;
  if (decode_ws_bytes(g, rows) > decode_scratch_capacity()) return ADAKV_EWORKSPACE;
  void* scratch = nullptr;
  if (decode_scratch(&scratch) != hipSuccess) return ADAKV_EHIP;
  const bool append = k_new != nullptr;
  return hip_status(launch_decode(g, rows, step + (append ? 1 : 0), q, k_new, v_new, k_flat, v_flat, seg_start,
                                  seg_len, out, static_cast<char*>(scratch), static_cast<hipStream_t>(stream)));
}

adakv_status adakv_decode_attn(const adakv_shape* shape, const adakv_alloc* alloc, const void* q, const void* k_new,
                               const void* v_new, void* k_flat, void* v_flat, const int64_t* seg_start,
                               const int32_t* seg_len, int32_t reserve, int32_t step, float* out, void* ws,
                               size_t ws_bytes, void* stream) {
  Geo g{};
  int64_t rows = 0;
  adakv_status st = check_decode(shape, alloc, q, k_new, v_new, k_flat, v_flat, seg_start, seg_len, reserve, step,
                                 out, g, rows);
  if (st != ADAKV_OK) return st;
  if (!aligned16(ws)) return ADAKV_EINVAL;
  if (ws_bytes < decode_ws_bytes(g, rows)) return ADAKV_EWORKSPACE;
  const bool append = k_new != nullptr;
  return hip_status(launch_decode(g, rows, step + (append ? 1 : 0), q, k_new, v_new, k_flat, v_flat, seg_start,
                                  seg_len, out, static_cast<char*>(ws), static_cast<hipStream_t>(stream)));
}

}  // extern "C"
