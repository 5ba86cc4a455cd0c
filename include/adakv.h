/*
 * adakv.h -- C ABI of libadakv.so: head-wise adaptive KV-cache eviction on
 * AMD Instinct MI355X (gfx950).
 *
 * The path, per layer instance (one layer of one sequence):
 *   adakv_score        observation-window scores of every prefix token
 *   adakv_score_lse    the same with the window softmax normaliser supplied
 *   adakv_lse_from_causal  that normaliser from the one a causal prefill leaves
 *   adakv_allocate     layer-wide top-B -> per-head budgets -> per-head selection
 *   adakv_compact      selected rows + window rows -> one flat variable-length cache
 *   adakv_decode_attn  decode attention over the flat cache (optional append)
 *   adakv_decode_attn_noalloc  the same without a workspace argument
 *   adakv_lava_online_allocate / adakv_lava_online_compact
 *                      LAVa's layer-by-layer prefill with re-compression
 *
 * Conventions shared by every call
 *   - Every buffer argument is DEVICE memory owned by the caller.  The library
 *     never allocates, frees or keeps pointers after a call returns.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without waiting: the host is never synchronised.
 *   - Arguments are checked on the host before anything is launched.  A bad
 *     argument returns its status code and launches nothing.  ADAKV_EHIP means
 *     the HIP runtime reported an error when a kernel was launched.
 *   - Every pointer must be 16-byte aligned.  Arrays are dense, row-major, in
 *     the shapes given below, with I = shape.n_inst, p = n - w, G = hq / hkv.
 *   - Results are deterministic: the same inputs give bit-identical outputs.
 *   - Calls are stateless and may run concurrently on different streams with
 *     different workspaces.
 *
 * Sources (page title, then section / equation / algorithm):
 *   [AdaKV-notes]  "Ada-KV: Optimizing KV Cache Eviction by Adaptive Budget
 *                  Allocation for Efficient LLM Inference" (papercache.org notes)
 *   [AdaKV-paper]  the same paper, arXiv 2407.11550 HTML, Sections 3-4
 *   [LAVa-notes]   "LAVa: Layer-wise KV Cache Eviction with Dynamic Budget
 *                  Allocation" (papercache.org notes)
 *   [CKV-notes]    "CriticalKV: Optimizing KV Cache Eviction from an Output
 *                  Perturbation Perspective" (papernotes.org)
 *   [LaProx]       "重构长上下文 LLM 推理中的 KV 缓存淘汰问题" (a translation of
 *                  arXiv 2605.07234, the LaProx paper)
 */
#ifndef ADAKV_H
#define ADAKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ADAKV_OK = 0,
  ADAKV_EINVAL = 1,        /* a NULL pointer, a bad size or a bad combination   */
  ADAKV_EUNSUPPORTED = 2,  /* valid but not built: head dim, dtype, window, ... */
  ADAKV_ECAPACITY = 3,     /* an append would pass the reserved rows            */
  ADAKV_EWORKSPACE = 4,    /* ws_bytes smaller than adakv_workspace_bytes()     */
  ADAKV_EHIP = 5           /* the HIP runtime reported an error on launch       */
} adakv_status;

typedef enum { ADAKV_BF16 = 0, ADAKV_F32 = 1 } adakv_dtype;

typedef enum {
  ADAKV_SCORE_SNAPKV = 0,      /* Ada-KV / SnapKV window attention            */
  ADAKV_SCORE_LAVA = 1,        /* LAVa score (attention x value-norm maximum) */
  ADAKV_SCORE_CRITICALKV = 2,  /* Ada-KV score + CriticalKV composite         */
  ADAKV_SCORE_LAPROX = 3       /* LaProx: ||A[:,t]||_2 x ||(V W_O)[t,:]||_2    */
} adakv_scorer;

typedef enum {
  ADAKV_ALLOC_ADA = 0,          /* Ada-KV budgets with safeguard, per-head top-k   */
  ADAKV_ALLOC_LAVA_LAYERS = 1,  /* LAVa entropy layer budgets, flattened top-k    */
  ADAKV_ALLOC_ADA_CRITICALKV = 2,/* Ada-KV budgets, CriticalKV two-stage selection */
  ADAKV_ALLOC_GLOBAL = 3,       /* one top-k over every head of every instance    */
  ADAKV_ALLOC_ADA_FLOOR = 4,    /* safeguard read as a per-head floor, then top-k */
  ADAKV_ALLOC_STREAMING = 5     /* StreamingLLM: sinks + most recent, no scores    */
} adakv_alloc_mode;

/* Geometry of one call.  Enumerations are carried as int32_t fields. */
typedef struct {
  int32_t n_inst;  /* I: independent instances (layer x sequence)            */
  int32_t hq;      /* query heads                                             */
  int32_t hkv;     /* KV heads; hq % hkv == 0                                 */
  int32_t d;       /* head dimension                                          */
  int32_t n;       /* cached tokens per head, window included                 */
  int32_t w;       /* observation window: the last w tokens of every head     */
  int32_t pool;    /* max-pool kernel, odd, 1 = off                           */
  int32_t dtype;   /* adakv_dtype of q, k, v, w_o and the flat cache           */
  int32_t scorer;  /* adakv_scorer                                            */
  int32_t hidden;  /* CriticalKV, LaProx: model hidden size D (rows of w_o)     */
  float eps;       /* CriticalKV: additive epsilon of the composite            */
  int32_t reserved0;
} adakv_shape;

/* Budget allocation settings. */
typedef struct {
  int32_t mode;       /* adakv_alloc_mode                                          */
  int32_t alpha_num;  /* Ada-KV safeguard alpha = alpha_num / alpha_den (0..1)     */
  int32_t alpha_den;
  int32_t ck_num;     /* CriticalKV stage-1 share = ck_num / ck_den (0..1)        */
  int32_t ck_den;
  int32_t sinks;      /* STREAMING: leading prefix tokens every head keeps (>= 0) */
  int64_t budget;     /* ADA / CRITICALKV / ADA_FLOOR / STREAMING: budget B of
                         every instance, window included (w*hkv <= B <= n*hkv).
                         LAVA_LAYERS: total budget over all I instances (the
                         layers of one sequence), windows included; the part
                         B' = budget - I*w*hkv must satisfy 0 <= B' <= hkv*p.
                         GLOBAL: total budget over all I instances, windows
                         included; 0 <= B' = budget - I*w*hkv <= I*hkv*p.   */
  const int64_t* inst_budget; /* ADA only; NULL or HOST memory: I per-instance
                         budgets B_i (window included, w*hkv <= B_i <= n*hkv)
                         used instead of `budget` for instance i, e.g. preset
                         layer budgets (Pyramid: SnapKV with a per-layer budget
                         and alpha = 0; Ada-Pyramid: the same with Ada-KV's
                         allocation, [AdaKV-paper] Section 4 "Baselines",
                         [AdaKV-notes] "集成到现有的缓存驱逐方法中").  Read during
                         the call; the same array must be passed to
                         adakv_compact and adakv_decode_attn.  Other modes
                         return ADAKV_EUNSUPPORTED when it is set.            */
} adakv_alloc;

/* Bytes of workspace every call below needs for this geometry (the maximum
 * over the calls).  `reserve` is the number of empty rows kept per head in the
 * flat cache (see adakv_compact).  Returns 0 for an invalid description. */
size_t adakv_workspace_bytes(const adakv_shape* shape, const adakv_alloc* alloc, int32_t reserve);

/* Observation-window scoring of every prefix token (the first p tokens).
 *
 *   SNAPKV      [AdaKV-notes] Algorithm 2 ("Ada-KV Integration"), steps 2-4:
 *               for query head i and window row r the logits
 *               q_win[i,r] . k[g,t] / sqrt(d) over the prefix t < p are
 *               softmaxed, every row is max pooled (stride 1, window cut at the
 *               ends), and the rows are averaged; GQA groups take the mean
 *               over their query heads ([AdaKV-paper] "Compatibility with Group
 *               Query Attention").  score[i,g,t] = that group mean.
 *   LAVA        [LAVa-notes] Definition 1 and "适配GQA架构": window row r attends
 *               causally to keys 0..p+r; the rows' weights are summed, the group
 *               takes the maximum over its heads, the result is scaled by
 *               max_t ||v[g,t]||_1 / w and max pooled over all n tokens; score
 *               holds the prefix part.
 *   CRITICALKV  score = the SNAPKV score (for the budgets); score2 = the
 *               composite of [CKV-notes] "两阶段贪心选择算法", under GQA the mean
 *               over the group's query heads of (A_i[t] + eps) * ||(v W^O_i)[t]||_1.
 *   LAPROX      [LaProx] Section 4.1, Algorithm 1: A_i = softmax of
 *               q_win[i] . k[g]^T / sqrt(d) with every window row over all n
 *               keys (no mask, as printed); score[i,g,t] = the mean over the
 *               group's query heads of ||A_i[:, t]||_2 * ||(v W^O_i)[t, :]||_2
 *               (window tokens score infinity there and are always kept, so
 *               only the prefix is scored).  No pooling: shape.pool must be 1.
 *               w_o is shared by every instance of the call: instances with
 *               different projections (layers) are scored in separate calls.
 *
 *   q_win  [I, hq, w, d]   dtype         the window queries
 *   k      [I, hkv, n, d]  dtype
 *   v      [I, hkv, n, d]  dtype         LAVA, CRITICALKV and LAPROX, else NULL
 *   w_o    [hidden, hq*d]  dtype         CRITICALKV and LAPROX, else NULL: the output
 *                                        projection in the nn.Linear layout
 *                                        (row c holds output feature c, so
 *                                        W^O_i of the pages is columns i*d..i*d+d-1
 *                                        transposed)
 *   score  [I, hkv, p]     float32 out
 *   score2 [I, hkv, p]     float32 out   CRITICALKV only, else NULL
 *   ws     >= adakv_workspace_bytes() bytes of device scratch
 *
 * Supported: bf16 with d in {64, 128}; f32 with d in {16, 64}; w <= 64;
 * pool in {1, 3, 5, 7}; G <= 8; CRITICALKV and LAPROX need bf16, d = 128 and
 * hidden a multiple of 64.  Other valid shapes return ADAKV_EUNSUPPORTED. */
adakv_status adakv_score(const adakv_shape* shape, const void* q_win, const void* k, const void* v,
                         const void* w_o, float* score, float* score2, void* ws, size_t ws_bytes,
                         void* stream);

/* Observation-window scoring with the window softmax normaliser supplied.
 *
 * The same scores as adakv_score, but the log-sum-exp of every window row's
 * logits over the row's key domain comes from the caller instead of a first
 * pass over the keys, so K is read once.  An attention pass over the window
 * rows (the prefill, which computes them anyway: [LAVa-notes] "时间复杂度与
 * 内存使用分析" counts the recent-attention recomputation separately from the
 * cache computation) leaves exactly this statistic behind.
 *
 *   row_lse [I, hq, w] float32   natural-log log-sum-exp of q_win[j,r].k[g,t]/sqrt(d)
 *                                over row r's domain: the prefix t < p for
 *                                SNAPKV and CRITICALKV (the domain adakv_score
 *                                normalises over), t <= p + r for LAVA, all
 *                                n keys for LAPROX.  Finite.
 * Every other argument, the outputs and the supported shapes are those of
 * adakv_score; ws may be the same size. */
adakv_status adakv_score_lse(const adakv_shape* shape, const void* q_win, const void* k, const void* v,
                             const void* w_o, const float* row_lse, float* score, float* score2, void* ws,
                             size_t ws_bytes, void* stream);

/* The window softmax normaliser of adakv_score_lse from a causal prefill's.
 *
 * An attention pass over the prompt with the causal mask leaves, for window
 * row r (position p + r) of query head j, L = the natural-log log-sum-exp of
 * z_t = q_win[i,j,r].k[i,g,t]/sqrt(d) over keys t = 0 .. p + r (g = j / G).
 * That is the LAVA domain ([LAVa-notes] Definition 1).  The other scorers'
 * domains differ from it by window keys only, so the call reads the w window
 * rows of K and rewrites L in float64:
 *   SNAPKV, CRITICALKV  prefix t < p ([AdaKV-notes] Algorithm 2, step 2):
 *                       out = L + ln(1 - sum_{t=p}^{p+r} exp(z_t - L))
 *   LAPROX              all n keys ([LaProx] Section 4.1, Algorithm 1):
 *                       out = L + ln(1 + sum_{t=p+r+1}^{n-1} exp(z_t - L))
 *   LAVA                out = L
 * out is what adakv_score_lse takes as row_lse.
 *
 *   q_win      [I, hq, w, d]  dtype
 *   k          [I, hkv, n, d] dtype    only rows p .. n-1 of each head are read
 *   lse_causal [I, hq, w] float32      L, finite
 *   lse_out    [I, hq, w] float32 out  may be lse_causal itself (in place)
 *   row_flag   [I, hq, w] int32 out, or NULL:
 *                0  the row is well conditioned;
 *                1  prefix domain, and the prefix holds less than 2^-7 of the
 *                   causal mass (1 - sum < 2^-7).  The subtraction multiplies
 *                   the absolute error of L by 1 / (1 - sum), so more than 7
 *                   bits of L's precision are lost; where rounding in L leaves
 *                   no positive share at all, out = L - 60 ln 2.  Score such
 *                   rows with adakv_score (two passes) instead;
 *                2  L, or the result, is not finite (out = L).
 * Supported shapes: those of adakv_score (pool, hidden and eps are not read).
 * No workspace; nothing is allocated. */
adakv_status adakv_lse_from_causal(const adakv_shape* shape, const void* q_win, const void* k,
                                   const float* lse_causal, float* lse_out, int32_t* row_flag, void* stream);

/* Budget allocation and selection.  Scores must be finite and >= 0 (-0.0 is
 * treated as +0.0).  Ranking: a larger score first; equal scores by the smaller
 * flat index g*p + t.
 *
 *   ADA         [AdaKV-notes] Algorithm 1 inside Algorithm 2: P = B - w*hkv
 *               (B = inst_budget[i] for instance i when given);
 *               the top P of all hkv*p scores give counts f_g; the safeguard
 *               (Algorithm 2, step 8) alpha*f_g + (1-alpha)*P/hkv is made
 *               integer exactly (floors, then one extra unit to the largest
 *               remainders, lower head first on equal remainders) so the
 *               budgets sum to P; then each head keeps its top B_g.  alpha
 *               weighs the adaptive counts as the formula is printed; the
 *               reading in which alpha weighs the uniform share instead
 *               ("smaller alpha, more aggressive allocation" in the notes'
 *               robustness analysis) is alpha_num/alpha_den = 1 - alpha.
 *   LAVA_LAYERS [LAVa-notes] "基于不确定性的层预算分配": instance l is layer l;
 *               e_l = entropy of the layer's normalised scores / (hkv*p);
 *               B' = budget - I*w*hkv is split in proportion to e_l (largest
 *               remainder, lower layer first); "动态头预算的逐层缓存驱逐": each
 *               layer keeps its top B'_l of the flattened scores (no safeguard).
 *   ADA_CRITICALKV  budgets as ADA on `score`; per head stage 1 keeps the top
 *               floor(B_g*ck_num/ck_den) by `score`, stage 2 the top rest by
 *               `score2` among the others ([CKV-notes] "两阶段贪心选择算法").
 *   ADA_FLOOR   the safeguard read as a floor ([AdaKV-notes] Algorithm 2 step 8
 *               keeps sparse heads from too small a budget): every head first
 *               keeps its own top f0 = floor(alpha_num*P / (alpha_den*hkv)),
 *               then the top P - hkv*f0 of all heads' remaining entries
 *               (Algorithm 1 on the rest); B_g = f0 + head g's share.  Of all
 *               splits with B_g >= f0 it keeps the largest total score.
 *   STREAMING   StreamingLLM ([AdaKV-paper] "Baselines" / "Parameters": 4 sink
 *               tokens and the most recent window): B_g = P/hkv (one more for
 *               the lowest P mod hkv heads); head g keeps prefix tokens
 *               0 .. min(sinks, B_g)-1 and its most recent remaining ones.
 *               score may be NULL.
 *   GLOBAL      [LaProx] Algorithm 1, TopK(p, B_total) with the window tokens
 *               at infinity, and the abstract's model-wide selection: the top
 *               B' = budget - I*w*hkv of all I*hkv*p scores, ranked by (-score,
 *               flat index (i*hkv + g)*p + t); B_g is head g's share.  Pass
 *               the layers of a sequence as the instances (n_inst = 1 gives a
 *               per-layer top-k).  Needs I*hkv*p < 2^31 and I*hkv <= 2^20.
 *
 *   score   [I, hkv, p] float32         score2 [I, hkv, p] float32 (CK only, else NULL)
 *   budgets [I, hkv]    int32 out       prefix budget B_g of every head
 *   sel     int32 out, sum of all budgets entries: instance i starts at
 *           sel_off[i]; inside it head g's selected token indices (in [0,p))
 *           follow head g-1's, each head ascending.  Its length is
 *           I*(budget - w*hkv) for ADA / CK (the sum over instances of
 *           inst_budget[i] - w*hkv when given) and budget - I*w*hkv for LAVA
 *           and GLOBAL.
 *   sel_off [I+1] int64 out
 *
 * Precondition check: the int32 at the start of ws is cleared by the call and
 * set to a nonzero value when a score it reads (score; score2 for CK) is
 * negative (other than -0.0), NaN or infinite.  Such a selection is
 * unspecified but stays inside its buffers.  Read the word after the stream
 * has passed the call; the next call on the same ws overwrites it.  STREAMING
 * reads no score and leaves it zero.
 */
adakv_status adakv_allocate(const adakv_shape* shape, const adakv_alloc* alloc, const float* score,
                            const float* score2, int32_t* budgets, int32_t* sel, int64_t* sel_off,
                            void* ws, size_t ws_bytes, void* stream);

/* Compaction into the flat cache ([AdaKV-notes] Algorithm 2 steps 10-11 and
 * [AdaKV-paper] "Variable-length Attention with Variable-sized Cache
 * Elements": all heads' retained caches concatenated into one tensor).
 * Segment s = i*hkv + g holds the selected prefix rows of (i, g) in ascending
 * token order, then its w window rows, then `reserve` rows left untouched for
 * decode appends.  The copy is bit-exact.
 *
 *   k, v        [I, hkv, n, d] dtype         as given to adakv_score
 *   budgets, sel, sel_off                    as written by adakv_allocate
 *   k_flat, v_flat [rows, d] dtype out       rows = (sum of budgets) + I*hkv*(w + reserve)
 *   seg_start   [I*hkv + 1] int64 out        first row of every segment
 *   seg_len     [I*hkv]     int32 out        B_g + w (rows written here)
 */
adakv_status adakv_compact(const adakv_shape* shape, const adakv_alloc* alloc, const void* k, const void* v,
                           const int32_t* budgets, const int32_t* sel, const int64_t* sel_off,
                           int32_t reserve, void* k_flat, void* v_flat, int64_t* seg_start,
                           int32_t* seg_len, void* stream);

/* LAVa online prefill ([LAVa-notes] "在线预填充与层预算调整"): prefill and
 * eviction run layer by layer, and after layer l is prefilled the lower layers
 * are compressed again with their same scores under budgets that shrink as
 * more layers share the memory.  The pages leave the schedule open; here,
 * after layer l the I = l + 1 layers present share B'(l) = total_budget -
 * I*w*hkv prefix entries by the LAVA_LAYERS entropy rule (same e_j, same
 * largest-remainder split), each layer's budget capped by its budget of the
 * previous step (and by hkv*p), so budgets never grow and every selection lies
 * inside the previous one.  Each layer keeps the top B_j of its flattened
 * scores (no safeguard).  The budgets may sum to less than B'(l) where a cap
 * binds: sel_off[I] holds the count.
 *
 * A layer's entropy e_j depends on its own scores only, so each is computed
 * once, at the step that adds the layer, and kept by the caller in layer_ent.
 * Because budgets never grow, the new top-B_j of an older layer is the first
 * B_j of its previous kept entries (same order, same scores): given the
 * previous step's budgets and sel, each older layer is re-selected from those
 * entries and only the newest layer's full scores are read (taken when the
 * previous step's older layers kept at most 32768 entries in all, at most 8192
 * each on average, and hkv <= 256; otherwise every layer is re-selected from
 * its full scores).  Both routes give the same outputs.
 *
 *   shape.n_inst  I = layers prefilled so far; scorer/pool as for the scores
 *   score         [I, hkv, p] float32, the LAVa scores of layers 0..I-1 (each
 *                 layer's own, as adakv_score wrote them when it was prefilled)
 *   prev_sel_off  [I] int64: sel_off of the previous step (layers 0..I-2);
 *                 NULL when I == 1.  Must not overlap sel_off.
 *   prev_budgets, prev_sel   the previous step's budgets and sel, both or
 *                 neither (NULL: every layer from its full scores; ignored
 *                 when I == 1).  Must not overlap budgets or sel.
 *   layer_ent     [I] float64, 8-byte aligned, in/out: entries 0..I-2 as the
 *                 earlier steps wrote them (read), entry I-1 written.  The
 *                 caller keeps it from step to step.
 *   budgets [I, hkv] int32 out, sel int32 out (capacity total_budget - I*w*hkv,
 *   layout as adakv_allocate), sel_off [I+1] int64 out.
 *   ws            >= adakv_workspace_bytes(shape, LAVA_LAYERS alloc, 0) bytes;
 *                 its first int32 reports broken score preconditions as for
 *                 adakv_allocate, for the scores this call reads in full (the
 *                 newest layer's alone on the incremental route).
 * Needs I <= 4096. */
adakv_status adakv_lava_online_allocate(const adakv_shape* shape, int64_t total_budget, const float* score,
                                        const int64_t* prev_sel_off, const int32_t* prev_budgets,
                                        const int32_t* prev_sel, double* layer_ent, int32_t* budgets,
                                        int32_t* sel, int64_t* sel_off, void* ws, size_t ws_bytes, void* stream);

/* The flat cache of layers 0..I-1 after an adakv_lava_online_allocate step:
 * the newest layer's rows (instance I-1) are gathered from its dense cache,
 * the lower layers' rows from the previous step's flat cache, where every kept
 * token still is (selections only shrink).  Layout as adakv_compact with no
 * reserve rows: segment s = i*hkv + g holds B_g selected rows then w window
 * rows.  The copy is bit-exact.
 *
 *   k_new, v_new     [hkv, n, d] dtype: the dense cache of layer I-1
 *   k_old, v_old     previous flat cache (layers 0..I-2), at least max_rows
 *                    rows like k_flat (rows at or past max_rows are not read),
 *                    seg_start_old [(I-1)*hkv+1], sel_old and sel_off_old [I]
 *                    of the previous step; all NULL when I == 1.  Reads of
 *                    sel and sel_old stay inside each layer's span of its
 *                    offsets even where budgets disagree with them (rows left
 *                    unwritten then).
 *   budgets, sel, sel_off   this step's adakv_lava_online_allocate outputs
 *   max_rows         rows of k_flat / v_flat; rows past it are not written
 *                    (B'(l) + I*hkv*w always suffices)
 *   k_flat, v_flat   [max_rows, d] out, must not overlap k_old / v_old
 *   seg_start [I*hkv+1] int64 out, seg_len [I*hkv] int32 out (B_g + w) */
adakv_status adakv_lava_online_compact(const adakv_shape* shape, const void* k_new, const void* v_new,
                                       const void* k_old, const void* v_old, const int64_t* seg_start_old,
                                       const int32_t* sel_old, const int64_t* sel_off_old, const int32_t* budgets,
                                       const int32_t* sel, const int64_t* sel_off, int64_t max_rows, void* k_flat,
                                       void* v_flat, int64_t* seg_start, int32_t* seg_len, void* stream);

/* Decode attention over the flat cache.  Segment s holds seg_len[s] rows from
 * adakv_compact plus the `step` rows appended by earlier decode calls.  If
 * k_new and v_new are given, this call appends one more row to every segment
 * (stored at seg_start[s] + seg_len[s] + step) before attending ([AdaKV-notes]
 * the cache update before the output formula).  Then
 *   out[i, j] = softmax(q[i,j] . K_s / sqrt(d)) V_s
 * over the rows of segment s = i*hkv + j/G.  seg_len is read only: a call
 * carries no state besides the appended rows, so the caller counts `step`.
 *
 *   q          [I, hq, d]    dtype
 *   k_new, v_new [I, hkv, d] dtype, both or neither (NULL = no append)
 *   k_flat, v_flat, seg_start, seg_len       from adakv_compact
 *   reserve    the reserve given to adakv_compact.  The library keeps no
 *              state, so it cannot check this against the call that built the
 *              cache: with a larger value an append that passes a segment's
 *              reserved rows (its end is seg_start[s + 1]) is dropped on the
 *              device: the row is neither stored nor attended, nothing past
 *              the segment is read or written, and the call still returns
 *              ADAKV_OK (out is then the attention over the rows already in
 *              the segment, as if k_new / v_new were NULL).
 *   step       rows appended since adakv_compact (0 for the first decode);
 *              an append with step >= reserve returns ADAKV_ECAPACITY, and
 *              step > reserve returns ADAKV_EINVAL
 *   out        [I, hq, d] float32 out
 * Needs G <= 8. */
adakv_status adakv_decode_attn(const adakv_shape* shape, const adakv_alloc* alloc, const void* q,
                               const void* k_new, const void* v_new, void* k_flat, void* v_flat,
                               const int64_t* seg_start, const int32_t* seg_len, int32_t reserve, int32_t step,
                               float* out, void* ws, size_t ws_bytes, void* stream);

/* adakv_decode_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and checks as
 * adakv_decode_attn; the split partials that adakv_decode_attn keeps in `ws`
 * live instead in a fixed device array inside the library, one copy per GPU
 * (8 MiB, held until the process ends; its address is looked up on the first
 * call on each device).  Nothing is allocated or freed by this call.
 *   - A shape whose partials would not fit returns ADAKV_EWORKSPACE (with the
 *     current split rule every supported shape fits: at most about 6.4 MB).
 *   - Every call on a GPU shares that GPU's array: calls that may overlap on
 *     one device (two streams, two host threads) race and must be ordered by
 *     the caller.  Each call writes every partial it reads, so nothing needs
 *     clearing between calls.
 *   - Errors: as adakv_decode_attn; ADAKV_EHIP also when the array's address
 *     cannot be obtained on the current device. */
adakv_status adakv_decode_attn_noalloc(const adakv_shape* shape, const adakv_alloc* alloc, const void* q,
                                       const void* k_new, const void* v_new, void* k_flat, void* v_flat,
                                       const int64_t* seg_start, const int32_t* seg_len, int32_t reserve,
                                       int32_t step, float* out, void* stream);

/* A short, static description of a status code. */
const char* adakv_strerror(adakv_status status);

/* Library version, major*10000 + minor*100 + patch. */
int32_t adakv_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ADAKV_H */
