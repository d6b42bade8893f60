/*
 * confkv.h — C ABI of the MI355X (gfx950) decode-step library for
 * confidence-gated KV-cache eviction (CONF-KV) and its KVpop fixed-budget
 * variant.
 *
 * One call, confkv_step, runs one decode step for every layer and batch row:
 *   1. a vocab-wide reduction of the logits gives the confidence
 *        c = w_e (1 - H / log V) + w_m sigmoid(z(1) - z(2)) + w_p p_max
 *      and c against tau picks the step's base budget per batch row
 *      ("Conf-KV" post on rcap.io, method paragraph and decoding-loop
 *      pseudocode; CONF-KV abstract on chatpaper.ai);
 *   2. decode attention of each query head over its KV head's retained rows,
 *      the recent window in FP16 and older rows INT8, dequantized in the
 *      kernel (CONF-KV abstract: blockwise softmax attention with mixed
 *      FP16/INT8 storage; Conf-KV post: the fused INT8 dequantization);
 *   3. the EMA of each row's attention mass and the score
 *        alpha * ema + (1 - alpha) * recency            (Conf-KV post);
 *   4. per KV head, eviction of the lowest-scoring rows down to the budget,
 *      sink and protected-window rows exempt          (Conf-KV post);
 *   5. in-place compaction of the survivors and INT8 storage of the row that
 *      leaves the FP16 window                          (Conf-KV post).
 * With policy KVPOP, steps 1 and 3 are replaced by the fixed budget
 * B = s + w + k over static per-token priorities ("Resumen Técnico: KVpop",
 * gist.science, §2.1 and §2.4), the priority of a row arriving when it leaves
 * the protected window (§2.3, delayed scoring).
 *
 * Conventions
 * -----------
 * - Every tensor pointer is a caller-owned DEVICE pointer, row-major, with the
 *   shape in brackets. fp16 values are passed as their uint16_t bit patterns.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream). Calls
 *   only enqueue work on it, except where a function says it synchronizes.
 * - Segment index: seg = (l * batch + b) * num_kv_heads + h. Query heads
 *   h*G .. h*G+G-1 (G = num_q_heads / num_kv_heads) share KV head h.
 * - Ownership: the caller allocates the device state buffer (size from
 *   confkv_state_bytes) and all inputs/outputs, and keeps inputs alive until
 *   the stream has passed the call. The library allocates only a host-side
 *   handle (and HIP events while profiling is on); it never allocates device
 *   memory.
 * - Errors: argument and shape checks run on the host before anything is
 *   enqueued and return CONFKV_EINVAL / CONFKV_ECAPACITY with the state
 *   unchanged. Faults found by the kernels (non-finite logits or scores, a
 *   segment outgrowing its capacity) set a sticky device error word that
 *   confkv_status (and every synchronizing call) reports. After any error
 *   the handle accepts only confkv_status, confkv_destroy, confkv_strerror.
 *   Nothing throws across this ABI. A handle is not thread-safe.
 */
#ifndef CONFKV_H
#define CONFKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CONFKV_ABI_VERSION 2

enum {
  CONFKV_OK = 0,
  CONFKV_EINVAL = -1,      /* bad argument, shape or config value            */
  CONFKV_ECAPACITY = -2,   /* capacity or state buffer too small             */
  CONFKV_EHIP = -3,        /* a HIP runtime call failed                      */
  CONFKV_ENONFINITE = -4,  /* NaN/Inf in logits or in a ranking score        */
  CONFKV_ESTATE = -5       /* handle destroyed or poisoned by an earlier error */
};

enum { CONFKV_POLICY_CONF = 0, CONFKV_POLICY_KVPOP = 1 };

/* How CONF ranks the rows inside the budget. The "Conf-KV" post's
 * matched-rate ablation keeps the confidence-gated schedule and swaps the
 * ranker: recency only (SCORE with alpha 0), attention only (SCORE with
 * alpha 1), or random victims (RANDOM). A fixed-budget sliding window is
 * SCORE with alpha 0 and n_low == n_high. */
enum { CONFKV_RANKER_SCORE = 0, CONFKV_RANKER_RANDOM = 1 };

typedef struct confkv_handle confkv_handle;

typedef struct confkv_config {
  int32_t abi_version;     /* CONFKV_ABI_VERSION                                   */
  int32_t num_layers;      /* L >= 1                                               */
  int32_t batch;           /* B >= 1                                               */
  int32_t num_q_heads;     /* Hq, a multiple of num_kv_heads; G in {1,2,4,5,8}     */
  int32_t num_kv_heads;    /* Hkv >= 1                                             */
  int32_t head_dim;        /* d in {64, 128}                                       */
  int32_t vocab;           /* V >= 2 (CONF); ignored for KVPOP                     */
  int32_t capacity;        /* rows older than the FP16 window that one segment can
                              hold; >= max(prefill_len, largest budget + 1,
                              num_sink + protect_last + 1). It counts the old
                              (INT8, or FP16 under KVPOP) region only: the W + 1
                              window slots are a fixed ring beside it, so the
                              rows a segment can hold are capacity + W + 1     */
  int32_t policy;          /* CONFKV_POLICY_CONF | CONFKV_POLICY_KVPOP             */
  int32_t n_low, n_high;   /* the two base budgets (rows per segment)              */
  int32_t protect_last;    /* P: the last P positions are never evicted (KVPOP: w) */
  int32_t fp16_window;     /* W: rows with pos > t - W stay FP16 (KVPOP: = w)      */
  int32_t num_sink;        /* s: positions < s are never evicted                   */
  float tau;               /* confidence threshold                                 */
  float alpha;             /* score = alpha * ema + (1 - alpha) * recency          */
  float ema_beta;          /* ema <- beta * ema + (1 - beta) * mass                */
  float w_entropy, w_margin, w_pmax;  /* 0.4, 0.3, 0.3                             */
  int32_t gate_literal;    /* 0: c >= tau -> min(n_low, n_high) (the pages' prose);
                              1: c >= tau -> n_high (the pseudocode as printed)   */
  int32_t pyramid;         /* 1: layer l gets floor(base*(3(L-1)-2l)/(2(L-1)))     */
  int32_t kvpop_k;         /* k of B = s + w + k (KVPOP)                           */
  int32_t old_int8;        /* 1: rows leaving the FP16 window are stored INT8
                              (per-token, per-head fp32 absmax scale, K and V
                              separately); 0: they stay FP16                      */
  float softmax_scale;     /* 0 -> 1/sqrt(d)                                       */
  int32_t record_scores;   /* 1: keep the last step's per-row positions, ranking
                              values and LSEs for confkv_read_last_step            */
  int32_t ranker;          /* CONFKV_RANKER_SCORE: alpha * ema + (1 - alpha) *
                              recency. CONFKV_RANKER_RANDOM (CONF only): every
                              row gets a fresh uniform rank each step, the top
                              24 bits of x = out(out(out(seed, t+1), seg+1),
                              pos+1) times 2^-24, where out(k, n) is the n-th
                              output of SplitMix64 (Steele, Lea and Flood 2014)
                              started from state k; the EMA is still kept     */
  uint32_t seed;           /* seed of CONFKV_RANKER_RANDOM                        */
} confkv_config;

/* Host-only check of a configuration with a given prefill length. Returns
 * CONFKV_OK, CONFKV_EINVAL or CONFKV_ECAPACITY. Touches no GPU. */
int confkv_validate(const confkv_config* cfg, int32_t prefill_len);

/* Bytes of device state the configuration needs, or 0 if it is invalid.
 * Host-only; touches no GPU. */
size_t confkv_state_bytes(const confkv_config* cfg);

/* Rows per segment in the buffers of confkv_read_cache/confkv_read_last_step:
 * capacity + fp16 window slots. Host-only. 0 if cfg is invalid. */
int32_t confkv_rows_max(const confkv_config* cfg);

/* Carve `state` (>= confkv_state_bytes, 256-byte aligned) and ingest an
 * optional prefill: prefill_k / prefill_v [L][B][Hkv][prefill_len][d] fp16 (both
 * NULL iff prefill_len == 0; KVPOP takes no prefill). Prefill rows get
 * positions 0..prefill_len-1 and EMA 0; those with pos <= prefill_len-1-W are
 * stored INT8 (if old_int8); nothing is attended or evicted here. The next
 * confkv_step decodes position prefill_len. Enqueues on `stream`; on success
 * *out receives a new handle. */
int confkv_init(const confkv_config* cfg, void* state, size_t state_bytes, void* stream,
                const uint16_t* prefill_k, const uint16_t* prefill_v, int32_t prefill_len,
                confkv_handle** out);

/* One decode step at position t (prefill_len + number of earlier steps):
 *   logits    [B][V]        fp32   CONF: required; KVPOP: must be NULL
 *   q         [L][B][Hq][d] fp16   this step's queries
 *   k_new     [L][B][Hkv][d] fp16  this step's key row (appended, pos = t)
 *   v_new     [L][B][Hkv][d] fp16  this step's value row
 *   prio_new  [L][B][Hkv]   fp32   KVPOP: priority of the row at position t-w,
 *                                  which leaves the protected window now
 *                                  (ignored where t-w < s); CONF: NULL
 *   out       [L][B][Hq][d] fp16   attention output (written)
 *   conf_out  [B] fp32, budget_out [B] int32: optional (NULL) copies of the
 *             confidence and the base budget of each batch row (CONF only;
 *             the per-layer budget applies the pyramid to the base).
 * Only enqueues work; no host synchronization. */
int confkv_step(confkv_handle* h, void* stream, const float* logits, const uint16_t* q,
                const uint16_t* k_new, const uint16_t* v_new, const float* prio_new, uint16_t* out,
                float* conf_out, int32_t* budget_out);

/* The same step split at the layer boundary, for a model whose layer l+1
 * takes its queries from layer l's output. In the pages' decoding loop the
 * model first runs every layer on the new token, extending each layer's
 * cache and producing the logits; then each layer updates its EMA and evicts
 * down to the budget that the logits' confidence picks ("Conf-KV" post,
 * decoding-loop pseudocode). So:
 *
 * confkv_attend(layer) appends the new row to that layer's segments, attends
 * over them and updates their EMA (steps 2 and 3 of confkv_step, one layer):
 *   q         [B][Hq][d]  fp16   the layer's queries at position t
 *   k_new     [B][Hkv][d] fp16   the layer's new key row (pos = t)
 *   v_new     [B][Hkv][d] fp16
 *   prio_new  [B][Hkv]    fp32   KVPOP: as in confkv_step; CONF: NULL
 *   out       [B][Hq][d]  fp16   attention output (written)
 * Each layer attends once per step, in any order. EINVAL (nothing enqueued)
 * for a layer out of range or already attended at this position.
 *
 * confkv_evict, after every layer has attended at position t, runs the
 * confidence reduction (CONF), ranks, selects, compacts and ages out for
 * every segment (steps 1, 4 and 5), then moves to position t + 1. logits,
 * conf_out and budget_out are those of confkv_step. EINVAL (nothing enqueued)
 * while a layer has not attended at t.
 *
 * With one workgroup per segment (confkv_set_attend_splits(h, 1)),
 * confkv_attend for every layer followed by confkv_evict leaves the state,
 * outputs, confidences and budgets bit-identical to one confkv_step on the
 * same inputs. confkv_step returns EINVAL between the first confkv_attend of
 * a position and its confkv_evict. Both only enqueue work. */
int confkv_attend(confkv_handle* h, void* stream, int32_t layer, const uint16_t* q, const uint16_t* k_new,
                  const uint16_t* v_new, const float* prio_new, uint16_t* out);
int confkv_evict(confkv_handle* h, void* stream, const float* logits, float* conf_out, int32_t* budget_out);

/* One layer holds only B * Hkv segments, too few workgroups to fill the GPU
 * when each takes a whole segment. confkv_attend therefore splits each
 * segment's rows over several workgroups (split-K) and combines their
 * partial softmax statistics and outputs by the log-sum-exp rule (CONF-KV
 * abstract: blockwise online-softmax attention); the EMA is then updated
 * from the combined normaliser. The split result equals the whole-segment
 * one up to float rounding (not bit for bit).
 * confkv_set_attend_splits: 0 (default) chooses the split count per call,
 * 1 takes one workgroup per segment (bit-identical to confkv_step), 2..32
 * asks for that many (raised where one split's rows would not fit on chip;
 * one workgroup per segment where no count up to 32 fits). EINVAL outside
 * 0..32. confkv_attend_splits returns the count the next confkv_attend will
 * use (-1 for an unknown handle). Host-only. */
int confkv_set_attend_splits(confkv_handle* h, int32_t splits);
int32_t confkv_attend_splits(const confkv_handle* h);

/* The next token of each batch row from a step's logits: the decoding loop
 * of the "Conf-KV" post ends each step by drawing x_t from the same
 * p = softmax(logits) whose confidence set the budget (temperature 1, no
 * truncation).
 *   logits     [B][V] fp32
 *   u          [B] fp32 in [0, 1), or NULL. NULL: greedy, the largest logit
 *              (lowest index among equal maxima). Otherwise an inverse-CDF
 *              draw: the smallest j with p_0 + ... + p_j > u[b], the sums
 *              formed in binary64 (a u within about 1e-12 of a running sum
 *              may land on either neighbour; where rounding leaves u past
 *              the last sum, the last token with p_j > 0).
 *   token_out  [B] int32 (written); -1 for a row holding a non-finite logit,
 *              which also sets the sticky CONFKV_ENONFINITE.
 * CONF only (EINVAL for KVPOP, which has no vocabulary). Touches no cache
 * state, so it may come anywhere between steps; it shares a scratch area
 * with nothing else but itself, so two draws on one handle must be ordered
 * on one stream. Only enqueues work. */
int confkv_sample(confkv_handle* h, void* stream, const float* logits, const float* u, int32_t* token_out);

/* KVpop prefill (or teacher-forced pass) over seq_len = S positions whose
 * static priorities are all known, with the multi-query mask of
 * "Resumen Técnico: KVpop" §2.4: query q sees key j iff
 *   j <= q and (j < s or j >= q - w or j in topk(C_q)),  C_q = [s, q-1-w],
 * top-k by (priority descending, position ascending). That is exactly the
 * set a decode step at t = q attends to (§2.1 budget, §2.3 delayed scoring).
 * The mask is never stored: per (batch row, KV head) a sort ranks the
 * priorities, one pass over q moves the k-th-rank threshold, and the
 * attention kernel tests each (query, key) pair against it. One layer per
 * call; the handle's config supplies B, Hq, Hkv, d, s (num_sink),
 * w (protect_last), k (kvpop_k) and the softmax scale. KVPOP only. The
 * decode cache is not touched.
 *   q     [B][Hq][S][d]  fp16      k, v [B][Hkv][S][d] fp16
 *   prio  [B][Hkv][S]    fp32      (non-finite: sticky CONFKV_ENONFINITE)
 *   out   [B][Hq][S][d]  fp16      lse [B][Hq][S] fp32 or NULL
 *   workspace: device, 256-byte aligned, at least
 *     confkv_kvpop_prefill_workspace(h, S) bytes (0: invalid handle or S).
 *     Afterwards it holds, each part starting at a 256-byte boundary:
 *     sort keys [B*Hkv][N] uint64 (N the power of two >= max(S - s, 1)),
 *     ranks [B*Hkv][S] int32 (0 for the highest priority, -1 for sinks),
 *     thresholds [B*Hkv][S] int32 (the k-th smallest rank of C_q; S while
 *     |C_q| < k; -1 when k = 0).
 * 1 <= S <= 131072; EINVAL where one query tile's key list (s + k + w + 40
 * entries) would not fit on chip. Only enqueues work. */
size_t confkv_kvpop_prefill_workspace(const confkv_handle* h, int32_t seq_len);
int confkv_kvpop_prefill(confkv_handle* h, void* stream, int32_t seq_len, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, const float* prio, uint16_t* out, float* lse, void* workspace,
                         size_t workspace_bytes);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * masked prefill as confkv_kvpop_prefill, same arguments and results, with
 * no workspace argument. Its sort keys, ranks and thresholds live in a
 * library-owned device array of CONFKV_NOALLOC_SCRATCH_BYTES (16 MiB), one
 * copy per GPU, taken when the library's code is loaded on that GPU and held
 * until the process ends. The call allocates and frees nothing.
 * - ECAPACITY, with nothing enqueued, when the workspace this S needs
 *   (confkv_kvpop_prefill_workspace(h, S)) exceeds that size; for instance
 *   B*Hkv = 64 with S = 16384 needs exactly 16 MiB.
 * - Every call on one GPU uses that GPU's single array: calls that overlap on
 *   one GPU (several streams, or several host threads) race and give wrong
 *   results; calls in one stream's order do not. Each call rewrites every
 *   byte it reads, so nothing carries over from an earlier call.
 * - The ranks and thresholds are not handed back (use confkv_kvpop_prefill
 *   for them). Other errors as confkv_kvpop_prefill. Only enqueues work. */
#define CONFKV_NOALLOC_SCRATCH_BYTES (16u << 20)
int confkv_kvpop_prefill_noalloc(confkv_handle* h, void* stream, int32_t seq_len, const uint16_t* q,
                                 const uint16_t* k, const uint16_t* v, const float* prio, uint16_t* out,
                                 float* lse);

/* The training target of KVpop's scorer ("Resumen Técnico: KVpop" §2.2): for
 * each key position t, the log of the attention mass that the future queries
 * d >= t + w give it, summed over the query heads of its KV head,
 *   target[t] = log sum_g sum_{d >= t + w} exp(scale * q[d, g] . k[t] - lse[d, g]),
 * computed by the transposed pass the summary names: keys and queries swap
 * roles in the MFMA and each query's normaliser lse is reused, so no
 * attention map is formed. -inf where no query counts (t + w >= S).
 *   q [B][Hq][S][d] fp16, k [B][Hkv][S][d] fp16,
 *   lse [B][Hq][S] fp32 (for instance the one confkv_kvpop_prefill writes),
 *   target [B][Hkv][S] fp32 (written).
 * KVPOP only (w = protect_last); 1 <= S <= 131072. Only enqueues work. */
int confkv_kvpop_future_target(confkv_handle* h, void* stream, int32_t seq_len, const uint16_t* q, const uint16_t* k,
                               const float* lse, float* target);

/* Gather the logical contents of segments [seg_first, seg_first+seg_count) in
 * ascending position order. The ranking score is not part of the cache (the
 * step forms it from ema, position and the step's t, then ranks and evicts
 * in the same kernel); a step's scores are read, with the rows it saw, by
 * confkv_read_last_step under record_scores. Per segment i, rows 0..len[i]-1 of each
 * [seg_count][rows_max] / [seg_count][rows_max][d] output are written (rows_max
 * = confkv_rows_max); later rows are left untouched. Any output except len may
 * be NULL. FP16 rows appear in k16/v16 and have zero k8/v8/scales; INT8 rows
 * appear in k8/v8 + k_scale/v_scale and have zero k16/v16. ema is 0 for KVPOP
 * and prio is 0 for CONF (and for rows still inside the window). Synchronizes
 * `stream` and returns the sticky error status. */
int confkv_read_cache(confkv_handle* h, void* stream, int32_t seg_first, int32_t seg_count, int32_t* len,
                      int32_t* pos, float* ema, float* prio, uint16_t* k16, uint16_t* v16, int8_t* k8,
                      int8_t* v8, float* k_scale, float* v_scale, uint8_t* is_int8);

/* Requires record_scores. For segments [seg_first, seg_first+seg_count) copy
 * what the last step saw before evicting:
 *   meta  [count][4] int32: staged rows, live rows, per-layer budget, evicted
 *   pos   [count][rows_max] int32: position of each staged row (-1: empty slot)
 *   score [count][rows_max] fp32: the ranking value (CONF: alpha*ema+(1-alpha)*rec
 *         as stored in fp32; KVPOP: the priority) of each staged row
 *   lse   [count][G] fp32: log-sum-exp of each query head's scores
 * Any pointer may be NULL. Synchronizes `stream`. */
int confkv_read_last_step(confkv_handle* h, void* stream, int32_t seg_first, int32_t seg_count,
                          int32_t* meta, int32_t* pos, float* score, float* lse);

/* Totals over all segments since init (or the last reset), written to the
 * HOST array totals[4]: KV bytes read by attention (K+V rows and INT8 scales),
 * rows attended, rows moved by compaction or age-out, rows evicted.
 * Synchronizes `stream`. */
int confkv_stats(confkv_handle* h, void* stream, uint64_t* totals, int32_t reset);

/* Profiling of the step's kernels with HIP events on the step's stream.
 * confkv_profile(h, mask) records an event pair around each launch of the
 * kernels in mask (0 stops recording; EINVAL outside 0 .. CONFKV_PROFILE_ALL):
 * the fused attend+evict kernel of confkv_step, the logits reducer (of
 * confkv_step and confkv_evict), the kernels of confkv_attend and the kernel
 * of confkv_evict. Each event record costs a few microseconds of stream time,
 * so a throughput measurement times only the kernels it needs.
 * confkv_profile_read synchronizes and writes HOST values: total milliseconds
 * and launch counts of the fused kernel and of the reducer, then (if reset)
 * clears them. confkv_profile_kernel does the same for one kernel: 0 fused
 * step, 1 logits reducer, 2 attend, 3 evict (EINVAL otherwise). */
/* A measurement aid, not part of the decode step: a plain streaming kernel
 * over `bytes` of device memory at `src`, enqueued on `stream`, giving the
 * HBM bandwidth a simple read or copy attains on this part, the reference
 * beside the published peak when the step's kernels are measured.
 *   copy = 0: read only; `dst` is a scratch of at least 1 KiB (nothing is
 *             normally written to it);
 *   copy = 1: copy `bytes` from `src` to `dst` (buffers must not overlap).
 * src and dst 16-byte aligned; bytes a positive multiple of 16; caller-owned
 * device pointers. EINVAL on bad arguments, with nothing enqueued. */
int confkv_bandwidth_probe(void* stream, const void* src, void* dst, size_t bytes, int32_t copy);

#define CONFKV_PROFILE_STEP 1
#define CONFKV_PROFILE_REDUCE 2
#define CONFKV_PROFILE_ATTEND 4
#define CONFKV_PROFILE_EVICT 8
#define CONFKV_PROFILE_ALL 15
int confkv_profile(confkv_handle* h, int32_t mask);
int confkv_profile_read(confkv_handle* h, double* fused_ms, int64_t* fused_launches, double* reduce_ms,
                        int64_t* reduce_launches, int32_t reset);
int confkv_profile_kernel(confkv_handle* h, int32_t kernel, double* ms, int64_t* launches, int32_t reset);

/* Position the next confkv_step decodes. -1 for a NULL handle. */
int64_t confkv_position(const confkv_handle* h);

/* Synchronize the last stream used and return the sticky device error word
 * as a status code (CONFKV_OK if none). */
int confkv_status(confkv_handle* h);

/* Free the handle (not the state buffer). Safe on NULL. */
int confkv_destroy(confkv_handle* h);

/* Static string for a status code. */
const char* confkv_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* CONFKV_H */
