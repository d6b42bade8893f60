// Device-state layout and kernel parameter blocks shared by the host ABI
// (api.hip) and the kernels (kernels.hip). Internal: not part of the C ABI.
//
// Per segment seg = (l*B + b)*Hkv + h the state holds two regions:
//   ring  — the FP16 window: Wr = W + 1 slots, a row at position p lives in
//           slot p mod Wr; a position of -1 marks an empty or evicted slot. At
//           step t the live slots hold positions in [t-W, t].
//   old   — rows older than the window, densely packed in [0, n_old) in no
//           particular order: INT8 codes + fp32 absmax scales (old_int8) or
//           FP16. Every old position is below every ring position.
// Row counts are padded to multiples of 32 (cap32, Wr32); padding rows stay
// finite (zeroed at init) and are masked out of every computation.
// K is stored row-major ([row][d]). V is stored in 32-row transposed tiles so
// that one 16-byte load per lane is one MFMA B-operand slice (8 consecutive
// rows of one column) and a wave's load covers 1 KiB of contiguous memory:
// inside a tile, element (row r, column c), with q = r/8, e = r%8,
// cb = c/16, j = c%16, lives at
//   INT8: 1024*(cb/2) + 16*(16q + j) + 8*(cb%2) + e   bytes
//   FP16:  512*cb     +  8*(16q + j) + e              halves
// All arrays are segment-major structure-of-arrays; each array base is
// 256-byte aligned.
#pragma once
#include <stdint.h>

namespace confkv {

constexpr int kThreads = 256;          // fused-step workgroup
constexpr int kChunk = 4096;           // logits per reducer workgroup (256 x 16)
constexpr int kStatFields = 4;         // kv bytes, rows attended, rows moved, rows evicted
constexpr uint32_t kErrNonFinite = 1u, kErrCapacity = 2u, kErrInternal = 4u;
// What one launch of the step kernel covers: the whole step for every
// segment; append + attention + EMA for one layer; or ranking, selection,
// compaction and age-out for every segment after all layers have attended.
enum { kModeStep = 0, kModeAttend = 1, kModeEvict = 2 };

// Selection in the HBM-staged instance (segments whose rows do not fit LDS
// staging): a histogram of the keys' top kSelBinBits bits in LDS, whose
// space then holds up to kSelCandCap candidate keys (8 bytes) and rows (4
// bytes); a victim bitmask of one bit per stage row follows it in LDS when
// it fits kSelBitsLdsMax bytes, else it lives in the segment's HBM stage.
constexpr int kSelBinBits = 13;
constexpr int kSelBins = 1 << kSelBinBits;
constexpr int kSelLdsBytes = kSelBins * 4;
constexpr int kSelCandCap = 2560;
constexpr int kSelBitsLdsMax = 32 * 1024;
static_assert(kSelCandCap * 12 <= kSelLdsBytes, "the candidates reuse the histogram's LDS");
// victim bitmask words for a stage-row count: whole 64-row groups
inline constexpr int64_t sel_bits_words(int64_t rows) { return ((rows + 63) / 64) * 2; }
// Attention of the HBM-staged instance: rows per LDS chunk (a multiple of 32)
// for G score planes and one V-scale plane within kSelLdsBytes.
inline constexpr int hbm_chunk_rows(int G) { return (kSelLdsBytes / (4 * (G + 1))) & ~31; }

struct ConfPartial {                   // one logits chunk: m = top1
  double S;                            // sum exp(z - m)
  double T;                            // sum exp(z - m) * (z - m)
  float m, top2;
  uint32_t nonfinite, pad;
};

struct SamplePartial {                 // one logits chunk for the next-token draw
  double S;                            // sum exp(z - m) (only for a random draw)
  float m;                             // the chunk's largest logit (NaN if idx < 0)
  int32_t idx;                         // its lowest index; -1: a non-finite logit
};

struct SplitML {                       // one split's softmax statistics for one head
  float m;                             // maximum of its scores (-inf: no valid row)
  float l;                             // sum of exp(s - m)
};

struct Layout {
  int32_t L, B, Hq, Hkv, G, D, V;
  int32_t S;          // segments
  int32_t cap;        // old rows per segment
  int32_t W;          // FP16 window (rows with pos > t - W stay in the ring)
  int32_t Wr;         // ring slots = W + 1
  int32_t cap32;      // cap rounded up to 32
  int32_t Wr32;       // Wr rounded up to 32
  int32_t rows_max;   // cap32 + Wr32: staged rows per segment upper bound
  int32_t planes;     // staging planes per segment = max(G, 4)
  int32_t chunks;     // logits chunks per batch row
  int32_t old_bytes;  // bytes per element of an old row (1 int8, 2 fp16)
  // ring
  uint16_t* ring_k;   // [S][Wr32][D] row-major
  uint16_t* ring_v;   // [S][Wr32/32] transposed FP16 tiles
  // old
  uint8_t* old_k;     // [S][cap32][D * old_bytes] row-major
  uint8_t* old_v;     // [S][cap32/32] transposed tiles
  float* old_ks;      // [S][cap32] (old_int8)
  float* old_vs;
  // row state of both regions: old row i at [i], ring slot r at [cap32 + r]
  int32_t* row_pos;   // [S][rows_max]
  float* row_ema;     // [S][rows_max]
  float* row_prio;    // [S][rows_max]
  int32_t* seg_nold;  // [S]
  uint64_t* seg_stats;  // [S][kStatFields]
  float* stage;       // [S][planes][rows_max]: the step's HBM staging where LDS does not hold a
                      // segment's rows; the split attend's raw scores (planes 0..G-1)
  // split-K attend of one layer (reused by every layer)
  int32_t ns_max;     // most splits per segment
  float* sk_o;        // [B*Hkv][ns_max][G][D] unnormalised partial outputs
  SplitML* sk_ml;     // [B*Hkv][ns_max][G]
  float* sk_lse;      // [S][G] log-sum-exp of each head after the split attend's combine
  // confidence reducer
  ConfPartial* partials;  // [B][chunks]
  SamplePartial* spart;   // [B][chunks] (next-token draw)
  uint32_t* err;          // [1]
  uint64_t* stats_total;  // [kStatFields]
  // last-step record (record_scores)
  int32_t* rec_meta;  // [S][4]
  int32_t* rec_pos;   // [S][rows_max]
  float* rec_score;   // [S][rows_max]
  float* rec_lse;     // [S][G]
};

struct Params {
  float tau, alpha, beta, w_e, w_m, w_p, sm_scale;
  int32_t n_low, n_high, P, s, kvpop_k, policy, gate_literal, pyramid, old_int8, record;
  int32_t ranker;  // 0: alpha-blend score; 1: SplitMix64 random rank
  uint32_t seed;
};

struct StepArgs {
  int32_t t;                 // position decoded this step
  int32_t seg0;              // attend: first segment of the layer (inputs are that layer's)
  int32_t ns;                // split-K attend: workgroups per segment
  int32_t lds_rows;          // staged-row capacity of the LDS planes (LDS variant)
  int32_t sel_bits_lds;      // HBM-staged variant: 1 when the victim bitmask is in LDS
  int32_t ema_from_scores;   // evict: the layers attended split-K; update the EMA from the
                             // stored scores and log-sum-exps first
  const uint16_t* q;         // [L][B][Hq][D] (attend: [B][Hq][D])
  const uint16_t* k_new;     // [L][B][Hkv][D] (attend: [B][Hkv][D])
  const uint16_t* v_new;
  const float* prio_new;     // [L][B][Hkv] (attend: [B][Hkv]) or null
  uint16_t* out;             // [L][B][Hq][D] (attend: [B][Hq][D])
  float* conf_out;           // [B] or null (CONF; step and evict)
  int32_t* budget_out;       // [B] or null (CONF; step and evict)
};

// KVpop prefill over S known priorities with the multi-query mask.
struct KvpopPrefillArgs {
  int32_t B, Hq, Hkv, G, D, S;
  int32_t sinks, window, topk;  // s, w, k of B = s + w + k
  int32_t N;                 // sort length: the power of two >= max(S - s, 1)
  int32_t list_cap;          // key-list entries per query tile
  float scale;
  const uint16_t* q;         // [B][Hq][S][D]
  const uint16_t* k;         // [B][Hkv][S][D]
  const uint16_t* v;
  const float* prio;         // [B][Hkv][S]
  uint16_t* out;             // [B][Hq][S][D]
  float* lse;                // [B][Hq][S] or null
  uint64_t* sort;            // workspace [B*Hkv][N]
  int32_t* rank;             // workspace [B*Hkv][S]
  int32_t* thr;              // workspace [B*Hkv][S]
  uint32_t* err;             // the handle's sticky error word
};

// Launchers (kernels.hip). All enqueue on `stream` and return the launch status.
int launch_init(const Layout& lay, const Params& par, void* state, size_t state_bytes, const uint16_t* pk,
                const uint16_t* pv, int32_t P0, void* stream);
int launch_conf_reduce(const Layout& lay, const float* logits, void* stream);
int launch_sample(const Layout& lay, const float* logits, const float* u, int32_t* token, void* stream);
int launch_fused_step(const Layout& lay, const Params& par, const StepArgs& a, bool use_lds, int lds_bytes,
                      void* stream);
int launch_attend_split(const Layout& lay, const Params& par, const StepArgs& a, int lds_bytes, void* stream);
int launch_attend(const Layout& lay, const Params& par, const StepArgs& a, bool use_lds, int lds_bytes,
                  void* stream);
int launch_evict(const Layout& lay, const Params& par, const StepArgs& a, bool use_lds, int lds_bytes,
                 void* stream);
int launch_read_cache(const Layout& lay, int32_t seg_first, int32_t seg_count, int32_t* len, int32_t* pos,
                      float* ema, float* prio, uint16_t* k16, uint16_t* v16, int8_t* k8, int8_t* v8,
                      float* ks, float* vs, uint8_t* is8, int32_t old_int8, void* stream);
int launch_stats_total(const Layout& lay, int32_t reset, void* stream);
int launch_kvpop_prefill(const KvpopPrefillArgs& pa, void* stream);
int launch_kvpop_target(const KvpopPrefillArgs& pa, const float* lse, float* target, void* stream);
int kvpop_prefill_attend_lds(int D, int list_cap, bool with_buffers);
int fused_max_dynamic_lds();

}  // namespace confkv
