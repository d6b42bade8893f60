// Host side of the C ABI declared in include/confkv.h: configuration checks,
// carving of the caller's state buffer, and the per-step launch sequence.
// Nothing here computes a step; every stage runs in kernels.hip.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <unordered_set>
#include <vector>

#include "confkv.h"
#include "layout.h"

#define CONFKV_API extern "C" __attribute__((visibility("default")))

using namespace confkv;

namespace confkv {
int launch_stream_probe(const void* src, void* dst, size_t bytes, int32_t copy, void* stream);  // probe.hip
}

// Workspace of confkv_kvpop_prefill_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends. Host code never passes its name
// to a kernel or a copy (on the host it is only a stand-in for the symbol);
// it uses the device address taken by hipGetSymbolAddress for each device.
static __device__ __align__(256) uint8_t scratch[CONFKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr uint32_t kMagic = 0xC0F4B1E5u;
constexpr uint32_t kDead = 0xDEADDEADu;
constexpr int kMaxProfilePairs = 1 << 15;
constexpr int kSplitMax = 32;        // most workgroups per segment in a split-K attend
constexpr int kSplitTarget = 1024;   // workgroups an automatic split-K attend aims for (one per CU slot)
constexpr int kSplitMinTiles = 4;    // 32-row tiles per split at least, when splitting for occupancy

struct EventPool {
  int bit = 0;                 // this kernel's bit in the profiling mask
  std::vector<hipEvent_t> ev;  // pairs: start, stop
  size_t used = 0;             // pairs recorded since the last read
  double ms = 0.0;
  int64_t n = 0;
};

}  // namespace

struct confkv_handle {
  uint32_t magic;
  confkv_config cfg;
  Layout lay;
  Params par;
  void* state;
  size_t state_bytes;
  int64_t t;           // position decoded by the next step
  int64_t rows_bound;  // upper bound on rows any segment retains before the next step
  int64_t keep_max;    // no segment keeps more rows than this after an eviction
  int poisoned;
  hipStream_t last_stream;
  int prof;  // mask of the kernels whose launches get an event pair
  EventPool pf, pr;    // fused kernel, logits reducer
  EventPool pa, pe;    // attend kernel, evict kernel
  std::vector<uint8_t> attended;  // per layer: attended at position t by confkv_attend
  int32_t n_attended;             // layers attended at t (0: no split step under way)
  int32_t attend_splits;          // 0: automatic; 1: one workgroup per segment; >= 2: that many
  int32_t step_split;             // the layers attended at t used the split-K attend
};

namespace {

int group_ok(int g) { return g == 1 || g == 2 || g == 4 || g == 5 || g == 8; }

int64_t window_of(const confkv_config* c) {
  return c->policy == CONFKV_POLICY_KVPOP ? c->protect_last : c->fp16_window;
}

// Largest per-layer budget the configuration can produce.
int64_t budget_max(const confkv_config* c) {
  if (c->policy == CONFKV_POLICY_KVPOP) return (int64_t)c->num_sink + c->protect_last + c->kvpop_k;
  const int64_t top = std::max(c->n_low, c->n_high);
  return (c->pyramid && c->num_layers > 1) ? (3 * top) / 2 : top;
}

int64_t keep_bound(const confkv_config* c) {
  return std::max<int64_t>(budget_max(c), (int64_t)c->num_sink + c->protect_last);
}

bool finite_all(std::initializer_list<float> v) {
  for (float x : v)
    if (!isfinite(x)) return false;
  return true;
}

int check_cfg(const confkv_config* c, int32_t P0) {
  if (!c) return CONFKV_EINVAL;
  if (c->abi_version != CONFKV_ABI_VERSION) return CONFKV_EINVAL;
  if (c->num_layers < 1 || c->batch < 1 || c->num_kv_heads < 1 || c->num_q_heads < 1) return CONFKV_EINVAL;
  if (c->num_q_heads % c->num_kv_heads) return CONFKV_EINVAL;
  if (!group_ok(c->num_q_heads / c->num_kv_heads)) return CONFKV_EINVAL;
  if (c->head_dim != 64 && c->head_dim != 128) return CONFKV_EINVAL;
  if (c->policy != CONFKV_POLICY_CONF && c->policy != CONFKV_POLICY_KVPOP) return CONFKV_EINVAL;
  if (c->protect_last < 0 || c->fp16_window < 0 || c->num_sink < 0 || P0 < 0) return CONFKV_EINVAL;
  if (c->old_int8 != 0 && c->old_int8 != 1) return CONFKV_EINVAL;
  if (c->ranker != CONFKV_RANKER_SCORE && c->ranker != CONFKV_RANKER_RANDOM) return CONFKV_EINVAL;
  if (c->ranker == CONFKV_RANKER_RANDOM && c->policy != CONFKV_POLICY_CONF) return CONFKV_EINVAL;
  if (!finite_all({c->softmax_scale}) || c->softmax_scale < 0.0f) return CONFKV_EINVAL;
  if (c->policy == CONFKV_POLICY_CONF) {
    if (c->vocab < 2 || c->n_low < 0 || c->n_high < 0) return CONFKV_EINVAL;
    if (!finite_all({c->tau, c->alpha, c->ema_beta, c->w_entropy, c->w_margin, c->w_pmax})) return CONFKV_EINVAL;
  } else {
    if (c->kvpop_k < 0 || P0 != 0) return CONFKV_EINVAL;
  }
  const int64_t W = window_of(c);
  if (W > (1 << 16)) return CONFKV_EINVAL;
  if (c->capacity < 1) return CONFKV_ECAPACITY;
  const int64_t need = std::max<int64_t>({(int64_t)P0, keep_bound(c) + 1, 1});
  if ((int64_t)c->capacity < need) return CONFKV_ECAPACITY;
  // index arithmetic of the kernels stays in range
  const int64_t S = (int64_t)c->num_layers * c->batch * c->num_kv_heads;
  if (S > (1 << 30) || (int64_t)c->capacity > (1 << 30)) return CONFKV_EINVAL;
  if (S * ((int64_t)c->capacity + W + 1) * c->head_dim * 2 > (int64_t)1 << 50) return CONFKV_ECAPACITY;
  return CONFKV_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Carve the state; with base == nullptr only the size is computed.
size_t carve(const confkv_config* c, uint8_t* base, Layout* L) {
  Layout lay;
  memset(&lay, 0, sizeof(lay));
  lay.L = c->num_layers;
  lay.B = c->batch;
  lay.Hq = c->num_q_heads;
  lay.Hkv = c->num_kv_heads;
  lay.G = c->num_q_heads / c->num_kv_heads;
  lay.D = c->head_dim;
  lay.V = c->policy == CONFKV_POLICY_CONF ? c->vocab : 0;
  lay.S = c->num_layers * c->batch * c->num_kv_heads;
  lay.cap = c->capacity;
  lay.W = (int32_t)window_of(c);
  lay.Wr = lay.W + 1;
  lay.cap32 = (lay.cap + 31) & ~31;
  lay.Wr32 = (lay.Wr + 31) & ~31;
  lay.rows_max = lay.cap32 + lay.Wr32;
  lay.planes = std::max(lay.G, 4);
  lay.chunks = lay.V > 0 ? (lay.V + kChunk - 1) / kChunk : 0;
  lay.old_bytes = c->old_int8 ? 1 : 2;
  const size_t S = (size_t)lay.S, D = (size_t)lay.D, Wr = (size_t)lay.Wr32, cap = (size_t)lay.cap32;
  size_t off = 0;
  auto take = [&](size_t bytes) -> uint8_t* {
    const size_t o = align256(off);
    off = o + std::max<size_t>(bytes, 1);
    return base ? base + o : nullptr;
  };
  lay.ring_k = (uint16_t*)take(S * Wr * D * 2);
  lay.ring_v = (uint16_t*)take(S * Wr * D * 2);
  lay.old_k = take(S * cap * D * lay.old_bytes);
  lay.old_v = take(S * cap * D * lay.old_bytes);
  lay.old_ks = (float*)take(S * cap * 4);
  lay.old_vs = (float*)take(S * cap * 4);
  lay.row_pos = (int32_t*)take(S * (size_t)lay.rows_max * 4);
  lay.row_ema = (float*)take(S * (size_t)lay.rows_max * 4);
  lay.row_prio = (float*)take(S * (size_t)lay.rows_max * 4);
  lay.seg_nold = (int32_t*)take(S * 4);
  lay.seg_stats = (uint64_t*)take(S * kStatFields * 8);
  lay.stage = (float*)take(S * lay.planes * (size_t)lay.rows_max * 4);
  const size_t segs_l = (size_t)lay.B * lay.Hkv;
  lay.ns_max = kSplitMax;
  lay.sk_o = (float*)take(segs_l * kSplitMax * lay.G * D * 4);
  lay.sk_ml = (SplitML*)take(segs_l * kSplitMax * lay.G * sizeof(SplitML));
  lay.sk_lse = (float*)take(S * lay.G * 4);
  lay.partials = (ConfPartial*)take((size_t)lay.B * std::max(lay.chunks, 1) * sizeof(ConfPartial));
  lay.spart = (SamplePartial*)take((size_t)lay.B * std::max(lay.chunks, 1) * sizeof(SamplePartial));
  lay.err = (uint32_t*)take(4);
  lay.stats_total = (uint64_t*)take(kStatFields * 8);
  if (c->record_scores) {
    lay.rec_meta = (int32_t*)take(S * 16);
    lay.rec_pos = (int32_t*)take(S * lay.rows_max * 4);
    lay.rec_score = (float*)take(S * lay.rows_max * 4);
    lay.rec_lse = (float*)take(S * lay.G * 4);
  }
  if (L) *L = lay;
  return align256(off);
}

Params make_params(const confkv_config* c) {
  Params p;
  memset(&p, 0, sizeof(p));
  p.tau = c->tau;
  p.alpha = c->alpha;
  p.beta = c->ema_beta;
  p.w_e = c->w_entropy;
  p.w_m = c->w_margin;
  p.w_p = c->w_pmax;
  p.sm_scale = c->softmax_scale > 0.0f ? c->softmax_scale : (float)(1.0 / sqrt((double)c->head_dim));
  p.n_low = c->n_low;
  p.n_high = c->n_high;
  p.P = c->protect_last;
  p.s = c->num_sink;
  p.kvpop_k = c->kvpop_k;
  p.policy = c->policy;
  p.gate_literal = c->gate_literal ? 1 : 0;
  p.pyramid = c->pyramid ? 1 : 0;
  p.old_int8 = c->old_int8;
  p.record = c->record_scores ? 1 : 0;
  p.ranker = c->ranker;
  p.seed = c->seed;
  return p;
}

// Device address of `scratch` per device id, taken once per device with that
// device current (at confkv_init, or at the first no-allocation call there).
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return CONFKV_EHIP;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return CONFKV_EHIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CONFKV_OK;
}

// Handles handed out and not yet destroyed; a destroyed or foreign pointer is
// never dereferenced.
std::mutex g_mu;
std::unordered_set<const confkv_handle*> g_live;

bool live(const confkv_handle* h) {
  if (!h) return false;
  std::lock_guard<std::mutex> lk(g_mu);
  return g_live.count(h) != 0;
}

int record_event(confkv_handle* h, EventPool& pool, hipStream_t s, bool start) {
  if (!(h->prof & pool.bit)) return 0;
  const size_t idx = 2 * pool.used + (start ? 0 : 1);
  if (pool.used >= (size_t)kMaxProfilePairs) return 0;
  while (pool.ev.size() <= idx) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return -1;
    pool.ev.push_back(e);
  }
  if (hipEventRecord(pool.ev[idx], s) != hipSuccess) return -1;
  if (!start) ++pool.used;
  return 0;
}

int collect(EventPool& pool) {
  for (size_t i = 0; i < pool.used; ++i) {
    float ms = 0.0f;
    if (hipEventSynchronize(pool.ev[2 * i + 1]) != hipSuccess) return -1;
    if (hipEventElapsedTime(&ms, pool.ev[2 * i], pool.ev[2 * i + 1]) != hipSuccess) return -1;
    pool.ms += ms;
    pool.n += 1;
  }
  pool.used = 0;
  return 0;
}

// Staging of a launch: LDS planes sized for the most rows a segment can hold
// at this step, or the HBM stage when they do not fit. The HBM-staged
// instance takes LDS for its selection (histogram, candidates and, when it
// fits, the victim bitmask over every stage row).
struct Staging {
  bool use_lds;
  int32_t lds_rows;
  int lds_bytes;
  int32_t sel_bits_lds;
};

Staging staging(const confkv_handle* h, int planes) {
  const Layout& lay = h->lay;
  const int64_t old32 = (std::min<int64_t>(h->rows_bound, lay.cap) + 31) & ~(int64_t)31;
  const int64_t lds_rows = old32 + lay.Wr32;
  const int64_t lds_bytes = lds_rows * planes * 4;
  Staging st;
  st.use_lds = lds_bytes <= fused_max_dynamic_lds();
  st.lds_rows = st.use_lds ? (int32_t)lds_rows : 0;
  st.lds_bytes = st.use_lds ? (int)lds_bytes : 0;
  st.sel_bits_lds = 0;
  if (!st.use_lds) {
    const int64_t bits_bytes = sel_bits_words(lay.rows_max) * 4;
    st.sel_bits_lds = bits_bytes <= kSelBitsLdsMax ? 1 : 0;
    st.lds_bytes = kSelLdsBytes + (st.sel_bits_lds ? (int)bits_bytes : 0);
  }
  return st;
}

// Workgroups per segment for one layer's attend: 1 selects the whole-segment
// kernel. Automatic: enough splits for about kSplitTarget workgroups, at least
// kSplitMinTiles 32-row tiles per split, and few enough rows per split for
// the LDS.
int attend_splits(const confkv_handle* h) {
  const Layout& lay = h->lay;
  const int64_t segs = (int64_t)lay.B * lay.Hkv;
  const int64_t tiles = ((std::min<int64_t>(h->rows_bound, lay.cap) + 31) >> 5) + (lay.Wr32 >> 5);
  auto lds_ok = [&](int64_t ns) {
    return ((tiles + ns - 1) / ns) * 32 * (lay.G + 1) * 4 <= (int64_t)fused_max_dynamic_lds();
  };
  int64_t ns;
  if (h->attend_splits == 1) return 1;
  if (h->attend_splits >= 2) {
    ns = std::min<int64_t>(h->attend_splits, tiles);
  } else {
    ns = std::min<int64_t>({(kSplitTarget + segs - 1) / segs, tiles / kSplitMinTiles, (int64_t)kSplitMax});
  }
  while (ns <= kSplitMax && ns >= 2 && !lds_ok(ns)) ++ns;
  if (ns < 2 || ns > kSplitMax || !lds_ok(ns)) return 1;
  return (int)ns;
}

void advance(confkv_handle* h) {
  h->t += 1;
  h->rows_bound = std::min(h->rows_bound + 1, h->keep_max);
}

int device_status(confkv_handle* h) {
  if (hipStreamSynchronize(h->last_stream) != hipSuccess) {
    h->poisoned = 1;
    return CONFKV_EHIP;
  }
  uint32_t err = 0;
  if (hipMemcpy(&err, h->lay.err, 4, hipMemcpyDeviceToHost) != hipSuccess) {
    h->poisoned = 1;
    return CONFKV_EHIP;
  }
  if (!err) return CONFKV_OK;
  h->poisoned = 1;
  if (err & kErrNonFinite) return CONFKV_ENONFINITE;
  if (err & kErrCapacity) return CONFKV_ECAPACITY;
  return CONFKV_EHIP;
}

}  // namespace

CONFKV_API int confkv_validate(const confkv_config* cfg, int32_t prefill_len) { return check_cfg(cfg, prefill_len); }

CONFKV_API size_t confkv_state_bytes(const confkv_config* cfg) {
  if (check_cfg(cfg, 0) != CONFKV_OK) return 0;
  return carve(cfg, nullptr, nullptr);
}

CONFKV_API int32_t confkv_rows_max(const confkv_config* cfg) {
  if (check_cfg(cfg, 0) != CONFKV_OK) return 0;
  Layout lay;
  carve(cfg, nullptr, &lay);
  return lay.rows_max;
}

CONFKV_API int confkv_init(const confkv_config* cfg, void* state, size_t state_bytes, void* stream,
                           const uint16_t* prefill_k, const uint16_t* prefill_v, int32_t prefill_len,
                           confkv_handle** out) {
  if (!out) return CONFKV_EINVAL;
  *out = nullptr;
  const int rc = check_cfg(cfg, prefill_len);
  if (rc != CONFKV_OK) return rc;
  if (!state || ((uintptr_t)state & 255)) return CONFKV_EINVAL;
  if (state_bytes < carve(cfg, nullptr, nullptr)) return CONFKV_ECAPACITY;
  if (prefill_len > 0 && (!prefill_k || !prefill_v)) return CONFKV_EINVAL;
  if (prefill_len == 0 && (prefill_k || prefill_v)) return CONFKV_EINVAL;
  void* scratch_ptr = nullptr;
  if (scratch_on_current_device(&scratch_ptr) != CONFKV_OK) return CONFKV_EHIP;
  confkv_handle* h = new (std::nothrow) confkv_handle();
  if (!h) return CONFKV_EHIP;
  h->magic = kMagic;
  h->cfg = *cfg;
  carve(cfg, (uint8_t*)state, &h->lay);
  h->par = make_params(cfg);
  h->state = state;
  h->state_bytes = state_bytes;
  h->t = prefill_len;
  h->rows_bound = prefill_len;
  h->keep_max = keep_bound(cfg);
  h->poisoned = 0;
  h->last_stream = (hipStream_t)stream;
  h->prof = 0;
  h->pf.bit = CONFKV_PROFILE_STEP;
  h->pr.bit = CONFKV_PROFILE_REDUCE;
  h->pa.bit = CONFKV_PROFILE_ATTEND;
  h->pe.bit = CONFKV_PROFILE_EVICT;
  h->attended.assign((size_t)cfg->num_layers, 0);
  h->n_attended = 0;
  h->attend_splits = 0;
  h->step_split = 0;
  if (launch_init(h->lay, h->par, state, carve(cfg, nullptr, nullptr), prefill_k, prefill_v, prefill_len, stream) !=
      0) {
    h->magic = kDead;
    delete h;
    return CONFKV_EHIP;
  }
  {
    std::lock_guard<std::mutex> lk(g_mu);
    g_live.insert(h);
  }
  *out = h;
  return CONFKV_OK;
}

CONFKV_API int confkv_step(confkv_handle* h, void* stream, const float* logits, const uint16_t* q,
                           const uint16_t* k_new, const uint16_t* v_new, const float* prio_new, uint16_t* out,
                           float* conf_out, int32_t* budget_out) {
  if (!live(h)) return CONFKV_ESTATE;
  if (h->poisoned) return CONFKV_ESTATE;
  if (!q || !k_new || !v_new || !out) return CONFKV_EINVAL;
  const bool conf = h->cfg.policy == CONFKV_POLICY_CONF;
  if (conf && (!logits || prio_new)) return CONFKV_EINVAL;
  if (!conf && (logits || !prio_new || conf_out || budget_out)) return CONFKV_EINVAL;
  if (h->t >= (int64_t)INT32_MAX - 1) return CONFKV_EINVAL;
  if (h->n_attended) return CONFKV_EINVAL;  // a split step is under way
  hipStream_t s = (hipStream_t)stream;
  h->last_stream = s;
  const Layout& lay = h->lay;
  if (conf) {
    if (record_event(h, h->pr, s, true)) goto hip_fail;
    if (launch_conf_reduce(lay, logits, stream) != 0) goto hip_fail;
    if (record_event(h, h->pr, s, false)) goto hip_fail;
  }
  {
    StepArgs a;
    memset(&a, 0, sizeof(a));
    a.t = (int32_t)h->t;
    a.seg0 = 0;
    a.q = q;
    a.k_new = k_new;
    a.v_new = v_new;
    a.prio_new = prio_new;
    a.out = out;
    a.conf_out = conf_out;
    a.budget_out = budget_out;
    const Staging sg = staging(h, lay.planes);
    a.lds_rows = sg.lds_rows;
    a.sel_bits_lds = sg.sel_bits_lds;
    if (record_event(h, h->pf, s, true)) goto hip_fail;
    if (launch_fused_step(lay, h->par, a, sg.use_lds, sg.lds_bytes, stream) != 0) goto hip_fail;
    if (record_event(h, h->pf, s, false)) goto hip_fail;
  }
  advance(h);
  return CONFKV_OK;
hip_fail:
  h->poisoned = 1;
  return CONFKV_EHIP;
}

CONFKV_API int confkv_attend(confkv_handle* h, void* stream, int32_t layer, const uint16_t* q,
                             const uint16_t* k_new, const uint16_t* v_new, const float* prio_new, uint16_t* out) {
  if (!live(h)) return CONFKV_ESTATE;
  if (h->poisoned) return CONFKV_ESTATE;
  if (!q || !k_new || !v_new || !out) return CONFKV_EINVAL;
  const bool conf = h->cfg.policy == CONFKV_POLICY_CONF;
  if (conf == (prio_new != nullptr)) return CONFKV_EINVAL;
  if (layer < 0 || layer >= h->lay.L || h->attended[(size_t)layer]) return CONFKV_EINVAL;
  if (h->t >= (int64_t)INT32_MAX - 1) return CONFKV_EINVAL;
  const Layout& lay = h->lay;
  StepArgs a;
  memset(&a, 0, sizeof(a));
  a.t = (int32_t)h->t;
  a.seg0 = layer * lay.B * lay.Hkv;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.prio_new = prio_new;
  a.out = out;
  hipStream_t s = (hipStream_t)stream;
  h->last_stream = s;
  const int ns = attend_splits(h);
  int rc;
  if (ns >= 2) {
    const int64_t tiles = ((std::min<int64_t>(h->rows_bound, lay.cap) + 31) >> 5) + (lay.Wr32 >> 5);
    a.ns = ns;
    a.lds_rows = (int32_t)(((tiles + ns - 1) / ns) * 32);
    if (record_event(h, h->pa, s, true)) goto hip_fail;
    rc = launch_attend_split(lay, h->par, a, a.lds_rows * (lay.G + 1) * 4, stream);  // planes + V scales
  } else {
    const Staging sg = staging(h, lay.planes);
    a.lds_rows = sg.lds_rows;
    if (record_event(h, h->pa, s, true)) goto hip_fail;
    rc = launch_attend(lay, h->par, a, sg.use_lds, sg.lds_bytes, stream);
  }
  if (rc != 0 || record_event(h, h->pa, s, false)) goto hip_fail;
  h->step_split = ns >= 2 ? 1 : 0;  // the same for every layer of a step
  h->attended[(size_t)layer] = 1;
  h->n_attended += 1;
  return CONFKV_OK;
hip_fail:
  h->poisoned = 1;
  return CONFKV_EHIP;
}

CONFKV_API int confkv_set_attend_splits(confkv_handle* h, int32_t splits) {
  if (!live(h)) return CONFKV_ESTATE;
  if (splits < 0 || splits > kSplitMax) return CONFKV_EINVAL;
  if (h->n_attended) return CONFKV_EINVAL;  // not inside a split step: its layers share one mode
  h->attend_splits = splits;
  return CONFKV_OK;
}

CONFKV_API int32_t confkv_attend_splits(const confkv_handle* h) {
  if (!live(h)) return -1;
  return attend_splits(h);
}

CONFKV_API int confkv_evict(confkv_handle* h, void* stream, const float* logits, float* conf_out,
                            int32_t* budget_out) {
  if (!live(h)) return CONFKV_ESTATE;
  if (h->poisoned) return CONFKV_ESTATE;
  const bool conf = h->cfg.policy == CONFKV_POLICY_CONF;
  if (conf && !logits) return CONFKV_EINVAL;
  if (!conf && (logits || conf_out || budget_out)) return CONFKV_EINVAL;
  if (h->n_attended != h->lay.L) return CONFKV_EINVAL;  // every layer attends before the eviction
  const Layout& lay = h->lay;
  hipStream_t s = (hipStream_t)stream;
  h->last_stream = s;
  if (conf && (record_event(h, h->pr, s, true) || launch_conf_reduce(lay, logits, stream) != 0 ||
               record_event(h, h->pr, s, false))) {
    h->poisoned = 1;
    return CONFKV_EHIP;
  }
  StepArgs a;
  memset(&a, 0, sizeof(a));
  a.t = (int32_t)h->t;
  a.conf_out = conf_out;
  a.budget_out = budget_out;
  const Staging sg = staging(h, 4);  // keys (two planes) and the compaction lists
  a.lds_rows = sg.lds_rows;
  a.sel_bits_lds = sg.sel_bits_lds;
  a.ema_from_scores = h->step_split;
  if (record_event(h, h->pe, s, true) || launch_evict(lay, h->par, a, sg.use_lds, sg.lds_bytes, stream) != 0 ||
      record_event(h, h->pe, s, false)) {
    h->poisoned = 1;
    return CONFKV_EHIP;
  }
  std::fill(h->attended.begin(), h->attended.end(), (uint8_t)0);
  h->n_attended = 0;
  advance(h);
  return CONFKV_OK;
}

CONFKV_API int confkv_sample(confkv_handle* h, void* stream, const float* logits, const float* u,
                             int32_t* token_out) {
  if (!live(h)) return CONFKV_ESTATE;
  if (h->poisoned) return CONFKV_ESTATE;
  if (h->cfg.policy != CONFKV_POLICY_CONF || !logits || !token_out) return CONFKV_EINVAL;
  h->last_stream = (hipStream_t)stream;
  if (launch_sample(h->lay, logits, u, token_out, stream) != 0) {
    h->poisoned = 1;
    return CONFKV_EHIP;
  }
  return CONFKV_OK;
}

namespace {
constexpr int64_t kPrefillMaxLen = 1 << 17;

struct PrefillSizes {
  int64_t N, sort_bytes, rank_bytes, total;
};

PrefillSizes prefill_sizes(const confkv_handle* h, int64_t S) {
  const int64_t segs = (int64_t)h->lay.B * h->lay.Hkv;
  int64_t N = 1;
  while (N < std::max<int64_t>(S - h->cfg.num_sink, 1)) N <<= 1;
  PrefillSizes z;
  z.N = N;
  z.sort_bytes = (int64_t)align256((size_t)(segs * N * 8));
  z.rank_bytes = (int64_t)align256((size_t)(segs * S * 4));
  // the thresholds follow the ranks: the attend kernel's 16-byte reads may run
  // up to 60 bytes past the last segment's ranks, into the thresholds
  z.total = z.sort_bytes + 2 * z.rank_bytes;
  return z;
}

int prefill_list_cap(const confkv_handle* h, int64_t S) {
  const confkv_config& c = h->cfg;
  return (int)(std::min<int64_t>(c.num_sink, S) + std::min<int64_t>(c.kvpop_k, S) + c.protect_last + 32 + 8);
}
}  // namespace

CONFKV_API size_t confkv_kvpop_prefill_workspace(const confkv_handle* h, int32_t seq_len) {
  if (!live(h) || h->cfg.policy != CONFKV_POLICY_KVPOP || seq_len < 1 || seq_len > kPrefillMaxLen) return 0;
  return (size_t)prefill_sizes(h, seq_len).total;
}

namespace {
// Checks shared by the two prefill entry points (the workspace aside).
int prefill_args_ok(const confkv_handle* h, int32_t seq_len, const uint16_t* q, const uint16_t* k,
                    const uint16_t* v, const float* prio, const uint16_t* out) {
  if (!live(h)) return CONFKV_ESTATE;
  if (h->poisoned) return CONFKV_ESTATE;
  if (h->cfg.policy != CONFKV_POLICY_KVPOP) return CONFKV_EINVAL;
  if (seq_len < 1 || seq_len > kPrefillMaxLen) return CONFKV_EINVAL;
  if (!q || !k || !v || !prio || !out) return CONFKV_EINVAL;
  return CONFKV_OK;
}

// Enqueue the rank, threshold and masked attention kernels with the given
// workspace (sort keys, ranks, thresholds; every byte rewritten per call).
int kvpop_prefill_enqueue(confkv_handle* h, void* stream, int32_t seq_len, const uint16_t* q, const uint16_t* k,
                          const uint16_t* v, const float* prio, uint16_t* out, float* lse, void* workspace) {
  const PrefillSizes z = prefill_sizes(h, seq_len);
  const int cap = prefill_list_cap(h, seq_len);
  if (kvpop_prefill_attend_lds(h->lay.D, cap, true) > fused_max_dynamic_lds()) return CONFKV_EINVAL;
  KvpopPrefillArgs pa;
  memset(&pa, 0, sizeof(pa));
  pa.B = h->lay.B;
  pa.Hq = h->lay.Hq;
  pa.Hkv = h->lay.Hkv;
  pa.G = h->lay.G;
  pa.D = h->lay.D;
  pa.S = seq_len;
  pa.sinks = h->cfg.num_sink;
  pa.window = h->cfg.protect_last;
  pa.topk = h->cfg.kvpop_k;
  pa.N = (int32_t)z.N;
  pa.list_cap = cap;
  pa.scale = h->par.sm_scale;
  pa.q = q;
  pa.k = k;
  pa.v = v;
  pa.prio = prio;
  pa.out = out;
  pa.lse = lse;
  uint8_t* ws = (uint8_t*)workspace;
  pa.sort = (uint64_t*)ws;
  pa.rank = (int32_t*)(ws + z.sort_bytes);
  pa.thr = (int32_t*)(ws + z.sort_bytes + z.rank_bytes);
  pa.err = h->lay.err;
  h->last_stream = (hipStream_t)stream;
  if (launch_kvpop_prefill(pa, stream) != 0) {
    h->poisoned = 1;
    return CONFKV_EHIP;
  }
  return CONFKV_OK;
}
}  // namespace

CONFKV_API int confkv_kvpop_prefill(confkv_handle* h, void* stream, int32_t seq_len, const uint16_t* q,
                                    const uint16_t* k, const uint16_t* v, const float* prio, uint16_t* out,
                                    float* lse, void* workspace, size_t workspace_bytes) {
  const int rc = prefill_args_ok(h, seq_len, q, k, v, prio, out);
  if (rc != CONFKV_OK) return rc;
  if (!workspace || ((uintptr_t)workspace & 255)) return CONFKV_EINVAL;
  if (workspace_bytes < (size_t)prefill_sizes(h, seq_len).total) return CONFKV_ECAPACITY;
  return kvpop_prefill_enqueue(h, stream, seq_len, q, k, v, prio, out, lse, workspace);
}

CONFKV_API int confkv_kvpop_prefill_noalloc(confkv_handle* h, void* stream, int32_t seq_len, const uint16_t* q,
                                            const uint16_t* k, const uint16_t* v, const float* prio, uint16_t* out,
                                            float* lse) {
  const int rc = prefill_args_ok(h, seq_len, q, k, v, prio, out);
  if (rc != CONFKV_OK) return rc;
  if ((size_t)prefill_sizes(h, seq_len).total > (size_t)CONFKV_NOALLOC_SCRATCH_BYTES) return CONFKV_ECAPACITY;
  void* ws = nullptr;
  if (scratch_on_current_device(&ws) != CONFKV_OK) return CONFKV_EHIP;
  return kvpop_prefill_enqueue(h, stream, seq_len, q, k, v, prio, out, lse, ws);
}

CONFKV_API int confkv_kvpop_future_target(confkv_handle* h, void* stream, int32_t seq_len, const uint16_t* q,
                                         const uint16_t* k, const float* lse, float* target) {
  if (!live(h)) return CONFKV_ESTATE;
  if (h->poisoned) return CONFKV_ESTATE;
  if (h->cfg.policy != CONFKV_POLICY_KVPOP) return CONFKV_EINVAL;
  if (seq_len < 1 || seq_len > kPrefillMaxLen) return CONFKV_EINVAL;
  if (!q || !k || !lse || !target) return CONFKV_EINVAL;
  KvpopPrefillArgs pa;
  memset(&pa, 0, sizeof(pa));
  pa.B = h->lay.B;
  pa.Hq = h->lay.Hq;
  pa.Hkv = h->lay.Hkv;
  pa.G = h->lay.G;
  pa.D = h->lay.D;
  pa.S = seq_len;
  pa.window = h->cfg.protect_last;
  pa.scale = h->par.sm_scale;
  pa.q = q;
  pa.k = k;
  pa.err = h->lay.err;
  h->last_stream = (hipStream_t)stream;
  if (launch_kvpop_target(pa, lse, target, stream) != 0) {
    h->poisoned = 1;
    return CONFKV_EHIP;
  }
  return CONFKV_OK;
}

CONFKV_API int confkv_read_cache(confkv_handle* h, void* stream, int32_t seg_first, int32_t seg_count, int32_t* len,
                                 int32_t* pos, float* ema, float* prio, uint16_t* k16, uint16_t* v16, int8_t* k8,
                                 int8_t* v8, float* k_scale, float* v_scale, uint8_t* is_int8) {
  if (!live(h) || h->poisoned) return CONFKV_ESTATE;
  if (!len || seg_first < 0 || seg_count < 1 || seg_first + (int64_t)seg_count > h->lay.S) return CONFKV_EINVAL;
  h->last_stream = (hipStream_t)stream;
  if (launch_read_cache(h->lay, seg_first, seg_count, len, pos, ema, prio, k16, v16, k8, v8, k_scale, v_scale,
                        is_int8, h->cfg.old_int8, stream) != 0) {
    h->poisoned = 1;
    return CONFKV_EHIP;
  }
  return device_status(h);
}

CONFKV_API int confkv_read_last_step(confkv_handle* h, void* stream, int32_t seg_first, int32_t seg_count,
                                     int32_t* meta, int32_t* pos, float* score, float* lse) {
  if (!live(h) || h->poisoned) return CONFKV_ESTATE;
  if (!h->cfg.record_scores) return CONFKV_EINVAL;
  if (seg_first < 0 || seg_count < 1 || seg_first + (int64_t)seg_count > h->lay.S) return CONFKV_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  h->last_stream = s;
  const Layout& L = h->lay;
  const size_t rm = (size_t)L.rows_max;
  bool ok = true;
  if (meta)
    ok &= hipMemcpyAsync(meta, L.rec_meta + (size_t)seg_first * 4, (size_t)seg_count * 16, hipMemcpyDeviceToDevice,
                         s) == hipSuccess;
  if (pos)
    ok &= hipMemcpyAsync(pos, L.rec_pos + (size_t)seg_first * rm, (size_t)seg_count * rm * 4,
                         hipMemcpyDeviceToDevice, s) == hipSuccess;
  if (score)
    ok &= hipMemcpyAsync(score, L.rec_score + (size_t)seg_first * rm, (size_t)seg_count * rm * 4,
                         hipMemcpyDeviceToDevice, s) == hipSuccess;
  if (lse)
    ok &= hipMemcpyAsync(lse, L.rec_lse + (size_t)seg_first * L.G, (size_t)seg_count * L.G * 4,
                         hipMemcpyDeviceToDevice, s) == hipSuccess;
  if (!ok) {
    h->poisoned = 1;
    return CONFKV_EHIP;
  }
  return device_status(h);
}

CONFKV_API int confkv_stats(confkv_handle* h, void* stream, uint64_t* totals, int32_t reset) {
  if (!live(h) || h->poisoned) return CONFKV_ESTATE;
  if (!totals) return CONFKV_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  h->last_stream = s;
  if (launch_stats_total(h->lay, reset, stream) != 0 ||
      hipMemcpyAsync(totals, h->lay.stats_total, kStatFields * 8, hipMemcpyDeviceToHost, s) != hipSuccess) {
    h->poisoned = 1;
    return CONFKV_EHIP;
  }
  return device_status(h);
}

CONFKV_API int confkv_profile(confkv_handle* h, int32_t enable) {
  if (!live(h)) return CONFKV_ESTATE;
  if (enable < 0 || enable > CONFKV_PROFILE_ALL) return CONFKV_EINVAL;
  h->prof = enable;
  return CONFKV_OK;
}

CONFKV_API int confkv_profile_read(confkv_handle* h, double* fused_ms, int64_t* fused_launches, double* reduce_ms,
                                   int64_t* reduce_launches, int32_t reset) {
  if (!live(h)) return CONFKV_ESTATE;
  if (collect(h->pf) || collect(h->pr)) {
    h->poisoned = 1;
    return CONFKV_EHIP;
  }
  if (fused_ms) *fused_ms = h->pf.ms;
  if (fused_launches) *fused_launches = h->pf.n;
  if (reduce_ms) *reduce_ms = h->pr.ms;
  if (reduce_launches) *reduce_launches = h->pr.n;
  if (reset) {
    h->pf.ms = h->pr.ms = 0.0;
    h->pf.n = h->pr.n = 0;
  }
  return CONFKV_OK;
}

CONFKV_API int confkv_profile_kernel(confkv_handle* h, int32_t kernel, double* ms, int64_t* launches,
                                    int32_t reset) {
  if (!live(h)) return CONFKV_ESTATE;
  EventPool* pools[4] = {&h->pf, &h->pr, &h->pa, &h->pe};
  if (kernel < 0 || kernel > 3) return CONFKV_EINVAL;
  EventPool& p = *pools[kernel];
  if (collect(p)) {
    h->poisoned = 1;
    return CONFKV_EHIP;
  }
  if (ms) *ms = p.ms;
  if (launches) *launches = p.n;
  if (reset) {
    p.ms = 0.0;
    p.n = 0;
  }
  return CONFKV_OK;
}

CONFKV_API int confkv_bandwidth_probe(void* stream, const void* src, void* dst, size_t bytes, int32_t copy) {
  if (!src || !dst || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return CONFKV_EINVAL;
  if (bytes < 16 || (bytes & 15) || (copy != 0 && copy != 1)) return CONFKV_EINVAL;
  return launch_stream_probe(src, dst, bytes, copy, stream) == 0 ? CONFKV_OK : CONFKV_EHIP;
}

CONFKV_API int64_t confkv_position(const confkv_handle* h) { return live(h) ? h->t : -1; }

CONFKV_API int confkv_status(confkv_handle* h) {
  if (!live(h)) return CONFKV_ESTATE;
  return device_status(h);
}

CONFKV_API int confkv_destroy(confkv_handle* h) {
  if (!h) return CONFKV_OK;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_live.erase(h)) return CONFKV_ESTATE;
  }
  for (hipEvent_t e : h->pf.ev) (void)hipEventDestroy(e);
  for (hipEvent_t e : h->pr.ev) (void)hipEventDestroy(e);
  for (hipEvent_t e : h->pa.ev) (void)hipEventDestroy(e);
  for (hipEvent_t e : h->pe.ev) (void)hipEventDestroy(e);
  h->magic = kDead;
  delete h;
  return CONFKV_OK;
}

CONFKV_API const char* confkv_strerror(int code) {
  switch (code) {
    case CONFKV_OK: return "ok";
    case CONFKV_EINVAL: return "invalid argument, shape or configuration";
    case CONFKV_ECAPACITY: return "capacity or state buffer too small";
    case CONFKV_EHIP: return "HIP runtime error";
    case CONFKV_ENONFINITE: return "non-finite logits or ranking score";
    case CONFKV_ESTATE: return "handle destroyed or poisoned by an earlier error";
    default: return "unknown status code";
  }
}
