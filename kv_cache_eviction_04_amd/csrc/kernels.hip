// HIP kernels for gfx950 (MI355X): one decode step of confidence-gated KV
// eviction (CONF-KV) and its KVpop fixed-budget variant.
//
// Kernels
//   conf_reduce_kernel  logits -> (max, sum e, sum e*(z-m), top1, top2) per
//                       chunk; each segment workgroup merges its row's
//                       chunks into the confidence c and the base budget.
//   fused_step_kernel   one workgroup per segment (layer, batch row, KV head):
//                       append -> QK on MFMA -> max -> exp/sum -> PV on MFMA
//                       -> out -> mass/EMA/score/key -> select -> compact ->
//                       age-out; also the attend-only and evict-only halves.
//   init / ingest       zero the state and store the prefill.
//   read_cache          logical (ascending position) read-out for checking.
// The split-K attend, the next-token draw and the KVpop prefill live in
// split_attend.hip, sample.hip and kvpop_prefill.hip.
//
// Sources: "Conf-KV" post (rcap.io), method paragraph and decoding-loop
// pseudocode; CONF-KV abstract (chatpaper.ai); "Resumen Técnico: KVpop"
// (gist.science) §2.1, §2.3, §2.4.
#include "device.h"

namespace confkv {

// ======================================================= logits -> confidence
// [Conf-KV post, pseudocode] p = softmax(logits); c mixes the normalized
// entropy, sigmoid of the top-2 log-prob gap and p_max. Per chunk (reducer
// kernel): M = max z, S = sum e^(z-M), T = sum e^(z-M)(z-M) (fp64
// accumulation of fp32 exponentials), top-2 values. Merged over chunks (by
// each segment of the row) with M* = max M_c:
//   S* = sum S_c e^(M_c-M*),  T* = sum e^(M_c-M*) (T_c + (M_c-M*) S_c),
// so H = log S* - T*/S*, p_max = 1/S*, margin = top1 - top2.
__device__ __forceinline__ void top2_merge(float& a1, float& a2, float b1, float b2) {
  const float hi = fmaxf(a1, b1), lo = fminf(a1, b1);
  a2 = fmaxf(lo, fmaxf(a2, b2));
  a1 = hi;
}

// One workgroup per (chunk, batch row): the chunk's partial (M, S, T, top-2,
// non-finite flag). The segments of the row merge the partials themselves.
__global__ void __launch_bounds__(256) conf_reduce_kernel(Layout lay, const float* logits) {
  __shared__ float s_t1[4], s_t2[4];
  __shared__ double s_S[4], s_T[4];
  __shared__ uint32_t s_bad[4];
  const int b = blockIdx.y, ci = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int V = lay.V;
  const float* z = logits + (size_t)b * V;
  const int begin = ci * kChunk, end = min(V, begin + kChunk);

  // all 16 loads first (index clamped into the chunk), then the arithmetic
  float x[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) x[j] = z[min(begin + tid + 256 * j, end - 1)];
  float t1 = -INFINITY, t2 = -INFINITY;
  uint32_t bad = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const bool in = begin + tid + 256 * j < end;
    const bool fin = isfinite(x[j]);
    bad |= (in && !fin) ? 1u : 0u;
    x[j] = (in && fin) ? x[j] : -INFINITY;
    t2 = fmaxf(t2, fminf(t1, x[j]));
    t1 = fmaxf(t1, x[j]);
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float o1 = __shfl_xor(t1, o, 64), o2 = __shfl_xor(t2, o, 64);
    top2_merge(t1, t2, o1, o2);
    bad |= __shfl_xor(bad, o, 64);
  }
  if (lane == 0) {
    s_t1[wave] = t1;
    s_t2[wave] = t2;
    s_bad[wave] = bad;
  }
  __syncthreads();
  float M = s_t1[0], M2 = s_t2[0];
  for (int w = 1; w < 4; ++w) top2_merge(M, M2, s_t1[w], s_t2[w]);
  bad = s_bad[0] | s_bad[1] | s_bad[2] | s_bad[3];

  double S = 0.0, T = 0.0;
  if (M > -INFINITY) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float dz = x[j] - M;
      const float e = x[j] > -INFINITY ? expf(dz) : 0.0f;
      S += (double)e;
      T += e > 0.0f ? (double)e * (double)dz : 0.0;
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    S += __shfl_xor(S, o, 64);
    T += __shfl_xor(T, o, 64);
  }
  if (lane == 0) {
    s_S[wave] = S;
    s_T[wave] = T;
  }
  __syncthreads();
  if (tid == 0) {
    ConfPartial P;
    P.S = s_S[0] + s_S[1] + s_S[2] + s_S[3];
    P.T = s_T[0] + s_T[1] + s_T[2] + s_T[3];
    P.m = M;
    P.top2 = M2;
    P.nonfinite = bad;
    P.pad = 0;
    lay.partials[(size_t)b * lay.chunks + ci] = P;
  }
}

// Merge of a batch row's chunk partials by one wave (partial c on lane c % 64,
// the first 64 preloaded into `first`), then c and the step's base budget for
// every lane. The chunk sums were accumulated in fp64; the merge and the final
// terms run in fp32, whose error (~1e-7 on c) is far below what the gate
// needs: H = log S + E[M - z] adds two non-negative terms, so nothing cancels.
// A non-finite logit or confidence raises the error and takes the larger
// budget.
__device__ __forceinline__ void mst_merge_f(float& pm, float& pS, float& pT, float qm, float qS, float qT) {
  if (qm == -INFINITY) return;
  const float mx = fmaxf(pm, qm);
  const float f1 = pm > -INFINITY ? expf(pm - mx) : 0.0f, f2 = expf(qm - mx);
  pT = f1 * (pT + (pm > -INFINITY ? (pm - mx) * pS : 0.0f)) + f2 * (qT + (qm - mx) * qS);
  pS = f1 * pS + f2 * qS;
  pm = mx;
}
__device__ __forceinline__ void row_confidence(const Layout& lay, const Params& par, int b, int lane,
                                               const ConfPartial& first, float& c_out, int& base_out) {
  const ConfPartial* parts = lay.partials + (size_t)b * lay.chunks;
  float a1 = -INFINITY, a2 = -INFINITY;
  float pm = -INFINITY, pS = 0.0f, pT = 0.0f;
  uint32_t badall = 0;
  for (int c0 = 0; c0 < lay.chunks; c0 += 64) {
    const int c = c0 + lane;
    if (c < lay.chunks) {
      const ConfPartial P = c0 == 0 ? first : parts[c];
      badall |= P.nonfinite;
      top2_merge(a1, a2, P.m, P.top2);
      mst_merge_f(pm, pS, pT, P.m, (float)P.S, (float)P.T);
    }
  }
  // lanes >= chunks hold empty partials; with at most 32 chunks the upper
  // half of the wave has nothing to contribute
  for (int o = lay.chunks > 32 ? 32 : 16; o > 0; o >>= 1) {
    const float o1 = __shfl_xor(a1, o, 64), o2 = __shfl_xor(a2, o, 64);
    top2_merge(a1, a2, o1, o2);
    badall |= __shfl_xor(badall, o, 64);
    const float qm = __shfl_xor(pm, o, 64), qS = __shfl_xor(pS, o, 64), qT = __shfl_xor(pT, o, 64);
    mst_merge_f(pm, pS, pT, qm, qS, qT);
  }
  const float H = logf(pS) - pT / pS;
  const float Hn = H / logf((float)lay.V);
  const float sig = 1.0f / (1.0f + expf(-(a1 - a2)));
  const float cval = par.w_e * (1.0f - Hn) + par.w_m * sig + par.w_p * (1.0f / pS);
  if (badall || !isfinite(cval)) {
    if (lane == 0) atomicOr(lay.err, kErrNonFinite);
    base_out = max(par.n_low, par.n_high);
    c_out = NAN;
  } else {
    const bool confident = cval >= par.tau;
    if (par.gate_literal)
      base_out = confident ? par.n_high : par.n_low;
    else
      base_out = confident ? min(par.n_low, par.n_high) : max(par.n_low, par.n_high);
    c_out = cval;
  }
}

template <bool kLds>
struct Stage {
  float* p;
  int rs;  // row stride of a plane (a multiple of 32)
  __device__ __forceinline__ float& at(int plane, int i) const { return p[plane * rs + i]; }
  __device__ __forceinline__ const float4& at4(int plane, int i) const {
    return *reinterpret_cast<const float4*>(p + plane * rs + i);
  }
  __device__ __forceinline__ uint64_t key(int i) const {
    return ((uint64_t)__builtin_bit_cast(uint32_t, p[rs + i]) << 32) | __builtin_bit_cast(uint32_t, p[i]);
  }
  __device__ __forceinline__ void set_key(int i, uint64_t k) const {
    p[i] = __builtin_bit_cast(float, (uint32_t)k);
    p[rs + i] = __builtin_bit_cast(float, (uint32_t)(k >> 32));
  }
  __device__ __forceinline__ int32_t* list(int plane) const { return reinterpret_cast<int32_t*>(p + plane * rs); }
};

// Walks over the staged keys. An HBM-staged key costs a memory round trip, so
// that instance loads 8 keys of a thread before using them; one at a time, a
// thread's walk over a 32K-row segment would be some 128 round trips in a
// row. f(i, key) is called in ascending i within a thread.
template <bool kLds>
constexpr int kKeyBatch = kLds ? 1 : 8;
// rows i = tid, tid + 256, ... below n
template <bool kLds, class F>
__device__ __forceinline__ void for_keys(const Stage<kLds>& st, int n, F&& f) {
  constexpr int U = kKeyBatch<kLds>;
  for (int i0 = threadIdx.x; i0 < n; i0 += kThreads * U) {
    uint64_t k[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + kThreads * u;
      k[u] = i < n ? st.key(i) : ~0ull;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i0 + kThreads * u < n) f(i0 + kThreads * u, k[u]);
  }
}
// rows lo .. hi-1, in order
template <bool kLds, class F>
__device__ __forceinline__ void for_keys_range(const Stage<kLds>& st, int lo, int hi, F&& f) {
  constexpr int U = kKeyBatch<kLds>;
  for (int i0 = lo; i0 < hi; i0 += U) {
    uint64_t k[U];
#pragma unroll
    for (int u = 0; u < U; ++u) k[u] = i0 + u < hi ? st.key(i0 + u) : ~0ull;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i0 + u < hi) f(i0 + u, k[u]);
  }
}

// The e-th smallest key (e >= 1) over keys [0, rows): an 8-bit-digit radix
// select from the most significant digit down. Keys are unique, so once the
// selected digit's bin holds a single key, that key is the answer and one
// minimum pass over the keys under the prefix finds it.
template <bool kLds>
__device__ uint64_t radix_select(const Stage<kLds>& st, int rows, uint32_t e, uint32_t* hist, uint32_t* red,
                                 int32_t* sh, uint64_t* red64) {
  uint64_t prefix = 0, mask = 0;
  const int tid = threadIdx.x;
  for (int shift = 56; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for_keys(st, rows, [&](int, uint64_t k) {
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    });
    __syncthreads();
    const uint32_t cnt = hist[tid];
    uint32_t total;
    const uint32_t excl = block_excl_scan_u32(cnt, red, &total);
    if (excl < e && e <= excl + cnt) {
      sh[0] = tid;
      sh[1] = (int32_t)excl;
      sh[2] = (int32_t)cnt;
    }
    __syncthreads();
    const uint32_t bin = (uint32_t)sh[0];
    e -= (uint32_t)sh[1];
    prefix |= (uint64_t)bin << shift;
    mask |= (uint64_t)0xFFu << shift;
    const bool single = sh[2] == 1;
    __syncthreads();
    if (single && shift > 0) {
      uint64_t mk = ~0ull;
      for_keys(st, rows, [&](int, uint64_t k) {
        if ((k & mask) == prefix && k < mk) mk = k;
      });
      return block_min_u64(mk, red64);
    }
  }
  return prefix;
}

// Count bin in the histogram h for the calling lanes: lanes whose bin equals
// the first active lane's add together with one atomic (neighbouring rows
// usually share a bin), the others one by one.
__device__ __forceinline__ void hist_add(uint32_t* h, uint32_t bin) {
  const uint32_t b0 = __builtin_amdgcn_readfirstlane(bin);
  const uint64_t same = __ballot(bin == b0);
  if (bin == b0) {
    if ((int)(threadIdx.x & 63) == __ffsll((unsigned long long)same) - 1)
      atomicAdd(&h[b0], (uint32_t)__popcll(same));
  } else {
    atomicAdd(&h[bin], 1u);
  }
}

// Bits [0, x) of a 32-bit word (x clamped to 0 .. 32).
__device__ __forceinline__ uint32_t bits_below(int x) {
  return x <= 0 ? 0u : (x >= 32 ? ~0u : (1u << x) - 1u);
}

// One workgroup per segment. Stage-row index space: old rows [0, n_old32)
// (rows >= n_old are padding), ring slots [n_old32, n_old32 + Wr32).
template <int D, int G, bool kLds, int MODE>
__global__ void __launch_bounds__(kThreads, (G <= 5 ? CONFKV_OCC : 3)) fused_step_kernel(Layout lay, Params par, StepArgs a) {
  constexpr bool kAtt = MODE != kModeEvict;  // append, attention, output (and the EMA update)
  constexpr bool kEv = MODE != kModeAttend;  // keys, selection, compaction, age-out
  constexpr int LPR = D / 16;          // lanes per row for row-wise work
  constexpr int RPB = kThreads / LPR;  // rows per block iteration for row-wise work
  constexpr int KS = D / 32;           // MFMA k-steps over d
  constexpr int NCB = D / 16;          // 16-column blocks of d
  constexpr int PL = G > 4 ? G : 4;    // staging planes
  constexpr int CBW = NCB / 4;         // PV column blocks per wave (waves split d)
  constexpr int NP8 = 4;               // 16-row INT8 K tiles in flight per wave
  constexpr int NP16 = 2;              // 16-row FP16 K tiles in flight per wave
  constexpr int NV8 = 8;               // 32-row INT8 V tiles in flight per wave
  constexpr int NV16 = 4;              // 32-row FP16 V tiles in flight per wave
  constexpr int KB = !kLds ? CONFKV_KB_HBM : (G <= 4 ? CONFKV_KB : CONFKV_KB_WIDE);  // rows per thread in flight in the key phase
  static_assert(LPR == 4 || LPR == 8, "head_dim 64 or 128");
  static_assert(G <= 16, "a GQA group fits one MFMA tile");

  __shared__ float red_m[4][G], red_l[4][G];
  __shared__ uint32_t red_u[4];
  __shared__ uint64_t red_k[4];
  __shared__ uint32_t hist[256];
  __shared__ int32_t sh[8];
  __shared__ int32_t sh_out_live, sh_base;
  __shared__ uint32_t sh_cand;  // HBM-staged selection: candidates gathered
  __shared__ float sh_mrun[G], sh_lrun[G];  // HBM-staged attention: running maxima and sums
  __shared__ uint32_t sel_cnt[4][2];  // per wave: live rows, eligible rows
  __shared__ uint64_t sel_key[4];     // per wave: smallest key
  __shared__ int32_t sel_row[4];      // per wave: its stage row
  extern __shared__ __attribute__((aligned(16))) float dyn_lds[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid % LPR, rg = tid / LPR;
  const int lq = lane >> 4, lj = lane & 15;  // MFMA lane coordinates
  // Attend launches cover one layer (segments seg0 .. seg0 + B*Hkv - 1, its
  // inputs indexed from 0); the other modes cover every segment.
  const int si = blockIdx.x;
  const int seg = MODE == kModeAttend ? a.seg0 + si : si;
  const int b = (seg / lay.Hkv) % lay.B, l = seg / (lay.Hkv * lay.B);
  const int t = a.t, Wr = lay.Wr, Wr32 = lay.Wr32, ob = lay.old_bytes;
  const bool kvpop = par.policy == 1;

  uint16_t* rk = lay.ring_k + (size_t)seg * Wr32 * D;
  uint16_t* rvt = lay.ring_v + (size_t)seg * Wr32 * D;
  const size_t obase = (size_t)seg * lay.cap32;
  uint8_t* okp = lay.old_k + obase * D * ob;
  uint8_t* ovt = lay.old_v + obase * D * ob;
  float* oks = lay.old_ks + obase;
  float* ovs = lay.old_vs + obase;
  const size_t sbase = (size_t)seg * lay.rows_max;  // row state: old rows, then ring slots at cap32
  int32_t* opos = lay.row_pos + sbase;
  float* oema = lay.row_ema + sbase;
  float* oprio = lay.row_prio + sbase;
  int32_t* rpos = opos + lay.cap32;
  float* rema = oema + lay.cap32;
  float* rprio = oprio + lay.cap32;

  // The host sizes the LDS planes for the most rows a segment can hold. Should
  // a segment hold more, the step is computed on a clamped row count (every
  // access stays in bounds) and an internal error is raised at the end; the
  // state is then invalid and every later call refuses to run.
  const int n_old_raw = lay.seg_nold[seg];
  const int n_old = kLds ? min(n_old_raw, a.lds_rows - Wr32) : n_old_raw;
  const int n_old32 = (n_old + 31) & ~31;
  const int rows = n_old32 + Wr32;
  Stage<kLds> st;
  if constexpr (kLds) {
    st.p = dyn_lds;
    st.rs = a.lds_rows;
  } else {
    st.p = lay.stage + (size_t)seg * lay.planes * lay.rows_max;
    st.rs = lay.rows_max;
  }
  // HBM-staged selection: the key histogram (later the candidates) in LDS and
  // the victim bitmask, in LDS after it or else in the upper half of stage
  // plane 2 (the compaction's hole list, at most half the old rows, sits in
  // the lower half).
  uint32_t* const hsel = reinterpret_cast<uint32_t*>(dyn_lds);
  uint32_t* vbits = nullptr;
  if constexpr (!kLds && kEv)
    vbits = a.sel_bits_lds ? hsel + kSelBins : reinterpret_cast<uint32_t*>(st.p + 2 * st.rs + st.rs / 2);

  // The new row (pos t) goes to ring slot t mod Wr; the row at t - W leaves
  // the FP16 window at the end of the step; under KVpop the row at t - w gets
  // its priority now.
  const int slot_new = t % Wr;
  const int pos_out = t - lay.W;
  const int pos_prio = (kvpop && t - par.P >= par.s) ? t - par.P : -1;
  float prio_now = 0.0f;

  // rows of this thread in flight in the weight and key passes
  int32_t kpos[KB];
  float kev[KB], ksv[KB];
  // Row state of stage row i sits at one index of the unified row arrays
  // (old row i, or ring slot i - n_old32 at cap32 + slot), so every row issues
  // the same three loads with no branch between them; padding rows read valid
  // padding entries and are masked after. Slots in which no row of the wave
  // is below the stage-row count are not loaded (nothing reads them).
  const float* uev = kvpop ? oprio : oema;
  auto load_rows = [&](int i0) {
    const int wrow0 = i0 - tid + 64 * wave;  // the wave's first row of slot 0
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (wrow0 + kThreads * u >= rows) break;  // no row of the wave in this slot or later ones
      const int i = i0 + kThreads * u;
      const int r = i - n_old32;
      const int ix = r < 0 ? i : lay.cap32 + min(r, Wr32 - 1);
      kpos[u] = opos[ix];
      kev[u] = uev[ix];
      if constexpr (kAtt && kLds) ksv[u] = ovs[min(i, lay.cap32 - 1)];  // V scales: LDS-staged weights only
    }
  };
  // HBM-staged attention: the raw scores of the same rows, for their mass
  float ksc[kLds ? 1 : KB][G];
  auto load_scores = [&](int i0) {
    if constexpr (!kLds && kAtt) {
      const int wrow0 = i0 - tid + 64 * wave;
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        if (wrow0 + kThreads * u >= rows) break;
        const int i = min(i0 + kThreads * u, rows - 1);
#pragma unroll
        for (int g = 0; g < G; ++g) ksc[u][g] = st.at(g, i);
      }
    }
  };
  // the raw loaded state of stage row i, masked: position (-1: no row), EMA or
  // priority. Until the attend pass has stored the new row's state (an evict
  // launch comes after it), the new row and the delayed priority are
  // substituted here.
  auto row_state = [&](int i, int32_t pl, float el, int32_t& p, float& ev) {
    const int r = i - n_old32;
    const bool is_old = i < n_old, is_ring = r >= 0 && r < Wr;
    if constexpr (MODE == kModeEvict) {
      p = (is_old || is_ring) ? pl : -1;
      ev = el;
    } else {
      p = is_old ? pl : (is_ring ? (r == slot_new ? t : pl) : -1);
      ev = (is_old || (is_ring && r != slot_new)) ? el : 0.0f;
      if (kvpop && is_ring && p == pos_prio && p >= 0) ev = prio_now;
    }
  };
  auto row_scale = [&](int i, float sv) { return (i < n_old && par.old_int8 && sv > 0.0f) ? sv : 1.0f; };
  float inv_l[G];  // 1 / sum of p per head (attention)
  float Mf[G];     // HBM-staged: the final maximum score per head
  float finv = 1.0f;  // 1 / the power-of-two prescale of the PV weights
  if constexpr (!kAtt) {
    if (tid == 0) sh_out_live = 0;
  }

  if constexpr (kAtt) {
    // ---- q as MFMA A operands (row g = lane%16; zero rows g >= G). INT8 K tiles
    // take d in the order their 16-byte loads deliver it, FP16 tiles in theirs.
    const uint16_t* qrow = a.q + ((size_t)si * G + (lj < G ? lj : 0)) * D;
    half8 qa8[KS], qa16[KS];
    auto load_q16 = [&]() {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const uint4 u16 = *reinterpret_cast<const uint4*>(qrow + 8 * (lq + 4 * kk));
        qa16[kk] = lj < G ? as_h8(u16) : half8{};
      }
    };
    auto load_q8 = [&]() {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const uint4 u8 = *reinterpret_cast<const uint4*>(qrow + 16 * (lq + 4 * (kk >> 1)) + 8 * (kk & 1));
        qa8[kk] = lj < G ? as_h8(u8) : half8{};
      }
    };
    if constexpr (kLds) load_q16();

    // ---- the new row (pos t): its data is loaded now and appended to the ring
    // after the ring QK (below), so these loads do not hold up the first tiles.
    // (The HBM-staged variant loads it when it appends the row.)
    const uint16_t* kn = a.k_new + (size_t)si * D;
    if (pos_prio >= 0) prio_now = a.prio_new[si];
    uint4 kn4 = uint4{0u, 0u, 0u, 0u};
    uint16_t vn1 = 0;
    auto load_new_row = [&]() {
      kn4 = reinterpret_cast<const uint4*>(kn)[tid % (D / 8)];
      vn1 = a.v_new[(size_t)si * D + tid % D];
    };
    if constexpr (kLds) load_new_row();
    const int32_t pos_prio_slot = pos_prio >= 0 ? rpos[pos_prio % Wr] : -1;

    // ---- append the new row (pos t, ema 0) into ring slot t mod Wr. The slot's
    // previous row (pos t - Wr) left the window at the end of the last step.
    // Nothing reads these stores back before a barrier: the ring QK takes the
    // new row's K from k_new, and the row-state passes substitute its position,
    // EMA and (KVpop) the delayed priority.
    auto append_row = [&]() {
      if (tid < D / 8) reinterpret_cast<uint4*>(rk + (size_t)slot_new * D)[tid] = kn4;
      if (tid < D) rvt[vt16(slot_new, tid, D)] = vn1;
      if (tid == 0) {
        rpos[slot_new] = t;
        rema[slot_new] = 0.0f;
        rprio[slot_new] = 0.0f;
        // [KVpop summary §2.3] delayed scoring: the row at t - w gets its
        // priority now, as it stops being protected.
        if (pos_prio >= 0 && pos_prio_slot == pos_prio) rprio[pos_prio % Wr] = prio_now;
        sh_out_live = 0;
      }
    };

    // ---- PV on MFMA over 32-row tiles: O[g][col] += sum_row w[g][row] V[row][col]
    // with A = w as its fp16 hi and lo parts and B = V from the transposed
    // tiles; lane (lq, lj) receives O[4*lq + r][16*cb + lj]. Waves split the
    // columns: wave w owns column blocks CBW*w .. CBW*w+CBW-1 and streams every
    // row, so no cross-wave reduction is needed.
    // The weights of 8 consecutive rows of head lj (lanes lj < G; zero for the
    // others), stored as fp16 (hi | lo << 16) pairs, into hi and lo A operands.
    auto wpack = [&](const float4& p0, const float4& p1, half8& ahi, half8& alo) {
      const uint32_t wd[8] = {__builtin_bit_cast(uint32_t, p0.x), __builtin_bit_cast(uint32_t, p0.y),
                              __builtin_bit_cast(uint32_t, p0.z), __builtin_bit_cast(uint32_t, p0.w),
                              __builtin_bit_cast(uint32_t, p1.x), __builtin_bit_cast(uint32_t, p1.y),
                              __builtin_bit_cast(uint32_t, p1.z), __builtin_bit_cast(uint32_t, p1.w)};
      uint4 h, lw;
      h.x = __builtin_amdgcn_perm(wd[1], wd[0], 0x05040100u);
      h.y = __builtin_amdgcn_perm(wd[3], wd[2], 0x05040100u);
      h.z = __builtin_amdgcn_perm(wd[5], wd[4], 0x05040100u);
      h.w = __builtin_amdgcn_perm(wd[7], wd[6], 0x05040100u);
      lw.x = __builtin_amdgcn_perm(wd[1], wd[0], 0x07060302u);
      lw.y = __builtin_amdgcn_perm(wd[3], wd[2], 0x07060302u);
      lw.z = __builtin_amdgcn_perm(wd[5], wd[4], 0x07060302u);
      lw.w = __builtin_amdgcn_perm(wd[7], wd[6], 0x07060302u);
      ahi = as_h8(h);
      alo = as_h8(lw);
    };
    // V tiles: a lane loads 8 consecutive rows (lane group lq); lanes whose
    // rows all lie past the region's nvalid rows read lane group 0's (same
    // lines, no traffic), and their weights are 0.
    auto vload16 = [&](const uint16_t* vbase, int nvalid, int tt, PV16Buf<CBW>& bf) {
      const uint16_t* tb = vbase + (size_t)tt * 32 * D + 8 * (32 * tt + 8 * lq < nvalid ? lane : lj);
#pragma unroll
      for (int k = 0; k < CBW; ++k) bf.v[k] = ldnt4(tb + 512 * (CBW * wave + k));
    };
    auto load_pv8 = [&](int tt, PV8Buf& bf) {
      const uint8_t* tb = ovt + (size_t)tt * 32 * D + 16 * (32 * tt + 8 * lq < n_old ? lane : lj);
      if constexpr (CBW == 2) {
        bf.v = ldnt4(tb + 1024 * wave);
      } else {
        const uint2 h = ldnt2(tb + 1024 * (wave >> 1) + 8 * (wave & 1));
        bf.v = make_uint4(h.x, h.y, 0u, 0u);
      }
    };
    auto mm16 = [&](floatx4(&acc)[CBW], const PV16Buf<CBW>& bf, const half8& ahi, const half8& alo) {
#pragma unroll
      for (int k = 0; k < CBW; ++k) {
        acc[k] = mfma16(ahi, as_h8(bf.v[k]), acc[k]);
        acc[k] = mfma16(alo, as_h8(bf.v[k]), acc[k]);
      }
    };
    auto mm8 = [&](floatx4(&acc)[CBW], const PV8Buf& bf, const half8& ahi, const half8& alo) {
      half8 blo, bhi;
      i8x16_to_h8(bf.v, blo, bhi);
      acc[0] = mfma16(ahi, blo, acc[0]);
      acc[0] = mfma16(alo, blo, acc[0]);
      if constexpr (CBW == 2) {
        acc[1] = mfma16(ahi, bhi, acc[1]);
        acc[1] = mfma16(alo, bhi, acc[1]);
      }
    };
    const float sm = par.sm_scale;

    if constexpr (kLds) {
    // ---- QK on MFMA: S[g][row] = sum_d q[g][d] K[row][d] for 16-row tiles;
    // lane (lq, lj) receives S[4*lq + r][row lj]. The ring goes first (its
    // tiles do not depend on the old-region count), then the old region. Each
    // wave takes a contiguous share of the tiles, stages s in LDS and keeps a
    // running max per head.
    float mrun[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    float sv_max = 0.0f;
    {
      const int nt_ring = (Wr + 15) >> 4;  // tiles wholly past slot Wr-1 are skipped
      const int ta = (wave * nt_ring) >> 2, tb = ((wave + 1) * nt_ring) >> 2;
      pipelined<CONFKV_QK16_NPB, QK16Buf<KS>>(
          ta, tb,
          [&](int tt, QK16Buf<KS>& bf) {
            const int r = 16 * tt + lj;
            // lanes past the last slot read the tile's first row (same lines, no traffic)
            const uint16_t* kr = r == slot_new ? kn : rk + (size_t)(r < Wr ? r : 16 * tt) * D;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) bf.kc[kk] = ldnt4(kr + 8 * (lq + 4 * kk));
            bf.pr = rpos[r];
          },
          [&](int tt, const QK16Buf<KS>& bf) {
            floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) acc = mfma16(qa16[kk], as_h8(bf.kc[kk]), acc);
            const int r = 16 * tt + lj;
            const bool valid = r < Wr && (bf.pr >= 0 || r == slot_new);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int g = 4 * lq + rr;
              if (g < G) {
                const float sc = valid ? acc[rr] * sm : -INFINITY;
                st.at(g, n_old32 + r) = sc;
                mrun[rr] = fmaxf(mrun[rr], sc);
              }
            }
          });
      // ring slots past the last QK tile
      for (int r = tid + 16 * nt_ring; r < Wr32; r += kThreads)
#pragma unroll
        for (int g = 0; g < G; ++g) st.at(g, n_old32 + r) = -INFINITY;
    }
    append_row();

    // 16-row tiles holding at least one old row; lanes past the last row read
    // the tile's first row, and a trailing tile without rows is not read
    const int nt_old = (n_old + 15) >> 4;
    for (int i = 16 * nt_old + tid; i < n_old32; i += kThreads)
#pragma unroll
      for (int g = 0; g < G; ++g) st.at(g, i) = -INFINITY;
    {
      const int ta = (wave * nt_old) >> 2, tb = ((wave + 1) * nt_old) >> 2;
      if (par.old_int8) {
        load_q8();
        pipelined<CONFKV_QK8_NPB, QK8Buf>(
            ta, tb,
            [&](int tt, QK8Buf& bf) {
              const int row = 16 * tt + lj, rl = row < n_old ? row : 16 * tt;
              const uint8_t* kr = okp + (size_t)rl * D;
              bf.k0 = ldnt4(kr + 16 * lq);
              if constexpr (D == 128) bf.k1 = ldnt4(kr + 16 * (lq + 4));
              bf.sk = oks[rl];
              bf.sv = ovs[rl];
            },
            [&](int tt, const QK8Buf& bf) {
              half8 b0, b1;
              floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
              i8x16_to_h8(bf.k0, b0, b1);
              acc = mfma16(qa8[0], b0, acc);
              acc = mfma16(qa8[1], b1, acc);
              if constexpr (D == 128) {
                half8 b2, b3;
                i8x16_to_h8(bf.k1, b2, b3);
                acc = mfma16(qa8[2], b2, acc);
                acc = mfma16(qa8[3], b3, acc);
              }
              const int row = 16 * tt + lj;
              const bool valid = row < n_old;
              sv_max = fmaxf(sv_max, valid ? bf.sv : 0.0f);
              const float f = bf.sk * sm;
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int g = 4 * lq + r;
                if (g < G) {
                  const float sc = valid ? acc[r] * f : -INFINITY;
                  st.at(g, row) = sc;
                  mrun[r] = fmaxf(mrun[r], sc);
                }
              }
            });
      } else {
        pipelined<CONFKV_QK16_NPB, QK16Buf<KS>>(
            ta, tb,
            [&](int tt, QK16Buf<KS>& bf) {
              const int row = 16 * tt + lj, rl = row < n_old ? row : 16 * tt;
              const uint16_t* kr = reinterpret_cast<const uint16_t*>(okp) + (size_t)rl * D;
#pragma unroll
              for (int kk = 0; kk < KS; ++kk) bf.kc[kk] = ldnt4(kr + 8 * (lq + 4 * kk));
            },
            [&](int tt, const QK16Buf<KS>& bf) {
              floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
              for (int kk = 0; kk < KS; ++kk) acc = mfma16(qa16[kk], as_h8(bf.kc[kk]), acc);
              const int row = 16 * tt + lj;
              const bool valid = row < n_old;
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int g = 4 * lq + r;
                if (g < G) {
                  const float sc = valid ? acc[r] * sm : -INFINITY;
                  st.at(g, row) = sc;
                  mrun[r] = fmaxf(mrun[r], sc);
                }
              }
            });
      }
    }
    // per-head maxima: over the 16 lanes of each lane group, then per wave
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float m = mrun[r];
      m = row16_reduce(m, [](float x, float y) { return fmaxf(x, y); });
      const int g = 4 * lq + r;
      if (lj == 0 && g < G) red_m[wave][g] = m;
    }
    sv_max = wave_max(sv_max);
    if (lane == 0) red_u[wave] = __builtin_bit_cast(uint32_t, sv_max);

    load_rows(tid);
    __syncthreads();
    float M[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float m = red_m[0][g];
#pragma unroll
      for (int w = 1; w < 4; ++w) m = fmaxf(m, red_m[w][g]);
      M[g] = m;
    }
    float svm = 0.0f;
    for (int w = 0; w < 4; ++w) svm = fmaxf(svm, __builtin_bit_cast(float, red_u[w]));
    // PV weights are prescaled by a power of two that keeps p*sV*f below 2^14
    // (fp16 range) while lifting small weights out of the fp16 subnormals.
    int fexp = 10;
    if (svm > 0.0f) {
      int e2;
      frexpf(svm, &e2);
      fexp = min(10, max(-30, 14 - e2));
    }
    const float fscale = ldexpf(1.0f, fexp);
    finv = ldexpf(1.0f, -fexp);

    // ---- weight pass, once per (row, head): p = exp(s - M_g), l_g = sum p, and
    // the PV weight w = p * scale * f stored in place of s as an fp16 pair
    // (hi | lo << 16) with hi + lo = w to about 22 bits. scale is the row's V
    // scale for INT8 rows with a nonzero scale, else 1.
    float lpart[G];
#pragma unroll
    for (int g = 0; g < G; ++g) lpart[g] = 0.0f;
    for (int i0 = tid; i0 < rows; i0 += kThreads * KB) {
      if (i0 != tid) load_rows(i0);
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int i = i0 + kThreads * u;
        if (i < rows) {
          const float scf = row_scale(i, ksv[u]) * fscale;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float p = __expf(st.at(g, i) - M[g]);
            lpart[g] += p;
            const float wv = p * scf;
            const _Float16 hi = (_Float16)wv, lo = (_Float16)(wv - (float)hi);
            st.at(g, i) = __builtin_bit_cast(float, (uint32_t)__builtin_bit_cast(uint16_t, hi) |
                                                        ((uint32_t)__builtin_bit_cast(uint16_t, lo) << 16));
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float v = wave_sum(lpart[g]);
      if (lane == 0) red_l[wave][g] = v;
    }
    __syncthreads();
    float Lsum[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      Lsum[g] = red_l[0][g] + red_l[1][g] + red_l[2][g] + red_l[3][g];
      inv_l[g] = 1.0f / Lsum[g];
    }
    // 1/l of the output rows 4*lq + r (lane-varying head index: from LDS)
    float il4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int g = 4 * lq + r;
      if (g < G) il4[r] = 1.0f / (red_l[0][g] + red_l[1][g] + red_l[2][g] + red_l[3][g]);
    }

    // ---- PV from the LDS weights
    floatx4 O[CBW];
#pragma unroll
    for (int k = 0; k < CBW; ++k) O[k] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    auto wfrag = [&](int srow, half8& ahi, half8& alo) {
      float4 p0{0.0f, 0.0f, 0.0f, 0.0f}, p1{0.0f, 0.0f, 0.0f, 0.0f};
      if (lj < G) {
        p0 = st.at4(lj, srow);
        p1 = st.at4(lj, srow + 4);
      }
      wpack(p0, p1, ahi, alo);
    };
    auto pv16 = [&](const uint16_t* vbase, int srow0, int ntiles, int nvalid) {
      pipelined<CONFKV_PV16_NPB, PV16Buf<CBW>>(
          0, ntiles, [&](int tt, PV16Buf<CBW>& bf) { vload16(vbase, nvalid, tt, bf); },
          [&](int tt, const PV16Buf<CBW>& bf) {
            half8 ahi, alo;
            wfrag(srow0 + 32 * tt + 8 * lq, ahi, alo);
            mm16(O, bf, ahi, alo);
          });
    };
    const int nv_old = n_old32 >> 5;
    if (par.old_int8) {
      pipelined<CONFKV_PV8_NPB, PV8Buf>(0, nv_old, load_pv8, [&](int tt, const PV8Buf& bf) {
        half8 ahi, alo;
        wfrag(32 * tt + 8 * lq, ahi, alo);
        mm8(O, bf, ahi, alo);
      });
    } else {
      pv16(reinterpret_cast<const uint16_t*>(ovt), 0, nv_old, n_old);
    }
    pv16(rvt, n_old32, (Wr + 31) >> 5, Wr);
#pragma unroll
    for (int k = 0; k < CBW; ++k) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int g = 4 * lq + r;
        if (g < G) {
          const int col = 16 * (CBW * wave + k) + lj;
          a.out[((size_t)si * G + g) * D + col] = f2h(O[k][r] * finv * il4[r]);
        }
      }
    }
    if (par.record && tid == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) lay.rec_lse[(size_t)seg * G + g] = M[g] + logf(Lsum[g]);
    }
    } else {
    // ---- Segments too long for LDS staging stream through LDS in chunks of
    // CH rows: the old region's, then (after the new row is appended) the
    // ring's. Per chunk: QK on MFMA (scores into the LDS chunk, and into the
    // HBM stage for the key pass), the chunk's per-head maxima, the weights
    // p = exp(s - M) against the running maxima M, with the row's V scale and
    // a power-of-two prescale folded in, packed in place as fp16 hi/lo pairs,
    // and PV on MFMA from them. Online softmax: a chunk that raises a head's
    // maximum rescales that head's running sum and output rows by
    // exp(M_old - M_new). The output accumulates in units of the current
    // chunk's prescale: a new prescale rescales it by the ratio of the two
    // (a power of two, exact). The running maxima and sums, the same in every
    // thread, are kept in LDS (sh_mrun, sh_lrun).
    constexpr int CH = hbm_chunk_rows(G);
    float* const cs = dyn_lds;            // [G][CH] scores, then weights
    float* const cvs = dyn_lds + G * CH;  // [CH] V scale of each INT8 row (1 for the others)
    if (tid < G) {
      sh_mrun[tid] = -INFINITY;
      sh_lrun[tid] = 0.0f;
    }
    int fexp_run = 0;  // prescale exponent the output is held in
    floatx4 O[CBW];
#pragma unroll
    for (int k = 0; k < CBW; ++k) O[k] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    // stage rows [c0, c1) (multiples of 32) of the ring (slot r = row - n_old32) or of the old region
    auto run_chunk = [&](const bool ring, const int c0, const int c1) {
      const bool int8 = !ring && par.old_int8;
      // q in the order this region's K tiles deliver d, loaded per chunk (a
      // cache hit) so that no operand set stays live through the PV
      half8 qa[KS];
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const uint16_t* qp = int8 ? qrow + 16 * (lq + 4 * (kk >> 1)) + 8 * (kk & 1) : qrow + 8 * (lq + 4 * kk);
        const uint4 u = *reinterpret_cast<const uint4*>(qp);
        qa[kk] = lj < G ? as_h8(u) : half8{};
      }
      const int vend = ring ? min(c1, n_old32 + Wr) : min(c1, n_old);  // past the chunk's last row
      // 16-row tiles holding a row; the chunk's rows past them score -inf
      const int t0 = c0 >> 4, t1 = max(t0, (vend + 15) >> 4);
      for (int i = 16 * t1 + tid; i < c1; i += kThreads) {
#pragma unroll
        for (int g = 0; g < G; ++g) cs[g * CH + i - c0] = -INFINITY;
        cvs[i - c0] = 1.0f;
      }
      float mrun[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      float sv_max = 0.0f;
      auto put = [&](const floatx4& acc, int row, bool valid, float f) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int g = 4 * lq + r;
          if (g < G) {
            const float sc = valid ? acc[r] * f : -INFINITY;
            cs[g * CH + row - c0] = sc;
            st.at(g, row) = sc;
            mrun[r] = fmaxf(mrun[r], sc);
          }
        }
      };
      const int nt = t1 - t0;
      const int ta = t0 + ((wave * nt) >> 2), tb = t0 + (((wave + 1) * nt) >> 2);
      if (ring) {
        pipelined<CONFKV_QK16_NPB, QK16Buf<KS>>(
            ta, tb,
            [&](int tt, QK16Buf<KS>& bf) {
              const int r = 16 * tt + lj - n_old32;
              // lanes past the last slot read the tile's first slot (same lines, no traffic)
              const uint16_t* kr = r == slot_new ? kn : rk + (size_t)(r < Wr ? r : 16 * tt - n_old32) * D;
#pragma unroll
              for (int kk = 0; kk < KS; ++kk) bf.kc[kk] = ldnt4(kr + 8 * (lq + 4 * kk));
              bf.pr = rpos[r];
            },
            [&](int tt, const QK16Buf<KS>& bf) {
              floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
              for (int kk = 0; kk < KS; ++kk) acc = mfma16(qa[kk], as_h8(bf.kc[kk]), acc);
              const int r = 16 * tt + lj - n_old32;
              put(acc, 16 * tt + lj, r < Wr && (bf.pr >= 0 || r == slot_new), sm);
            });
      } else if (int8) {
        pipelined<CONFKV_QK8_NPB, QK8Buf>(
            ta, tb,
            [&](int tt, QK8Buf& bf) {
              const int row = 16 * tt + lj, rl = row < n_old ? row : 16 * tt;
              const uint8_t* kr = okp + (size_t)rl * D;
              bf.k0 = ldnt4(kr + 16 * lq);
              if constexpr (D == 128) bf.k1 = ldnt4(kr + 16 * (lq + 4));
              bf.sk = oks[rl];
              bf.sv = ovs[rl];
            },
            [&](int tt, const QK8Buf& bf) {
              half8 b0, b1;
              floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
              i8x16_to_h8(bf.k0, b0, b1);
              acc = mfma16(qa[0], b0, acc);
              acc = mfma16(qa[1], b1, acc);
              if constexpr (D == 128) {
                half8 b2, b3;
                i8x16_to_h8(bf.k1, b2, b3);
                acc = mfma16(qa[2], b2, acc);
                acc = mfma16(qa[3], b3, acc);
              }
              const int row = 16 * tt + lj;
              const bool valid = row < n_old;
              sv_max = fmaxf(sv_max, valid ? bf.sv : 0.0f);
              if (lq == 0) cvs[row - c0] = (valid && bf.sv > 0.0f) ? bf.sv : 1.0f;
              put(acc, row, valid, bf.sk * sm);
            });
      } else {
        pipelined<CONFKV_QK16_NPB, QK16Buf<KS>>(
            ta, tb,
            [&](int tt, QK16Buf<KS>& bf) {
              const int row = 16 * tt + lj, rl = row < n_old ? row : 16 * tt;
              const uint16_t* kr = reinterpret_cast<const uint16_t*>(okp) + (size_t)rl * D;
#pragma unroll
              for (int kk = 0; kk < KS; ++kk) bf.kc[kk] = ldnt4(kr + 8 * (lq + 4 * kk));
            },
            [&](int tt, const QK16Buf<KS>& bf) {
              floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
              for (int kk = 0; kk < KS; ++kk) acc = mfma16(qa[kk], as_h8(bf.kc[kk]), acc);
              const int row = 16 * tt + lj;
              put(acc, row, row < n_old, sm);
            });
      }
      // the chunk's maxima, the new running maxima and the rescale factors
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float m = row16_reduce(mrun[r], [](float x, float y) { return fmaxf(x, y); });
        const int g = 4 * lq + r;
        if (lj == 0 && g < G) red_m[wave][g] = m;
      }
      sv_max = wave_max(sv_max);
      if (lane == 0) red_u[wave] = __builtin_bit_cast(uint32_t, sv_max);
      __syncthreads();
      float Mn[G], corr[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mc = fmaxf(fmaxf(red_m[0][g], red_m[1][g]), fmaxf(red_m[2][g], red_m[3][g]));
        const float mo = sh_mrun[g];
        Mn[g] = fmaxf(mo, mc);
        corr[g] = Mn[g] == -INFINITY ? 1.0f : __expf(mo - Mn[g]);
      }
      float svm = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) svm = fmaxf(svm, __builtin_bit_cast(float, red_u[w]));
      // prescale keeping p*sV*f below 2^14 (fp16 range) while lifting small
      // weights out of the fp16 subnormals
      int fexp = 10;
      if (svm > 0.0f) {
        int e2;
        frexpf(svm, &e2);
        fexp = min(10, max(-30, 14 - e2));
      }
      const float fsc = ldexpf(1.0f, fexp), fratio = ldexpf(1.0f, fexp - fexp_run);
      fexp_run = fexp;
      // weights of the chunk's rows, in place
      float lpart[G];
#pragma unroll
      for (int g = 0; g < G; ++g) lpart[g] = 0.0f;
      for (int i = c0 + tid; i < c1; i += kThreads) {
        const int ii = i - c0;
        const float scf = (int8 ? cvs[ii] : 1.0f) * fsc;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float p = Mn[g] == -INFINITY ? 0.0f : __expf(cs[g * CH + ii] - Mn[g]);
          lpart[g] += p;
          const float wv = p * scf;
          const _Float16 hi = (_Float16)wv, lo = (_Float16)(wv - (float)hi);
          cs[g * CH + ii] = __builtin_bit_cast(float, (uint32_t)__builtin_bit_cast(uint16_t, hi) |
                                                          ((uint32_t)__builtin_bit_cast(uint16_t, lo) << 16));
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float v = wave_sum(lpart[g]);
        if (lane == 0) red_l[wave][g] = v;
      }
      __syncthreads();
      if (tid < G) {
        float c = 1.0f, m = -INFINITY;
#pragma unroll
        for (int g = 0; g < G; ++g)
          if (g == tid) {
            c = corr[g];
            m = Mn[g];
          }
        sh_lrun[tid] = sh_lrun[tid] * c + ((red_l[0][tid] + red_l[1][tid]) + (red_l[2][tid] + red_l[3][tid]));
        sh_mrun[tid] = m;
      }
      // the output rows 4*lq + r (a lane-dependent head) to the new maxima and prescale
      float c4[4] = {fratio, fratio, fratio, fratio};
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int g = 0; g < G; ++g)
          if (g == 4 * lq + r) c4[r] = corr[g] * fratio;
#pragma unroll
      for (int k = 0; k < CBW; ++k)
#pragma unroll
        for (int r = 0; r < 4; ++r) O[k][r] *= c4[r];
      auto wfrag = [&](int wl, half8& ahi, half8& alo) {  // chunk row wl
        float4 p0{0.0f, 0.0f, 0.0f, 0.0f}, p1{0.0f, 0.0f, 0.0f, 0.0f};
        if (lj < G) {
          p0 = *reinterpret_cast<const float4*>(cs + lj * CH + wl);
          p1 = *reinterpret_cast<const float4*>(cs + lj * CH + wl + 4);
        }
        wpack(p0, p1, ahi, alo);
      };
      if (ring) {
        const int rt0 = (c0 - n_old32) >> 5, rt1 = min((c1 - n_old32) >> 5, (Wr + 31) >> 5);
        pipelined<CONFKV_PV16_NPB, PV16Buf<CBW>>(
            rt0, rt1, [&](int tt, PV16Buf<CBW>& bf) { vload16(rvt, Wr, tt, bf); },
            [&](int tt, const PV16Buf<CBW>& bf) {
              half8 ahi, alo;
              wfrag(n_old32 + 32 * tt + 8 * lq - c0, ahi, alo);
              mm16(O, bf, ahi, alo);
            });
      } else if (int8) {
        pipelined<CONFKV_PV8_NPB, PV8Buf>(c0 >> 5, c1 >> 5, load_pv8, [&](int tt, const PV8Buf& bf) {
          half8 ahi, alo;
          wfrag(32 * tt + 8 * lq - c0, ahi, alo);
          mm8(O, bf, ahi, alo);
        });
      } else {
        const uint16_t* ov16 = reinterpret_cast<const uint16_t*>(ovt);
        pipelined<CONFKV_PV16_NPB, PV16Buf<CBW>>(
            c0 >> 5, c1 >> 5, [&](int tt, PV16Buf<CBW>& bf) { vload16(ov16, n_old, tt, bf); },
            [&](int tt, const PV16Buf<CBW>& bf) {
              half8 ahi, alo;
              wfrag(32 * tt + 8 * lq - c0, ahi, alo);
              mm16(O, bf, ahi, alo);
            });
      }
      __syncthreads();  // every wave has read the chunk's LDS before the next chunk writes it
    };
    for (int c0 = 0; c0 < n_old32; c0 += CH) run_chunk(false, c0, min(c0 + CH, n_old32));
    load_new_row();
    append_row();
    for (int c0 = n_old32; c0 < rows; c0 += CH) run_chunk(true, c0, min(c0 + CH, rows));
#pragma unroll
    for (int g = 0; g < G; ++g) {
      Mf[g] = sh_mrun[g];
      inv_l[g] = 1.0f / sh_lrun[g];
    }
    const float fiv = ldexpf(1.0f, -fexp_run);
    float il4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int g = 0; g < G; ++g)
        if (g == 4 * lq + r) il4[r] = inv_l[g];
#pragma unroll
    for (int k = 0; k < CBW; ++k) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int g = 4 * lq + r;
        if (g < G) {
          const int col = 16 * (CBW * wave + k) + lj;
          a.out[((size_t)si * G + g) * D + col] = f2h(O[k][r] * fiv * il4[r]);
        }
      }
    }
    if (par.record && tid == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) lay.rec_lse[(size_t)seg * G + g] = Mf[g] + logf(sh_lrun[g]);
    }
    }
  }  // attention

  // An attend launch under KVpop has no per-row pass left: the priorities
  // need no update and the ranking waits for the evict launch.
  if constexpr (MODE == kModeAttend) {
    if (kvpop) {
      if (tid == 0 && n_old != n_old_raw) atomicOr(lay.err, kErrInternal);
      return;
    }
  }
  // ---- an evict launch after split-K attends (CONF): every live row's EMA
  // from the scores the split attends stored and the heads' log-sum-exps
  // [Conf-KV post: EMA of the attention mass], mass = mean over the G heads
  // of exp(s - LSE). A thread updates the rows its key pass reads next.
  if constexpr (MODE == kModeEvict) {
    if (a.ema_from_scores && !kvpop) {
      const float* sco = lay.stage + (size_t)seg * lay.planes * lay.rows_max;
      float lse[G];
#pragma unroll
      for (int g = 0; g < G; ++g) lse[g] = lay.sk_lse[(size_t)seg * G + g];
      constexpr int RB = 4;
      for (int i0 = tid; i0 < rows; i0 += kThreads * RB) {
        int32_t p[RB];
        float ev[RB], sc[RB][G];
#pragma unroll
        for (int u = 0; u < RB; ++u) {
          const int i = min(i0 + kThreads * u, rows - 1);
          const int r = i - n_old32;
          const int ix = r < 0 ? i : lay.cap32 + min(r, Wr32 - 1);
          p[u] = opos[ix];
          ev[u] = oema[ix];
#pragma unroll
          for (int g = 0; g < G; ++g) sc[u][g] = sco[(size_t)g * lay.rows_max + i];
        }
#pragma unroll
        for (int u = 0; u < RB; ++u) {
          const int i = i0 + kThreads * u;
          if (i >= rows) continue;
          const int r = i - n_old32;
          const bool is_old = i < n_old, is_ring = r >= 0 && r < Wr;
          const bool is_new = is_ring && r == slot_new;
          if (!(is_old || (is_ring && (is_new || p[u] >= 0)))) continue;
          float mass = 0.0f;
#pragma unroll
          for (int g = 0; g < G; ++g) mass += __expf(sc[u][g] - lse[g]);
          mass *= 1.0f / (float)G;
          oema[is_old ? i : lay.cap32 + r] = par.beta * (is_new ? 0.0f : ev[u]) + (1.0f - par.beta) * mass;
        }
      }
    }
  }
  // the row pass starts from the first rows again (an evict launch, and the
  // HBM-staged attention, which has no weight pass over them, load them here first)
  if (MODE == kModeEvict || !kLds || rows > kThreads * KB) {
    int i0 = tid;
    asm volatile("" : "+v"(i0));  // recompute the addresses rather than keep them live
    load_rows(i0);
    load_scores(i0);
  }
  // prefetch of the row that may leave the FP16 window at the end of the step
  // (16 consecutive elements of K or V per lane for lanes 0 .. 2*LPR-1)
  // One half per register (K: 16 consecutive halves of the row; V: the same
  // columns from the transposed tile, 8 halves apart), combined only at the
  // age-out, so nothing here waits for the loads.
  uint32_t aro[16];
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) aro[jj] = 0u;
  if (kEv && pos_out >= 0 && wave == 0 && lane < 2 * LPR) {
    const int slot = pos_out % Wr, cc = lane % LPR;
    const bool isv = lane >= LPR;
    const uint16_t* src = isv ? rvt + vt16(slot, 16 * cc, D) : rk + (size_t)slot * D + cc * 16;
    const int stride = isv ? 8 : 1;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) aro[jj] = src[stride * jj];
  }
  // this row's logits partials, merged by wave 0 after the key pass
  ConfPartial part0;
  if (kEv && !kvpop && wave == 0 && lane < lay.chunks) part0 = lay.partials[(size_t)b * lay.chunks + lane];
  if constexpr (!kLds && kEv)
    for (int j = tid; j < kSelBins; j += kThreads) hsel[j] = 0u;
  // every wave's PV has read the weights that the keys overwrite (evict: the
  // flag sh_out_live is cleared; HBM-staged: the histogram is cleared)
  if constexpr (kEv) __syncthreads();
  // ---- mass, EMA, score, key. [Conf-KV post] ema of the attention mass,
  // score = alpha*ema + (1-alpha)*recency; KVpop ranks by its priority.
  // p_gi = (hi + lo) / (scale_i * f) from the stored weight. Keys overwrite
  // planes 0/1 of the row just read (same thread). An attend launch stops at
  // the EMA; an evict launch takes the EMA the attend launches stored.
  uint32_t n_live = 0, n_elig = 0;
  uint64_t kmin = ~0ull;  // this thread's smallest key and its stage row
  int32_t imin = -1;
  const float inv_t1 = 1.0f / (float)(t + 1);  // recency (pos+1)/(t+1) as a product, within an ulp
  // random ranker: this step's and segment's generator state; a row's rank
  // is the top 24 bits of out(k2, pos + 1) times 2^-24
  const uint64_t rnd_k2 = splitmix64_out(splitmix64_out(par.seed, (uint64_t)t + 1), (uint64_t)seg + 1);
  // one row: its state, EMA (to store when est), score and key
  auto key_row = [&](int i, int u, int32_t& pos, float& e_out, bool& est, float& score, uint64_t& key) {
    key = ~0ull;
    score = NAN;
    est = false;
    e_out = 0.0f;
    float ev_u;
    row_state(i, kpos[u], kev[u], pos, ev_u);
    if (pos >= 0) {
      ++n_live;
      if (!kvpop) {
        float e = ev_u;
        if constexpr (kAtt) {
          float mass = 0.0f;
          if constexpr (kLds) {
            const float inv_scf = __builtin_amdgcn_rcpf(row_scale(i, ksv[u])) * finv;
#pragma unroll
            for (int g = 0; g < G; ++g) {
              const uint32_t wd = __builtin_bit_cast(uint32_t, st.at(g, i));
              const float wv = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd & 0xFFFFu)) +
                               (float)__builtin_bit_cast(_Float16, (uint16_t)(wd >> 16));
              mass = fmaf(wv, inv_l[g], mass);
            }
            mass *= inv_scf * (1.0f / (float)G);
          } else {  // from the raw scores in the HBM stage
#pragma unroll
            for (int g = 0; g < G; ++g) mass = fmaf(__expf(ksc[u][g] - Mf[g]), inv_l[g], mass);
            mass *= 1.0f / (float)G;
          }
          e = par.beta * ev_u + (1.0f - par.beta) * mass;
          e_out = e;
          est = true;
        }
        if (par.ranker == 0) {
          const float rec = (float)(pos + 1) * inv_t1;
          score = par.alpha * e + (1.0f - par.alpha) * rec;
        } else {
          score = (float)(uint32_t)(splitmix64_out(rnd_k2, (uint64_t)pos + 1) >> 40) * 0x1p-24f;
        }
      } else {
        score = ev_u;
      }
      if constexpr (kEv) {
        const bool elig = pos >= par.s && pos <= t - par.P;
        if (!isfinite(score)) {
          atomicOr(lay.err, kErrNonFinite);
        } else if (elig) {
          key = rank_key(score, pos);
          ++n_elig;
          if (key < kmin) {
            kmin = key;
            imin = i;
          }
        }
        if (pos == pos_out && i >= n_old32) sh_out_live = 1;
      }
    }
  };
  auto store_row = [&](int i, int32_t pos, float e, bool est, float score, uint64_t key) {
    if constexpr (kAtt) {
      if (est) oema[i < n_old32 ? i : lay.cap32 + (i - n_old32)] = e;  // unified row-state index
    }
    if constexpr (kEv) {
      st.set_key(i, key);
      if constexpr (!kLds) hist_add(hsel, (uint32_t)(key >> (64 - kSelBinBits)));
      if (par.record) {
        lay.rec_pos[(size_t)seg * lay.rows_max + i] = pos;
        lay.rec_score[(size_t)seg * lay.rows_max + i] = pos >= 0 ? score : NAN;
      }
    }
  };
  if constexpr (kLds) {
    for (int i0 = tid; i0 < rows; i0 += kThreads * KB) {
      if (i0 != tid) load_rows(i0);
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int i = i0 + kThreads * u;
        if (i < rows) {
          int32_t pos;
          float e, score;
          bool est;
          uint64_t key;
          key_row(i, u, pos, e, est, score, key);
          store_row(i, pos, e, est, score, key);
        }
      }
    }
  } else {
    // A batch's results wait in registers while the next batch's loads are
    // issued, and are stored after them: loads and stores share one counter,
    // so loads issued after the stores would wait for those stores too.
    for (int i0 = tid; i0 < rows; i0 += kThreads * KB) {
      int32_t pos[KB];
      float e[KB], score[KB];
      bool est[KB];
      uint64_t key[KB];
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int i = i0 + kThreads * u;
        if (i < rows) key_row(i, u, pos[u], e[u], est[u], score[u], key[u]);
      }
      if (i0 + kThreads * KB < rows) {
        load_rows(i0 + kThreads * KB);
        load_scores(i0 + kThreads * KB);
      }
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int i = i0 + kThreads * u;
        if (i < rows) store_row(i, pos[u], e[u], est[u], score[u], key[u]);
      }
    }
  }
  if constexpr (MODE == kModeAttend) {
    if (tid == 0 && n_old != n_old_raw) atomicOr(lay.err, kErrInternal);
    return;
  }
  if (!kvpop && wave == 0) {
    float cval;
    int base;
    row_confidence(lay, par, b, lane, part0, cval, base);
    if (lane == 0) {
      sh_base = base;
      if (l == 0 && seg % lay.Hkv == 0) {  // the row's first segment reports it
        if (a.conf_out) a.conf_out[b] = cval;
        if (a.budget_out) a.budget_out[b] = base;
      }
    }
  }
  // One block reduction gives the live and eligible counts and the smallest
  // key with its row. With one victim (the steady state) that is the whole
  // selection; more victims continue from it.
  {
    n_live = wave_sum_u32(n_live);
    n_elig = wave_sum_u32(n_elig);
    wave_argmin_u64(kmin, imin);
    if (lane == 0) {
      sel_cnt[wave][0] = n_live;
      sel_cnt[wave][1] = n_elig;
      sel_key[wave] = kmin;
      sel_row[wave] = imin;
    }
    __syncthreads();
    n_live = sel_cnt[0][0] + sel_cnt[1][0] + sel_cnt[2][0] + sel_cnt[3][0];
    n_elig = sel_cnt[0][1] + sel_cnt[1][1] + sel_cnt[2][1] + sel_cnt[3][1];
    kmin = sel_key[0];
    imin = sel_row[0];
#pragma unroll
    for (int w = 1; w < 4; ++w)
      if (sel_key[w] < kmin) {
        kmin = sel_key[w];
        imin = sel_row[w];
      }
  }

  // ---- budget and selection of the e lowest keys among the eligible rows.
  int budget;
  if (!kvpop) {
    const long long base = sh_base;
    budget = (par.pyramid && lay.L > 1)
                 ? (int)((base * (long long)(3 * (lay.L - 1) - 2 * l)) / (long long)(2 * (lay.L - 1)))
                 : (int)base;
  } else {
    budget = par.s + par.P + par.kvpop_k;
  }
  uint32_t e = 0;
  if ((int)n_live > budget) e = min((uint32_t)((int)n_live - budget), n_elig);
  uint64_t T = e > 0 ? kmin : 0;  // victims: key <= T (no key is 0); the first is the smallest key
  if constexpr (kLds) {
    if (e > 1 && e <= 8) {
      for (uint32_t r = 1; r < e; ++r) {
        uint64_t mk = ~0ull;
        for_keys(st, rows, [&](int, uint64_t k) {
          if (k > T && k < mk) mk = k;
        });
        T = block_min_u64(mk, red_k);
      }
    } else if (e > 8) {
      T = radix_select(st, rows, e, hist, red_u, sh, red_k);
    }
  } else if (e > 1) {
    // Victims into the bitmask. The bin holding the e-th smallest key: each
    // thread sums 32 consecutive bins, a block scan places them.
    constexpr int BPT = kSelBins / kThreads;
    {
      uint32_t cnt = 0;
#pragma unroll 8
      for (int j = 0; j < BPT; ++j) cnt += hsel[BPT * tid + j];
      uint32_t total;
      const uint32_t excl = block_excl_scan_u32(cnt, red_u, &total);
      if (excl < e && e <= excl + cnt) {
        uint32_t acc = excl;
        for (int j = 0; j < BPT; ++j) {
          const uint32_t c = hsel[BPT * tid + j];
          if (acc + c >= e) {
            sh[0] = BPT * tid + j;
            sh[1] = (int32_t)acc;
            break;
          }
          acc += c;
        }
      }
      if (tid == 0) sh_cand = 0u;
      __syncthreads();
    }
    const uint32_t tb = (uint32_t)sh[0];
    const uint32_t e2 = e - (uint32_t)sh[1];  // victims still to choose inside bin tb
    uint64_t* ckey = reinterpret_cast<uint64_t*>(dyn_lds);
    int32_t* crow = reinterpret_cast<int32_t*>(ckey + kSelCandCap);
    // One pass over the keys' high words: rows of lower bins are victims
    // (a wave stores the bitmask words of its 64 consecutive rows); the keys
    // of bin tb are gathered as candidates while there is room (their low
    // words are loaded after the pass, all at once).
    {
      constexpr int U = 16;
      const int wrow0 = 64 * wave;
      for (int i0 = 0; i0 < rows; i0 += kThreads * U) {
        uint32_t hw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = i0 + kThreads * u + tid;
          hw[u] = i < rows ? __builtin_bit_cast(uint32_t, st.at(1, i)) : ~0u;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int w0 = i0 + kThreads * u + wrow0;  // the wave's first row (a multiple of 64)
          if (w0 >= rows) break;                     // wave-uniform
          const int i = w0 + lane;
          const uint32_t bn = hw[u] >> (32 - kSelBinBits);
          const uint64_t below = __ballot(i < rows && bn < tb);
          const uint64_t inbin = __ballot(i < rows && bn == tb);
          if (lane == 0) vbits[w0 >> 5] = (uint32_t)below;
          if (lane == 32 && w0 + 32 < rows) vbits[(w0 >> 5) + 1] = (uint32_t)(below >> 32);
          if (inbin != 0ull) {
            const int leader = __ffsll((unsigned long long)inbin) - 1;
            uint32_t base = 0u;
            if (lane == leader) base = atomicAdd(&sh_cand, (uint32_t)__popcll(inbin));
            base = __shfl(base, leader, 64);
            if ((inbin >> lane) & 1ull) {
              const uint32_t idx = base + (uint32_t)__popcll(inbin & ((1ull << lane) - 1ull));
              if (idx < (uint32_t)kSelCandCap) {
                ckey[idx] = (uint64_t)hw[u] << 32;
                crow[idx] = i;
              }
            }
          }
        }
      }
    }
    __syncthreads();
    const uint32_t nc = sh_cand;
    if (nc <= (uint32_t)kSelCandCap) {
      // The e2 smallest candidates (keys are unique). A thread holds
      // candidates j = tid + 256 q. Their low words first; then a histogram
      // of the next 8 key bits (51..43 down) names the sub-bin holding the
      // e2-th smallest, below which every candidate is a victim; inside it a
      // candidate's rank is the number of smaller ones there.
      constexpr int CPT = (kSelCandCap + kThreads - 1) / kThreads;
      {
        uint32_t lw[CPT];
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
          const uint32_t j = tid + kThreads * q;
          lw[q] = j < nc ? __builtin_bit_cast(uint32_t, st.at(0, crow[j])) : 0u;
        }
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
          const uint32_t j = tid + kThreads * q;
          if (j < nc) ckey[j] |= lw[q];
        }
      }
      hist[tid] = 0u;
      __syncthreads();
      auto sub = [](uint64_t k) { return (uint32_t)(k >> (64 - kSelBinBits - 8)) & 0xFFu; };
#pragma unroll
      for (int q = 0; q < CPT; ++q) {
        const uint32_t j = tid + kThreads * q;
        if (j < nc) hist_add(hist, sub(ckey[j]));
      }
      __syncthreads();
      {
        const uint32_t cnt = hist[tid];
        uint32_t total;
        const uint32_t excl = block_excl_scan_u32(cnt, red_u, &total);
        if (excl < e2 && e2 <= excl + cnt) {
          sh[0] = tid;
          sh[1] = (int32_t)excl;
        }
        __syncthreads();
      }
      const uint32_t tb2 = (uint32_t)sh[0], e3 = e2 - (uint32_t)sh[1];
#pragma unroll
      for (int q = 0; q < CPT; ++q) {
        const uint32_t j = tid + kThreads * q;
        if (j < nc) {
          const uint64_t kj = ckey[j];
          const uint32_t sj = sub(kj);
          bool v = sj < tb2;
          if (sj == tb2) {
            uint32_t r = 0;
            for (uint32_t k = 0; k < nc; ++k) {
              const uint64_t kk = ckey[k];
              r += (sub(kk) == tb2 && kk < kj) ? 1u : 0u;
            }
            v = r < e3;
          }
          if (v) {
            const int rr = crow[j];
            atomicOr(&vbits[rr >> 5], 1u << (rr & 31));
          }
        }
      }
    } else {
      // too many keys share the bin: a radix select over the staged keys
      // gives the e-th smallest key, and the bin's keys up to it are victims
      T = radix_select(st, rows, e, hist, red_u, sh, red_k);
      for_keys(st, rows, [&](int i, uint64_t k) {
        if ((uint32_t)(k >> (64 - kSelBinBits)) == tb && k <= T) atomicOr(&vbits[i >> 5], 1u << (i & 31));
      });
    }
    __syncthreads();
  }
  // is stage row i a victim
  auto victim = [&](int i) -> bool {
    if constexpr (!kLds) {
      if (e > 1) return (vbits[i >> 5] >> (i & 31)) & 1u;
    }
    return st.key(i) <= T;
  };

  // ---- compaction of the old region. The row leaving the FP16 window (if it
  // survived) takes the lowest victim's slot; the other victims below the new
  // count m become holes, filled in ascending order by the survivors at or
  // above m. The steady state (one old victim, one aged-out row) moves nothing.
  const int slot_out = pos_out >= 0 ? pos_out % Wr : 0;
  const bool age = pos_out >= 0 && sh_out_live && !victim(n_old32 + slot_out);
  uint32_t ev_old = 0;
  int vmin = n_old, vmax = -1;
  if (e == 1) {
    if (imin < n_old) {  // the one victim is an old row
      ev_old = 1;
      vmin = vmax = imin;
    }
  } else if (e > 1) {
    if constexpr (kLds) {
      for_keys(st, n_old, [&](int i, uint64_t k) {
        if (k <= T) {
          ++ev_old;
          vmin = min(vmin, i);
          vmax = max(vmax, i);
        }
      });
    } else {
      for (int w = tid; w < ((n_old + 31) >> 5); w += kThreads) {
        const uint32_t bw = vbits[w] & bits_below(n_old - 32 * w);
        if (bw) {
          ev_old += (uint32_t)__popc(bw);
          vmin = min(vmin, 32 * w + __ffs(bw) - 1);
          vmax = max(vmax, 32 * w + 31 - __clz(bw));
        }
      }
    }
    for (int o = 32; o > 0; o >>= 1) {
      ev_old += __shfl_xor(ev_old, o, 64);
      vmin = min(vmin, __shfl_xor(vmin, o, 64));
      vmax = max(vmax, __shfl_xor(vmax, o, 64));
    }
    if (lane == 0) {
      sh[wave] = vmin;
      sh[4 + wave] = vmax;
      red_u[wave] = ev_old;
    }
    __syncthreads();
    ev_old = red_u[0] + red_u[1] + red_u[2] + red_u[3];
    vmin = min(min(sh[0], sh[1]), min(sh[2], sh[3]));
    vmax = max(max(sh[4], sh[5]), max(sh[6], sh[7]));
    __syncthreads();
  }
  const bool into_hole = age && ev_old > 0;         // aged-out row goes to slot vmin
  const int rem = (int)ev_old - (into_hole ? 1 : 0);  // victims left to compact away
  const int m = n_old - rem;                          // old rows after compaction (+1 if appended)
  uint32_t moved = 0;
  if (rem == 1) {
    const int v = into_hole ? vmax : vmin;  // the one remaining victim
    if (v < m) {                            // move the last row (a survivor) into it
      const int src = n_old - 1;
      moved = 1;
      if (rg == 0) {
        const size_t rb = (size_t)D * ob;
        const int cbytes = 16 * ob;
        for (int off = 0; off < cbytes; off += 16)
          *reinterpret_cast<uint4*>(okp + v * rb + c * cbytes + off) =
              *reinterpret_cast<const uint4*>(okp + src * rb + c * cbytes + off);
        if (ob == 1) {
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) ovt[vt8(v, 16 * c + jj, D)] = ovt[vt8(src, 16 * c + jj, D)];
        } else {
          uint16_t* v16 = reinterpret_cast<uint16_t*>(ovt);
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) v16[vt16(v, 16 * c + jj, D)] = v16[vt16(src, 16 * c + jj, D)];
        }
        if (c == 0) {
          opos[v] = opos[src];
          oema[v] = oema[src];
          oprio[v] = oprio[src];
          oks[v] = oks[src];
          ovs[v] = ovs[src];
        }
      }
    }
  } else if (rem > 1) {
    int32_t* holes = st.list(2);
    int32_t* srcs = st.list(3);
    uint32_t nh, kt = 0;        // rows and whole tiles to move
    int32_t* tdst = nullptr;    // tiles of holes (HBM-staged variant)
    int32_t* tsrc = nullptr;    // tiles of sources
    if constexpr (kLds) {
      // victim predicate for the hole fill: vmin is not a hole when it takes the aged-out row
      auto hole = [&](int i, uint64_t k) { return k <= T && !(into_hole && i == vmin); };
      const int per = (n_old + kThreads - 1) / kThreads;
      const int lo = min(n_old, tid * per), hi = min(n_old, lo + per);
      uint32_t hv = 0, sv = 0;
      for_keys_range(st, lo, hi, [&](int i, uint64_t k) {
        const bool v = hole(i, k);
        hv += (v && i < m) ? 1u : 0u;
        sv += (!v && i >= m) ? 1u : 0u;
      });
      uint32_t ns;
      uint32_t ho = block_excl_scan_u32(hv, red_u, &nh);
      uint32_t so = block_excl_scan_u32(sv, red_u, &ns);
      for_keys_range(st, lo, hi, [&](int i, uint64_t k) {
        const bool v = hole(i, k);
        const bool to_hole = v && i < m, to_src = !v && i >= m;
        if (to_hole) holes[ho] = i;
        if (to_src) srcs[so] = i;
        ho += to_hole ? 1u : 0u;
        so += to_src ? 1u : 0u;
      });
    } else {
      // From the bitmask, whose words are the 32-row tiles: a thread takes
      // whole words of consecutive rows. Holes are the victims below m (vmin
      // excepted when it takes the aged-out row), sources the survivors at or
      // above m. The old region keeps no row order, so any pairing of holes
      // with sources will do: a tile of 32 holes is filled from a tile of 32
      // sources as a whole (such tiles paired in ascending order; the copy is
      // contiguous K rows, one V tile and the row state), and the remaining
      // holes and sources pair row by row in ascending order.
      const int per = (((n_old + kThreads - 1) / kThreads) + 31) & ~31;
      const int lo = min(n_old, tid * per), hi = min(n_old, lo + per);
      // this thread's words [w0, w1): none when its range is empty
      const int w0 = lo >> 5, w1 = lo < hi ? (hi + 31) >> 5 : w0;
      auto hole_src = [&](int w, uint32_t& hw, uint32_t& sw) {
        const uint32_t bw = vbits[w], in = bits_below(hi - 32 * w), lt_m = bits_below(m - 32 * w);
        hw = bw & in & lt_m;
        if (into_hole && (vmin >> 5) == w) hw &= ~(1u << (vmin & 31));
        sw = ~bw & in & ~lt_m;
      };
      auto hole_tile = [&](uint32_t hw, int w) { return hw == ~0u && 32 * w + 32 <= m; };
      auto src_tile = [&](uint32_t sw, int w) { return sw == ~0u && 32 * w >= m; };
      uint32_t fh = 0, fs = 0;
      for (int w = w0; w < w1; ++w) {
        uint32_t hw, sw;
        hole_src(w, hw, sw);
        fh += hole_tile(hw, w) ? 1u : 0u;
        fs += src_tile(sw, w) ? 1u : 0u;
      }
      uint32_t nfh, nfs;
      const uint32_t fho = block_excl_scan_u32(fh, red_u, &nfh);
      const uint32_t fso = block_excl_scan_u32(fs, red_u, &nfs);
      kt = min(nfh, nfs);
      // rows outside the paired tiles
      uint32_t hv = 0, sv = 0;
      {
        uint32_t a = fho, b = fso;
        for (int w = w0; w < w1; ++w) {
          uint32_t hw, sw;
          hole_src(w, hw, sw);
          if (hole_tile(hw, w) && a++ < kt) hw = 0u;
          if (src_tile(sw, w) && b++ < kt) sw = 0u;
          hv += (uint32_t)__popc(hw);
          sv += (uint32_t)__popc(sw);
        }
      }
      uint32_t ns;
      uint32_t ho = block_excl_scan_u32(hv, red_u, &nh);
      uint32_t so = block_excl_scan_u32(sv, red_u, &ns);
      // row lists, then the tile lists, in the LDS the selection used when they fit
      if (8 * (nh + kt) <= (uint32_t)kSelLdsBytes) {
        holes = reinterpret_cast<int32_t*>(dyn_lds);
        srcs = holes + nh;
        tdst = srcs + nh;
        tsrc = tdst + kt;
      } else {
        tdst = holes + nh;
        tsrc = srcs + nh;
      }
      {
        uint32_t a = fho, b = fso;
        for (int w = w0; w < w1; ++w) {
          uint32_t hw, sw;
          hole_src(w, hw, sw);
          if (hole_tile(hw, w)) {
            if (a < kt) {
              tdst[a] = w;
              hw = 0u;
            }
            ++a;
          }
          if (src_tile(sw, w)) {
            if (b < kt) {
              tsrc[b] = w;
              sw = 0u;
            }
            ++b;
          }
          for (; hw; hw &= hw - 1u) holes[ho++] = 32 * w + __ffs(hw) - 1;
          for (; sw; sw &= sw - 1u) srcs[so++] = 32 * w + __ffs(sw) - 1;
        }
      }
    }
    __syncthreads();
    moved = nh + 32 * kt;
    // whole tiles: each thread copies 16-byte units of the K rows and of the
    // V tile, and one row-state value; four tiles per iteration, every load
    // before any store
    if constexpr (!kLds) {
      const int units = 2 * D * ob;  // 16-byte units in a tile's K rows (as in its V tile)
      constexpr int TU = 4;
      for (int i0 = 0; i0 < (int)kt; i0 += TU) {
        uint4 kv[TU][4];
        uint32_t sv4[TU];
#pragma unroll
        for (int u = 0; u < TU; ++u) {
          const int i = min(i0 + u, (int)kt - 1);  // past the list: the last pair again
          const size_t sb = (size_t)tsrc[i] * units;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int j = tid + kThreads * h;
            kv[u][2 * h] = kv[u][2 * h + 1] = uint4{0u, 0u, 0u, 0u};
            if (j < units) {
              kv[u][2 * h] = reinterpret_cast<const uint4*>(okp)[sb + j];
              kv[u][2 * h + 1] = reinterpret_cast<const uint4*>(ovt)[sb + j];
            }
          }
          const int r = 32 * tsrc[i] + (tid & 31), f = tid >> 5;  // row state: 5 arrays x 32 rows
          sv4[u] = 0u;
          if (f < 5) {
            const uint32_t* arr = f == 0 ? reinterpret_cast<const uint32_t*>(opos)
                                : f == 1 ? reinterpret_cast<const uint32_t*>(oema)
                                : f == 2 ? reinterpret_cast<const uint32_t*>(oprio)
                                : f == 3 ? reinterpret_cast<const uint32_t*>(oks)
                                         : reinterpret_cast<const uint32_t*>(ovs);
            sv4[u] = arr[r];
          }
        }
#pragma unroll
        for (int u = 0; u < TU; ++u) {
          if (i0 + u < (int)kt) {
            const size_t db = (size_t)tdst[i0 + u] * units;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int j = tid + kThreads * h;
              if (j < units) {
                reinterpret_cast<uint4*>(okp)[db + j] = kv[u][2 * h];
                reinterpret_cast<uint4*>(ovt)[db + j] = kv[u][2 * h + 1];
              }
            }
            const int r = 32 * tdst[i0 + u] + (tid & 31), f = tid >> 5;
            if (f < 5) {
              uint32_t* arr = f == 0 ? reinterpret_cast<uint32_t*>(opos)
                            : f == 1 ? reinterpret_cast<uint32_t*>(oema)
                            : f == 2 ? reinterpret_cast<uint32_t*>(oprio)
                            : f == 3 ? reinterpret_cast<uint32_t*>(oks)
                                     : reinterpret_cast<uint32_t*>(ovs);
              arr[r] = sv4[u];
            }
          }
        }
      }
    }
    // A lane group moves two rows per iteration and issues every load of both
    // before any store (a source is never a hole, so nothing overlaps).
    const size_t rb = (size_t)D * ob;
    const int cbytes = 16 * ob;  // bytes of a K row per lane
    uint16_t* v16 = reinterpret_cast<uint16_t*>(ovt);
    struct MoveRow {
      uint4 k0, k1;
      uint32_t v[16];
      int32_t p;
      float f[4];
    };
    auto load_row = [&](int sr, MoveRow& m) __attribute__((always_inline)) {
      m.k0 = *reinterpret_cast<const uint4*>(okp + sr * rb + c * cbytes);
      m.k1 = uint4{0u, 0u, 0u, 0u};
      if (ob == 2) m.k1 = *reinterpret_cast<const uint4*>(okp + sr * rb + c * cbytes + 16);
      if (ob == 1) {
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) m.v[jj] = ovt[vt8(sr, 16 * c + jj, D)];
      } else {
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) m.v[jj] = v16[vt16(sr, 16 * c + jj, D)];
      }
      m.p = opos[sr];
      m.f[0] = oema[sr];
      m.f[1] = oprio[sr];
      m.f[2] = oks[sr];
      m.f[3] = ovs[sr];
    };
    auto store_row = [&](int dr, const MoveRow& m) __attribute__((always_inline)) {
      *reinterpret_cast<uint4*>(okp + dr * rb + c * cbytes) = m.k0;
      if (ob == 2) *reinterpret_cast<uint4*>(okp + dr * rb + c * cbytes + 16) = m.k1;
      if (ob == 1) {
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) ovt[vt8(dr, 16 * c + jj, D)] = (uint8_t)m.v[jj];
      } else {
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) v16[vt16(dr, 16 * c + jj, D)] = (uint16_t)m.v[jj];
      }
      if (c == 0) {
        opos[dr] = m.p;
        oema[dr] = m.f[0];
        oprio[dr] = m.f[1];
        oks[dr] = m.f[2];
        ovs[dr] = m.f[3];
      }
    };
    for (int r0 = rg; r0 < (int)nh; r0 += 2 * RPB) {
      const int r1 = r0 + RPB;
      const bool two = r1 < (int)nh;
      const int s0 = srcs[r0], d0 = holes[r0];
      const int s1 = two ? srcs[r1] : s0, d1 = two ? holes[r1] : d0;  // no second row: reload the first
      MoveRow m0, m1;
      load_row(s0, m0);
      load_row(s1, m1);
      store_row(d0, m0);
      store_row(d1, m1);  // without a second row: the first row's values again
    }
  }
  if (e == 1) {
    if (tid == 0 && imin >= n_old32) rpos[imin - n_old32] = -1;
  } else if (e > 1) {
    for (int r = tid; r < Wr; r += kThreads)
      if (victim(n_old32 + r)) rpos[r] = -1;
  }

  // ---- age-out: the row at t - W leaves the FP16 window; if it survived it
  // is stored in the old region (quantized when old rows are INT8), in the
  // lowest victim's slot or appended at m.
  int n_old_new = m;
  bool aged = false;
  if (age) {
    const int dst = into_hole ? vmin : m;
    if (dst >= lay.cap) {
      if (tid == 0) atomicOr(lay.err, kErrCapacity);
    } else {
      const int slot = slot_out;
      if (wave == 0 && lane < 2 * LPR) {
        const bool isv = lane >= LPR;
        const int cc = lane % LPR;
        float x[16];
        {
#pragma unroll
          for (int j = 0; j < 16; ++j) x[j] = half_lo(aro[j]);
        }
        if (par.old_int8) {
          int8_t codes[16];
          const float scale = quantize16<LPR>(x, codes);
          if (!isv) {
            *reinterpret_cast<uint4*>(okp + (size_t)dst * D + cc * 16) = pack16(codes);
            if (cc == 0) oks[dst] = scale;
          } else {
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) ovt[vt8(dst, 16 * cc + jj, D)] = (uint8_t)codes[jj];
            if (cc == 0) ovs[dst] = scale;
          }
        } else {
          if (!isv) {
            uint4* d4 = reinterpret_cast<uint4*>(okp + ((size_t)dst * D + cc * 16) * 2);
            uint32_t w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) w[j] = aro[2 * j] | (aro[2 * j + 1] << 16);
            d4[0] = make_uint4(w[0], w[1], w[2], w[3]);
            d4[1] = make_uint4(w[4], w[5], w[6], w[7]);
          } else {
            uint16_t* v16 = reinterpret_cast<uint16_t*>(ovt);
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) v16[vt16(dst, 16 * cc + jj, D)] = f2h(x[jj]);
          }
          if (cc == 0) (isv ? ovs : oks)[dst] = 0.0f;
        }
        if (lane == 0) {
          opos[dst] = pos_out;
          oema[dst] = rema[slot];
          oprio[dst] = rprio[slot];
          rpos[slot] = -1;
        }
      }
      aged = true;
      if (!into_hole) n_old_new = m + 1;
    }
  }
  if (tid == 0) {
    if (n_old != n_old_raw) atomicOr(lay.err, kErrInternal);
    lay.seg_nold[seg] = n_old_new;
    const uint64_t live_ring = (uint64_t)n_live - (uint64_t)n_old;
    const uint64_t old_row = par.old_int8 ? (uint64_t)(2 * D + 8) : (uint64_t)(4 * D);
    unsigned long long* sp = reinterpret_cast<unsigned long long*>(lay.seg_stats + (size_t)seg * kStatFields);
    atomicAdd(sp + 0, (unsigned long long)((uint64_t)n_old * old_row + live_ring * (uint64_t)(4 * D)));
    atomicAdd(sp + 1, (unsigned long long)n_live);
    atomicAdd(sp + 2, (unsigned long long)(moved + (aged ? 1u : 0u)));
    atomicAdd(sp + 3, (unsigned long long)e);
    if (par.record) {
      int32_t* mp = lay.rec_meta + (size_t)seg * 4;
      mp[0] = rows;
      mp[1] = (int32_t)n_live;
      mp[2] = budget;
      mp[3] = (int32_t)e;
    }
  }
}

// ================================================================ init/ingest
__global__ void zero_kernel(uint4* p, size_t n16) {
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x) p[i] = z;
}

__global__ void init_meta_kernel(Layout lay, int32_t n_old_init) {
  const int seg = blockIdx.x, tid = threadIdx.x;
  for (int r = tid; r < lay.Wr32; r += blockDim.x) lay.row_pos[(size_t)seg * lay.rows_max + lay.cap32 + r] = -1;
  if (tid == 0) lay.seg_nold[seg] = n_old_init;
}

// Prefill rows 32*blockIdx.x .. +31 of segment blockIdx.y. Rows with
// pos <= P0-1-W go to old row pos (quantized when old rows are INT8), the rest
// to ring slot pos mod Wr. Old V rows are assembled into their transposed tile
// in LDS and written out in 16-byte chunks.
template <int D>
__global__ void __launch_bounds__(256) ingest_kernel(Layout lay, Params par, const uint16_t* pk, const uint16_t* pv,
                                                     int32_t P0) {
  constexpr int LPR = D / 16;
  __shared__ uint16_t tile[32 * D];  // old V rows of this block, row-major (codes or halves)
  const int seg = blockIdx.y, blk = blockIdx.x, tid = threadIdx.x, c = tid % LPR, rr = tid / LPR;
  const int n_old_init = max(0, P0 - lay.W);
  const int ob = lay.old_bytes;
  const size_t obase = (size_t)seg * lay.cap32;
  for (int i = tid; i < 32 * D; i += 256) tile[i] = 0;
  __syncthreads();
  const int p = 32 * blk + rr;
  if (rr < 32 && p < P0) {  // whole lane groups share p
    float xk[16], xv[16];
    load16h(pk + ((size_t)seg * P0 + p) * D + c * 16, xk);
    load16h(pv + ((size_t)seg * P0 + p) * D + c * 16, xv);
    if (p < n_old_init) {
      const size_t row = obase + p;
      if (par.old_int8) {
        int8_t ck[16], cv[16];
        const float sk = quantize16<LPR>(xk, ck);
        const float sv = quantize16<LPR>(xv, cv);
        *reinterpret_cast<uint4*>(lay.old_k + row * D + c * 16) = pack16(ck);
        uint8_t* t8 = reinterpret_cast<uint8_t*>(tile);
#pragma unroll
        for (int e = 0; e < 16; ++e) t8[rr * D + 16 * c + e] = (uint8_t)cv[e];
        if (c == 0) {
          lay.old_ks[row] = sk;
          lay.old_vs[row] = sv;
        }
      } else {
        uint16_t* dk = reinterpret_cast<uint16_t*>(lay.old_k) + row * D + c * 16;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          dk[e] = f2h(xk[e]);
          tile[rr * D + 16 * c + e] = f2h(xv[e]);
        }
      }
      if (c == 0) lay.row_pos[(size_t)seg * lay.rows_max + p] = p;
    } else {
      const int slot = p % lay.Wr;
      uint16_t* dk = lay.ring_k + ((size_t)seg * lay.Wr32 + slot) * D + c * 16;
      uint16_t* dv = lay.ring_v + (size_t)seg * lay.Wr32 * D;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        dk[e] = f2h(xk[e]);
        dv[vt16(slot, 16 * c + e, D)] = f2h(xv[e]);
      }
      if (c == 0) lay.row_pos[(size_t)seg * lay.rows_max + lay.cap32 + slot] = p;
    }
  }
  __syncthreads();
  if (32 * blk < n_old_init) {
    if (ob == 1) {
      // 16-byte chunk ch = 64*k + lane of the tile: columns 16*(2k) + j and
      // 16*(2k+1) + j, rows 8q .. 8q+7 (lane = 16q + j)
      const uint8_t* t8 = reinterpret_cast<const uint8_t*>(tile);
      uint8_t* dst = lay.old_v + (obase + 32 * (size_t)blk) * D;
      for (int ch = tid; ch < 2 * D; ch += 256) {
        const int k = ch >> 6, ln = ch & 63, q = ln >> 4, j = ln & 15;
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            w[2 * h + (e >> 2)] |= (uint32_t)t8[(8 * q + e) * D + 16 * (2 * k + h) + j] << (8 * (e & 3));
        reinterpret_cast<uint4*>(dst)[ch] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    } else {
      uint16_t* dst = reinterpret_cast<uint16_t*>(lay.old_v) + (obase + 32 * (size_t)blk) * D;
      for (int ch = tid; ch < 4 * D; ch += 256) {
        const int cb = ch >> 6, ln = ch & 63, q = ln >> 4, j = ln & 15;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = (uint32_t)tile[(8 * q + 2 * e) * D + 16 * cb + j] |
                 ((uint32_t)tile[(8 * q + 2 * e + 1) * D + 16 * cb + j] << 16);
        reinterpret_cast<uint4*>(dst)[ch] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }
}

// ================================================================ read-back
// Staged row i of segment seg_first + blockIdx.y goes to its logical rank:
// old rows first (all older than every ring row), each region ordered by
// position (ranks by counting smaller positions; a checking path).
__global__ void __launch_bounds__(256) read_cache_kernel(Layout lay, int32_t seg_first, int32_t* len, int32_t* pos_o,
                                                         float* ema_o, float* prio_o, uint16_t* k16, uint16_t* v16,
                                                         int8_t* k8, int8_t* v8, float* ks_o, float* vs_o,
                                                         uint8_t* is8_o, int32_t old_int8) {
  const int si = blockIdx.y, seg = seg_first + si;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int D = lay.D, Wr = lay.Wr;
  const int n_old = lay.seg_nold[seg];
  const int32_t* opos = lay.row_pos + (size_t)seg * lay.rows_max;
  const int32_t* rpos = opos + lay.cap32;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    int live = 0;
    for (int r = 0; r < Wr; ++r) live += rpos[r] >= 0;
    len[si] = n_old + live;
  }
  if (i >= n_old + Wr) return;
  const bool in_old = i < n_old;
  const int row = in_old ? i : i - n_old;
  const int32_t pos = in_old ? opos[row] : rpos[row];
  if (pos < 0) return;
  int rank = 0;
  if (in_old) {
    for (int j = 0; j < n_old; ++j) rank += opos[j] < pos;
  } else {
    rank = n_old;
    for (int r = 0; r < Wr; ++r) rank += (rpos[r] >= 0 && rpos[r] < pos);
  }
  const size_t orow = (size_t)si * lay.rows_max + rank;
  const bool row8 = in_old && old_int8;
  if (pos_o) pos_o[orow] = pos;
  if (is8_o) is8_o[orow] = row8 ? 1 : 0;
  const size_t src = in_old ? (size_t)seg * lay.cap32 + row : (size_t)seg * lay.Wr32 + row;
  const size_t us = (size_t)seg * lay.rows_max + (in_old ? row : lay.cap32 + row);
  if (ema_o) ema_o[orow] = lay.row_ema[us];
  if (prio_o) prio_o[orow] = lay.row_prio[us];
  if (ks_o) ks_o[orow] = row8 ? lay.old_ks[src] : 0.0f;
  if (vs_o) vs_o[orow] = row8 ? lay.old_vs[src] : 0.0f;
  const size_t vbase = (in_old ? (size_t)seg * lay.cap32 : (size_t)seg * lay.Wr32) * D;
  for (int e = 0; e < D; ++e) {
    uint16_t hk = 0, hv = 0;
    int8_t ck = 0, cv = 0;
    if (row8) {
      ck = (int8_t)lay.old_k[src * D + e];
      cv = (int8_t)lay.old_v[vbase + vt8(row, e, D)];
    } else if (in_old) {
      hk = reinterpret_cast<const uint16_t*>(lay.old_k)[src * D + e];
      hv = reinterpret_cast<const uint16_t*>(lay.old_v)[vbase + vt16(row, e, D)];
    } else {
      hk = lay.ring_k[src * D + e];
      hv = lay.ring_v[vbase + vt16(row, e, D)];
    }
    if (k16) k16[orow * D + e] = hk;
    if (v16) v16[orow * D + e] = hv;
    if (k8) k8[orow * D + e] = ck;
    if (v8) v8[orow * D + e] = cv;
  }
}

__global__ void __launch_bounds__(256) stats_total_kernel(Layout lay, int32_t reset) {
  __shared__ unsigned long long red[4][kStatFields];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  unsigned long long sum[kStatFields] = {0, 0, 0, 0};
  for (int s = tid; s < lay.S; s += 256)
    for (int f = 0; f < kStatFields; ++f) {
      sum[f] += lay.seg_stats[(size_t)s * kStatFields + f];
      if (reset) lay.seg_stats[(size_t)s * kStatFields + f] = 0;
    }
  for (int f = 0; f < kStatFields; ++f) {
    unsigned long long v = sum[f];
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0) red[wave][f] = v;
  }
  __syncthreads();
  if (tid < kStatFields) lay.stats_total[tid] = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
}

// ================================================================ launchers
int launch_init(const Layout& lay, const Params& par, void* state, size_t state_bytes, const uint16_t* pk,
                const uint16_t* pv, int32_t P0, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const size_t n16 = state_bytes / 16;
  hipLaunchKernelGGL(zero_kernel, dim3(2048), dim3(256), 0, s, reinterpret_cast<uint4*>(state), n16);
  if (hipGetLastError() != hipSuccess) return -3;
  const int32_t n_old_init = P0 > lay.W ? P0 - lay.W : 0;
  hipLaunchKernelGGL(init_meta_kernel, dim3(lay.S), dim3(256), 0, s, lay, n_old_init);
  if (hipGetLastError() != hipSuccess) return -3;
  if (P0 > 0) {
    const dim3 grid((P0 + 31) / 32, lay.S);
    if (lay.D == 64)
      hipLaunchKernelGGL(ingest_kernel<64>, grid, dim3(256), 0, s, lay, par, pk, pv, P0);
    else
      hipLaunchKernelGGL(ingest_kernel<128>, grid, dim3(256), 0, s, lay, par, pk, pv, P0);
  }
  return ok_or_err();
}

int launch_conf_reduce(const Layout& lay, const float* logits, void* stream) {
  hipLaunchKernelGGL(conf_reduce_kernel, dim3(lay.chunks, lay.B), dim3(256), 0, (hipStream_t)stream, lay, logits);
  return ok_or_err();
}

template <int D, int G, int MODE>
static void launch_fused_dg(const Layout& lay, const Params& par, const StepArgs& a, int grid, bool use_lds,
                            int lds_bytes, hipStream_t s) {
  if (use_lds)
    hipLaunchKernelGGL((fused_step_kernel<D, G, true, MODE>), dim3(grid), dim3(kThreads), lds_bytes, s, lay, par, a);
  else
    hipLaunchKernelGGL((fused_step_kernel<D, G, false, MODE>), dim3(grid), dim3(kThreads),
                       MODE == kModeAttend ? kSelLdsBytes : lds_bytes, s, lay, par, a);
}

template <int D, int MODE>
static int launch_fused_d(const Layout& lay, const Params& par, const StepArgs& a, int grid, bool use_lds,
                          int lds_bytes, hipStream_t s) {
  switch (lay.G) {
    case 1: launch_fused_dg<D, 1, MODE>(lay, par, a, grid, use_lds, lds_bytes, s); break;
    case 2: launch_fused_dg<D, 2, MODE>(lay, par, a, grid, use_lds, lds_bytes, s); break;
    case 4: launch_fused_dg<D, 4, MODE>(lay, par, a, grid, use_lds, lds_bytes, s); break;
    case 5: launch_fused_dg<D, 5, MODE>(lay, par, a, grid, use_lds, lds_bytes, s); break;
    case 8: launch_fused_dg<D, 8, MODE>(lay, par, a, grid, use_lds, lds_bytes, s); break;
    default: return -1;
  }
  return ok_or_err();
}

template <int MODE>
static int launch_mode(const Layout& lay, const Params& par, const StepArgs& a, int grid, bool use_lds, int lds_bytes,
                       hipStream_t s) {
  if (lay.D == 64) return launch_fused_d<64, MODE>(lay, par, a, grid, use_lds, lds_bytes, s);
  if (lay.D == 128) return launch_fused_d<128, MODE>(lay, par, a, grid, use_lds, lds_bytes, s);
  return -1;
}

int launch_fused_step(const Layout& lay, const Params& par, const StepArgs& a, bool use_lds, int lds_bytes,
                      void* stream) {
  return launch_mode<kModeStep>(lay, par, a, lay.S, use_lds, lds_bytes, (hipStream_t)stream);
}

int launch_attend(const Layout& lay, const Params& par, const StepArgs& a, bool use_lds, int lds_bytes,
                  void* stream) {
  return launch_mode<kModeAttend>(lay, par, a, lay.B * lay.Hkv, use_lds, lds_bytes, (hipStream_t)stream);
}

int launch_evict(const Layout& lay, const Params& par, const StepArgs& a, bool use_lds, int lds_bytes,
                 void* stream) {
  return launch_mode<kModeEvict>(lay, par, a, lay.S, use_lds, lds_bytes, (hipStream_t)stream);
}

int launch_read_cache(const Layout& lay, int32_t seg_first, int32_t seg_count, int32_t* len, int32_t* pos,
                      float* ema, float* prio, uint16_t* k16, uint16_t* v16, int8_t* k8, int8_t* v8, float* ks,
                      float* vs, uint8_t* is8, int32_t old_int8, void* stream) {
  const dim3 grid((lay.rows_max + 255) / 256, seg_count);
  hipLaunchKernelGGL(read_cache_kernel, grid, dim3(256), 0, (hipStream_t)stream, lay, seg_first, len, pos, ema, prio,
                     k16, v16, k8, v8, ks, vs, is8, old_int8);
  return ok_or_err();
}

int launch_stats_total(const Layout& lay, int32_t reset, void* stream) {
  hipLaunchKernelGGL(stats_total_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream, lay, reset);
  return ok_or_err();
}

int fused_max_dynamic_lds() { return 64 * 1024; }

}  // namespace confkv
