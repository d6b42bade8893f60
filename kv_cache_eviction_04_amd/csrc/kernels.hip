// HIP kernels for gfx950 (MI355X): one decode step of confidence-gated KV
// eviction (CONF-KV) and its KVpop fixed-budget variant.
//
// Kernels
//   conf_reduce_kernel  logits -> (max, sum e, sum e*(z-m), top1, top2) per
//                       chunk; the last chunk of a batch row to finish merges
//                       them into the confidence c and the base budget.
//   fused_step_kernel   one workgroup per segment (layer, batch row, KV head):
//                       append -> QK pass -> max -> exp/sum -> PV pass -> out
//                       -> mass/EMA/score/key -> select -> compact -> age-out.
//   init / ingest       carve the state and store the prefill.
//   read_cache          logical (ascending position) read-out for checking.
//
// Sources: "Conf-KV" post (rcap.io), method paragraph and decoding-loop
// pseudocode; CONF-KV abstract (chatpaper.ai); "Resumen Técnico: KVpop"
// (gist.science) §2.1, §2.3, §2.4.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "layout.h"

namespace confkv {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ float half_lo(uint32_t u) { return (float)__builtin_bit_cast(h2, u)[0]; }
__device__ __forceinline__ float half_hi(uint32_t u) { return (float)__builtin_bit_cast(h2, u)[1]; }
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// ---------------------------------------------------------------- lane groups
// A row of d elements is spread over LPR = d/16 consecutive lanes, 16 elements
// (16 bytes of INT8 or 32 bytes of FP16) each. Reductions inside a group use
// DPP: quad_perm swaps (xor 1, xor 2) and, for 8-lane groups, the half-row
// mirror (lane i <-> 7-i), which pairs the two quads.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  if constexpr (LPR == 8) v += dpp<0x141>(v);
  return v;
}
template <int LPR>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  if constexpr (LPR == 8) v = fmaxf(v, dpp<0x141>(v));
  return v;
}

// Four signed INT8 codes -> two fp16 pairs, exactly: bias each byte to
// unsigned (x + 128), splice it under the fp16 exponent of 1024 (0x64xx is
// 1024 + xx), then subtract 1152.
__device__ __forceinline__ void i8x4_to_h2(uint32_t w, h2& lo, h2& hi) {
  const uint32_t x = w ^ 0x80808080u;
  const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  lo = as_h2(__builtin_amdgcn_perm(0x64646464u, x, 0x04010400u)) - bias;
  hi = as_h2(__builtin_amdgcn_perm(0x64646464u, x, 0x04030402u)) - bias;
}

__device__ __forceinline__ uint32_t orderable(float f) {
  if (f == 0.0f) f = 0.0f;  // -0 ranks as +0
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// Larger key = kept first: score descending, then position ascending.
__device__ __forceinline__ uint64_t rank_key(float score, int32_t pos) {
  return ((uint64_t)orderable(score) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)pos);
}

// ------------------------------------------------------------ block helpers
// 256 threads = 4 wavefronts of 64.
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t w = __shfl_xor(v, o, 64);
    v = w < v ? w : v;
  }
  return v;
}
__device__ __forceinline__ uint32_t block_sum_u32(uint32_t v, uint32_t* red) {
  v = wave_sum_u32(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const uint32_t r = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return r;
}
__device__ __forceinline__ uint64_t block_min_u64(uint64_t v, uint64_t* red) {
  v = wave_min_u64(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint64_t r = red[0];
  for (int w = 1; w < 4; ++w) r = red[w] < r ? red[w] : r;
  __syncthreads();
  return r;
}
// Exclusive prefix sum over the block in thread order; *total gets the sum.
__device__ __forceinline__ uint32_t block_excl_scan_u32(uint32_t v, uint32_t* red, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = v;
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) red[wave] = inc;
  __syncthreads();
  uint32_t off = 0;
  for (int w = 0; w < wave; ++w) off += red[w];
  *total = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return off + inc - v;
}

// ----------------------------------------------------------------- INT8 row
// Absmax quantization of the 16 elements a lane holds; the group of LPR lanes
// holds one row. scale = fl32(amax / 127) and code = rne(fl32(x / scale)),
// clamped to [-127, 127]; amax == 0 gives scale 0 and zero codes. Both
// quotients are formed in binary64 and rounded once to binary32, which is the
// correctly rounded binary32 quotient (53 >= 2*24 + 2), independent of the
// compiler's float-division mode.
template <int LPR>
__device__ __forceinline__ void quantize16(const uint16_t* src, uint8_t* dst_codes, float* dst_scale, bool lead) {
  const uint4 a = reinterpret_cast<const uint4*>(src)[0];
  const uint4 b = reinterpret_cast<const uint4*>(src)[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  float x[16];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[2 * j] = half_lo(w[j]);
    x[2 * j + 1] = half_hi(w[j]);
  }
  float am = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) am = fmaxf(am, fabsf(x[e]));
  am = group_max<LPR>(am);
  uint32_t packed[4] = {0u, 0u, 0u, 0u};
  float scale = 0.0f;
  if (am > 0.0f) {
    scale = (float)((double)am / 127.0);
    const double sd = (double)scale;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float r = rintf((float)((double)x[e] / sd));
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      packed[e >> 2] |= ((uint32_t)(uint8_t)(int8_t)(int)r) << (8 * (e & 3));
    }
  }
  *reinterpret_cast<uint4*>(dst_codes) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  if (lead) *dst_scale = scale;
}

// ======================================================= logits -> confidence
// [Conf-KV post, pseudocode] p = softmax(logits); c mixes the normalized
// entropy, sigmoid of the top-2 log-prob gap and p_max. Per chunk: M = max z,
// S = sum e^(z-M), T = sum e^(z-M)(z-M) (fp64 accumulation of fp32
// exponentials), top-2 values. Merged over chunks with M* = max M_c:
//   S* = sum S_c e^(M_c-M*),  T* = sum e^(M_c-M*) (T_c + (M_c-M*) S_c),
// so H = log S* - T*/S*, p_max = 1/S*, margin = top1 - top2.
__device__ __forceinline__ void top2_merge(float& a1, float& a2, float b1, float b2) {
  const float hi = fmaxf(a1, b1), lo = fminf(a1, b1);
  a2 = fmaxf(lo, fmaxf(a2, b2));
  a1 = hi;
}

__global__ void __launch_bounds__(256) conf_reduce_kernel(Layout lay, Params par, const float* logits, float* conf_out,
                                                          int32_t* budget_out) {
  __shared__ float s_t1[4], s_t2[4];
  __shared__ double s_S[4], s_T[4];
  __shared__ uint32_t s_bad[4];
  __shared__ int s_last;
  const int b = blockIdx.y, ci = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int V = lay.V;
  const float* z = logits + (size_t)b * V;
  const int begin = ci * kChunk, end = min(V, begin + kChunk);

  float x[16];
  float t1 = -INFINITY, t2 = -INFINITY;
  uint32_t bad = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int idx = begin + tid + 256 * j;
    x[j] = -INFINITY;
    if (idx < end) {
      const float v = z[idx];
      if (!isfinite(v)) {
        bad = 1;
      } else {
        x[j] = v;
        if (v > t1) {
          t2 = t1;
          t1 = v;
        } else if (v > t2) {
          t2 = v;
        }
      }
    }
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
      if (x[j] > -INFINITY) {
        const float dz = x[j] - M;
        const float e = expf(dz);
        S += (double)e;
        T += (double)e * (double)dz;
      }
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
    __threadfence();
    const uint32_t prev = atomicAdd(&lay.row_counter[b], 1u);
    s_last = (prev == (uint32_t)(lay.chunks - 1));
  }
  __syncthreads();
  if (!s_last || wave != 0) return;
  __threadfence();

  // Last chunk of row b: wave 0 merges the partials, one chunk per lane.
  const ConfPartial* parts = lay.partials + (size_t)b * lay.chunks;
  float a1 = -INFINITY, a2 = -INFINITY;
  double pm = -INFINITY, pS = 0.0, pT = 0.0;
  uint32_t badall = 0;
  for (int c0 = 0; c0 < lay.chunks; c0 += 64) {
    const int c = c0 + lane;
    if (c < lay.chunks) {
      const ConfPartial P = parts[c];
      badall |= P.nonfinite;
      top2_merge(a1, a2, P.m, P.top2);
      // fold chunk c into this lane's running (m, S, T)
      const double m2 = (double)P.m;
      if (m2 > -INFINITY) {
        const double mx = fmax(pm, m2);
        const double f1 = pm > -INFINITY ? exp(pm - mx) : 0.0, f2 = exp(m2 - mx);
        pT = f1 * (pT + (pm > -INFINITY ? (pm - mx) * pS : 0.0)) + f2 * (P.T + (m2 - mx) * P.S);
        pS = f1 * pS + f2 * P.S;
        pm = mx;
      }
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float o1 = __shfl_xor(a1, o, 64), o2 = __shfl_xor(a2, o, 64);
    top2_merge(a1, a2, o1, o2);
    badall |= __shfl_xor(badall, o, 64);
    const double qm = __shfl_xor(pm, o, 64), qS = __shfl_xor(pS, o, 64), qT = __shfl_xor(pT, o, 64);
    if (qm > -INFINITY) {
      const double mx = fmax(pm, qm);
      const double f1 = pm > -INFINITY ? exp(pm - mx) : 0.0, f2 = exp(qm - mx);
      pT = f1 * (pT + (pm > -INFINITY ? (pm - mx) * pS : 0.0)) + f2 * (qT + (qm - mx) * qS);
      pS = f1 * pS + f2 * qS;
      pm = mx;
    }
  }
  if (lane != 0) return;
  const double Sx = pS, Tx = pT;
  const double H = log(Sx) - Tx / Sx;
  const double Hn = H / log((double)V);
  const double margin = (double)a1 - (double)a2;
  const double sig = 1.0 / (1.0 + exp(-margin));
  const double cval = (double)par.w_e * (1.0 - Hn) + (double)par.w_m * sig + (double)par.w_p * (1.0 / Sx);
  int base;
  float cout;
  if (badall || !isfinite(cval)) {
    atomicOr(lay.err, kErrNonFinite);
    base = max(par.n_low, par.n_high);
    cout = NAN;
  } else {
    const bool confident = cval >= (double)par.tau;
    if (par.gate_literal)
      base = confident ? par.n_high : par.n_low;
    else
      base = confident ? min(par.n_low, par.n_high) : max(par.n_low, par.n_high);
    cout = (float)cval;
  }
  lay.row_conf[b] = cout;
  lay.row_base[b] = base;
  if (conf_out) conf_out[b] = cout;
  if (budget_out) budget_out[b] = base;
  lay.row_counter[b] = 0;
}

// ================================================== fused attend+evict step
template <bool kLds>
struct Stage {
  float* p;
  int rs;  // row stride of a plane
  __device__ __forceinline__ float& at(int plane, int i) const { return p[plane * rs + i]; }
  __device__ __forceinline__ uint64_t key(int i) const {
    return ((uint64_t)__builtin_bit_cast(uint32_t, p[rs + i]) << 32) | __builtin_bit_cast(uint32_t, p[i]);
  }
  __device__ __forceinline__ void set_key(int i, uint64_t k) const {
    p[i] = __builtin_bit_cast(float, (uint32_t)k);
    p[rs + i] = __builtin_bit_cast(float, (uint32_t)(k >> 32));
  }
  __device__ __forceinline__ int32_t* list(int plane) const { return reinterpret_cast<int32_t*>(p + plane * rs); }
};

// The e-th smallest key (e >= 1) over keys [0, rows): an 8-bit-digit radix
// select from the most significant digit down.
template <bool kLds>
__device__ uint64_t radix_select(const Stage<kLds>& st, int rows, uint32_t e, uint32_t* hist, uint32_t* red,
                                 int32_t* sh) {
  uint64_t prefix = 0, mask = 0;
  const int tid = threadIdx.x;
  for (int shift = 56; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < rows; i += kThreads) {
      const uint64_t k = st.key(i);
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    const uint32_t cnt = hist[tid];
    uint32_t total;
    const uint32_t excl = block_excl_scan_u32(cnt, red, &total);
    if (excl < e && e <= excl + cnt) {
      sh[0] = tid;
      sh[1] = (int32_t)excl;
    }
    __syncthreads();
    const uint32_t bin = (uint32_t)sh[0];
    e -= (uint32_t)sh[1];
    prefix |= (uint64_t)bin << shift;
    mask |= (uint64_t)0xFFu << shift;
    __syncthreads();
  }
  return prefix;
}

template <int D, int G, bool kLds>
__global__ void __launch_bounds__(kThreads, (G <= 2 ? 4 : (G <= 4 ? 3 : 2))) fused_step_kernel(Layout lay, Params par, StepArgs a) {
  constexpr int LPR = D / 16;          // lanes per row
  constexpr int RPB = kThreads / LPR;  // rows per block iteration
  constexpr int PL = G > 4 ? G : 4;    // staging planes
  constexpr int U8 = 8;                // INT8 rows per lane in flight (16 B each)
  constexpr int U16 = 4;               // FP16 rows per lane in flight (32 B each)
  static_assert(LPR == 4 || LPR == 8, "head_dim 64 or 128");

  __shared__ float red_f[4][G];
  __shared__ uint32_t red_u[4];
  __shared__ uint64_t red_k[4];
  __shared__ float obuf[G * D];
  __shared__ uint32_t hist[256];
  __shared__ int32_t sh[4];
  extern __shared__ float dyn_lds[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid % LPR, rg = tid / LPR;
  const int seg = blockIdx.x;
  const int h = seg % lay.Hkv, b = (seg / lay.Hkv) % lay.B, l = seg / (lay.Hkv * lay.B);
  (void)h;
  const int t = a.t, Wr = lay.Wr, ob = lay.old_bytes;
  const bool kvpop = par.policy == 1;

  uint16_t* rk = lay.ring_k + (size_t)seg * Wr * D;
  uint16_t* rv = lay.ring_v + (size_t)seg * Wr * D;
  int32_t* rpos = lay.ring_pos + (size_t)seg * Wr;
  float* rema = lay.ring_ema + (size_t)seg * Wr;
  float* rprio = lay.ring_prio + (size_t)seg * Wr;
  const size_t obase = (size_t)seg * lay.cap;
  uint8_t* okp = lay.old_k + obase * D * ob;
  uint8_t* ovp = lay.old_v + obase * D * ob;
  float* oks = lay.old_ks + obase;
  float* ovs = lay.old_vs + obase;
  int32_t* opos = lay.old_pos + obase;
  float* oema = lay.old_ema + obase;
  float* oprio = lay.old_prio + obase;

  const int n_old = lay.seg_nold[seg];
  const int rows = n_old + Wr;
  Stage<kLds> st;
  if constexpr (kLds) {
    st.p = dyn_lds;
    st.rs = a.lds_rows;
    if (rows > a.lds_rows) {  // the host bound on rows was wrong: refuse, touch nothing
      if (tid == 0) atomicOr(lay.err, kErrInternal);
      return;
    }
  } else {
    st.p = lay.stage + (size_t)seg * PL * lay.rows_max;
    st.rs = lay.rows_max;
  }

  // ---- append the new row (pos t, ema 0) into ring slot t mod Wr. The slot's
  // previous row (pos t - Wr) left the window at the end of the last step.
  const int slot_new = t % Wr;
  {
    const uint4* kn = reinterpret_cast<const uint4*>(a.k_new + (size_t)seg * D);
    const uint4* vn = reinterpret_cast<const uint4*>(a.v_new + (size_t)seg * D);
    if (tid < D / 8)
      reinterpret_cast<uint4*>(rk + (size_t)slot_new * D)[tid] = kn[tid];
    else if (tid < D / 4)
      reinterpret_cast<uint4*>(rv + (size_t)slot_new * D)[tid - D / 8] = vn[tid - D / 8];
    if (tid == 0) {
      rpos[slot_new] = t;
      rema[slot_new] = 0.0f;
      rprio[slot_new] = 0.0f;
      // [KVpop summary §2.3] delayed scoring: the row at t - w gets its
      // priority now, as it stops being protected.
      const int pl = t - par.P;
      if (kvpop && pl >= par.s) {
        const int sl = pl % Wr;
        if (rpos[sl] == pl) rprio[sl] = a.prio_new[seg];
      }
    }
  }
  __syncthreads();

  // ---- QK pass: s_gi = (q_g . k_i) * scale_i * sm_scale, staged per row.
  h2 qh[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint4* qp = reinterpret_cast<const uint4*>(a.q + ((size_t)seg * G + g) * D + c * 16);
    const uint4 x0 = qp[0], x1 = qp[1];
    qh[g][0] = as_h2(x0.x); qh[g][1] = as_h2(x0.y); qh[g][2] = as_h2(x0.z); qh[g][3] = as_h2(x0.w);
    qh[g][4] = as_h2(x1.x); qh[g][5] = as_h2(x1.y); qh[g][6] = as_h2(x1.z); qh[g][7] = as_h2(x1.w);
  }
  const float sm = par.sm_scale;
  float mloc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) mloc[g] = -INFINITY;

  if (par.old_int8) {
    for (int i0 = rg; i0 < n_old; i0 += RPB * U8) {
      uint4 kk[U8];
      float sc[U8];
#pragma unroll
      for (int u = 0; u < U8; ++u) {
        const int i = i0 + u * RPB;
        if (i < n_old) {
          kk[u] = *reinterpret_cast<const uint4*>(okp + (size_t)i * D + c * 16);
          sc[u] = oks[i];
        }
      }
#pragma unroll
      for (int u = 0; u < U8; ++u) {
        const int i = i0 + u * RPB;
        if (i < n_old) {
          h2 kh[8];
          i8x4_to_h2(kk[u].x, kh[0], kh[1]);
          i8x4_to_h2(kk[u].y, kh[2], kh[3]);
          i8x4_to_h2(kk[u].z, kh[4], kh[5]);
          i8x4_to_h2(kk[u].w, kh[6], kh[7]);
          const float f = sc[u] * sm;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_fdot2(kh[j], qh[g][j], acc, false);
            const float s = group_sum<LPR>(acc) * f;
            if (c == 0) st.at(g, i) = s;
            mloc[g] = fmaxf(mloc[g], s);
          }
        }
      }
    }
  } else {
    for (int i0 = rg; i0 < n_old; i0 += RPB * U16) {
      uint4 k0[U16], k1[U16];
#pragma unroll
      for (int u = 0; u < U16; ++u) {
        const int i = i0 + u * RPB;
        if (i < n_old) {
          const uint4* p = reinterpret_cast<const uint4*>(okp + ((size_t)i * D + c * 16) * 2);
          k0[u] = p[0];
          k1[u] = p[1];
        }
      }
#pragma unroll
      for (int u = 0; u < U16; ++u) {
        const int i = i0 + u * RPB;
        if (i < n_old) {
          const h2 kh[8] = {as_h2(k0[u].x), as_h2(k0[u].y), as_h2(k0[u].z), as_h2(k0[u].w),
                            as_h2(k1[u].x), as_h2(k1[u].y), as_h2(k1[u].z), as_h2(k1[u].w)};
#pragma unroll
          for (int g = 0; g < G; ++g) {
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_fdot2(kh[j], qh[g][j], acc, false);
            const float s = group_sum<LPR>(acc) * sm;
            if (c == 0) st.at(g, i) = s;
            mloc[g] = fmaxf(mloc[g], s);
          }
        }
      }
    }
  }
  for (int r0 = rg; r0 < Wr; r0 += RPB * U16) {
    uint4 k0[U16], k1[U16];
    bool live[U16];
#pragma unroll
    for (int u = 0; u < U16; ++u) {
      const int r = r0 + u * RPB;
      live[u] = false;
      if (r < Wr) {
        live[u] = rpos[r] >= 0;
        if (live[u]) {
          const uint4* p = reinterpret_cast<const uint4*>(rk + (size_t)r * D + c * 16);
          k0[u] = p[0];
          k1[u] = p[1];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U16; ++u) {
      const int r = r0 + u * RPB;
      if (r < Wr) {
        if (live[u]) {
          const h2 kh[8] = {as_h2(k0[u].x), as_h2(k0[u].y), as_h2(k0[u].z), as_h2(k0[u].w),
                            as_h2(k1[u].x), as_h2(k1[u].y), as_h2(k1[u].z), as_h2(k1[u].w)};
#pragma unroll
          for (int g = 0; g < G; ++g) {
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_fdot2(kh[j], qh[g][j], acc, false);
            const float s = group_sum<LPR>(acc) * sm;
            if (c == 0) st.at(g, n_old + r) = s;
            mloc[g] = fmaxf(mloc[g], s);
          }
        } else if (c == 0) {
#pragma unroll
          for (int g = 0; g < G; ++g) st.at(g, n_old + r) = -INFINITY;
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float v = wave_max(mloc[g]);
    if (lane == 0) red_f[wave][g] = v;
  }
  __syncthreads();
  float M[G];
#pragma unroll
  for (int g = 0; g < G; ++g) M[g] = fmaxf(fmaxf(red_f[0][g], red_f[1][g]), fmaxf(red_f[2][g], red_f[3][g]));
  __syncthreads();

  // ---- p_gi = exp(s_gi - M_g) in place; l_g = sum_i p_gi.
  float lsum[G];
#pragma unroll
  for (int g = 0; g < G; ++g) lsum[g] = 0.0f;
  for (int i = tid; i < rows; i += kThreads) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float p = __expf(st.at(g, i) - M[g]);
      st.at(g, i) = p;
      lsum[g] += p;
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float v = wave_sum(lsum[g]);
    if (lane == 0) red_f[wave][g] = v;
  }
  __syncthreads();
  float inv_l[G], Lsum[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    Lsum[g] = red_f[0][g] + red_f[1][g] + red_f[2][g] + red_f[3][g];
    inv_l[g] = 1.0f / Lsum[g];
  }

  // ---- PV pass: acc_g += p_gi * v-hat_i. INT8 rows fold the V scale into
  // the weight and use biased-unsigned codes (u = code + 128); the bias is
  // removed once at the end: sum w (u - 128) = sum w u - 128 sum w.
  float acc[G][16];
  float bias[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    bias[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[g][e] = 0.0f;
  }
  if (par.old_int8) {
    for (int i0 = rg; i0 < n_old; i0 += RPB * U8) {
      uint4 vv[U8];
      float sc[U8];
#pragma unroll
      for (int u = 0; u < U8; ++u) {
        const int i = i0 + u * RPB;
        if (i < n_old) {
          vv[u] = *reinterpret_cast<const uint4*>(ovp + (size_t)i * D + c * 16);
          sc[u] = ovs[i];
        }
      }
#pragma unroll
      for (int u = 0; u < U8; ++u) {
        const int i = i0 + u * RPB;
        if (i < n_old) {
          const uint32_t w4[4] = {vv[u].x ^ 0x80808080u, vv[u].y ^ 0x80808080u, vv[u].z ^ 0x80808080u,
                                  vv[u].w ^ 0x80808080u};
          float f[16];
#pragma unroll
          for (int e = 0; e < 16; ++e) f[e] = (float)((w4[e >> 2] >> (8 * (e & 3))) & 0xFFu);
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float w = st.at(g, i) * sc[u];
            bias[g] += w;
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[g][e] = fmaf(w, f[e], acc[g][e]);
          }
        }
      }
    }
  } else {
    for (int i0 = rg; i0 < n_old; i0 += RPB * U16) {
      uint4 v0[U16], v1[U16];
#pragma unroll
      for (int u = 0; u < U16; ++u) {
        const int i = i0 + u * RPB;
        if (i < n_old) {
          const uint4* p = reinterpret_cast<const uint4*>(ovp + ((size_t)i * D + c * 16) * 2);
          v0[u] = p[0];
          v1[u] = p[1];
        }
      }
#pragma unroll
      for (int u = 0; u < U16; ++u) {
        const int i = i0 + u * RPB;
        if (i < n_old) {
          const uint32_t w8[8] = {v0[u].x, v0[u].y, v0[u].z, v0[u].w, v1[u].x, v1[u].y, v1[u].z, v1[u].w};
          float f[16];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            f[2 * j] = half_lo(w8[j]);
            f[2 * j + 1] = half_hi(w8[j]);
          }
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float w = st.at(g, i);
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[g][e] = fmaf(w, f[e], acc[g][e]);
          }
        }
      }
    }
  }
  for (int r0 = rg; r0 < Wr; r0 += RPB * U16) {
    uint4 v0[U16], v1[U16];
    bool live[U16];
#pragma unroll
    for (int u = 0; u < U16; ++u) {
      const int r = r0 + u * RPB;
      live[u] = false;
      if (r < Wr) {
        live[u] = rpos[r] >= 0;
        if (live[u]) {
          const uint4* p = reinterpret_cast<const uint4*>(rv + (size_t)r * D + c * 16);
          v0[u] = p[0];
          v1[u] = p[1];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U16; ++u) {
      const int r = r0 + u * RPB;
      if (r < Wr && live[u]) {
        const uint32_t w8[8] = {v0[u].x, v0[u].y, v0[u].z, v0[u].w, v1[u].x, v1[u].y, v1[u].z, v1[u].w};
        float f[16];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          f[2 * j] = half_lo(w8[j]);
          f[2 * j + 1] = half_hi(w8[j]);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float w = st.at(g, n_old + r);
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[g][e] = fmaf(w, f[e], acc[g][e]);
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float v = fmaf(-128.0f, bias[g], acc[g][e]);
      for (int o = LPR; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
      acc[g][e] = v;
    }
  }
  // Lanes 0..LPR-1 of each wave hold the wave's sums; add the waves in order.
  for (int w = 0; w < 4; ++w) {
    if (wave == w && lane < LPR) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int idx = g * D + lane * 16 + e;
          obuf[idx] = (w == 0 ? 0.0f : obuf[idx]) + acc[g][e];
        }
      }
    }
    __syncthreads();
  }
  for (int idx = tid; idx < G * D; idx += kThreads)
    a.out[(size_t)seg * G * D + idx] = f2h(obuf[idx] * inv_l[idx / D]);

  // ---- mass, EMA, score, key. [Conf-KV post] ema of the attention mass,
  // score = alpha*ema + (1-alpha)*recency; KVpop ranks by its priority.
  // Keys overwrite planes 0/1 of the row just read (same thread).
  uint32_t n_live = 0, n_elig = 0;
  const float inv_t1 = 1.0f;  // (kept explicit below: IEEE division per row)
  (void)inv_t1;
  for (int i = tid; i < rows; i += kThreads) {
    const bool in_old = i < n_old;
    const int r = i - n_old;
    const int32_t pos = in_old ? opos[i] : rpos[r];
    uint64_t key = ~0ull;
    float score = NAN;
    if (pos >= 0) {
      ++n_live;
      if (!kvpop) {
        float mass = 0.0f;
#pragma unroll
        for (int g = 0; g < G; ++g) mass = fmaf(st.at(g, i), inv_l[g], mass);
        mass *= (1.0f / (float)G);
        float* ep = in_old ? (oema + i) : (rema + r);
        const float e = par.beta * (*ep) + (1.0f - par.beta) * mass;
        *ep = e;
        const float rec = (float)(pos + 1) / (float)(t + 1);
        score = par.alpha * e + (1.0f - par.alpha) * rec;
      } else {
        score = in_old ? oprio[i] : rprio[r];
      }
      const bool elig = pos >= par.s && pos <= t - par.P;
      if (!isfinite(score)) {
        atomicOr(lay.err, kErrNonFinite);
      } else if (elig) {
        key = rank_key(score, pos);
        ++n_elig;
      }
    }
    st.set_key(i, key);
    if (par.record) {
      lay.rec_pos[(size_t)seg * lay.rows_max + i] = pos;
      lay.rec_score[(size_t)seg * lay.rows_max + i] = pos >= 0 ? score : NAN;
    }
  }
  n_live = block_sum_u32(n_live, red_u);
  n_elig = block_sum_u32(n_elig, red_u);

  // ---- budget and selection of the e lowest keys among the eligible rows.
  int budget;
  if (!kvpop) {
    const long long base = lay.row_base[b];
    budget = (par.pyramid && lay.L > 1)
                 ? (int)((base * (long long)(3 * (lay.L - 1) - 2 * l)) / (long long)(2 * (lay.L - 1)))
                 : (int)base;
  } else {
    budget = par.s + par.P + par.kvpop_k;
  }
  uint32_t e = 0;
  if ((int)n_live > budget) e = min((uint32_t)((int)n_live - budget), n_elig);
  uint64_t T = 0;  // victims: key <= T (no key is 0)
  if (e > 0 && e <= 8) {
    for (uint32_t r = 0; r < e; ++r) {
      uint64_t m = ~0ull;
      for (int i = tid; i < rows; i += kThreads) {
        const uint64_t k = st.key(i);
        if (k > T && k < m) m = k;
      }
      T = block_min_u64(m, red_k);
    }
  } else if (e > 8) {
    T = radix_select(st, rows, e, hist, red_u, sh);
  }

  // ---- compaction of the old region: victims below the new count m become
  // holes, filled in ascending order by the survivors at or above m.
  uint32_t ev_old = 0;
  if (e > 0)
    for (int i = tid; i < n_old; i += kThreads) ev_old += st.key(i) <= T ? 1u : 0u;
  ev_old = block_sum_u32(ev_old, red_u);
  const int m = n_old - (int)ev_old;
  uint32_t moved = 0;
  if (ev_old > 0) {
    const int per = (n_old + kThreads - 1) / kThreads;
    const int lo = min(n_old, tid * per), hi = min(n_old, lo + per);
    uint32_t hv = 0, sv = 0;
    for (int i = lo; i < hi; ++i) {
      const bool v = st.key(i) <= T;
      hv += (v && i < m) ? 1u : 0u;
      sv += (!v && i >= m) ? 1u : 0u;
    }
    uint32_t nh, ns;
    uint32_t ho = block_excl_scan_u32(hv, red_u, &nh);
    uint32_t so = block_excl_scan_u32(sv, red_u, &ns);
    int32_t* holes = st.list(2);
    int32_t* srcs = st.list(3);
    for (int i = lo; i < hi; ++i) {
      const bool v = st.key(i) <= T;
      if (v && i < m) holes[ho++] = i;
      if (!v && i >= m) srcs[so++] = i;
    }
    __syncthreads();
    moved = nh;
    for (int r = rg; r < (int)nh; r += RPB) {
      const int src = srcs[r], dst = holes[r];
      const size_t rb = (size_t)D * ob;
      const int cb = 16 * ob;  // bytes per lane
      for (int off = 0; off < cb; off += 16) {
        *reinterpret_cast<uint4*>(okp + dst * rb + c * cb + off) =
            *reinterpret_cast<const uint4*>(okp + src * rb + c * cb + off);
        *reinterpret_cast<uint4*>(ovp + dst * rb + c * cb + off) =
            *reinterpret_cast<const uint4*>(ovp + src * rb + c * cb + off);
      }
      if (c == 0) {
        opos[dst] = opos[src];
        oema[dst] = oema[src];
        oprio[dst] = oprio[src];
        oks[dst] = oks[src];
        ovs[dst] = ovs[src];
      }
    }
  }
  if (e > 0)
    for (int r = tid; r < Wr; r += kThreads)
      if (st.key(n_old + r) <= T) rpos[r] = -1;
  __syncthreads();

  // ---- age-out: the row at t - W leaves the FP16 window; if it survived it
  // is appended to the old region, quantized when old rows are INT8.
  int n_old_new = m;
  bool aged = false;
  const int pos_out = t - lay.W;
  if (pos_out >= 0 && wave == 0) {
    const int slot = pos_out % Wr;
    const bool alive = rpos[slot] == pos_out;
    if (alive) {
      if (m >= lay.cap) {
        if (lane == 0) atomicOr(lay.err, kErrCapacity);
      } else {
        if (lane < 2 * LPR) {
          const bool isv = lane >= LPR;
          const int cc = lane % LPR;
          const uint16_t* src = (isv ? rv : rk) + (size_t)slot * D + cc * 16;
          uint8_t* dst = (isv ? ovp : okp) + (size_t)m * D * ob;
          if (par.old_int8) {
            quantize16<LPR>(src, dst + cc * 16, (isv ? ovs : oks) + m, cc == 0);
          } else {
            const uint4* s4 = reinterpret_cast<const uint4*>(src);
            uint4* d4 = reinterpret_cast<uint4*>(dst + cc * 32);
            d4[0] = s4[0];
            d4[1] = s4[1];
          }
        }
        if (lane == 0) {
          opos[m] = pos_out;
          oema[m] = rema[slot];
          oprio[m] = rprio[slot];
          if (!par.old_int8) {
            oks[m] = 0.0f;
            ovs[m] = 0.0f;
          }
          rpos[slot] = -1;
        }
        aged = true;
        n_old_new = m + 1;
      }
    }
  }
  if (tid == 0) {
    lay.seg_nold[seg] = n_old_new;
    const uint64_t live_ring = (uint64_t)n_live - (uint64_t)n_old;
    const uint64_t old_row = par.old_int8 ? (uint64_t)(2 * D + 8) : (uint64_t)(4 * D);
    uint64_t* sp = lay.seg_stats + (size_t)seg * kStatFields;
    sp[0] += (uint64_t)n_old * old_row + live_ring * (uint64_t)(4 * D);
    sp[1] += n_live;
    sp[2] += moved + (aged ? 1u : 0u);
    sp[3] += e;
    if (par.record) {
      int32_t* mp = lay.rec_meta + (size_t)seg * 4;
      mp[0] = rows;
      mp[1] = (int32_t)n_live;
      mp[2] = budget;
      mp[3] = (int32_t)e;
#pragma unroll
      for (int g = 0; g < G; ++g) lay.rec_lse[(size_t)seg * G + g] = M[g] + logf(Lsum[g]);
    }
  }
}

// ================================================================ init/ingest
__global__ void init_meta_kernel(Layout lay, int32_t n_old_init) {
  const int seg = blockIdx.x, tid = threadIdx.x;
  for (int r = tid; r < lay.Wr; r += blockDim.x) {
    lay.ring_pos[(size_t)seg * lay.Wr + r] = -1;
    lay.ring_ema[(size_t)seg * lay.Wr + r] = 0.0f;
    lay.ring_prio[(size_t)seg * lay.Wr + r] = 0.0f;
  }
  if (tid < kStatFields) lay.seg_stats[(size_t)seg * kStatFields + tid] = 0;
  if (tid == 0) lay.seg_nold[seg] = n_old_init;
  if (seg == 0) {
    for (int i = tid; i < lay.B; i += blockDim.x) {
      lay.row_counter[i] = 0;
      lay.row_base[i] = 0;
      lay.row_conf[i] = 0.0f;
    }
    if (tid == 0) *lay.err = 0;
  }
}

// Prefill row p of segment seg: pos <= P0-1-W goes to old row p (quantized when
// old rows are INT8), the rest to ring slot p mod Wr.
template <int D>
__global__ void __launch_bounds__(256) ingest_kernel(Layout lay, Params par, const uint16_t* pk, const uint16_t* pv,
                                                     int32_t P0) {
  constexpr int LPR = D / 16, RPB = 256 / LPR;
  const int seg = blockIdx.y, tid = threadIdx.x, c = tid % LPR;
  const int p = blockIdx.x * RPB + tid / LPR;
  if (p >= P0) return;  // whole lane groups leave together
  const int n_old_init = max(0, P0 - lay.W);
  const uint16_t* ks = pk + ((size_t)seg * P0 + p) * D + c * 16;
  const uint16_t* vs = pv + ((size_t)seg * P0 + p) * D + c * 16;
  const int ob = lay.old_bytes;
  if (p < n_old_init) {
    const size_t row = (size_t)seg * lay.cap + p;
    uint8_t* dk = lay.old_k + row * D * ob;
    uint8_t* dv = lay.old_v + row * D * ob;
    if (par.old_int8) {
      quantize16<LPR>(ks, dk + c * 16, lay.old_ks + row, c == 0);
      quantize16<LPR>(vs, dv + c * 16, lay.old_vs + row, c == 0);
    } else {
      reinterpret_cast<uint4*>(dk + c * 32)[0] = reinterpret_cast<const uint4*>(ks)[0];
      reinterpret_cast<uint4*>(dk + c * 32)[1] = reinterpret_cast<const uint4*>(ks)[1];
      reinterpret_cast<uint4*>(dv + c * 32)[0] = reinterpret_cast<const uint4*>(vs)[0];
      reinterpret_cast<uint4*>(dv + c * 32)[1] = reinterpret_cast<const uint4*>(vs)[1];
      if (c == 0) {
        lay.old_ks[row] = 0.0f;
        lay.old_vs[row] = 0.0f;
      }
    }
    if (c == 0) {
      lay.old_pos[row] = p;
      lay.old_ema[row] = 0.0f;
      lay.old_prio[row] = 0.0f;
    }
  } else {
    const int slot = p % lay.Wr;
    const size_t row = (size_t)seg * lay.Wr + slot;
    uint4* dk = reinterpret_cast<uint4*>(lay.ring_k + row * D + c * 16);
    uint4* dv = reinterpret_cast<uint4*>(lay.ring_v + row * D + c * 16);
    dk[0] = reinterpret_cast<const uint4*>(ks)[0];
    dk[1] = reinterpret_cast<const uint4*>(ks)[1];
    dv[0] = reinterpret_cast<const uint4*>(vs)[0];
    dv[1] = reinterpret_cast<const uint4*>(vs)[1];
    if (c == 0) {
      lay.ring_pos[row] = p;
      lay.ring_ema[row] = 0.0f;
      lay.ring_prio[row] = 0.0f;
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
  const int D = lay.D, Wr = lay.Wr, ob = lay.old_bytes;
  const int n_old = lay.seg_nold[seg];
  const int32_t* opos = lay.old_pos + (size_t)seg * lay.cap;
  const int32_t* rpos = lay.ring_pos + (size_t)seg * Wr;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    int live = 0;
    for (int r = 0; r < Wr; ++r) live += rpos[r] >= 0;
    len[si] = n_old + live;
  }
  if (i >= n_old + Wr) return;
  const bool in_old = i < n_old;
  const int32_t pos = in_old ? opos[i] : rpos[i - n_old];
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
  const size_t src = in_old ? (size_t)seg * lay.cap + i : (size_t)seg * Wr + (i - n_old);
  if (ema_o) ema_o[orow] = in_old ? lay.old_ema[src] : lay.ring_ema[src];
  if (prio_o) prio_o[orow] = in_old ? lay.old_prio[src] : lay.ring_prio[src];
  if (ks_o) ks_o[orow] = row8 ? lay.old_ks[src] : 0.0f;
  if (vs_o) vs_o[orow] = row8 ? lay.old_vs[src] : 0.0f;
  for (int e = 0; e < D; ++e) {
    uint16_t hk = 0, hv = 0;
    int8_t ck = 0, cv = 0;
    if (row8) {
      ck = (int8_t)lay.old_k[src * D + e];
      cv = (int8_t)lay.old_v[src * D + e];
    } else if (in_old) {
      hk = reinterpret_cast<const uint16_t*>(lay.old_k)[src * D + e];
      hv = reinterpret_cast<const uint16_t*>(lay.old_v)[src * D + e];
    } else {
      hk = lay.ring_k[src * D + e];
      hv = lay.ring_v[src * D + e];
    }
    if (k16) k16[orow * D + e] = hk;
    if (v16) v16[orow * D + e] = hv;
    if (k8) k8[orow * D + e] = ck;
    if (v8) v8[orow * D + e] = cv;
  }
  (void)ob;
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
static inline int ok_or_err() { return hipGetLastError() == hipSuccess ? 0 : -3; }

int launch_init(const Layout& lay, const Params& par, const uint16_t* pk, const uint16_t* pv, int32_t P0,
                void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int32_t n_old_init = P0 > lay.W ? P0 - lay.W : 0;
  hipLaunchKernelGGL(init_meta_kernel, dim3(lay.S), dim3(256), 0, s, lay, n_old_init);
  if (hipGetLastError() != hipSuccess) return -3;
  if (P0 > 0) {
    const int rpb = 256 / (lay.D / 16);
    const dim3 grid((P0 + rpb - 1) / rpb, lay.S);
    if (lay.D == 64)
      hipLaunchKernelGGL(ingest_kernel<64>, grid, dim3(256), 0, s, lay, par, pk, pv, P0);
    else
      hipLaunchKernelGGL(ingest_kernel<128>, grid, dim3(256), 0, s, lay, par, pk, pv, P0);
  }
  return ok_or_err();
}

int launch_conf_reduce(const Layout& lay, const Params& par, const float* logits, float* conf_out,
                       int32_t* budget_out, void* stream) {
  hipLaunchKernelGGL(conf_reduce_kernel, dim3(lay.chunks, lay.B), dim3(256), 0, (hipStream_t)stream, lay, par,
                     logits, conf_out, budget_out);
  return ok_or_err();
}

template <int D, int G>
static void launch_fused_dg(const Layout& lay, const Params& par, const StepArgs& a, bool use_lds, int lds_bytes,
                            hipStream_t s) {
  if (use_lds)
    hipLaunchKernelGGL((fused_step_kernel<D, G, true>), dim3(lay.S), dim3(kThreads), lds_bytes, s, lay, par, a);
  else
    hipLaunchKernelGGL((fused_step_kernel<D, G, false>), dim3(lay.S), dim3(kThreads), 0, s, lay, par, a);
}

template <int D>
static int launch_fused_d(const Layout& lay, const Params& par, const StepArgs& a, bool use_lds, int lds_bytes,
                          hipStream_t s) {
  switch (lay.G) {
    case 1: launch_fused_dg<D, 1>(lay, par, a, use_lds, lds_bytes, s); break;
    case 2: launch_fused_dg<D, 2>(lay, par, a, use_lds, lds_bytes, s); break;
    case 4: launch_fused_dg<D, 4>(lay, par, a, use_lds, lds_bytes, s); break;
    case 5: launch_fused_dg<D, 5>(lay, par, a, use_lds, lds_bytes, s); break;
    case 8: launch_fused_dg<D, 8>(lay, par, a, use_lds, lds_bytes, s); break;
    default: return -1;
  }
  return ok_or_err();
}

int launch_fused_step(const Layout& lay, const Params& par, const StepArgs& a, bool use_lds, int lds_bytes,
                      void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (lay.D == 64) return launch_fused_d<64>(lay, par, a, use_lds, lds_bytes, s);
  if (lay.D == 128) return launch_fused_d<128>(lay, par, a, use_lds, lds_bytes, s);
  return -1;
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
