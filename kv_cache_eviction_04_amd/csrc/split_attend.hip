// HIP kernels for gfx950 (MI355X): one layer's attention at the layer
// boundary, split over several workgroups per segment (split-K), and its
// log-sum-exp combine.
//
// Sources: CONF-KV abstract (chatpaper.ai); "Conf-KV" post (rcap.io), method
// paragraph; "Resumen Técnico: KVpop" (gist.science) §2.3.
#include "device.h"

namespace confkv {

// ========================================================= split-K attend
// One layer's attend with ns workgroups per segment, for launches whose
// B*Hkv segments alone would leave most CUs idle. Split c of a segment takes
// the run of 32-row stage tiles [c*T/ns, (c+1)*T/ns) (T tiles in all: the
// old region, then the ring) and computes, per query head, its own maximum
// m_c, sum l_c = sum exp(s - m_c) and unnormalised PV partial O_c, and
// stores the raw scores s of its rows in the segment's HBM stage (planes
// 0..G-1). The split holding the new row's slot appends it. A second launch,
// one workgroup per segment, combines [CONF-KV abstract: blockwise
// online-softmax attention]:
//   M = max_c m_c, L = sum_c l_c e^(m_c - M), out = sum_c O_c e^(m_c - M) / L,
//   LSE = M + log L,
// and stores each head's LSE. Under CONF the evict launch after the last
// layer updates every live row's EMA from the stored scores and LSEs (mass =
// mean over the G heads of exp(s - LSE)), for all layers at once. The launch
// boundary orders split and combine: a device-scope fence per workgroup
// would write back and invalidate its XCD's whole L2.
// Arithmetic per split is that of the whole-segment kernel.
template <int D, int G>
__global__ void __launch_bounds__(kThreads, (G <= 4 ? CONFKV_OCC : 3)) attend_split_kernel(Layout lay, Params par,
                                                                                           StepArgs a) {
  constexpr int KS = D / 32;           // MFMA k-steps over d
  constexpr int NCB = D / 16;          // 16-column blocks of d
  constexpr int CBW = NCB / 4;         // PV column blocks per wave
  static_assert(G <= 16, "a GQA group fits one MFMA tile");

  __shared__ float red_m[4][G], red_l[4][G];
  __shared__ uint32_t red_u[4];
  extern __shared__ float dyn_lds[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lq = lane >> 4, lj = lane & 15;
  const int ns = a.ns;
  const int sl = blockIdx.x / ns, c = blockIdx.x - sl * ns;  // local segment, split
  const int seg = a.seg0 + sl;
  const int t = a.t, Wr = lay.Wr, Wr32 = lay.Wr32;
  const bool kvpop = par.policy == 1;

  uint16_t* rk = lay.ring_k + (size_t)seg * Wr32 * D;
  uint16_t* rvt = lay.ring_v + (size_t)seg * Wr32 * D;
  const size_t obase = (size_t)seg * lay.cap32;
  const uint8_t* okp = lay.old_k + obase * D * lay.old_bytes;
  const uint8_t* ovt = lay.old_v + obase * D * lay.old_bytes;
  const float* oks = lay.old_ks + obase;
  const float* ovs = lay.old_vs + obase;
  const size_t sbase = (size_t)seg * lay.rows_max;
  int32_t* opos = lay.row_pos + sbase;
  float* oema = lay.row_ema + sbase;
  int32_t* rpos = opos + lay.cap32;
  float* rema = oema + lay.cap32;
  float* rprio = lay.row_prio + sbase + lay.cap32;

  const int n_old = lay.seg_nold[seg];
  const int n_old32 = (n_old + 31) & ~31;
  const int rows = n_old32 + Wr32;
  const int T = rows >> 5;
  const int r0 = (int)(((long long)c * T) / ns) * 32;
  int r1 = (int)(((long long)(c + 1) * T) / ns) * 32;
  // The host sizes the LDS planes for the longest run a split can get;
  // should a run be longer, it is cut (every access stays in bounds) and an
  // internal error is raised.
  const bool cut = r1 - r0 > a.lds_rows;
  if (cut) r1 = r0 + a.lds_rows;
  const int rs = a.lds_rows;
  auto st = [&](int g, int j) -> float& { return dyn_lds[g * rs + j]; };
  float* svl = dyn_lds + G * rs;  // V scales of the run's old rows (from the QK loads)

  const int slot_new = t % Wr;
  const int i_new = n_old32 + slot_new;
  const bool owner = i_new >= r0 && i_new < r1;  // this split appends the new row
  const int pos_prio = (kvpop && t - par.P >= par.s) ? t - par.P : -1;
  const uint16_t* kn = a.k_new + (size_t)sl * D;

  // ---- q as MFMA A operands (see the whole-segment kernel)
  const uint16_t* qrow = a.q + ((size_t)sl * G + (lj < G ? lj : 0)) * D;
  half8 qa8[KS], qa16[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const uint4 u16 = *reinterpret_cast<const uint4*>(qrow + 8 * (lq + 4 * kk));
    qa16[kk] = lj < G ? as_h8(u16) : half8{};
  }
  uint4 kn4 = make_uint4(0u, 0u, 0u, 0u);
  uint16_t vn1 = 0;
  float prio_now = 0.0f;
  int32_t pos_prio_slot = -1;
  if (owner) {
    kn4 = reinterpret_cast<const uint4*>(kn)[tid % (D / 8)];
    vn1 = a.v_new[(size_t)sl * D + tid % D];
    if (pos_prio >= 0) {
      prio_now = a.prio_new[sl];
      pos_prio_slot = rpos[pos_prio % Wr];
    }
  }

  const float sm = par.sm_scale;
  float mrun[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  float sv_max = 0.0f;
  // ---- ring QK over this run's ring slots [ra, rb)
  const int ra = max(r0, n_old32) - n_old32, rb = r1 - n_old32;
  if (rb > ra) {
    const int nt_ring = (Wr + 15) >> 4;
    const int g0 = ra >> 4, g1 = min(rb >> 4, nt_ring);
    const int n = max(g1 - g0, 0);
    const int ta = g0 + ((wave * n) >> 2), tb = g0 + (((wave + 1) * n) >> 2);
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
              st(g, n_old32 + r - r0) = sc;
              mrun[rr] = fmaxf(mrun[rr], sc);
            }
          }
        });
    for (int r = max(ra, 16 * nt_ring) + tid; r < rb; r += kThreads)
#pragma unroll
      for (int g = 0; g < G; ++g) st(g, n_old32 + r - r0) = -INFINITY;
  }
  // ---- append of the new row by the split that holds its slot (the slot's
  // previous row left the window at the end of the last step)
  if (owner) {
    if (tid < D / 8) reinterpret_cast<uint4*>(rk + (size_t)slot_new * D)[tid] = kn4;
    if (tid < D) rvt[vt16(slot_new, tid, D)] = vn1;
    if (tid == 0) {
      rpos[slot_new] = t;
      rema[slot_new] = 0.0f;
      rprio[slot_new] = 0.0f;
      // [KVpop summary §2.3] delayed scoring
      if (pos_prio >= 0 && pos_prio_slot == pos_prio) rprio[pos_prio % Wr] = prio_now;
    }
  }
  // ---- old-region QK over this run's old rows [r0, oe)
  const int oe = min(r1, n_old32);
  if (oe > r0) {
    const int n = (oe - r0) >> 4;
    const int ta = (r0 >> 4) + ((wave * n) >> 2), tb = (r0 >> 4) + (((wave + 1) * n) >> 2);
    if (par.old_int8) {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const uint4 u8 = *reinterpret_cast<const uint4*>(qrow + 16 * (lq + 4 * (kk >> 1)) + 8 * (kk & 1));
        qa8[kk] = lj < G ? as_h8(u8) : half8{};
      }
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
            if (valid) sv_max = fmaxf(sv_max, bf.sv);
            if (lq == 0) svl[row - r0] = bf.sv;
            const float f = bf.sk * sm;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int g = 4 * lq + r;
              if (g < G) {
                const float sc = valid ? acc[r] * f : -INFINITY;
                st(g, row - r0) = sc;
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
                st(g, row - r0) = sc;
                mrun[r] = fmaxf(mrun[r], sc);
              }
            }
          });
    }
  }
  // ---- the first batch of this run's INT8 V tiles, loaded now so that the
  // loads overlap the maxima barrier and the weight pass
  const int pv_t0 = r0 >> 5, pv_t1 = oe > r0 ? oe >> 5 : pv_t0;
  constexpr int NPRE = CONFKV_PV8_NPB;
  PV8Buf vpre[NPRE];
  auto load_pv8 = [&](int tt, PV8Buf& bf) {
    const uint8_t* tb = ovt + (size_t)tt * 32 * D + 16 * (32 * tt + 8 * lq < n_old ? lane : lj);
    if constexpr (CBW == 2) {
      bf.v = ldnt4(tb + 1024 * wave);
    } else {
      const uint2 hh = ldnt2(tb + 1024 * (wave >> 1) + 8 * (wave & 1));
      bf.v = make_uint4(hh.x, hh.y, 0u, 0u);
    }
  };
  if (par.old_int8) {
#pragma unroll
    for (int u = 0; u < NPRE; ++u)
      if (pv_t0 + u < pv_t1) load_pv8(pv_t0 + u, vpre[u]);
  }
  // ---- this run's maxima per head and of the INT8 V scales
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float m = mrun[r];
    m = row16_reduce(m, [](float x, float y) { return fmaxf(x, y); });
    const int g = 4 * lq + r;
    if (lj == 0 && g < G) red_m[wave][g] = m;
  }
  sv_max = wave_max(sv_max);
  if (lane == 0) red_u[wave] = __builtin_bit_cast(uint32_t, sv_max);
  __syncthreads();
  float Mc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) Mc[g] = fmaxf(fmaxf(red_m[0][g], red_m[1][g]), fmaxf(red_m[2][g], red_m[3][g]));
  float svm = 0.0f;
  for (int w = 0; w < 4; ++w) svm = fmaxf(svm, __builtin_bit_cast(float, red_u[w]));
  int fexp = 10;
  if (svm > 0.0f) {
    int e2;
    frexpf(svm, &e2);
    fexp = min(10, max(-30, 14 - e2));
  }
  const float fscale = ldexpf(1.0f, fexp), finv = ldexpf(1.0f, -fexp);

  // ---- weights: p = exp(s - m_c) (0 for a run without a valid row), the
  // raw scores kept for the evict launch's EMA pass
  float lpart[G];
#pragma unroll
  for (int g = 0; g < G; ++g) lpart[g] = 0.0f;
  float* sco = lay.stage + (size_t)seg * lay.planes * lay.rows_max;  // planes 0..G-1 of the segment's stage
  for (int j = tid; j < r1 - r0; j += kThreads) {
    const int i = r0 + j;
    const float sv = (i < n_old && par.old_int8) ? svl[j] : 0.0f;
    const float scf = ((i < n_old && par.old_int8 && sv > 0.0f) ? sv : 1.0f) * fscale;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float s = st(g, j);
      if (!kvpop) sco[(size_t)g * lay.rows_max + i] = s;
      const float p = Mc[g] == -INFINITY ? 0.0f : __expf(s - Mc[g]);
      lpart[g] += p;
      const float wv = p * scf;
      const _Float16 hi = (_Float16)wv, lo = (_Float16)(wv - (float)hi);
      st(g, j) = __builtin_bit_cast(float, (uint32_t)__builtin_bit_cast(uint16_t, hi) |
                                                ((uint32_t)__builtin_bit_cast(uint16_t, lo) << 16));
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float v = wave_sum(lpart[g]);
    if (lane == 0) red_l[wave][g] = v;
  }
  __syncthreads();

  // ---- PV over this run's 32-row tiles (waves split the columns)
  floatx4 O[CBW];
#pragma unroll
  for (int k = 0; k < CBW; ++k) O[k] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  auto weights = [&](int j, half8& ahi, half8& alo) {  // local stage row j
    if (lj < G) {
      const float4 p0 = *reinterpret_cast<const float4*>(&st(lj, j));
      const float4 p1 = *reinterpret_cast<const float4*>(&st(lj, j + 4));
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
    } else {
      ahi = half8{};
      alo = half8{};
    }
  };
  // tiles [t0, t1) of vbase, local stage row j0 + 32*(tt-t0); lanes whose 8
  // rows lie past the region's nvalid rows read lane group 0's
  auto pv16 = [&](const uint16_t* vbase, int j0, int t0, int t1, int nvalid) {
    pipelined<CONFKV_PV16_NPB, PV16Buf<CBW>>(
        t0, t1,
        [&](int tt, PV16Buf<CBW>& bf) {
          const uint16_t* tb = vbase + (size_t)tt * 32 * D + 8 * (32 * tt + 8 * lq < nvalid ? lane : lj);
#pragma unroll
          for (int k = 0; k < CBW; ++k) bf.v[k] = ldnt4(tb + 512 * (CBW * wave + k));
        },
        [&](int tt, const PV16Buf<CBW>& bf) {
          half8 ahi, alo;
          weights(j0 + 32 * (tt - t0) + 8 * lq, ahi, alo);
#pragma unroll
          for (int k = 0; k < CBW; ++k) {
            O[k] = mfma16(ahi, as_h8(bf.v[k]), O[k]);
            O[k] = mfma16(alo, as_h8(bf.v[k]), O[k]);
          }
        });
  };
  if (oe > r0) {
    const int t0 = r0 >> 5, t1 = oe >> 5;
    if (par.old_int8) {
      auto pv8 = [&](int tt, const PV8Buf& bf) {
        half8 ahi, alo, blo, bhi;
        weights(32 * tt - r0 + 8 * lq, ahi, alo);
        i8x16_to_h8(bf.v, blo, bhi);
        O[0] = mfma16(ahi, blo, O[0]);
        O[0] = mfma16(alo, blo, O[0]);
        if constexpr (CBW == 2) {
          O[1] = mfma16(ahi, bhi, O[1]);
          O[1] = mfma16(alo, bhi, O[1]);
        }
      };
#pragma unroll
      for (int u = 0; u < NPRE; ++u)
        if (t0 + u < t1) pv8(t0 + u, vpre[u]);
      pipelined<CONFKV_PV8_NPB, PV8Buf>(t0 + NPRE, t1, load_pv8, pv8);
    } else {
      pv16(reinterpret_cast<const uint16_t*>(ovt), 0, t0, t1, n_old);
    }
  }
  if (rb > ra) pv16(rvt, max(r0, n_old32) - r0, ra >> 5, rb >> 5, Wr);

  // ---- this split's partials: O_c (unnormalised, f removed), m_c, l_c
  const size_t pbase = (size_t)sl * lay.ns_max + c;
#pragma unroll
  for (int k = 0; k < CBW; ++k) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int g = 4 * lq + r;
      if (g < G) lay.sk_o[(pbase * G + g) * D + 16 * (CBW * wave + k) + lj] = O[k][r] * finv;
    }
  }
  if (tid < G) {
    const float l = red_l[0][tid] + red_l[1][tid] + red_l[2][tid] + red_l[3][tid];
    lay.sk_ml[pbase * G + tid] = SplitML{Mc[tid], l};
  }
  if (tid == 0 && cut) atomicOr(lay.err, kErrInternal);
}

// The combine of a split-K attend: one workgroup per segment of the layer.
// The splits' statistics go through LDS once; every load that follows is
// issued in batches, so the combine costs a few load latencies.
template <int D, int G>
__global__ void __launch_bounds__(kThreads) attend_combine_kernel(Layout lay, Params par, StepArgs a) {
  constexpr int KMAX = 32;  // most splits per segment
  __shared__ float sh_m[G][KMAX], sh_l[G][KMAX], sh_f[G][KMAX];
  __shared__ float sh_lse[G];
  const int tid = threadIdx.x;
  const int ns = a.ns;
  const int sl = blockIdx.x, seg = a.seg0 + sl;
  const size_t pbase = (size_t)sl * lay.ns_max;
  // the first KPRE splits' partials of this thread's output elements are
  // loaded before the statistics, so both round trips overlap
  constexpr int EPT = (G * D + kThreads - 1) / kThreads;
  constexpr int KPRE = 8;
  const float* po = lay.sk_o + pbase * G * D;
  float pre[EPT][KPRE];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid + kThreads * j;
#pragma unroll
    for (int k = 0; k < KPRE; ++k) pre[j][k] = (e < G * D && k < ns) ? po[(size_t)k * G * D + e] : 0.0f;
  }
  if (tid < G * ns) {
    const int k = tid / G, g = tid - k * G;
    const SplitML ml = lay.sk_ml[(pbase + k) * G + g];
    sh_m[g][k] = ml.m;
    sh_l[g][k] = ml.l;
  }
  __syncthreads();
  // per head: M = max m_k, L = sum l_k e^(m_k - M); weights e^(m_k - M) / L
  if (tid < G) {
    float M = -INFINITY;
    for (int k = 0; k < ns; ++k) M = fmaxf(M, sh_m[tid][k]);
    float L = 0.0f;
    for (int k = 0; k < ns; ++k) L += sh_m[tid][k] == -INFINITY ? 0.0f : sh_l[tid][k] * __expf(sh_m[tid][k] - M);
    const float il = 1.0f / L;
    for (int k = 0; k < ns; ++k) sh_f[tid][k] = sh_m[tid][k] == -INFINITY ? 0.0f : __expf(sh_m[tid][k] - M) * il;
    sh_lse[tid] = M + logf(L);
  }
  __syncthreads();
  // out = sum_k O_k * e^(m_k - M) / L; splits past the first KPRE eight loads at a time
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid + kThreads * j;
    if (e < G * D) {
      const int g = e / D;
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < KPRE; ++k) acc += k < ns ? pre[j][k] * sh_f[g][k] : 0.0f;
      for (int k0 = KPRE; k0 < ns; k0 += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = k0 + u < ns ? po[(size_t)(k0 + u) * G * D + e] : 0.0f;
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += k0 + u < ns ? v[u] * sh_f[g][k0 + u] : 0.0f;
      }
      a.out[(size_t)sl * G * D + e] = f2h(acc);
    }
  }
  if (tid < G) {
    lay.sk_lse[(size_t)seg * G + tid] = sh_lse[tid];
    if (par.record) lay.rec_lse[(size_t)seg * G + tid] = sh_lse[tid];
  }
}

template <int D, int G>
static int launch_split_dg(const Layout& lay, const Params& par, const StepArgs& a, int lds_bytes, hipStream_t s) {
  hipLaunchKernelGGL((attend_split_kernel<D, G>), dim3(lay.B * lay.Hkv * a.ns), dim3(kThreads), lds_bytes, s, lay,
                     par, a);
  if (hipGetLastError() != hipSuccess) return -3;
  hipLaunchKernelGGL((attend_combine_kernel<D, G>), dim3(lay.B * lay.Hkv), dim3(kThreads), 0, s, lay, par, a);
  return ok_or_err();
}

template <int D>
static int launch_split_d(const Layout& lay, const Params& par, const StepArgs& a, int lds_bytes, hipStream_t s) {
  switch (lay.G) {
    case 1: return launch_split_dg<D, 1>(lay, par, a, lds_bytes, s);
    case 2: return launch_split_dg<D, 2>(lay, par, a, lds_bytes, s);
    case 4: return launch_split_dg<D, 4>(lay, par, a, lds_bytes, s);
    case 5: return launch_split_dg<D, 5>(lay, par, a, lds_bytes, s);
    case 8: return launch_split_dg<D, 8>(lay, par, a, lds_bytes, s);
    default: return -1;
  }
}

int launch_attend_split(const Layout& lay, const Params& par, const StepArgs& a, int lds_bytes, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (a.ns < 2 || a.ns > lay.ns_max) return -1;
  if (lay.D == 64) return launch_split_d<64>(lay, par, a, lds_bytes, s);
  if (lay.D == 128) return launch_split_d<128>(lay, par, a, lds_bytes, s);
  return -1;
}

}  // namespace confkv
