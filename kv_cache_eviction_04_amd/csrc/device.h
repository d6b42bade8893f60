// Device helpers shared by the HIP kernels (internal, not part of the C ABI):
// fp16 and INT8 MFMA operands, V-tile addressing, wave and block reductions,
// the INT8 row quantizer, ranking keys, SplitMix64, and the tile loops and
// loads of the attention passes with their tuning constants.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "layout.h"

namespace confkv {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ half8 as_h8(uint4 u) { return __builtin_bit_cast(half8, u); }
__device__ __forceinline__ float half_lo(uint32_t u) { return (float)__builtin_bit_cast(h2, u)[0]; }
__device__ __forceinline__ float half_hi(uint32_t u) { return (float)__builtin_bit_cast(h2, u)[1]; }
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
__device__ __forceinline__ float h2f(uint16_t u) { return (float)__builtin_bit_cast(_Float16, u); }

__device__ __forceinline__ floatx4 mfma16(half8 a, half8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- V tiles
// Element offset of (row, col) in a segment's transposed V storage (see
// layout.h): rows in tiles of 32, each tile 32*D elements.
__device__ __forceinline__ size_t vt8(int row, int col, int D) {
  const int r = row & 31, q = r >> 3, e = r & 7, cb = col >> 4, j = col & 15;
  return (size_t)(row >> 5) * 32 * D + 1024 * (cb >> 1) + 16 * (16 * q + j) + 8 * (cb & 1) + e;
}
__device__ __forceinline__ size_t vt16(int row, int col, int D) {
  const int r = row & 31, q = r >> 3, e = r & 7, cb = col >> 4, j = col & 15;
  return (size_t)(row >> 5) * 32 * D + 512 * cb + 8 * (16 * q + j) + e;
}

// ---------------------------------------------------------------- lane groups
// Row-wise work (quantization, moves) spreads a row of d elements over
// LPR = d/16 consecutive lanes, 16 elements each. Group reductions use DPP:
// quad_perm swaps (xor 1, xor 2) and, for 8-lane groups, the half-row mirror
// (lane i <-> 7-i), which pairs the two quads.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
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
// 16 codes -> codes 0..7 and 8..15 as fp16 MFMA operands.
__device__ __forceinline__ void i8x16_to_h8(uint4 w, half8& a, half8& b) {
  h2 t0, t1, t2, t3, t4, t5, t6, t7;
  i8x4_to_h2(w.x, t0, t1);
  i8x4_to_h2(w.y, t2, t3);
  i8x4_to_h2(w.z, t4, t5);
  i8x4_to_h2(w.w, t6, t7);
  a = half8{t0[0], t0[1], t1[0], t1[1], t2[0], t2[1], t3[0], t3[1]};
  b = half8{t4[0], t4[1], t5[0], t5[1], t6[0], t6[1], t7[0], t7[1]};
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

// Random ranks for the random-victim ranker: SplitMix64 (Steele, Lea and
// Flood, OOPSLA 2014). out(k, n) is the n-th output of the generator started
// from state k: the state advances by the golden-ratio increment and the
// output function applies two xor-shift-multiply rounds and an xor-shift.
__device__ __forceinline__ uint64_t splitmix64_out(uint64_t k, uint64_t n) {
  uint64_t z = k + n * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// ------------------------------------------------------------ block helpers
// 256 threads = 4 wavefronts of 64.
//
// Wave reductions run inside each row of 16 lanes by DPP moves (quad
// permutes for lane distances 1 and 2, then the half-row and row mirrors),
// with no LDS round trip, and then combine the four rows' results read from
// lanes 0, 16, 32 and 48. After the quad steps every lane of a quad holds the
// same value, so pairing by mirror gives the same operands as pairing by XOR.
// They must be called with every lane of the wave active; the result is the
// same in every lane.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, dpp_u32<CTRL>(__builtin_bit_cast(uint32_t, v)));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
template <class Op>
__device__ __forceinline__ float row16_reduce(float v, Op op) {
  v = op(v, dpp_f32<kDppXor1>(v));
  v = op(v, dpp_f32<kDppXor2>(v));
  v = op(v, dpp_f32<kDppHalfMirror>(v));
  return op(v, dpp_f32<kDppMirror>(v));
}
__device__ __forceinline__ float lane_f32(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_reduce(v, [](float x, float y) { return x + y; });
  return (lane_f32(v, 0) + lane_f32(v, 16)) + (lane_f32(v, 32) + lane_f32(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row16_reduce(v, [](float x, float y) { return fmaxf(x, y); });
  return fmaxf(fmaxf(lane_f32(v, 0), lane_f32(v, 16)), fmaxf(lane_f32(v, 32), lane_f32(v, 48)));
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += dpp_u32<kDppXor1>(v);
  v += dpp_u32<kDppXor2>(v);
  v += dpp_u32<kDppHalfMirror>(v);
  v += dpp_u32<kDppMirror>(v);
  return (uint32_t)(__builtin_amdgcn_readlane((int)v, 0) + __builtin_amdgcn_readlane((int)v, 16) +
                    __builtin_amdgcn_readlane((int)v, 32) + __builtin_amdgcn_readlane((int)v, 48));
}
// The wave's smallest 64-bit key and the index held with it (the index of
// the lane holding the minimum when keys are unique).
template <int CTRL>
__device__ __forceinline__ void argmin_step(uint64_t& k, int32_t& i) {
  const uint32_t lo = dpp_u32<CTRL>((uint32_t)k), hi = dpp_u32<CTRL>((uint32_t)(k >> 32));
  const int32_t j = (int32_t)dpp_u32<CTRL>((uint32_t)i);
  const uint64_t w = ((uint64_t)hi << 32) | lo;
  if (w < k) {
    k = w;
    i = j;
  }
}
__device__ __forceinline__ void wave_argmin_u64(uint64_t& k, int32_t& i) {
  argmin_step<kDppXor1>(k, i);
  argmin_step<kDppXor2>(k, i);
  argmin_step<kDppHalfMirror>(k, i);
  argmin_step<kDppMirror>(k, i);
  uint64_t best = ~0ull;
  int32_t bi = -1;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint64_t w = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(k >> 32), 16 * r) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)k, 16 * r);
    const int32_t j = __builtin_amdgcn_readlane(i, 16 * r);
    if (r == 0 || w < best) {
      best = w;
      bi = j;
    }
  }
  k = best;
  i = bi;
}
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
  int32_t unused = 0;
  wave_argmin_u64(v, unused);
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
template <int NW = 4>
__device__ __forceinline__ uint32_t block_excl_scan_u32(uint32_t v, uint32_t* red, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = v;
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) red[wave] = inc;
  __syncthreads();
  uint32_t off = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    off += w < wave ? red[w] : 0u;
    all += red[w];
  }
  *total = all;
  __syncthreads();
  return off + inc - v;
}

// ----------------------------------------------------------------- INT8 row
// Absmax quantization of the 16 elements a lane holds; the group of LPR lanes
// holds one row. scale = fl32(amax / 127) and code = rne(fl32(x / scale)),
// clamped to [-127, 127]; amax == 0 gives scale 0 and zero codes. Both
// quotients are formed in binary64 and rounded once to binary32, which is the
// correctly rounded binary32 quotient (53 >= 2*24 + 2), independent of the
// compiler's float-division mode. Returns the group's scale; codes[e] holds
// the code of element e.
template <int LPR>
__device__ __forceinline__ float quantize16(const float (&x)[16], int8_t (&codes)[16]) {
  float am = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) am = fmaxf(am, fabsf(x[e]));
  am = group_max<LPR>(am);
  float scale = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) codes[e] = 0;
  if (am > 0.0f) {
    scale = (float)((double)am / 127.0);
    const double sd = (double)scale;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float r = rintf((float)((double)x[e] / sd));
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      codes[e] = (int8_t)(int)r;
    }
  }
  return scale;
}
__device__ __forceinline__ void load16h(const uint16_t* src, float (&x)[16]) {
  const uint4 a = reinterpret_cast<const uint4*>(src)[0];
  const uint4 b = reinterpret_cast<const uint4*>(src)[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[2 * j] = half_lo(w[j]);
    x[2 * j + 1] = half_hi(w[j]);
  }
}
__device__ __forceinline__ uint4 pack16(const int8_t (&c)[16]) {
  uint32_t p[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 16; ++e) p[e >> 2] |= ((uint32_t)(uint8_t)c[e]) << (8 * (e & 3));
  return make_uint4(p[0], p[1], p[2], p[3]);
}

// ========================================== tile loops and loads of the attention passes
typedef unsigned int u4v __attribute__((ext_vector_type(4)));
typedef unsigned int u2v __attribute__((ext_vector_type(2)));
// Tuning constants of the fused kernel (defaults measured on MI355X).
#ifndef CONFKV_NT
#define CONFKV_NT 0        // K/V tile loads marked non-temporal
#endif
#ifndef CONFKV_PIPE
#define CONFKV_PIPE 0      // 0: load a batch, then compute it; 1: two-stage pipeline
#endif
#ifndef CONFKV_QK8_NPB
#define CONFKV_QK8_NPB 4   // INT8 K tiles per batch
#endif
#ifndef CONFKV_QK16_NPB
#define CONFKV_QK16_NPB 2  // FP16 K tiles per batch
#endif
#ifndef CONFKV_PV8_NPB
#define CONFKV_PV8_NPB 8   // INT8 V tiles per batch
#endif
#ifndef CONFKV_PV16_NPB
#define CONFKV_PV16_NPB 4  // FP16 V tiles per batch
#endif
#ifndef CONFKV_KB
#define CONFKV_KB 10       // key-phase rows per thread loaded ahead, groups of up to 4
#endif                     // query heads (2560 staged rows in one round)
#ifndef CONFKV_KB_WIDE
#define CONFKV_KB_WIDE 6   // the same for larger groups, which have fewer registers left
#endif
#ifndef CONFKV_KB_HBM
#define CONFKV_KB_HBM 6    // the same for HBM-staged segments, whose batches also hold the
#endif                     // rows' scores and their results until the next batch is loaded
#ifndef CONFKV_OCC
#define CONFKV_OCC 4       // waves per SIMD the fused kernel is compiled for (G <= 5; a few
                           // spills at G = 5 cost less than a fourth of the occupancy)
#endif
// Streaming loads of K/V tiles: read once per step, so marked non-temporal.
__device__ __forceinline__ uint4 ldnt4(const void* p) {
#if CONFKV_NT
  const u4v v = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
#else
  return *reinterpret_cast<const uint4*>(p);
#endif
}
__device__ __forceinline__ uint2 ldnt2(const void* p) {
#if CONFKV_NT
  const u2v v = __builtin_nontemporal_load(reinterpret_cast<const u2v*>(p));
  return make_uint2(v[0], v[1]);
#else
  return *reinterpret_cast<const uint2*>(p);
#endif
}

// Tile loop over [t0, t1) (uniform across the wavefront). Batched: issue the
// loads of NPB tiles, then compute them. Two-stage: while one batch is
// computed, the loads of the next are in flight (twice the registers).
template <int NPB, class Buf, class LoadF, class CompF>
__device__ __forceinline__ void pipelined(int t0, int t1, LoadF&& load, CompF&& comp) {
  if (t0 >= t1) return;
#if !CONFKV_PIPE
  for (int base = t0; base < t1; base += NPB) {
    Buf A[NPB];
    // Every slot of the batch is loaded, those past the range with the range's
    // last tile (same lines, in flight already: no extra HBM traffic). With no
    // branch between the loads, each tile's compute waits for that tile's
    // loads only, not for the whole batch.
#pragma unroll
    for (int u = 0; u < NPB; ++u) {
      load(min(base + u, t1 - 1), A[u]);
      __builtin_amdgcn_sched_barrier(0);  // keep the loads in tile order
    }
#pragma unroll
    for (int u = 0; u < NPB; ++u)
      if (base + u < t1) comp(base + u, A[u]);
  }
  return;
#endif
  Buf A[NPB], B[NPB];
#pragma unroll
  for (int u = 0; u < NPB; ++u)
    if (t0 + u < t1) load(t0 + u, A[u]);
  for (int base = t0; base < t1; base += 2 * NPB) {
#pragma unroll
    for (int u = 0; u < NPB; ++u)
      if (base + NPB + u < t1) load(base + NPB + u, B[u]);
#pragma unroll
    for (int u = 0; u < NPB; ++u)
      if (base + u < t1) comp(base + u, A[u]);
#pragma unroll
    for (int u = 0; u < NPB; ++u)
      if (base + 2 * NPB + u < t1) load(base + 2 * NPB + u, A[u]);
#pragma unroll
    for (int u = 0; u < NPB; ++u)
      if (base + NPB + u < t1) comp(base + NPB + u, B[u]);
  }
}
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
struct QK8Buf {
  uint4 k0, k1;
  float sk, sv;
};
template <int KS>
struct QK16Buf {
  uint4 kc[KS];
  int32_t pr;
};
struct PV8Buf {
  uint4 v;
};
template <int CBW>
struct PV16Buf {
  uint4 v[CBW];
};

static inline int ok_or_err() { return hipGetLastError() == hipSuccess ? 0 : -3; }

}  // namespace confkv
