// HIP kernels for gfx950 (MI355X): the next-token draw of the decoding loop
// (greedy or inverse-CDF) over the same logits the confidence reads.
//
// Source: "Conf-KV" post (rcap.io), decoding-loop pseudocode.
#include "device.h"

namespace confkv {

// ================================================================= sampling
// [Conf-KV post, pseudocode] the step ends with x_t = sample(p), p the softmax
// of the same logits. Greedy: the largest logit, lowest index among equal
// maxima. Random: the smallest j with p_0 + ... + p_j > u for the caller's
// uniform u of the row, the sums formed in binary64 from e_j = exp(z_j - M).
// Pass 1 (one workgroup per 4096-logit chunk and row): the chunk's maximum,
// its lowest index, and sum e^(z - m_c). Pass 2 (one workgroup per row): the
// row's maximum and token for greedy; for a draw, the chunk where the scaled
// running sum crosses u * total, then an ordered scan inside that chunk.
__global__ void __launch_bounds__(256) sample_reduce_kernel(Layout lay, const float* logits, int32_t want_sum) {
  __shared__ uint64_t s_k[4];
  __shared__ double s_S[4];
  const int b = blockIdx.y, ci = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int V = lay.V;
  const float* z = logits + (size_t)b * V;
  const int begin = ci * kChunk, end = min(V, begin + kChunk);
  float x[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) x[j] = z[min(begin + tid + 256 * j, end - 1)];
  // key: (~orderable(z) << 32) | index — the smallest key is the largest
  // logit at its lowest index; a non-finite logit forces the key 0
  uint64_t key = ~0ull;
  bool bad = false;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int i = begin + tid + 256 * j;
    if (i < end) {
      bad |= !isfinite(x[j]);
      const uint64_t k = ((uint64_t)(~orderable(x[j])) << 32) | (uint32_t)i;
      key = k < key ? k : key;
    }
  }
  if (bad) key = 0;
  key = block_min_u64(key, s_k);
  SamplePartial out;
  out.idx = key == 0 ? -1 : (int32_t)(uint32_t)key;
  out.m = key == 0 ? NAN : z[out.idx];
  out.S = 0.0;
  if (want_sum && key != 0) {
    const double m = (double)out.m;
    double S = 0.0;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (begin + tid + 256 * j < end) S += exp((double)x[j] - m);
    for (int o = 32; o > 0; o >>= 1) S += __shfl_xor(S, o, 64);
    if (lane == 0) s_S[wave] = S;
    __syncthreads();
    out.S = (s_S[0] + s_S[1]) + (s_S[2] + s_S[3]);
  }
  if (tid == 0) {
    lay.spart[(size_t)b * lay.chunks + ci] = out;
    if (key == 0) atomicOr(lay.err, kErrNonFinite);
  }
}

// Exclusive prefix sum of doubles over the block in thread order.
__device__ __forceinline__ double block_excl_scan_f64(double v, double* red, double* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double inc = v;
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) red[wave] = inc;
  __syncthreads();
  double off = 0.0;
  for (int w = 0; w < wave; ++w) off += red[w];
  *total = ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();
  return off + inc - v;
}

__global__ void __launch_bounds__(256) sample_pick_kernel(Layout lay, const float* logits, const float* u,
                                                          int32_t* token) {
  __shared__ float s_m[4];
  __shared__ int32_t s_i[4];
  __shared__ double s_red[4];
  __shared__ int32_t s_chunk, s_pick;
  __shared__ double s_base, s_target;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int C = lay.chunks;
  const SamplePartial* sp = lay.spart + (size_t)b * C;
  // row maximum and its lowest index; any flagged chunk makes the row invalid
  float m = -INFINITY;
  int32_t idx = INT32_MAX;
  bool bad = false;
  for (int c = tid; c < C; c += 256) {
    const SamplePartial p = sp[c];
    if (p.idx < 0) {
      bad = true;
    } else if (p.m > m || (p.m == m && p.idx < idx)) {
      m = p.m;
      idx = p.idx;
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(m, o, 64);
    const int32_t oi = __shfl_xor(idx, o, 64);
    if (om > m || (om == m && oi < idx)) {
      m = om;
      idx = oi;
    }
  }
  bad = __any(bad);
  if (lane == 0) {
    s_m[wave] = m;
    s_i[wave] = bad ? -1 : idx;
  }
  __syncthreads();
  float M = s_m[0];
  int32_t I = s_i[0];
  bool row_bad = s_i[0] < 0;
  for (int w = 1; w < 4; ++w) {
    row_bad |= s_i[w] < 0;
    if (s_m[w] > M || (s_m[w] == M && s_i[w] < I)) {
      M = s_m[w];
      I = s_i[w];
    }
  }
  if (row_bad) {
    if (tid == 0) token[b] = -1;
    return;
  }
  if (!u) {
    if (tid == 0) token[b] = I;
    return;
  }
  // the chunk where the running sum of e_j (in units of exp(-M)) passes u * total
  if (tid == 0) {
    const double Md = (double)M;
    double total = 0.0;
    for (int c = 0; c < C; ++c) total += sp[c].S * exp((double)sp[c].m - Md);
    const double target = (double)u[b] * total;
    double acc = 0.0;
    int k = -1, last = 0;
    for (int c = 0; c < C; ++c) {
      const double wc = sp[c].S * exp((double)sp[c].m - Md);
      if (wc > 0.0) last = c;
      if (k < 0 && acc + wc > target && wc > 0.0) {
        k = c;
        break;
      }
      acc += wc;
    }
    if (k < 0) {  // u * total not reached through rounding: the last chunk with mass
      k = last;
      double a2 = 0.0;
      for (int c = 0; c < k; ++c) a2 += sp[c].S * exp((double)sp[c].m - Md);
      acc = a2;
    }
    s_chunk = k;
    s_base = acc;
    s_target = target;
    s_pick = INT32_MAX;
  }
  __syncthreads();
  const int k = s_chunk;
  const double base = s_base, target = s_target, Md = (double)M;
  const int V = lay.V;
  const float* z = logits + (size_t)b * V;
  const int begin = k * kChunk, end = min(V, begin + kChunk);
  // thread tid scans 16 consecutive logits of the chunk, in index order
  double e[16], loc = 0.0;
  int lastpos = -1;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int i = begin + 16 * tid + j;
    e[j] = i < end ? exp((double)z[i] - Md) : 0.0;
    loc += e[j];
    if (e[j] > 0.0) lastpos = i;
  }
  double chunk_total;
  const double pre = base + block_excl_scan_f64(loc, s_red, &chunk_total);
  if (pre <= target && pre + loc > target) {
    // the crossing is in this thread's range; should the one-term-at-a-time
    // sum stop short of it by rounding, the range's last token with mass
    int pick = lastpos;
    double run = pre;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      run += e[j];
      if (run > target && e[j] > 0.0) {
        pick = begin + 16 * tid + j;
        break;
      }
    }
    atomicMin(&s_pick, pick);
  }
  __syncthreads();
  if (s_pick == INT32_MAX) {  // the chunk's own sum stops short of the target: its last token with mass
    int lp = lastpos;
    for (int o = 32; o > 0; o >>= 1) lp = max(lp, __shfl_xor(lp, o, 64));
    if (lane == 0) s_i[wave] = lp;
    __syncthreads();
    if (tid == 0) token[b] = max(max(s_i[0], s_i[1]), max(s_i[2], s_i[3]));
    return;
  }
  if (tid == 0) token[b] = s_pick;
}

int launch_sample(const Layout& lay, const float* logits, const float* u, int32_t* token, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(sample_reduce_kernel, dim3(lay.chunks, lay.B), dim3(256), 0, s, lay, logits,
                     (int32_t)(u != nullptr));
  if (hipGetLastError() != hipSuccess) return -3;
  hipLaunchKernelGGL(sample_pick_kernel, dim3(lay.B), dim3(256), 0, s, lay, logits, u, token);
  return ok_or_err();
}

}  // namespace confkv
