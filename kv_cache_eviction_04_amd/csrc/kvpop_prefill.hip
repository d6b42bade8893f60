// HIP kernels for gfx950 (MI355X): KVpop's prefill over S tokens with known
// priorities under the multi-query sink + window + top-k mask, and the
// scorer's future-attention training target.
//
// Source: "Resumen Técnico: KVpop" (gist.science) §2.1, §2.2, §2.4.
#include <float.h>

#include "device.h"

namespace confkv {

constexpr int kRankBlock = 8192;  // keys per LDS block of the rank sort (64 KB)
constexpr int kMaxChunks = 1024;  // 32-key chunks of one query tile's key list, at most
constexpr int kThrChunk = 256;    // queries per workgroup of the threshold pass (a multiple of 256)
constexpr int kThrThreads = 256;

// ==================================================== KVpop prefill mask
// [KVpop summary §2.4] The k long-range slots follow a running threshold over
// static priorities, so the sparse mask of a prefill over S known priorities
// is generated inside the attention kernel, never stored as S x S. Query q
// may see key j iff
//   j <= q and (j < s or j >= q - w or rank(j) <= thr(q)),
// where rank orders positions >= s by (priority descending, position
// ascending) and thr(q) is the k-th smallest rank among [s, q-1-w]: the rows
// a decode step at q attends to. Per segment (batch row, KV head): a sort
// gives the ranks, one pass over q moves the threshold, and the attention
// kernel evaluates the predicate per (query, key).

// Ranks: keys (orderable priority << 32 | ~position) sorted descending by a
// bitonic network over the segment's N (a power of two) keys in the
// workspace, then rank[position] = sorted index (-1 for sinks). A pass
// (k, jj) compares i with i ^ jj, so every pass with jj below the block size
// B (up to 8192 keys, 64 KB) pairs keys of one block: those run in LDS, and
// only the passes with jj >= B go through global memory. Direction:
// descending where i & k is 0. Two launches: the first sorts every block
// (k = 2 .. B) with one workgroup per (block, segment); the second, one
// workgroup per segment, runs each larger k (its global passes, then its
// passes below B block by block in LDS) and scatters the ranks.
__device__ __forceinline__ void rank_cmpx(uint64_t* X, int i, int ixj, int gi, int k) {
  const uint64_t a = X[i], b = X[ixj];
  const bool desc = (gi & k) == 0;
  if (desc ? (a < b) : (a > b)) {
    X[i] = b;
    X[ixj] = a;
  }
}
// Passes (k, jj) for k = k_lo .. k_hi (powers of two) and jj from
// min(k, 8192)/2 down to 1 (larger strides pair keys of different blocks and
// are done before, in global memory) over an 8192-key block in LDS (in LDS
// on entry and on return), 1024 threads: thread t keeps keys 8t .. 8t+7 in registers for
// the passes with jj < 512, whose partners are in the same wave: jj < 8 in
// the thread, 8 <= jj < 512 in lane t ^ (jj/8), exchanged by shuffles. Only
// the passes with jj >= 512 pair keys of different waves and go through
// LDS, with a barrier each. gbase: the block's first index in the segment.
__device__ void rank_block_regs(uint64_t* sblk, int gbase, int k_lo, int k_hi) {
  const int t = threadIdx.x;
  uint64_t x[8];
  bool in_regs = false;
  for (int k = k_lo; k <= k_hi; k <<= 1) {
    int jj = min(k, kRankBlock) >> 1;  // larger strides pair keys of different blocks: done before
    for (; jj >= 512; jj >>= 1) {
      if (in_regs) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sblk[8 * t + e] = x[e];
        __syncthreads();
        in_regs = false;
      }
      for (int i = t; i < kRankBlock; i += 1024) {
        const int ixj = i ^ jj;
        if (ixj > i) rank_cmpx(sblk, i, ixj, gbase + i, k);
      }
      __syncthreads();
    }
    if (!in_regs) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = sblk[8 * t + e];
      in_regs = true;
    }
    for (; jj >= 8; jj >>= 1) {
      const int d = jj >> 3;
      const bool lower = (t & d) == 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint64_t y = __shfl_xor(x[e], d, 64);
        const bool desc = ((gbase + 8 * t + e) & k) == 0;
        x[e] = (lower == desc) ? (x[e] > y ? x[e] : y) : (x[e] < y ? x[e] : y);
      }
    }
    for (; jj >= 1; jj >>= 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if ((e & jj) == 0) {
          const int f = e | jj;
          const bool desc = ((gbase + 8 * t + e) & k) == 0;
          const uint64_t a = x[e], b = x[f];
          if (desc ? (a < b) : (a > b)) {
            x[e] = b;
            x[f] = a;
          }
        }
      }
    }
  }
  if (in_regs) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sblk[8 * t + e] = x[e];
    __syncthreads();
  }
}
// passes (k, jj) for jj from min(k, B)/2 down to 1 on block b in LDS, for k
// from 2 to B (k0 = 0: the block's own sort, loading the keys from the
// priorities) or for k = k0 alone (the keys from the workspace)
__device__ void rank_block_passes(const KvpopPrefillArgs& pa, uint64_t* sblk, int seg, int b, int k0) {
  const int tid = threadIdx.x;
  const int S = pa.S, s = pa.sinks, N = pa.N, B = min(N, kRankBlock);
  const float* pr = pa.prio + (size_t)seg * S;
  uint64_t* A = pa.sort + (size_t)seg * N;
  const int base = b * B;
  for (int i = tid; i < B; i += 1024) {
    const int j = s + base + i;
    if (k0 == 0) {
      sblk[i] = j < S ? rank_key(pr[j], j) : 0ull;  // padding sorts last
      if (j < S && !isfinite(pr[j])) atomicOr(pa.err, kErrNonFinite);
    } else {
      sblk[i] = A[base + i];
    }
  }
  __syncthreads();
  if (B == kRankBlock) {
    rank_block_regs(sblk, base, k0 ? k0 : 2, k0 ? k0 : B);
  } else {
    for (int k = k0 ? k0 : 2; k <= (k0 ? k0 : B); k <<= 1) {
      for (int jj = min(k, B) >> 1; jj > 0; jj >>= 1) {
        for (int i = tid; i < B; i += 1024) {
          const int ixj = i ^ jj;
          if (ixj > i) rank_cmpx(sblk, i, ixj, base + i, k);
        }
        __syncthreads();
      }
    }
  }
  for (int i = tid; i < B; i += 1024) A[base + i] = sblk[i];
  __syncthreads();
}
__global__ void __launch_bounds__(1024) kvpop_rank_blocks_kernel(KvpopPrefillArgs pa) {
  extern __shared__ uint64_t sblk[];  // [B]
  rank_block_passes(pa, sblk, blockIdx.y, blockIdx.x, 0);
}
__global__ void __launch_bounds__(1024) kvpop_rank_kernel(KvpopPrefillArgs pa) {
  extern __shared__ uint64_t sblk[];  // [B]
  const int tid = threadIdx.x, seg = blockIdx.x;
  const int S = pa.S, s = pa.sinks, N = pa.N, B = min(N, kRankBlock);
  uint64_t* A = pa.sort + (size_t)seg * N;
  int32_t* rank = pa.rank + (size_t)seg * S;
  for (int j = tid; j < min(s, S); j += 1024) rank[j] = -1;
  for (int k = 2 * B; k <= N; k <<= 1) {
    for (int jj = k >> 1; jj >= B; jj >>= 1) {
      for (int i = tid; i < N; i += 1024) {
        const int ixj = i ^ jj;
        if (ixj > i) rank_cmpx(A, i, ixj, i, k);
      }
      __syncthreads();
    }
    for (int b = 0; b < N / B; ++b) rank_block_passes(pa, sblk, seg, b, k);
  }
  for (int i = tid; i < S - s; i += 1024) rank[0xFFFFFFFFu - (uint32_t)A[i]] = i;
}

// Thresholds: one pass over q. Position q-1-w joins the candidates at query
// q; a bitmap over ranks holds the candidates. With n candidates, thr = S
// (all pass) while n < k, the largest rank at n = k, and after that an
// inserted rank below thr moves thr to the next candidate rank below it
// (the old k-th is pushed out). k = 0 gives thr = -1 (none pass). Once
// n >= k a rank above thr is never the threshold again (thr only moves
// down, and the search for the next rank runs below it), so it is not
// entered in the bitmap.
// The state before any query a follows from its definition, not only from
// the walk: the candidates are then the M = a - 1 - w - s positions
// [s, a-2-w] (position a-1-w joins at query a), thr is their k-th smallest
// rank (S while M < k), and a bitmap holding all their ranks serves as well
// as the walk's (the ranks above thr that it also holds are never visited).
// So each workgroup takes one chunk of 256 queries of a segment: its 256
// threads enter the ranks that precede the chunk's first query into the
// bitmap and find thr there by a scan over the words' popcounts, and then
// one wave walks the chunk.
// The wave walks the chunk's queries in batches of 64: lane i loads the
// rank that joins at query q0 + i (four batches at a time, loaded a group
// ahead), and lane i keeps the threshold of query q0 + i until the batch is
// stored. A batch that leaves n below k only enters its ranks; the batch in
// which n reaches k is stepped through query by query (readlane). After
// that only the ranks below the batch's starting thr can move it, so a
// ballot picks them and they are taken in query order. The bitmap word that
// holds thr is also kept in a register, so a move of thr within that word
// needs no LDS access; inserts are LDS atomic ORs whose result is not
// waited for.
__device__ __forceinline__ int wave_max_i32(int v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}
__global__ void __launch_bounds__(kThrThreads) kvpop_threshold_kernel(KvpopPrefillArgs pa) {
  extern __shared__ uint32_t kbits[];  // ceil(N/32) words
  __shared__ uint32_t red[kThrThreads / 64];
  __shared__ int sh_t, sh_max;
  const int tid = threadIdx.x, lane = tid & 63, seg = blockIdx.y;
  const int S = pa.S, s = pa.sinks, w = pa.window, k = pa.topk, nw = (pa.N + 31) >> 5;
  const int a = blockIdx.x * kThrChunk, b_end = min(a + kThrChunk, S);  // this chunk's queries
  const int32_t* rank = pa.rank + (size_t)seg * S;
  int32_t* thr = pa.thr + (size_t)seg * S;
  for (int i = tid; i < nw; i += kThrThreads) kbits[i] = 0u;
  if (tid == 0) sh_max = -1;
  __syncthreads();
  // ---- the state before query a: the ranks of positions [s, s + M)
  const int M = max(0, a - 1 - w - s);
  int mx = -1;
  for (int i = tid; i < M; i += kThrThreads) {
    const int r = rank[s + i];
    atomicOr(&kbits[r >> 5], 1u << (r & 31));
    mx = max(mx, r);
  }
  mx = wave_max_i32(mx);
  if (lane == 0) atomicMax(&sh_max, mx);
  __syncthreads();
  if (k > 0 && M >= k) {
    // thr(a): the k-th smallest entered rank. Each thread counts a run of
    // words; the one whose run holds the k-th set bit finds it.
    const int wpt = (nw + kThrThreads - 1) / kThrThreads;
    const int w0 = min(nw, tid * wpt), w1 = min(nw, w0 + wpt);
    uint32_t cnt = 0;
    for (int i = w0; i < w1; ++i) cnt += __popc(kbits[i]);
    uint32_t total;
    const uint32_t excl = block_excl_scan_u32<kThrThreads / 64>(cnt, red, &total);
    if (excl < (uint32_t)k && (uint32_t)k <= excl + cnt) {
      uint32_t acc = excl;
      for (int i = w0; i < w1; ++i) {
        uint32_t word = kbits[i];
        const uint32_t pc = __popc(word);
        if (acc + pc >= (uint32_t)k) {
          for (uint32_t j = acc + 1; j < (uint32_t)k; ++j) word &= word - 1;  // drop the lower set bits
          sh_t = (i << 5) + __builtin_ctz(word);
          break;
        }
        acc += pc;
      }
    }
    __syncthreads();
  }
  if (tid >= 64) return;  // one wave walks the chunk
  int n = M, t = k > 0 ? (M >= k ? sh_t : S) : -1, maxr = sh_max;
  int wt = 0;        // the bitmap word holding thr once n >= k,
  uint32_t ct = 0u;  // and a copy of it kept up to date
  if (k > 0 && M >= k) {
    wt = t >> 5;
    ct = kbits[wt];
  }
  // insert rank r below thr and move thr to the next candidate rank below it
  auto move = [&](int r) {
    const uint32_t bit = 1u << (r & 31);
    if (lane == 0) atomicOr(&kbits[r >> 5], bit);  // LDS operations of a wave complete in order
    if ((r >> 5) == wt) ct |= bit;
    int wi = wt;
    uint32_t word = ct & ((1u << (t & 31)) - 1u);
    if (word == 0u) {
      do word = kbits[--wi];
      while (word == 0u);
      wt = wi;
      ct = word;
    }
    t = (wi << 5) + 31 - __clz((int)word);
  };
  auto rank_at = [&](int q0) {
    const int q = q0 + lane, p = q - 1 - w;
    return (q < b_end && p >= s) ? rank[p] : -2;
  };
  constexpr int NB = 4;  // batches whose ranks are loaded together
  int rv[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) rv[j] = rank_at(a + 64 * j);
  for (int g0 = a; g0 < b_end; g0 += 64 * NB) {
    int rn[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) rn[j] = g0 + 64 * (NB + j) < b_end ? rank_at(g0 + 64 * (NB + j)) : -2;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int q0 = g0 + 64 * j, q = q0 + lane;
      if (q0 >= b_end) break;
      const int r_l = rv[j];
      int tv = t;
      const uint64_t valid = __ballot(r_l >= 0);
      const int nv = __popcll(valid);
      if (k > 0 && n >= k) {
        // thr only moves down, so only ranks below the batch's starting thr
        // can move it; the others change nothing
        n += nv;
        uint64_t cand = __ballot(r_l >= 0 && r_l < t);
        while (cand) {
          const int i = __builtin_ctzll(cand);
          cand &= cand - 1;
          const int r = __builtin_amdgcn_readlane(r_l, i);
          if (r < t) {
            move(r);
            tv = lane >= i ? t : tv;
          }
        }
      } else if (k > 0 && n + nv < k) {
        // every rank of the batch is entered and thr stays S
        if (r_l >= 0) atomicOr(&kbits[r_l >> 5], 1u << (r_l & 31));
        maxr = max(maxr, wave_max_i32(r_l));
        n += nv;
      } else {
        const int cnt = min(64, b_end - q0);
        for (int i = 0; i < cnt; ++i) {
          const int r = __builtin_amdgcn_readlane(r_l, i);
          if (r >= 0 && k > 0) {
            ++n;
            if (n <= k) {
              if (lane == 0) atomicOr(&kbits[r >> 5], 1u << (r & 31));
              maxr = max(maxr, r);
              if (n == k) {
                t = maxr;
                wt = t >> 5;
                ct = kbits[wt];
              }
            } else if (r < t) {
              move(r);
            }
          }
          tv = lane == i ? t : tv;
        }
      }
      if (q < b_end) thr[q] = tv;
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) rv[j] = rn[j];
  }
}

// Work item of a workgroup of a (tiles x segments) grid, XCD-aware. The
// dispatcher deals workgroups out round-robin over the 8 XCDs, each with its
// own L2, so XCD x = lin % 8 is given the contiguous run of work items that
// starts at x * (n / 8) + min(x, n % 8), in order; work items run tile-fastest
// within a segment. Neighbouring tiles of a segment share most of their keys
// (prefill) or their later query rows (target), and so meet in one L2. The
// map is a bijection on [0, n) whatever the dispatch order.
__device__ __forceinline__ void xcd_tile_seg(int& tile, int& seg) {
  const int n = gridDim.x * gridDim.y;
  const int lin = blockIdx.x + blockIdx.y * gridDim.x;
  const int x = lin & 7;
  const int work = x * (n >> 3) + min(x, n & 7) + (lin >> 3);
  seg = work / gridDim.x;
  tile = work - seg * gridDim.x;
}

// Max and sum over the four 16-lane rows of a wave (lanes j, j+16, j+32,
// j+48), in every lane, with gfx950's row-swap instructions: VALU work, no
// LDS round trip. v_permlane16_swap exchanges the odd rows of its first
// operand with the even rows of its second, so with both set to x they end
// up holding rows (0, 0, 2, 2) and (1, 1, 3, 3) of x; v_permlane32_swap does
// the same for the two halves. Combining the pair gives every lane the same
// value, in the same order as a shuffle-xor reduction. This compiler's
// builtins for these instructions return the first operand for both
// results, hence the asm; s_nop 1 gives the two wait states a swap needs
// after a VALU write of its operands (and the same again before a VALU
// reads its results).
__device__ __forceinline__ void row_swap(float& a, float& b, int half) {
  if (half)
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  else
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
// The maximum is taken in the same asm block as the swaps: written as
// fmaxf on the swaps' results, each operand would first be canonicalised
// (the compiler cannot see that a swap only moves values), two VALU
// instructions more per step. The operands are scores or -inf, never NaN.
__device__ __forceinline__ float rows_max(float x) {
  float a = x, b;
  asm("v_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1\n\tv_max_f32 %0, %0, %1\n\t"
      "v_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1\n\tv_max_f32 %0, %0, %1"
      : "+v"(a), "=&v"(b));
  return a;
}
// max(a, b) of two non-NaN values without the canonicalising moves
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float rows_sum(float x) {
  float a = x, b = x;
  row_swap(a, b, 0);
  a = a + b;
  b = a;
  row_swap(a, b, 1);
  return a + b;
}

constexpr float kLog2e = 1.4426950408889634f;  // log2(e)
constexpr float kLn2 = 0.6931471805599453f;    // ln(2)

// 16-byte piece swizzle of row r of the LDS V tile (rows of D halves). The PV
// operand of a lane group is read by gfx950's transposing LDS read: each lane
// of a 16-lane group names 8 bytes (4 columns) of one of 4 rows, and lane j
// receives column j of the 4 rows. A half-wave so reads 32 bytes of each of 8
// rows that differ in bits 0, 1 and 3 (D = 128: rows are 256 bytes, one bank
// line each) or in bits 1 and 3 within each parity (D = 64: 128-byte rows,
// odd rows on the upper half of the banks). XOR-ing the piece index with an
// even value taken from those bits puts the 8 rows on distinct banks.
template <int D>
__device__ __forceinline__ int vtile_swizzle(int r) {
  return D == 128 ? 2 * ((r & 3) | (((r >> 3) & 1) << 2)) : 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1));
}

// 16-byte piece swizzle of row r of the LDS K tile (rows of D halves, no
// padding). QK reads one piece of 16 rows per 16-lane group: rows
// 8(j/4) + j%4 (+4) for lane j, which differ in bits 0, 1, 3 and 4; XOR-ing
// the piece index with those bits puts the 16 reads on distinct banks (D =
// 128; at D = 64, two rows per bank line, bits 1, 3 and 4).
template <int D>
__device__ __forceinline__ int ktile_swizzle(int r) {
  return D == 128 ? ((r & 3) | (((r >> 3) & 3) << 2)) : (((r >> 1) & 1) | (((r >> 3) & 3) << 1));
}

// LDS of one chunk buffer of the prefill attention: K then V, 32 rows of D
// halves each.
template <int D>
constexpr int kChunkHalves = 2 * 32 * D;

typedef short short4v __attribute__((ext_vector_type(4)));
typedef _Float16 half4v __attribute__((ext_vector_type(4)));

// Masked prefill attention: one workgroup per 32 queries of a segment (16
// when a wave serves two query heads). The key list holds the sinks, the
// long-range keys that pass the first query's threshold (a superset for the
// later queries, whose thresholds are no larger), found from the earlier
// positions' ranks or from the rank-sorted keys, whichever reads less, and
// the contiguous run [q0 - w, q1). Per 32-key chunk the K rows and V rows
// (row-major, 16-byte pieces swizzled per row) go through LDS once for all
// the workgroup's queries, loaded straight from global memory into one of
// two buffers while the other is computed. With 8 waves (groups of up to 4
// query heads) wave w takes head w % 4 for the 16 queries of block w / 4;
// with 4 waves (larger groups) wave w takes heads w, w+4, ... for 16
// queries. Per row block: S^T = K Q^T on MFMA, the predicate per (key,
// query), online softmax per query in the base-2 domain, and O^T = V^T P^T
// with the weights rounded once to fp16 (the sums l stay fp32, so the LSE
// is not affected).
template <int D, int G, int NT>
__global__ void __launch_bounds__(NT, NT == 512 ? 4 : 3) kvpop_prefill_attend_kernel(KvpopPrefillArgs pa) {
  constexpr int KS = D / 32, NCB = D / 16;
  constexpr int NW = NT / 64;                   // waves
  constexpr bool kWavePerBlock = NW == 8;       // 8 waves: one (head, 16-query block) per wave
  static_assert(!kWavePerBlock || G <= 4, "8 waves serve groups of up to 4 heads");
  constexpr int HPW = kWavePerBlock ? 1 : (G + 3) / 4;          // query heads per wave
  constexpr int QT = kWavePerBlock ? 1 : (HPW == 1 ? 2 : 1);     // 16-query blocks per head and wave
  constexpr int QB = kWavePerBlock ? 32 : 16 * QT;               // queries per workgroup
  constexpr int NR = HPW * QT;                  // 16-row blocks per wave
  static_assert(D == 64 || D == 128, "tile swizzles");
  constexpr int PIECES = kChunkHalves<D> / 8;      // 16-byte pieces of a chunk: K then V
  constexpr int PPT = (PIECES + NT - 1) / NT;
  // two chunk buffers, distinct objects: the compiler then sees that the
  // reads of one never wait for the loads in flight into the other
  __shared__ __align__(16) uint16_t cbuf0[kChunkHalves<D>], cbuf1[kChunkHalves<D>];
  extern __shared__ __align__(16) int32_t plds[];
  int32_t* lpos = plds;
  int32_t* lrank = lpos + ((pa.list_cap + 31) & ~31);  // 16-byte aligned for vector reads
  __shared__ uint32_t red[NW];
  __shared__ uint32_t easy_bits[kMaxChunks / 32];  // chunk c: bit c % 32 of word c / 32

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane >> 4, lj = lane & 15;
  const int S = pa.S, s = pa.sinks, w = pa.window;
  if (tid < kMaxChunks / 32) easy_bits[tid] = 0u;  // cleared before the list's barrier
  int tile, seg;
  xcd_tile_seg(tile, seg);
  const int b = seg / pa.Hkv, h = seg - b * pa.Hkv;
  const int q0 = QB * tile, q1 = min(q0 + QB, S);
  const int32_t* rank = pa.rank + (size_t)seg * S;
  const int32_t* thr = pa.thr + (size_t)seg * S;
  const uint16_t* kseg = pa.k + (size_t)seg * S * D;
  const uint16_t* vseg = pa.v + (size_t)seg * S * D;

  // ---- key list: sinks, long-range keys passing thr(q0), contiguous run
  const int n_sink = min(s, q1);
  const int g_end = max(s, q0 - w);            // long-range positions [s, g_end)
  const int thr0 = thr[q0];
  // The long-range keys are the positions in [s, g_end) whose rank is at
  // most thr0. Two ways to find them, whichever reads fewer bytes: the
  // ranks of [s, g_end) (4 bytes each), or the sorted keys of ranks
  // 0 .. thr0 (8 bytes each; the rank sort leaves rank i's key at entry i),
  // keeping those below g_end. Late tiles take the second: their top-k set
  // is a small share of the positions before them.
  const int nr = max(0, min(thr0 + 1, S - s));
  const bool by_rank = 2 * nr < g_end - s && pa.N >= 2;
  uint32_t cnt = 0, ng, off;
  if (by_rank) {
    // Each thread takes a run of 8 sorted entries per round (four 16-byte
    // loads; entry 0 is 16-byte aligned as N >= 2); a round may read up to
    // 7 entries past nr, inside the segment's N entries or the workspace's
    // next part (the ranks). Count, scan, then write in rank order.
    const uint64_t* A = pa.sort + (size_t)seg * pa.N;
    const int per = (((nr + NT - 1) / NT) + 7) & ~7;
    const int ia = min(nr, tid * per), ib = min(nr, tid * per + per);
    auto load8 = [&](int i, uint64_t (&kv)[8]) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const ulonglong2 v = *reinterpret_cast<const ulonglong2*>(A + i + 2 * u);
        kv[2 * u] = v.x;
        kv[2 * u + 1] = v.y;
      }
    };
    for (int i = ia; i < ib; i += 8) {
      uint64_t kv[8];
      load8(i, kv);
#pragma unroll
      for (int e = 0; e < 8; ++e) cnt += (i + e < ib && (int)(0xFFFFFFFFu - (uint32_t)kv[e]) < g_end) ? 1u : 0u;
    }
    off = block_excl_scan_u32<NW>(cnt, red, &ng);
    for (int i = ia; i < ib; i += 8) {
      uint64_t kv[8];
      load8(i, kv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int pos = (int)(0xFFFFFFFFu - (uint32_t)kv[e]);
        if (i + e < ib && pos < g_end) {
          if (n_sink + (int)off < pa.list_cap) {
            lpos[n_sink + off] = pos;
            lrank[n_sink + off] = i + e;
          }
          ++off;
        }
      }
    }
  } else {
    // Each thread scans a run of ranks that starts 16-byte aligned in memory
    // (at most 3 before s: the previous segment's, or for the first segment
    // none before the array), 16 ranks per round as four 16-byte loads in
    // flight. A round starts below g_end <= S and may read up to 15 ranks
    // past the segment's end: the next segment's, or for the last segment
    // the start of the thresholds, which follow the ranks in the workspace.
    // Ranks before s and from g_end on are skipped. Count, scan, then write
    // in ascending position order.
    const int a0 = s - (int)(((size_t)seg * S + s) & 3);  // rank + a0 is 16-byte aligned
    const int span = g_end - a0;
    const int per = (((span + NT - 1) / NT) + 15) & ~15;
    const int ga = a0 + min(span, tid * per), gb = a0 + min(span, tid * per + per);
    auto load16 = [&](int j, int (&r)[16]) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int4 v = *reinterpret_cast<const int4*>(rank + j + 4 * u);
        r[4 * u] = v.x;
        r[4 * u + 1] = v.y;
        r[4 * u + 2] = v.z;
        r[4 * u + 3] = v.w;
      }
    };
    for (int j = ga; j < gb; j += 16) {
      int r[16];
      load16(j, r);
#pragma unroll
      for (int e = 0; e < 16; ++e) cnt += (j + e >= s && j + e < gb && r[e] <= thr0) ? 1u : 0u;
    }
    off = block_excl_scan_u32<NW>(cnt, red, &ng);
    for (int j = ga; j < gb; j += 16) {
      int r[16];
      load16(j, r);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if (j + e >= s && j + e < gb && r[e] <= thr0) {
          if (n_sink + (int)off < pa.list_cap) {
            lpos[n_sink + off] = j + e;
            lrank[n_sink + off] = r[e];
          }
          ++off;
        }
      }
    }
  }
  const int c0 = g_end;
  const int n_cont = max(0, q1 - c0);
  const int nk = n_sink + (int)ng + n_cont;
  for (int i = tid; i < n_sink; i += NT) {
    lpos[i] = i;
    lrank[i] = -1;
  }
  for (int i = tid; i < n_cont; i += NT) {
    if (n_sink + (int)ng + i < pa.list_cap) {
      lpos[n_sink + ng + i] = c0 + i;
      lrank[n_sink + ng + i] = rank[c0 + i];
    }
  }
  if (tid == 0 && nk > pa.list_cap) atomicOr(pa.err, kErrInternal);  // cannot happen: host bound
  __syncthreads();
  const int nkc = min(nk, pa.list_cap);
  const int nchunks = (nkc + 31) >> 5;

  // Thresholds do not increase with the query, so thr(q1 - 1) is the
  // tile's smallest: a key at or before q0 and below g_end (a sink, or a
  // long-range key) whose rank passes it is allowed for every query of the
  // tile, and a chunk of such keys needs no per-pair predicate. Thread i
  // checks list entry i; a wave's 64 entries are two chunks, whose flags are
  // the halves of its ballot, ORed into an LDS bitmask.
  const int thr_min = thr[q1 - 1];
  const int easy_end = min(q0 + 1, g_end);
  for (int b0 = 0; b0 < 32 * nchunks; b0 += NT) {
    const int li = b0 + tid;
    const bool ok = li < nkc && lpos[li] < easy_end && lrank[li] <= thr_min;
    const uint64_t bal = __ballot(ok);
    if (lane == 0) {
      const int c = (b0 + 64 * wave) >> 5;  // even
      const uint32_t bits = ((uint32_t)bal == 0xFFFFFFFFu ? 1u : 0u) | ((uint32_t)(bal >> 32) == 0xFFFFFFFFu ? 2u : 0u);
      if (bits) atomicOr(&easy_bits[c >> 5], bits << (c & 31));
    }
  }
  __syncthreads();
  // ---- 32-key chunks, loaded global -> LDS (gfx950): lane l of a wave
  // writes the 16 bytes at the wave's LDS base + 16 l, so piece e of the
  // buffer (K pieces, then V pieces, row by row) is loaded by the thread
  // NT u + e and holds the global piece that the row's swizzle maps there.
  // Keys past the list's end repeat its last entry (masked).
  // The list reads that give the addresses come first, the loads after: an
  // LDS read issued behind a load into LDS waits for it unless the compiler
  // can tell the two apart, which it cannot for the (dynamic) lists.
  auto issue_chunk = [&](int c, uint16_t* buf) {
    const uint16_t* src[PPT];
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int e = tid + NT * u;
      const bool isv = e >= PIECES / 2;
      const int pe = isv ? e - PIECES / 2 : e;
      const int row = pe / (D / 8), slot = pe - row * (D / 8);
      const int pos = lpos[min(32 * c + row, nkc - 1)];
      const int piece = slot ^ (isv ? vtile_swizzle<D>(row) : ktile_swizzle<D>(row));
      src[u] = (isv ? vseg : kseg) + (size_t)pos * D + 8 * piece;
    }
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int e = tid + NT * u;
      if (PIECES % NT == 0 || e < PIECES) {
        const int wbase = __builtin_amdgcn_readfirstlane(8 * (tid - lane + NT * u));  // halves, wave-uniform
        __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src[u],
                                         (__attribute__((address_space(3))) void*)(buf + wbase), 16, 0, 0);
      }
    }
  };
  // the first chunk's loads go out now, ahead of the queries' loads below
  if (nchunks > 0) issue_chunk(0, cbuf0);

  // ---- row blocks of this wave: head rb_head(rb), query block rb_qblk(rb). The
  // MFMA computes S^T = K Q^T with the chunk's K rows in a permuted order, so
  // that lane (lq, lj) receives query lj's scores against keys 8lq .. 8lq+7
  // of the chunk: the softmax of a query stays in one lane group, and its
  // eight weights are at once the lane's B operand of O^T = V^T P^T.
  // Scores and maxima are kept in base-2 units (scale * log2(e) folded in).
  const float sl2 = pa.scale * kLog2e;
  auto rb_head = [&](int rb) { return kWavePerBlock ? (wave & 3) : wave + 4 * (rb / QT); };
  auto rb_qblk = [&](int rb) { return kWavePerBlock ? (wave >> 2) : rb % QT; };
  // row block rb serves a head (always so when G is a multiple of 4)
  auto active = [&](int rb) { return G % 4 == 0 || rb_head(rb) < G; };
  half8 qb[NR][KS];
  float m[NR], l[NR];
  int thr_q[NR];
  floatx4 O[NR][NCB];
#pragma unroll
  for (int rb = 0; rb < NR; ++rb) {
    const int g = rb_head(rb), qt = rb_qblk(rb);
    const int hq = h * G + (g < G ? g : 0);
    const int qrow = q0 + 16 * qt + lj;
    const uint16_t* qp = pa.q + (((size_t)b * pa.Hq + hq) * S + min(qrow, S - 1)) * D;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const uint4 u = *reinterpret_cast<const uint4*>(qp + 8 * (lq + 4 * kk));
      qb[rb][kk] = qrow < q1 ? as_h8(u) : half8{};
    }
    m[rb] = -INFINITY;
    l[rb] = 0.0f;
    thr_q[rb] = qrow < q1 ? thr[qrow] : -1;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) O[rb][cb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  // row lj of permuted block kb holds key 8*(lj/4) + 4*kb + lj%4 of the chunk
  const int kperm0 = 8 * (lj >> 2) + (lj & 3);
  // PV operand of column block cb: keys 8lq .. 8lq+7 of column 16cb + lj, as
  // two transposing reads of rows 8lq + lj/4 and 8lq + 4 + lj/4 (same
  // swizzle), columns 16cb + 4(lj%4) .. +3
  const int vrow = 8 * lq + (lj >> 2);
  const int vsw = vtile_swizzle<D>(vrow);
  const int voff = 32 * D + vrow * D + 4 * (lj & 1);  // halves into a chunk buffer

  // one chunk: wait for this wave's loads of it, barrier (every wave's loads
  // landed; every wave is done with the other buffer), start the next
  // chunk's loads into the other buffer, compute this one
  auto step = [&](const int c, const uint16_t* buf, uint16_t* nbuf) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    const bool chunk_easy = (__builtin_amdgcn_readfirstlane(easy_bits[c >> 5]) >> (c & 31)) & 1u;
    // this lane's eight keys of the chunk (list entries 32c + 8lq .. +7), for
    // the per-pair predicate of a chunk that needs it. List reads come
    // before the loads into LDS are issued (see issue_chunk).
    int kpos[8], krank[8];
    if (!chunk_easy) {
      const int li0 = 32 * c + 8 * lq;
      const uint4 p0 = *reinterpret_cast<const uint4*>(lpos + li0);
      const uint4 p1 = *reinterpret_cast<const uint4*>(lpos + li0 + 4);
      const uint4 r0v = *reinterpret_cast<const uint4*>(lrank + li0);
      const uint4 r1v = *reinterpret_cast<const uint4*>(lrank + li0 + 4);
      const int pp[8] = {(int)p0.x, (int)p0.y, (int)p0.z, (int)p0.w, (int)p1.x, (int)p1.y, (int)p1.z, (int)p1.w};
      const int rr[8] = {(int)r0v.x, (int)r0v.y, (int)r0v.z, (int)r0v.w,
                         (int)r1v.x, (int)r1v.y, (int)r1v.z, (int)r1v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool in = li0 + e < nkc;
        kpos[e] = in ? pp[e] : INT32_MAX;  // out of the list: never <= a query
        krank[e] = rr[e];
      }
    }
    if (c + 1 < nchunks) issue_chunk(c + 1, nbuf);
#pragma unroll
    for (int rb = 0; rb < NR; ++rb) {
      if (!active(rb)) continue;
      const int qr = q0 + 16 * rb_qblk(rb) + lj;
      floatx4 acc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        acc[kb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        const int krow = kperm0 + 4 * kb;
        const uint16_t* kr = buf + krow * D;
        const int ksw = ktile_swizzle<D>(krow);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
          acc[kb] = mfma16(as_h8(*reinterpret_cast<const uint4*>(kr + 8 * ((lq + 4 * kk) ^ ksw))), qb[rb][kk], acc[kb]);
      }
      // raw scores (masked pairs -inf); the scale goes into the maximum
      // (rounding is monotone, so the scaled maximum is the maximum of the
      // scaled scores) and into one FMA per weight
      float sc[8];
      float mt = -INFINITY;
      if (chunk_easy) {
        // No mask: a query row past the tile's end has zero Q, so finite
        // scores of its own, and its output and LSE are never stored.
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sc[e] = acc[e >> 2][e & 3];
          mt = fmaxf(mt, sc[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = kpos[e];
          const bool ok = qr < q1 && j <= qr && (j < s || j >= qr - w || krank[e] <= thr_q[rb]);
          sc[e] = ok ? acc[e >> 2][e & 3] : -INFINITY;
          mt = fmaxf(mt, sc[e]);
        }
      }
      mt = rows_max(mt) * sl2;
      const float mn = max_raw(m[rb], mt);
      // all masked so far (mn = -inf): every score of the row is -inf too, and
      // a finite reference gives exp2(-inf) = 0 for the weights and alpha
      const float ms = max_raw(mn, -FLT_MAX);
      const float alpha = __builtin_amdgcn_exp2f(m[rb] - ms);
      float ls = 0.0f;
      half8 ph;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = __builtin_amdgcn_exp2f(fmaf(sc[e], sl2, -ms));
        ls = e == 0 ? pe : ls + pe;
        ph[e] = (_Float16)pe;
      }
      ls = rows_sum(ls);
      l[rb] = l[rb] * alpha + ls;
      m[rb] = mn;
      // the output is rescaled only when some query's maximum moved (alpha 1
      // elsewhere: skipping leaves every bit as it is)
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) O[rb][cb] *= alpha;
      }
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const uint16_t* vp = buf + voff + 8 * ((2 * cb + ((lj & 3) >> 1)) ^ vsw);
        typedef __attribute__((address_space(3))) short4v lds_s4;
        const half4v a0 = __builtin_bit_cast(half4v, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)vp));
        const half4v a1 = __builtin_bit_cast(half4v, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(vp + 4 * D)));
        const half8 av = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        O[rb][cb] = mfma16(av, ph, O[rb][cb]);
      }
    }
  };
  for (int c = 0; c < nchunks; c += 2) {
    step(c, cbuf0, cbuf1);
    if (c + 1 < nchunks) step(c + 1, cbuf1, cbuf0);
  }
  // ---- output rows and LSE (natural log: m * ln 2 + ln l). Lane (lq, lj)
  // holds O^T[column 16cb + 4lq + r][query lj].
#pragma unroll
  for (int rb = 0; rb < NR; ++rb) {
    const int g = rb_head(rb), qt = rb_qblk(rb);
    if (g >= G) continue;
    const int hq = h * G + g;
    const int qr = q0 + 16 * qt + lj;
    if (qr < q1) {
      const float il = 1.0f / l[rb];
      uint16_t* orow = pa.out + (((size_t)b * pa.Hq + hq) * S + qr) * D;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const uint32_t lo = (uint32_t)f2h(O[rb][cb][0] * il) | ((uint32_t)f2h(O[rb][cb][1] * il) << 16);
        const uint32_t hi = (uint32_t)f2h(O[rb][cb][2] * il) | ((uint32_t)f2h(O[rb][cb][3] * il) << 16);
        *reinterpret_cast<uint2*>(orow + 16 * cb + 4 * lq) = make_uint2(lo, hi);
      }
      if (pa.lse && lq == 0) pa.lse[((size_t)b * pa.Hq + hq) * S + qr] = m[rb] * kLn2 + logf(l[rb]);
    }
  }
}


// Future-attention target [KVpop summary §2.2], the transposed pass: for key
// t of a segment, log sum over the group's query heads g and the queries
// d >= t + w of exp(s[d, g, t] - LSE[d, g]), with the queries' normalisers
// handed in, so no attention map is formed. One workgroup per 64*kTgtTiles
// keys; wave w takes kTgtTiles 16-row MFMA A tiles of them. The later
// queries stream through LDS in stages of four (16-query tile, head) pairs,
// double-buffered and shared by the four waves; the MFMA gives
// S^T[key][query] and each lane accumulates the masked exponentials. Every
// workgroup streams the Q rows of all queries after its keys, so the keys
// per workgroup set how often Q is read again.
#ifndef CONFKV_TGT_TILES
#define CONFKV_TGT_TILES 4
#endif
constexpr int kTgtTiles = CONFKV_TGT_TILES;   // 16-key A tiles per wave
constexpr int kTgtKeys = 64 * kTgtTiles;      // keys per workgroup
template <int D, int G>
__global__ void __launch_bounds__(kThreads, 2) kvpop_target_kernel(KvpopPrefillArgs pa, const float* lse_in,
                                                                float* target) {
  constexpr int KS = D / 32;
  constexpr int QSTR = D + 8;                 // staged row stride (halves)
  constexpr int NP = 4;                       // (tile, head) pairs per stage
  constexpr int RP = D / 8;                   // 16-byte pieces per row
  constexpr int PPT = NP * 16 * RP / kThreads;
  static_assert(PPT * kThreads == NP * 16 * RP, "stage pieces divide the block");
  __shared__ __align__(16) uint16_t qs[2][NP][16][QSTR];
  __shared__ float ls[2][NP][16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the full-tile test is a scalar branch
  const int lq = lane >> 4, lj = lane & 15;
  const int S = pa.S, w = pa.window;
  int tile, seg;
  xcd_tile_seg(tile, seg);
  const int b = seg / pa.Hkv, h = seg - b * pa.Hkv;
  const int t0b = kTgtKeys * tile;             // the workgroup's first key
  const int t0 = t0b + 16 * kTgtTiles * wave;  // this wave's first key
  const uint16_t* kseg = pa.k + (size_t)seg * S * D;
  const float sl2 = pa.scale * kLog2e;

  half8 ka[kTgtTiles][KS];
#pragma unroll
  for (int kb = 0; kb < kTgtTiles; ++kb) {
    const int t = t0 + 16 * kb + lj;
    const uint16_t* kr = kseg + (size_t)min(t, S - 1) * D;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const uint4 u = *reinterpret_cast<const uint4*>(kr + 8 * (lq + 4 * kk));
      ka[kb][kk] = t < S ? as_h8(u) : half8{};
    }
  }
  float acc[kTgtTiles][4];
#pragma unroll
  for (int kb = 0; kb < kTgtTiles; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[kb][r] = 0.0f;

  // (query tile, head) pairs from the first tile holding a counted query
  const int x0 = (min(t0b + w, S) >> 4) * G, x1 = ((S + 15) >> 4) * G;
  const int nst = (x1 - x0 + NP - 1) / NP;
  uint4 pre[PPT];
  float plse = 0.0f;
  auto load_stage = [&](int st) {
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int e = tid + kThreads * u;
      const int pr = e / (16 * RP), rem = e - pr * 16 * RP, row = rem / RP, piece = rem - row * RP;
      const int x = x0 + NP * st + pr;
      if (x < x1) {
        const int tile = x / G, g = x - tile * G;
        const int d = min(16 * tile + row, S - 1);
        pre[u] = *reinterpret_cast<const uint4*>(pa.q + (((size_t)b * pa.Hq + h * G + g) * S + d) * D + 8 * piece);
      } else {
        pre[u] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    if (tid < NP * 16) {
      const int pr = tid >> 4, row = tid & 15;
      const int x = x0 + NP * st + pr;
      if (x < x1) {
        const int tile = x / G, g = x - tile * G;
        plse = lse_in[((size_t)b * pa.Hq + h * G + g) * S + min(16 * tile + row, S - 1)];
      }
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int e = tid + kThreads * u;
      const int pr = e / (16 * RP), rem = e - pr * 16 * RP, row = rem / RP, piece = rem - row * RP;
      *reinterpret_cast<uint4*>(&qs[buf][pr][row][8 * piece]) = pre[u];
    }
    if (tid < NP * 16) ls[buf][tid >> 4][tid & 15] = plse;
  };
  if (nst > 0) {
    load_stage(0);
    store_stage(0);
  }
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) load_stage(st + 1);
#pragma unroll
    for (int pr = 0; pr < NP; ++pr) {
      const int x = x0 + NP * st + pr;
      if (x >= x1) break;
      const int d0 = 16 * (x / G), d = d0 + lj;
      half8 qb[KS];
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) qb[kk] = as_h8(*reinterpret_cast<const uint4*>(&qs[buf][pr][lj][8 * (lq + 4 * kk)]));
      // exp(s*scale - lse) = 2^(c*scale*log2(e) - lse*log2(e)): one FMA and one exp2
      const float nl2 = -ls[buf][pr][lj] * kLog2e;
      auto qk = [&](int kb) {
        floatx4 c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) c = mfma16(ka[kb][kk], qb[kk], c);
        return c;
      };
      // every query of this tile counts for every key of this wave (a branch
      // uniform over the wave)
      if (d0 >= t0 + 16 * kTgtTiles - 1 + w && d0 + 15 < S) {
        // the products of key tile kb + 1 are issued before the
        // exponentials of tile kb, so the matrix unit works while they run
        floatx4 c = qk(0);
#pragma unroll
        for (int kb = 0; kb < kTgtTiles; ++kb) {
          floatx4 cn = c;
          if (kb + 1 < kTgtTiles) cn = qk(kb + 1);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[kb][r] += __builtin_amdgcn_exp2f(fmaf(c[r], sl2, nl2));
          c = cn;
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < kTgtTiles; ++kb) {
          const floatx4 c = qk(kb);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = t0 + 16 * kb + 4 * lq + r;
            const bool counted = d < S && d >= t + w;
            acc[kb][r] += counted ? __builtin_amdgcn_exp2f(fmaf(c[r], sl2, nl2)) : 0.0f;
          }
        }
      }
    }
    if (st + 1 < nst) store_stage(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int kb = 0; kb < kTgtTiles; ++kb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float a = acc[kb][r];
      for (int o = 1; o < 16; o <<= 1) a += __shfl_xor(a, o, 64);
      const int t = t0 + 16 * kb + 4 * lq + r;
      if (lj == 0 && t < S) target[(size_t)seg * S + t] = a > 0.0f ? logf(a) : -INFINITY;
    }
  }
}

template <int D>
static int launch_kvpop_attend_d(const KvpopPrefillArgs& pa, int lds_bytes, hipStream_t s) {
  const int qb = pa.G <= 4 ? 32 : 16;  // queries per workgroup (see the kernel)
  const dim3 grid((pa.S + qb - 1) / qb, pa.B * pa.Hkv);
  switch (pa.G) {  // 8 waves for groups of up to 4 heads, 4 for larger ones
    case 1: hipLaunchKernelGGL((kvpop_prefill_attend_kernel<D, 1, 512>), grid, dim3(512), lds_bytes, s, pa); break;
    case 2: hipLaunchKernelGGL((kvpop_prefill_attend_kernel<D, 2, 512>), grid, dim3(512), lds_bytes, s, pa); break;
    case 4: hipLaunchKernelGGL((kvpop_prefill_attend_kernel<D, 4, 512>), grid, dim3(512), lds_bytes, s, pa); break;
    case 5: hipLaunchKernelGGL((kvpop_prefill_attend_kernel<D, 5, 256>), grid, dim3(256), lds_bytes, s, pa); break;
    case 8: hipLaunchKernelGGL((kvpop_prefill_attend_kernel<D, 8, 256>), grid, dim3(256), lds_bytes, s, pa); break;
    default: return -1;
  }
  return ok_or_err();
}

// LDS of the attention kernel: the key lists (dynamic) and, with
// with_buffers, the two chunk buffers (static).
int kvpop_prefill_attend_lds(int D, int list_cap, bool with_buffers) {
  return ((list_cap + 31) & ~31) * 8 + (with_buffers ? 2 * 2 * 32 * D * 2 : 0);
}

int launch_kvpop_prefill(const KvpopPrefillArgs& pa, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int segs = pa.B * pa.Hkv;
  const int rb = std::min(pa.N, kRankBlock);
  hipLaunchKernelGGL(kvpop_rank_blocks_kernel, dim3(pa.N / rb, segs), dim3(1024), (size_t)rb * 8, s, pa);
  if (hipGetLastError() != hipSuccess) return -3;
  hipLaunchKernelGGL(kvpop_rank_kernel, dim3(segs), dim3(1024), (size_t)rb * 8, s, pa);
  if (hipGetLastError() != hipSuccess) return -3;
  hipLaunchKernelGGL(kvpop_threshold_kernel, dim3((pa.S + kThrChunk - 1) / kThrChunk, segs), dim3(kThrThreads),
                     ((pa.N + 31) / 32) * 4, s, pa);
  if (hipGetLastError() != hipSuccess) return -3;
  const int lds = kvpop_prefill_attend_lds(pa.D, pa.list_cap, false);
  if (pa.D == 64) return launch_kvpop_attend_d<64>(pa, lds, s);
  if (pa.D == 128) return launch_kvpop_attend_d<128>(pa, lds, s);
  return -1;
}

template <int D>
static int launch_target_d(const KvpopPrefillArgs& pa, const float* lse, float* target, hipStream_t s) {
  const dim3 grid((pa.S + kTgtKeys - 1) / kTgtKeys, pa.B * pa.Hkv);
  switch (pa.G) {
    case 1: hipLaunchKernelGGL((kvpop_target_kernel<D, 1>), grid, dim3(kThreads), 0, s, pa, lse, target); break;
    case 2: hipLaunchKernelGGL((kvpop_target_kernel<D, 2>), grid, dim3(kThreads), 0, s, pa, lse, target); break;
    case 4: hipLaunchKernelGGL((kvpop_target_kernel<D, 4>), grid, dim3(kThreads), 0, s, pa, lse, target); break;
    case 5: hipLaunchKernelGGL((kvpop_target_kernel<D, 5>), grid, dim3(kThreads), 0, s, pa, lse, target); break;
    case 8: hipLaunchKernelGGL((kvpop_target_kernel<D, 8>), grid, dim3(kThreads), 0, s, pa, lse, target); break;
    default: return -1;
  }
  return ok_or_err();
}

int launch_kvpop_target(const KvpopPrefillArgs& pa, const float* lse, float* target, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (pa.D == 64) return launch_target_d<64>(pa, lse, target, s);
  if (pa.D == 128) return launch_target_d<128>(pa, lse, target, s);
  return -1;
}

}  // namespace confkv
