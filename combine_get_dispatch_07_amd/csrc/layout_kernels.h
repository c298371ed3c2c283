// Dispatch layout kernels: top-k expert ids -> is_token_in_rank, per-rank and
// per-expert token counts, and the dispatch plan (per-token rank bitmask and
// per-64-token-chunk exclusive prefix counts per rank).
//
// Follows the is_token_in_rank filter of "DeepEP：年度总结中的计算通信重叠摘记"
// (notes.kuangjux.top), section 节点内通信: a token is marked only for the
// ranks that own one of its top-k experts.
//
// One lane per token, one wave per 64-token chunk.  Per-rank chunk counts come
// from wave ballots (one ballot + popcount per rank), expert counts from an
// LDS histogram; all counting is integer, so results do not depend on
// scheduling.  Inter-block prefix sums are done by a second, single-block
// kernel rather than by blocks waiting on each other.
#pragma once

#include "device_common.h"

namespace moe {

#ifndef MOE_LAYOUT_BLOCK
#define MOE_LAYOUT_BLOCK 256
#endif
constexpr int kLayoutBlock = MOE_LAYOUT_BLOCK;  // tokens per block, multi-block path
constexpr int kFusedMaxTokens = 1024;  // up to this many tokens one block does everything
constexpr int kFusedMaxChunks = kFusedMaxTokens / kWave;

struct LayoutArgs {
  const int32_t* topk_idx;
  int32_t* tokens_per_rank;
  int32_t* tokens_per_expert;
  uint8_t* mask;           // [T, R] bytes
  uint64_t* token_ranks;   // plan: [T] rank bitmask
  int32_t* chunk_base;     // plan: [R, NC] chunk counts, then exclusive prefix per rank
  int32_t* block_expert;   // plan scratch: [NB, E] per-block expert histogram
  int32_t* ws_rank_offsets;// plan: [R + 1]
  uint64_t rank_magic;
  int T, k, E, R, NC, NB;
  int mask_words;          // 1: mask rows written as 32-bit words (R % 4 == 0, aligned)
  int ids_vec4;            // 1: id rows read as 16-byte vectors (k % 4 == 0, 16-byte aligned)
};

// Rank bitmask of token t; valid expert ids are added to the LDS histogram.
// The id loads are issued together, unconditionally, from clamped addresses
// (a load under a lane-dependent branch or between LDS atomics would be
// waited for on its own, one memory round trip each).  KI: ids held per lane
// (k <= KI).
template <int KI>
__device__ __forceinline__ uint64_t token_rank_mask(const LayoutArgs& a, int t, int* hist) {
  if (a.T == 0) return 0;  // no rows to read (topk_idx may be absent)
  const int32_t* row = a.topk_idx + (size_t)min(t, a.T - 1) * a.k;
  int ids[KI];
  if (a.ids_vec4) {  // rows are 16-byte aligned: 4 ids per load
    const int4* row4 = reinterpret_cast<const int4*>(row);
#pragma unroll
    for (int j = 0; j < KI / 4; ++j) {
      const int4 q = row4[min(j, (a.k >> 2) - 1)];
      ids[4 * j] = q.x;
      ids[4 * j + 1] = q.y;
      ids[4 * j + 2] = q.z;
      ids[4 * j + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < KI; ++j) ids[j] = row[min(j, a.k - 1)];
  }
  uint64_t m = 0;
  if (t < a.T) {
#pragma unroll
    for (int j = 0; j < KI; ++j) {
      const int e = ids[j];
      if (j < a.k && (unsigned)e < (unsigned)a.E) {
        m |= 1ull << rank_of(e, a.rank_magic);
        atomicAdd(&hist[e], 1);
      }
    }
  }
  return m;
}

__device__ __forceinline__ void write_mask_row(const LayoutArgs& a, int t, uint64_t m) {
  uint8_t* dst = a.mask + (size_t)t * a.R;
  if (a.mask_words) {
    uint32_t* d32 = reinterpret_cast<uint32_t*>(dst);
    for (int w = 0; w < (a.R >> 2); ++w) {
      const uint32_t b = (uint32_t)(m >> (4 * w)) & 0xfu;
      d32[w] = (b & 1u) | ((b & 2u) << 7) | ((b & 4u) << 14) | ((b & 8u) << 21);
    }
  } else {
    for (int r = 0; r < a.R; ++r) dst[r] = (uint8_t)((m >> r) & 1u);
  }
}

// Adds each lane's rank bits m to the per-rank counters cnt[0..63] (LDS)
// with one atomic add per set bit: at most min(k, R) adds per lane, where one
// ballot per rank would take R dependent steps.  Integer adds: the result
// does not depend on their order.
__device__ __forceinline__ void add_rank_bits(uint64_t m, int* cnt) {
  for (uint64_t b = m; b; b &= b - 1) atomicAdd(&cnt[__builtin_ctzll(b)], 1);
}

// Lane r (< R) returns how many lanes of the wave have bit r set in m; `cnt`
// is 64 ints of LDS private to the wave.
__device__ __forceinline__ int wave_rank_counts(uint64_t m, int R, int lane, int* cnt) {
  cnt[lane] = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  add_rank_bits(m, cnt);
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  return lane < R ? cnt[lane] : 0;
}

// Wave 0: per-rank totals -> tokens_per_rank and the exclusive rank offsets.
__device__ __forceinline__ void publish_rank_offsets(const LayoutArgs& a, const int* total, int lane) {
  const int v = lane < a.R ? total[lane] : 0;
  const int incl = wave_inclusive_scan(v, lane);
  if (lane < a.R) {
    a.tokens_per_rank[lane] = v;
    a.ws_rank_offsets[lane] = incl - v;
  }
  if (lane == a.R - 1) a.ws_rank_offsets[a.R] = incl;
}

// The whole layout in one block of at least ceil(T/64) waves (at most 16):
// thread i owns token i, wave w chunk w; waves beyond the last chunk count
// nothing.  hist: E ints of LDS.  Returns after wave 0 has published the rank
// offsets; rank_total then holds the per-rank token counts.
template <int KI>
__device__ __forceinline__ void layout_one_block(const LayoutArgs& a, int* hist, int* chunk_cnt,
                                                 int (*wave_cnt)[kWave], int* rank_total) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  for (int e = tid; e < a.E; e += blockDim.x) hist[e] = 0;
  __syncthreads();

  const uint64_t m = token_rank_mask<KI>(a, tid, hist);
  if (tid < a.T) {
    a.token_ranks[tid] = m;
    write_mask_row(a, tid, m);
  }
  const int cnt = wave_rank_counts(m, a.R, lane, wave_cnt[wave]);
  if (lane < a.R) chunk_cnt[lane * kFusedMaxChunks + wave] = cnt;
  __syncthreads();

  for (int e = tid; e < a.E; e += blockDim.x) a.tokens_per_expert[e] = hist[e];
  if (tid < a.R) {  // at most 16 chunks: a serial scan per rank is shortest
    int run = 0;
    for (int c = 0; c < a.NC; ++c) {
      a.chunk_base[tid * a.NC + c] = run;
      run += chunk_cnt[tid * kFusedMaxChunks + c];
    }
    rank_total[tid] = run;
  }
  __syncthreads();
  if (wave == 0) publish_rank_offsets(a, rank_total, lane);
}

// T <= kFusedMaxTokens: one block of ceil(T/64) waves (at least one) does
// everything in one launch.  Dynamic LDS: hist[E]; static: chunk counts [R][16].
template <int KI>
__global__ __launch_bounds__(kFusedMaxTokens) void layout_fused_kernel(LayoutArgs a) {
  extern __shared__ int hist[];
  __shared__ int chunk_cnt[kWave * kFusedMaxChunks];
  __shared__ int wave_cnt[kFusedMaxChunks][kWave];
  __shared__ int rank_total[kWave];
  layout_one_block<KI>(a, hist, chunk_cnt, wave_cnt, rank_total);
}

// Multi-block path, pass 1: mask rows, token bitmasks, chunk counts, block histograms.
template <int KI>
__global__ __launch_bounds__(kLayoutBlock) void layout_count_kernel(LayoutArgs a) {
  extern __shared__ int hist[];  // [E]
  __shared__ int wave_cnt[kLayoutBlock / kWave][kWave];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  for (int e = tid; e < a.E; e += kLayoutBlock) hist[e] = 0;
  __syncthreads();

  const int t = blockIdx.x * kLayoutBlock + tid;
  const uint64_t m = token_rank_mask<KI>(a, t, hist);
  if (t < a.T) {
    a.token_ranks[t] = m;
    write_mask_row(a, t, m);
  }
  const int chunk = t >> 6;
  const int cnt = wave_rank_counts(m, a.R, lane, wave_cnt[tid >> 6]);
  if (chunk < a.NC && lane < a.R) a.chunk_base[lane * a.NC + chunk] = cnt;
  __syncthreads();
  for (int e = tid; e < a.E; e += kLayoutBlock) a.block_expert[(size_t)blockIdx.x * a.E + e] = hist[e];
}

// Multi-block path, pass 2 (one block): expert totals, per-rank chunk prefix, rank offsets.
__global__ __launch_bounds__(1024) void layout_finalize_kernel(LayoutArgs a) {
  __shared__ int rank_total[kWave];
  __shared__ int part_sum[1024];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int nwaves = blockDim.x >> 6;
  // Expert totals: with E < blockDim, P = blockDim / E threads per expert each
  // sum every P-th block row (independent loads, many in flight), then one
  // thread adds the P partials.  Integer sums: the order does not matter.
  const int P = a.E >= (int)blockDim.x ? 1 : (int)blockDim.x / a.E;
  for (int i = tid; i < P * a.E; i += blockDim.x) {
    const int e = i % a.E, part = i / a.E;
    int s = 0;
#pragma unroll 8
    for (int b = part; b < a.NB; b += P) s += a.block_expert[(size_t)b * a.E + e];
    if (P == 1)
      a.tokens_per_expert[e] = s;
    else
      part_sum[i] = s;
  }
  for (int r = wave; r < a.R; r += nwaves) {
    int* row = a.chunk_base + (size_t)r * a.NC;
    int carry = 0;
    for (int c0 = 0; c0 < a.NC; c0 += kWave) {
      const int c = c0 + lane;
      const int v = c < a.NC ? row[c] : 0;
      const int incl = wave_inclusive_scan(v, lane);
      if (c < a.NC) row[c] = carry + incl - v;
      carry += __builtin_amdgcn_readlane(incl, kWave - 1);
    }
    if (lane == 0) rank_total[r] = carry;
  }
  __syncthreads();
  if (P > 1) {
    for (int e = tid; e < a.E; e += blockDim.x) {
      int s = 0;
      for (int q = 0; q < P; ++q) s += part_sum[q * a.E + e];
      a.tokens_per_expert[e] = s;
    }
  }
  if (wave == 0) publish_rank_offsets(a, rank_total, lane);
}

}  // namespace moe
