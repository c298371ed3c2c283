// Low-latency (per-expert) receive layout: dispatch into one fixed-capacity
// buffer per expert, [E, cap, H], as the low-latency decode mode of the DeepEP
// pages keeps one buffer per local expert ("DeepEP：面向MoE的高吞吐低延迟GPU通信库",
// ssnai.com; "DeepEP：年度总结中的计算通信重叠摘记", notes.kuangjux.top, section
// 节点间通信).  One receive row per (token, distinct valid expert); the row of
// token t in expert e's buffer is the number of earlier tokens naming e.
//
// Positions are computed without any ordering race: a wave owns 64 tokens and
// builds, in LDS, one 64-bit membership mask per expert (atomicOr is order-
// independent); a token's position inside its chunk is popcount(mask[e] &
// lanes_below), and per-expert chunk counts are scanned across chunks.
#pragma once

#include "device_common.h"
#include "dispatch_kernels.h"

namespace moe {

constexpr int kLlFusedMaxTokens = 1024;  // one block of up to 16 waves does the whole layout
constexpr int kLlFusedMaxExperts = 512;  // 16 masks of E x 8 bytes fit in 64 KB of LDS

struct LlLayoutArgs {
  const int32_t* topk_idx;
  int32_t* slot_local;  // plan: [T, k] position inside the token's chunk, or -1
  int32_t* chunk_base;  // plan: [E, NC] chunk counts, then exclusive prefix per expert
  int32_t* recv_count;  // out: [E]
  int T, k, E, NC;
};

// Builds this wave's expert masks for its 64 tokens and writes in-chunk slot
// positions.  `mask` is this wave's [E] array in LDS, already zeroed.  The
// token's ids are loaded once (all loads issued together) and kept in
// registers for both passes.
__device__ __forceinline__ void ll_chunk_positions(const LlLayoutArgs& a, int chunk, int lane,
                                                   unsigned long long* mask) {
  constexpr int kMaxK = 32;  // the library's top-k limit
  const int t = chunk * kWave + lane;
  const unsigned long long bit = 1ull << lane;
  const bool live = t < a.T;
  const int32_t* row = a.topk_idx + (size_t)min(t, max(a.T - 1, 0)) * a.k;
  int ids[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) ids[j] = live && j < a.k ? row[j] : -1;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if ((unsigned)ids[j] < (unsigned)a.E) atomicOr(&mask[ids[j]], bit);
  __syncthreads();
  if (live) {
    const unsigned long long below = bit - 1ull;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < a.k)
        a.slot_local[(size_t)t * a.k + j] = (unsigned)ids[j] < (unsigned)a.E ? __popcll(mask[ids[j]] & below) : -1;
    }
  }
}

// Multi-block pass 1: one 64-token chunk per block (one wave).  Dynamic LDS: E x u64.
__global__ __launch_bounds__(kWave) void ll_count_kernel(LlLayoutArgs a) {
  extern __shared__ unsigned long long mask[];
  const int lane = threadIdx.x;
  for (int e = lane; e < a.E; e += kWave) mask[e] = 0ull;
  __syncthreads();
  ll_chunk_positions(a, blockIdx.x, lane, mask);
  for (int e = lane; e < a.E; e += kWave) a.chunk_base[(size_t)e * a.NC + blockIdx.x] = __popcll(mask[e]);
}

// Multi-block pass 2: one wave per expert scans its chunk counts.
__global__ __launch_bounds__(256) void ll_scan_kernel(LlLayoutArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= a.E) return;
  int* row = a.chunk_base + (size_t)e * a.NC;
  int carry = 0;
  for (int c0 = 0; c0 < a.NC; c0 += kWave) {
    const int c = c0 + lane;
    const int v = c < a.NC ? row[c] : 0;
    const int incl = wave_inclusive_scan(v, lane);
    if (c < a.NC) row[c] = carry + incl - v;
    carry += __builtin_amdgcn_readlane(incl, kWave - 1);
  }
  if (lane == 0) a.recv_count[e] = carry;
}

// T <= 1024 and E <= 512: one block, wave w owns chunk w.  Dynamic LDS: waves x E x u64.
__global__ __launch_bounds__(kLlFusedMaxTokens) void ll_layout_fused_kernel(LlLayoutArgs a) {
  extern __shared__ unsigned long long masks[];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int nwaves = blockDim.x >> 6;
  for (int i = tid; i < nwaves * a.E; i += blockDim.x) masks[i] = 0ull;
  __syncthreads();
  ll_chunk_positions(a, wave, lane, masks + (size_t)wave * a.E);
  __syncthreads();
  for (int e = tid; e < a.E; e += blockDim.x) {  // serial scan over at most 16 chunks
    int run = 0;
    for (int c = 0; c < a.NC; ++c) {
      a.chunk_base[(size_t)e * a.NC + c] = run;
      run += __popcll(masks[(size_t)c * a.E + e]);
    }
    a.recv_count[e] = run;
  }
}

struct LlDispatchArgs {
  const uint16_t* x;
  const int32_t* topk_idx;
  const int32_t* slot_local;
  const int32_t* chunk_base;
  void* recv_x;         // [E, cap, H]
  float* recv_scales;   // [E, cap, H/128]
  int32_t* recv_src_idx;  // [E, cap]
  int32_t* slot_pos;      // [T, k]
  int T, H, H8, k, E, NC, cap;
  int slices, items;
};

template <int U, bool kFp8>
__global__ __launch_bounds__(kDispatchBlock) void ll_dispatch_kernel(LlDispatchArgs a) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = blockIdx.x * (kDispatchBlock / kWave) + wave;
  if (item >= a.items) return;
  const int t = item / a.slices;
  const int s = item - t * a.slices;
  const int chunk = t >> 6;

  // lane j < k: slot j's expert, receive position, and whether it is the first
  // slot naming it.  Loads are unconditional from clamped addresses, so the x
  // slice and the ids are in flight together (the chunk base needs the id).
  const int jl = min(lane, a.k - 1);
  const int e_raw = a.topk_idx[(size_t)t * a.k + jl];
  const int local = a.slot_local[(size_t)t * a.k + jl];
  const int c0 = s * (U * kWave) + lane;
  const u32x4* xrow = reinterpret_cast<const u32x4*>(a.x + (size_t)t * a.H);
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(xrow + min(c0 + u * kWave, a.H8 - 1));
  const int e = lane < a.k ? e_raw : -1;
  const bool valid = (unsigned)e < (unsigned)a.E;
  const int base = a.chunk_base[(size_t)(valid ? e : 0) * a.NC + chunk];
  int pos = valid ? base + local : -1;
  if ((unsigned)pos >= (unsigned)a.cap) pos = -1;  // only a plan from another layout gets here
  bool first = pos >= 0;
  for (int j = 0; j < a.k; ++j) {  // an earlier slot naming the same expert sends the row
    const int other = __builtin_amdgcn_readlane(e, j);
    first = first && !(j < lane && other == e);
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (c0 + u * kWave >= a.H8) v[u] = u32x4{0u, 0u, 0u, 0u};
  u32x2 q[U];
  float sc[U];
  if constexpr (kFp8) quantize_slice<U>(v, q, sc);

  if (s == 0 && lane < a.k) a.slot_pos[(size_t)t * a.k + lane] = pos;
  uint64_t todo = __ballot(first);
  while (todo) {
    const int j = __builtin_ctzll(todo);
    todo &= todo - 1;
    const int ej = __builtin_amdgcn_readlane(e, j);
    const int pj = __builtin_amdgcn_readlane(pos, j);
    const size_t row = (size_t)ej * a.cap + pj;
    if (s == 0 && lane == 0) a.recv_src_idx[row] = t;
    store_slice<U, kFp8>(a.recv_x, a.recv_scales, (size_t)row, a.H, a.H8, c0, lane, v, q, sc);
  }
}

// ---------------------------------------------------------------------------
// Small batches (T <= 1024): layout and dispatch in one launch.  Block t < T
// owns token t.  Its waves take the hidden slices (one each) and, in 64-token
// batches (one each), all T tokens' ids: a slot's position is the number of
// earlier tokens naming its expert (ballot counts added into LDS), and the
// token writes recv_count[e] = position + 1 for each expert no later token
// names.  Block T writes recv_count[e] = 0 for the experts no token names.
// All loads are issued together from clamped, always valid addresses and
// masked afterwards (a load under a lane-dependent branch would be waited for
// before the branch joins, one memory round trip per load).  Same rows,
// positions and counts as the two-pass path.  KI: ids held per lane (k <= KI).
constexpr int kLlSmallMaxTokens = 1024;
constexpr int kLlSmallMaxWaves = 16;

template <int U, bool kFp8, int KI>
__global__ __launch_bounds__(kLlSmallMaxWaves * kWave) void ll_dispatch_small_kernel(LlDispatchArgs a,
                                                                                      int32_t* recv_count) {
#pragma clang fp contract(off)
  __shared__ int cnt[kMaxTopk];    // slot j: earlier tokens naming its expert
  __shared__ int after[kMaxTopk];  // slot j: later tokens naming its expert
  __shared__ unsigned char named[kMaxExperts];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (a.T == 0) {  // no tokens (topk_idx may be absent): every count is 0
    for (int e = threadIdx.x; e < a.E; e += blockDim.x) recv_count[e] = 0;
    return;
  }

  // This wave's batch of tokens: lane l holds token 64 * wave + l's ids.
  const int u = wave * kWave + lane;
  const bool has_batch = wave * kWave < a.T;
  int ids[KI];
  {
    const int32_t* row = a.topk_idx + (size_t)min(u, a.T - 1) * a.k;
#pragma unroll
    for (int i = 0; i < KI; ++i) ids[i] = row[min(i, a.k - 1)];
  }

  if (blockIdx.x == a.T) {  // experts no token names
    for (int e = threadIdx.x; e < a.E; e += blockDim.x) named[e] = 0;
    __syncthreads();
    if (u < a.T) {
#pragma unroll
      for (int i = 0; i < KI; ++i)
        if (i < a.k && (unsigned)ids[i] < (unsigned)a.E) named[ids[i]] = 1;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < a.E; e += blockDim.x)
      if (!named[e]) recv_count[e] = 0;
    return;
  }

  const int t = blockIdx.x;
  const int e_raw = a.topk_idx[(size_t)t * a.k + min(lane, a.k - 1)];
  const int c0 = wave * (U * kWave) + lane;
  const u32x4* xrow = reinterpret_cast<const u32x4*>(a.x + (size_t)t * a.H);
  u32x4 v[U];
#pragma unroll
  for (int uu = 0; uu < U; ++uu) v[uu] = __builtin_nontemporal_load(xrow + min(c0 + uu * kWave, a.H8 - 1));
  if (threadIdx.x < kMaxTopk) {
    cnt[threadIdx.x] = 0;
    after[threadIdx.x] = 0;
  }
#pragma unroll
  for (int i = 0; i < KI; ++i) ids[i] = i < a.k ? ids[i] : -1;
  // lane j < k: slot j's expert, and whether it is the first slot naming it
  const int e = lane < a.k ? e_raw : -1;
  const bool valid = lane < a.k && (unsigned)e < (unsigned)a.E;
  bool first = valid;
  for (int j = 0; j < a.k; ++j) {
    const int other = __builtin_amdgcn_readlane(e, j);
    first = first && !(j < lane && other == e);
  }
  __syncthreads();

  if (has_batch) {
    const int d = t - wave * kWave;  // lanes l < d hold earlier tokens, l > d later ones
    const uint64_t below = d <= 0 ? 0ull : d >= kWave ? ~0ull : (1ull << d) - 1ull;
    const uint64_t above = d < 0 ? ~0ull : d >= kWave - 1 ? 0ull : ~((1ull << d << 1) - 1ull);
    const uint64_t live = __ballot(u < a.T);
    int n_before = 0, n_after = 0;  // lane j: slot j's counts over this batch
    for (int j = 0; j < a.k; ++j) {
      const int ej = __builtin_amdgcn_readlane(e, j);
      bool hit = false;
#pragma unroll
      for (int i = 0; i < KI; ++i) hit = hit || ids[i] == ej;
      const uint64_t m = __ballot(hit) & live;
      n_before = lane == j ? __popcll(m & below) : n_before;
      n_after = lane == j ? __popcll(m & above) : n_after;
    }
    if (lane < a.k) {
      if (n_before) atomicAdd(&cnt[lane], n_before);
      if (n_after) atomicAdd(&after[lane], n_after);
    }
  }

#pragma unroll
  for (int uu = 0; uu < U; ++uu)
    if (c0 + uu * kWave >= a.H8) v[uu] = u32x4{0u, 0u, 0u, 0u};
  u32x2 q[U];
  float sc[U];
  if constexpr (kFp8) quantize_slice<U>(v, q, sc);
  __syncthreads();

  int pos = valid ? cnt[lane] : -1;
  if (pos >= a.cap) pos = -1;  // unreachable: cap >= T is checked on the host
  if (wave == 0) {
    if (lane < a.k) a.slot_pos[(size_t)t * a.k + lane] = pos;
    if (first && pos >= 0 && after[lane] == 0) recv_count[e] = pos + 1;  // the last token naming e
  }
  uint64_t todo = __ballot(first && pos >= 0);
  while (todo) {
    const int j = __builtin_ctzll(todo);
    todo &= todo - 1;
    const int ej = __builtin_amdgcn_readlane(e, j);
    const int pj = __builtin_amdgcn_readlane(pos, j);
    const size_t row = (size_t)ej * a.cap + pj;
    if (wave == 0 && lane == 0) a.recv_src_idx[row] = t;
    store_slice<U, kFp8>(a.recv_x, a.recv_scales, (size_t)row, a.H, a.H8, c0, lane, v, q, sc);
  }
}

}  // namespace moe
