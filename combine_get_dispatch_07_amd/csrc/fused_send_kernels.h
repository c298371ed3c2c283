// The send side in one launch: top-k routing, its layout and the dispatch.
// "DeepEP：年度总结中的计算通信重叠摘记" (notes.kuangjux.top), section 节点内通信,
// notes that DeepEP runs top-k together with the sparse exchange so that no CPU
// step and no launch gap separates them; here the routing blocks and the
// packing blocks share one launch.
//
// Blocks take role tickets from a counter in the workspace when they start:
// the first `producers` tickets route tokens exactly as the one-launch router
// kernel does (ids, weights, token rank bitmasks, expert counts; the last of
// them to finish also writes the layout's outputs and the plan).  Every later
// ticket is a dispatch block: it loads its x slices, waits until the last routing
// block raises the ready flag (every routing block has handed over its tokens
// by then), then loads all T token bitmasks and
// computes its rows itself -- per 64-token batch, one ballot per rank gives the
// batch's tokens going to that rank; their prefix over batches and ranks gives
// each destination row -- so the packing does not wait for the plan's last
// step.  A dispatch block only ever waits for routing blocks, every one of
// which took its role ticket (so it is running) before any dispatch block did
// and never waits: the launch completes whatever the number of resident blocks.
// Data handed from routing to dispatch blocks goes through the L2
// (put_coherent / get_coherent); the last block to leave resets the sync words.
#pragma once

#include "device_common.h"
#include "dispatch_kernels.h"
#include "layout_kernels.h"
#include "router_kernels.h"

namespace moe {

// Waves per block of the fused launch.  Every block takes a role ticket and an
// exit ticket from one counter each, and same-address atomics serialise (a few
// ns apiece), so blocks are large: a routing block routes with its first
// kRouterSmallWaves waves, a dispatch block packs one item per wave.
constexpr int kFusedWaves = 16;
static_assert(kRouterSmallWaves <= kFusedWaves, "routing waves fit a fused block");
static_assert(kFusedMaxChunks <= kFusedWaves, "one 64-token batch per wave");

// Polls of the ready flag before a dispatch block gives up (several seconds):
// reached only if the routing blocks never complete, which no input can cause.
constexpr uint32_t kReadySpins = 1u << 22;

struct FusedSendArgs {
  RouterArgs r;   // the routing and its layout
  DispatchArgs d;
  int producers;  // routing blocks
};

// The block's role ticket (same value in every thread).
__device__ __forceinline__ uint32_t draw_role(SyncWords* sync) {
  __shared__ uint32_t role;
  if (threadIdx.x == 0) role = __hip_atomic_fetch_add(&sync->role, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  return role;
}

// Dispatch blocks: thread 0 polls the ready flag, which the last routing block
// raises once every routing block's hand-off writes have completed (a line of
// its own: the routing blocks' ticket atomics do not queue behind the polls).
__device__ __forceinline__ bool wait_producers(const SyncWords* sync) {
  __shared__ uint32_t seen;
  if (threadIdx.x == 0) {
    uint32_t v = get_coherent(&sync->ready);
    for (uint32_t spin = 0; v == 0u && spin < kReadySpins; ++spin) {
      __builtin_amdgcn_s_sleep(8);  // about 0.2 us between polls
      v = get_coherent(&sync->ready);
    }
    seen = v;
  }
  __syncthreads();
  return seen != 0u;
}

// Every block once, at its end: the last one to leave resets the sync words
// for the next launch (every block has taken its role and seen the flag).
__device__ __forceinline__ void leave(SyncWords* sync, uint32_t blocks) {
  if (threadIdx.x == 0) {
    const uint32_t n = __hip_atomic_fetch_add(&sync->exits, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (n == blocks - 1) {
      clear_word(&sync->role);
      clear_word(&sync->ticket);
      clear_word(&sync->ready);
      clear_word(&sync->exits);
    }
  }
}

// A dispatch block: wave w takes item kFusedWaves (role - producers) + w.
// tok_m: T bitmasks of LDS; cnt: per batch and rank, the batch's tokens going to
// the rank, then their exclusive prefix over batches; seg: rank offsets (LDS).
template <int U, bool kFp8>
__device__ __forceinline__ void fused_dispatch_block(const FusedSendArgs& f, uint32_t role, SyncWords* sync,
                                                     uint64_t* tok_m, int (*cnt)[kWave], int* seg) {
  const DispatchArgs& a = f.d;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = ((int)role - f.producers) * kFusedWaves + wave;
  const bool live = item < a.items;
  const int t = live ? item / a.slices : 0;
  const int s = item - t * a.slices;
  u32x4 v[U];
  if (live) load_item_slice<U, kFp8>(a, item, lane, v);  // x does not depend on the routing
  if (!wait_producers(sync)) return;

  // wave w < number of batches: the bitmasks of tokens 64 w .. 64 w + 63 (through the L2), and the
  // item's slot ids and weights
  const int nb = (a.T + kWave - 1) / kWave;
  const int u = wave * kWave + lane;
  const uint64_t m_raw = get_coherent(&a.token_ranks[min(u, a.T - 1)]);
  const int jl = min(lane, a.k - 1);
  int ej_raw = -1;
  float wj_raw = 0.0f;
  if (live && (kFp8 || s == 0)) {
    ej_raw = get_coherent(&a.topk_idx[(size_t)t * a.k + jl]);
    wj_raw = get_coherent(&a.topk_w[(size_t)t * a.k + jl]);
  }
  if (wave < nb) {
    const uint64_t m = u < a.T ? m_raw : 0ull;
    tok_m[u] = m;
    int c = 0;  // lane r: the batch's tokens going to rank r
    for (int r = 0; r < a.R; ++r) {
      const int n = __popcll(__ballot((m >> r) & 1ull));
      c = lane == r ? n : c;
    }
    cnt[wave][lane] = c;
  }
  __syncthreads();
  if (wave == 0) {  // lane r: prefix over batches, then the rank offsets
    int run = 0;
    for (int b = 0; b < nb; ++b) {
      const int c = cnt[b][lane];
      cnt[b][lane] = run;
      run += c;
    }
    const int total = lane < a.R ? run : 0;
    seg[lane] = wave_inclusive_scan(total, lane) - total;
  }
  __syncthreads();
  if (!live) return;
  const int tb = t >> 6;
  const uint64_t lm = tok_m[min(tb * kWave + lane, nb * kWave - 1)];
  const int chunk_row = lane < a.R ? seg[lane] + cnt[tb][lane] : 0;
  pack_item<U, kFp8>(a, t, s, lane, v, lm, chunk_row, ej_raw, wj_raw);
}

// Routing, layout and dispatch of T <= kFusedMaxTokens tokens in one launch.
template <int P, int KS, int U, bool kFp8>
__global__ __launch_bounds__(kFusedWaves * kWave) void route_dispatch_kernel(FusedSendArgs f) {
  __shared__ int cnt[kFusedMaxChunks][kWave];
  __shared__ int offs[kWave + 1];
  __shared__ uint64_t tok_m[kFusedMaxTokens];
  SyncWords* sync = f.r.lay.sync;
  const uint32_t role = draw_role(sync);
  if ((int)role < f.producers)
    router_small_produce<P, KS, true>(f.r, role, f.producers, cnt, offs);
  else
    fused_dispatch_block<U, kFp8>(f, role, sync, tok_m, cnt, offs);
  leave(sync, gridDim.x);
}

}  // namespace moe
