// Top-k gating fused with the dispatch layout.
//
// "DeepEP：年度总结中的计算通信重叠摘记" (notes.kuangjux.top), section 节点内通信, notes
// that DeepEP computes top-k together with the sparse exchange so that no CPU
// step separates them; its section 计算-通信重叠 names DeepSeek's group-limited
// gating as the routing DeepEP was built around.  Per token, from fp32 logits:
//   * group-limited gating: G equal contiguous groups, score = largest logit,
//     the best KG groups kept (ties to the lower group);
//   * top-k among the eligible experts by logit, ties to the lower id, slots in
//     descending order;
//   * weights: softmax over the k selected logits, or the sigmoid gate
//     normalised over the k selected (fp32, expf);
// and, in the same pass, what the layout kernels compute from the ids: the
// token's rank bitmask and is_token_in_rank row, per-64-token-chunk rank counts
// and per-block expert histograms.
//
// Work split: 8 lanes per token, lane p holding experts [p*V, p*V + V),
// V = E / 8, so a wave routes 8 tokens and a block of 8 waves one 64-token
// layout chunk.  Each lane sorts its V candidates into a register list of the
// best KL (insertion with a constant per-position comparison, so equal logits
// keep the earlier, lower id); the token's k picks are then k rounds of a max
// over the 8 list heads, keyed by (logit, lower id), whose owner pops its head.
// Logits are compared through an order-preserving unsigned key (-0.0 folded
// into +0.0), so every selection decision is exact.
#pragma once

#include "device_common.h"
#include "layout_kernels.h"

namespace moe {

constexpr int kRouterLanes = 8;                           // lanes per token
constexpr int kRouterTokensPerWave = kWave / kRouterLanes;  // 8
constexpr int kRouterBlock = 512;                         // 8 waves = one 64-token chunk
constexpr int kRouterFusedMaxTokens = 128;                // one block of up to 16 waves does all
constexpr int kRouterMaxExperts = 512;                    // V <= 64

struct RouterArgs {
  const float* logits;  // [T, E]
  int32_t* topk_idx;    // [T, k]
  float* topk_w;        // [T, k]
  LayoutArgs lay;       // outputs and plan, as the layout kernels fill them
  int V;                // experts per lane, E / 8
  int G, KG;            // groups, kept groups (G = 1: no group limit)
  int sigmoid;          // 0: softmax over the selected, 1: normalised sigmoid
  int vec4;             // 1: logit rows read as 16-byte vectors
};

// Order-preserving map of fp32 bits to uint32 (larger float, larger key),
// with -0.0 folded into +0.0.  Finite and infinite logits map to keys
// >= 0x007fffff; the bit pattern 0xffffffff (a NaN, never a valid logit) maps
// to 0, which marks "not eligible".
constexpr uint32_t kNoLogit = 0xffffffffu;

__device__ __forceinline__ uint32_t logit_key(uint32_t u) {
  u = u == 0x80000000u ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_logit(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Routes tokens t0 + (lane >> 3); returns the token's rank bitmask (same in its
// 8 lanes; 0 for t >= T) and adds its experts to the LDS histogram.
template <int VMAX, int KL>
__device__ __forceinline__ uint64_t route_token(const RouterArgs& a, int t, int lane, int* hist) {
#pragma clang fp contract(off)
  const LayoutArgs& L = a.lay;
  const int p = lane & (kRouterLanes - 1);
  const int gbase = lane & ~(kRouterLanes - 1);
  const bool live = t < L.T;

  // 1. this lane's V logits as bits (all loads issued before any is used);
  //    kNoLogit beyond V or for t >= T, so the sort below needs no conditions
  uint32_t xb[VMAX];
  const float* row = a.logits + (size_t)min(t, max(L.T - 1, 0)) * L.E + (size_t)p * a.V;
  if (a.vec4) {
#pragma unroll
    for (int v = 0; v < VMAX; v += 4) {
      u32x4 q = {kNoLogit, kNoLogit, kNoLogit, kNoLogit};
      if (live && v < a.V) q = *reinterpret_cast<const u32x4*>(row + v);
#pragma unroll
      for (int i = 0; i < 4; ++i) xb[v + i] = q[i];
    }
  } else {
    const uint32_t* rowb = reinterpret_cast<const uint32_t*>(row);
#pragma unroll
    for (int v = 0; v < VMAX; ++v) xb[v] = live && v < a.V ? rowb[v] : kNoLogit;
  }

  // 2. per-lane sorted list of the best KL candidates.  Positions v ascend
  //    with the expert id, so a strict comparison keeps equal logits in id order.
  uint32_t lk[KL];
  int li[KL];  // position v within the lane (a constant per insertion), expert = p * V + v
#pragma unroll
  for (int i = 0; i < KL; ++i) {
    lk[i] = 0u;
    li[i] = 0;
  }
#pragma unroll
  for (int v = 0; v < VMAX; ++v) {
    const uint32_t nk = logit_key(xb[v]);
    bool c[KL];
#pragma unroll
    for (int i = 0; i < KL; ++i) c[i] = nk > lk[i];  // true from the insertion point on
#pragma unroll
    for (int i = KL - 1; i > 0; --i) {
      lk[i] = c[i] ? (c[i - 1] ? lk[i - 1] : nk) : lk[i];
      li[i] = c[i] ? (c[i - 1] ? li[i - 1] : v) : li[i];
    }
    lk[0] = c[0] ? nk : lk[0];
    li[0] = c[0] ? v : li[0];
  }

  // 3. group-limited gating: 8 / G consecutive lanes form one group, so the
  //    group score is the largest list head among them; a lane of a group that
  //    is not kept empties its list.
  if (a.G > 1) {
    const int lpg = kRouterLanes / a.G;
    uint32_t m = lk[0];
    for (int s = 1; s < lpg; s <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, s, kWave));
    const int g = p / lpg;
    int better = 0;
    for (int q = 0; q < a.G; ++q) {
      const uint32_t sq = (uint32_t)__shfl((int)m, gbase + q * lpg, kWave);
      better += (sq > m || (sq == m && q < g)) ? 1 : 0;
    }
    if (better >= a.KG) {
#pragma unroll
      for (int i = 0; i < KL; ++i) lk[i] = 0u;
    }
  }

  // 4. k rounds over the 8 heads; slot j is kept by lane j % 8
  constexpr int kSlots = KL / kRouterLanes;  // slots per lane (k <= KL)
  int sid[kSlots];
  uint32_t skey[kSlots];
#pragma unroll
  for (int q = 0; q < kSlots; ++q) {
    sid[q] = -1;
    skey[q] = 0u;
  }
  uint64_t ranks = 0;
  uint32_t key0 = 0u;
  for (int j = 0; j < L.k; ++j) {
    const uint64_t mine = ((uint64_t)lk[0] << 32) | (uint32_t)~(p * a.V + li[0]);
    uint64_t best = mine;
#pragma unroll
    for (int s = 1; s < kRouterLanes; s <<= 1) {
      const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)best, s, kWave);
      const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(best >> 32), s, kWave);
      const uint64_t o = ((uint64_t)hi << 32) | lo;
      best = o > best ? o : best;
    }
    const int id = (int)~(uint32_t)best;
    const uint32_t bk = (uint32_t)(best >> 32);
    if (j == 0) key0 = bk;
    ranks |= 1ull << rank_of(id, L.rank_magic);
#pragma unroll
    for (int q = 0; q < kSlots; ++q) {  // no dynamic register indexing
      if (j == q * kRouterLanes + p) {
        sid[q] = id;
        skey[q] = bk;
      }
    }
    if (best == mine) {  // the owner pops its head
#pragma unroll
      for (int i = 0; i + 1 < KL; ++i) {
        lk[i] = lk[i + 1];
        li[i] = li[i + 1];
      }
      lk[KL - 1] = 0u;
      li[KL - 1] = 0;
    }
  }

  // 5. weights, summed in a fixed order (per lane, then a butterfly over the 8 lanes)
  float ev[kSlots];
  float sum = 0.0f;
#pragma unroll
  for (int q = 0; q < kSlots; ++q) {
    const float l = key_logit(skey[q]);
    float e = a.sigmoid ? 1.0f / (1.0f + expf(-l)) : expf(l - key_logit(key0));
    e = sid[q] >= 0 ? e : 0.0f;
    ev[q] = e;
    sum = sum + e;
  }
#pragma unroll
  for (int s = 1; s < kRouterLanes; s <<= 1) sum = sum + __shfl_xor(sum, s, kWave);

  if (live) {
#pragma unroll
    for (int q = 0; q < kSlots; ++q) {
      const int j = q * kRouterLanes + p;
      if (j < L.k) {
        a.topk_idx[(size_t)t * L.k + j] = sid[q];
        a.topk_w[(size_t)t * L.k + j] = ev[q] / sum;
        atomicAdd(&hist[sid[q]], 1);
      }
    }
    // layout outputs of this token: bitmask and is_token_in_rank row
    if (p == 0) L.token_ranks[t] = ranks;
    uint8_t* dst = L.mask + (size_t)t * L.R;
    if (L.mask_words) {
      uint32_t* d32 = reinterpret_cast<uint32_t*>(dst);
      for (int w = p; w < (L.R >> 2); w += kRouterLanes) {
        const uint32_t b = (uint32_t)(ranks >> (4 * w)) & 0xfu;
        d32[w] = (b & 1u) | ((b & 2u) << 7) | ((b & 4u) << 14) | ((b & 8u) << 21);
      }
    } else {
      for (int r = p; r < L.R; r += kRouterLanes) dst[r] = (uint8_t)((ranks >> r) & 1u);
    }
  }
  return live ? ranks : 0;
}

// T > kRouterFusedMaxTokens: block b routes chunk b (64 tokens) and writes its
// chunk counts and expert histogram; layout_finalize_kernel (NB = NC) follows.
template <int VMAX, int KL>
__global__ __launch_bounds__(kRouterBlock) void router_count_kernel(RouterArgs a) {
  extern __shared__ int hist[];  // [E]
  __shared__ uint64_t chunk_masks[kWave];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const LayoutArgs& L = a.lay;
  for (int e = tid; e < L.E; e += kRouterBlock) hist[e] = 0;
  __syncthreads();

  const int tw = wave * kRouterTokensPerWave + (lane >> 3);  // token within the chunk
  const uint64_t m = route_token<VMAX, KL>(a, blockIdx.x * kWave + tw, lane, hist);
  if ((lane & (kRouterLanes - 1)) == 0) chunk_masks[tw] = m;
  __syncthreads();

  if (wave == 0) {
    const int cnt = wave_rank_counts(chunk_masks[lane], L.R, lane);
    if (lane < L.R) L.chunk_base[lane * L.NC + blockIdx.x] = cnt;
  }
  for (int e = tid; e < L.E; e += kRouterBlock) L.block_expert[(size_t)blockIdx.x * L.E + e] = hist[e];
}

// T <= kRouterFusedMaxTokens: one block of ceil(T / 8) waves (at least one)
// routes every token and finishes the layout (at most two chunks).
template <int VMAX, int KL>
__global__ __launch_bounds__(kRouterFusedMaxTokens * kRouterLanes) void router_layout_fused_kernel(RouterArgs a) {
  extern __shared__ int hist[];  // [E]
  __shared__ uint64_t masks[kRouterFusedMaxTokens];
  __shared__ int chunk_cnt[2][kWave];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const LayoutArgs& L = a.lay;
  for (int e = tid; e < L.E; e += blockDim.x) hist[e] = 0;
  for (int i = tid; i < kRouterFusedMaxTokens; i += blockDim.x) masks[i] = 0;
  __syncthreads();

  const int t = wave * kRouterTokensPerWave + (lane >> 3);
  const uint64_t m = route_token<VMAX, KL>(a, t, lane, hist);
  if ((lane & (kRouterLanes - 1)) == 0 && t < kRouterFusedMaxTokens) masks[t] = m;
  __syncthreads();

  if (wave < 2) {  // chunk `wave`: per-rank token counts
    const int cnt = wave_rank_counts(masks[wave * kWave + lane], L.R, lane);
    if (lane < L.R) chunk_cnt[wave][lane] = cnt;
  }
  for (int e = tid; e < L.E; e += blockDim.x) L.tokens_per_expert[e] = hist[e];
  __syncthreads();
  if (wave == 0) {
    int c0 = 0, total = 0;
    if (lane < L.R) {
      c0 = chunk_cnt[0][lane];
      total = c0 + (L.NC > 1 ? chunk_cnt[1][lane] : 0);
      if (L.NC > 0) L.chunk_base[lane * L.NC] = 0;
      if (L.NC > 1) L.chunk_base[lane * L.NC + 1] = c0;
    }
    const int incl = wave_inclusive_scan(lane < L.R ? total : 0, lane);
    if (lane < L.R) {
      L.tokens_per_rank[lane] = total;
      L.ws_rank_offsets[lane] = incl - total;
    }
    if (lane == L.R - 1) L.ws_rank_offsets[L.R] = incl;
  }
}

}  // namespace moe
