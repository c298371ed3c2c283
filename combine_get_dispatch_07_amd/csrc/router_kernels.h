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
// and what the layout kernels compute from the ids: the token's rank bitmask
// and is_token_in_rank row, per-64-token-chunk rank counts and expert counts.
// One launch at every batch size: the routing block that finishes last
// completes the plan (prefix sums, offsets, totals), so no host step or second
// launch separates routing from the layout.  Batches above 1024 tokens route
// one 64-token chunk per block (router_count_kernel); smaller ones use 4-wave
// blocks of 16 or 32 tokens to spread the routing over more CUs
// (router_small_kernel).
//
// Work split: P lanes per token (16 when E % 16 == 0, else 8), lane p
// holding experts [p*V, p*V + V), V = E / P.  Candidates are ordered by (logit key, then lower expert id).
// Each lane keeps a sorted register list of its KL best; the token's k picks
// are k rounds of a max over the P list heads (DPP lane exchanges, 32-bit
// operations only: 64-bit compares cost several times more on this GPU) whose
// owner pops its head.  A lane that runs out of list entries while picks
// remain rebuilds its list from the candidates after its last pick
// ("refill"), so KL bounds only the work, not k.
#pragma once

#include "device_common.h"
#include "layout_kernels.h"

namespace moe {

constexpr int kRouterList = 4;  // KL: list entries per lane
constexpr int kRouterSmallWaves = 4;  // waves per block of router_small_kernel
constexpr int kRouterMaxK = 16;  // slots per token handled (one or two per lane)

struct RouterArgs {
  const float* logits;  // [T, E]
  int32_t* topk_idx;    // [T, k]
  float* topk_w;        // [T, k]
  LayoutArgs lay;       // outputs and plan, as the layout kernels fill them
  int V;                // experts per lane, E / P
  int G, KG;            // groups, kept groups (G = 1: no group limit)
  int sigmoid;          // 0: softmax over the selected, 1: normalised sigmoid
  int vec4;             // 1: logit rows read as 16-byte vectors
};

// Order-preserving map fp32 -> uint32 (larger float, larger key).  x + 0.0
// turns -0.0 into +0.0 (IEEE addition; the compiler may not drop it), so the
// two zeros are one key.  Every finite or infinite logit maps to a key of at
// least 0x007fffff; 0 marks "no candidate".
__device__ __forceinline__ uint32_t logit_key(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ float key_logit(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

template <int N>
__device__ __forceinline__ uint32_t lanes_or(uint32_t x) {
  return lanes_reduce<N>(x, [](uint32_t u, uint32_t v) { return u | v; });
}

// Runtime group width (2, 4 or 8 lanes of the token's P) for group scores.
template <int P>
__device__ __forceinline__ uint32_t group_max(uint32_t x, int lpg) {
  if (lpg >= 2) x = max(x, dpp32<kXor1>(x));
  if (lpg >= 4) x = max(x, dpp32<kXor2>(x));
  if (P >= 16 && lpg >= 8) x = max(x, dpp32<kMirror8>(x));
  return x;
}

// A lane's list: its best candidates, keys descending (0 = empty), with their
// expert ids.  Candidates are offered in ascending id order, so a new one loses
// every tie with an entry already listed and `key > lk[i]` alone decides where
// it goes; entries below the insertion point shift down, the last falls off.
// Keys move with min / max; ids with bitwise selects on all-ones / zero masks.
// The empty asm hides the masks from the optimiser, which would otherwise turn
// the nested selects into branches.
__device__ __forceinline__ uint32_t bitsel(uint32_t m, uint32_t a, uint32_t b) { return (a & m) | (b & ~m); }

template <int KL>
__device__ __forceinline__ void list_insert(uint32_t (&lk)[KL], int (&li)[KL], uint32_t key, int id) {
  uint32_t gt[KL];
#pragma unroll
  for (int i = 0; i < KL; ++i) {
    gt[i] = key > lk[i] ? ~0u : 0u;  // all ones from the insertion point on
    __asm__("" : "+v"(gt[i]));
  }
#pragma unroll
  for (int i = KL - 1; i > 0; --i) {
    li[i] = (int)bitsel(gt[i], bitsel(gt[i - 1], (uint32_t)li[i - 1], (uint32_t)id), (uint32_t)li[i]);
    lk[i] = max(lk[i], min(key, lk[i - 1]));
  }
  li[0] = (int)bitsel(gt[0], (uint32_t)id, (uint32_t)li[0]);
  lk[0] = max(lk[0], key);
}

// Offers the lane's V candidates (ids id0 + v) to the list: all of them, or
// with `refill`, only those ordered after the lane's last pick (fk, fid).  Up
// to 16 candidates (four 16-byte loads) are loaded at once; longer rows go
// through a rolled loop that keeps the code small, with the load two 16-byte
// chunks ahead issued before the current chunk is inserted (the empty asm
// keeps the compiler from sinking it).  `row` must be readable for V values.
template <int KL>
__device__ __forceinline__ void list_fill(uint32_t (&lk)[KL], int (&li)[KL], const float* row, int V, bool vec4,
                                          int id0, bool live, bool refill, uint32_t fk, int fid) {
  auto offer = [&](uint32_t u, int v) {
    uint32_t key = live ? logit_key(__uint_as_float(u)) : 0u;
    const int id = id0 + v;
    if (refill) key = (key < fk || (key == fk && id > fid)) ? key : 0u;
    list_insert<KL>(lk, li, key, id);
  };
  if (vec4 && V <= 16) {  // up to four 16-byte loads: all issued before the first is used
    const u32x4* r4 = reinterpret_cast<const u32x4*>(row);
    const int n4 = V >> 2;
    u32x4 c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = r4[min(i, n4 - 1)];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < n4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) offer(c[i][j], 4 * i + j);
      }
  } else if (vec4) {
    const u32x4* r4 = reinterpret_cast<const u32x4*>(row);
    const int n4 = V >> 2;
    u32x4 c0 = r4[0];
    u32x4 c1 = r4[min(1, n4 - 1)];
#pragma unroll 1
    for (int c = 0; c < n4; ++c) {
      const u32x4 cur = c0;
      c0 = c1;
      c1 = r4[min(c + 2, n4 - 1)];
      __asm__ volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < 4; ++i) offer(cur[i], 4 * c + i);
    }
  } else {
    const uint32_t* r1 = reinterpret_cast<const uint32_t*>(row);
    uint32_t c0 = r1[0];
    uint32_t c1 = r1[min(1, V - 1)];
#pragma unroll 1
    for (int v = 0; v < V; ++v) {
      const uint32_t cur = c0;
      c0 = c1;
      c1 = r1[min(v + 2, V - 1)];
      __asm__ volatile("" ::: "memory");
      offer(cur, v);
    }
  }
}

// Routes token t with the P lanes of its lane group: returns its rank bitmask
// (same in the P lanes; 0 for t >= T), the expert ids of the lane's slots
// j = q * P + p in `sel` (-1: none) and their weights in `wt`; store_route
// writes the last two.
template <int P, int KS>
__device__ __forceinline__ uint64_t route_token(const RouterArgs& a, int t, int lane, int (&sel)[KS],
                                                float (&wt)[KS]) {
#pragma clang fp contract(off)
  constexpr int KL = kRouterList;
  const LayoutArgs& L = a.lay;
  const int p = lane & (P - 1);
  const int gbase = lane & ~(P - 1);
  const bool live = t < L.T;

  // 1-2. the lane's best KL candidates (rows t >= T read row T - 1 and offer nothing)
  const float* row = a.logits + (size_t)min(t, L.T - 1) * L.E + (size_t)p * a.V;
  const int id0 = p * a.V;
  uint32_t lk[KL];
  int li[KL];
#pragma unroll
  for (int i = 0; i < KL; ++i) {
    lk[i] = 0u;
    li[i] = 0;
  }
  list_fill<KL>(lk, li, row, a.V, a.vec4 != 0, id0, live, false, 0u, 0);
  bool exhausted = lk[0] == 0u;

  // 3. group-limited gating: P / G consecutive lanes form one group, so the
  //    group score is the largest list head among them; lanes of groups that
  //    are not kept empty their lists.
  if (a.G > 1) {
    const int lpg = P / a.G;
    const uint32_t m = group_max<P>(lk[0], lpg);
    const int g = p / lpg;
    int better = 0;
    for (int q = 0; q < a.G; ++q) {
      const uint32_t sq = (uint32_t)__shfl((int)m, gbase + q * lpg, kWave);
      better += (sq > m || (sq == m && q < g)) ? 1 : 0;
    }
    if (better >= a.KG) {
#pragma unroll
      for (int i = 0; i < KL; ++i) lk[i] = 0u;
      exhausted = true;
    }
  }

  // 4. k rounds over the P heads; slot j is kept by lane j % P.  Per round:
  //    the largest head key, then the lowest id among the heads with that key
  //    (two lane reductions); the owner pops its head (bitwise selects).
  uint32_t skey[KS];
#pragma unroll
  for (int q = 0; q < KS; ++q) {
    sel[q] = -1;
    skey[q] = 0u;
  }
  uint32_t key0 = 0u, fk = 0u;
  int fid = 0;
  for (int j = 0; j < L.k; ++j) {
    const uint32_t bk = lanes_max<P>(lk[0]);
    const uint32_t bn = lanes_max<P>(lk[0] == bk ? ~(uint32_t)li[0] : 0u);
    const int id = (int)~bn;
    if (j == 0) key0 = bk;
#pragma unroll
    for (int q = 0; q < KS; ++q) {  // no dynamic register indexing
      const bool mine_slot = j == q * P + p;
      sel[q] = mine_slot ? id : sel[q];
      skey[q] = mine_slot ? bk : skey[q];
    }
    uint32_t own = lk[0] == bk && li[0] == id ? ~0u : 0u;  // the owner pops its head
    __asm__("" : "+v"(own));
    fk = bitsel(own, bk, fk);
    fid = (int)bitsel(own, (uint32_t)id, (uint32_t)fid);
#pragma unroll
    for (int i = 0; i + 1 < KL; ++i) {
      lk[i] = bitsel(own, lk[i + 1], lk[i]);
      li[i] = (int)bitsel(own, (uint32_t)li[i + 1], (uint32_t)li[i]);
    }
    lk[KL - 1] = bitsel(own, 0u, lk[KL - 1]);
    if (j >= KL - 1 && j + 1 < L.k) {  // a lane can run dry only after KL pops
      const bool need = !exhausted && lk[0] == 0u;
      if (__ballot(need)) {  // rare: a lane gave all KL of its entries
        if (need) list_fill<KL>(lk, li, row, a.V, a.vec4 != 0, id0, live, true, fk, fid);
        exhausted = exhausted || (need && lk[0] == 0u);
      }
    }
  }

  // 5. weights, summed in a fixed order (per lane, then over the P lanes), and
  //    the rank bitmask
  float ev[KS];
  float sum = 0.0f;
  uint32_t rlo = 0u, rhi = 0u;
#pragma unroll
  for (int q = 0; q < KS; ++q) {
    const float lg = key_logit(skey[q]);
    float e = a.sigmoid ? 1.0f / (1.0f + expf(-lg)) : expf(lg - key_logit(key0));
    e = sel[q] >= 0 ? e : 0.0f;
    ev[q] = e;
    sum = sum + e;
    if (sel[q] >= 0) {
      const int r = rank_of(sel[q], L.rank_magic) & 63;  // (ids of rows t >= T are discarded)
      rlo |= r < 32 ? 1u << r : 0u;
      rhi |= r >= 32 ? 1u << (r - 32) : 0u;
    }
  }
  sum = lanes_sum<P>(sum);
  const uint64_t ranks = ((uint64_t)lanes_or<P>(rhi) << 32) | lanes_or<P>(rlo);

#pragma unroll
  for (int q = 0; q < KS; ++q) {
    wt[q] = ev[q] / sum;
    sel[q] = live ? sel[q] : -1;
  }
  return live ? ranks : 0;
}

// Writes the ids and weights route_token returned for token t (lane p of its
// P lanes holds slots q * P + p), through the L2: a dispatch in the same launch
// may read them.
template <int P, int KS>
__device__ __forceinline__ void store_route(const RouterArgs& a, int t, int p, const int (&sel)[KS],
                                            const float (&wt)[KS]) {
  const LayoutArgs& L = a.lay;
  if (t >= L.T) return;
#pragma unroll
  for (int q = 0; q < KS; ++q) {
    const int j = q * P + p;
    if (j < L.k) {
      put_coherent(&a.topk_idx[(size_t)t * L.k + j], sel[q]);
      put_coherent(&a.topk_w[(size_t)t * L.k + j], wt[q]);
    }
  }
}

// Writes token t's rank bitmask (lane p == 0 of its P lanes) and its
// is_token_in_rank row (spread over the P lanes).
template <int P, bool kBitmask = true>
__device__ __forceinline__ void write_token_layout(const LayoutArgs& L, int t, int p, uint64_t m) {
  if (t >= L.T) return;
  if (kBitmask && p == 0) L.token_ranks[t] = m;
  uint8_t* dst = L.mask + (size_t)t * L.R;
  if (L.mask_words) {
    uint32_t* d32 = reinterpret_cast<uint32_t*>(dst);
    for (int w = p; w < (L.R >> 2); w += P) {
      const uint32_t b = (uint32_t)(m >> (4 * w)) & 0xfu;
      d32[w] = (b & 1u) | ((b & 2u) << 7) | ((b & 4u) << 14) | ((b & 8u) << 21);
    }
  } else {
    for (int r = p; r < L.R; r += P) dst[r] = (uint8_t)((m >> r) & 1u);
  }
}

// T > kFusedMaxTokens (so T >= 1): block b routes chunk b (64 tokens, 64 / P
// per wave) and writes what layout_count_kernel writes for it (rank bitmasks,
// mask rows, the chunk's counts, rank and expert totals added to the
// accumulators); the block that finishes last turns the counts into receive
// rows.  Dynamic LDS: hist[E].
template <int P, int KS>
__global__ __launch_bounds__(kWave * P) void router_count_kernel(RouterArgs a) {
  extern __shared__ int hist[];  // [E]
  __shared__ int chunk_cnt[kWave];  // per-rank token counts of this chunk
  __shared__ int tile[kCountTile];
  __shared__ int offs[kWave];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const LayoutArgs& L = a.lay;
  for (int e = tid; e < L.E; e += kWave * P) hist[e] = 0;
  if (tid < kWave) chunk_cnt[tid] = 0;
  __syncthreads();

  const int tw = tid / P;  // token within the chunk
  const int t = blockIdx.x * kWave + tw;
  const int p = lane & (P - 1);
  int sel[KS];
  float wt[KS];
  const uint64_t m = route_token<P, KS>(a, t, lane, sel, wt);
#pragma unroll
  for (int q = 0; q < KS; ++q)
    if (sel[q] >= 0) atomicAdd(&hist[sel[q]], 1);
  if (p == 0) add_rank_bits(m, chunk_cnt);
  // every store after the counting: the compiler waits for outstanding stores
  // before reusing their registers, which would stall the counting on them
  write_token_layout<P>(L, t, p, m);
  store_route<P, KS>(a, t, p, sel, wt);
  __syncthreads();

  // what the last block reads: the chunk's counts and the totals
  if (tid < L.R) {
    const int c = chunk_cnt[tid];
    put_coherent(&L.chunk_base[tid * L.NC + blockIdx.x], c);
    if (c) atomicAdd(&L.rank_acc[tid], c);
  }
  for (int e = tid; e < L.E; e += kWave * P)
    if (hist[e]) atomicAdd(&L.expert_acc[e], hist[e]);

  if (!last_block_done(&L.sync->ticket, gridDim.x)) return;
  finalize_chunk_rows(L, tile, offs);
  if (tid == 0) clear_word(&L.sync->ticket);
}

// Plan of a batch of at most kFusedMaxTokens tokens from the token bitmasks
// handed over by the routing blocks, by one block of any number of waves:
// per-chunk rank counts (one ballot per rank over the chunk's 64 tokens), rank
// offsets and totals, the chunks' receive rows; tokens per expert from the
// accumulator, which is cleared for the next call.  offs: 65 ints of LDS.
__device__ __forceinline__ void finalize_small_plan(const LayoutArgs& a, int (*cnt)[kWave], int* offs) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int nthreads = blockDim.x, nwaves = nthreads >> 6;
  for (int c = wave; c < a.NC; c += nwaves) {
    const int t = c * kWave + lane;
    const uint64_t m_raw = get_coherent(&a.token_ranks[min(t, a.T - 1)]);
    const uint64_t m = t < a.T ? m_raw : 0ull;
    int mine = 0;
    for (int r = 0; r < a.R; ++r) {
      const int n = __popcll(__ballot((m >> r) & 1ull));
      mine = lane == r ? n : mine;
    }
    cnt[c][lane] = mine;
  }
  for (int e = tid; e < a.E; e += nthreads) {
    a.tokens_per_expert[e] = get_coherent(&a.expert_acc[e]);
    put_coherent(&a.expert_acc[e], 0);
  }
  __syncthreads();
  small_chunk_rows(a, cnt, offs);
}

// 1 <= T <= kFusedMaxTokens: block b of nblocks (kRouterSmallWaves waves)
// routes tokens [b * TPB, b * TPB + TPB), TPB = kRouterSmallWaves * 64 / P,
// writes ids, weights, bitmasks (handed to the last block) and mask rows, and
// adds its expert counts to the workspace accumulator; the block that finishes
// last computes the rest of the plan and returns true.  Every thread of the
// block must call it.  offs: 65 ints of LDS (offs[r] = segment offset of rank
// r, offs[64] = receive rows, valid in the block that returns true).  With
// kSignal, the last block raises the ready flag as soon as it has drawn its
// ticket (every routing block's hand-off has completed then), before computing
// the plan, for others in the same launch; the ticket and the flag are then left
// for whoever resets the sync words.
template <int P, int KS, bool kSignal = false>
__device__ __forceinline__ bool router_small_produce(const RouterArgs& a, int b, int nblocks,
                                                     int (*cnt)[kWave], int* offs) {
  constexpr int kThreads = kRouterSmallWaves * kWave;  // routing threads; further waves only join in
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const LayoutArgs& L = a.lay;
  if (tid < kThreads) {  // whole waves: the others skip the routing instead of running it on no token
    const int t = b * (kThreads / P) + tid / P;
    const int p = lane & (P - 1);
    int sel[KS];
    float wt[KS];
    const uint64_t m = route_token<P, KS>(a, t, lane, sel, wt);
    // the mask row first: its loop reuses registers, and the compiler waits
    // for outstanding stores before reusing theirs
    write_token_layout<P, false>(L, t, p, m);
    if (p == 0 && t < L.T) put_coherent(&L.token_ranks[t], m);
#pragma unroll
    for (int q = 0; q < KS; ++q)
      if (sel[q] >= 0) atomicAdd(&L.expert_acc[sel[q]], 1);
    store_route<P, KS>(a, t, p, sel, wt);
  }

  if (!last_block_done(&L.sync->ticket, nblocks)) return false;
  if (kSignal && tid == 0) put_coherent(&L.sync->ready, 1u);
  finalize_small_plan(L, cnt, offs);
  if (!kSignal && tid == 0) clear_word(&L.sync->ticket);
  return true;
}

template <int P, int KS>
__global__ __launch_bounds__(kRouterSmallWaves * kWave) void router_small_kernel(RouterArgs a) {
  __shared__ int cnt[kFusedMaxChunks][kWave];
  __shared__ int offs[kWave + 1];
  router_small_produce<P, KS>(a, blockIdx.x, gridDim.x, cnt, offs);
}

}  // namespace moe
