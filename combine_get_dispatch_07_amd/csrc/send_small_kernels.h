// Layout and dispatch in one launch for small batches (T <= 1024): the rank
// layout ("DeepEP：年度总结中的计算通信重叠摘记", notes.kuangjux.top, section
// 节点内通信: a token goes only to the ranks that own one of its experts) and the
// packed dispatch into destination-contiguous receive segments (the mlqm.cn
// rocSHMEM notes, section 3.2), computed together so that a decode step needs
// one launch where the separate calls need two.
//
// Block T computes the layout exactly as layout_fused_kernel does (mask rows,
// token bitmasks, counts, the dispatch plan, rank offsets) and also publishes
// the dispatch's rank_offsets and num_recv.  Block t < T owns token t: its
// waves take the hidden slices (one each) and, in 64-token batches (one each),
// the rank bitmasks of all T tokens; per rank r a ballot over a batch counts the
// tokens going to r (the rank totals, from which every block derives the
// segment offsets itself) and those before t going to r (the token's row inside
// the segment).  Rows, metadata and bytes are those of moe_get_dispatch_layout
// followed by moe_dispatch.  All loads of a block are issued together, from
// clamped addresses, before anything waits on them.
#pragma once

#include "device_common.h"
#include "dispatch_kernels.h"
#include "layout_kernels.h"

namespace moe {

constexpr int kSendSmallMaxTokens = 1024;
constexpr int kSendSmallMaxWaves = 16;

struct SendSmallArgs {
  LayoutArgs lay;
  DispatchArgs d;
};

// U: 64-lane groups of 16-byte pieces per wave (1 or 2); KI: ids held per lane (k <= KI).
// Dynamic LDS: E ints (the expert histogram of the layout block).
template <int U, bool kFp8, int KI>
__global__ __launch_bounds__(kSendSmallMaxWaves * kWave) void send_small_kernel(SendSmallArgs args) {
#pragma clang fp contract(off)
  extern __shared__ int hist[];
  __shared__ int chunk_cnt[kFusedMaxChunks][kWave];
  __shared__ int wave_cnt[kFusedMaxChunks][kWave];
  __shared__ int rank_total[kWave + 1];  // layout block: offsets; token blocks: tokens per rank
  __shared__ int before[kWave];      // token blocks: tokens before t going to each rank
  __shared__ uint64_t mstage[kFusedMaxTokens];  // layout block: the tokens' rank bitmasks
  const LayoutArgs& L = args.lay;
  const DispatchArgs& a = args.d;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  if (blockIdx.x == a.T) {  // the layout, then the dispatch's segment offsets and row count
    layout_one_block<KI>(L, hist, chunk_cnt, wave_cnt, rank_total, mstage);
    if (wave == 0) {
      if (lane < a.R) a.rank_offsets[lane] = rank_total[lane];
      if (lane == 0) {
        a.rank_offsets[a.R] = rank_total[kWave];
        *a.num_recv = rank_total[kWave];
      }
    }
    return;
  }

  // Loads: the ids of this wave's 64-token batch (lane l: token 64 * wave + l),
  // the token's slot ids and weights (lane j: slot j) and this wave's x slice.
  const int t = blockIdx.x;
  const int u = wave * kWave + lane;
  const bool has_batch = wave * kWave < a.T;
  int ids[KI];
  {
    const int32_t* row = a.topk_idx + (size_t)min(u, a.T - 1) * a.k;
#pragma unroll
    for (int i = 0; i < KI; ++i) ids[i] = row[min(i, a.k - 1)];
  }
  const int jl = min(lane, a.k - 1);
  const int ej_raw = a.topk_idx[(size_t)t * a.k + jl];
  const float wj_raw = a.topk_w[(size_t)t * a.k + jl];
  const int c0 = wave * (U * kWave) + lane;
  const u32x4* xrow = reinterpret_cast<const u32x4*>(a.x + (size_t)t * a.H);
  u32x4 v[U];
#pragma unroll
  for (int uu = 0; uu < U; ++uu) v[uu] = __builtin_nontemporal_load(xrow + min(c0 + uu * kWave, a.H8 - 1));
  if (threadIdx.x < kWave) {
    rank_total[threadIdx.x] = 0;
    before[threadIdx.x] = 0;
  }

  // The token's slots and rank bitmask (wave-uniform).
  const int ej = lane < a.k ? ej_raw : -1;
  const float wj = lane < a.k ? wj_raw : 0.0f;
  const bool valid = (unsigned)ej < (unsigned)a.E;
  const int rj = valid ? rank_of(ej, a.rank_magic) : -1;
  uint64_t mine = 0;
  for (int j = 0; j < a.k; ++j) {
    const int r = __builtin_amdgcn_readlane(rj, j);
    if (r >= 0) mine |= 1ull << r;
  }
  __syncthreads();

  if (has_batch) {
    uint64_t m = 0;  // rank bitmask of token u
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int e = ids[i];
      if (i < a.k && (unsigned)e < (unsigned)a.E) m |= 1ull << rank_of(e, a.rank_magic);
    }
    if (u >= a.T) m = 0;
    const int d = t - wave * kWave;  // lanes l < d hold tokens before t
    const uint64_t below = d <= 0 ? 0ull : d >= kWave ? ~0ull : (1ull << d) - 1ull;
    int tot = 0, bef = 0;  // lane r: this batch's tokens going to r, and those before t
    for (int r = 0; r < a.R; ++r) {
      const uint64_t bal = __ballot((m >> r) & 1ull);
      tot = lane == r ? __popcll(bal) : tot;
      bef = lane == r ? __popcll(bal & below) : bef;
    }
    if (lane < a.R) {
      if (tot) atomicAdd(&rank_total[lane], tot);
      if (bef) atomicAdd(&before[lane], bef);
    }
  }

#pragma unroll
  for (int uu = 0; uu < U; ++uu)
    if (c0 + uu * kWave >= a.H8) v[uu] = u32x4{0u, 0u, 0u, 0u};
  u32x2 q[U];
  float sc[U];
  if constexpr (kFp8) quantize_slice<U>(v, q, sc);
  __syncthreads();

  // lane r < R: the segment offset of rank r (exclusive scan of the totals) plus
  // the tokens before t going to r = the token's row on rank r.
  const int total = lane < a.R ? rank_total[lane] : 0;
  const int incl = wave_inclusive_scan(total, lane);
  const int rank_row = lane < a.R ? incl - total + before[lane] : 0;

  const bool meta = wave == 0;
  int my_row = -1;  // lane r: receive row of (t, r)
  for (uint64_t todo = mine & a.rank_bits; todo; todo &= todo - 1) {
    const int r = __builtin_ctzll(todo);
    const int row = __builtin_amdgcn_readlane(rank_row, r);
    if ((unsigned)row >= (unsigned)a.capacity) continue;  // unreachable: capacity is checked on the host
    my_row = lane == r ? row : my_row;
    store_slice<U, kFp8>(a.recv_x, a.recv_scales, (size_t)row, a.H, a.H8, c0, lane, v, q, sc);
    if (meta) {
      if (lane == 0) a.recv_src_idx[row] = t;
      if (lane < a.k) {
        const int local = rj == r ? ej - r * a.L : -1;
        a.recv_topk_idx[(size_t)row * a.k + lane] = local;
        a.recv_topk_w[(size_t)row * a.k + lane] = local >= 0 ? wj : 0.0f;
      }
    }
  }
  if (meta && lane < a.R) a.send_row[(size_t)t * a.R + lane] = my_row;
}

}  // namespace moe
