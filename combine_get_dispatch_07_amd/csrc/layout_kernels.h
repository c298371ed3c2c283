// Dispatch layout kernels: top-k expert ids -> is_token_in_rank, per-rank and
// per-expert token counts, and the dispatch plan: each token's rank bitmask
// and, per rank and 64-token chunk, the receive row of the chunk's first token
// going to that rank (segment offset plus the tokens of earlier chunks).
//
// Follows the is_token_in_rank filter of "DeepEP：年度总结中的计算通信重叠摘记"
// (notes.kuangjux.top), section 节点内通信: a token is marked only for the
// ranks that own one of its top-k experts.
//
// One lane per token, one wave per 64-token chunk.  Per-rank chunk counts come
// from LDS atomics on the set rank bits, expert counts from an LDS histogram;
// all counting is integer, so results do not depend on scheduling.  Up to 1024
// tokens one block does everything.  Above, count blocks run in parallel and
// add their rank and expert totals to accumulators in the workspace; the block
// that finishes last ("last block done": every block takes a ticket from a
// counter in the workspace) turns the chunk counts into receive rows and
// resets the counter and the accumulators.  No block ever waits for another.
#pragma once

#include "device_common.h"

namespace moe {

#ifndef MOE_LAYOUT_BLOCK
#define MOE_LAYOUT_BLOCK 256
#endif
constexpr int kLayoutBlock = MOE_LAYOUT_BLOCK;  // tokens per block, multi-block path
constexpr int kFusedMaxTokens = 1024;  // up to this many tokens one block does everything
constexpr int kFusedMaxChunks = kFusedMaxTokens / kWave;
constexpr int kCountTile = 8192;  // chunk counts staged in LDS per pass of the finalisation

// Words at the start of the workspace that coordinate the blocks of one launch.
// They are zero between calls: the caller zero-fills a new workspace once, and
// every launch that uses them leaves them zero again.  Each word has a 4 KiB
// line of its own: many blocks hit them at once (role and exit tickets, polls
// of the ready flag), and one shared line would serialise all of them.
constexpr int kSyncStride = 4096 / sizeof(uint32_t);
struct SyncWords {
  uint32_t ticket;  // count (or routing) blocks finished: last-block-done
  uint32_t pad0[kSyncStride - 1];
  uint32_t role;    // role tickets taken (routing and dispatch in one launch)
  uint32_t pad1[kSyncStride - 1];
  uint32_t exits;   // blocks of that launch that are done with the sync words
  uint32_t pad2[kSyncStride - 1];
  uint32_t ready;   // 1 once every routing block of that launch has handed over its tokens
  uint32_t pad3[kSyncStride - 1];
};
constexpr int kSyncBytes = sizeof(SyncWords);

struct LayoutArgs {
  SyncWords* sync;
  int32_t* expert_acc;      // [E] expert counts summed across blocks (zero between calls)
  int32_t* rank_acc;        // [R] tokens per rank summed across blocks (zero between calls)
  const int32_t* topk_idx;
  int32_t* tokens_per_rank;
  int32_t* tokens_per_expert;
  uint8_t* mask;            // [T, R] bytes
  uint64_t* token_ranks;    // plan: [T] rank bitmask
  int32_t* chunk_base;      // plan: [R, NC] receive row of the chunk's first token on rank r
                            // (per-chunk counts while the count blocks run)
  int32_t* ws_rank_offsets; // plan: [R + 1]
  int32_t* out_rank_offsets;// [R + 1] and [1]: the dispatch's rank_offsets and num_recv, when the
  int32_t* out_num_recv;    // layout runs in the same launch as the dispatch (else null)
  uint64_t rank_magic;
  int T, k, E, R, NC, NB;
  int mask_words;           // 1: mask rows written as 32-bit words (R % 4 == 0, aligned)
  int mask_shift;           // log2(R) when R is a power of two >= 4 and the rows start 16-byte
                            // aligned: whole waves write their rows as 16-byte pieces; else -1
  int ids_vec4;             // 1: id rows read as 16-byte vectors (k % 4 == 0, 16-byte aligned)
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

// The is_token_in_rank rows of the 64 tokens [t0, t0 + 64) of one wave (those
// below T), R = 2^mask_shift bytes each, as 16-byte pieces: lane l writes
// pieces l, l + 64, ... of the wave's 64 R contiguous bytes, so each store
// instruction covers 1 KiB, where one lane per token writing its own row
// would touch a cache line per lane and instruction.  mw: the 64 tokens' rank
// bitmasks in LDS, written by this wave before the call.
__device__ __forceinline__ void write_wave_mask_rows(const LayoutArgs& a, int t0, int lane, const uint64_t* mw) {
  const int sh = a.mask_shift;
  const int nbytes = min(kWave, a.T - t0) << sh;  // a multiple of R >= 4
  uint8_t* base = a.mask + ((size_t)t0 << sh);
  for (int q = lane; (q << 4) < nbytes; q += kWave) {
    const int b0 = q << 4;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int b = b0 + 4 * k;
      const uint32_t nib = (uint32_t)(mw[b >> sh] >> (b & ((1 << sh) - 1))) & 0xfu;
      w[k] = (nib & 1u) | ((nib & 2u) << 7) | ((nib & 4u) << 14) | ((nib & 8u) << 21);
    }
    if (b0 + 16 <= nbytes) {
      *reinterpret_cast<u32x4*>(base + b0) = u32x4{w[0], w[1], w[2], w[3]};
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (b0 + 4 * k < nbytes) *reinterpret_cast<uint32_t*>(base + b0 + 4 * k) = w[k];
    }
  }
}

// Token t's outputs: its rank bitmask (plan) and its is_token_in_rank row,
// either by its own lane or, with mask_shift >= 0, staged in mw (the wave's 64
// masks in LDS) and written by the whole wave.  Every lane of the wave calls it.
__device__ __forceinline__ void write_token_outputs(const LayoutArgs& a, int t, int lane, uint64_t m, uint64_t* mw) {
  if (t < a.T) a.token_ranks[t] = m;
  if (a.mask_shift >= 0) {
    mw[lane] = m;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int t0 = t - lane;
    if (t0 < a.T) write_wave_mask_rows(a, t0, lane, mw);
  } else if (t < a.T) {
    write_mask_row(a, t, m);
  }
}

// Adds each lane's rank bits m to the per-rank counters cnt[0..63] (LDS)
// with one atomic add per set bit: at most min(k, R) adds per lane, fewer
// steps than one ballot per rank when R is large.  Integer adds: the result
// does not depend on their order.
__device__ __forceinline__ void add_rank_bits(uint64_t m, int* cnt) {
  for (uint64_t b = m; b; b &= b - 1) atomicAdd(&cnt[__builtin_ctzll(b)], 1);
}

// Lane r (< R) returns how many lanes of the wave have bit r set in m; `cnt`
// is 64 ints of LDS private to the wave.  Up to kBallotRanks ranks: one ballot
// per rank (scalar work, no LDS); above, one LDS atomic per set bit, where the
// set bits of all lanes hit the same few counters far less often.
#ifndef MOE_BALLOT_RANKS
#define MOE_BALLOT_RANKS 16
#endif
constexpr int kBallotRanks = MOE_BALLOT_RANKS;
__device__ __forceinline__ int wave_rank_counts(uint64_t m, int R, int lane, int* cnt) {
  if (R <= kBallotRanks) {
    int mine = 0;
    for (int r = 0; r < R; ++r) {
      const int c = __popcll(__ballot((m >> r) & 1ull));
      mine = lane == r ? c : mine;
    }
    return mine;
  }
  cnt[lane] = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  add_rank_bits(m, cnt);
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  return lane < R ? cnt[lane] : 0;
}

// Wave 0: per-rank totals (lane r: total of rank r) -> tokens_per_rank and the
// exclusive rank offsets; returns lane r's offset.
__device__ __forceinline__ int publish_rank_offsets(const LayoutArgs& a, int v, int lane) {
  v = lane < a.R ? v : 0;
  const int incl = wave_inclusive_scan(v, lane);
  if (lane < a.R) {
    a.tokens_per_rank[lane] = v;
    a.ws_rank_offsets[lane] = incl - v;
  }
  if (lane == a.R - 1) a.ws_rank_offsets[a.R] = incl;
  if (a.out_rank_offsets != nullptr) {
    if (lane < a.R) a.out_rank_offsets[lane] = incl - v;
    if (lane == a.R - 1) {
      a.out_rank_offsets[a.R] = incl;
      *a.out_num_recv = incl;
    }
  }
  return incl - v;
}

// Receive rows of the chunks of a batch of at most kFusedMaxTokens tokens, by
// one block: cnt[c][r] holds the chunk counts (LDS); lanes r < R of wave 0
// compute the rank totals, the offsets (published; offs[r], and offs[64] = the
// number of receive rows) and the row of each chunk's first token.  offs: 65
// ints of LDS.  Every thread of the block must call it.
__device__ __forceinline__ void small_chunk_rows(const LayoutArgs& a, const int (*cnt)[kWave], int* offs) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  if (tid < kWave) {
    int total = 0;
    for (int c = 0; c < a.NC; ++c) total += cnt[c][lane];
    const int off = publish_rank_offsets(a, total, lane);
    offs[lane] = off;
    if (lane == a.R - 1) offs[kWave] = off + total;
  }
  __syncthreads();
  if (tid < a.R) {  // at most 16 chunks: a serial scan per rank is shortest
    int run = offs[tid];
    for (int c = 0; c < a.NC; ++c) {
      put_coherent(&a.chunk_base[tid * a.NC + c], run);
      run += cnt[c][tid];
    }
  }
}

// The whole layout in one block of at least ceil(T/64) waves (at most 16):
// thread i owns token i, wave w chunk w; waves beyond the last chunk count
// nothing.  hist: E ints of LDS; mstage: 64 u64 of LDS per wave.  Returns (in
// every thread) once the plan is written; offs[r] then holds the segment
// offset of rank r and offs[64] the number of receive rows.
template <int KI>
__device__ __forceinline__ void layout_one_block(const LayoutArgs& a, int* hist, int (*cnt)[kWave],
                                                 int (*wave_cnt)[kWave], int* offs, uint64_t* mstage) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  for (int e = tid; e < a.E; e += blockDim.x) hist[e] = 0;
  __syncthreads();

  const uint64_t m = token_rank_mask<KI>(a, tid, hist);
  cnt[wave][lane] = wave_rank_counts(m, a.R, lane, wave_cnt[wave]);
  write_token_outputs(a, tid, lane, m, mstage + wave * kWave);
  __syncthreads();

  for (int e = tid; e < a.E; e += blockDim.x) a.tokens_per_expert[e] = hist[e];
  small_chunk_rows(a, cnt, offs);
  __syncthreads();
}

// T <= kFusedMaxTokens: one block of ceil(T/64) waves (at least one) does
// everything in one launch.  Dynamic LDS: hist[E].
template <int KI>
__global__ __launch_bounds__(kFusedMaxTokens) void layout_fused_kernel(LayoutArgs a) {
  extern __shared__ int hist[];
  __shared__ int cnt[kFusedMaxChunks][kWave];
  __shared__ int wave_cnt[kFusedMaxChunks][kWave];
  __shared__ int offs[kWave + 1];
  __shared__ uint64_t mstage[kFusedMaxTokens];
  layout_one_block<KI>(a, hist, cnt, wave_cnt, offs, mstage);
}

// Last-block-done.  Every wave of the block, having written with put_coherent
// (or agent-scope atomics) everything the last block will read, waits for those
// writes to complete; then one thread takes a ticket.  Returns true, in every
// thread, in the block that drew the last of `blocks` tickets: every other
// block's hand-off writes completed before its ticket was taken, so that block
// reads them with get_coherent.  No thread waits for another block.
__device__ __forceinline__ bool last_block_done(uint32_t* ticket, uint32_t blocks) {
  __shared__ uint32_t drawn;
  wait_own_stores();
  __syncthreads();
  if (threadIdx.x == 0) drawn = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  return drawn == blocks - 1;
}

// Resets a sync word for the next launch (all tickets of this one are taken).
__device__ __forceinline__ void clear_word(uint32_t* w) { put_coherent(w, 0u); }

// kBatch chunk counts of a tile (rank-major: element i = rank i / nc, chunk
// c0 + i % nc) for element i0 + u * stride, u < kBatch, from clamped addresses,
// all issued before any is used.
template <int kBatch>
__device__ __forceinline__ void load_count_batch(const LayoutArgs& a, int (&v)[kBatch], int i0, int stride, int n,
                                                 int nc, int c0) {
  if (nc == a.NC) {  // the tile holds every chunk: element i is chunk_base[i] (no division)
#pragma unroll
    for (int u = 0; u < kBatch; ++u) v[u] = get_coherent(&a.chunk_base[min(i0 + u * stride, n - 1)]);
    return;
  }
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    const int i = min(i0 + u * stride, n - 1);
    v[u] = get_coherent(&a.chunk_base[(i / nc) * a.NC + c0 + i % nc]);
  }
}

// Plan finalisation of the multi-block paths, by the block that finished last
// (any number of waves): rank offsets from the rank accumulator, expert totals
// from the expert accumulator (both cleared for the next call), then the chunk
// counts, kCountTile at a time, staged in LDS (tile), scanned per rank (one
// wave per rank) and written back as receive rows.  The rank totals, the first
// expert totals and the first tile's chunk counts (at most two batches of
// loads per thread) are loaded together, so shapes whose counts fit one tile
// take one round of loads.  offs: 64 ints of LDS.  Every thread of the block
// must call it.
__device__ __forceinline__ void finalize_chunk_rows(const LayoutArgs& a, int* tile, int* offs) {
  constexpr int kBatch = 16;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int nthreads = blockDim.x, nwaves = nthreads >> 6;
  const int TC = kCountTile / a.R;  // chunks of every rank per tile (R <= 64: at least 128)

  // the first tile: up to two batches of loads per thread, all issued before any is used
  const int nc0 = min(TC, a.NC), n0 = a.R * nc0;
  const int rv = get_coherent(&a.rank_acc[min(lane, a.R - 1)]);
  const int ev = get_coherent(&a.expert_acc[min(tid, a.E - 1)]);
  int v[kBatch], w[kBatch];
  load_count_batch<kBatch>(a, v, tid, nthreads, n0, nc0, 0);
  const bool two = n0 > kBatch * nthreads;  // block-uniform
  if (two) load_count_batch<kBatch>(a, w, tid + kBatch * nthreads, nthreads, n0, nc0, 0);

  if (wave == 0) {
    offs[lane] = publish_rank_offsets(a, rv, lane);
    if (lane < a.R) put_coherent(&a.rank_acc[lane], 0);
  }
  for (int e = tid; e < a.E; e += nthreads) {
    a.tokens_per_expert[e] = e == tid ? ev : get_coherent(&a.expert_acc[e]);
    put_coherent(&a.expert_acc[e], 0);
  }
  for (int c0 = 0; c0 < a.NC; c0 += TC) {
    const int nc = min(TC, a.NC - c0), n = a.R * nc;
    for (int i0 = tid; i0 < n; i0 += kBatch * nthreads) {
      const bool first = c0 == 0 && i0 == tid, second = c0 == 0 && i0 == tid + kBatch * nthreads;
      if (!first && !second) load_count_batch<kBatch>(a, v, i0, nthreads, n, nc, c0);
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (i0 + u * nthreads < n) tile[i0 + u * nthreads] = second ? w[u] : v[u];
    }
    __syncthreads();
    if (nc <= kWave) {  // one chunk per lane: one wave scan per rank
      for (int r = wave; r < a.R; r += nwaves) {
        const int c = lane < nc ? tile[r * nc + lane] : 0;
        const int incl = wave_inclusive_scan(c, lane);
        if (lane < nc) put_coherent(&a.chunk_base[r * a.NC + c0 + lane], offs[r] + incl - c);
        if (lane == kWave - 1) offs[r] += incl;
      }
    } else {  // 64 chunks at a time, the carry between them through a readlane (contiguous stores)
      for (int r = wave; r < a.R; r += nwaves) {
        int run = offs[r];
        for (int j0 = 0; j0 < nc; j0 += kWave) {
          const int j = j0 + lane;
          const int c = j < nc ? tile[r * nc + j] : 0;
          const int incl = wave_inclusive_scan(c, lane);
          if (j < nc) put_coherent(&a.chunk_base[r * a.NC + c0 + j], run + incl - c);
          run += __builtin_amdgcn_readlane(incl, kWave - 1);
        }
        if (lane == 0) offs[r] = run;
      }
    }
    __syncthreads();
  }
}

// Multi-block path (T > kFusedMaxTokens): count block b of nblocks counts
// tokens [256 b, 256 b + 256) -- mask rows, token bitmasks, the counts of its
// four chunks, rank and expert totals added to the accumulators -- and the
// block that finishes last turns the counts into receive rows and returns true.
// Every thread of the block must call it.  hist: E ints of LDS; tile:
// kCountTile ints; offs: 64 ints; mstage: kLayoutBlock u64.
template <int KI>
__device__ __forceinline__ bool layout_count_produce(const LayoutArgs& a, int b, int nblocks, int* hist,
                                                     int (*wave_cnt)[kWave], int* tile, int* offs,
                                                     uint64_t* mstage) {
  constexpr int kChunks = kLayoutBlock / kWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  for (int e = tid; e < a.E; e += kLayoutBlock) hist[e] = 0;
  __syncthreads();

  const int t = b * kLayoutBlock + tid;
  const uint64_t m = token_rank_mask<KI>(a, t, hist);
  const int cnt = wave_rank_counts(m, a.R, lane, wave_cnt[wave]);
  const int chunk = b * kChunks + wave;
  if (chunk < a.NC && lane < a.R) {
    put_coherent(&a.chunk_base[lane * a.NC + chunk], cnt);
    if (cnt) atomicAdd(&a.rank_acc[lane], cnt);
  }
  __syncthreads();
  for (int e = tid; e < a.E; e += kLayoutBlock)
    if (hist[e]) atomicAdd(&a.expert_acc[e], hist[e]);
  // The plain output stores come last: the compiler waits for outstanding
  // stores before reusing their registers, and here that wait is the one the
  // ticket needs anyway rather than a round trip of its own mid-block.
  write_token_outputs(a, t, lane, m, mstage + wave * kWave);

  if (!last_block_done(&a.sync->ticket, nblocks)) return false;
  finalize_chunk_rows(a, tile, offs);
  if (tid == 0) clear_word(&a.sync->ticket);
  return true;
}

// One launch of the multi-block layout.  Dynamic LDS: hist[E].
template <int KI>
__global__ __launch_bounds__(kLayoutBlock) void layout_count_kernel(LayoutArgs a) {
  extern __shared__ int hist[];  // [E]
  __shared__ int wave_cnt[kLayoutBlock / kWave][kWave];
  __shared__ int tile[kCountTile];
  __shared__ int offs[kWave];
  __shared__ uint64_t mstage[kLayoutBlock];
  layout_count_produce<KI>(a, blockIdx.x, gridDim.x, hist, wave_cnt, tile, offs, mstage);
}

}  // namespace moe
