// Combine kernels: gather expert outputs back to their source tokens as a
// top-k weighted fp32 sum, rounded to bf16.
//
// Follows "DeepEP：年度总结中的计算通信重叠摘记" (notes.kuangjux.top), section
// 节点内通信 (combine returns what dispatch sent), and the mlqm.cn rocSHMEM
// notes, section 3.2 (the receive buffer is reused for the returning rows).
// Per token and channel: acc = +0; for j = 0..k-1 over valid slots,
// acc = fl32(acc + fl32(w_j * y[row(t, j)])); out = bf16_rne(acc).
// row(t, j) is send_row[t, rank(e_j)] for the rank layout, or
// e_j * cap + slot_pos[t, j] for the per-expert (low-latency) layout.  The
// same gather with weight 1 over the token's distinct rank rows (ranks
// ascending) is the dispatch backward: grad_x[t] = sum_r grad_recv[send_row[t, r]].
//
// A gather, not a scatter: each (token, 512-channel slice) is owned by one
// wave, so there are no float atomics and the summation order is fixed.  A
// persistent grid of waves loops over items.  Slot metadata comes from one
// round of vector loads (lane j = slot j, lane r = rank r) made wave-uniform
// with readlane.
#pragma once

#include "device_common.h"

namespace moe {

// Output rows are written once and not re-read here: nontemporal stores keep
// them from displacing expert-output lines in L2 (measured faster).
#ifndef MOE_COMBINE_NT_STORE
#define MOE_COMBINE_NT_STORE 1
#endif
// Expert-output rows are read once: nontemporal loads (measured faster).
#ifndef MOE_COMBINE_NT_LOAD
#define MOE_COMBINE_NT_LOAD 1
#endif

// One 16-byte piece of an expert-output row.
__device__ __forceinline__ u32x4 load_y(const u32x4* p) {
#if MOE_COMBINE_NT_LOAD
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

constexpr int kCombineBlock = 256;
constexpr int kSlotBatch = 8;

// How term j of token t finds its row of y and its weight.
enum RowMode : int {
  kRankSlots = 0,    // j = slot: row send_row[t, rank(e_j)], weight topk_w[t, j]
  kExpertSlots = 1,  // j = slot: row e_j * cap + slot_pos[t, j], weight topk_w[t, j]
  kRankRows = 2,     // j-th rank the token was sent to (ascending): row send_row[t, r_j], weight 1
};

struct CombineArgs {
  const uint16_t* y;
  const int32_t* topk_idx;
  const float* topk_w;
  const int32_t* send_row;  // rank layout: [T, R]
  const int32_t* slot_pos;  // per-expert layout: [T, k]
  uint16_t* out;
  uint64_t rank_magic;
  int T, H, H8, k, E, R;
  int cap;         // per-expert layout: rows per expert
  int num_y_rows;  // rows of y; slots whose row falls outside are skipped
  int terms;       // terms per token: k, or min(k, R) for kRankRows
  int slices;
  int items;
};

struct RawMeta {
  int id, rr;  // lane j: slot j's expert id; lane r (rank layout) or j (per-expert): row datum
  float w;
};

// Unconditional loads from clamped, always valid addresses (masked in resolve_row).
template <int kMode>
__device__ __forceinline__ RawMeta load_raw_meta(const CombineArgs& a, int item, int lane) {
  const int t = min(item, a.items - 1) / a.slices;
  RawMeta m;
  if constexpr (kMode == kRankRows) {
    m.id = 0;
    m.w = 1.0f;
    m.rr = a.send_row[(size_t)t * a.R + min(lane, a.R - 1)];
  } else {
    const int j = min(lane, a.k - 1);
    m.id = a.topk_idx[(size_t)t * a.k + j];
    m.w = a.topk_w[(size_t)t * a.k + j];
    if constexpr (kMode == kExpertSlots)
      m.rr = a.slot_pos[(size_t)t * a.k + j];
    else
      m.rr = a.send_row[(size_t)t * a.R + min(lane, a.R - 1)];
  }
  return m;
}

// Lane j: the y row of term j, or -1.
template <int kMode>
__device__ __forceinline__ int resolve_row(const CombineArgs& a, const RawMeta& m, int item, int lane) {
  if constexpr (kMode == kRankRows) {
    // The token's rows on the ranks it was sent to, moved into lanes 0..n-1 in
    // ascending rank order (so the sum order is unchanged); other lanes get -1.
    // A token reaches at most min(k, R) ranks, so terms = min(k, R) lanes
    // suffice however many ranks there are.
    const bool valid = item < a.items && lane < a.R && (unsigned)m.rr < (unsigned)a.num_y_rows;
    const uint64_t vm = __ballot(valid);
    const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(vm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)vm, 0));
    const int n = __popcll(vm);
    const int dst = valid ? below : n + (lane - below);  // a permutation of the 64 lanes
    return __builtin_amdgcn_ds_permute(dst << 2, valid ? m.rr : -1);
  }
  bool valid = item < a.items && lane < a.terms;
  int row;
  if constexpr (kMode == kExpertSlots) {
    valid = valid && (unsigned)m.id < (unsigned)a.E;
    row = valid && m.rr >= 0 && m.rr < a.cap ? m.id * a.cap + m.rr : -1;
  } else {
    valid = valid && (unsigned)m.id < (unsigned)a.E;
    row = __shfl(m.rr, valid ? rank_of(m.id, a.rank_magic) : 0, kWave);
  }
  return valid && (unsigned)row < (unsigned)a.num_y_rows ? row : -1;
}

__device__ __forceinline__ void store_out(u32x4* orow, int c, const float (&acc)[8]) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32_to_bf16_rne(acc[2 * i]) | (f32_to_bf16_rne(acc[2 * i + 1]) << 16);
#if MOE_COMBINE_NT_STORE
  __builtin_nontemporal_store(o, orow + c);
#else
  orow[c] = o;
#endif
}

__device__ __forceinline__ void accumulate(float (&acc)[8], float w, const u32x4& v) {
#pragma clang fp contract(off)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float p0 = w * bf16_lo(v[i]);
    const float p1 = w * bf16_hi(v[i]);
    acc[2 * i] = acc[2 * i] + p0;
    acc[2 * i + 1] = acc[2 * i + 1] + p1;
  }
}

// ---------------------------------------------------------------------------
// terms <= 8: two-deep software pipeline.  Vector loads retire in order against
// one counter, so per item i the loop issues, in this order: (1) the metadata
// of item i+2, (2) the payload of item i+1; then it waits only for item i's
// payload (accumulate, store) and for item i+2's metadata (resolve its rows),
// while item i+1's payload stays in flight.  For the wait counts to be exact
// on every path, every load is issued unconditionally from a clamped, always
// valid address and masked afterwards, and the two payload buffers alternate
// by unrolling instead of being copied.  Requires num_y_rows >= 1.
struct SlotRows {
  int row[kSlotBatch];
  float w[kSlotBatch];
};

template <int kMode>
__device__ __forceinline__ SlotRows resolve_rows(const CombineArgs& a, const RawMeta& m, int item, int lane) {
  const int row = resolve_row<kMode>(a, m, item, lane);
  SlotRows r;
#pragma unroll
  for (int j = 0; j < kSlotBatch; ++j) {
    r.row[j] = __builtin_amdgcn_readlane(row, j);
    r.w[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m.w), j));
  }
  return r;
}

__device__ __forceinline__ void load_payload(const CombineArgs& a, const SlotRows& r, int item, int lane,
                                             u32x4 (&v)[kSlotBatch]) {
  const int c = min((min(item, a.items - 1) % a.slices) * kWave + lane, a.H8 - 1);
#pragma unroll
  for (int j = 0; j < kSlotBatch; ++j) {
    const u32x4* yrow = reinterpret_cast<const u32x4*>(a.y + (size_t)max(r.row[j], 0) * a.H);
    v[j] = load_y(yrow + c);
  }
}

template <int kMode>
__device__ __forceinline__ void combine_stage(const CombineArgs& a, int item, int nw, int lane, SlotRows& cur,
                                              SlotRows& nxt, const u32x4 (&pc)[kSlotBatch],
                                              u32x4 (&pn)[kSlotBatch]) {
  const RawMeta m2 = load_raw_meta<kMode>(a, item + 2 * nw, lane);
  load_payload(a, nxt, item + nw, lane, pn);

  const int t = item / a.slices;
  const int c = (item - t * a.slices) * kWave + lane;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < kSlotBatch; ++j)
    if (cur.row[j] >= 0) accumulate(acc, cur.w[j], pc[j]);
  if (c < a.H8) store_out(reinterpret_cast<u32x4*>(a.out + (size_t)t * a.H), c, acc);
  cur = nxt;
  nxt = resolve_rows<kMode>(a, m2, item + 2 * nw, lane);
}

template <int kMode>
__global__ __launch_bounds__(kCombineBlock) void combine_pipelined_kernel(CombineArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = gridDim.x * (kCombineBlock / kWave);
  int item = blockIdx.x * (kCombineBlock / kWave) + wave;
  if (item >= a.items) return;

  const RawMeta m0 = load_raw_meta<kMode>(a, item, lane);
  const RawMeta m1 = load_raw_meta<kMode>(a, item + nw, lane);
  SlotRows cur = resolve_rows<kMode>(a, m0, item, lane);
  u32x4 buf_a[kSlotBatch], buf_b[kSlotBatch];
  load_payload(a, cur, item, lane, buf_a);
  SlotRows nxt = resolve_rows<kMode>(a, m1, item + nw, lane);
  for (;;) {
    combine_stage<kMode>(a, item, nw, lane, cur, nxt, buf_a, buf_b);
    item += nw;
    if (item >= a.items) break;
    combine_stage<kMode>(a, item, nw, lane, cur, nxt, buf_b, buf_a);
    item += nw;
    if (item >= a.items) break;
  }
}

// ---------------------------------------------------------------------------
// Any number of terms (up to 64): persistent loop, terms in batches of 8 (rows of a batch
// are loaded before any is accumulated); the next item's metadata is fetched
// behind the current payload.  Requires num_y_rows >= 1.
template <int kMode>
__global__ __launch_bounds__(kCombineBlock) void combine_persistent_kernel(CombineArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = gridDim.x * (kCombineBlock / kWave);
  int item = blockIdx.x * (kCombineBlock / kWave) + wave;
  if (item >= a.items) return;

  RawMeta m = load_raw_meta<kMode>(a, item, lane);
  for (; item < a.items; item += nw) {
    const int t = item / a.slices;
    const int c = (item - t * a.slices) * kWave + lane;
    const int cc = min(c, a.H8 - 1);
    const int slot_row = resolve_row<kMode>(a, m, item, lane);
    const float slot_w = m.w;
    m = load_raw_meta<kMode>(a, item + nw, lane);  // next item's metadata, in flight meanwhile

    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int j0 = 0; j0 < a.terms; j0 += kSlotBatch) {
      int row[kSlotBatch];
      float w[kSlotBatch];
      u32x4 v[kSlotBatch];
#pragma unroll
      for (int jj = 0; jj < kSlotBatch; ++jj) {  // lanes >= terms hold row -1
        row[jj] = __builtin_amdgcn_readlane(slot_row, j0 + jj);
        w[jj] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(slot_w), j0 + jj));
        v[jj] = load_y(reinterpret_cast<const u32x4*>(a.y + (size_t)max(row[jj], 0) * a.H) + cc);
      }
#pragma unroll
      for (int jj = 0; jj < kSlotBatch; ++jj)
        if (row[jj] >= 0) accumulate(acc, w[jj], v[jj]);
    }
    if (c < a.H8) store_out(reinterpret_cast<u32x4*>(a.out + (size_t)t * a.H), c, acc);
  }
}

}  // namespace moe
