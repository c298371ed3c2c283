// Combine kernel: gathers expert outputs back to their source tokens as a
// top-k weighted fp32 sum, rounded to bf16.
//
// Follows "DeepEP：年度总结中的计算通信重叠摘记" (notes.kuangjux.top), section
// 节点内通信 (combine returns what dispatch sent), and the mlqm.cn rocSHMEM
// notes, section 3.2 (the receive buffer is reused for the returning rows).
// Per token and channel: acc = +0; for j = 0..k-1 over valid slots,
// acc = fl32(acc + fl32(w_j * y[send_row[t, rank(e_j)]])); out = bf16_rne(acc).
//
// A gather, not a scatter: each (token, hidden slice) is owned by one wave, so
// there are no float atomics and the summation order is fixed.  Slot rows and
// weights come from one round of vector loads (lane j = slot j, lane r =
// rank r) and are made wave-uniform with readlane; up to 8 slots' rows are loaded
// before any is accumulated, so 8 * U 16-byte loads per lane are in flight.
#pragma once

#include "device_common.h"

namespace moe {

#ifndef MOE_COMBINE_NT_LOADS
#define MOE_COMBINE_NT_LOADS 0
#endif
// Output rows are written once and not re-read here: nontemporal stores keep
// them from displacing expert-output lines in L2 (measured faster).
#ifndef MOE_COMBINE_NT_STORE
#define MOE_COMBINE_NT_STORE 1
#endif

constexpr int kCombineBlock = 256;
constexpr int kSlotBatch = 8;

struct CombineArgs {
  const uint16_t* y;
  const int32_t* topk_idx;
  const float* topk_w;
  const int32_t* send_row;
  uint16_t* out;
  uint64_t rank_magic;
  int T, H, H8, k, E, R;
  int num_y_rows;
  int slices;
  int items;
};

template <int U>
__global__ __launch_bounds__(kCombineBlock) void combine_kernel(CombineArgs a) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = blockIdx.x * (kCombineBlock / kWave) + wave;
  if (item >= a.items) return;
  const int t = item / a.slices;
  const int s = item - t * a.slices;
  const int c0 = s * (U * kWave) + lane;

  // One round of vector loads for the item's metadata: lane j < k holds slot j
  // (expert id, weight), lane r < R holds this token's receive row on rank r.
  const int slot_id = lane < a.k ? a.topk_idx[(size_t)t * a.k + lane] : -1;
  const float slot_w = lane < a.k ? a.topk_w[(size_t)t * a.k + lane] : 0.0f;
  const int rank_row = lane < a.R ? a.send_row[(size_t)t * a.R + lane] : -1;
  const bool valid = (unsigned)slot_id < (unsigned)a.E;
  const int slot_rank = valid ? rank_of(slot_id, a.rank_magic) : 0;
  int slot_row = __shfl(rank_row, slot_rank, kWave);
  slot_row = valid && (unsigned)slot_row < (unsigned)a.num_y_rows ? slot_row : -1;

  float acc[U][8];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[u][i] = 0.0f;

  for (int j0 = 0; j0 < a.k; j0 += kSlotBatch) {
    int row[kSlotBatch];
    float w[kSlotBatch];
#pragma unroll
    for (int jj = 0; jj < kSlotBatch; ++jj) {  // wave-uniform; lanes >= k hold row -1
      row[jj] = __builtin_amdgcn_readlane(slot_row, j0 + jj);
      w[jj] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(slot_w), j0 + jj));
    }
    u32x4 v[kSlotBatch][U];
#pragma unroll
    for (int jj = 0; jj < kSlotBatch; ++jj) {
      if (row[jj] >= 0) {
        const u32x4* yrow = reinterpret_cast<const u32x4*>(a.y + (size_t)row[jj] * a.H);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + u * kWave;
#if MOE_COMBINE_NT_LOADS
          v[jj][u] = c < a.H8 ? __builtin_nontemporal_load(yrow + c) : u32x4{0u, 0u, 0u, 0u};
#else
          v[jj][u] = c < a.H8 ? yrow[c] : u32x4{0u, 0u, 0u, 0u};
#endif
        }
      }
    }
#pragma unroll
    for (int jj = 0; jj < kSlotBatch; ++jj) {
      if (row[jj] >= 0) {
        const float wj = w[jj];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p0 = wj * bf16_lo(v[jj][u][i]);
            const float p1 = wj * bf16_hi(v[jj][u][i]);
            acc[u][2 * i] = acc[u][2 * i] + p0;
            acc[u][2 * i + 1] = acc[u][2 * i + 1] + p1;
          }
        }
      }
    }
  }

  u32x4* orow = reinterpret_cast<u32x4*>(a.out + (size_t)t * a.H);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = c0 + u * kWave;
    if (c < a.H8) {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = f32_to_bf16_rne(acc[u][2 * i]) | (f32_to_bf16_rne(acc[u][2 * i + 1]) << 16);
      orow[c] = o;
    }
  }
}

// Persistent variant: a fixed grid of waves loops over items (item += total
// waves).  The next item's metadata loads are issued right after the current
// item's payload loads, so they are in flight while the payload arrives and no
// wave starts cold.  Same arithmetic, same order, same results.
template <int U>
__global__ __launch_bounds__(kCombineBlock) void combine_persistent_kernel(CombineArgs a) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = gridDim.x * (kCombineBlock / kWave);
  int item = blockIdx.x * (kCombineBlock / kWave) + wave;
  if (item >= a.items) return;

  // raw metadata of the current item (lane j: slot j; lane r: rank r)
  int t = item / a.slices;
  int raw_id = lane < a.k ? a.topk_idx[(size_t)t * a.k + lane] : -1;
  float raw_w = lane < a.k ? a.topk_w[(size_t)t * a.k + lane] : 0.0f;
  int raw_rr = lane < a.R ? a.send_row[(size_t)t * a.R + lane] : -1;

  for (; item < a.items; item += nw) {
    t = item / a.slices;
    const int s = item - t * a.slices;
    const int c0 = s * (U * kWave) + lane;
    const bool valid = (unsigned)raw_id < (unsigned)a.E;
    const int slot_rank = valid ? rank_of(raw_id, a.rank_magic) : 0;
    int slot_row = __shfl(raw_rr, slot_rank, kWave);
    slot_row = valid && (unsigned)slot_row < (unsigned)a.num_y_rows ? slot_row : -1;
    const float slot_w = raw_w;

    float acc[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[u][i] = 0.0f;

    for (int j0 = 0; j0 < a.k; j0 += kSlotBatch) {
      int row[kSlotBatch];
      float w[kSlotBatch];
#pragma unroll
      for (int jj = 0; jj < kSlotBatch; ++jj) {
        row[jj] = __builtin_amdgcn_readlane(slot_row, j0 + jj);
        w[jj] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(slot_w), j0 + jj));
      }
      u32x4 v[kSlotBatch][U];
#pragma unroll
      for (int jj = 0; jj < kSlotBatch; ++jj) {
        if (row[jj] >= 0) {
          const u32x4* yrow = reinterpret_cast<const u32x4*>(a.y + (size_t)row[jj] * a.H);
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int c = c0 + u * kWave;
            v[jj][u] = c < a.H8 ? yrow[c] : u32x4{0u, 0u, 0u, 0u};
          }
        }
      }
      if (j0 == 0) {  // prefetch the next item's metadata behind this payload
        const int nitem = item + nw;
        if (nitem < a.items) {
          const int nt = nitem / a.slices;
          raw_id = lane < a.k ? a.topk_idx[(size_t)nt * a.k + lane] : -1;
          raw_w = lane < a.k ? a.topk_w[(size_t)nt * a.k + lane] : 0.0f;
          raw_rr = lane < a.R ? a.send_row[(size_t)nt * a.R + lane] : -1;
        }
      }
#pragma unroll
      for (int jj = 0; jj < kSlotBatch; ++jj) {
        if (row[jj] >= 0) {
          const float wj = w[jj];
#pragma unroll
          for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float p0 = wj * bf16_lo(v[jj][u][i]);
              const float p1 = wj * bf16_hi(v[jj][u][i]);
              acc[u][2 * i] = acc[u][2 * i] + p0;
              acc[u][2 * i + 1] = acc[u][2 * i + 1] + p1;
            }
          }
        }
      }
    }

    u32x4* orow = reinterpret_cast<u32x4*>(a.out + (size_t)t * a.H);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave;
      if (c < a.H8) {
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[i] = f32_to_bf16_rne(acc[u][2 * i]) | (f32_to_bf16_rne(acc[u][2 * i + 1]) << 16);
        orow[c] = o;
      }
    }
  }
}

// Two-deep software pipeline for k <= 8 (one slot batch) and num_y_rows >= 1.
// Vector loads retire in order against one counter, so per item i the loop
// issues, in this order: (1) the metadata of item i+2, (2) the payload of item
// i+1; then it waits only for item i's payload (accumulate, store) and for item
// i+2's metadata (resolve its rows), while item i+1's payload stays in flight.
// For the wait counts to be exact on every path, every load is issued
// unconditionally from a clamped, always valid address and masked afterwards,
// and the two payload buffers alternate by unrolling instead of being copied.
struct SlotRows {
  int row[kSlotBatch];
  float w[kSlotBatch];
};

struct RawMeta {
  int id, rr;
  float w;
};

__device__ __forceinline__ RawMeta load_raw_meta(const CombineArgs& a, int item, int lane) {
  const int t = min(item, a.items - 1) / a.slices;
  RawMeta m;
  m.id = a.topk_idx[(size_t)t * a.k + min(lane, a.k - 1)];
  m.w = a.topk_w[(size_t)t * a.k + min(lane, a.k - 1)];
  m.rr = a.send_row[(size_t)t * a.R + min(lane, a.R - 1)];
  return m;
}

__device__ __forceinline__ SlotRows resolve_rows(const CombineArgs& a, const RawMeta& m, int item, int lane) {
  const bool valid = item < a.items && lane < a.k && (unsigned)m.id < (unsigned)a.E;
  const int rank = valid ? rank_of(m.id, a.rank_magic) : 0;
  int row = __shfl(m.rr, rank, kWave);
  row = valid && (unsigned)row < (unsigned)a.num_y_rows ? row : -1;
  SlotRows r;
#pragma unroll
  for (int j = 0; j < kSlotBatch; ++j) {
    r.row[j] = __builtin_amdgcn_readlane(row, j);
    r.w[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m.w), j));
  }
  return r;
}

template <int U>
__device__ __forceinline__ void load_payload(const CombineArgs& a, const SlotRows& r, int item, int lane,
                                             u32x4 (&v)[kSlotBatch][U]) {
  const int c0 = (min(item, a.items - 1) % a.slices) * (U * kWave) + lane;
#pragma unroll
  for (int j = 0; j < kSlotBatch; ++j) {
    const u32x4* yrow = reinterpret_cast<const u32x4*>(a.y + (size_t)max(r.row[j], 0) * a.H);
#pragma unroll
    for (int u = 0; u < U; ++u) v[j][u] = yrow[min(c0 + u * kWave, a.H8 - 1)];
  }
}

// One pipeline stage: see the comment above.  `pc` holds item's payload,
// `pn` receives item + nw's; on return cur/nxt have advanced by one item.
template <int U>
__device__ __forceinline__ void combine_stage(const CombineArgs& a, int item, int nw, int lane, SlotRows& cur,
                                              SlotRows& nxt, const u32x4 (&pc)[kSlotBatch][U],
                                              u32x4 (&pn)[kSlotBatch][U]) {
#pragma clang fp contract(off)
  const RawMeta m2 = load_raw_meta(a, item + 2 * nw, lane);
  load_payload<U>(a, nxt, item + nw, lane, pn);

  const int t = item / a.slices;
  const int c0 = (item - t * a.slices) * (U * kWave) + lane;
  float acc[U][8];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[u][i] = 0.0f;
#pragma unroll
  for (int j = 0; j < kSlotBatch; ++j) {
    if (cur.row[j] >= 0) {
      const float wj = cur.w[j];
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p0 = wj * bf16_lo(pc[j][u][i]);
          const float p1 = wj * bf16_hi(pc[j][u][i]);
          acc[u][2 * i] = acc[u][2 * i] + p0;
          acc[u][2 * i + 1] = acc[u][2 * i + 1] + p1;
        }
      }
    }
  }
  u32x4* orow = reinterpret_cast<u32x4*>(a.out + (size_t)t * a.H);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = c0 + u * kWave;
    if (c < a.H8) {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = f32_to_bf16_rne(acc[u][2 * i]) | (f32_to_bf16_rne(acc[u][2 * i + 1]) << 16);
#if MOE_COMBINE_NT_STORE
      __builtin_nontemporal_store(o, orow + c);
#else
      orow[c] = o;
#endif
    }
  }
  cur = nxt;
  nxt = resolve_rows(a, m2, item + 2 * nw, lane);
}

template <int U>
__global__ __launch_bounds__(kCombineBlock) void combine_pipelined_kernel(CombineArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = gridDim.x * (kCombineBlock / kWave);
  int item = blockIdx.x * (kCombineBlock / kWave) + wave;
  if (item >= a.items) return;

  const RawMeta m0 = load_raw_meta(a, item, lane);
  const RawMeta m1 = load_raw_meta(a, item + nw, lane);
  SlotRows cur = resolve_rows(a, m0, item, lane);
  u32x4 buf_a[kSlotBatch][U], buf_b[kSlotBatch][U];
  load_payload<U>(a, cur, item, lane, buf_a);
  SlotRows nxt = resolve_rows(a, m1, item + nw, lane);
  for (;;) {
    combine_stage<U>(a, item, nw, lane, cur, nxt, buf_a, buf_b);
    item += nw;
    if (item >= a.items) break;
    combine_stage<U>(a, item, nw, lane, cur, nxt, buf_b, buf_a);
    item += nw;
    if (item >= a.items) break;
  }
}

}  // namespace moe
