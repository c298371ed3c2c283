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

}  // namespace moe
