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
// weights are wave-uniform (scalar loads); up to 8 slots' rows are loaded
// before any is accumulated, so 8 * U 16-byte loads per lane are in flight.
#pragma once

#include "device_common.h"

namespace moe {

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

  const int32_t* ids = a.topk_idx + (size_t)t * a.k;
  const float* ws = a.topk_w + (size_t)t * a.k;
  const int32_t* rows_of_rank = a.send_row + (size_t)t * a.R;

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
      const int j = j0 + jj;
      row[jj] = -1;
      w[jj] = 0.0f;
      if (j < a.k) {
        const int e = ids[j];
        if ((unsigned)e < (unsigned)a.E) {
          const int rr = rows_of_rank[rank_of(e, a.rank_magic)];
          if ((unsigned)rr < (unsigned)a.num_y_rows) {
            row[jj] = rr;
            w[jj] = ws[j];
          }
        }
      }
    }
    u32x4 v[kSlotBatch][U];
#pragma unroll
    for (int jj = 0; jj < kSlotBatch; ++jj) {
      if (row[jj] >= 0) {
        const u32x4* yrow = reinterpret_cast<const u32x4*>(a.y + (size_t)row[jj] * a.H);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + u * kWave;
          v[jj][u] = c < a.H8 ? __builtin_nontemporal_load(yrow + c) : u32x4{0u, 0u, 0u, 0u};
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

}  // namespace moe
