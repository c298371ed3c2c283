// Backward of combine and dispatch (training).
//
// The DeepEP pages describe a library for training as well as inference and
// note that its backward pass needs its own integration
// ("DeepEP：面向MoE的高吞吐低延迟GPU通信库", ssnai.com).  Each backward is the
// adjoint of its forward step:
//   combine backward:  grad_y[send_row[t, r]] = sum over slots j of t on rank
//                      r, ascending, of fl32(w_tj * g[t]) (fp32, then bf16 RNE);
//                      grad_w[t, j] = <g[t], y[row(t, j)]> (fp32 dot product);
//   dispatch backward: grad_x[t] = sum over ranks r, ascending, of
//                      grad_recv[send_row[t, r]] (the rank-rows gather in
//                      combine_kernels.h); grad_topk_w[t, j] =
//                      grad_recv_w[row(t, j), j] (below).
#pragma once

#include "combine_kernels.h"
#include "device_common.h"

namespace moe {

constexpr int kBwdMaxWaves = 16;  // upper bound of waves per block (one block per token)
constexpr int kMaxTopk = 32;

struct CombineBwdArgs {
  const uint16_t* g;  // [T, H] gradient of the combine output
  const uint16_t* y;  // [num_y_rows, H] combine input (expert outputs)
  const int32_t* topk_idx;
  const float* topk_w;
  const int32_t* send_row;
  uint16_t* grad_y;  // [num_y_rows, H]
  float* grad_w;     // [T, k]
  uint64_t rank_magic;
  int T, H, H8, k, E, R, num_y_rows;
};

template <int KB>  // slots handled in registers: 8 or 32 (k <= KB)
__global__ __launch_bounds__(kBwdMaxWaves * kWave) void combine_backward_kernel(CombineBwdArgs a) {
#pragma clang fp contract(off)
  __shared__ float partial[kBwdMaxWaves][KB];
  const int nwaves = blockDim.x / kWave;  // wave w takes slices w, w + nwaves, ...
  const int t = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // lane j < k: slot j's weight, rank and y row; lane r < R: this token's row on rank r
  const int j = min(lane, a.k - 1);
  const int id = a.topk_idx[(size_t)t * a.k + j];
  const float w = a.topk_w[(size_t)t * a.k + j];
  const int rank_row = a.send_row[(size_t)t * a.R + min(lane, a.R - 1)];
  bool valid = lane < a.k && (unsigned)id < (unsigned)a.E;
  const int rank = valid ? rank_of(id, a.rank_magic) : 0;
  const int row = __shfl(rank_row, rank, kWave);
  valid = valid && (unsigned)row < (unsigned)a.num_y_rows;

  int srank[KB], srow[KB];
  float sw[KB];
  uint64_t ranks = 0;
#pragma unroll
  for (int jj = 0; jj < KB; ++jj) {  // wave-uniform copies of the slot metadata
    const bool v = __builtin_amdgcn_readlane((int)valid, jj) != 0;
    srank[jj] = v ? __builtin_amdgcn_readlane(rank, jj) : -1;
    srow[jj] = v ? __builtin_amdgcn_readlane(row, jj) : -1;
    sw[jj] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), jj));
    if (v) ranks |= 1ull << srank[jj];
  }

  float dot[KB];
#pragma unroll
  for (int jj = 0; jj < KB; ++jj) dot[jj] = 0.0f;

  const int slices = (a.H8 + kWave - 1) / kWave;
  const u32x4* grow = reinterpret_cast<const u32x4*>(a.g + (size_t)t * a.H);
  // k <= 8: software pipeline over this wave's slices -- the next slice's g and
  // y loads are issued before the current slice's grad_y rows are stored.
  // k > 8: slots in batches of 8 per slice, without prefetch.
  constexpr bool kPrefetch = KB <= 8;
  u32x4 gv, yv[kPrefetch ? KB : 1];
  auto load_slice = [&](int s_) {
    const int cc = min(s_ * kWave + lane, a.H8 - 1);
    gv = grow[cc];
    if constexpr (kPrefetch) {
#pragma unroll
      for (int jj = 0; jj < KB; ++jj)
        yv[jj] = reinterpret_cast<const u32x4*>(a.y + (size_t)max(srow[jj], 0) * a.H)[cc];
    }
  };
  int s = wave;
  if (s < slices) load_slice(s);
  for (; s < slices; s += nwaves) {
    const int c = s * kWave + lane;
    const int cc = min(c, a.H8 - 1);
    float gf[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gf[2 * i] = bf16_lo(gv[i]);
      gf[2 * i + 1] = bf16_hi(gv[i]);
    }
    // dot products of g with every slot's y row
#pragma unroll
    for (int b = 0; b < KB; b += 8) {
      u32x4 yb[8];
      if constexpr (!kPrefetch) {
        if (b >= a.k) break;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          yb[jj] = reinterpret_cast<const u32x4*>(a.y + (size_t)max(srow[b + jj], 0) * a.H)[cc];
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const u32x4& v = kPrefetch ? yv[jj] : yb[jj];
        if (srow[b + jj] >= 0 && c < a.H8) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p0 = gf[2 * i] * bf16_lo(v[i]);
            const float p1 = gf[2 * i + 1] * bf16_hi(v[i]);
            dot[b + jj] = dot[b + jj] + p0;
            dot[b + jj] = dot[b + jj] + p1;
          }
        }
      }
    }
    if (s + nwaves < slices) load_slice(s + nwaves);  // in flight during the stores below
    // grad_y rows: one per destination rank, its slots added in ascending order
    for (uint64_t todo = ranks; todo; todo &= todo - 1) {
      const int r = __builtin_ctzll(todo);
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
      int dst_row = 0;
#pragma unroll
      for (int jj = 0; jj < KB; ++jj) {
        if (srank[jj] == r) {
          dst_row = srow[jj];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float p = sw[jj] * gf[i];
            acc[i] = acc[i] + p;
          }
        }
      }
      if (c < a.H8) store_out(reinterpret_cast<u32x4*>(a.grad_y + (size_t)dst_row * a.H), c, acc);
    }
  }

  // fixed-order reductions: across lanes (xor tree), then across the block's waves
#pragma unroll
  for (int jj = 0; jj < KB; ++jj) {
    float v = dot[jj];
#pragma unroll
    for (int m = kWave / 2; m >= 1; m >>= 1) v = v + __shfl_xor(v, m, kWave);
    if (lane == 0) partial[wave][jj] = v;
  }
  __syncthreads();
  if (threadIdx.x < a.k) {  // wave 0, lane j: its own `valid` is slot j's
    float sum = 0.0f;
    for (int q = 0; q < nwaves; ++q) sum = sum + partial[q][threadIdx.x];
    a.grad_w[(size_t)t * a.k + threadIdx.x] = valid ? sum : 0.0f;
  }
}

// grad_topk_w[t, j] = grad_recv_w[send_row[t, rank(e_tj)], j] for valid slots, else 0.
struct WeightGradArgs {
  const float* grad_recv_w;  // [num_rows, k]
  const int32_t* topk_idx;
  const int32_t* send_row;
  float* grad_topk_w;  // [T, k]
  uint64_t rank_magic;
  int T, k, E, R, num_rows;
};

__global__ __launch_bounds__(256) void gather_weight_grad_kernel(WeightGradArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.T * a.k) return;
  const int t = (int)(i / a.k), j = (int)(i - (int64_t)t * a.k);
  const int e = a.topk_idx[i];
  float v = 0.0f;
  if ((unsigned)e < (unsigned)a.E) {
    const int row = a.send_row[(size_t)t * a.R + rank_of(e, a.rank_magic)];
    if ((unsigned)row < (unsigned)a.num_rows) v = a.grad_recv_w[(size_t)row * a.k + j];
  }
  a.grad_topk_w[i] = v;
}

}  // namespace moe
