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

constexpr int kNarrowTopk = 8;  // slots whose y rows the narrow variant keeps in flight

// Slot metadata of token t, one slot per lane: lane j < k holds slot j's weight,
// destination rank and y row; `valid` is false for lanes >= k, invalid ids and
// rows outside y.  Lane r < R also holds the token's row on rank r.
struct BwdSlots {
  float w;
  int rank, row, rank_row;
  bool valid;
};

__device__ __forceinline__ BwdSlots bwd_slots(const CombineBwdArgs& a, int t, int lane) {
  BwdSlots m;
  const int j = min(lane, a.k - 1);
  const int id = a.topk_idx[(size_t)t * a.k + j];
  m.w = a.topk_w[(size_t)t * a.k + j];
  m.rank_row = a.send_row[(size_t)t * a.R + min(lane, a.R - 1)];
  m.valid = lane < a.k && (unsigned)id < (unsigned)a.E;
  m.rank = m.valid ? rank_of(id, a.rank_magic) : 0;
  m.row = __shfl(m.rank_row, m.rank, kWave);
  m.valid = m.valid && (unsigned)m.row < (unsigned)a.num_y_rows;
  return m;
}

// Fixed-order reduction of the dot products: across lanes (a DPP tree within
// each row of 16 lanes, then rows 0 + 16 and 32 + 48, then those two), then
// across the block's waves in ascending order.  dot[p] for p < n is reduced;
// wave 0, lane j < k writes slot j's total, taken from dot[pos] (pos: lane j's
// index into dot).
template <int N>
__device__ __forceinline__ void bwd_reduce_dots(const CombineBwdArgs& a, const float (&dot)[N], int n,
                                                float (&partial)[kBwdMaxWaves][kMaxTopk], int t, int lane,
                                                int wave, int nwaves, bool valid, int pos) {
#pragma clang fp contract(off)
#pragma unroll
  for (int jj = 0; jj < N; ++jj) {
    if (jj < n) {
      const int r = __float_as_int(lanes_sum<16>(dot[jj]));
      const float lo = __int_as_float(__builtin_amdgcn_readlane(r, 0)) +
                       __int_as_float(__builtin_amdgcn_readlane(r, 16));
      const float hi = __int_as_float(__builtin_amdgcn_readlane(r, 32)) +
                       __int_as_float(__builtin_amdgcn_readlane(r, 48));
      if (lane == 0) partial[wave][jj] = lo + hi;
    }
  }
  __syncthreads();
  if (threadIdx.x < a.k) {  // wave 0, lane j: its own `valid` is slot j's
    float sum = 0.0f;
    for (int q = 0; q < nwaves; ++q) sum = sum + partial[q][pos];
    a.grad_w[(size_t)t * a.k + threadIdx.x] = valid ? sum : 0.0f;
  }
}

// k <= 8: one block per token, wave w takes hidden slices w, w + nwaves, ...
// A software pipeline issues the next slice's g and y loads before the
// current slice's grad_y rows are stored.
__global__ __launch_bounds__(kBwdMaxWaves * kWave) void combine_backward_kernel(CombineBwdArgs a) {
#pragma clang fp contract(off)
  constexpr int KB = kNarrowTopk;
  __shared__ float partial[kBwdMaxWaves][kMaxTopk];
  const int nwaves = blockDim.x / kWave;
  const int t = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const BwdSlots m = bwd_slots(a, t, lane);

  int srank[KB], srow[KB];
  float sw[KB];
  uint64_t ranks = 0;
#pragma unroll
  for (int jj = 0; jj < KB; ++jj) {  // wave-uniform copies of the slot metadata
    const bool v = __builtin_amdgcn_readlane((int)m.valid, jj) != 0;
    srank[jj] = v ? __builtin_amdgcn_readlane(m.rank, jj) : -1;
    srow[jj] = v ? __builtin_amdgcn_readlane(m.row, jj) : -1;
    sw[jj] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m.w), jj));
    if (v) ranks |= 1ull << srank[jj];
  }

  float dot[KB];
#pragma unroll
  for (int jj = 0; jj < KB; ++jj) dot[jj] = 0.0f;

  const int slices = (a.H8 + kWave - 1) / kWave;
  const u32x4* grow = reinterpret_cast<const u32x4*>(a.g + (size_t)t * a.H);
  u32x4 gv, yv[KB];
  auto load_slice = [&](int s_) {
    const int cc = min(s_ * kWave + lane, a.H8 - 1);
    gv = grow[cc];
#pragma unroll
    for (int jj = 0; jj < KB; ++jj)
      yv[jj] = reinterpret_cast<const u32x4*>(a.y + (size_t)max(srow[jj], 0) * a.H)[cc];
  };
  int s = wave;
  if (s < slices) load_slice(s);
  for (; s < slices; s += nwaves) {
    const int c = s * kWave + lane;
    float gf[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gf[2 * i] = bf16_lo(gv[i]);
      gf[2 * i + 1] = bf16_hi(gv[i]);
    }
    // dot products of g with every slot's y row
#pragma unroll
    for (int jj = 0; jj < KB; ++jj) {
      if (srow[jj] >= 0 && c < a.H8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p0 = gf[2 * i] * bf16_lo(yv[jj][i]);
          const float p1 = gf[2 * i + 1] * bf16_hi(yv[jj][i]);
          dot[jj] = dot[jj] + p0;
          dot[jj] = dot[jj] + p1;
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
  bwd_reduce_dots(a, dot, a.k, partial, t, lane, wave, nwaves, m.valid, lane);
}

// 8 < k <= 32: the slot metadata stays one slot per lane and is read with
// readlane where it is used.  Slots on one rank share that rank's y row, so the
// dot products are taken once per distinct row (at most min(k, R) of them, in
// ascending rank order) and handed to every slot on the rank; per slice the y
// rows are loaded 8 at a time.  grad_y rows take each rank's slots from a
// ballot, in ascending slot order.
__global__ __launch_bounds__(kBwdMaxWaves * kWave) void combine_backward_wide_kernel(CombineBwdArgs a) {
#pragma clang fp contract(off)
  __shared__ float partial[kBwdMaxWaves][kMaxTopk];
  const int nwaves = blockDim.x / kWave;
  const int t = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const BwdSlots m = bwd_slots(a, t, lane);
  const uint64_t vmask = __ballot(m.valid);
  uint64_t ranks = 0;
  for (uint64_t todo = vmask; todo; todo &= todo - 1)
    ranks |= 1ull << __builtin_amdgcn_readlane(m.rank, __builtin_ctzll(todo));
  // Lane p < nrows: the p-th distinct row (ascending rank); lane j: slot j's index p.
  const int nrows = __popcll(ranks);
  const bool has = (ranks >> lane) & 1ull;
  const uint64_t below = lane == 0 ? 0ull : ranks & (~0ull >> (kWave - lane));
  const int dst = has ? __popcll(below) : nrows + lane - __popcll(below);  // a permutation of the lanes
  const int drow = __builtin_amdgcn_ds_permute(dst << 2, has ? m.rank_row : -1);
  const int pos = __popcll(ranks & ((1ull << m.rank) - 1ull));

  float dot[kMaxTopk];
#pragma unroll
  for (int jj = 0; jj < kMaxTopk; ++jj) dot[jj] = 0.0f;

  const int slices = (a.H8 + kWave - 1) / kWave;
  const u32x4* grow = reinterpret_cast<const u32x4*>(a.g + (size_t)t * a.H);
  for (int s = wave; s < slices; s += nwaves) {
    const int c = s * kWave + lane;
    const int cc = min(c, a.H8 - 1);
    const u32x4 gv = grow[cc];
    float gf[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gf[2 * i] = bf16_lo(gv[i]);
      gf[2 * i + 1] = bf16_hi(gv[i]);
    }
#pragma unroll
    for (int b = 0; b < kMaxTopk; b += 8) {
      if (b >= nrows) break;
      int brow[8];
      u32x4 yb[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        brow[jj] = __builtin_amdgcn_readlane(drow, b + jj);
        yb[jj] = reinterpret_cast<const u32x4*>(a.y + (size_t)max(brow[jj], 0) * a.H)[cc];
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        if (brow[jj] >= 0 && c < a.H8) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p0 = gf[2 * i] * bf16_lo(yb[jj][i]);
            const float p1 = gf[2 * i + 1] * bf16_hi(yb[jj][i]);
            dot[b + jj] = dot[b + jj] + p0;
            dot[b + jj] = dot[b + jj] + p1;
          }
        }
      }
    }
    for (uint64_t todo = ranks; todo; todo &= todo - 1) {
      const int r = __builtin_ctzll(todo);
      const uint64_t on_r = __ballot(m.valid && m.rank == r);
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
      const int dst_row = __builtin_amdgcn_readlane(m.rank_row, r);
      for (uint64_t sl = on_r; sl; sl &= sl - 1) {
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m.w), __builtin_ctzll(sl)));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p = wj * gf[i];
          acc[i] = acc[i] + p;
        }
      }
      if (c < a.H8) store_out(reinterpret_cast<u32x4*>(a.grad_y + (size_t)dst_row * a.H), c, acc);
    }
  }
  bwd_reduce_dots(a, dot, nrows, partial, t, lane, wave, nwaves, m.valid, pos);
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
