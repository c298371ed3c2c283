// Dispatch kernel: stable prefix-sum slot assignment plus the row pack, bf16
// bit copy or FP8 E4M3 with one fp32 scale per 128 channels.
//
// Follows "DeepEP：年度总结中的计算通信重叠摘记" (notes.kuangjux.top), section
// 节点内通信 (rows go only to ranks in is_token_in_rank; FP8 halves the bytes
// moved), and the mlqm.cn rocSHMEM notes, section 3.2 (rows are packed into a
// preallocated receive buffer).  Receive row of (t, r) = rank_offsets[r] +
// #{t' < t : t' goes to r}: segments in rank order, tokens ascending.
//
// Work item = (token, hidden slice); one wave per item.  A wave reads the
// 64 rank bitmasks of its token's chunk (one per lane); a ballot per
// destination rank plus the chunk's precomputed base gives the row.  The
// slice is loaded once with 16-byte loads (each instruction reads 1 KiB
// contiguous), quantised once if FP8, and stored to every destination row
// with nontemporal stores (the receive rows are not re-read by this kernel).
#pragma once

#include "device_common.h"

namespace moe {

// Source rows are read once.  Measured at 4096 tokens with the rows out of every cache: ordinary
// loads are ~1.5% faster than nontemporal ones for the bf16 copy, nontemporal ones ~9% faster for
// the FP8 pack; stores are nontemporal for both (ordinary stores were 3-16% slower).
template <bool kNt>
__device__ __forceinline__ u32x4 load_source(const u32x4* p) {
  if constexpr (kNt)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

#ifndef MOE_DISPATCH_BLOCK
#define MOE_DISPATCH_BLOCK 256
#endif
constexpr int kDispatchBlock = MOE_DISPATCH_BLOCK;  // 4 waves: 4 work items per block
constexpr int kFp8Block = 128;       // channels per FP8 scale
constexpr float kAmaxFloor = 1e-4f;
constexpr float kE4m3Max = 448.0f;

struct DispatchArgs {
  const uint16_t* x;
  const int32_t* topk_idx;
  const float* topk_w;
  const uint64_t* token_ranks;
  const int32_t* chunk_base;     // [R, NC] receive row of each chunk's first token on rank r
  const int32_t* ws_rank_offsets;
  void* recv_x;
  float* recv_scales;
  int32_t* recv_src_idx;
  int32_t* recv_topk_idx;
  float* recv_topk_w;
  int32_t* rank_offsets;
  int32_t* send_row;
  int32_t* num_recv;
  uint64_t rank_magic;
  uint64_t rank_bits;  // (1 << R) - 1
  int T, H, H8, k, E, R, L, NC;
  int capacity;  // receive rows allocated; rows at or beyond it are never written
  int slices;    // hidden slices per token
  int items;   // T * slices
};

// Eight bf16 channels of one lane -> eight E4M3 codes, given the block scale:
// q = E4M3_RNE(fl32(x / s)), IEEE division, then the hardware conversion.
__device__ __forceinline__ u32x2 quantize8(u32x4 v, float s) {
#pragma clang fp contract(off)
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(v[i]) / s;
    f[2 * i + 1] = bf16_hi(v[i]) / s;
  }
  u32x2 out;
#pragma unroll
  for (int w = 0; w < 2; ++w)
    out[w] = e4m3_pack2<true>(f[4 * w + 2], f[4 * w + 3], e4m3_pack2<false>(f[4 * w], f[4 * w + 1], 0u));
  return out;
}

// Standalone E4M3 encoding (moe_encode_e4m3): four values per thread.
__global__ __launch_bounds__(256) void encode_e4m3_kernel(const float* in, uint8_t* out, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = i + j < n ? in[i + j] : 0.0f;
  const uint32_t q = e4m3_pack2<true>(v[2], v[3], e4m3_pack2<false>(v[0], v[1], 0u));
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (i + j < n) out[i + j] = (uint8_t)(q >> (8 * j));
}

// |x| maximum over the 16 lanes (128 channels) sharing a scale, as fp32.
__device__ __forceinline__ float block_amax(u32x4 v) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = max(m, v[i] & 0x7fffu);
    m = max(m, (v[i] >> 16) & 0x7fffu);
  }
  // bf16 magnitudes order like their bit patterns, so the maximum is exact;
  // DPP lane moves within each row of 16 lanes (every lane must be active)
  return __uint_as_float(lanes_max<16>(m) << 16);
}

// FP8 codes and block scales of a wave's slice, this lane's U 16-byte pieces:
// one scale per 128 channels (16 lanes), s = fl32(max(amax, 1e-4) / 448).
template <int U>
__device__ __forceinline__ void quantize_slice(const u32x4 (&v)[U], u32x2 (&q)[U], float (&sc)[U]) {
#pragma clang fp contract(off)
#pragma unroll
  for (int u = 0; u < U; ++u) {
    sc[u] = fmaxf(block_amax(v[u]), kAmaxFloor) / kE4m3Max;
    q[u] = quantize8(v[u], sc[u]);
  }
}

// Writes this lane's pieces of a slice (piece u covers 16-byte column c0 + 64u
// of the row) to receive row `row`: the bf16 bits, or the E4M3 codes and, from
// the first lane of each 16, the block scale.  Nontemporal stores: the receive
// rows are not read again by the dispatch.
template <int U, bool kFp8>
__device__ __forceinline__ void store_slice(void* recv_x, float* recv_scales, size_t row, int H, int H8, int c0,
                                            int lane, const u32x4 (&v)[U], const u32x2 (&q)[U],
                                            const float (&sc)[U]) {
  if constexpr (kFp8) {
    u32x2* dst = reinterpret_cast<u32x2*>(static_cast<uint8_t*>(recv_x) + row * H);
    float* sdst = recv_scales + row * (H / kFp8Block);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave;
      if (c < H8) {
        __builtin_nontemporal_store(q[u], dst + c);
        if ((lane & 15) == 0) sdst[c >> 4] = sc[u];
      }
    }
  } else {
    u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(recv_x) + row * H);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave;
      if (c < H8) __builtin_nontemporal_store(v[u], dst + c);
    }
  }
}

// This lane's U 16-byte pieces of the x slice of `item` (clamped addresses).
template <int U, bool kFp8>
__device__ __forceinline__ void load_item_slice(const DispatchArgs& a, int item, int lane, u32x4 (&v)[U]) {
  const int t = item / a.slices;
  const int c0 = (item - t * a.slices) * (U * kWave) + lane;
  const u32x4* xrow = reinterpret_cast<const u32x4*>(a.x + (size_t)t * a.H);
#pragma unroll
  for (int u = 0; u < U; ++u) v[u] = load_source<kFp8>(xrow + min(c0 + u * kWave, a.H8 - 1));
}

// Packs item (token t, slice s) once everything it needs is in registers:
//   v        this lane's pieces of the x slice;
//   lm       lane l: rank bitmask of token 64 (t / 64) + l of t's chunk (0 past T);
//   chunk_row lane r < R: receive row of the chunk's first token going to rank r;
//   ej_raw, wj_raw lane j < k: expert id and weight of slot j (read only when s == 0
//            for bf16; every wave for FP8).
// For each destination rank the row is chunk_row + the chunk's tokens before t
// going to that rank (a ballot); the slice is quantised once if FP8 and stored
// to every destination; the first slice's wave writes the row metadata and
// send_row.
template <int U, bool kFp8>
__device__ __forceinline__ void pack_item(const DispatchArgs& a, int t, int s, int lane, u32x4 (&v)[U], uint64_t lm,
                                          int chunk_row, int ej_raw, float wj_raw) {
#pragma clang fp contract(off)
  const int c0 = s * (U * kWave) + lane;
  const uint64_t mine = readlane64(lm, t & (kWave - 1)) & a.rank_bits;
  const int tl = t & (kWave - 1);
  const uint64_t lanes_below = tl == 0 ? 0ull : (~0ull >> (kWave - tl));
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (c0 + u * kWave >= a.H8) v[u] = u32x4{0u, 0u, 0u, 0u};

  u32x2 q[U];
  float sc[U];
  if constexpr (kFp8) quantize_slice<U>(v, q, sc);

  // Slot metadata: lane j < k holds slot j of this token.
  const bool meta = s == 0;
  const int ej = lane < a.k ? ej_raw : -1;
  const float wj = lane < a.k ? wj_raw : 0.0f;
  const int rj = (unsigned)ej < (unsigned)a.E ? rank_of(ej, a.rank_magic) : -1;

  int my_row = -1;  // lane r: receive row of (t, r)
  uint64_t todo = mine;
  while (todo) {
    const int r = __builtin_ctzll(todo);
    todo &= todo - 1;
    const uint64_t before = __ballot((lm >> r) & 1ull) & lanes_below;
    const int row = __builtin_amdgcn_readlane(chunk_row, r) + __popcll(before);
    if ((unsigned)row >= (unsigned)a.capacity) continue;  // only a plan from another layout gets here
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

// No load sits under a lane-dependent branch: each is issued from a clamped,
// always valid address and masked afterwards.  A load under such a branch makes
// the compiler wait for it before the branch joins, which would serialise the
// loads (one memory round trip each) in this latency-bound kernel.
template <int U, bool kFp8>
__device__ __forceinline__ void dispatch_item(const DispatchArgs& a, int item, int lane) {
  const int t = item / a.slices;
  const int s = item - t * a.slices;
  const int chunk = t >> 6;
  const int tt = (chunk << 6) + lane;
  const int rl = min(lane, a.R - 1);
  const int jl = min(lane, a.k - 1);

  // All loads first: the chunk's rank bitmasks (one per lane), the row of the
  // chunk's first token on rank lane, the x slice, and the slot metadata (lane
  // j = slot j).
  const uint64_t lm_raw = a.token_ranks[min(tt, a.T - 1)];
  const int cb = a.chunk_base[rl * a.NC + chunk];
  u32x4 v[U];
  load_item_slice<U, kFp8>(a, item, lane, v);
  // Only the first slice's wave writes the slot metadata.  bf16 rows are split into many slices,
  // and loading the slots in that wave alone took 0.4-1 us off the prefill copy; for FP8 every
  // wave loading them measured faster.  The branch is wave-uniform, so no lane waits at its join.
  int ej_raw = -1;
  float wj_raw = 0.0f;
  if (kFp8 || s == 0) {
    ej_raw = a.topk_idx[(size_t)t * a.k + jl];
    wj_raw = a.topk_w[(size_t)t * a.k + jl];
  }
  pack_item<U, kFp8>(a, t, s, lane, v, tt < a.T ? lm_raw : 0ull, lane < a.R ? cb : 0, ej_raw, wj_raw);
}

template <int U, bool kFp8>
__global__ __launch_bounds__(kDispatchBlock) void dispatch_kernel(DispatchArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = blockIdx.x * (kDispatchBlock / kWave) + wave;
  if (item < a.items) dispatch_item<U, kFp8>(a, item, lane);
  if (blockIdx.x == 0 && wave == 0) {  // publish the segment offsets and the row count
    const int off = a.ws_rank_offsets[lane < a.R ? lane : a.R];
    if (lane < a.R) a.rank_offsets[lane] = off;
    if (lane == 0) {
      const int total = a.ws_rank_offsets[a.R];
      a.rank_offsets[a.R] = total;
      *a.num_recv = total;
    }
  }
}

}  // namespace moe
