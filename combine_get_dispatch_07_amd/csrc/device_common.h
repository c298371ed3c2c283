// Device helpers shared by the layout, dispatch and combine kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxTopk = 32;       // the library's limits (checked on the host)
constexpr int kMaxExperts = 4096;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Rank owning expert e: floor(e / L), computed as (e * ceil(2^32 / L)) >> 32.
// Exact for e, L < 2^16 (the error term e * (magic * L - 2^32) stays below 2^32).
__device__ __forceinline__ int rank_of(int e, uint64_t magic) {
  return (int)(((uint64_t)(uint32_t)e * magic) >> 32);
}

// 64-bit value of `lane` in a wave-uniform (scalar) register pair.
__device__ __forceinline__ uint64_t readlane64(uint64_t v, int lane) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

// Inclusive prefix sum over the 64 lanes of a wave, with DPP lane moves (no
// LDS round trips): shifts by 1, 2, 4 and 8 within each row of 16 lanes
// (lanes shifted in from outside a row read 0), then lane 15 of rows 0 and 2
// is added to rows 1 and 3, then lane 31 to rows 2 and 3.  Every lane of the
// wave must be active.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ int dpp_or_zero(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, kRowMask, 0xf, false);
}

__device__ __forceinline__ int wave_inclusive_scan(int v, int /*lane*/) {
  v += dpp_or_zero<0x111, 0xf>(v);  // row_shr:1
  v += dpp_or_zero<0x112, 0xf>(v);  // row_shr:2
  v += dpp_or_zero<0x114, 0xf>(v);  // row_shr:4
  v += dpp_or_zero<0x118, 0xf>(v);  // row_shr:8
  v += dpp_or_zero<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_or_zero<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Lane exchanges inside aligned groups of P = 8 or 16 lanes (DPP, no LDS
// round trip): kXor1 / kXor2 swap neighbours / pairs within a quad, kMirror8
// maps lane i of a half row to lane 7 - i, kMirror16 lane i of a row to 15 - i.
// After the steps for the smaller groups every lane of a group holds the
// group's result, so each mirror step combines two such groups.
constexpr int kXor1 = 0xb1;       // quad_perm [1, 0, 3, 2]
constexpr int kXor2 = 0x4e;       // quad_perm [2, 3, 0, 1]
constexpr int kMirror8 = 0x141;   // row_half_mirror
constexpr int kMirror16 = 0x140;  // row_mirror

// Every source lane of these patterns exists, so bound_ctrl (read 0 from a
// missing lane) never applies; it lets the compiler fold the move into the
// instruction that consumes it.
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kCtrl, 0xf, 0xf, true);
}

// op over aligned groups of N lanes (N = 1, 2, 4, 8 or 16), result in all of them.
template <int N, typename Op>
__device__ __forceinline__ uint32_t lanes_reduce(uint32_t x, Op op) {
  if constexpr (N >= 2) x = op(x, dpp32<kXor1>(x));
  if constexpr (N >= 4) x = op(x, dpp32<kXor2>(x));
  if constexpr (N >= 8) x = op(x, dpp32<kMirror8>(x));
  if constexpr (N >= 16) x = op(x, dpp32<kMirror16>(x));
  return x;
}

template <int N>
__device__ __forceinline__ uint32_t lanes_max(uint32_t x) {
  return lanes_reduce<N>(x, [](uint32_t u, uint32_t v) { return max(u, v); });
}

// The same value in all N lanes: a fixed tree of pairwise sums, up to the
// order of operands of each addition, which does not change a sum.
template <int N>
__device__ __forceinline__ float lanes_sum(float x) {
  return __uint_as_float(lanes_reduce<N>(__float_as_uint(x), [](uint32_t u, uint32_t v) {
    return __float_as_uint(__uint_as_float(u) + __uint_as_float(v));
  }));
}

// bf16 halves of a 32-bit word, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// fp32 -> OCP E4M3 ("fn": bias 7, max 448, no infinities) codes of two values,
// round to nearest even, sign kept (-0 and negative values that round to zero
// give 0x80), with gfx950's v_cvt_pk_fp8_f32: the codes land in bytes 0-1
// (kHi false) or 2-3 (kHi true) of `old`, whose other half is kept.  Checked
// against round-to-nearest-even over every fp32 magnitude below 464, the range
// the per-block scaling produces (|x / s| <= 448 (1 + 2^-23)^2); larger or
// non-finite inputs are outside that contract.
template <bool kHi>
__device__ __forceinline__ uint32_t e4m3_pack2(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, kHi);
}

// Hand-off of data between the blocks of one launch.  On gfx950 every XCD has
// its own L2, and an agent-scope release or acquire fence writes back or
// invalidates a whole L2, which is slow.  So data one block hands to another is
// written and read with agent-scope atomic stores and loads (relaxed), which go
// through the L2 to the device-coherent level (the sc1 bit), and ordering comes
// from waits alone: a writer waits for its own stores to complete before the
// atomic that signals them (wait_own_stores), and a reader issues its loads
// only once the signalling atomic's value has arrived.  Nothing else of the
// block needs to reach another block in the same launch.
template <typename T>
__device__ __forceinline__ void put_coherent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
__device__ __forceinline__ T get_coherent(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// This wave's earlier vector-memory operations (stores and atomics included)
// have completed: s_waitcnt vmcnt(0), with the expcnt and lgkmcnt fields at
// their "no wait" maxima (7 and 15).
__device__ __forceinline__ void wait_own_stores() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xf << 8));
}

}  // namespace moe
