// Host side of the C ABI declared in include/moe_ep.h: argument checks, the
// workspace (dispatch plan) carve-up, launch shapes and kernel launches.
// Everything is checked before the first HIP call, so a rejected call touches
// neither the GPU nor any memory.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>

#include "moe_ep.h"

#include "backward_kernels.h"
#include "combine_kernels.h"
#include "device_common.h"
#include "dispatch_kernels.h"
#include "layout_kernels.h"
#include "ll_kernels.h"
#include "router_kernels.h"
#include "send_small_kernels.h"
#include "fused_send_kernels.h"

namespace {

constexpr int kMaxTopk = moe::kMaxTopk;
constexpr int kMaxRanks = 64;
constexpr int kMaxExperts = moe::kMaxExperts;
constexpr size_t kPlanAlign = 256;
constexpr int kMaxDevices = 64;
constexpr int kMaxCuMaskWords = 32;  // up to 1024 compute units
// Wide FP8 dispatch slices only when they still give this many waves.
constexpr long kMinFp8Waves = 4096;

struct PlanLayout {
  size_t sync, expert_acc, rank_acc, token_ranks, chunk_base, rank_offsets, total;
  int NC, NB;
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

moe_status check_shape(const moe_shape* s) {
  if (s == nullptr) return MOE_ERR_INVALID_ARG;
  const int64_t T = s->num_tokens, H = s->hidden, k = s->num_topk, E = s->num_experts,
                R = s->num_ranks;
  if (T < 0 || H <= 0 || H % 8 != 0 || k < 1 || E < 1 || R < 1) return MOE_ERR_INVALID_ARG;
  if (k > kMaxTopk || R > kMaxRanks || E > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (R > E || E % R != 0 || k > E) return MOE_ERR_INVALID_ARG;
  // T <= 2^30 leaves int headroom for the token-derived launch arithmetic (T + 63, T + 1, ...).
  if (T > (int64_t)1 << 30 || T * k > INT32_MAX || T * R > INT32_MAX || T * std::min(k, R) > INT32_MAX)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

PlanLayout plan_layout(const moe_shape& s) {
  PlanLayout p{};
  const size_t T = (size_t)s.num_tokens, R = (size_t)s.num_ranks, E = (size_t)s.num_experts;
  p.NC = (int)((T + moe::kWave - 1) / moe::kWave);
  p.NB = (int)((T + moe::kLayoutBlock - 1) / moe::kLayoutBlock);
  size_t off = 0;
  p.sync = off;  // sync words and the two accumulators: zero between calls
  off = align_up(off + moe::kSyncBytes, kPlanAlign);
  p.expert_acc = off;
  off = align_up(off + E * sizeof(int32_t), kPlanAlign);
  p.rank_acc = off;
  off = align_up(off + R * sizeof(int32_t), kPlanAlign);
  p.token_ranks = off;
  off = align_up(off + T * sizeof(uint64_t), kPlanAlign);
  p.chunk_base = off;
  off = align_up(off + R * (size_t)p.NC * sizeof(int32_t), kPlanAlign);
  p.rank_offsets = off;
  off = align_up(off + (R + 1) * sizeof(int32_t), kPlanAlign);
  p.total = off;
  return p;
}

uint64_t rank_magic(const moe_shape& s) {
  const uint64_t L = (uint64_t)(s.num_experts / s.num_ranks);
  return ((1ull << 32) + L - 1) / L;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// A pointer may be NULL exactly when the array it stands for is empty.
bool present(const void* p, int64_t elements) { return p != nullptr || elements == 0; }

// Dispatch work item = (token, slice of U*512 channels).  bf16 rows favour
// narrow slices (many short waves keep the most stores in flight).  FP8 rows
// favour wide slices when there are enough tokens to fill the chip: one wave
// then quantises the whole row and writes each destination's scale row as a
// unit instead of 16-byte fragments from many waves.
int pick_dispatch_chunks_per_lane(int T, int H8, bool fp8) {
  if (!fp8) return 1;
  static const int kOptions[] = {14, 7, 4, 2};
  const int groups = (H8 + moe::kWave - 1) / moe::kWave;  // 64-lane chunk groups per row
  for (int u : kOptions) {
    if (u > groups) continue;
    const long slices = (groups + u - 1) / u;
    if ((long)T * slices >= kMinFp8Waves) return u;
  }
  return 1;
}

moe_status last_launch_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

template <bool kFp8>
void launch_dispatch(int U, dim3 grid, hipStream_t stream, const moe::DispatchArgs& a) {
  const dim3 block(moe::kDispatchBlock);
  switch (U) {
    case 14: hipLaunchKernelGGL((moe::dispatch_kernel<14, kFp8>), grid, block, 0, stream, a); break;
    case 7: hipLaunchKernelGGL((moe::dispatch_kernel<7, kFp8>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((moe::dispatch_kernel<4, kFp8>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((moe::dispatch_kernel<2, kFp8>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((moe::dispatch_kernel<1, kFp8>), grid, block, 0, stream, a); break;
  }
}

// Waves per token in the combine backward (each takes every MOE_BWD_WAVES-th slice).
#ifndef MOE_BWD_WAVES
#define MOE_BWD_WAVES 7
#endif
static_assert(MOE_BWD_WAVES >= 1 && MOE_BWD_WAVES <= moe::kBwdMaxWaves, "waves per block");

// Small-batch low-latency dispatch in one launch (0: always the two-pass path).
#ifndef MOE_LL_SMALL
#define MOE_LL_SMALL 1
#endif
// Resident combine waves per CU in the persistent launch: one block of 4
// waves, one per SIMD, each with two items' payload in flight.  Fewer
// concurrent streams keep the rows being read at any time close together.
#ifndef MOE_COMBINE_WAVES_PER_CU
#define MOE_COMBINE_WAVES_PER_CU 4
#endif
// Layout and dispatch in one launch for small batches in moe_layout_dispatch (0: two launches).
#ifndef MOE_SEND_SMALL
#define MOE_SEND_SMALL 1
#endif
#ifndef MOE_COMBINE_MAX_WAVES_PER_CU
#define MOE_COMBINE_MAX_WAVES_PER_CU 16
#endif

// Compute units of the current device, queried once per device.
int device_cu_count() {
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Streams made by moe_stream_create_cu_range and the number of CUs each may
// use, so that a launch learns its stream's CU budget from a table lookup
// instead of asking the runtime for the stream's mask on every call.  Slots are
// claimed and released with compare-and-swap; a lookup scans them only while
// some stream is registered.
constexpr int kMaxCuStreams = 64;
struct CuStream {
  std::atomic<hipStream_t> stream{nullptr};
  std::atomic<int> cus{0};
};
CuStream g_cu_streams[kMaxCuStreams];
std::atomic<int> g_cu_stream_count{0};

bool register_cu_stream(hipStream_t stream, int cus) {
  for (CuStream& slot : g_cu_streams) {
    hipStream_t empty = nullptr;
    if (slot.stream.load(std::memory_order_relaxed) == nullptr &&
        slot.stream.compare_exchange_strong(empty, stream, std::memory_order_acq_rel)) {
      slot.cus.store(cus, std::memory_order_release);
      g_cu_stream_count.fetch_add(1, std::memory_order_acq_rel);
      return true;
    }
  }
  return false;
}

void unregister_cu_stream(hipStream_t stream) {
  for (CuStream& slot : g_cu_streams) {
    hipStream_t s = stream;
    if (slot.stream.load(std::memory_order_acquire) == stream) {
      slot.cus.store(0, std::memory_order_relaxed);
      if (slot.stream.compare_exchange_strong(s, nullptr, std::memory_order_acq_rel))
        g_cu_stream_count.fetch_sub(1, std::memory_order_acq_rel);
      return;
    }
  }
}

// Compute units a launch on `stream` can use: the registered budget of a
// stream made by moe_stream_create_cu_range, else all of the device's CUs.
int stream_cu_count(hipStream_t stream) {
  if (stream != nullptr && g_cu_stream_count.load(std::memory_order_acquire) > 0) {
    for (const CuStream& slot : g_cu_streams) {
      if (slot.stream.load(std::memory_order_acquire) == stream) {
        const int cus = slot.cus.load(std::memory_order_acquire);
        if (cus > 0) return std::min(cus, device_cu_count());
      }
    }
  }
  return device_cu_count();
}

int device_xcc_count() {
  int dev = 0, xcc = 1;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&xcc, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcc <= 0) {
    (void)hipGetLastError();
    return 1;
  }
  return xcc;
}

__global__ __launch_bounds__(256) void zero_fill_kernel(moe::u32x4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = moe::u32x4{0u, 0u, 0u, 0u};
}

__global__ __launch_bounds__(256) void zero_fill_f32_kernel(float* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0.0f;
}

// Combine over T tokens: one wave per (token, 512-channel slice) item, on a
// persistent grid.  With no rows of y every slot is skipped and out is +0.
template <int kMode>
moe_status launch_combine(moe::CombineArgs& a, void* out, hipStream_t stream) {
  const size_t out16 = (size_t)a.T * a.H8;
  if (a.num_y_rows == 0) {
    const unsigned blocks = (unsigned)std::min<size_t>((out16 + 255) / 256, 4096);
    hipLaunchKernelGGL(zero_fill_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<moe::u32x4*>(out), out16);
    return last_launch_status();
  }
  a.slices = (a.H8 + moe::kWave - 1) / moe::kWave;
  if ((int64_t)a.T * a.slices > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  a.items = a.T * a.slices;
  const int waves_per_block = moe::kCombineBlock / moe::kWave;
  // A stream limited to fewer CUs keeps about the full chip's number of waves in
  // flight (each CU then serves a larger share of the bandwidth), up to
  // MOE_COMBINE_MAX_WAVES_PER_CU.
  const long cus = stream_cu_count(stream);
  const long per_cu = std::min<long>(MOE_COMBINE_MAX_WAVES_PER_CU,
                                     std::max<long>(MOE_COMBINE_WAVES_PER_CU,
                                                    (long)MOE_COMBINE_WAVES_PER_CU * device_cu_count() / cus));
  const long resident = cus * per_cu / waves_per_block;
  const dim3 grid((unsigned)std::min<long>((a.items + waves_per_block - 1) / waves_per_block, resident));
  const dim3 block(moe::kCombineBlock);
  a.terms = kMode == moe::kRankRows ? std::min(a.k, a.R) : a.k;
  if (a.terms <= moe::kSlotBatch)
    hipLaunchKernelGGL((moe::combine_pipelined_kernel<kMode>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((moe::combine_persistent_kernel<kMode>), grid, block, 0, stream, a);
  return last_launch_status();
}

struct LlPlanLayout {
  size_t slot_local, chunk_base, total;
  int NC;
};

LlPlanLayout ll_plan_layout(const moe_shape& s) {
  LlPlanLayout p{};
  p.NC = (s.num_tokens + moe::kWave - 1) / moe::kWave;
  size_t off = 0;
  p.slot_local = off;
  off = align_up(off + (size_t)s.num_tokens * s.num_topk * sizeof(int32_t), kPlanAlign);
  p.chunk_base = off;
  off = align_up(off + (size_t)s.num_experts * p.NC * sizeof(int32_t), kPlanAlign);
  p.total = std::max(off, kPlanAlign);  // never empty: callers always pass a real allocation
  return p;
}

template <bool kFp8, int KI>
void launch_ll_small_t(int U, dim3 grid, dim3 block, hipStream_t stream, const moe::LlDispatchArgs& a,
                       int32_t* recv_count) {
  if (U == 2)
    hipLaunchKernelGGL((moe::ll_dispatch_small_kernel<2, kFp8, KI>), grid, block, 0, stream, a, recv_count);
  else
    hipLaunchKernelGGL((moe::ll_dispatch_small_kernel<1, kFp8, KI>), grid, block, 0, stream, a, recv_count);
}

void launch_ll_small(int U, bool fp8, dim3 grid, dim3 block, hipStream_t stream, const moe::LlDispatchArgs& a,
                     int32_t* recv_count) {
  const bool narrow = a.k <= 8;  // ids held per lane: 8, else the top-k limit
  if (fp8 && narrow)
    launch_ll_small_t<true, 8>(U, grid, block, stream, a, recv_count);
  else if (fp8)
    launch_ll_small_t<true, moe::kMaxTopk>(U, grid, block, stream, a, recv_count);
  else if (narrow)
    launch_ll_small_t<false, 8>(U, grid, block, stream, a, recv_count);
  else
    launch_ll_small_t<false, moe::kMaxTopk>(U, grid, block, stream, a, recv_count);
}

template <bool kFp8>
void launch_ll_dispatch(int U, dim3 grid, hipStream_t stream, const moe::LlDispatchArgs& a) {
  const dim3 block(moe::kDispatchBlock);
  switch (U) {
    case 14: hipLaunchKernelGGL((moe::ll_dispatch_kernel<14, kFp8>), grid, block, 0, stream, a); break;
    case 7: hipLaunchKernelGGL((moe::ll_dispatch_kernel<7, kFp8>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((moe::ll_dispatch_kernel<4, kFp8>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((moe::ll_dispatch_kernel<2, kFp8>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((moe::ll_dispatch_kernel<1, kFp8>), grid, block, 0, stream, a); break;
  }
}


// One launch at every size; the routing block that finishes last finalises the plan.
template <int P, int KS>
void launch_router(int T, size_t lds, hipStream_t stream, const moe::RouterArgs& a) {
  if (T == 0) {  // no tokens: one block writes zero counts and offsets
    hipLaunchKernelGGL(moe::layout_fused_kernel<8>, dim3(1), dim3(moe::kWave), lds, stream, a.lay);
  } else if (T <= moe::kFusedMaxTokens) {  // small blocks spread the routing over many CUs
    constexpr int tokens_per_block = moe::kRouterSmallWaves * moe::kWave / P;
    const int blocks = (T + tokens_per_block - 1) / tokens_per_block;
    hipLaunchKernelGGL((moe::router_small_kernel<P, KS>), dim3(blocks), dim3(moe::kRouterSmallWaves * moe::kWave), 0,
                       stream, a);
  } else {
    hipLaunchKernelGGL((moe::router_count_kernel<P, KS>), dim3(a.lay.NC), dim3(moe::kWave * P), lds, stream, a);
  }
}

// log2(R) when R is a power of two >= 4 and is_token_in_rank is 16-byte aligned (a wave's rows are
// then 16-byte aligned too: 64 R bytes per wave), else -1.
int mask_shift(const moe_shape& s, const void* is_token_in_rank) {
  const int R = s.num_ranks;
  if (R < 4 || (R & (R - 1)) != 0 || !aligned(is_token_in_rank, 16)) return -1;
  return __builtin_ctz((unsigned)R);
}

// Layout arguments after every check moe_get_dispatch_layout makes (shape already checked).
moe_status layout_args(const moe_shape& s, const int32_t* topk_idx, int32_t* tokens_per_rank,
                       int32_t* tokens_per_expert, uint8_t* is_token_in_rank, void* workspace, size_t workspace_bytes,
                       moe::LayoutArgs& a) {
  const int64_t T = s.num_tokens;
  if (!present(topk_idx, T) || !present(is_token_in_rank, T) || !tokens_per_rank || !tokens_per_expert ||
      !workspace)
    return MOE_ERR_INVALID_ARG;
  if (!aligned(topk_idx, 4) || !aligned(tokens_per_rank, 4) || !aligned(tokens_per_expert, 4) ||
      !aligned(workspace, kPlanAlign))
    return MOE_ERR_INVALID_ARG;
  const PlanLayout p = plan_layout(s);
  if (workspace_bytes < p.total) return MOE_ERR_INVALID_ARG;

  char* ws = static_cast<char*>(workspace);
  a = moe::LayoutArgs{};
  a.sync = reinterpret_cast<moe::SyncWords*>(ws + p.sync);
  a.expert_acc = reinterpret_cast<int32_t*>(ws + p.expert_acc);
  a.rank_acc = reinterpret_cast<int32_t*>(ws + p.rank_acc);
  a.topk_idx = topk_idx;
  a.tokens_per_rank = tokens_per_rank;
  a.tokens_per_expert = tokens_per_expert;
  a.mask = is_token_in_rank;
  a.token_ranks = reinterpret_cast<uint64_t*>(ws + p.token_ranks);
  a.chunk_base = reinterpret_cast<int32_t*>(ws + p.chunk_base);
  a.ws_rank_offsets = reinterpret_cast<int32_t*>(ws + p.rank_offsets);
  a.rank_magic = rank_magic(s);
  a.T = s.num_tokens;
  a.k = s.num_topk;
  a.E = s.num_experts;
  a.R = s.num_ranks;
  a.NC = p.NC;
  a.NB = p.NB;
  a.mask_words = (s.num_ranks % 4 == 0 && aligned(is_token_in_rank, 4)) ? 1 : 0;
  a.mask_shift = mask_shift(s, is_token_in_rank);
  a.ids_vec4 = (s.num_topk % 4 == 0 && aligned(topk_idx, 16)) ? 1 : 0;
  return MOE_OK;
}

void launch_layout(const moe::LayoutArgs& a, hipStream_t stream) {
  const size_t hist_bytes = (size_t)a.E * sizeof(int);
  const bool narrow = a.k <= 8;  // ids held per lane: 8, else the top-k limit
  if (a.T <= moe::kFusedMaxTokens) {
    const int threads = std::max(moe::kWave, (a.T + moe::kWave - 1) / moe::kWave * moe::kWave);
    if (narrow)
      hipLaunchKernelGGL(moe::layout_fused_kernel<8>, dim3(1), dim3(threads), hist_bytes, stream, a);
    else
      hipLaunchKernelGGL(moe::layout_fused_kernel<moe::kMaxTopk>, dim3(1), dim3(threads), hist_bytes, stream, a);
  } else {  // one launch: the count block that finishes last finalises the plan
    if (narrow)
      hipLaunchKernelGGL(moe::layout_count_kernel<8>, dim3(a.NB), dim3(moe::kLayoutBlock), hist_bytes, stream, a);
    else
      hipLaunchKernelGGL(moe::layout_count_kernel<moe::kMaxTopk>, dim3(a.NB), dim3(moe::kLayoutBlock), hist_bytes,
                         stream, a);
  }
}

// Dispatch arguments after every check moe_dispatch makes (shape already checked); U is the
// slice width the launch uses.
moe_status dispatch_args(const moe_shape& s, moe_dtype dtype, const void* x, const int32_t* topk_idx,
                         const float* topk_w, const void* workspace, size_t workspace_bytes, int32_t recv_capacity,
                         void* recv_x, float* recv_scales, int32_t* recv_src_idx, int32_t* recv_topk_idx,
                         float* recv_topk_w, int32_t* rank_offsets, int32_t* send_row, int32_t* num_recv,
                         moe::DispatchArgs& a, int& U) {
  if (dtype != MOE_BF16 && dtype != MOE_FP8_E4M3) return MOE_ERR_INVALID_ARG;
  const bool fp8 = dtype == MOE_FP8_E4M3;
  if (fp8 && s.hidden % moe::kFp8Block != 0) return MOE_ERR_INVALID_ARG;
  const int64_t T = s.num_tokens, cap = recv_capacity;
  if (!present(x, T) || !present(topk_idx, T) || !present(topk_w, T) || !present(send_row, T) || !workspace ||
      !present(recv_x, cap) || !present(recv_src_idx, cap) || !present(recv_topk_idx, cap) ||
      !present(recv_topk_w, cap) || (fp8 && !present(recv_scales, cap)) || !rank_offsets || !num_recv)
    return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(recv_x, 16) || !aligned(topk_idx, 4) || !aligned(topk_w, 4) ||
      !aligned(workspace, kPlanAlign) || !aligned(recv_src_idx, 4) || !aligned(recv_topk_idx, 4) ||
      !aligned(recv_topk_w, 4) || !aligned(rank_offsets, 4) || !aligned(send_row, 4) ||
      !aligned(num_recv, 4) || (fp8 && !aligned(recv_scales, 4)))
    return MOE_ERR_INVALID_ARG;
  const PlanLayout p = plan_layout(s);
  if (workspace_bytes < p.total) return MOE_ERR_INVALID_ARG;
  if (recv_capacity < 0) return MOE_ERR_INVALID_ARG;
  if (recv_capacity < s.num_tokens * std::min(s.num_topk, s.num_ranks)) return MOE_ERR_CAPACITY;

  const char* ws = static_cast<const char*>(workspace);
  a = moe::DispatchArgs{};
  a.x = static_cast<const uint16_t*>(x);
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.token_ranks = reinterpret_cast<const uint64_t*>(ws + p.token_ranks);
  a.chunk_base = reinterpret_cast<const int32_t*>(ws + p.chunk_base);
  a.ws_rank_offsets = reinterpret_cast<const int32_t*>(ws + p.rank_offsets);
  a.recv_x = recv_x;
  a.recv_scales = recv_scales;
  a.recv_src_idx = recv_src_idx;
  a.recv_topk_idx = recv_topk_idx;
  a.recv_topk_w = recv_topk_w;
  a.rank_offsets = rank_offsets;
  a.send_row = send_row;
  a.num_recv = num_recv;
  a.rank_magic = rank_magic(s);
  a.rank_bits = s.num_ranks == 64 ? ~0ull : ((1ull << s.num_ranks) - 1);
  a.T = s.num_tokens;
  a.H = s.hidden;
  a.H8 = s.hidden / 8;
  a.k = s.num_topk;
  a.E = s.num_experts;
  a.R = s.num_ranks;
  a.L = s.num_experts / s.num_ranks;
  a.NC = p.NC;
  a.capacity = recv_capacity;
#ifdef MOE_FORCE_DISPATCH_U
  U = MOE_FORCE_DISPATCH_U;
#else
  U = pick_dispatch_chunks_per_lane(s.num_tokens, a.H8, fp8);
#endif
  const int groups = (a.H8 + moe::kWave - 1) / moe::kWave;
  a.slices = (groups + U - 1) / U;
  if ((int64_t)s.num_tokens * a.slices > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  a.items = s.num_tokens * a.slices;
  return MOE_OK;
}

void launch_dispatch_args(const moe::DispatchArgs& a, int U, bool fp8, hipStream_t stream) {
  const int waves_per_block = moe::kDispatchBlock / moe::kWave;
  const dim3 grid(std::max(1, (a.items + waves_per_block - 1) / waves_per_block));
  if (fp8)
    launch_dispatch<true>(U, grid, stream, a);
  else
    launch_dispatch<false>(U, grid, stream, a);
}

template <int U>
void launch_send_small_t(bool fp8, bool narrow, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                         const moe::SendSmallArgs& a) {
  if (fp8 && narrow)
    hipLaunchKernelGGL((moe::send_small_kernel<U, true, 8>), grid, block, lds, stream, a);
  else if (fp8)
    hipLaunchKernelGGL((moe::send_small_kernel<U, true, moe::kMaxTopk>), grid, block, lds, stream, a);
  else if (narrow)
    hipLaunchKernelGGL((moe::send_small_kernel<U, false, 8>), grid, block, lds, stream, a);
  else
    hipLaunchKernelGGL((moe::send_small_kernel<U, false, moe::kMaxTopk>), grid, block, lds, stream, a);
}

// Layout and dispatch in one launch (T <= 1024, hidden <= 16384): returns false when the
// batch is outside that range and nothing was launched.
bool launch_send_small(const moe::LayoutArgs& lay, const moe::DispatchArgs& d, bool fp8, hipStream_t stream) {
  if (!MOE_SEND_SMALL || d.T > moe::kSendSmallMaxTokens) return false;
  const int groups = (d.H8 + moe::kWave - 1) / moe::kWave;
  const int U = groups <= moe::kSendSmallMaxWaves ? 1 : groups <= 2 * moe::kSendSmallMaxWaves ? 2 : 0;
  if (U == 0) return false;
  moe::SendSmallArgs a{lay, d};
  a.d.slices = (groups + U - 1) / U;
  a.d.items = d.T * a.d.slices;
  const int waves = std::max({a.d.slices, (d.T + moe::kWave - 1) / moe::kWave, 1});
  const dim3 grid(d.T + 1), block(waves * moe::kWave);
  const size_t lds = (size_t)lay.E * sizeof(int);
  const bool narrow = d.k <= 8;  // ids held per lane: 8, else the top-k limit
  if (U == 1)
    launch_send_small_t<1>(fp8, narrow, grid, block, lds, stream, a);
  else
    launch_send_small_t<2>(fp8, narrow, grid, block, lds, stream, a);
  return true;
}

// Router arguments after every check moe_route_layout makes (shape already checked).
moe_status route_args(const moe_shape& s, const moe_router* router, const float* logits, int32_t* topk_idx,
                      float* topk_w, int32_t* tokens_per_rank, int32_t* tokens_per_expert, uint8_t* is_token_in_rank,
                      void* workspace, size_t workspace_bytes, moe::RouterArgs& a) {
  if (router == nullptr) return MOE_ERR_INVALID_ARG;
  const int64_t T = s.num_tokens;
  const int E = s.num_experts, k = s.num_topk, G = router->num_groups, KG = router->topk_groups;
  if (router->gate != MOE_GATE_SOFTMAX && router->gate != MOE_GATE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (G < 1 || KG < 1 || KG > G) return MOE_ERR_INVALID_ARG;
  if (E % 8 != 0 || k > moe::kRouterMaxK) return MOE_ERR_UNSUPPORTED;
  if (G != 1 && G != 2 && G != 4 && G != 8) return MOE_ERR_UNSUPPORTED;
  if (E % G != 0 || k > KG * (E / G)) return MOE_ERR_INVALID_ARG;
  if (!present(logits, T) || !present(topk_idx, T) || !present(topk_w, T) || !present(is_token_in_rank, T) ||
      !tokens_per_rank || !tokens_per_expert || !workspace)
    return MOE_ERR_INVALID_ARG;
  if (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4) || !aligned(tokens_per_rank, 4) ||
      !aligned(tokens_per_expert, 4) || !aligned(workspace, kPlanAlign))
    return MOE_ERR_INVALID_ARG;
  const PlanLayout p = plan_layout(s);
  if (workspace_bytes < p.total) return MOE_ERR_INVALID_ARG;

  char* ws = static_cast<char*>(workspace);
  a = moe::RouterArgs{};
  a.lay.sync = reinterpret_cast<moe::SyncWords*>(ws + p.sync);
  a.lay.expert_acc = reinterpret_cast<int32_t*>(ws + p.expert_acc);
  a.lay.rank_acc = reinterpret_cast<int32_t*>(ws + p.rank_acc);
  a.logits = logits;
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.lay.topk_idx = topk_idx;
  a.lay.tokens_per_rank = tokens_per_rank;
  a.lay.tokens_per_expert = tokens_per_expert;
  a.lay.mask = is_token_in_rank;
  a.lay.token_ranks = reinterpret_cast<uint64_t*>(ws + p.token_ranks);
  a.lay.chunk_base = reinterpret_cast<int32_t*>(ws + p.chunk_base);
  a.lay.ws_rank_offsets = reinterpret_cast<int32_t*>(ws + p.rank_offsets);
  a.lay.rank_magic = rank_magic(s);
  a.lay.T = s.num_tokens;
  a.lay.k = k;
  a.lay.E = E;
  a.lay.R = s.num_ranks;
  a.lay.NC = p.NC;
  a.lay.NB = p.NC;  // one routing block per 64-token chunk
  a.lay.mask_words = (s.num_ranks % 4 == 0 && aligned(is_token_in_rank, 4)) ? 1 : 0;
  a.lay.mask_shift = mask_shift(s, is_token_in_rank);
  a.lay.ids_vec4 = (k % 4 == 0 && aligned(topk_idx, 16)) ? 1 : 0;  // the layout kernel's reads of the ids
  a.V = E % 16 == 0 ? E / 16 : E / 8;  // experts per lane: 16 or 8 lanes per token
  a.G = G;
  a.KG = KG;
  a.sigmoid = router->gate == MOE_GATE_SIGMOID ? 1 : 0;
  a.vec4 = (a.V % 4 == 0 && aligned(logits, 16)) ? 1 : 0;
  return MOE_OK;
}

void launch_router_any(const moe::RouterArgs& a, hipStream_t stream) {
  const size_t lds = (size_t)a.lay.E * sizeof(int);
  if (a.lay.E % 16 == 0)  // 16 lanes per token, one slot per lane
    launch_router<16, 1>(a.lay.T, lds, stream, a);
  else if (a.lay.k <= 8)
    launch_router<8, 1>(a.lay.T, lds, stream, a);
  else
    launch_router<8, 2>(a.lay.T, lds, stream, a);
}

// Routing, layout and dispatch in one launch (route_dispatch_kernel).
#ifndef MOE_FUSED_ROUTE
#define MOE_FUSED_ROUTE 1
#endif

template <int P, int KS, bool kFp8>
void launch_route_dispatch_t(int U, dim3 grid, hipStream_t stream, const moe::FusedSendArgs& f) {
  const dim3 block(moe::kFusedWaves * moe::kWave);
  if (U == 2)
    hipLaunchKernelGGL((moe::route_dispatch_kernel<P, KS, 2, kFp8>), grid, block, 0, stream, f);
  else
    hipLaunchKernelGGL((moe::route_dispatch_kernel<P, KS, 1, kFp8>), grid, block, 0, stream, f);
}

// 1 <= T <= 1024: the routing blocks (16 or 32 tokens each) and the dispatch
// blocks of one launch; returns false (nothing launched) outside that range.
// Dispatch slices are one or two 64-lane groups of 16-byte pieces.
bool launch_route_dispatch(moe::RouterArgs r, moe::DispatchArgs d, bool fp8, hipStream_t stream) {
  const int T = d.T;
  if (!MOE_FUSED_ROUTE || T < 1 || T > moe::kFusedMaxTokens) return false;
  const int P = r.lay.E % 16 == 0 ? 16 : 8;
  const int KS = (P == 8 && r.lay.k > 8) ? 2 : 1;
  const int groups = (d.H8 + moe::kWave - 1) / moe::kWave;
  const int U = (fp8 && groups >= 2 && (long)T * ((groups + 1) / 2) >= kMinFp8Waves) ? 2 : 1;
  d.slices = (groups + U - 1) / U;
  d.items = T * d.slices;
  r.lay.out_rank_offsets = d.rank_offsets;
  r.lay.out_num_recv = d.num_recv;
  moe::FusedSendArgs f{r, d, 0};
  const int tokens_per_producer = moe::kRouterSmallWaves * moe::kWave / P;
  f.producers = (T + tokens_per_producer - 1) / tokens_per_producer;
  const dim3 grid(f.producers + (d.items + moe::kFusedWaves - 1) / moe::kFusedWaves);
  if (P == 16 && fp8) launch_route_dispatch_t<16, 1, true>(U, grid, stream, f);
  else if (P == 16) launch_route_dispatch_t<16, 1, false>(U, grid, stream, f);
  else if (KS == 1 && fp8) launch_route_dispatch_t<8, 1, true>(U, grid, stream, f);
  else if (KS == 1) launch_route_dispatch_t<8, 1, false>(U, grid, stream, f);
  else if (fp8) launch_route_dispatch_t<8, 2, true>(U, grid, stream, f);
  else launch_route_dispatch_t<8, 2, false>(U, grid, stream, f);
  return true;
}

// Device memory of moe_layout_dispatch_noalloc: the plan (workspace) kept in a
// file-scope array, for callers that cannot allocate.  Every device the library
// runs on holds its own copy until the process ends.  Static device memory is
// zero-filled when the code object is loaded, and every launch leaves the
// plan's sync words and accumulators zero again, as a caller-allocated
// workspace requires.  In host code the name `scratch` is only a host-side
// stand-in: its device address comes from hipGetSymbolAddress, once per
// device (scratch_ptr), and only that address is passed to kernels.
constexpr size_t kScratchBytes = 4u << 20;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

// Address of this device's `scratch`, looked up on the first call on each
// device; nullptr if the lookup fails.
void* scratch_ptr() {
  static std::atomic<void*> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  void* p = cached[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
    (void)hipGetLastError();
    return nullptr;
  }
  cached[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_CAPACITY: return "MOE_ERR_CAPACITY";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: break;  // MOE_STATUS_MAX_ENUM and any other value
  }
  return "MOE_ERR_UNKNOWN";
}

size_t moe_workspace_bytes(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  return plan_layout(*shape).total;
}

int32_t moe_max_recv_rows(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return -1;
  return shape->num_tokens * std::min(shape->num_topk, shape->num_ranks);
}

moe_status moe_get_dispatch_layout(const moe_shape* shape, const int32_t* topk_idx,
                                   int32_t* tokens_per_rank, int32_t* tokens_per_expert,
                                   uint8_t* is_token_in_rank, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  moe::LayoutArgs a;
  st = layout_args(*shape, topk_idx, tokens_per_rank, tokens_per_expert, is_token_in_rank, workspace,
                   workspace_bytes, a);
  if (st != MOE_OK) return st;
  launch_layout(a, stream);
  return last_launch_status();
}

moe_status moe_route_layout(const moe_shape* shape, const moe_router* router, const float* logits,
                            int32_t* topk_idx, float* topk_w, int32_t* tokens_per_rank,
                            int32_t* tokens_per_expert, uint8_t* is_token_in_rank, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  moe::RouterArgs a;
  st = route_args(*shape, router, logits, topk_idx, topk_w, tokens_per_rank, tokens_per_expert, is_token_in_rank,
                  workspace, workspace_bytes, a);
  if (st != MOE_OK) return st;
  launch_router_any(a, stream);
  return last_launch_status();
}

moe_status moe_route_dispatch(const moe_shape* shape, const moe_router* router, moe_dtype dtype, const float* logits,
                              const void* x, int32_t* topk_idx, float* topk_w, int32_t* tokens_per_rank,
                              int32_t* tokens_per_expert, uint8_t* is_token_in_rank, void* workspace,
                              size_t workspace_bytes, int32_t recv_capacity, void* recv_x, float* recv_scales,
                              int32_t* recv_src_idx, int32_t* recv_topk_idx, float* recv_topk_w,
                              int32_t* rank_offsets, int32_t* send_row, int32_t* num_recv, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  moe::RouterArgs r;
  st = route_args(*shape, router, logits, topk_idx, topk_w, tokens_per_rank, tokens_per_expert, is_token_in_rank,
                  workspace, workspace_bytes, r);
  if (st != MOE_OK) return st;
  moe::DispatchArgs d;
  int U = 1;
  st = dispatch_args(*shape, dtype, x, topk_idx, topk_w, workspace, workspace_bytes, recv_capacity, recv_x,
                     recv_scales, recv_src_idx, recv_topk_idx, recv_topk_w, rank_offsets, send_row, num_recv, d, U);
  if (st != MOE_OK) return st;
  const bool fp8 = dtype == MOE_FP8_E4M3;
  if (!launch_route_dispatch(r, d, fp8, stream)) {
    launch_router_any(r, stream);
    launch_dispatch_args(d, U, fp8, stream);
  }
  return last_launch_status();
}

moe_status moe_dispatch(const moe_shape* shape, moe_dtype dtype, const void* x,
                        const int32_t* topk_idx, const float* topk_w, const void* workspace,
                        size_t workspace_bytes, int32_t recv_capacity, void* recv_x,
                        float* recv_scales, int32_t* recv_src_idx, int32_t* recv_topk_idx,
                        float* recv_topk_w, int32_t* rank_offsets, int32_t* send_row,
                        int32_t* num_recv, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  moe::DispatchArgs a;
  int U = 1;
  st = dispatch_args(*shape, dtype, x, topk_idx, topk_w, workspace, workspace_bytes, recv_capacity, recv_x,
                     recv_scales, recv_src_idx, recv_topk_idx, recv_topk_w, rank_offsets, send_row, num_recv, a, U);
  if (st != MOE_OK) return st;
  launch_dispatch_args(a, U, dtype == MOE_FP8_E4M3, stream);
  return last_launch_status();
}

moe_status moe_layout_dispatch(const moe_shape* shape, moe_dtype dtype, const void* x, const int32_t* topk_idx,
                               const float* topk_w, int32_t* tokens_per_rank, int32_t* tokens_per_expert,
                               uint8_t* is_token_in_rank, void* workspace, size_t workspace_bytes,
                               int32_t recv_capacity, void* recv_x, float* recv_scales, int32_t* recv_src_idx,
                               int32_t* recv_topk_idx, float* recv_topk_w, int32_t* rank_offsets,
                               int32_t* send_row, int32_t* num_recv, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  moe::LayoutArgs lay;
  st = layout_args(*shape, topk_idx, tokens_per_rank, tokens_per_expert, is_token_in_rank, workspace,
                   workspace_bytes, lay);
  if (st != MOE_OK) return st;
  moe::DispatchArgs d;
  int U = 1;
  st = dispatch_args(*shape, dtype, x, topk_idx, topk_w, workspace, workspace_bytes, recv_capacity, recv_x,
                     recv_scales, recv_src_idx, recv_topk_idx, recv_topk_w, rank_offsets, send_row, num_recv, d, U);
  if (st != MOE_OK) return st;
  const bool fp8 = dtype == MOE_FP8_E4M3;
  if (!launch_send_small(lay, d, fp8, stream)) {
    launch_layout(lay, stream);
    launch_dispatch_args(d, U, fp8, stream);
  }
  return last_launch_status();
}

moe_status moe_layout_dispatch_noalloc(const moe_shape* shape, moe_dtype dtype, const void* x,
                                       const int32_t* topk_idx, const float* topk_w, int32_t* tokens_per_rank,
                                       int32_t* tokens_per_expert, uint8_t* is_token_in_rank, int32_t recv_capacity,
                                       void* recv_x, float* recv_scales, int32_t* recv_src_idx,
                                       int32_t* recv_topk_idx, float* recv_topk_w, int32_t* rank_offsets,
                                       int32_t* send_row, int32_t* num_recv, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (plan_layout(*shape).total > kScratchBytes) return MOE_ERR_UNSUPPORTED;
  // every argument check of moe_layout_dispatch first (with a stand-in address
  // if the array's address is unavailable), so errors are reported alike
  void* ws = scratch_ptr();
  void* ws_checked = ws != nullptr ? ws : reinterpret_cast<void*>(kPlanAlign);
  moe::LayoutArgs lay;
  st = layout_args(*shape, topk_idx, tokens_per_rank, tokens_per_expert, is_token_in_rank, ws_checked, kScratchBytes,
                   lay);
  if (st != MOE_OK) return st;
  moe::DispatchArgs d;
  int U = 1;
  st = dispatch_args(*shape, dtype, x, topk_idx, topk_w, ws_checked, kScratchBytes, recv_capacity, recv_x,
                     recv_scales, recv_src_idx, recv_topk_idx, recv_topk_w, rank_offsets, send_row, num_recv, d, U);
  if (st != MOE_OK) return st;
  if (ws == nullptr) return MOE_ERR_HIP;
  return moe_layout_dispatch(shape, dtype, x, topk_idx, topk_w, tokens_per_rank, tokens_per_expert,
                             is_token_in_rank, ws, kScratchBytes, recv_capacity, recv_x, recv_scales, recv_src_idx,
                             recv_topk_idx, recv_topk_w, rank_offsets, send_row, num_recv, stream);
}

moe_status moe_combine(const moe_shape* shape, const void* y, int32_t num_y_rows,
                       const int32_t* topk_idx, const float* topk_w, const int32_t* send_row,
                       void* out, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape s = *shape;
  if (num_y_rows < 0) return MOE_ERR_INVALID_ARG;
  const int64_t T = s.num_tokens;
  if (!present(y, num_y_rows) || !present(topk_idx, T) || !present(topk_w, T) || !present(send_row, T) ||
      !present(out, T))
    return MOE_ERR_INVALID_ARG;
  if (!aligned(y, 16) || !aligned(out, 16) || !aligned(topk_idx, 4) || !aligned(topk_w, 4) ||
      !aligned(send_row, 4))
    return MOE_ERR_INVALID_ARG;
  if (s.num_tokens == 0) return MOE_OK;

  moe::CombineArgs a{};
  a.y = static_cast<const uint16_t*>(y);
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.send_row = send_row;
  a.out = static_cast<uint16_t*>(out);
  a.rank_magic = rank_magic(s);
  a.T = s.num_tokens;
  a.H = s.hidden;
  a.H8 = s.hidden / 8;
  a.k = s.num_topk;
  a.E = s.num_experts;
  a.R = s.num_ranks;
  a.num_y_rows = num_y_rows;
  return launch_combine<moe::kRankSlots>(a, out, stream);
}

size_t moe_ll_workspace_bytes(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  return ll_plan_layout(*shape).total;
}

moe_status moe_dispatch_ll(const moe_shape* shape, moe_dtype dtype, const void* x, const int32_t* topk_idx,
                           void* workspace, size_t workspace_bytes, int32_t expert_capacity, void* recv_x,
                           float* recv_scales, int32_t* recv_src_idx, int32_t* recv_count, int32_t* slot_pos,
                           hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape s = *shape;
  if (dtype != MOE_BF16 && dtype != MOE_FP8_E4M3) return MOE_ERR_INVALID_ARG;
  const bool fp8 = dtype == MOE_FP8_E4M3;
  if (fp8 && s.hidden % moe::kFp8Block != 0) return MOE_ERR_INVALID_ARG;
  if (expert_capacity < 0) return MOE_ERR_INVALID_ARG;
  if (expert_capacity < s.num_tokens) return MOE_ERR_CAPACITY;
  const int64_t T = s.num_tokens, rows = (int64_t)s.num_experts * expert_capacity;
  if (rows > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (!present(x, T) || !present(topk_idx, T) || !present(slot_pos, T) || !workspace || !recv_count ||
      !present(recv_x, rows) || !present(recv_src_idx, rows) || (fp8 && !present(recv_scales, rows)))
    return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(recv_x, 16) || !aligned(topk_idx, 4) || !aligned(workspace, kPlanAlign) ||
      !aligned(recv_src_idx, 4) || !aligned(recv_count, 4) || !aligned(slot_pos, 4) ||
      (fp8 && !aligned(recv_scales, 4)))
    return MOE_ERR_INVALID_ARG;
  const LlPlanLayout p = ll_plan_layout(s);
  if (workspace_bytes < p.total) return MOE_ERR_INVALID_ARG;

  moe::LlDispatchArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.topk_idx = topk_idx;
  a.recv_x = recv_x;
  a.recv_scales = recv_scales;
  a.recv_src_idx = recv_src_idx;
  a.slot_pos = slot_pos;
  a.T = s.num_tokens;
  a.H = s.hidden;
  a.H8 = s.hidden / 8;
  a.k = s.num_topk;
  a.E = s.num_experts;
  a.NC = p.NC;
  a.cap = expert_capacity;
#if MOE_LL_SMALL
  {  // small batch: one launch, one block per token (hidden up to 16384: 16 waves of 2 x 512 channels)
    const int groups = (a.H8 + moe::kWave - 1) / moe::kWave;
    const int U = groups <= moe::kLlSmallMaxWaves ? 1 : groups <= 2 * moe::kLlSmallMaxWaves ? 2 : 0;
    if (s.num_tokens <= moe::kLlSmallMaxTokens && U > 0) {
      const int waves = std::max({(groups + U - 1) / U, (s.num_tokens + moe::kWave - 1) / moe::kWave, 1});
      a.slices = (groups + U - 1) / U;
      a.items = s.num_tokens * a.slices;
      launch_ll_small(U, fp8, dim3(s.num_tokens + 1), dim3(waves * moe::kWave), stream, a, recv_count);
      return last_launch_status();
    }
  }
#endif

  char* ws = static_cast<char*>(workspace);
  moe::LlLayoutArgs la{};
  la.topk_idx = topk_idx;
  la.slot_local = reinterpret_cast<int32_t*>(ws + p.slot_local);
  la.chunk_base = reinterpret_cast<int32_t*>(ws + p.chunk_base);
  la.recv_count = recv_count;
  la.T = s.num_tokens;
  la.k = s.num_topk;
  la.E = s.num_experts;
  la.NC = p.NC;
  const int nwaves = std::max(1, p.NC);
  const size_t fused_lds = (size_t)nwaves * s.num_experts * sizeof(unsigned long long);
  if (s.num_tokens <= moe::kLlFusedMaxTokens && fused_lds <= 64 * 1024) {
    hipLaunchKernelGGL(moe::ll_layout_fused_kernel, dim3(1), dim3(nwaves * moe::kWave), fused_lds, stream, la);
  } else {
    hipLaunchKernelGGL(moe::ll_count_kernel, dim3(p.NC), dim3(moe::kWave),
                       (size_t)s.num_experts * sizeof(unsigned long long), stream, la);
    hipLaunchKernelGGL(moe::ll_scan_kernel, dim3((s.num_experts + 3) / 4), dim3(256), 0, stream, la);
  }
  st = last_launch_status();
  if (st != MOE_OK || s.num_tokens == 0) return st;

  a.slot_local = la.slot_local;
  a.chunk_base = la.chunk_base;
  const int U = pick_dispatch_chunks_per_lane(s.num_tokens, a.H8, fp8);
  const int groups = (a.H8 + moe::kWave - 1) / moe::kWave;
  a.slices = (groups + U - 1) / U;
  if ((int64_t)s.num_tokens * a.slices > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  a.items = s.num_tokens * a.slices;
  const int waves_per_block = moe::kDispatchBlock / moe::kWave;
  const dim3 grid((a.items + waves_per_block - 1) / waves_per_block);
  if (fp8)
    launch_ll_dispatch<true>(U, grid, stream, a);
  else
    launch_ll_dispatch<false>(U, grid, stream, a);
  return last_launch_status();
}

moe_status moe_encode_e4m3(const float* values, uint8_t* codes, int64_t n, hipStream_t stream) {
  if (n < 0 || ((!values || !codes) && n > 0)) return MOE_ERR_INVALID_ARG;
  if (n == 0) return MOE_OK;
  const int64_t blocks = (n + 1023) / 1024;  // 256 threads of 4 values
  if (blocks > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(moe::encode_e4m3_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, values, codes, n);
  return last_launch_status();
}

moe_status moe_combine_ll(const moe_shape* shape, const void* y, int32_t expert_capacity, const int32_t* topk_idx,
                          const float* topk_w, const int32_t* slot_pos, void* out, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape s = *shape;
  if (expert_capacity < 0) return MOE_ERR_INVALID_ARG;
  const int64_t T = s.num_tokens, rows = (int64_t)s.num_experts * expert_capacity;
  if (rows > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (!present(y, rows) || !present(topk_idx, T) || !present(topk_w, T) || !present(slot_pos, T) ||
      !present(out, T))
    return MOE_ERR_INVALID_ARG;
  if (!aligned(y, 16) || !aligned(out, 16) || !aligned(topk_idx, 4) || !aligned(topk_w, 4) ||
      !aligned(slot_pos, 4))
    return MOE_ERR_INVALID_ARG;
  if (s.num_tokens == 0) return MOE_OK;

  moe::CombineArgs a{};
  a.y = static_cast<const uint16_t*>(y);
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.slot_pos = slot_pos;
  a.out = static_cast<uint16_t*>(out);
  a.T = s.num_tokens;
  a.H = s.hidden;
  a.H8 = s.hidden / 8;
  a.k = s.num_topk;
  a.E = s.num_experts;
  a.R = s.num_ranks;
  a.cap = expert_capacity;
  a.num_y_rows = (int)rows;
  return launch_combine<moe::kExpertSlots>(a, out, stream);
}

moe_status moe_combine_backward(const moe_shape* shape, const void* grad_out, const void* y, int32_t num_y_rows,
                                const int32_t* topk_idx, const float* topk_w, const int32_t* send_row,
                                void* grad_y, float* grad_topk_w, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape s = *shape;
  if (num_y_rows < 0) return MOE_ERR_INVALID_ARG;
  const int64_t T = s.num_tokens;
  if (!present(grad_out, T) || !present(y, num_y_rows) || !present(topk_idx, T) || !present(topk_w, T) ||
      !present(send_row, T) || !present(grad_y, num_y_rows) || !present(grad_topk_w, T))
    return MOE_ERR_INVALID_ARG;
  if (!aligned(grad_out, 16) || !aligned(y, 16) || !aligned(grad_y, 16) || !aligned(topk_idx, 4) ||
      !aligned(topk_w, 4) || !aligned(send_row, 4) || !aligned(grad_topk_w, 4))
    return MOE_ERR_INVALID_ARG;
  if (s.num_tokens == 0) return MOE_OK;
  if (num_y_rows == 0) {  // no expert rows: grad_y has no row to write and every weight gradient is +0
    const size_t n = (size_t)s.num_tokens * s.num_topk;
    const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(zero_fill_f32_kernel, dim3(blocks), dim3(256), 0, stream, grad_topk_w, n);
    return last_launch_status();
  }

  moe::CombineBwdArgs a{};
  a.g = static_cast<const uint16_t*>(grad_out);
  a.y = static_cast<const uint16_t*>(y);
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.send_row = send_row;
  a.grad_y = static_cast<uint16_t*>(grad_y);
  a.grad_w = grad_topk_w;
  a.rank_magic = rank_magic(s);
  a.T = s.num_tokens;
  a.H = s.hidden;
  a.H8 = s.hidden / 8;
  a.k = s.num_topk;
  a.E = s.num_experts;
  a.R = s.num_ranks;
  a.num_y_rows = num_y_rows;
  const int slices = (a.H8 + moe::kWave - 1) / moe::kWave;
  const dim3 grid(s.num_tokens), block(std::min(slices, MOE_BWD_WAVES) * moe::kWave);
  if (s.num_topk <= moe::kNarrowTopk)
    hipLaunchKernelGGL(moe::combine_backward_kernel, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(moe::combine_backward_wide_kernel, grid, block, 0, stream, a);
  return last_launch_status();
}

moe_status moe_dispatch_backward(const moe_shape* shape, const void* grad_recv_x, int32_t num_recv_rows,
                                 const float* grad_recv_topk_w, const int32_t* topk_idx, const int32_t* send_row,
                                 void* grad_x, float* grad_topk_w, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape s = *shape;
  if (num_recv_rows < 0) return MOE_ERR_INVALID_ARG;
  if ((grad_recv_topk_w == nullptr) != (grad_topk_w == nullptr)) return MOE_ERR_INVALID_ARG;
  const bool weights = grad_topk_w != nullptr;
  const int64_t T = s.num_tokens;
  if (!present(grad_recv_x, num_recv_rows) || !present(send_row, T) || !present(grad_x, T) ||
      (weights && (!present(topk_idx, T) || !present(grad_recv_topk_w, num_recv_rows))))
    return MOE_ERR_INVALID_ARG;
  if (!aligned(grad_recv_x, 16) || !aligned(grad_x, 16) || !aligned(send_row, 4) || !aligned(topk_idx, 4) ||
      !aligned(grad_recv_topk_w, 4) || !aligned(grad_topk_w, 4))
    return MOE_ERR_INVALID_ARG;
  if (s.num_tokens == 0) return MOE_OK;

  moe::CombineArgs a{};
  a.y = static_cast<const uint16_t*>(grad_recv_x);
  a.send_row = send_row;
  a.out = static_cast<uint16_t*>(grad_x);
  a.T = s.num_tokens;
  a.H = s.hidden;
  a.H8 = s.hidden / 8;
  a.k = s.num_topk;
  a.E = s.num_experts;
  a.R = s.num_ranks;
  a.num_y_rows = num_recv_rows;
  st = launch_combine<moe::kRankRows>(a, grad_x, stream);
  if (st != MOE_OK || !weights) return st;

  moe::WeightGradArgs wa{};
  wa.grad_recv_w = grad_recv_topk_w;
  wa.topk_idx = topk_idx;
  wa.send_row = send_row;
  wa.grad_topk_w = grad_topk_w;
  wa.rank_magic = rank_magic(s);
  wa.T = s.num_tokens;
  wa.k = s.num_topk;
  wa.E = s.num_experts;
  wa.R = s.num_ranks;
  wa.num_rows = num_recv_rows;
  const int64_t n = (int64_t)s.num_tokens * s.num_topk;
  hipLaunchKernelGGL(moe::gather_weight_grad_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, wa);
  return last_launch_status();
}

moe_status moe_stream_create_cu_range(int32_t first_cu, int32_t num_cus, hipStream_t* stream) {
  if (stream == nullptr) return MOE_ERR_INVALID_ARG;
  *stream = nullptr;
  const int cus = device_cu_count(), xcc = device_xcc_count();
  if (first_cu == 0 && (num_cus <= 0 || num_cus >= cus))
    return hipStreamCreateWithFlags(stream, hipStreamNonBlocking) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  if (first_cu < 0 || num_cus <= 0 || first_cu % xcc != 0 || num_cus % xcc != 0 || first_cu + num_cus > cus ||
      (cus + 31) / 32 > kMaxCuMaskWords)
    return MOE_ERR_INVALID_ARG;
  uint32_t mask[kMaxCuMaskWords] = {0};
  for (int i = first_cu; i < first_cu + num_cus; ++i) mask[i / 32] |= 1u << (i % 32);
  if (hipExtStreamCreateWithCUMask(stream, (uint32_t)((cus + 31) / 32), mask) != hipSuccess) {
    (void)hipGetLastError();  // do not leave the failure for the next unrelated call
    *stream = nullptr;
    return MOE_ERR_HIP;
  }
  if (!register_cu_stream(*stream, num_cus)) {  // more than kMaxCuStreams alive at once
    (void)hipStreamDestroy(*stream);
    *stream = nullptr;
    return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

moe_status moe_stream_destroy(hipStream_t stream) {
  if (stream == nullptr) return MOE_ERR_INVALID_ARG;
  unregister_cu_stream(stream);
  return hipStreamDestroy(stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
