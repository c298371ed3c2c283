// Achievable HBM bandwidth on this GPU for the access mixes of the library's
// kernels: plain streaming kernels (no gather, no metadata) that read NR and
// write NW equally long streams of 16-byte vectors, swept over grid sizes, over
// nontemporal vs ordinary loads and stores and over the spacing of the streams
// (back to back, or staggered by a little over 1 MiB so that equal offsets do
// not meet on the same HBM channels); the best of each mix is printed as one
// JSON line.  Mixes: read only, write only, copy (1:1),
// 5 reads : 1 write (the combine's mix at top-8 over 8 ranks, ~5.3 rows per
// token), 1 read : 5 writes (the dispatch's) and 5 reads : 5 writes (close to
// the combine backward's: g and the token's rows read, one row per rank written).  A measurement aid, not part
// of the library: bench.py (beside it) reports it next to the kernels' fraction of peak.
//
//   hipcc --offload-arch=gfx950 -O3 hbm_ceiling.hip -o hbm_ceiling && ./hbm_ceiling
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                              \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "HIP error %d at line %d\n", (int)e_, __LINE__);        \
      return 1;                                                               \
    }                                                                         \
  } while (0)

constexpr int kBlock = 256;

// Grid-stride loop over n vectors, U consecutive strides per iteration (all
// of an iteration's loads issued before its stores).  Stream r starts at
// r * pitch (pitch >= n); every access is below NR * pitch (src) or NW * pitch (dst).
template <int NR, int NW, int U, bool NT>
__global__ __launch_bounds__(kBlock) void stream_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        size_t n, size_t pitch, uint32_t* sink) {
  const size_t st = (size_t)gridDim.x * kBlock;
  size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x;
  u32x4 keep = {0u, 0u, 0u, 0u};
  for (; i + (U - 1) * st < n; i += U * st) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      v[u] = u32x4{(uint32_t)i, 1u, 2u, 3u};
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const u32x4* p = src + r * pitch + i + u * st;
        v[u] ^= NT ? __builtin_nontemporal_load(p) : *p;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        u32x4* p = dst + w * pitch + i + u * st;
        if (NT)
          __builtin_nontemporal_store(v[u], p);
        else
          *p = v[u];
      }
      keep ^= v[u];
    }
  }
  for (; i < n; i += st) {  // tail
    u32x4 v = {(uint32_t)i, 1u, 2u, 3u};
    for (int r = 0; r < NR; ++r) v ^= src[r * pitch + i];
    for (int w = 0; w < NW; ++w) dst[w * pitch + i] = v;
    keep ^= v;
  }
  if (NW == 0 && (keep.x ^ keep.y ^ keep.z ^ keep.w) == 0x9e3779b9u) sink[0] = 1u;  // keeps the loads
}

struct Best {
  double gbs = 0;
  int grid = 0;
  bool nt = false;
  size_t pitch = 0;
};

constexpr size_t kStagger = ((size_t)1 << 16) + 256 + 16;  // vectors: 1 MiB + 4 KiB + 256 B

template <int NR, int NW, int U, bool NT>
int sweep(const u32x4* src, u32x4* dst, size_t n, uint32_t* sink, hipEvent_t e0, hipEvent_t e1, Best& best) {
  const int grids[] = {256, 512, 1024, 2048, 4096};
  const size_t pitches[] = {n, n + kStagger};
  const double bytes = 16.0 * (double)n * (NR + NW);
  for (size_t pitch : pitches) {
    for (int g : grids) {
      for (int i = 0; i < 3; ++i)
        hipLaunchKernelGGL((stream_kernel<NR, NW, U, NT>), dim3(g), dim3(kBlock), 0, 0, src, dst, n, pitch, sink);
      CHECK(hipGetLastError());
      CHECK(hipEventRecord(e0, 0));
      for (int i = 0; i < 10; ++i)
        hipLaunchKernelGGL((stream_kernel<NR, NW, U, NT>), dim3(g), dim3(kBlock), 0, 0, src, dst, n, pitch, sink);
      CHECK(hipEventRecord(e1, 0));
      CHECK(hipEventSynchronize(e1));
      float ms = 0;
      CHECK(hipEventElapsedTime(&ms, e0, e1));
      const double gbs = bytes / (ms / 10 * 1e-3) / 1e9;
      if (gbs > best.gbs) best = Best{gbs, g, NT, pitch};
    }
  }
  return 0;
}

template <int NR, int NW, int U>
int measure(const char* name, const u32x4* src, u32x4* dst, size_t n, uint32_t* sink, hipEvent_t e0,
            hipEvent_t e1, bool last) {
  Best best;
  if (sweep<NR, NW, U, false>(src, dst, n, sink, e0, e1, best)) return 1;
  if (sweep<NR, NW, U, true>(src, dst, n, sink, e0, e1, best)) return 1;
  printf("\"%s\": {\"GB_per_s\": %.0f, \"grid\": %d, \"block\": %d, \"nontemporal\": %s, \"staggered\": %s}%s",
         name, best.gbs, best.grid, kBlock, best.nt ? "true" : "false", best.pitch != n ? "true" : "false",
         last ? "" : ", ");
  return 0;
}

int main() {
  const size_t stream_bytes = (size_t)256 << 20;  // 256 MiB per stream: far beyond the 256 MB last-level cache in total
  const size_t n = stream_bytes / 16;
  u32x4 *src, *dst;
  uint32_t* sink;
  const size_t alloc = 5 * (n + kStagger) * 16;  // five streams at the larger pitch
  CHECK(hipMalloc(&src, alloc));
  CHECK(hipMalloc(&dst, alloc));
  CHECK(hipMalloc(&sink, sizeof(uint32_t)));
  CHECK(hipMemset(src, 1, alloc));
  CHECK(hipMemset(dst, 0, alloc));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  printf("{\"stream_MiB\": %zu, ", stream_bytes >> 20);
  if (measure<1, 0, 8>("read", src, dst, n, sink, e0, e1, false)) return 1;
  if (measure<0, 1, 4>("write", src, dst, n, sink, e0, e1, false)) return 1;
  if (measure<1, 1, 4>("copy", src, dst, n, sink, e0, e1, false)) return 1;
  if (measure<5, 1, 2>("read5_write1", src, dst, n, sink, e0, e1, false)) return 1;
  if (measure<1, 5, 2>("read1_write5", src, dst, n, sink, e0, e1, false)) return 1;
  if (measure<5, 5, 1>("read5_write5", src, dst, n, sink, e0, e1, true)) return 1;
  printf("}\n");
  CHECK(hipDeviceSynchronize());
  CHECK(hipFree(src));
  CHECK(hipFree(dst));
  CHECK(hipFree(sink));
  return 0;
}
