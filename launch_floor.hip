// The shortest launches on this GPU, as a floor for the latency-bound (decode
// sized) kernels of the library: an empty one-wave kernel, and a one-wave
// kernel whose lane 0 loads one 16-byte value and stores it.  bench.py times
// them beside the decode launches (and rocprofv3 traces them in the same run).
// A measurement aid, not part of the library.
//
//   hipcc --offload-arch=gfx950 -O3 -shared -fPIC launch_floor.hip -o liblaunch_floor.so
#include <hip/hip_runtime.h>

#include <cstdint>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64) void floor_empty_kernel() {}

__global__ __launch_bounds__(64) void floor_load_store_kernel(const u32x4* src, u32x4* dst) {
  if (threadIdx.x == 0) *dst = *src;
}

extern "C" {

// 0 on success, else the HIP error code of the launch.
int floor_empty(hipStream_t stream) {
  hipLaunchKernelGGL(floor_empty_kernel, dim3(1), dim3(64), 0, stream);
  return (int)hipGetLastError();
}

// src, dst: device pointers, 16-byte aligned.
int floor_load_store(const void* src, void* dst, hipStream_t stream) {
  if (src == nullptr || dst == nullptr || (uintptr_t)src % 16 != 0 || (uintptr_t)dst % 16 != 0) return -1;
  hipLaunchKernelGGL(floor_load_store_kernel, dim3(1), dim3(64), 0, stream, static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst));
  return (int)hipGetLastError();
}

}  // extern "C"
