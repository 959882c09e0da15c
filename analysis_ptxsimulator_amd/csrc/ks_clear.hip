// ks_clear.hip -- zeroing of device buffers that a run must find cleared (the cache
// model's per-warp state): a kernel of the library's own rather than a memset, so
// that a run can be captured in a HIP graph.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ks_launch.h"

// Zeroes n16 16-byte words at p with a grid-stride loop of 16-byte stores.
__global__ void ks_clear_kernel(uint4* p, uint64_t n16) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

hipError_t ks_launch_clear(void* p, uint64_t bytes, hipStream_t s) {
  if (((uintptr_t)p & 15u) || (bytes & 15u)) return hipErrorInvalidValue;
  const uint64_t n16 = bytes / 16u;
  if (n16 == 0) return hipSuccess;
  uint64_t blocks = (n16 + 255u) / 256u;
  if (blocks > 8192) blocks = 8192;  // 32 workgroups per compute unit, then grid-stride
  hipLaunchKernelGGL(ks_clear_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, (uint4*)p, n16);
  return hipGetLastError();
}
