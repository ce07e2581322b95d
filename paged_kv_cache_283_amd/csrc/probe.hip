// Streaming read and copy probes: the practical HBM ceilings the decode
// kernel's achieved bandwidth is compared with.  Grid-stride, 16-byte accesses.
#include "device_common.hpp"
#include "launch.hpp"

namespace pkv {

__global__ void __launch_bounds__(256) probe_read_kernel(const u32x4* src, size_t n16, float* sink) {
  uint32_t x = 0u;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  // Keeps the loads alive; the value itself is meaningless.
  if (x == 0x9e3779b9u) sink[(blockIdx.x * blockDim.x + threadIdx.x) & 1023] = (float)x;
}

__global__ void __launch_bounds__(256) probe_copy_kernel(u32x4* dst, const u32x4* src, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

hipError_t launch_probe_read(const void* src, size_t bytes, float* sink, hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(probe_read_kernel, dim3(256 * 32), dim3(256), 0, st, reinterpret_cast<const u32x4*>(src), n16,
                     sink);
  return hipGetLastError();
}

hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(probe_copy_kernel, dim3(256 * 32), dim3(256), 0, st, reinterpret_cast<u32x4*>(dst),
                     reinterpret_cast<const u32x4*>(src), n16);
  return hipGetLastError();
}

}  // namespace pkv
