// Streaming read and copy probes: the practical HBM ceilings the kernels'
// achieved bandwidth is compared with.  Each workgroup streams one contiguous
// chunk with four independent 16-byte non-temporal loads in flight per thread
// (measured on MI355X: ~7.1 TB/s read, against ~6.0 TB/s for a grid-stride
// loop with one load in flight).
#include "device_common.hpp"
#include "launch.hpp"

namespace pkv {

namespace {
constexpr int kProbeGroups = 2048;   // 8 workgroups of 256 threads per CU
}

__global__ void __launch_bounds__(256) probe_read_kernel(const u32x4* src, size_t n16, float* sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b0 = (size_t)blockIdx.x * per;
  const size_t b1 = b0 + per < n16 ? b0 + per : n16;
  uint32_t x = 0u;
  size_t i = b0 + threadIdx.x;
  for (; i + 3 * 256 < b1; i += 4 * 256) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + 256);
    const u32x4 c = __builtin_nontemporal_load(src + i + 512);
    const u32x4 d = __builtin_nontemporal_load(src + i + 768);
    x ^= a[0] ^ b[1] ^ c[2] ^ d[3];
  }
  for (; i < b1; i += 256) x ^= __builtin_nontemporal_load(src + i)[0];
  // Keeps the loads alive; the value itself is meaningless.
  if (x == 0x9e3779b9u) sink[(blockIdx.x * blockDim.x + threadIdx.x) & 1023] = (float)x;
}

__global__ void __launch_bounds__(256) probe_copy_kernel(u32x4* dst, const u32x4* src, size_t n16) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b0 = (size_t)blockIdx.x * per;
  const size_t b1 = b0 + per < n16 ? b0 + per : n16;
  size_t i = b0 + threadIdx.x;
  for (; i + 3 * 256 < b1; i += 4 * 256) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + 256);
    const u32x4 c = __builtin_nontemporal_load(src + i + 512);
    const u32x4 d = __builtin_nontemporal_load(src + i + 768);
    dst[i] = a;
    dst[i + 256] = b;
    dst[i + 512] = c;
    dst[i + 768] = d;
  }
  for (; i < b1; i += 256) dst[i] = src[i];
}

hipError_t launch_probe_read(const void* src, size_t bytes, float* sink, hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(probe_read_kernel, dim3(kProbeGroups), dim3(256), 0, st, reinterpret_cast<const u32x4*>(src),
                     n16, sink);
  return hipGetLastError();
}

hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(probe_copy_kernel, dim3(kProbeGroups), dim3(256), 0, st, reinterpret_cast<u32x4*>(dst),
                     reinterpret_cast<const u32x4*>(src), n16);
  return hipGetLastError();
}

}  // namespace pkv
