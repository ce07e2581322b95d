// Block swap between the HBM pool and a pinned host arena, for gfx950.
//
// Page "KV Cache 与 PagedAttention：显存复用与长上下文推理", "三大运行时组件": the block
// allocator manages the pool by blocks and can swap them out to CPU RAM; page
// "系统优化" 4.5 "CPU Offloading": the KV of inactive requests waits in CPU
// memory and is loaded back when needed.
//
// One launch moves a batch of (pool block, host slot) pairs: one workgroup
// per pair copies the block's K and V tiles of every KV head (and, for 8-bit
// pools, both scale rows) with 16-byte accesses.  The host arena is pinned,
// device-accessible memory laid out like the pool ([slots][Hkv][tile]), so the
// kernel reads or writes it directly over the host link; no staging copy.
#include "device_common.hpp"
#include "launch.hpp"

namespace pkv {

__global__ void __launch_bounds__(256) kv_swap_kernel(uint8_t* k_pool, uint8_t* v_pool, float* k_scale, float* v_scale,
                                                    uint8_t* host_k, uint8_t* host_v, float* host_ks, float* host_vs,
                                                    const int32_t* pairs, int num_blocks, int host_slots,
                                                    size_t block_bytes, int scale_floats, int to_host) {
  const int pr = blockIdx.x;
  const int blk = pairs[2 * pr], slot = pairs[2 * pr + 1];
  if (blk < 0 || blk >= num_blocks || slot < 0 || slot >= host_slots) return;
  u32x4* pk = reinterpret_cast<u32x4*>(k_pool + (size_t)blk * block_bytes);
  u32x4* pv = reinterpret_cast<u32x4*>(v_pool + (size_t)blk * block_bytes);
  u32x4* hk = reinterpret_cast<u32x4*>(host_k + (size_t)slot * block_bytes);
  u32x4* hv = reinterpret_cast<u32x4*>(host_v + (size_t)slot * block_bytes);
  const size_t n16 = block_bytes / 16;
  if (to_host) {
    for (size_t i = threadIdx.x; i < n16; i += blockDim.x) {
      hk[i] = pk[i];
      hv[i] = pv[i];
    }
  } else {
    for (size_t i = threadIdx.x; i < n16; i += blockDim.x) {
      pk[i] = hk[i];
      pv[i] = hv[i];
    }
  }
  if (k_scale != nullptr) {
    float* ps = k_scale + (size_t)blk * scale_floats;
    float* qs = v_scale + (size_t)blk * scale_floats;
    float* hs = host_ks + (size_t)slot * scale_floats;
    float* gs = host_vs + (size_t)slot * scale_floats;
    for (int i = threadIdx.x; i < scale_floats; i += blockDim.x) {
      if (to_host) {
        hs[i] = ps[i];
        gs[i] = qs[i];
      } else {
        ps[i] = hs[i];
        qs[i] = gs[i];
      }
    }
  }
}

hipError_t launch_kv_swap(void* k_pool, void* v_pool, float* k_scale, float* v_scale, int kv_dtype, void* host_k,
                          void* host_v, float* host_k_scale, float* host_v_scale, const int32_t* pairs, int num_pairs,
                          int num_blocks, int host_slots, int num_kv_heads, int head_dim, int to_host,
                          hipStream_t st) {
  if (num_pairs == 0) return hipSuccess;
  const int eb = kv_dtype == DT_F32 ? 4 : (is_code8(kv_dtype) ? 1 : 2);
  const size_t block_bytes = (size_t)num_kv_heads * kBlockSize * head_dim * eb;
  const bool q = is_quantised(kv_dtype);
  hipLaunchKernelGGL(kv_swap_kernel, dim3(num_pairs), dim3(256), 0, st, reinterpret_cast<uint8_t*>(k_pool),
                     reinterpret_cast<uint8_t*>(v_pool), q ? k_scale : nullptr, q ? v_scale : nullptr,
                     reinterpret_cast<uint8_t*>(host_k), reinterpret_cast<uint8_t*>(host_v),
                     q ? host_k_scale : nullptr, q ? host_v_scale : nullptr, pairs, num_blocks, host_slots,
                     block_bytes, num_kv_heads * kBlockSize, to_host);
  return hipGetLastError();
}

}  // namespace pkv
