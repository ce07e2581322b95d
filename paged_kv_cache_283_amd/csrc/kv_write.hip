// KV-cache maintenance kernels for gfx950: decode slot lookup, token write
// (with FP8 quantisation) and whole-block copy for copy-on-write.
//
// Page "KV Cache 与 PagedAttention：显存复用与长上下文推理" (plumephp.com/ai-kv-cache-paged-attention):
//   "PagedAttention 的设计" -- a token lives in the physical block its sequence's
//     block table names for logical block p / 16, at offset p % 16;
//   "量化原理" -- FP8 (E4M3) or INT8 storage with per-token or per-channel scales;
//   "三大运行时组件" and copy_on_write -- a shared block is copied before a write.
// Pool layout: K [NB][Hkv][D/X][16][X] (16-byte chunks of X elements),
// V [NB][Hkv][D/(16Y)][16][4][Y][4] (16-byte chunks of 4 tokens x Y dims), per-token
// scales [NB][Hkv][16], per-channel scales [Hkv][D] (static, given by the caller).
#include "device_common.hpp"
#include "fp8_e4m3.hpp"
#include "launch.hpp"

namespace pkv {

__global__ void __launch_bounds__(256) decode_slots_kernel(const int32_t* tables, int stride, const int32_t* lens,
                                                         int num_seqs, int num_blocks, int64_t* slots) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= num_seqs) return;
  const int L = lens[s];
  if (L < 1 || L > stride * kBlockSize) { slots[s] = -1; return; }
  const int p = L - 1;
  const int b = tables[(size_t)s * stride + p / kBlockSize];
  slots[s] = (b < 0 || b >= num_blocks) ? (int64_t)-1 : (int64_t)b * kBlockSize + p % kBlockSize;
}

__global__ void __launch_bounds__(256) token_slots_kernel(const int32_t* tables, int stride, int num_seqs,
                                                        const int32_t* seq_ids, const int32_t* positions,
                                                        int num_tokens, int num_blocks, int64_t* slots) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= num_tokens) return;
  const int s = seq_ids[t], p = positions[t];
  if (s < 0 || s >= num_seqs || p < 0 || p >= stride * kBlockSize) { slots[t] = -1; return; }
  const int b = tables[(size_t)s * stride + p / kBlockSize];
  slots[t] = (b < 0 || b >= num_blocks) ? (int64_t)-1 : (int64_t)b * kBlockSize + p % kBlockSize;
}

template <int SRC>
__device__ __forceinline__ float src_to_f32(const void* p, size_t i) {
  if constexpr (SRC == DT_F32) return reinterpret_cast<const float*>(p)[i];
  else if constexpr (SRC == DT_BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  else return f16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
}

// One 8-bit code of the quotient x / scale: E4M3FN (round to nearest even,
// saturating to +-448) or INT8 (nearest integer, ties to even -- v_rndne_f32 --
// saturated to +-127, two's complement).
template <int KVT>
__device__ __forceinline__ uint32_t encode8(float q) {
  if constexpr (code_set(KVT) == DT_INT8) {
    const float r = fminf(fmaxf(__builtin_rintf(q), -127.f), 127.f);
    return (uint32_t)(int32_t)r & 0xffu;
  } else {
    return e4m3fn_encode(q);
  }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
  return x;
}

// Where token t goes: slots[t], or -- for the decode append -- position
// lens[t] - 1 of sequence t through its table row.
struct SlotSource {
  const int64_t* slots;    // non-null: explicit slots
  const int32_t* tables;   // else: decode append
  const int32_t* lens;
  int stride;
};

__device__ __forceinline__ int64_t token_slot(const SlotSource& ss, int t, int num_blocks) {
  if (ss.slots != nullptr) return ss.slots[t];
  const int L = ss.lens[t];
  if (L < 1 || L > ss.stride * kBlockSize) return -1;
  const int b = ss.tables[(size_t)t * ss.stride + (L - 1) / kBlockSize];
  return (b < 0 || b >= num_blocks) ? (int64_t)-1 : (int64_t)b * kBlockSize + (L - 1) % kBlockSize;
}

// One wave per (token, KV head) row; K and V of the row handled together.
template <int SRC, int KVT, int D>
__global__ void __launch_bounds__(256) kv_write_kernel(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                                     float* k_scale, float* v_scale, const SlotSource ss,
                                                     int num_tokens, int num_blocks, int num_kv_heads) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (long)num_tokens * num_kv_heads) return;
  const int t = (int)(row / num_kv_heads);
  const int h = (int)(row % num_kv_heads);
  const int64_t slot = token_slot(ss, t, num_blocks);
  if (slot < 0 || slot >= (int64_t)num_blocks * kBlockSize) return;
  const size_t tile = (size_t)(slot / kBlockSize) * num_kv_heads + h;
  const int o = (int)(slot % kBlockSize);
  const size_t src = (size_t)row * D;
  constexpr int PER = D / 64;
  if constexpr (is_quantised(KVT)) {
    constexpr float kMaxCode = KVT == DT_INT8 ? 127.f : 448.f;
    float kx[PER], vx[PER];
    float kmax = 0.f, vmax = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      kx[e] = src_to_f32<SRC>(k_new, src + e * 64 + lane);
      vx[e] = src_to_f32<SRC>(v_new, src + e * 64 + lane);
      kmax = fmaxf(kmax, fabsf(kx[e]));
      vmax = fmaxf(vmax, fabsf(vx[e]));
    }
    kmax = wave_max(kmax);
    vmax = wave_max(vmax);
    const float ks = __fdiv_rn(kmax, kMaxCode);
    const float vs = __fdiv_rn(vmax, kMaxCode);
    uint8_t* kp = reinterpret_cast<uint8_t*>(k_pool);
    uint8_t* vp = reinterpret_cast<uint8_t*>(v_pool);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int d = e * 64 + lane;
      const uint32_t kc = ks == 0.f ? 0u : encode8<KVT>(__fdiv_rn(kx[e], ks));
      const uint32_t vc = vs == 0.f ? 0u : encode8<KVT>(__fdiv_rn(vx[e], vs));
      kp[tile * kBlockSize * D + k_chunk_offset<1>(o, d)] = (uint8_t)kc;
      vp[tile * kBlockSize * D + v_chunk_offset<1>(o, d)] = (uint8_t)vc;
    }
    if (lane == 0) {
      k_scale[tile * kBlockSize + o] = ks;
      v_scale[tile * kBlockSize + o] = vs;
    }
  } else if constexpr (is_channel_scaled(KVT)) {
    // Static scales [Hkv][D]: the code of x / scale[h][d] (fp32 division).
    uint8_t* kp = reinterpret_cast<uint8_t*>(k_pool);
    uint8_t* vp = reinterpret_cast<uint8_t*>(v_pool);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int d = e * 64 + lane;
      const float kx = src_to_f32<SRC>(k_new, src + d);
      const float vx = src_to_f32<SRC>(v_new, src + d);
      const uint32_t kc = encode8<KVT>(__fdiv_rn(kx, k_scale[(size_t)h * D + d]));
      const uint32_t vc = encode8<KVT>(__fdiv_rn(vx, v_scale[(size_t)h * D + d]));
      kp[tile * kBlockSize * D + k_chunk_offset<1>(o, d)] = (uint8_t)kc;
      vp[tile * kBlockSize * D + v_chunk_offset<1>(o, d)] = (uint8_t)vc;
    }
  } else {
    using T = typename std::conditional<KVT == DT_F32, uint32_t, uint16_t>::type;
    const T* ks = reinterpret_cast<const T*>(k_new);
    const T* vs = reinterpret_cast<const T*>(v_new);
    T* kp = reinterpret_cast<T*>(k_pool);
    T* vp = reinterpret_cast<T*>(v_pool);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int d = e * 64 + lane;
      kp[tile * kBlockSize * D + k_chunk_offset<sizeof(T)>(o, d)] = ks[src + d];
      vp[tile * kBlockSize * D + v_chunk_offset<sizeof(T)>(o, d)] = vs[src + d];
    }
  }
}

// Copy whole blocks src -> dst: K tile, V tile and (per-token FP8/INT8) both scale rows, all KV heads.
__global__ void __launch_bounds__(256) block_copy_kernel(uint8_t* k_pool, uint8_t* v_pool, float* k_scale, float* v_scale,
                                                       const int32_t* pairs, int num_blocks, size_t block_bytes,
                                                       int scale_floats) {
  const int pr = blockIdx.y;
  const int src = pairs[2 * pr], dst = pairs[2 * pr + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
  const size_t n16 = block_bytes / 16;
  const u32x4* ks = reinterpret_cast<const u32x4*>(k_pool + (size_t)src * block_bytes);
  const u32x4* vs = reinterpret_cast<const u32x4*>(v_pool + (size_t)src * block_bytes);
  u32x4* kd = reinterpret_cast<u32x4*>(k_pool + (size_t)dst * block_bytes);
  u32x4* vd = reinterpret_cast<u32x4*>(v_pool + (size_t)dst * block_bytes);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x) {
    kd[i] = ks[i];
    vd[i] = vs[i];
  }
  if (k_scale != nullptr && blockIdx.x == 0) {
    for (int i = threadIdx.x; i < scale_floats; i += blockDim.x) {
      k_scale[(size_t)dst * scale_floats + i] = k_scale[(size_t)src * scale_floats + i];
      v_scale[(size_t)dst * scale_floats + i] = v_scale[(size_t)src * scale_floats + i];
    }
  }
}

namespace {

template <int SRC, int KVT>
hipError_t write_d(const void* k_new, const void* v_new, void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                   const SlotSource& ss, int num_tokens, int num_blocks, int num_kv_heads, int head_dim,
                   hipStream_t st) {
  const long rows = (long)num_tokens * num_kv_heads;
  dim3 grid((unsigned)((rows + 3) / 4));
  if (head_dim == 64)
    hipLaunchKernelGGL((kv_write_kernel<SRC, KVT, 64>), grid, dim3(256), 0, st, k_new, v_new, k_pool, v_pool, k_scale,
                       v_scale, ss, num_tokens, num_blocks, num_kv_heads);
  else
    hipLaunchKernelGGL((kv_write_kernel<SRC, KVT, 128>), grid, dim3(256), 0, st, k_new, v_new, k_pool, v_pool,
                       k_scale, v_scale, ss, num_tokens, num_blocks, num_kv_heads);
  return hipGetLastError();
}

hipError_t write_any(const void* k_new, const void* v_new, int src_dtype, void* k_pool, void* v_pool, float* k_scale,
                     float* v_scale, int kv_dtype, const SlotSource& ss, int num_tokens, int num_blocks,
                     int num_kv_heads, int head_dim, hipStream_t st) {
  if (num_tokens == 0) return hipSuccess;
#define PKV_WRITE(S, K) write_d<S, K>(k_new, v_new, k_pool, v_pool, k_scale, v_scale, ss, num_tokens, num_blocks, \
                                      num_kv_heads, head_dim, st)
  if (kv_dtype == DT_FP8) {
    if (src_dtype == DT_F32) return PKV_WRITE(DT_F32, DT_FP8);
    if (src_dtype == DT_BF16) return PKV_WRITE(DT_BF16, DT_FP8);
    return PKV_WRITE(DT_F16, DT_FP8);
  }
  if (kv_dtype == DT_INT8) {
    if (src_dtype == DT_F32) return PKV_WRITE(DT_F32, DT_INT8);
    if (src_dtype == DT_BF16) return PKV_WRITE(DT_BF16, DT_INT8);
    return PKV_WRITE(DT_F16, DT_INT8);
  }
  if (kv_dtype == DT_FP8_CH) {
    if (src_dtype == DT_F32) return PKV_WRITE(DT_F32, DT_FP8_CH);
    if (src_dtype == DT_BF16) return PKV_WRITE(DT_BF16, DT_FP8_CH);
    return PKV_WRITE(DT_F16, DT_FP8_CH);
  }
  if (kv_dtype == DT_INT8_CH) {
    if (src_dtype == DT_F32) return PKV_WRITE(DT_F32, DT_INT8_CH);
    if (src_dtype == DT_BF16) return PKV_WRITE(DT_BF16, DT_INT8_CH);
    return PKV_WRITE(DT_F16, DT_INT8_CH);
  }
  if (kv_dtype == DT_F32) return PKV_WRITE(DT_F32, DT_F32);
  if (kv_dtype == DT_BF16) return PKV_WRITE(DT_BF16, DT_BF16);
  return PKV_WRITE(DT_F16, DT_F16);
#undef PKV_WRITE
}

}  // namespace

hipError_t launch_decode_slots(const int32_t* tables, int stride, const int32_t* lens, int num_seqs, int num_blocks,
                               int64_t* slots, hipStream_t st) {
  if (num_seqs == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_slots_kernel, dim3((num_seqs + 255) / 256), dim3(256), 0, st, tables, stride, lens,
                     num_seqs, num_blocks, slots);
  return hipGetLastError();
}

hipError_t launch_token_slots(const int32_t* tables, int stride, int num_seqs, const int32_t* seq_ids,
                              const int32_t* positions, int num_tokens, int num_blocks, int64_t* slots,
                              hipStream_t st) {
  if (num_tokens == 0) return hipSuccess;
  hipLaunchKernelGGL(token_slots_kernel, dim3((num_tokens + 255) / 256), dim3(256), 0, st, tables, stride, num_seqs,
                     seq_ids, positions, num_tokens, num_blocks, slots);
  return hipGetLastError();
}

hipError_t launch_kv_write(const void* k_new, const void* v_new, int src_dtype, void* k_pool, void* v_pool,
                           float* k_scale, float* v_scale, int kv_dtype, const int64_t* slots, int num_tokens,
                           int num_blocks, int num_kv_heads, int head_dim, hipStream_t st) {
  const SlotSource ss{slots, nullptr, nullptr, 0};
  return write_any(k_new, v_new, src_dtype, k_pool, v_pool, k_scale, v_scale, kv_dtype, ss, num_tokens, num_blocks,
                   num_kv_heads, head_dim, st);
}

hipError_t launch_kv_append(const void* k_new, const void* v_new, int src_dtype, void* k_pool, void* v_pool,
                            float* k_scale, float* v_scale, int kv_dtype, const int32_t* tables, int stride,
                            const int32_t* lens, int num_seqs, int num_blocks, int num_kv_heads, int head_dim,
                            hipStream_t st) {
  const SlotSource ss{nullptr, tables, lens, stride};
  return write_any(k_new, v_new, src_dtype, k_pool, v_pool, k_scale, v_scale, kv_dtype, ss, num_seqs, num_blocks,
                   num_kv_heads, head_dim, st);
}

hipError_t launch_block_copy(void* k_pool, void* v_pool, float* k_scale, float* v_scale, int kv_dtype,
                             const int32_t* pairs, int num_pairs, int num_blocks, int num_kv_heads, int head_dim,
                             hipStream_t st) {
  if (num_pairs == 0) return hipSuccess;
  const int eb = kv_dtype == DT_F32 ? 4 : (is_code8(kv_dtype) ? 1 : 2);
  const size_t block_bytes = (size_t)num_kv_heads * kBlockSize * head_dim * eb;
  const int scale_floats = num_kv_heads * kBlockSize;
  const unsigned chunks = (unsigned)((block_bytes / 16 + 255) / 256);
  dim3 grid(chunks < 64 ? chunks : 64, num_pairs);
  hipLaunchKernelGGL(block_copy_kernel, grid, dim3(256), 0, st, reinterpret_cast<uint8_t*>(k_pool),
                     reinterpret_cast<uint8_t*>(v_pool), is_quantised(kv_dtype) ? k_scale : nullptr,
                     is_quantised(kv_dtype) ? v_scale : nullptr, pairs, num_blocks, block_bytes, scale_floats);
  return hipGetLastError();
}

}  // namespace pkv
