// Element codecs of the KV-cache write (the write kernels and the attention
// kernel's fused append): 8-bit codes of a quotient value / scale, the stored
// bits of a source element, and stores of one element.  Page "KV Cache 与 PagedAttention：显存复用与长上下文推理",
// "量化原理": FP8 (E4M3) or INT8 storage with per-token or per-channel scales.
#pragma once

#include "device_common.hpp"
#include "fp8_e4m3.hpp"

namespace pkv {

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

// Value of a raw source element (16 or 32 bits, zero-extended).
template <int SRC>
__device__ __forceinline__ float raw_to_f32(uint32_t r) {
  if constexpr (SRC == DT_F32) return __uint_as_float(r);
  else if constexpr (SRC == DT_BF16) return bf16_to_f32(r);
  else return f16_to_f32(r);
}

// Stored bits of one element from its raw source bits: the bits themselves
// (pool dtype = source dtype), or the 8-bit code of value / scale, where the
// scale is the row's (per-token formats; 0 gives code 0) or the channel's.
template <int SRC, int KVT>
__device__ __forceinline__ uint32_t stored_code(uint32_t raw, float scale) {
  if constexpr (is_quantised(KVT)) return scale == 0.f ? 0u : encode8<KVT>(__fdiv_rn(raw_to_f32<SRC>(raw), scale));
  else if constexpr (is_channel_scaled(KVT)) return encode8<KVT>(__fdiv_rn(raw_to_f32<SRC>(raw), scale));
  else return raw;
}

template <int SRC>
__device__ __forceinline__ uint32_t load_raw(const void* p, size_t i) {
  if constexpr (SRC == DT_F32) return reinterpret_cast<const uint32_t*>(p)[i];
  else return reinterpret_cast<const uint16_t*>(p)[i];
}

// Maximum over the 64 lanes of the wave.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
  return x;
}

// Largest code magnitude of an 8-bit format (absmax maps to it).
template <int KVT>
constexpr float max_code8() { return code_set(KVT) == DT_INT8 ? 127.f : 448.f; }

template <int EB>
__device__ __forceinline__ void store_elem(uint8_t* dst, uint32_t v) {
  if constexpr (EB == 1) *dst = (uint8_t)v;
  else if constexpr (EB == 2) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)v;
  else *reinterpret_cast<uint32_t*>(dst) = v;
}

}  // namespace pkv
