// Element codecs of the KV-cache write: 8-bit codes of a quotient value / scale
// and stores of one element.  Page "KV Cache 与 PagedAttention：显存复用与长上下文推理",
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

template <int EB>
__device__ __forceinline__ void store_elem(uint8_t* dst, uint32_t v) {
  if constexpr (EB == 1) *dst = (uint8_t)v;
  else if constexpr (EB == 2) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)v;
  else *reinterpret_cast<uint32_t*>(dst) = v;
}

}  // namespace pkv
