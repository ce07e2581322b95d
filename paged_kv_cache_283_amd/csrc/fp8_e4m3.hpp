// OCP FP8 E4M3FN encoding for the KV write path (bias 7, largest finite 448,
// no infinities, S.1111.111 = NaN).  Page "KV Cache 与 PagedAttention：显存复用与长上下文推理"
// (plumephp.com/ai-kv-cache-paged-attention), "量化原理": FP16 -> FP8 E4M3 with
// per-token scaling.
//
// Rounding: to nearest, ties to even; magnitudes from 448 up (infinity too)
// saturate to 448 instead of becoming NaN; NaN gives 0x7F.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

__device__ __forceinline__ uint32_t e4m3fn_encode(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float ax = fabsf(x);
  if (ax != ax) return 0x7fu;
  if (ax >= 448.f) return sign | 0x7eu;
  if (ax < 0.015625f) {
    // Below the smallest normal 2^-6 the grid is uniform with step 2^-9:
    // scaling by 512 is exact, rintf rounds half to even; 8 lands on 2^-6 (code 0x08).
    return sign | (uint32_t)rintf(ax * 512.f);
  }
  const uint32_t au = __float_as_uint(ax);
  int exp = (int)(au >> 23) - 127;              // -6 .. 8
  uint32_t man = au & 0x7fffffu;
  uint32_t keep = man >> 20;                    // 3 mantissa bits
  const uint32_t rest = man & 0xfffffu;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ++keep;
  if (keep == 8u) { keep = 0u; ++exp; }
  return sign | ((uint32_t)(exp + 7) << 3) | keep;
}

}  // namespace pkv
