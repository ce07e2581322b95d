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

// gfx950's v_cvt_pk_fp8_f32 converts to OCP E4M3 with round-to-nearest-even,
// subnormals included (checked against the reference encoder on every code
// value, every midpoint between neighbouring codes and the floats adjacent to
// it, and millions of random values); the clamp to +-448 gives the
// saturation, and NaN is mapped to 0x7F first.
__device__ __forceinline__ uint32_t e4m3fn_encode(float x) {
  if (x != x) return 0x7fu;
  const float c = fminf(fmaxf(x, -448.f), 448.f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xffu;
}

}  // namespace pkv
