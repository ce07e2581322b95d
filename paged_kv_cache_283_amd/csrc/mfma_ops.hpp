// MFMA operand helpers shared by the attention kernels (gfx950).
//
// K tiles feed the A operand of a 16x16x32 (16-bit) or 16x16x4 (f32) MFMA with
// row = token; the query rows feed B with column = (query token, head).  The
// helpers convert and pack operands and name the head dims each lane holds.
#pragma once

#include "device_common.hpp"

namespace pkv {

template <int KVT>
struct KvType {
  static constexpr int kBytes = KVT == DT_F32 ? 4 : (is_code8(KVT) ? 1 : 2);
  static constexpr bool kOp32 = KVT == DT_F32;   // fp32 MFMA operands
  static constexpr bool kOpF16 = KVT == DT_F16;  // f16 MFMA operands (bf16 otherwise)
};

// Convert one float to the 16-bit MFMA operand type, and the residual.
template <bool F16>
__device__ __forceinline__ uint32_t to_op16(float f) {
  if constexpr (F16) return f32_to_f16_bits(f);
  else return f32_to_bf16_rne(f);
}
template <bool F16>
__device__ __forceinline__ float from_op16(uint32_t b) {
  if constexpr (F16) return f16_to_f32(b);
  else return bf16_to_f32(b);
}

template <int QT>
__device__ __forceinline__ float load_q_elem(const void* q, size_t idx) {
  if constexpr (QT == DT_F32) return reinterpret_cast<const float*>(q)[idx];
  else if constexpr (QT == DT_BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(q)[idx]);
  else return f16_to_f32(reinterpret_cast<const uint16_t*>(q)[idx]);
}

template <bool F16>
__device__ __forceinline__ f32x4 mfma_k32(const uint32_t* a, const uint32_t* b, f32x4 c) {
  u32x4 av = {a[0], a[1], a[2], a[3]};
  u32x4 bv = {b[0], b[1], b[2], b[3]};
  if constexpr (F16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av), __builtin_bit_cast(f16x8, bv), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), c, 0, 0, 0);
  }
}

template <bool F16>
__device__ __forceinline__ f32x4 mfma_k32v(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (F16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
}

// Two floats as packed 16-bit MFMA operands: the bf16 high parts (the upper 16
// bits, truncated) and the bf16 truncation of the residuals f - high, so that
// high + low carries about 16 significant bits.  One v_perm_b32 packs each pair.
__device__ __forceinline__ void split_bf16_pair(float f0, float f1, uint32_t& hi, uint32_t& lo) {
  const uint32_t u0 = __float_as_uint(f0), u1 = __float_as_uint(f1);
  hi = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
  const float r0 = f0 - __uint_as_float(u0 & 0xffff0000u);
  const float r1 = f1 - __uint_as_float(u1 & 0xffff0000u);
  lo = __builtin_amdgcn_perm(__float_as_uint(r1), __float_as_uint(r0), 0x07060302u);
}

template <bool F16>
__device__ __forceinline__ f32x4 mfma_k16(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f32x4 c) {
  u32x2 av = {a0, a1};
  u32x2 bv = {b0, b1};
  if constexpr (F16) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, av), __builtin_bit_cast(f16x4, bv), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, av), __builtin_bit_cast(s16x4, bv), c, 0, 0, 0);
  }
}

__device__ __forceinline__ f32x4 mfma_f32_k4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// First head-dim of the 8 consecutive dims row group j contributes to QK step
// st (16-bit and 8-bit K: one 16x16x32 MFMA per step).  With 16-byte K chunks of
// X elements, load u of row group j is chunk 4u + j.
template <int KVT>
__device__ __forceinline__ int qk_dim16(int st, int j) {
  if constexpr (is_code8(KVT)) return (4 * (st / 2) + j) * 16 + 8 * (st % 2);       // X = 16: two steps per chunk
  else return (4 * st + j) * 8;                                               // X = 8: one step per chunk
}
// Head-dim row group j contributes to step st of the fp32 16x16x4 MFMA (X = 4).
__device__ __forceinline__ int qk_dim_f32(int st, int j) { return (4 * (st / 4) + j) * 4 + st % 4; }


}  // namespace pkv
