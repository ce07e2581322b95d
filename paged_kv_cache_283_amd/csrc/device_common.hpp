// Device-side helpers shared by the gfx950 kernels: dtype codes, vector types,
// storage conversions and the wave64 cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "geometry.hpp"

namespace pkv {

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2, DT_FP8 = 3, DT_INT8 = 4, DT_FP8_CH = 5, DT_INT8_CH = 6 };

// Storage formats with 8-bit codes and one scale per (token, KV head), stored per block.
__host__ __device__ constexpr bool is_quantised(int kv) { return kv == DT_FP8 || kv == DT_INT8; }
// Storage formats with 8-bit codes and one static scale per (KV head, channel).
__host__ __device__ constexpr bool is_channel_scaled(int kv) { return kv == DT_FP8_CH || kv == DT_INT8_CH; }
// Any 8-bit code format.
__host__ __device__ constexpr bool is_code8(int kv) { return is_quantised(kv) || is_channel_scaled(kv); }
// The code set of an 8-bit format: DT_FP8 (E4M3FN) or DT_INT8.
__host__ __device__ constexpr int code_set(int kv) { return (kv == DT_INT8 || kv == DT_INT8_CH) ? DT_INT8 : DT_FP8; }

constexpr int kWave = 64;          // CDNA wavefront width

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// Element e (0/1) of a word holding two 16-bit values.
__device__ __forceinline__ uint32_t half_word(uint32_t w, int e) { return e ? (w >> 16) : (w & 0xffffu); }

// Four OCP E4M3FN codes (one word) -> four bf16 values (two words; byte 0 in
// the low half of lo), exactly: every E4M3 value is a bf16 value.  The gfx950
// v_cvt_scalef32_pk_bf16_fp8 converts two codes per instruction (scale 1; the
// NaN codes give NaN).
__device__ __forceinline__ void fp8x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}

// Four int8 codes (one word, two's complement) -> four bf16 values code + 128
// (two words; byte 0 in the low half of lo), exactly: 0..255 needs 8
// significant bits.  XOR 0x80 turns each code into the unsigned byte
// code + 128, v_cvt_f32_ubyte* converts it, and one v_perm_b32 per pair keeps
// the two high halves.  The attention kernels take the bias out of their sums
// (q . (c + 128) = q . c + 128 sum q; sum_p P_p (c_p + 128) = sum_p P_p c_p +
// 128 sum_p P_p), so no per-code subtraction is needed.
constexpr float kInt8Bias = 128.f;
__device__ __forceinline__ void int8x4_to_bf16x4_biased(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const uint32_t b = w ^ 0x80808080u;
  const float f0 = (float)(b & 0xffu);
  const float f1 = (float)((b >> 8) & 0xffu);
  const float f2 = (float)((b >> 16) & 0xffu);
  const float f3 = (float)(b >> 24);
  // bytes 2, 3 of src1 then bytes 2, 3 of src0 (src1 is bytes 0-3 of the pair)
  lo = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  hi = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
}

// Four int8 codes -> four f16 values code + 1152 (two words), exactly: XOR
// 0x80 gives the unsigned byte b = code + 128, and f16 bits 0x6400 | b are
// 1024 + b (exponent 10, b in the low mantissa bits); one v_perm_b32 per pair
// interleaves the bytes with 0x64.
constexpr float kInt8BiasF16 = 1152.f;
__device__ __forceinline__ void int8x4_to_f16x4_biased(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const uint32_t b = w ^ 0x80808080u;
  lo = __builtin_amdgcn_perm(0x64646464u, b, 0x04010400u);
  hi = __builtin_amdgcn_perm(0x64646464u, b, 0x04030402u);
}

// 8-bit codes of storage format KV -> bf16 MFMA operands: E4M3 values exactly,
// INT8 codes biased by kInt8Bias (code_biased<KV>).
template <int KV>
__host__ __device__ constexpr bool code_biased() { return code_set(KV) == DT_INT8; }
template <int KV>
__device__ __forceinline__ void code8x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  if constexpr (code_biased<KV>()) int8x4_to_bf16x4_biased(w, lo, hi);
  else fp8x4_to_bf16x4(w, lo, hi);
}

// Wave64 butterfly reductions over lanes that differ in bits 4 and 5 of the
// lane id (the four 16-lane rows of an MFMA accumulator), with the gfx950
// row-swap instructions: permlane16_swap(x, x) hands every lane the value of
// its partner 16 lanes away in one of the two results and keeps its own in the
// other, so max/sum of the pair is symmetric in the two; permlane32_swap does
// the same for the partner 32 lanes away.
__device__ __forceinline__ float row_max4(float x) {
  const uint32_t u = __float_as_uint(x);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t v = __float_as_uint(x);
  auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row_sum4(float x) {
  const uint32_t u = __float_as_uint(x);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t v = __float_as_uint(x);
  auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Element offset of K element (token o, dim d) inside a (block, KV head) tile
// stored as [D/X][16][X] with X = 16 bytes of elements.
template <int EB>
__device__ __forceinline__ int k_chunk_offset(int o, int d) {
  constexpr int X = 16 / EB;
  return ((d / X) * kBlockSize + o) * X + d % X;
}

// Element offset of V element (token o, dim d) inside a (block, KV head) tile
// stored in 16-byte chunks: chunk (g, c, j) holds tokens 4j..4j+3 of the Y = 4/EB
// dims 16 (g Y + u) + c, u < Y (u-major, then token), i.e. the tile is
// [D/(16 Y)][16][4][Y][4].  One lane's chunk is the PV operand of Y MFMA tiles.
template <int EB>
__device__ __forceinline__ int v_chunk_offset(int o, int d) {
  constexpr int Y = 4 / EB;
  const int t = d / 16;
  return ((((t / Y) * 16 + d % 16) * 4 + o / 4) * Y + t % Y) * 4 + o % 4;
}

// Logical block of virtual (attended) block vb: sink blocks first, then the window.
__device__ __forceinline__ int logical_block(int vb, int n_sink_blocks, int win_start) {
  return vb < n_sink_blocks ? vb : win_start + (vb - n_sink_blocks);
}

// Store one float of an output row in the requested dtype.
__device__ __forceinline__ void store_out(void* out, size_t idx, int dtype, float v) {
  if (dtype == DT_F32) {
    reinterpret_cast<float*>(out)[idx] = v;
  } else if (dtype == DT_BF16) {
    reinterpret_cast<uint16_t*>(out)[idx] = (uint16_t)f32_to_bf16_rne(v);
  } else {
    reinterpret_cast<uint16_t*>(out)[idx] = (uint16_t)f32_to_f16_bits(v);
  }
}

}  // namespace pkv
