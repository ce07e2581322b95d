// KV-cache maintenance kernels for gfx950: decode slot lookup, token write
// (with 8-bit quantisation) and whole-block copy for copy-on-write.
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
#include "kv_codec.hpp"
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

// One wave per (token, KV head) row, K and V together: the decode append,
// whose tokens are one per sequence (no chunk of the layout holds two of
// them), where latency is all that counts.  The source loads go out before the
// slot lookup they do not depend on.
template <int SRC, int KVT, int D>
__global__ void __launch_bounds__(256) kv_row_kernel(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                                   float* k_scale, float* v_scale, const SlotSource ss,
                                                   int num_tokens, int num_blocks, int num_kv_heads) {
  constexpr int EB = KVT == DT_F32 ? 4 : (is_code8(KVT) ? 1 : 2);
  constexpr int PER = D / kWave;
  constexpr float kMaxCode = code_set(KVT) == DT_INT8 ? 127.f : 448.f;
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (long)num_tokens * num_kv_heads) return;
  const int t = (int)(row / num_kv_heads), h = (int)(row % num_kv_heads);
  uint32_t kr[PER], vr[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    kr[e] = load_raw<SRC>(k_new, (size_t)row * D + e * kWave + lane);
    vr[e] = load_raw<SRC>(v_new, (size_t)row * D + e * kWave + lane);
  }
  const int64_t slot = token_slot(ss, t, num_blocks);
  if (slot < 0 || slot >= (int64_t)num_blocks * kBlockSize) return;
  const size_t tile = (size_t)(slot / kBlockSize) * num_kv_heads + h;
  const int o = (int)(slot % kBlockSize);
  float ks = 0.f, vs = 0.f;
  if constexpr (is_quantised(KVT)) {
    float km = 0.f, vm = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      km = fmaxf(km, fabsf(raw_to_f32<SRC>(kr[e])));
      vm = fmaxf(vm, fabsf(raw_to_f32<SRC>(vr[e])));
    }
    ks = __fdiv_rn(wave_max(km), kMaxCode);
    vs = __fdiv_rn(wave_max(vm), kMaxCode);
    if (lane == 0) {
      k_scale[tile * kBlockSize + o] = ks;
      v_scale[tile * kBlockSize + o] = vs;
    }
  }
  uint8_t* kp = reinterpret_cast<uint8_t*>(k_pool) + tile * kBlockSize * D * EB;
  uint8_t* vp = reinterpret_cast<uint8_t*>(v_pool) + tile * kBlockSize * D * EB;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int d = e * kWave + lane;
    const float kc = is_channel_scaled(KVT) ? k_scale[(size_t)h * D + d] : ks;
    const float vc = is_channel_scaled(KVT) ? v_scale[(size_t)h * D + d] : vs;
    store_elem<EB>(kp + (size_t)k_chunk_offset<EB>(o, d) * EB, stored_code<SRC, KVT>(kr[e], kc));
    store_elem<EB>(vp + (size_t)v_chunk_offset<EB>(o, d) * EB, stored_code<SRC, KVT>(vr[e], vc));
  }
}

// Tokens staged per workgroup of the slot-list write, and its threads (8 per
// staged K or V row in the scale pass).
constexpr int kWriteGroup = 16;
constexpr int kWriteThreads = 16 * kWriteGroup;

// One workgroup per 16 consecutive tokens and one KV head.  The tokens' K and
// V rows are staged in LDS, so the pool is written in whole 16-byte
// chunks wherever the layout allows: a K chunk holds X dims of one token, so
// every token's K goes out as D/X chunks whatever its slot; a V chunk holds 4
// consecutive rows of a block, so the 4 tokens of such a quad go out as whole
// chunks when all 4 are in this workgroup with consecutive slots (any
// prefill or bulk fill), and element by element otherwise (a decode step:
// one token per sequence).  8-bit formats quantise each row with its own
// scale (absmax / largest code) or by the static channel scales.
template <int SRC, int KVT, int D>
__global__ void __launch_bounds__(kWriteThreads) kv_write_kernel(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                                     float* k_scale, float* v_scale, const SlotSource ss,
                                                     int num_tokens, int num_blocks, int num_kv_heads) {
  constexpr int EB = KVT == DT_F32 ? 4 : (is_code8(KVT) ? 1 : 2);   // bytes per stored element
  constexpr int X = 16 / EB;                                       // elements per K chunk
  constexpr int Y = 4 / EB;                                        // dims per V chunk
  constexpr int kThreads = kWriteThreads;
  constexpr float kMaxCode = code_set(KVT) == DT_INT8 ? 127.f : 448.f;
  // Raw source bits of K and V.  f32 sources: one word per element, rows
  // padded by one word so that threads reading the same dim of consecutive
  // rows hit different LDS banks.  16-bit sources: packed as loaded, rows
  // padded by 16 bytes, so a 16-byte LDS read yields 8 consecutive dims (the
  // scale pass and the K chunks read them that way).  16-bit pools (fed from
  // their own dtype, bits copied as they are): a workgroup whose 16 tokens
  // fill one tile in slot order (bulk fills, prefills) builds each K chunk
  // from one 16-byte LDS read and each V chunk from eight 2-byte ones, with
  // no per-element packing.
  constexpr bool PACK16 = KVT == DT_BF16 || KVT == DT_F16;
  constexpr bool H16 = SRC != DT_F32;
  static_assert(!PACK16 || SRC == KVT, "16-bit pools take their own dtype");
  static_assert(!H16 || KVT != DT_F32, "f32 pools take f32");
  constexpr int kRow = D + 1;
  constexpr int kRowH = D + 8;
  __shared__ uint32_t s_src[H16 ? 1 : 2][H16 ? 1 : kWriteGroup][H16 ? 1 : kRow];   // [K, V][token][dim]
  __shared__ __attribute__((aligned(16))) uint16_t s_h[H16 ? 2 : 1][H16 ? kWriteGroup : 1][H16 ? kRowH : 8];
  __shared__ int s_full;                       // PACK16: the 16 tokens are rows 0..15 of one tile
  __shared__ int64_t s_slot[kWriteGroup];      // -1: token skipped
  __shared__ float s_scale[2][kWriteGroup];
  __shared__ float s_cs[is_channel_scaled(KVT) ? 2 : 1][is_channel_scaled(KVT) ? D : 1];   // K, V channel scales of head h
  __shared__ int s_lead[kWriteGroup];          // V: 1 leads a complete quad, 2 is covered by one, 0 neither
  __shared__ int s_quad[kWriteGroup / 4];      // the tokens that lead a quad, in order
  __shared__ int s_nquad, s_single;            // how many; whether any token is stored element by element

  const int tid = threadIdx.x;
  // KV head fastest: the heads of one token group read one contiguous stretch
  // of the source and write side-by-side tiles of the pool.
  const int h = (int)(blockIdx.x % (unsigned)num_kv_heads);
  const int t_base = (int)(blockIdx.x / (unsigned)num_kv_heads) * kWriteGroup;
  // Both rows of every token, with 16-byte loads: K and V, row o, elements
  // [8 p, 8 p + 8) (16-bit source) or [4 p, 4 p + 4) (f32).  All of a
  // thread's loads and the slot lookup go out before any of them is waited
  // for (one memory round trip per workgroup); rows of skipped tokens are
  // simply not stored.
  constexpr int kPer = 16 / (SRC == DT_F32 ? 4 : 2);
  constexpr int kUnits = 2 * kWriteGroup * D / kPer;   // 16-byte pieces of the group's K and V rows
  static_assert(kUnits % kThreads == 0, "whole loads per thread");
  constexpr int kLoads = kUnits / kThreads;
  u32x4 wv[kLoads];
#pragma unroll
  for (int it = 0; it < kLoads; ++it) {
    const int e = tid + it * kThreads;
    const int kv = e / (kWriteGroup * D / kPer), r = e % (kWriteGroup * D / kPer);
    const int o = r / (D / kPer), d0 = (r % (D / kPer)) * kPer;
    wv[it] = u32x4{0u, 0u, 0u, 0u};
    if (t_base + o < num_tokens)
      wv[it] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(kv == 0 ? k_new : v_new) +
                                               (((size_t)(t_base + o) * num_kv_heads + h) * D + d0) * (16 / kPer));
  }
  static_assert(2 * D <= kThreads, "one channel scale per thread");
  float cs = 0.f;
  if constexpr (is_channel_scaled(KVT))
    if (tid < 2 * D) cs = (tid < D ? k_scale : v_scale)[(size_t)h * D + tid % D];
  long long my_slot = -1;                      // lanes 0..15: token t_base + lane
  if (tid < kWriteGroup) {
    const int t = t_base + tid;
    int64_t sl = t < num_tokens ? token_slot(ss, t, num_blocks) : -1;
    if (sl >= (int64_t)num_blocks * kBlockSize) sl = -1;
    my_slot = sl < 0 ? -1 : sl;
    s_slot[tid] = my_slot;
  }
#pragma unroll
  for (int it = 0; it < kLoads; ++it) {
    const int e = tid + it * kThreads;
    const int kv = e / (kWriteGroup * D / kPer), r = e % (kWriteGroup * D / kPer);
    const int o = r / (D / kPer), d0 = (r % (D / kPer)) * kPer;
    const u32x4 w = wv[it];
    if constexpr (H16) {
      *reinterpret_cast<u32x4*>(&s_h[kv][o][d0]) = w;
    } else {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        if constexpr (SRC == DT_F32) s_src[kv][o][d0 + i] = w[i];
        else s_src[kv][o][d0 + i] = (w[i / 2] >> (16 * (i % 2))) & 0xffffu;
      }
    }
  }
  if constexpr (is_channel_scaled(KVT))
    if (tid < 2 * D) s_cs[tid / D][tid % D] = cs;
  __syncthreads();
  if (tid < kWave) {
    // V quads, in the first wave's registers: token o leads one when it and
    // the next 3 tokens hold rows 4k..4k+3 of one block in slot order (1); the
    // 3 others are covered (2).  A covered token's slot is not a multiple of
    // 4, so no token both leads and is covered.
    const long long n1 = __shfl_down(my_slot, 1, kWave), n2 = __shfl_down(my_slot, 2, kWave),
                    n3 = __shfl_down(my_slot, 3, kWave);
    const bool lead = tid + 3 < kWriteGroup && my_slot >= 0 && my_slot % 4 == 0 && n1 == my_slot + 1 &&
                      n2 == my_slot + 2 && n3 == my_slot + 3;
    const int l1 = __shfl_up((int)lead, 1, kWave), l2 = __shfl_up((int)lead, 2, kWave),
              l3 = __shfl_up((int)lead, 3, kWave);
    const bool covered = (tid >= 1 && l1) || (tid >= 2 && l2) || (tid >= 3 && l3);
    if (tid < kWriteGroup) s_lead[tid] = lead ? 1 : (covered ? 2 : 0);
    const unsigned long long lm = __builtin_amdgcn_ballot_w64(lead);
    if (lead) s_quad[__popcll(lm & ((1ull << tid) - 1ull))] = tid;
    const unsigned long long sm = __builtin_amdgcn_ballot_w64(tid < kWriteGroup && my_slot >= 0 && !lead && !covered);
    if (tid == 0) {
      s_nquad = __popcll(lm);
      s_single = sm != 0ull;
    }
    if constexpr (PACK16) {
      const long long s0 = __shfl(my_slot, 0, kWave);
      const bool ok = tid >= kWriteGroup || (s0 >= 0 && s0 % kBlockSize == 0 && my_slot == s0 + tid);
      const bool full = __builtin_amdgcn_ballot_w64(!ok) == 0ull;
      if (tid == 0) s_full = full ? 1 : 0;
    }
  }
  if constexpr (is_quantised(KVT)) {
    // 8 threads per (K or V, row): absmax, then the row's scale
    const int kv = tid / (8 * kWriteGroup), o = (tid / 8) % kWriteGroup, l = tid % 8;
    float m = 0.f;
    if constexpr (H16) {
      for (int p = l; p < D / 8; p += 8) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(&s_h[kv][o][8 * p]);
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(raw_to_f32<SRC>((w[i / 2] >> (16 * (i % 2))) & 0xffffu)));
      }
    } else {
      for (int d = l; d < D; d += 8) m = fmaxf(m, fabsf(raw_to_f32<SRC>(s_src[kv][o][d])));
    }
#pragma unroll
    for (int off = 4; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 8));
    const float sc = __fdiv_rn(m, kMaxCode);
    if (l == 0) {
      s_scale[kv][o] = sc;
      const int64_t sl = s_slot[o];
      if (sl >= 0)
        (kv == 0 ? k_scale : v_scale)[((size_t)(sl / kBlockSize) * num_kv_heads + h) * kBlockSize + sl % kBlockSize] = sc;
    }
  }
  __syncthreads();

  // Stored bits of element (token o, dim d) of K (kv 0) or V (kv 1), from its
  // raw source bits.
  auto code_from = [&](int kv, int o, int d, uint32_t raw) -> uint32_t {
    if constexpr (PACK16) {
      return raw;
    } else {
      float sc = 0.f;
      if constexpr (is_quantised(KVT)) sc = s_scale[kv][o];
      if constexpr (is_channel_scaled(KVT)) sc = s_cs[kv][d];
      return stored_code<SRC, KVT>(raw, sc);
    }
  };
  auto code_of = [&](int kv, int o, int d) -> uint32_t {
    if constexpr (H16) return code_from(kv, o, d, s_h[kv][o][d]);
    else return code_from(kv, o, d, s_src[kv][o][d]);
  };
  // 16 bytes from 16 / EB element codes.
  auto pack = [&](const uint32_t* el) {
    u32x4 w = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16 / EB; ++i) {
      if constexpr (EB == 4) w[i] = el[i];
      else w[i * EB / 4] |= (el[i] & ((1u << (EB * 8)) - 1u)) << ((i * EB * 8) % 32);
    }
    return w;
  };
  uint8_t* kp = reinterpret_cast<uint8_t*>(k_pool);
  uint8_t* vp = reinterpret_cast<uint8_t*>(v_pool);

  if constexpr (PACK16) {
    if (s_full) {   // one whole tile, rows in slot order
      const size_t tile = (size_t)(s_slot[0] / kBlockSize) * num_kv_heads + h;
      uint8_t* kt = kp + tile * kBlockSize * D * EB;
      uint8_t* vt = vp + tile * kBlockSize * D * EB;
      // K chunk (c, o): dims 8c .. 8c + 7 of row o, at (c * 16 + o) * 16
      for (int q = tid; q < kWriteGroup * (D / X); q += kThreads) {
        const int o = q % kWriteGroup, c = q / kWriteGroup;
        *reinterpret_cast<u32x4*>(kt + (size_t)(c * kBlockSize + o) * 16) =
            *reinterpret_cast<const u32x4*>(&s_h[0][o][X * c]);
      }
      // V chunk q = (g * 16 + c) * 4 + jq: dims 16 (2g + u) + c, u < 2, of rows
      // 4 jq .. 4 jq + 3, element order [u][row]
      for (int q = tid; q < kWriteGroup * D / 8; q += kThreads) {
        const int jq = q % 4, c = (q / 4) % kBlockSize, g = q / (4 * kBlockSize);
        uint32_t w4[4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int d = 16 * (2 * g + u) + c;
          w4[2 * u] = (uint32_t)s_h[1][4 * jq][d] | ((uint32_t)s_h[1][4 * jq + 1][d] << 16);
          w4[2 * u + 1] = (uint32_t)s_h[1][4 * jq + 2][d] | ((uint32_t)s_h[1][4 * jq + 3][d] << 16);
        }
        *reinterpret_cast<u32x4*>(vt + (size_t)q * 16) = u32x4{w4[0], w4[1], w4[2], w4[3]};
      }
      return;
    }
  }

  // K chunks and the V chunks of complete quads in one loop, so that every
  // thread takes a share of both (the K chunks alone occupy only half the
  // threads of an 8-bit pool's workgroup, the quads' V chunks another half).
  // K: chunk c of token o = dims c X .. c X + X - 1 at [c][row][*] of its tile.
  // V: chunk (g, c) of the quad led by token o holds dims 16 (g Y + u) + c,
  // u < Y, of its 4 rows, element order [u][row].
  constexpr int nK = kWriteGroup * (D / X);
  const int nKV = nK + s_nquad * (D / Y);
  for (int q = tid; q < nKV; q += kThreads) {
    uint32_t el[16 / EB];
    if (q < nK) {
      const int o = q % kWriteGroup, c = q / kWriteGroup;
      const int64_t sl = s_slot[o];
      if (sl < 0) continue;
      if constexpr (H16) {
#pragma unroll
        for (int j = 0; j < X / 8; ++j) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(&s_h[0][o][c * X + 8 * j]);
#pragma unroll
          for (int i = 0; i < 8; ++i)
            el[8 * j + i] = code_from(0, o, c * X + 8 * j + i, (w[i / 2] >> (16 * (i % 2))) & 0xffffu);
        }
      } else {
#pragma unroll
        for (int i = 0; i < X; ++i) el[i] = code_of(0, o, c * X + i);
      }
      const size_t tile = (size_t)(sl / kBlockSize) * num_kv_heads + h;
      *reinterpret_cast<u32x4*>(kp + tile * kBlockSize * D * EB + ((size_t)c * kBlockSize + sl % kBlockSize) * 16) =
          pack(el);
    } else {
      const int v = q - nK;
      const int o = s_quad[v / (D / Y)], gc = v % (D / Y);
      const int64_t sl = s_slot[o];
      const int g = gc / kBlockSize, c = gc % kBlockSize;
#pragma unroll
      for (int u = 0; u < Y; ++u) {
#pragma unroll
        for (int e = 0; e < 4; ++e) el[u * 4 + e] = code_of(1, o + e, kBlockSize * (g * Y + u) + c);
      }
      const size_t tile = (size_t)(sl / kBlockSize) * num_kv_heads + h;
      const int jq = (int)(sl % kBlockSize) / 4;
      *reinterpret_cast<u32x4*>(vp + tile * kBlockSize * D * EB + (((size_t)g * kBlockSize + c) * 4 + jq) * 16) =
          pack(el);
    }
  }
  if (!s_single) return;
  // V, other tokens: element by element
  for (int q = tid; q < kWriteGroup * D; q += kThreads) {
    const int o = q / D, d = q % D;
    const int64_t sl = s_slot[o];
    if (sl < 0 || s_lead[o] != 0) continue;
    const size_t tile = (size_t)(sl / kBlockSize) * num_kv_heads + h;
    uint8_t* dst = vp + (tile * kBlockSize * D + v_chunk_offset<EB>((int)(sl % kBlockSize), d)) * EB;
    store_elem<EB>(dst, code_of(1, o, d));
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

template <int SRC, int KVT, int D>
void launch_write(const void* k_new, const void* v_new, void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                  const SlotSource& ss, int num_tokens, int num_blocks, int num_kv_heads, hipStream_t st) {
  if (ss.slots != nullptr) {
    dim3 grid((unsigned)((num_tokens + kWriteGroup - 1) / kWriteGroup) * (unsigned)num_kv_heads);
    hipLaunchKernelGGL((kv_write_kernel<SRC, KVT, D>), grid, dim3(kWriteThreads), 0, st, k_new, v_new, k_pool, v_pool,
                       k_scale, v_scale, ss, num_tokens, num_blocks, num_kv_heads);
  } else {
    const long rows = (long)num_tokens * num_kv_heads;
    hipLaunchKernelGGL((kv_row_kernel<SRC, KVT, D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, k_new, v_new,
                       k_pool, v_pool, k_scale, v_scale, ss, num_tokens, num_blocks, num_kv_heads);
  }
}

template <int SRC, int KVT>
hipError_t write_d(const void* k_new, const void* v_new, void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                   const SlotSource& ss, int num_tokens, int num_blocks, int num_kv_heads, int head_dim,
                   hipStream_t st) {
  if (head_dim == 64)
    launch_write<SRC, KVT, 64>(k_new, v_new, k_pool, v_pool, k_scale, v_scale, ss, num_tokens, num_blocks,
                               num_kv_heads, st);
  else
    launch_write<SRC, KVT, 128>(k_new, v_new, k_pool, v_pool, k_scale, v_scale, ss, num_tokens, num_blocks,
                                num_kv_heads, st);
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
