// Cache compaction for gfx950: apply an eviction keep-set by moving the kept
// tokens to a dense prefix of fresh blocks.
//
// Page "系统优化" 4.2 (evict_tokens returns the cache restricted to the kept
// indices) and page "长上下文优化：注意力稀疏化与 KV Cache 管理", StreamingKVCache (the
// cache keeps sinks + window and drops the middle): after eviction the
// sequence holds only its kept tokens.  Here the token at logical position
// keep_idx[s][i] of the source table moves to logical position i of the
// destination table, so the sequence occupies ceil(n / 16) blocks and the
// source blocks can be released.
//
// One 256-thread workgroup per (KV head, destination block, sequence) writes
// whole 16-byte chunks of the destination tile: a K chunk is one token row's
// 16 bytes (read as one chunk of the source token's tile); a V chunk holds 4
// tokens x Y dims and is gathered element by element.  Chunks that hold both
// kept tokens and the unused tail of the last block are read, patched and
// written back, so the tail stays as it was.
#include "device_common.hpp"
#include "launch.hpp"

namespace pkv {

template <int EB>
struct Elem;
template <> struct Elem<1> { using T = uint8_t; };
template <> struct Elem<2> { using T = uint16_t; };
template <> struct Elem<4> { using T = uint32_t; };

template <int EB, int D>
__global__ void __launch_bounds__(256) kv_compact_kernel(uint8_t* k_pool, uint8_t* v_pool, float* k_scale,
                                                       float* v_scale, const int32_t* src_tables, int src_stride,
                                                       const int32_t* dst_tables, int dst_stride,
                                                       const int32_t* keep_idx, int keep_stride,
                                                       const int32_t* keep_count, int num_blocks, int num_kv_heads) {
  using T = typename Elem<EB>::T;
  constexpr int Y = 4 / EB;                         // dims per V chunk
  constexpr int KCH = D * EB / 16;                  // K chunks per token row
  constexpr int VCH = D / (16 * Y) * 16 * 4;        // V chunks per tile
  constexpr size_t kTile = (size_t)kBlockSize * D * EB;
  __shared__ int s_blk[kBlockSize];                 // source block of destination token o (-1: poison)
  __shared__ int s_off[kBlockSize];                 // its offset in that block
  // KV head fastest: the heads of one destination block write side-by-side
  // tiles and read the same kept tokens from side-by-side source tiles.
  const int s = blockIdx.z, h = (int)(blockIdx.x % (unsigned)num_kv_heads), db = (int)(blockIdx.x / (unsigned)num_kv_heads);
  const int tid = threadIdx.x;
  const int cnt = keep_count[s];
  if (cnt < 0 || cnt > keep_stride || cnt > dst_stride * kBlockSize) return;
  const int i0 = db * kBlockSize;
  if (i0 >= cnt) return;
  const int n = min(kBlockSize, cnt - i0);
  const int dphys = dst_tables[(size_t)s * dst_stride + db];
  if (dphys < 0 || dphys >= num_blocks) return;
  if (tid < kBlockSize) {
    int b = -1, o = 0;
    if (tid < n) {
      const int p = keep_idx[(size_t)s * keep_stride + i0 + tid];
      if (p >= 0 && p < src_stride * kBlockSize) {
        b = src_tables[(size_t)s * src_stride + p / kBlockSize];
        o = p % kBlockSize;
        if (b < 0 || b >= num_blocks) b = -1;
      }
    }
    s_blk[tid] = b;
    s_off[tid] = o;
  }
  __syncthreads();
  const size_t dtile = (size_t)dphys * num_kv_heads + h;

  // K: chunk (u, o) of the destination tile <- chunk (u, s_off[o]) of the source tile.
  for (int q = tid; q < KCH * kBlockSize; q += blockDim.x) {
    const int u = q / kBlockSize, o = q % kBlockSize;
    if (o >= n) continue;
    u32x4 v = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
    if (s_blk[o] >= 0) {
      const size_t stile = (size_t)s_blk[o] * num_kv_heads + h;
      v = *reinterpret_cast<const u32x4*>(k_pool + stile * kTile + ((size_t)u * kBlockSize + s_off[o]) * 16);
    }
    *reinterpret_cast<u32x4*>(k_pool + dtile * kTile + ((size_t)u * kBlockSize + o) * 16) = v;
  }

  // V: chunk (g, c, jj) of the destination holds tokens 4 jj .. 4 jj + 3; element
  // (u, e) of token o = 4 jj + e comes from chunk (g, c, s_off[o] / 4), element
  // (u, s_off[o] % 4) of the source token's tile.
  for (int q = tid; q < VCH; q += blockDim.x) {
    const int jj = q % 4;
    if (4 * jj >= n) continue;
    const int gc = q / 4;                            // g * 16 + c
    u32x4* dchunk = reinterpret_cast<u32x4*>(v_pool + dtile * kTile + (size_t)q * 16);
    u32x4 w = 4 * jj + 3 < n ? u32x4{0u, 0u, 0u, 0u} : *dchunk;
    T* we = reinterpret_cast<T*>(&w);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int o = 4 * jj + e;
      if (o >= n) continue;
      const int b = s_blk[o];
      const int so = s_off[o];
      const T* sc = reinterpret_cast<const T*>(v_pool + ((size_t)(b >= 0 ? b : 0) * num_kv_heads + h) * kTile +
                                               ((size_t)gc * 4 + so / 4) * 16);   // block 0 stands in for poison
#pragma unroll
      for (int u = 0; u < Y; ++u) we[u * 4 + e] = b >= 0 ? sc[u * 4 + so % 4] : (T)~(T)0;
    }
    *dchunk = w;
  }

  if (k_scale != nullptr && tid < n) {
    const int b = s_blk[tid];
    const size_t src_i = ((size_t)(b >= 0 ? b : 0) * num_kv_heads + h) * kBlockSize + s_off[tid];
    const size_t dst_i = dtile * kBlockSize + tid;
    k_scale[dst_i] = b >= 0 ? k_scale[src_i] : __builtin_nanf("");
    v_scale[dst_i] = b >= 0 ? v_scale[src_i] : __builtin_nanf("");
  }
}

// Keep map of a compacting attention call (paged_decode_attn_compact): thread
// (s, b) describes block b of sequence s -- which of its 16 positions the keep
// list holds (and the appended token at L - 1 when keep_last), the destination
// slot of its first kept token and the destination blocks they fall in.  The
// list is strictly ascending, so the first kept token of block b is entry
// lower_bound(16 b) and its rank is that index.  A list that is not ascending
// gives unspecified masks and slots, still inside the listed destination
// blocks; a count outside [0, min(keep_stride, L - keep_last)], or that with
// the appended token exceeds the destination table, poisons the sequence.
__global__ void __launch_bounds__(256) keep_map_kernel(const int32_t* keep_idx, int keep_stride,
                                                       const int32_t* keep_count, const int32_t* context_lens,
                                                       int max_context_len, const int32_t* dst_tables, int dst_stride,
                                                       int num_blocks, int map_stride, int keep_last,
                                                       KeepMapEntry* map) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  const int s = blockIdx.y;
  if (b >= map_stride) return;
  const int L = context_lens[s];
  const int n = keep_count[s];
  const int old_len = L - keep_last;             // positions the list refers to
  KeepMapEntry e{0, -1, -1, 0};
  const bool ok = L >= 1 && L <= max_context_len && n >= 0 && n <= keep_stride && n <= old_len &&
                  (long long)n + keep_last <= (long long)kBlockSize * dst_stride;
  const int p0 = b * kBlockSize;
  if (!ok) {
    e.w0 = (int)0x80000000u;
  } else if (p0 < L) {
    const int32_t* ki = keep_idx + (size_t)s * keep_stride;
    int lo = 0, hi = n;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (ki[mid] < p0) lo = mid + 1;
      else hi = mid;
    }
    uint32_t mask = 0;
    for (int i = lo; i < n && i < lo + kBlockSize; ++i) {
      const int p = ki[i];
      if (p >= p0 + kBlockSize) break;
      if (p >= p0 && p < old_len) mask |= 1u << (p - p0);
    }
    if (keep_last && L - 1 < p0 + kBlockSize) mask |= 1u << (L - 1 - p0);   // the appended token, rank n
    const int q = lo / kBlockSize;                 // destination block of the first kept token
    int d0 = q < dst_stride ? dst_tables[(size_t)s * dst_stride + q] : -1;
    int d1 = q + 1 < dst_stride ? dst_tables[(size_t)s * dst_stride + q + 1] : -1;
    if (d0 < 0 || d0 >= num_blocks) d0 = -1;
    if (d1 < 0 || d1 >= num_blocks) d1 = -1;
    e.w0 = (int)(mask | ((uint32_t)(lo % kBlockSize) << 16));
    e.dst0 = d0;
    e.dst1 = d1;
    e.rank = lo;
  }
  map[(size_t)s * map_stride + b] = e;
}

namespace {

template <int EB>
hipError_t compact_d(void* k_pool, void* v_pool, float* k_scale, float* v_scale, const int32_t* src_tables,
                     int src_stride, const int32_t* dst_tables, int dst_stride, const int32_t* keep_idx,
                     int keep_stride, const int32_t* keep_count, int num_seqs, int num_blocks, int num_kv_heads,
                     int head_dim, hipStream_t st) {
  dim3 grid((unsigned)((keep_stride + kBlockSize - 1) / kBlockSize) * (unsigned)num_kv_heads, 1, num_seqs);
  if (head_dim == 64)
    hipLaunchKernelGGL((kv_compact_kernel<EB, 64>), grid, dim3(256), 0, st, reinterpret_cast<uint8_t*>(k_pool),
                       reinterpret_cast<uint8_t*>(v_pool), k_scale, v_scale, src_tables, src_stride, dst_tables,
                       dst_stride, keep_idx, keep_stride, keep_count, num_blocks, num_kv_heads);
  else
    hipLaunchKernelGGL((kv_compact_kernel<EB, 128>), grid, dim3(256), 0, st, reinterpret_cast<uint8_t*>(k_pool),
                       reinterpret_cast<uint8_t*>(v_pool), k_scale, v_scale, src_tables, src_stride, dst_tables,
                       dst_stride, keep_idx, keep_stride, keep_count, num_blocks, num_kv_heads);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_compact(void* k_pool, void* v_pool, float* k_scale, float* v_scale, int kv_dtype,
                             const int32_t* src_tables, int src_stride, const int32_t* dst_tables, int dst_stride,
                             const int32_t* keep_idx, int keep_stride, const int32_t* keep_count, int num_seqs,
                             int num_blocks, int num_kv_heads, int head_dim, hipStream_t st) {
  if (num_seqs == 0 || keep_stride == 0) return hipSuccess;
  float* ks = is_quantised(kv_dtype) ? k_scale : nullptr;
  float* vs = is_quantised(kv_dtype) ? v_scale : nullptr;
  switch (kv_dtype) {
    case DT_F32:
      return compact_d<4>(k_pool, v_pool, ks, vs, src_tables, src_stride, dst_tables, dst_stride, keep_idx,
                          keep_stride, keep_count, num_seqs, num_blocks, num_kv_heads, head_dim, st);
    case DT_FP8:
    case DT_INT8:
    case DT_FP8_CH:
    case DT_INT8_CH:
      return compact_d<1>(k_pool, v_pool, ks, vs, src_tables, src_stride, dst_tables, dst_stride, keep_idx,
                          keep_stride, keep_count, num_seqs, num_blocks, num_kv_heads, head_dim, st);
    default:
      return compact_d<2>(k_pool, v_pool, ks, vs, src_tables, src_stride, dst_tables, dst_stride, keep_idx,
                          keep_stride, keep_count, num_seqs, num_blocks, num_kv_heads, head_dim, st);
  }
}

hipError_t launch_keep_map(const int32_t* keep_idx, int keep_stride, const int32_t* keep_count,
                           const int32_t* context_lens, int max_context_len, const int32_t* dst_tables,
                           int dst_stride, int num_blocks, int num_seqs, int map_stride, int keep_last,
                           KeepMapEntry* map, hipStream_t st) {
  if (num_seqs == 0 || map_stride == 0) return hipSuccess;
  dim3 grid((unsigned)((map_stride + 255) / 256), (unsigned)num_seqs);
  hipLaunchKernelGGL(keep_map_kernel, grid, dim3(256), 0, st, keep_idx, keep_stride, keep_count, context_lens,
                     max_context_len, dst_tables, dst_stride, num_blocks, map_stride, keep_last, map);
  return hipGetLastError();
}

}  // namespace pkv
