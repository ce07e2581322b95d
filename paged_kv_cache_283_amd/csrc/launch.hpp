// Host-side launchers of the gfx950 kernels (internal to the library).
// Arguments arrive here already validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pagedkv.h"

namespace pkv {

// (pool format, query dtype) pairs whose decode append the attention kernel
// takes in itself (paged_decode_append_attn): all but INT8 pools with f32
// queries, whose attention kernel would pass 256 VGPRs with the append code
// (one wave per SIMD instead of two); with 16-bit queries the INT8 kernel
// holds it at 250-252 and times the same as without it.
__host__ __device__ constexpr bool fused_append_built(int kv_dtype, int q_dtype) {
  return !((kv_dtype == PKV_INT8 || kv_dtype == PKV_INT8_CHANNEL) && q_dtype == PKV_F32);
}

// Per-call schedule the attention kernel hands to the merge kernel (workspace).
struct StreamHdr {
  int per;               // attended blocks of an even-numbered range
  int per_odd;           // attended blocks of an odd-numbered range (ranges alternate)
  int pad[2];
};

// Per attended block of a sequence, what the compacting attention call
// (paged_decode_attn_compact) does with its 16 tokens: bit t of w0's low 16
// bits keeps position 16 b + t (the rest are masked out of the attention);
// the kept tokens go, in order, to slots (w0 >> 16) & 15, +1, ... of physical
// block dst0, continuing at slot 0 of dst1 (-1: not stored); bit 31 of w0
// poisons the sequence (NaN output, nothing stored).  rank: the first kept
// token's destination position.
struct __attribute__((aligned(16))) KeepMapEntry {
  int w0, dst0, dst1, rank;
};

struct AttnArgs {
  void* out;
  int out_dtype;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;
  int table_stride;
  const int32_t* context_lens;
  int max_context_len;
  int num_seqs, num_blocks, num_q_heads, num_kv_heads;
  float scale_log2;     // softmax scale * log2(e): logits are kept in base 2
  int num_sinks, window;
  float* attn_mass;
  int mass_stride;
  // workspace views
  float* part_acc;      // [B][Hq][p_max][D]   unnormalised partial outputs
  float* part_ml;       // [B][Hq][p_max][2]   partition max (base-2) and exp-sum
  float* stash;         // [B][Hq][nv_pad]     base-2 logits per attended position (mass only)
  float* fin_ml;        // [B][Hq][2]          max and exp-sum of one-segment sequences (mass only)
  StreamHdr* hdr;       // schedule of this call
  int* seq_prefix;      // [B + 1]  attended-block prefix per sequence, then the total
  int p_max;
  int nv_pad;
  // Decode append fused in: the new token of every sequence (position
  // context_lens[s] - 1), [B][Hkv][D] in the pool's dtype (16-bit and f32
  // pools) or q's dtype (8-bit pools), enters the last block's operands from
  // here and is stored into the pools.  Null: the pools already hold it.
  const void* k_new;
  const void* v_new;
  void* k_store;        // the K and V pools, writable (fused append only)
  void* v_store;
  float* k_scale_store; // per-token scale arrays, writable (fused append, per-token 8-bit formats)
  float* v_scale_store;
  // Compaction fused in (16-bit pools): keep_map [B][map_stride] (see
  // KeepMapEntry); the kept tokens are stored through k_store / v_store.
  // With the H2O mass, attn_mass is the compacted score rows: entry i of
  // sequence s (the kept token of rank i) becomes mass_src[s][p] + this
  // step's mass of p, p its source position.
  const KeepMapEntry* keep_map;
  int map_stride;
  const float* mass_src;
  int mass_src_stride;
};

// Causal multi-query attention over the paged cache (chunked prefill).
struct PrefillArgs {
  void* out;
  int out_dtype;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;
  int table_stride;
  const int32_t* context_lens;
  const int32_t* query_start;   // [B + 1]: query rows of sequence s are [query_start[s], query_start[s + 1])
  int num_tokens;               // rows of q and out
  int max_context_len;
  int num_seqs, num_blocks, num_q_heads, num_kv_heads;
  float scale_log2;
  int tiles_per_pair;           // workgroups per (sequence, KV head), set by the launcher
};

hipError_t launch_prefill_attn(const PrefillArgs& a, int kv_dtype, int q_dtype, int head_dim, int max_query_len,
                               hipStream_t stream);

struct WorkspaceLayout {
  size_t acc_off, ml_off, hdr_off, prefix_off, stash_off, fin_off, total;
  int p_max, nv_pad;
};

WorkspaceLayout attn_workspace_layout(int num_seqs, int num_q_heads, int head_dim, int max_context_len,
                                      int num_sinks, int window, bool want_mass);

// Keep map of a compacting attention call: one entry per (sequence, block of
// max_context_len) from the sorted keep lists and the destination tables;
// keep_last adds position context_lens[s] - 1 (the appended token) after the
// listed ones.
hipError_t launch_keep_map(const int32_t* keep_idx, int keep_stride, const int32_t* keep_count,
                           const int32_t* context_lens, int max_context_len, const int32_t* dst_tables,
                           int dst_stride, int num_blocks, int num_seqs, int map_stride, int keep_last,
                           KeepMapEntry* map, hipStream_t stream);

// Size of the fixed per-device workspace behind paged_decode_attn_noalloc.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;

// Device address of that workspace on the current device (looked up once per
// device).
hipError_t static_scratch(void** ptr);

hipError_t launch_decode_attn(const AttnArgs& a, int kv_dtype, int q_dtype, int head_dim,
                              hipStream_t stream, hipEvent_t ev_main_begin, hipEvent_t ev_main_end);

hipError_t launch_decode_slots(const int32_t* tables, int stride, const int32_t* lens, int num_seqs,
                               int num_blocks, int64_t* slots, hipStream_t stream);

hipError_t launch_token_slots(const int32_t* tables, int stride, int num_seqs, const int32_t* seq_ids,
                              const int32_t* positions, int num_tokens, int num_blocks, int64_t* slots,
                              hipStream_t stream);

hipError_t launch_kv_write(const void* k_new, const void* v_new, int src_dtype, void* k_pool, void* v_pool,
                           float* k_scale, float* v_scale, int kv_dtype, const int64_t* slots,
                           int num_tokens, int num_blocks, int num_kv_heads, int head_dim, hipStream_t stream);

hipError_t launch_kv_append(const void* k_new, const void* v_new, int src_dtype, void* k_pool, void* v_pool,
                            float* k_scale, float* v_scale, int kv_dtype, const int32_t* tables, int stride,
                            const int32_t* lens, int num_seqs, int num_blocks, int num_kv_heads, int head_dim,
                            hipStream_t stream);

hipError_t launch_kv_swap(void* k_pool, void* v_pool, float* k_scale, float* v_scale, int kv_dtype, void* host_k,
                          void* host_v, float* host_k_scale, float* host_v_scale, const int32_t* pairs, int num_pairs,
                          int num_blocks, int host_slots, int num_kv_heads, int head_dim, int to_host,
                          hipStream_t stream);

hipError_t launch_block_copy(void* k_pool, void* v_pool, float* k_scale, float* v_scale, int kv_dtype,
                             const int32_t* pairs, int num_pairs, int num_blocks, int num_kv_heads,
                             int head_dim, hipStream_t stream);

hipError_t launch_keep_select(const float* scores, int stride, const int32_t* lens, int num_seqs, int max_len,
                              int num_sinks, int recent, int heavy, int all_candidates, int32_t* keep_idx,
                              int keep_stride, int32_t* keep_count, hipStream_t stream);

hipError_t launch_kv_compact(void* k_pool, void* v_pool, float* k_scale, float* v_scale, int kv_dtype,
                             const int32_t* src_tables, int src_stride, const int32_t* dst_tables, int dst_stride,
                             const int32_t* keep_idx, int keep_stride, const int32_t* keep_count, int num_seqs,
                             int num_blocks, int num_kv_heads, int head_dim, hipStream_t stream);

hipError_t launch_probe_read(const void* src, size_t bytes, float* sink, hipStream_t stream);
hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

}  // namespace pkv
