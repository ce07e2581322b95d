// Keep-set geometry shared by the host (workspace sizing, grids) and the
// kernels: which logical blocks of a sequence hold positions that decode
// attention reads.
//
// Kept positions follow page "长上下文优化：注意力稀疏化与 KV Cache 管理"
// (plumephp.com/llm-long-context-optimization), StreamingKVCache snippet, and
// page "系统优化" section 4.1: the first num_sinks positions plus the last
// `window` positions; window <= 0 keeps every position.  Blocks are 16 tokens
// (page "KV Cache 与 PagedAttention：显存复用与长上下文推理", "PagedAttention 的设计").
//
// Attended ("virtual") blocks are numbered densely: the sink blocks first,
// then the window blocks; a block that holds both is counted once.
#pragma once

#include <hip/hip_runtime.h>

namespace pkv {

constexpr int kBlockSize = 16;    // tokens per physical block
#ifndef PKV_PART_BLOCKS
#define PKV_PART_BLOCKS 16
#endif
constexpr int kPartBlocks = PKV_PART_BLOCKS;   // attended blocks per partial-output slot (256 tokens)

struct KeepGeom {
  int n_sink_blocks;  // virtual blocks [0, n_sink_blocks) are logical blocks 0..n_sink_blocks-1
  int win_start;      // virtual block n_sink_blocks is logical block win_start, and onwards
  int n_virtual;      // attended blocks of the sequence
};

__host__ __device__ inline KeepGeom keep_geometry(int len, int num_sinks, int window) {
  const int nb = (len + 15) / 16;
  if (window <= 0 || len <= num_sinks + window) return KeepGeom{0, 0, nb};
  const int nsb = (num_sinks + 15) / 16;
  int ws = (len - window) / 16;
  if (ws < nsb) ws = nsb;
  return KeepGeom{nsb, ws, nsb + (nb - ws)};
}

// Upper bound of n_virtual over all lengths 1..max_len.
__host__ __device__ inline int max_virtual_blocks(int max_len, int num_sinks, int window) {
  const int nb = (max_len + 15) / 16;
  if (window <= 0) return nb;
  const int bound = (num_sinks + 15) / 16 + (window + 15) / 16 + 1;
  return nb < bound ? nb : bound;
}

__host__ __device__ inline int num_partitions(int n_virtual) {
  return (n_virtual + kPartBlocks - 1) / kPartBlocks;
}

// Position p (< len) is attended.
__host__ __device__ inline bool is_kept(int p, int len, int num_sinks, int window) {
  return p < len && (window <= 0 || p < num_sinks || p >= len - window);
}

}  // namespace pkv
