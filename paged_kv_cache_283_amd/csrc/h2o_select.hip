// H2O keep-set selection for gfx950.
//
// Page "长上下文优化：注意力稀疏化与 KV Cache 管理" (plumephp.com/llm-long-context-optimization),
// H2OEviction.select: keep the most recent `recent` positions unconditionally
// and the highest accumulated scores among the earlier ones, budget in total,
// in ascending order.  Ties go to the lower position; NaN ranks like -inf.
//
// One workgroup per sequence.  The (budget - recent)-th largest score is found
// by an exact 4-pass radix select (8 bits per pass, LDS histogram) on
// order-preserving 32-bit keys; a final pass in position order takes every key
// above the threshold and the first still-needed keys equal to it, and
// compacts them with ballot prefix counts, which yields ascending output
// without a sort.
#include "device_common.hpp"
#include "launch.hpp"

namespace pkv {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;

__device__ __forceinline__ uint32_t score_key(float f) {
  if (f != f) return 0x007fffffu;         // NaN: same rank as -inf
  if (f == 0.f) f = 0.f;                  // -0 and +0 compare equal
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive count of `flag` over lower thread ids; *total gets the block count.
__device__ __forceinline__ int block_prefix_count(bool flag, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const unsigned long long bal = __ballot(flag);
  const int in_wave = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) s_wave[w] = __popcll(bal);
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) {
    const int n = s_wave[i];
    before += i < w ? n : 0;
    tot += n;
  }
  __syncthreads();
  *total = tot;
  return before + in_wave;
}

}  // namespace

__global__ void __launch_bounds__(kSelThreads) h2o_select_kernel(const float* scores, int stride, const int32_t* lens,
                                                               int max_len, int budget, int recent, int32_t* keep_idx,
                                                               int32_t* keep_count) {
  __shared__ int hist[256];
  __shared__ int s_wave[kSelWaves];
  __shared__ int s_pick[2];
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  const int L = lens[s];
  int32_t* out = keep_idx + (size_t)s * budget;
  if (L < 1 || L > max_len) {
    for (int i = tid; i < budget; i += kSelThreads) out[i] = -1;
    if (tid == 0) keep_count[s] = -1;
    return;
  }
  if (L <= budget) {
    for (int i = tid; i < budget; i += kSelThreads) out[i] = i < L ? i : -1;
    if (tid == 0) keep_count[s] = L;
    return;
  }
  const float* row = scores + (size_t)s * stride;
  const int cand = L - recent;
  const int k = budget - recent;
  for (int i = tid; i < recent; i += kSelThreads) out[k + i] = cand + i;
  if (tid == 0) keep_count[s] = budget;
  if (k == 0) return;

  // Radix select of the k-th largest key, most significant byte first.
  uint32_t prefix = 0u, mask = 0u;
  int need = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    for (int p = tid; p < cand; p += kSelThreads) {
      const uint32_t key = score_key(row[p]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int cum = 0, digit = 0;
      for (int d = 255; d >= 0; --d) {
        if (cum + hist[d] >= need) { digit = d; break; }
        cum += hist[d];
      }
      s_pick[0] = digit;
      s_pick[1] = need - cum;
    }
    __syncthreads();
    prefix |= (uint32_t)s_pick[0] << shift;
    mask |= 255u << shift;
    need = s_pick[1];
    __syncthreads();
  }
  const uint32_t thresh = prefix;   // the k-th largest key; `need` keys equal to it are taken

  int eq_seen = 0, written = 0;
  for (int base = 0; base < cand; base += kSelThreads) {
    const int p = base + tid;
    const uint32_t key = p < cand ? score_key(row[p]) : 0u;
    const bool eq = p < cand && key == thresh;
    const bool gt = p < cand && key > thresh;
    int eq_tot, sel_tot;
    const int eq_rank = eq_seen + block_prefix_count(eq, s_wave, &eq_tot);
    const bool sel = gt || (eq && eq_rank < need);
    const int pos = written + block_prefix_count(sel, s_wave, &sel_tot);
    if (sel && pos < k) out[pos] = p;
    eq_seen += eq_tot;
    written += sel_tot;
  }
}

hipError_t launch_h2o_select(const float* scores, int stride, const int32_t* lens, int num_seqs, int max_len,
                             int budget, int recent, int32_t* keep_idx, int32_t* keep_count, hipStream_t st) {
  if (num_seqs == 0) return hipSuccess;
  hipLaunchKernelGGL(h2o_select_kernel, dim3(num_seqs), dim3(kSelThreads), 0, st, scores, stride, lens, max_len,
                     budget, recent, keep_idx, keep_count);
  return hipGetLastError();
}

}  // namespace pkv
