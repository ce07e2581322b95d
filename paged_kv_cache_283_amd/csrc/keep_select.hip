// Eviction keep-sets for gfx950.
//
// Three rules of the pages share one shape: positions forced in (the first
// num_sinks and the last `recent`) united with the `heavy` highest accumulated
// scores of a candidate set, listed in ascending order.
//  * page "长上下文优化：注意力稀疏化与 KV Cache 管理" (plumephp.com/llm-long-context-optimization),
//    H2OEviction.select: the recent window plus the top scores of the earlier
//    positions (candidates = positions not forced, no sinks);
//  * page "KV Cache 与 PagedAttention：显存复用与长上下文推理", block 组合, should_cache:
//    sinks, recent window, and the top scores over every position
//    (candidates = all positions; the sets may overlap);
//  * page "系统优化" 4.2, evict_tokens: the top `budget` scores, nothing forced.
// Ties go to the lower position; NaN ranks like -inf; -0 equals +0.
//
// One workgroup per sequence.  The heavy-th largest candidate score is found
// by an exact 4-pass radix select (8 bits per pass, LDS histogram) on
// order-preserving 32-bit keys; a final pass in position order keeps forced
// positions, candidate keys above the threshold and the first still-needed
// keys equal to it, and compacts them with ballot prefix counts, which yields
// ascending output without a sort.
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

__global__ void __launch_bounds__(kSelThreads) keep_select_kernel(const float* scores, int stride, const int32_t* lens,
                                                                int max_len, int num_sinks, int recent, int heavy,
                                                                int all_candidates, int32_t* keep_idx, int keep_stride,
                                                                int32_t* keep_count) {
  __shared__ int hist[256];
  __shared__ int s_wave[kSelWaves];
  __shared__ int s_pick[2];
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  const int L = lens[s];
  int32_t* out = keep_idx + (size_t)s * keep_stride;
  if (L < 1 || L > max_len) {
    for (int i = tid; i < keep_stride; i += kSelThreads) out[i] = -1;
    if (tid == 0) keep_count[s] = -1;
    return;
  }
  const float* row = scores + (size_t)s * stride;
  // forced: p < sinks or p >= rec_lo; candidates: [c_lo, c_hi)
  const int sinks = min(num_sinks, L);
  const int rec_lo = L - min(recent, L);
  const int c_lo = all_candidates ? 0 : sinks;
  const int c_hi = all_candidates ? L : max(rec_lo, sinks);
  const int n_cand = c_hi - c_lo;
  const int k = min(heavy, n_cand);
  const bool take_all = k == n_cand;

  // Radix select of the k-th largest candidate key, most significant byte first.
  // The first kKeyRegs * 1024 candidate keys stay in registers across the
  // passes (loaded together, one memory latency); longer rows re-read the rest.
  constexpr int kKeyRegs = 8;
  uint32_t kc[kKeyRegs];
  float kf[kKeyRegs];   // the final pass's scores of positions tid + 1024 i, loaded with them
#pragma unroll
  for (int i = 0; i < kKeyRegs; ++i) {
    const int p = c_lo + tid + i * kSelThreads;
    kc[i] = p < c_hi ? score_key(row[p]) : 0u;
    const int q = tid + i * kSelThreads;
    kf[i] = q < L ? row[q] : 0.f;
  }
  uint32_t prefix = 0u, mask = 0u;
  int need = k;
  if (!take_all && k > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kKeyRegs; ++i) {
        if (c_lo + tid + i * kSelThreads < c_hi && (kc[i] & mask) == prefix)
          atomicAdd(&hist[(kc[i] >> shift) & 255u], 1);
      }
      for (int p = c_lo + tid + kKeyRegs * kSelThreads; p < c_hi; p += kSelThreads) {
        const uint32_t key = score_key(row[p]);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid < kWave) {
        // The digit holding the need-th largest remaining key, by the first
        // wave: lane l takes digits 255 - 4l .. 252 - 4l, a lane scan gives the
        // count of keys above its digits, and the one (lane, digit) where the
        // running count first reaches `need` records it.
        int h[4], local = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          h[e] = hist[255 - 4 * tid - e];
          local += h[e];
        }
        int incl = local;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
          const int t = __shfl_up(incl, off, kWave);
          if (tid >= off) incl += t;
        }
        int cum = incl - local;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c2 = cum + h[e];
          if (cum < need && c2 >= need) {
            s_pick[0] = 255 - 4 * tid - e;
            s_pick[1] = need - cum;
          }
          cum = c2;
        }
      }
      __syncthreads();
      prefix |= (uint32_t)s_pick[0] << shift;
      mask |= 255u << shift;
      need = s_pick[1];
      __syncthreads();
    }
  }
  const uint32_t thresh = prefix;   // the k-th largest key; `need` keys equal to it are taken

  int eq_seen = 0, written = 0;
  // One position per thread and step, in position order (the steps are
  // uniform, so the barriers inside are reached by every thread).
  auto step = [&](int p, float score) {
    const bool in_c = p >= c_lo && p < c_hi;
    const uint32_t key = in_c && !take_all && k > 0 ? score_key(score) : 0u;
    const bool eq = in_c && !take_all && k > 0 && key == thresh;
    int eq_tot, sel_tot;
    const int eq_rank = eq_seen + block_prefix_count(eq, s_wave, &eq_tot);
    const bool hv = in_c && (take_all || (k > 0 && (key > thresh || (eq && eq_rank < need))));
    const bool sel = p < L && (p < sinks || p >= rec_lo || hv);
    const int pos = written + block_prefix_count(sel, s_wave, &sel_tot);
    if (sel && pos < keep_stride) out[pos] = p;
    eq_seen += eq_tot;
    written += sel_tot;
  };
#pragma unroll
  for (int i = 0; i < kKeyRegs; ++i) {
    if (i * kSelThreads < L) step(i * kSelThreads + tid, kf[i]);
  }
  for (int base = kKeyRegs * kSelThreads; base < L; base += kSelThreads) {
    const int p = base + tid;
    step(p, p < L ? row[p] : 0.f);
  }
  for (int i = written + tid; i < keep_stride; i += kSelThreads) out[i] = -1;
  if (tid == 0) keep_count[s] = written;
}

hipError_t launch_keep_select(const float* scores, int stride, const int32_t* lens, int num_seqs, int max_len,
                              int num_sinks, int recent, int heavy, int all_candidates, int32_t* keep_idx,
                              int keep_stride, int32_t* keep_count, hipStream_t st) {
  if (num_seqs == 0) return hipSuccess;
  hipLaunchKernelGGL(keep_select_kernel, dim3(num_seqs), dim3(kSelThreads), 0, st, scores, stride, lens, max_len,
                     num_sinks, recent, heavy, all_candidates, keep_idx, keep_stride, keep_count);
  return hipGetLastError();
}

}  // namespace pkv
