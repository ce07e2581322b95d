// Causal multi-query attention over a paged KV cache for gfx950: the chunked
// prefill of a long prompt, or the continuation of a request whose prefix came
// from the prefix cache.
//
// Page "系统优化" 4.5 ("Chunked Prefill": a long prompt is processed in chunks
// interleaved with decode steps; "分页 KV Cache + 前缀缓存": the cache is paged and
// prefixes are shared) and page "KV Cache 与 PagedAttention：显存复用与长上下文推理",
// "共享场景的价值" (a prefix-cache hit skips the prefill of the shared part).
// The chunk of n_q query tokens of sequence s is its last n_q positions, whose
// K/V are already in the cache; query i (position p_i = L - n_q + i) attends to
// positions 0..p_i:
//   out[i][h] = sum_{p <= p_i} softmax_p(scale * q[i][h] . K[p][h/G]) * V[p][h/G]
//
// How, on gfx950: the decode kernel's MFMA tile with its 16 B-operand columns
// used as (query token, head) pairs -- 16/G tokens x G heads per wave -- so a
// wave computes S = K q^T for 16 query rows with one 16x16x32 MFMA per 32 head
// dims and PV with the probabilities straight from the QK accumulator.  Each
// column carries its own causal limit (a per-lane mask on the logits).  For
// long chunks a wave carries several such 16-column sets (PKV_PREFILL_SETS):
// each K/V tile it loads feeds one MFMA per set, so the tiles pulled from L2
// per query token drop by that factor.  A workgroup is 4 waves of consecutive
// query tokens of one (sequence, KV head); its waves walk the same blocks, so
// the tiles come from HBM once and from the caches for the other waves.  Work
// is split by query token only: every wave covers the whole causal range of
// its tokens, two blocks per step so that PV runs as 16x16x32 MFMAs over both
// blocks' 32 keys.
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"
#include "mfma_ops.hpp"

namespace pkv {

namespace {

constexpr int kPfWaves = 4;
constexpr int kPfTab = 1024;              // table entries staged per wave and chunk
constexpr float kPfRescaleSlack = 8.f;    // base-2 slack before accumulators are rescaled

}  // namespace

#ifndef PKV_PREFILL_SETS
#define PKV_PREFILL_SETS 2                // 16-column query sets per wave for long chunks
#endif


namespace {

}  // namespace

template <int KVT, int QT, int D, int CS>
__global__ void __launch_bounds__(256) prefill_kernel(const PrefillArgs a) {
  using KT = KvType<KVT>;
  constexpr int EB = KT::kBytes;
  constexpr bool OP32 = KT::kOp32;
  constexpr bool F16 = KT::kOpF16;
  constexpr int DPL = D / 4;
  constexpr int KW = DPL * EB / 4;
  constexpr int NT = D / 16;
  constexpr int VW = EB;
  constexpr bool CH = is_channel_scaled(KVT);   // static per-channel scales, folded into q and the output
  constexpr bool BIAS = code_biased<KVT>();      // INT8 operands are code + kInt8Bias
  constexpr bool QSAME = (!OP32) && (QT == (F16 ? DT_F16 : DT_BF16)) && !CH;
  constexpr bool QSPLIT = (!OP32) && !QSAME;
  constexpr int QW = OP32 ? 1 : DPL / 2;
  __shared__ int s_tab_all[kPfWaves][kPfTab];

  const int hq = a.num_q_heads;
  const int hkv = a.num_kv_heads;
  const int group = hq / hkv;
  const int tpw = 16 / group;                    // query tokens per column set
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int j = lane >> 4;
  int* s_tab = s_tab_all[wave];

  // Workgroup -> (sequence, KV head, tile).  With a pair count divisible by 8,
  // all tiles of a (sequence, KV head) go to one XCD (ids are dealt to the 8
  // XCDs in turn), so the waves re-reading its blocks share that XCD's L2.
  const int tiles = a.tiles_per_pair;
  const int pairs = a.num_seqs * hkv;
  int pair, tile;
  if ((pairs & 7) == 0) {
    const int xcd = blockIdx.x & 7, k = blockIdx.x >> 3;
    pair = (k / tiles) * 8 + xcd;
    tile = k % tiles;
  } else {
    pair = blockIdx.x / tiles;
    tile = blockIdx.x % tiles;
  }
  const int s = pair / hkv, kvh = pair % hkv;
  const int q0 = a.query_start[s];
  const int n_q = a.query_start[s + 1] - q0;
  const int L = a.context_lens[s];
  const int t0 = (tile * kPfWaves + wave) * CS * tpw;   // first query token of this wave
  if (q0 < 0 || n_q < 1 || n_q > a.num_tokens - q0 || t0 >= n_q) return;   // rows outside q/out: skip
  const int prefix = L - n_q;
  const bool seq_ok = L >= n_q && L <= a.max_context_len && L <= a.table_stride * kBlockSize;

  // ---- column c of set cs = (query token t0 + cs * tpw + c / G, head kvh * G + c % G)
  const int head = kvh * group + c % group;
  int tok[CS], pos[CS];
  bool col_ok[CS];
  uint32_t qhi[CS][QW];
  uint32_t qlo[CS][QSPLIT ? QW : 1];
  float qf[CS][OP32 ? DPL : 1];
#pragma unroll
  for (int cs = 0; cs < CS; ++cs) {
    tok[cs] = t0 + cs * tpw + c / group;
    col_ok[cs] = tok[cs] < n_q;
    pos[cs] = col_ok[cs] ? prefix + tok[cs] : -1;    // causal limit of the column (-1: no keys)
    const size_t qrow = ((size_t)(q0 + (col_ok[cs] ? tok[cs] : 0)) * hq + head) * D;
    if constexpr (OP32) {
#pragma unroll
      for (int st = 0; st < DPL; ++st)
        qf[cs][st] = col_ok[cs] ? load_q_elem<QT>(a.q, qrow + qk_dim_f32(st, j)) : 0.f;
    } else if constexpr (QSAME) {
      const uint16_t* qh = reinterpret_cast<const uint16_t*>(a.q) + qrow;
#pragma unroll
      for (int st = 0; st < QW / 4; ++st) {
        const u32x4 v = col_ok[cs] ? *reinterpret_cast<const u32x4*>(qh + qk_dim16<KVT>(st, j)) : u32x4{0, 0, 0, 0};
        qhi[cs][4 * st + 0] = v[0]; qhi[cs][4 * st + 1] = v[1]; qhi[cs][4 * st + 2] = v[2]; qhi[cs][4 * st + 3] = v[3];
      }
    } else {
#pragma unroll
      for (int st = 0; st < QW / 4; ++st) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int d0 = qk_dim16<KVT>(st, j) + 2 * w;
          float f0 = col_ok[cs] ? load_q_elem<QT>(a.q, qrow + d0) : 0.f;
          float f1 = col_ok[cs] ? load_q_elem<QT>(a.q, qrow + d0 + 1) : 0.f;
          if constexpr (CH) {   // q . (code * s) = (q * s) . code, with q * s carried as hi + lo
            f0 *= a.k_scale[(size_t)kvh * D + d0];
            f1 *= a.k_scale[(size_t)kvh * D + d0 + 1];
          }
          const uint32_t h0 = to_op16<F16>(f0), h1 = to_op16<F16>(f1);
          const uint32_t l0 = to_op16<F16>(f0 - from_op16<F16>(h0));
          const uint32_t l1 = to_op16<F16>(f1 - from_op16<F16>(h1));
          qhi[cs][4 * st + w] = h0 | (h1 << 16);
          qlo[cs][4 * st + w] = l0 | (l1 << 16);
        }
      }
    }
  }

  // Biased K operands add kInt8Bias * (sum of the column's q operand values) to every logit.
  float qbias[CS];
#pragma unroll
  for (int cs = 0; cs < CS; ++cs) {
    qbias[cs] = 0.f;
    if constexpr (BIAS) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < QW; ++w) {
        sum += from_op16<F16>(qhi[cs][w] & 0xffffu) + from_op16<F16>(qhi[cs][w] >> 16);
        if constexpr (QSPLIT) sum += from_op16<F16>(qlo[cs][w] & 0xffffu) + from_op16<F16>(qlo[cs][w] >> 16);
      }
      qbias[cs] = kInt8Bias * row_sum4(sum);
    }
  }

  float m_run[CS], l_run[CS];
  float p_run[CS];   // biased V operands: this lane's share of the sum of P operand values
  f32x4 acc[CS][NT];
#pragma unroll
  for (int cs = 0; cs < CS; ++cs) {
    p_run[cs] = 0.f;
    m_run[cs] = -INFINITY;
    l_run[cs] = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[cs][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bool bad = !seq_ok;

  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_pool);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v_pool);
  const int32_t* trow = a.block_tables + (size_t)s * a.table_stride;
  // Keys the wave needs: 0 .. prefix + its last token; keys below prefix + t0
  // are visible to every column (no mask there).
  const int t_last = min(t0 + CS * tpw, n_q) - 1;
  const int n_blocks = seq_ok ? (prefix + t_last) / kBlockSize + 1 : 0;
  const int all_visible = prefix + t0;
  int c0 = 0;

  struct Regs {
    // Held as the loaded 16-byte vectors: operands are then built by element
    // selects, never through a word array the compiler could widen into
    // memory accesses.
    u32x4 kq[KW / 4];
    u32x4 vq[NT * VW / 4];
    __device__ uint32_t k(int w) const { return kq[w / 4][w % 4]; }
    __device__ uint32_t v(int t, int e) const { return vq[(t * VW + e) / 4][(t * VW + e) % 4]; }
    __device__ void set_v(int t, int e, uint32_t x) { vq[(t * VW + e) / 4][(t * VW + e) % 4] = x; }
    f32x4 ks, vs;
    bool ok;
  };

  // Loads of block i's tiles into r (K and V halves separately, so a step can
  // refill K while it still uses V).  An entry outside the pool reads block 0
  // instead (in bounds) and marks r bad.
  auto tile_of = [&](Regs& r, int i) {
    const int phys = __builtin_amdgcn_readfirstlane(s_tab[i]);
    r.ok = phys >= 0 && phys < a.num_blocks;
    return (size_t)(r.ok ? phys : 0) * hkv + kvh;
  };
  auto load_k = [&](Regs& r, int i) {
    const size_t tile_i = tile_of(r, i);
    const uint8_t* kt = kbase + tile_i * (size_t)(kBlockSize * D * EB);
#pragma unroll
    for (int w = 0; w < KW / 4; ++w) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(kt + ((size_t)(4 * w + j) * kBlockSize + c) * 16);
      r.kq[w] = v;
    }
    if constexpr (is_quantised(KVT)) r.ks = *reinterpret_cast<const f32x4*>(a.k_scale + tile_i * kBlockSize + 4 * j);
  };
  auto load_v = [&](Regs& r, int i) {
    const size_t tile_i = tile_of(r, i);
    const uint8_t* vt = vbase + tile_i * (size_t)(kBlockSize * D * EB);
#pragma unroll
    for (int g = 0; g < NT * VW / 4; ++g) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(vt + ((size_t)(g * 16 + c) * 4 + j) * 16);
      r.vq[g] = v;
    }
    if constexpr (is_quantised(KVT)) r.vs = *reinterpret_cast<const f32x4*>(a.v_scale + tile_i * kBlockSize + 4 * j);
  };
  auto load = [&](Regs& r, int i) {
    load_k(r, i);
    load_v(r, i);
  };

  // S = K q^T of one block for every column set, sharing the converted K operand.
  auto qk = [&](const Regs& r, f32x4* sacc) {
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) sacc[cs] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (OP32) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
#pragma unroll
        for (int cs = 0; cs < CS; ++cs) sacc[cs] = mfma_f32_k4(__uint_as_float(r.k(e)), qf[cs][e], sacc[cs]);
      }
    } else {
#pragma unroll
      for (int st = 0; st < DPL / 8; ++st) {
        uint32_t av[4];
        if constexpr (is_code8(KVT)) {
          code8x4_to_bf16x4<KVT>(r.k(2 * st), av[0], av[1]);
          code8x4_to_bf16x4<KVT>(r.k(2 * st + 1), av[2], av[3]);
        } else {
          av[0] = r.k(4 * st); av[1] = r.k(4 * st + 1); av[2] = r.k(4 * st + 2); av[3] = r.k(4 * st + 3);
        }
#pragma unroll
        for (int cs = 0; cs < CS; ++cs) {
          sacc[cs] = mfma_k32<F16>(av, &qhi[cs][4 * st], sacc[cs]);
          if constexpr (QSPLIT) sacc[cs] = mfma_k32<F16>(av, &qlo[cs][4 * st], sacc[cs]);
        }
      }
    }
  };

  // Keys past the context (the unused tail of the last block): V zeroed.
  auto mask_tail = [&](Regs& r, int blk0, bool* in_ctx) {
#pragma unroll
    for (int e = 0; e < 4; ++e) in_ctx[e] = blk0 + 4 * j + e < L;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if constexpr (VW == 1) {
        const uint32_t msk = (in_ctx[0] ? 0xffu : 0u) | (in_ctx[1] ? 0xff00u : 0u) |
                             (in_ctx[2] ? 0xff0000u : 0u) | (in_ctx[3] ? 0xff000000u : 0u);
        r.set_v(t, 0, r.v(t, 0) & msk);
      } else if constexpr (VW == 2) {
        r.set_v(t, 0, r.v(t, 0) & ((in_ctx[0] ? 0xffffu : 0u) | (in_ctx[1] ? 0xffff0000u : 0u)));
        r.set_v(t, 1, r.v(t, 1) & ((in_ctx[2] ? 0xffffu : 0u) | (in_ctx[3] ? 0xffff0000u : 0u)));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) r.set_v(t, e, in_ctx[e] ? r.v(t, e) : 0u);
      }
    }
  };

  // V tile t of one block as the 16-bit PV A operand (two words: tokens 4j..4j+3 of dim 16t + c).
  auto v_operand = [&](const Regs& r, int t, uint32_t& v0, uint32_t& v1) {
    if constexpr (is_code8(KVT)) {
      code8x4_to_bf16x4<KVT>(r.v(t, 0), v0, v1);
    } else {
      v0 = r.v(t, 0);
      v1 = r.v(t, 1);
    }
  };

  // One step over the blocks i (ra) and i + 1 (rb, only if has_b): QK, the
  // online softmax over the step's keys, PV.  Each PV MFMA is a 16x16x32 whose
  // 32 keys are both blocks' 16: lane (c, j) holds tokens 4j..4j+3 of block i,
  // then of block i + 1, in the V operand and the probability operand alike,
  // so the contraction pairs them correctly and one instruction does the work
  // of two 16x16x16 ones (which run at half the rate per flop on gfx950).
  // Without a second block its logits are -inf and its V operand zero.
  // With refill, the next pair's K loads (blocks i + 2, i + 3) are issued as
  // soon as this step's QK MFMAs have consumed K.
  constexpr int NB = 2;
  auto compute = [&](Regs& ra, Regs& rb, int i, bool has_b, bool refill) {
    // (ra and rb are named explicitly, never selected by index: a reference
    // chosen at run time would keep the register buffers in memory.)
    f32x4 sacc[NB][CS];
    bool full[NB];
    bool in_ctx[NB][4];
    int blk0[NB];
    float ksc[NB][4], vsc[NB][4];
    bad |= !ra.ok || (has_b && !rb.ok);
    blk0[0] = (c0 + i) * kBlockSize;
    blk0[1] = blk0[0] + kBlockSize;
    qk(ra, sacc[0]);
    qk(rb, sacc[1]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ksc[0][e] = is_quantised(KVT) ? ra.ks[e] : 1.f;
      ksc[1][e] = is_quantised(KVT) ? rb.ks[e] : 1.f;
      vsc[0][e] = is_quantised(KVT) ? ra.vs[e] : 1.f;
      vsc[1][e] = is_quantised(KVT) ? rb.vs[e] : 1.f;
      in_ctx[0][e] = in_ctx[1][e] = true;
    }
    if (refill) {
      load_k(ra, i + 2);
      load_k(rb, i + 3);
    }
    full[0] = blk0[0] + kBlockSize <= all_visible;
    full[1] = blk0[1] + kBlockSize <= all_visible && has_b;
    if (!full[0]) mask_tail(ra, blk0[0], in_ctx[0]);
    if (!full[1]) mask_tail(rb, has_b ? blk0[1] : L, in_ctx[1]);   // an absent block lies wholly past L
    // ---- per column set: causal mask, online softmax, probabilities as PV operands
    uint32_t ph[CS][2 * NB], pl[CS][2 * NB];
    float pvv[CS][NB][4];
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) {
      float x[NB][4];
      float mx = -INFINITY;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = (BIAS ? sacc[b][cs][e] - qbias[cs] : sacc[b][cs][e]) * a.scale_log2;
          if constexpr (is_quantised(KVT)) v *= ksc[b][e];
          if (!full[b]) v = in_ctx[b][e] && blk0[b] + 4 * j + e <= pos[cs] ? v : -INFINITY;
          x[b][e] = v;
        }
        mx = fmaxf(mx, fmaxf(fmaxf(x[b][0], x[b][1]), fmaxf(x[b][2], x[b][3])));
      }
      const float mb = row_max4(mx);
      const bool need = mb > m_run[cs] + kPfRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(need) != 0ull) {
        const float m_new = need ? mb : m_run[cs];
        const float alpha = m_new == m_run[cs] ? 1.f : fast_exp2(m_run[cs] - m_new);
        l_run[cs] *= alpha;
        if constexpr (BIAS) p_run[cs] *= alpha;
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[cs][t] *= alpha;
        m_run[cs] = m_new;
      }
      const float mref = m_run[cs] == -INFINITY ? 0.f : m_run[cs];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float pr[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pr[e] = fast_exp2(x[b][e] - mref);
        l_run[cs] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (is_quantised(KVT)) pvv[cs][b][e] = in_ctx[b][e] ? pr[e] * vsc[b][e] : 0.f;
          else pvv[cs][b][e] = pr[e];
        }
        if constexpr (!OP32) {
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            const float f0 = pvv[cs][b][2 * w], f1 = pvv[cs][b][2 * w + 1];
            uint32_t h0, h1, l0, l1;
            if constexpr (F16) {
              h0 = f32_to_f16_bits(f0);
              h1 = f32_to_f16_bits(f1);
              l0 = f32_to_f16_bits(f0 - f16_to_f32(h0));
              l1 = f32_to_f16_bits(f1 - f16_to_f32(h1));
            } else {
              h0 = __float_as_uint(f0) >> 16;
              h1 = __float_as_uint(f1) >> 16;
              l0 = __float_as_uint(f0 - bf16_to_f32(h0)) >> 16;
              l1 = __float_as_uint(f1 - bf16_to_f32(h1)) >> 16;
              if constexpr (BIAS)
                p_run[cs] += (bf16_to_f32(h0) + bf16_to_f32(l0)) + (bf16_to_f32(h1) + bf16_to_f32(l1));
            }
            ph[cs][2 * b + w] = h0 | (h1 << 16);
            pl[cs][2 * b + w] = l0 | (l1 << 16);
          }
        }
      }
    }
    // ---- O^T += V^T P^T per set, sharing the converted V operand
    if constexpr (OP32) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
          for (int cs = 0; cs < CS; ++cs) {
            acc[cs][t] = mfma_f32_k4(__uint_as_float(ra.v(t, e)), pvv[cs][0][e], acc[cs][t]);
            acc[cs][t] = mfma_f32_k4(__uint_as_float(rb.v(t, e)), pvv[cs][1][e], acc[cs][t]);
          }
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        uint32_t av[4];
        v_operand(ra, t, av[0], av[1]);
        v_operand(rb, t, av[2], av[3]);
#pragma unroll
        for (int cs = 0; cs < CS; ++cs) {
          acc[cs][t] = mfma_k32<F16>(av, ph[cs], acc[cs][t]);
          acc[cs][t] = mfma_k32<F16>(av, pl[cs], acc[cs][t]);
        }
      }
    }
  };
  // An absent second block: defined (zero) operands; its keys are masked.
  auto clear = [&](Regs& r) {
#pragma unroll
    for (int w = 0; w < KW / 4; ++w) r.kq[w] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int g = 0; g < NT * VW / 4; ++g) r.vq[g] = u32x4{0u, 0u, 0u, 0u};
    r.ks = r.vs = f32x4{0.f, 0.f, 0.f, 0.f};
    r.ok = true;
  };

  for (; c0 < n_blocks; c0 += kPfTab) {
    const int n = min(kPfTab, n_blocks - c0);
    // 512 entries per memory latency: every lane issues 8 entry loads before
    // the first is waited for (indices past the chunk reload its last entry)
    for (int b0 = 0; b0 < n; b0 += kWave * 8) {
      int ent[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) ent[u] = trow[c0 + min(b0 + lane + kWave * u, n - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = b0 + lane + kWave * u;
        if (k < n) s_tab[k] = ent[u];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    // Pairs of blocks in two buffers: the next pair's K loads are issued as
    // soon as the QK MFMAs have consumed K, its V loads once PV has consumed V.
    Regs r0, r1;
    int i = 0;
    if (n > 0) load(r0, 0);
    if (n > 1) load(r1, 1);
    for (; i + 3 < n; i += 2) {   // steady state: the next pair exists, loads unconditional
      compute(r0, r1, i, true, true);
      load_v(r0, i + 2);
      load_v(r1, i + 3);
    }
    const int rem = n - i;        // 0..3 blocks left; r0, r1 hold blocks i, i + 1 where they exist
    if (rem >= 2) compute(r0, r1, i, true, false);
    if (rem % 2) {                // one block left over: paired with an absent one
      Regs rz;
      clear(rz);
      if (rem == 3) load(r0, i + 2);
      compute(r0, rz, rem == 3 ? i + 2 : i, false, false);
    }
    __builtin_amdgcn_wave_barrier();   // the next chunk rewrites this wave's s_tab
  }

#pragma unroll
  for (int cs = 0; cs < CS; ++cs) {
    float l = row_sum4(l_run[cs]);
    if (bad) l = __builtin_nanf("");
    const float vbias = BIAS ? kInt8Bias * row_sum4(p_run[cs]) : 0.f;   // biased V operands
    if (!col_ok[cs]) continue;
    const size_t orow = ((size_t)(q0 + tok[cs]) * hq + head) * D;
    const float inv = 1.f / l;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f32x4 o = acc[cs][t];
      if constexpr (BIAS) o -= vbias;
      if constexpr (CH) o *= *reinterpret_cast<const f32x4*>(a.v_scale + (size_t)kvh * D + 16 * t + 4 * j);
#pragma unroll
      for (int e = 0; e < 4; ++e) store_out(a.out, orow + 16 * t + 4 * j + e, a.out_dtype, o[e] * inv);
    }
  }
}

namespace {

template <int KVT, int QT>
hipError_t prefill_d(PrefillArgs a, int d, int max_query_len, hipStream_t st) {
  // Column sets per wave: PKV_PREFILL_SETS for chunks long enough to fill them, else one.
  const int tpw = 16 / (a.num_q_heads / a.num_kv_heads);
  const bool wide = max_query_len >= kPfWaves * tpw * PKV_PREFILL_SETS;
  const int per_wg = kPfWaves * tpw * (wide ? PKV_PREFILL_SETS : 1);
  a.tiles_per_pair = (max_query_len + per_wg - 1) / per_wg;
  const int pairs = a.num_seqs * a.num_kv_heads;
  const dim3 grid((unsigned)pairs * a.tiles_per_pair);
  if (wide) {
    if (d == 64) hipLaunchKernelGGL((prefill_kernel<KVT, QT, 64, PKV_PREFILL_SETS>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((prefill_kernel<KVT, QT, 128, PKV_PREFILL_SETS>), grid, dim3(256), 0, st, a);
  } else {
    if (d == 64) hipLaunchKernelGGL((prefill_kernel<KVT, QT, 64, 1>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((prefill_kernel<KVT, QT, 128, 1>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

template <int KVT>
hipError_t prefill_q(const PrefillArgs& a, int q_dtype, int d, int mq, hipStream_t st) {
  switch (q_dtype) {
    case DT_F32: return prefill_d<KVT, DT_F32>(a, d, mq, st);
    case DT_BF16: return prefill_d<KVT, DT_BF16>(a, d, mq, st);
    default: return prefill_d<KVT, DT_F16>(a, d, mq, st);
  }
}

}  // namespace

hipError_t launch_prefill_attn(const PrefillArgs& a, int kv_dtype, int q_dtype, int head_dim, int max_query_len,
                               hipStream_t st) {
  if (a.num_seqs == 0 || max_query_len < 1) return hipSuccess;
  switch (kv_dtype) {
    case DT_F32: return prefill_q<DT_F32>(a, q_dtype, head_dim, max_query_len, st);
    case DT_BF16: return prefill_q<DT_BF16>(a, q_dtype, head_dim, max_query_len, st);
    case DT_F16: return prefill_q<DT_F16>(a, q_dtype, head_dim, max_query_len, st);
    case DT_FP8: return prefill_q<DT_FP8>(a, q_dtype, head_dim, max_query_len, st);
    case DT_INT8: return prefill_q<DT_INT8>(a, q_dtype, head_dim, max_query_len, st);
    case DT_FP8_CH: return prefill_q<DT_FP8_CH>(a, q_dtype, head_dim, max_query_len, st);
    default: return prefill_q<DT_INT8_CH>(a, q_dtype, head_dim, max_query_len, st);
  }
}

}  // namespace pkv
