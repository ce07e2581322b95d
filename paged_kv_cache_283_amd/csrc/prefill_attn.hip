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
// blocks' 32 keys.  Steps whose keys every column of the wave sees (all but
// the last one or two of a wave) take a path with no mask at all, where the
// logit factor enters the exponent's fma; the factor's sign is folded into the
// query operands so that the running max is taken on the raw products.
// 16-bit pools stage each block pair once per workgroup in an LDS ring and run
// PV in f16 (bf16 V rewritten to f16 in the ring, one probability operand per
// tile); a workgroup whose values leave f16's range computes again with the
// bf16 high/low probability split.
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"
#include "mfma_ops.hpp"

namespace pkv {

#ifndef PKV_PREFILL_PRIO
#define PKV_PREFILL_PRIO 1   // wave priority over a run of MFMAs (0: leave it)
#endif

// Two waves share each SIMD: a wave's block of MFMAs runs at raised priority,
// so its next MFMA issues as soon as the matrix core takes it while the other
// wave's softmax VALU work fills the cycles in between.
__device__ __forceinline__ void mfma_phase(bool on) {
  if constexpr (PKV_PREFILL_PRIO > 0) {
    if (on) __builtin_amdgcn_s_setprio(PKV_PREFILL_PRIO);
    else __builtin_amdgcn_s_setprio(0);
  }
}

// Maximum for the softmax's running max: IEEE maximum (a NaN logit makes the
// max NaN, and the output is NaN either way), which gfx950 has as
// v_maximum3_f32; fmaxf's NaN-ignoring form needs every MFMA result
// canonicalised first (one v_max_f32 x, x per logit).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
// The same over the four 16-lane rows of an MFMA accumulator (lanes 16 and 32 apart).
__device__ __forceinline__ float row_vmax4(float x) {
  const uint32_t u = __float_as_uint(x);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t v = __float_as_uint(x);
  auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
// Two floats as one word of f16 MFMA operands, each rounded to nearest even
// (one v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2_t));
}
// A word of two bf16 values as two f16 values: exact over f16's normal range
// (bf16 carries 8 significant bits, f16 11), rounded to nearest below 2^-14,
// and +-inf above 65504 (round-to-nearest overflow).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return pack_f16x2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}

namespace {

constexpr int kPfWaves = 4;
constexpr int kPfTab = 1024;              // table entries staged per wave and chunk
constexpr float kPfRescaleSlack = 8.f;    // base-2 slack before accumulators are rescaled

}  // namespace

#ifndef PKV_PREFILL_SETS
#define PKV_PREFILL_SETS 2                // 16-column query sets per wave for long chunks
#endif
#ifndef PKV_PREFILL_STAGE
#define PKV_PREFILL_STAGE 1               // 16-bit pools: K/V block pairs staged once per workgroup in LDS
#endif
#ifndef PKV_PREFILL_STAGES
#define PKV_PREFILL_STAGES 4              // LDS ring slots (pairs in flight = slots - 1)
#endif
#ifndef PKV_PREFILL_ILV_LEAD
#define PKV_PREFILL_ILV_LEAD 8            // VALU instructions scheduled between the LDS reads and the first MFMA
#endif
#ifndef PKV_PREFILL_ILV_QK
#define PKV_PREFILL_ILV_QK 1              // VALU instructions scheduled after each QK MFMA of the next pair
#endif
#ifndef PKV_PREFILL_ILV_PV
#define PKV_PREFILL_ILV_PV 4              // ... after each PV MFMA of a column set but the last
#endif
#ifndef PKV_PREFILL_ILV_PVL
#define PKV_PREFILL_ILV_PVL 1             // ... after each PV MFMA of the last column set
#endif
#ifndef PKV_PREFILL_LATE_QK
#define PKV_PREFILL_LATE_QK 4             // QK MFMAs after the late LDS reads of a step (f16 rewrite)
#endif
#ifndef PKV_PREFILL_F16_ONE_MAX
#define PKV_PREFILL_F16_ONE_MAX 1         // f16 PV steps: the running max only from a chunk's first pair
#endif
#ifndef PKV_PREFILL_PV16
#define PKV_PREFILL_PV16 1                // 16-bit pools: PV as f16 x f16 with one probability operand
#endif

// One iteration of the LDS ring: this lane's K operand chunks of the next
// pair (slot at rk), its V operand chunks of the current pair (V rows at rv),
// the direct-to-LDS copy of one tile of a later pair into wr (LPS rows of
// 1 KiB: row k from src + k * 1024 to row row0 + row_step * k), and the table
// entry tab[next] (the tile the next iteration copies).  Every LDS access goes
// through the restrict parameters, so once inlined the compiler knows the copy
// writes none of what the reads return; otherwise each read waits for every
// copy in flight (vmcnt(0)) and the ring holds a single pair.
//
// With CONV, a later pair's V rows are rewritten in place from bf16 to f16
// and regrouped: rows 2g and 2g + 1 hold, per lane, chunk g of the first
// block's V tile (words 0-1: tile 2g, 2-3: tile 2g + 1) and of the second's;
// afterwards row t holds tile t's whole PV operand (first block's two words,
// then the second's), so the operand is one 16-byte read.  Wave w regroups
// chunk w (chunks past VQ: none).
__device__ __forceinline__ void regroup_v_f16(const u32x4& xa, const u32x4& xb, u32x4& t0, u32x4& t1) {
  t0 = u32x4{bf16x2_to_f16x2(xa[0]), bf16x2_to_f16x2(xa[1]), bf16x2_to_f16x2(xb[0]), bf16x2_to_f16x2(xb[1])};
  t1 = u32x4{bf16x2_to_f16x2(xa[2]), bf16x2_to_f16x2(xa[3]), bf16x2_to_f16x2(xb[2]), bf16x2_to_f16x2(xb[3])};
}
template <int VQ>
__device__ __forceinline__ void convert_v_rows(uint8_t* __restrict__ cv, int wave, int lane) {
  if (VQ >= 4 || wave < VQ) {
    const u32x4 xa = *reinterpret_cast<const u32x4*>(cv + (2 * wave) * 1024 + lane * 16);
    const u32x4 xb = *reinterpret_cast<const u32x4*>(cv + (2 * wave + 1) * 1024 + lane * 16);
    u32x4 t0, t1;
    regroup_v_f16(xa, xb, t0, t1);
    *reinterpret_cast<u32x4*>(cv + (2 * wave) * 1024 + lane * 16) = t0;
    *reinterpret_cast<u32x4*>(cv + (2 * wave + 1) * 1024 + lane * 16) = t1;
  }
}

// Direct-to-LDS copy of one K or V tile (LPS rows of 1 KiB; row k of the tile
// at base + k * 1024, lane l's 16 bytes from off + k * 1024, to LDS row
// row0 + row_step * k at dst).  A buffer load with the tile as its range: the
// compiler treats the global (flat-encoded) form as a possible LDS access that
// returns out of order, and then waits for every LDS read at the first use of
// one while a copy is in flight (always, in the ring).
template <int TB, int LPS>
__device__ __forceinline__ void copy_tile(const uint8_t* base, int off, uint8_t* __restrict__ dst, int row0,
                                          int row_step) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, TB, 0x00020000);
#pragma unroll
  for (int k = 0; k < LPS; ++k)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + (row0 + row_step * k) * 1024),
                                             16, off + k * 1024, 0, 0, 0);
}

template <int TB, int LPS, int KW4, int VQ, bool READ_V, bool CONV, class Body>
__device__ __forceinline__ int ring_io(const uint8_t* __restrict__ rk, const uint8_t* __restrict__ rv,
                                       uint8_t* __restrict__ wr, const int* __restrict__ tab, int next,
                                       const uint8_t* __restrict__ src, int src_off, int row0, int row_step, int c,
                                       int j, int lane,
                                       u32x4* ka, u32x4* kb, u32x4* va, u32x4* vb, uint8_t* __restrict__ cv,
                                       int wave, Body&& body) {
#pragma unroll
  for (int w = 0; w < KW4; ++w) {
    ka[w] = *reinterpret_cast<const u32x4*>(rk + ((4 * w + j) * kBlockSize + c) * 16);
    kb[w] = *reinterpret_cast<const u32x4*>(rk + TB + ((4 * w + j) * kBlockSize + c) * 16);
  }
  // Both are in lane order: lane l's 16 bytes of row r at r * 1024 + l * 16
  // (the copy of a V tile gathers each lane's chunk from where the pool keeps
  // it, so that these reads are conflict-free).
  auto read_v = [&](u32x4* dst, int parity) {
#pragma unroll
    for (int g = 0; g < VQ; ++g) dst[g] = *reinterpret_cast<const u32x4*>(rv + (2 * g + parity) * 1024 + lane * 16);
  };
  auto copy = [&]() { copy_tile<TB, LPS>(src, src_off, wr, row0, row_step); };
  int e = 0;
  if constexpr (!CONV) {
    if constexpr (READ_V) {
      read_v(va, 0);
      read_v(vb, 1);
      e = tab[next];
    }
    copy();
    __builtin_amdgcn_sched_barrier(0);   // the reads and the copy go out first, in their order
    body();
  } else {
    // Half the V reads go out with the K reads; the other half, the table
    // entry and the rewrite's reads go out inside the step's work (body,
    // whose scheduling hints place them after most of the QK MFMAs), so that
    // no more than 15 LDS reads are ever in flight (past that count the
    // first operand cannot be waited for alone: the wait is for all).  Every
    // ring access precedes the copy, issued last (a ring access after a copy
    // in the same iteration gets a wait for every copy in flight), and the
    // rewrite's arithmetic and stores follow the step's work.
    const bool conv_wave = VQ >= 4 || wave < VQ;
    u32x4 xa, xb;
    read_v(va, 0);
    __builtin_amdgcn_sched_barrier(0);
    read_v(vb, 1);
    e = tab[next];
    if (conv_wave) {
      xa = *reinterpret_cast<const u32x4*>(cv + (2 * wave) * 1024 + lane * 16);
      xb = *reinterpret_cast<const u32x4*>(cv + (2 * wave + 1) * 1024 + lane * 16);
    }
    body();
    __builtin_amdgcn_sched_barrier(0);
    if (conv_wave) {
      u32x4 t0, t1;
      regroup_v_f16(xa, xb, t0, t1);
      *reinterpret_cast<u32x4*>(cv + (2 * wave) * 1024 + lane * 16) = t0;
      *reinterpret_cast<u32x4*>(cv + (2 * wave + 1) * 1024 + lane * 16) = t1;
    }
    copy();
  }
  return e;
}

// Scheduling hint for the rest of the basic block: N MFMAs, each followed by
// up to V other vector-ALU instructions, so that one wave keeps the matrix
// core and the VALU busy together.
template <int N, int V>
__device__ __forceinline__ void interleave_mfma() {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
  }
}

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
  constexpr int VQ = NT * VW / 4;                // 16-byte V chunks per block
  // 16-bit pools: the workgroup's 4 waves walk the same blocks, so each block
  // pair is copied once into an LDS ring (direct global-to-LDS loads, one tile
  // per wave) and every wave builds its operands from there: the L2-to-CU
  // load instructions per MFMA drop by 4, and those are what bound the
  // register path (each wave loading every tile itself).
  constexpr bool STAGE = PKV_PREFILL_STAGE && EB == 2 && !OP32;
  constexpr int TB = kBlockSize * D * EB;        // bytes of one (block, KV head) tile
  constexpr int SB = 4 * TB;                     // one ring slot: K_a, K_b, then V_a / V_b by 1 KiB rows
  constexpr int NS = PKV_PREFILL_STAGES;
  constexpr int LPS = TB / 1024;                 // direct-to-LDS loads per wave and slot
  __shared__ int s_tab_all[STAGE ? 1 : kPfWaves][kPfTab];
  __shared__ __attribute__((aligned(16))) uint8_t s_ring[STAGE ? NS * SB : 16];
  __shared__ int s_redo;                         // f16 PV: some accumulator came out non-finite

  const int hq = a.num_q_heads;
  const int hkv = a.num_kv_heads;
  const int group = hq / hkv;
  const int tpw = 16 / group;                    // query tokens per column set
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int j = lane >> 4;
  int* s_tab = s_tab_all[STAGE ? 0 : wave];

  // Workgroup -> (sequence, KV head, tile).  With a pair count divisible by 8,
  // all tiles of a (sequence, KV head) go to one XCD (ids are dealt to the 8
  // XCDs in turn), so the waves re-reading its blocks share that XCD's L2.
  // Tiles are dealt last first: a later tile's tokens attend more keys, so
  // the longest workgroups start first and the short ones fill in at the end
  // (measured 1.07-1.10 -> 1.03 ms on 4 x 2048 after 6144).
  const int tiles = a.tiles_per_pair;
  const int pairs = a.num_seqs * hkv;
  int pair, tile;
  if ((pairs & 7) == 0) {
    const int xcd = blockIdx.x & 7, k = blockIdx.x >> 3;
    pair = (k / tiles) * 8 + xcd;
    tile = tiles - 1 - k % tiles;
  } else {
    pair = blockIdx.x / tiles;
    tile = tiles - 1 - blockIdx.x % tiles;
  }
  const int s = pair / hkv, kvh = pair % hkv;
  const int q0 = a.query_start[s];
  const int n_q = a.query_start[s + 1] - q0;
  const int L = a.context_lens[s];
  const int t0 = (tile * kPfWaves + wave) * CS * tpw;   // first query token of this wave
  const int t0_wg = tile * kPfWaves * CS * tpw;          // first query token of the workgroup
  // Rows outside q/out: skip.  With the LDS ring the workgroup stays together
  // (every wave takes part in the loads and barriers); a wave past the chunk
  // computes but stores nothing.
  if (q0 < 0 || n_q < 1 || n_q > a.num_tokens - q0 || (STAGE ? t0_wg : t0) >= n_q) return;
  const bool wave_live = t0 < n_q;
  const int prefix = L - n_q;
  const bool seq_ok = L >= n_q && L <= a.max_context_len && L <= a.table_stride * kBlockSize;

  // The logit factor's sign goes into q: q . k * scale = (-q) . k * |scale|, and
  // negating the 16-bit (or f32) operands flips sign bits only, so it is exact.
  // With a non-negative factor the largest logit is the largest raw product.
  const bool neg = a.scale_log2 < 0.f;
  const float sl2 = fabsf(a.scale_log2);
  const uint32_t qflip = neg ? 0x80008000u : 0u;

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
      for (int st = 0; st < DPL; ++st) {
        const float f = col_ok[cs] ? load_q_elem<QT>(a.q, qrow + qk_dim_f32(st, j)) : 0.f;
        qf[cs][st] = neg ? -f : f;
      }
    } else if constexpr (QSAME) {
      const uint16_t* qh = reinterpret_cast<const uint16_t*>(a.q) + qrow;
#pragma unroll
      for (int st = 0; st < QW / 4; ++st) {
        const u32x4 v = col_ok[cs] ? *reinterpret_cast<const u32x4*>(qh + qk_dim16<KVT>(st, j)) : u32x4{0, 0, 0, 0};
        qhi[cs][4 * st + 0] = v[0] ^ qflip; qhi[cs][4 * st + 1] = v[1] ^ qflip;
        qhi[cs][4 * st + 2] = v[2] ^ qflip; qhi[cs][4 * st + 3] = v[3] ^ qflip;
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
          qhi[cs][4 * st + w] = (h0 | (h1 << 16)) ^ qflip;
          qlo[cs][4 * st + w] = (l0 | (l1 << 16)) ^ qflip;
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
  // f16 PV steps: the column's normaliser, summed by one more MFMA from the
  // probability operands (every row of the result holds the column's sum).
  f32x4 lacc[CS];
#pragma unroll
  for (int cs = 0; cs < CS; ++cs) {
    p_run[cs] = 0.f;
    m_run[cs] = -INFINITY;
    l_run[cs] = 0.f;
    lacc[cs] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[cs][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bool bad = !seq_ok;

  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_pool);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v_pool);
  const int32_t* trow = a.block_tables + (size_t)s * a.table_stride;
  // Keys the wave needs: 0 .. prefix + its last token; keys below prefix + t0
  // are visible to every column (no mask there).
  // (with the ring: the last token of the workgroup, which all its waves walk to)
  const int t_last = min((STAGE ? t0_wg + kPfWaves * CS * tpw : t0 + CS * tpw), n_q) - 1;
  const int n_blocks = seq_ok ? (prefix + t_last) / kBlockSize + 1 : 0;
  const int all_visible = prefix + t0;
  int c0 = 0;

  // The two blocks (a, b) of one step, held as the loaded 16-byte vectors:
  // operands are built by element selects, never through a word array the
  // compiler could widen into memory accesses.  (Loading 16-bit V as 8-byte
  // pieces straight into each tile's operand quad saves the register moves that
  // assemble it, but doubles the load instructions, and the L2-to-CU path they
  // share is what bounds this kernel: measured 30% slower.)
  struct Pair {
    u32x4 ka[KW / 4], kb[KW / 4];
    u32x4 va[VQ], vb[VQ];
    f32x4 ksa, ksb, vsa, vsb;
    bool oka, okb;
  };
  // Word e of tile t of block a (B = false) or b (B = true).
  auto vword = [](const Pair& P, auto bsel, int t, int e) -> uint32_t {
    constexpr bool B = decltype(bsel)::value;
    return B ? P.vb[(t * VW + e) / 4][(t * VW + e) % 4] : P.va[(t * VW + e) / 4][(t * VW + e) % 4];
  };
  auto set_vword = [](Pair& P, auto bsel, int t, int e, uint32_t x) {
    constexpr bool B = decltype(bsel)::value;
    if constexpr (B) P.vb[(t * VW + e) / 4][(t * VW + e) % 4] = x;
    else P.va[(t * VW + e) / 4][(t * VW + e) % 4] = x;
  };
  constexpr std::false_type kA{};
  constexpr std::true_type kB{};
  // Two probabilities as packed 16-bit PV operands, high parts and residuals.
  auto pack_p = [](float f0, float f1, uint32_t& hw, uint32_t& lw) {
    if constexpr (F16) {
      const uint32_t h0 = f32_to_f16_bits(f0), h1 = f32_to_f16_bits(f1);
      const uint32_t l0 = f32_to_f16_bits(f0 - f16_to_f32(h0));
      const uint32_t l1 = f32_to_f16_bits(f1 - f16_to_f32(h1));
      hw = h0 | (h1 << 16);
      lw = l0 | (l1 << 16);
    } else {
      split_bf16_pair(f0, f1, hw, lw);
    }
  };

  // Loads of block i's tiles into half a or b of P (K and V separately, so a
  // step can refill K while it still uses V).  An entry outside the pool reads
  // block 0 instead (in bounds) and marks that half bad.
  auto tile_of = [&](int i, bool& ok) {
    const int phys = __builtin_amdgcn_readfirstlane(s_tab[i]);
    ok = phys >= 0 && phys < a.num_blocks;
    return (size_t)(ok ? phys : 0) * hkv + kvh;
  };
  auto load_k = [&](Pair& P, auto bsel, int i) {
    constexpr bool B = decltype(bsel)::value;
    bool ok;
    const size_t tile_i = tile_of(i, ok);
    const uint8_t* kt = kbase + tile_i * (size_t)(kBlockSize * D * EB);
#pragma unroll
    for (int w = 0; w < KW / 4; ++w) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(kt + ((size_t)(4 * w + j) * kBlockSize + c) * 16);
      if constexpr (B) P.kb[w] = v;
      else P.ka[w] = v;
    }
    if constexpr (is_quantised(KVT)) {
      const f32x4 sc = *reinterpret_cast<const f32x4*>(a.k_scale + tile_i * kBlockSize + 4 * j);
      if constexpr (B) P.ksb = sc;
      else P.ksa = sc;
    }
    if constexpr (B) P.okb = ok;
    else P.oka = ok;
  };
  auto load_v = [&](Pair& P, auto bsel, int i) {
    constexpr bool B = decltype(bsel)::value;
    bool ok;
    const size_t tile_i = tile_of(i, ok);
    const uint8_t* vt = vbase + tile_i * (size_t)(kBlockSize * D * EB);
#pragma unroll
    for (int g = 0; g < VQ; ++g) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(vt + ((size_t)(g * 16 + c) * 4 + j) * 16);
      if constexpr (B) P.vb[g] = v;
      else P.va[g] = v;
    }
    if constexpr (is_quantised(KVT)) {
      const f32x4 sc = *reinterpret_cast<const f32x4*>(a.v_scale + tile_i * kBlockSize + 4 * j);
      if constexpr (B) P.vsb = sc;
      else P.vsa = sc;
    }
  };

  // S = K q^T of one block for every column set, sharing the converted K operand.
  auto qk = [&](const u32x4* kq, f32x4* sacc) {
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) sacc[cs] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (OP32) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
#pragma unroll
        for (int cs = 0; cs < CS; ++cs)
          sacc[cs] = mfma_f32_k4(__uint_as_float(kq[e / 4][e % 4]), qf[cs][e], sacc[cs]);
      }
    } else {
#pragma unroll
      for (int st = 0; st < DPL / 8; ++st) {
        uint32_t av[4];
        if constexpr (is_code8(KVT)) {
          code8x4_to_bf16x4<KVT>(kq[st / 2][2 * (st % 2)], av[0], av[1]);
          code8x4_to_bf16x4<KVT>(kq[st / 2][2 * (st % 2) + 1], av[2], av[3]);
        } else {
          av[0] = kq[st][0]; av[1] = kq[st][1]; av[2] = kq[st][2]; av[3] = kq[st][3];
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
  auto mask_tail = [&](Pair& P, auto bsel, int blk0, bool* in_ctx) {
#pragma unroll
    for (int e = 0; e < 4; ++e) in_ctx[e] = blk0 + 4 * j + e < L;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if constexpr (VW == 1) {
        const uint32_t msk = (in_ctx[0] ? 0xffu : 0u) | (in_ctx[1] ? 0xff00u : 0u) |
                             (in_ctx[2] ? 0xff0000u : 0u) | (in_ctx[3] ? 0xff000000u : 0u);
        set_vword(P, bsel, t, 0, vword(P, bsel, t, 0) & msk);
      } else if constexpr (VW == 2) {
        set_vword(P, bsel, t, 0, vword(P, bsel, t, 0) & ((in_ctx[0] ? 0xffffu : 0u) | (in_ctx[1] ? 0xffff0000u : 0u)));
        set_vword(P, bsel, t, 1, vword(P, bsel, t, 1) & ((in_ctx[2] ? 0xffffu : 0u) | (in_ctx[3] ? 0xffff0000u : 0u)));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) set_vword(P, bsel, t, e, in_ctx[e] ? vword(P, bsel, t, e) : 0u);
      }
    }
  };

  // One step over the blocks i (half a) and i + 1 (half b, only if has_b): QK,
  // the online softmax over the step's keys, PV.  Each PV MFMA is a 16x16x32
  // whose 32 keys are both blocks' 16: lane (c, j) holds tokens 4j..4j+3 of
  // block i, then of block i + 1, in the V operand and the probability operand
  // alike, so the contraction pairs them correctly and one instruction does the
  // work of two 16x16x16 ones (which run at half the rate per flop on gfx950).
  // Without a second block its logits are -inf and its V operand zero.
  //
  // qk_step: S = K q^T for both blocks; with refill, the next pair's K loads
  // (blocks i + 2, i + 3) are issued as soon as the QK MFMAs have consumed K.
  constexpr int NB = 2;
  // The step's K scales (per-token formats) are taken before the refill overwrites them.
  auto qk_step = [&](Pair& P, f32x4 (&sacc)[NB][CS], f32x4 (&kscale)[NB], int i, bool has_b, bool refill) {
    bad |= !P.oka || (has_b && !P.okb);
    mfma_phase(true);
    qk(P.ka, sacc[0]);
    qk(P.kb, sacc[1]);
    mfma_phase(false);
    if constexpr (is_quantised(KVT)) {
      kscale[0] = P.ksa;
      kscale[1] = P.ksb;
    }
    if (refill) {
      load_k(P, kA, i + 2);
      load_k(P, kB, i + 3);
    }
  };
  // softmax_pv: the online softmax over the step's keys and PV.  Modes:
  //  kFull   every key of both blocks is inside the context and visible to
  //          every column: no mask is evaluated, and for formats without
  //          per-key scales the logit factor is applied inside the exponent,
  //          exp2(raw * |f| - (bias * |f| + m)), one fma per logit;
  //  kCausal every key is inside the context (the steady-state loop never
  //          reaches the sequence's last block), only the columns' causal
  //          limits apply;
  //  kAny    also keys past the context: their V values are zeroed.
  // Only kAny changes P, so the branch between kFull and kCausal in the loop
  // joins with the same operand registers.
  // pvf (16-bit pools read from the LDS ring only): the V operands hold f16
  // values, and each probability is one f16 operand (PV error within 2^-12 of
  // the output's scale), so one MFMA per tile instead of the high/low pair.
  auto softmax_pv = [&](Pair& P, f32x4 (&sacc)[NB][CS], const f32x4 (&kscale)[NB], int i, bool has_b, auto mode,
                        auto pvf) {
    constexpr int MODE = decltype(mode)::value;
    constexpr bool PVF = decltype(pvf)::value;
    constexpr bool RL = PVF && !F16;   // V rows regrouped in the ring: tile t's operand is row t
    constexpr bool FULL = MODE == 0;
    constexpr bool TAIL = MODE == 2;
    constexpr bool RAWMAX = FULL && !is_quantised(KVT);
    bool full[NB] = {true, true};
    bool in_ctx[NB][4];
    int blk0[NB];
    float ksc[NB][4], vsc[NB][4];
    blk0[0] = (c0 + i) * kBlockSize;
    blk0[1] = blk0[0] + kBlockSize;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ksc[0][e] = is_quantised(KVT) ? kscale[0][e] * sl2 : sl2;
      ksc[1][e] = is_quantised(KVT) ? kscale[1][e] * sl2 : sl2;
      vsc[0][e] = is_quantised(KVT) ? P.vsa[e] : 1.f;
      vsc[1][e] = is_quantised(KVT) ? P.vsb[e] : 1.f;
      in_ctx[0][e] = in_ctx[1][e] = true;
    }
    if constexpr (!FULL) {
      full[0] = blk0[0] + kBlockSize <= all_visible;
      full[1] = blk0[1] + kBlockSize <= all_visible && has_b;
    }
    if constexpr (TAIL && RL) {   // the operands are masked where they are built, below
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (!full[0]) in_ctx[0][e] = blk0[0] + 4 * j + e < L;
        if (!full[1]) in_ctx[1][e] = has_b && blk0[1] + 4 * j + e < L;
      }
    } else if constexpr (TAIL) {
      if (!full[0]) mask_tail(P, kA, blk0[0], in_ctx[0]);
      if (!full[1]) mask_tail(P, kB, has_b ? blk0[1] : L, in_ctx[1]);   // an absent block lies wholly past L
    }
    // ---- per column set: causal mask, online softmax, probabilities as PV operands
    uint32_t ph[CS][2 * NB], pl[CS][2 * NB];
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) {
      float x[NB][4];
      float mx = -INFINITY;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v;
          if constexpr (RAWMAX) {
            v = sacc[b][cs][e];
          } else {
            v = (BIAS ? sacc[b][cs][e] - qbias[cs] : sacc[b][cs][e]) * ksc[b][e];
            if (!full[b]) v = in_ctx[b][e] && blk0[b] + 4 * j + e <= pos[cs] ? v : -INFINITY;
          }
          x[b][e] = v;
        }
        mx = vmax(mx, vmax(vmax(x[b][0], x[b][1]), vmax(x[b][2], x[b][3])));
      }
      // the step's largest (scaled) logit of this column
      const float mb = RAWMAX ? (row_vmax4(mx) - qbias[cs]) * sl2 : row_vmax4(mx);
      const bool need = mb > m_run[cs] + kPfRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(need) != 0ull) {
        const float m_new = need ? mb : m_run[cs];
        const float alpha = m_new == m_run[cs] ? 1.f : fast_exp2(m_run[cs] - m_new);
        l_run[cs] *= alpha;
        lacc[cs] *= alpha;
        if constexpr (BIAS) p_run[cs] *= alpha;
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[cs][t] *= alpha;
        m_run[cs] = m_new;
      }
      const float mref = m_run[cs] == -INFINITY ? 0.f : m_run[cs];
      const float off = -(qbias[cs] * sl2) - mref;   // RAWMAX: exponent = raw * |f| + off
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float pr[4], pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pr[e] = fast_exp2(RAWMAX ? __builtin_fmaf(x[b][e], sl2, off) : x[b][e] - mref);
        l_run[cs] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (is_quantised(KVT)) pv[e] = in_ctx[b][e] ? pr[e] * vsc[b][e] : 0.f;
          else pv[e] = pr[e];
        }
        if constexpr (!OP32) {
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            const float f0 = pv[2 * w], f1 = pv[2 * w + 1];
            uint32_t hw, lw = 0;
            if constexpr (PVF) hw = pack_f16x2(f0, f1);
            else pack_p(f0, f1, hw, lw);
            if constexpr (!F16 && !PVF) {
              if constexpr (BIAS)
                p_run[cs] += (bf16_to_f32(hw & 0xffffu) + bf16_to_f32(lw & 0xffffu)) +
                             (bf16_to_f32(hw >> 16) + bf16_to_f32(lw >> 16));
            }
            ph[cs][2 * b + w] = hw;
            pl[cs][2 * b + w] = lw;
          }
        } else {
          // f32 pools: PV with the 16x16x4 f32 MFMA, one key per step
#pragma unroll
          for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t vw = b ? vword(P, kB, t, e) : vword(P, kA, t, e);
              acc[cs][t] = mfma_f32_k4(__uint_as_float(vw), pv[e], acc[cs][t]);
            }
          }
        }
      }
    }
    // ---- O^T += V^T P^T per set, sharing the converted V operand
    if constexpr (!OP32) {
      mfma_phase(true);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        u32x4 av;
        if constexpr (RL) {
          av = (t & 1) ? P.vb[t / 2] : P.va[t / 2];
          if constexpr (TAIL) {   // keys past the context: V zeroed (words 0-1 first block, 2-3 second)
#pragma unroll
            for (int w = 0; w < 4; ++w)
              av[w] &= (in_ctx[w / 2][2 * (w % 2)] ? 0xffffu : 0u) | (in_ctx[w / 2][2 * (w % 2) + 1] ? 0xffff0000u : 0u);
          }
        } else if constexpr (EB == 2) {
          av = u32x4{vword(P, kA, t, 0), vword(P, kA, t, 1), vword(P, kB, t, 0), vword(P, kB, t, 1)};
        } else {
          uint32_t v0, v1, v2, v3;
          code8x4_to_bf16x4<KVT>(vword(P, kA, t, 0), v0, v1);
          code8x4_to_bf16x4<KVT>(vword(P, kB, t, 0), v2, v3);
          av = u32x4{v0, v1, v2, v3};
        }
#pragma unroll
        for (int cs = 0; cs < CS; ++cs) {
          if constexpr (PVF) {
            acc[cs][t] = mfma_k32v<true>(av, u32x4{ph[cs][0], ph[cs][1], ph[cs][2], ph[cs][3]}, acc[cs][t]);
          } else {
            acc[cs][t] = mfma_k32v<F16>(av, u32x4{ph[cs][0], ph[cs][1], ph[cs][2], ph[cs][3]}, acc[cs][t]);
            acc[cs][t] = mfma_k32v<F16>(av, u32x4{pl[cs][0], pl[cs][1], pl[cs][2], pl[cs][3]}, acc[cs][t]);
          }
        }
      }
      mfma_phase(false);
    }
  };
  // An absent second block: defined (zero) operands; its keys are masked.
  auto clear_b = [&](Pair& P) {
#pragma unroll
    for (int w = 0; w < KW / 4; ++w) P.kb[w] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int g = 0; g < VQ; ++g) P.vb[g] = u32x4{0u, 0u, 0u, 0u};
    P.ksb = P.vsb = f32x4{0.f, 0.f, 0.f, 0.f};
    P.okb = true;
  };
  constexpr std::integral_constant<int, 0> kFull{};
  constexpr std::integral_constant<int, 1> kCausal{};
  constexpr std::integral_constant<int, 2> kAny{};

  // 16-bit pools: PV in f16 first (bf16 V rewritten to f16 in the ring); a V
  // value beyond f16's range turns into inf there and leaves an accumulator
  // non-finite, and then the workgroup computes again with the high/low
  // probability split, which is also what a non-finite q, K or V gives.
  constexpr bool PV16 = STAGE && PKV_PREFILL_PV16;
  if constexpr (PV16) {
    if (threadIdx.x == 0) s_redo = 0;   // ordered before its stores by the first barrier of the pass
  }
  if constexpr (STAGE) {
  auto stage_pass = [&](auto pvf) {
    constexpr bool PVF = decltype(pvf)::value;
    constexpr bool CONV = PVF && !F16;   // the V copies are bf16: rewritten to f16 in the ring
    // Pair q (blocks 2q, 2q + 1 of the chunk) has slot q % NS: K of its first
    // block, K of its second, then both V tiles by interleaved 1 KiB rows.  K
    // runs one pair ahead of V: iteration p reads V(p) and K(p + 1), so that
    // the QK MFMAs of pair p + 1 run beside the softmax VALU of pair p.  Wave 0
    // copies the first block's K tile, wave 1 the second's, waves 2 and 3 the
    // V tiles, each 1 KiB per instruction, byte for byte; in iteration p a wave
    // sends the copy of pair p + lead (K: NS ahead, V: NS - 1 ahead), before
    // the loop those of pairs 0 .. lead - 1.  Then the pair an iteration needs
    // was sent NS - 1 iterations earlier and its slot's previous pair was last
    // read an iteration earlier (every read of an iteration is consumed by its
    // MFMAs before the next barrier).  Pairs past the chunk reload its last
    // pair (their slots are never read), so every wave issues the same count
    // and the waits below are exact.
    const int lead = wave < 2 ? NS : NS - 1;
    const uint8_t* kvb = wave < 2 ? kbase : vbase;
    // Lane l copies the 16 bytes the operand reads of lane l need: a K row
    // holds them in lane order already; in a V row lane (c, j)'s chunk sits
    // at (4 c + j) * 16 (read there in lane order, a 16-byte read at a 64-byte
    // stride would hit each LDS bank four times).
    const int src_off = (wave < 2 ? lane : 4 * c + j) * 16;
    const int row0 = wave < 2 ? 0 : (wave & 1);   // K tiles: rows 0, 1, ..; V tiles interleaved
    const int row_step = wave < 2 ? 1 : 2;
    for (c0 = 0; c0 < n_blocks; c0 += kPfTab) {
      const int n = min(kPfTab, n_blocks - c0);
      for (int k = threadIdx.x; k < n; k += 256) s_tab[k] = trow[c0 + k];
      __syncthreads();                 // the ring is drained here: no copy in flight
      const int npairs = (n + 1) / 2;
      {
        // Every wave computes over every block of the chunk: an entry outside
        // the pool (its copies read block 0 instead) makes the result NaN.
        bool ok = true;
        for (int k = lane; k < n; k += kWave) {
          const int e = s_tab[k];
          ok = ok && e >= 0 && e < a.num_blocks;
        }
        bad = bad || __builtin_amdgcn_ballot_w64(!ok) != 0ull;
      }
      auto tile_blk = [&](int q) { return min(2 * min(q, npairs - 1) + (wave & 1), n - 1); };
      auto tile_src = [&](int phys) {
        return kvb + ((size_t)(phys >= 0 && phys < a.num_blocks ? phys : 0) * hkv + kvh) * TB;
      };
      auto tile_dst = [&](int q) { return s_ring + (q % NS) * SB + (wave < 2 ? wave * TB : 2 * TB); };
      for (int q = 0; q < lead; ++q) {
        copy_tile<TB, LPS>(tile_src(__builtin_amdgcn_readfirstlane(s_tab[tile_blk(q)])), src_off, tile_dst(q), row0,
                           row_step);
      }
      // The table entry of the tile this wave copies in the next iteration.
      int ent = s_tab[tile_blk(lead)];

      u32x4 kn_a[KW / 4], kn_b[KW / 4];   // K operands of the next pair
      f32x4 sacc[NB][CS];                 // S = K q^T of the current pair
      float lmx[CS];                      // this lane's largest raw product of the current pair, per set
      auto lane_max = [&](const f32x4 (&sx)[NB][CS], float (&m)[CS]) {
#pragma unroll
        for (int cs = 0; cs < CS; ++cs) {
          float mx = -INFINITY;
#pragma unroll
          for (int b = 0; b < NB; ++b)
            mx = vmax(mx, vmax(vmax(sx[b][cs][0], sx[b][cs][1]), vmax(sx[b][cs][2], sx[b][cs][3])));
          m[cs] = mx;
        }
      };

      // Iteration head: wait for this wave's copies of the pair needed now,
      // barrier (everyone's have landed, everyone is done with the previous
      // iteration), then the LDS reads and the next copy.
      auto ring_head = [&](int p, u32x4* va, u32x4* vb, auto read_v, auto&& body) {
        constexpr bool RV = decltype(read_v)::value;
        // With CONV, iteration p also rewrites V(p + 1), so the copies of
        // V(p + 1) must have landed here: one iteration's copies in flight
        // instead of two, and this wave's rewrite of the previous iteration
        // is finished before the barrier (lgkmcnt(0)).
        constexpr int kVm = LPS * (NS - (CONV ? 3 : 2));
        static_assert(kVm < 16 && NS >= 3, "vmcnt field");
        __builtin_amdgcn_s_waitcnt((CONV ? 0x0070 : 0x0F70) | kVm);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const uint8_t* src = tile_src(__builtin_amdgcn_readfirstlane(ent));
        const int e = ring_io<TB, LPS, KW / 4, VQ, RV, CONV>(
            s_ring + ((p + 1) % NS) * SB, s_ring + (p % NS) * SB + 2 * TB, tile_dst(p + lead), s_tab,
            tile_blk(p + 1 + lead), src, src_off, row0, row_step, c, j, lane, kn_a, kn_b, va, vb,
            s_ring + ((p + 1) % NS) * SB + 2 * TB, wave, body);
        if constexpr (RV) ent = e;
      };
      // QK of pair 0, its K operands loaded from the pool here (an LDS read
      // of the ring outside the loops makes the compiler wait for every copy
      // in flight before each read of the ring inside them).
      {
        const int e0 = __builtin_amdgcn_readfirstlane(s_tab[0]);
        const int e1 = __builtin_amdgcn_readfirstlane(s_tab[min(1, n - 1)]);
        const uint8_t* k0 = kbase + ((size_t)(e0 >= 0 && e0 < a.num_blocks ? e0 : 0) * hkv + kvh) * TB;
        const uint8_t* k1 = kbase + ((size_t)(e1 >= 0 && e1 < a.num_blocks ? e1 : 0) * hkv + kvh) * TB;
#pragma unroll
        for (int w = 0; w < KW / 4; ++w) {
          kn_a[w] = *reinterpret_cast<const u32x4*>(k0 + ((4 * w + j) * kBlockSize + c) * 16);
          kn_b[w] = *reinterpret_cast<const u32x4*>(k1 + ((4 * w + j) * kBlockSize + c) * 16);
        }
        qk(kn_a, sacc[0]);
        qk(kn_b, sacc[1]);
        lane_max(sacc, lmx);
      }
      // The first copies are waited for here, in the compiler's view too:
      // left in flight into the loop, they would make it wait for all copies
      // at every step.  So are all LDS and scalar loads: a scalar load still
      // pending at the loop's entry (a kernel argument used after it) makes
      // every first LDS wait of a step a wait for all of them (scalar loads
      // return out of order, so no partial count is safe).
      __builtin_amdgcn_s_waitcnt(0x0070);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if constexpr (CONV) convert_v_rows<VQ>(s_ring + 2 * TB, wave, lane);   // V(0); published by the first iteration's barrier
      // Pairs every column sees whole, software-pipelined: the running max of
      // pair p is checked first (this lane's largest product against the
      // rescale threshold; a rescale, rare, takes the column's max), then one
      // basic block interleaves the probabilities of each column set with the
      // QK MFMAs of pair p + 1 and the PV MFMAs of the previous set.
      // The exponent's offset per set, -m_run (0 while m_run is -inf), changed
      // only by a rescale.
      float offp[CS];
      auto set_off = [&]() {
#pragma unroll
        for (int cs = 0; cs < CS; ++cs) offp[cs] = -(qbias[cs] * sl2) - (m_run[cs] == -INFINITY ? 0.f : m_run[cs]);
      };
      set_off();
      auto pipe_step = [&](int p) {
        // f16 PV steps (with PKV_PREFILL_F16_ONE_MAX) take the running max
        // from a chunk's first pair only: a later logit up to 16 (base 2)
        // above it gives a probability up to 2^16, still an f16 value; past
        // that the probability is inf, the accumulators turn non-finite and
        // the workgroup computes again with the split path, which checks
        // every pair.  This saves the max over every later pair's products.
        constexpr bool kOneMax = PVF && PKV_PREFILL_F16_ONE_MAX;
        bool any = false;
        if (!kOneMax || p == 0) {
#pragma unroll
          for (int cs = 0; cs < CS; ++cs) any = any || lmx[cs] * sl2 > m_run[cs] + kPfRescaleSlack;
        }
        if (__builtin_amdgcn_ballot_w64(any) != 0ull) {
#pragma unroll
          for (int cs = 0; cs < CS; ++cs) {
            const float mb = (row_vmax4(lmx[cs]) - qbias[cs]) * sl2;
            const bool need = mb > m_run[cs] + kPfRescaleSlack;
            const float m_new = need ? mb : m_run[cs];
            const float alpha = m_new == m_run[cs] ? 1.f : fast_exp2(m_run[cs] - m_new);
            l_run[cs] *= alpha;
            lacc[cs] *= alpha;
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[cs][t] *= alpha;
            m_run[cs] = m_new;
          }
          set_off();
        }
        // From here on one basic block: the LDS reads, the copy, then the
        // MFMAs interleaved with the VALU work (the body below).
        u32x4 va[VQ], vb[VQ];
        uint32_t ph[CS][2 * NB], pl[CS][2 * NB];
        auto probs = [&](int cs) {
          const float off = offp[cs];   // exponent = raw * |f| + off
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            float pr[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) pr[e] = fast_exp2(__builtin_fmaf(sacc[b][cs][e], sl2, off));
            if constexpr (!PVF) l_run[cs] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
#pragma unroll
            for (int w = 0; w < 2; ++w) {
              if constexpr (PVF) ph[cs][2 * b + w] = pack_f16x2(pr[2 * w], pr[2 * w + 1]);
              else pack_p(pr[2 * w], pr[2 * w + 1], ph[cs][2 * b + w], pl[cs][2 * b + w]);
            }
          }
        };
        // PV of one column set, two tiles at a time (high parts, then low
        // parts): an MFMA never waits on the one just before it.
        auto pv = [&](int cs) {
#pragma unroll
          for (int t = 0; t < NT; t += 2) {
            u32x4 av[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              if constexpr (CONV)   // regrouped rows: tile t's operand is row t
                av[u] = ((t + u) & 1) ? vb[(t + u) / 2] : va[(t + u) / 2];
              else
                av[u] = u32x4{va[(2 * (t + u)) / 4][(2 * (t + u)) % 4], va[(2 * (t + u) + 1) / 4][(2 * (t + u) + 1) % 4],
                              vb[(2 * (t + u)) / 4][(2 * (t + u)) % 4], vb[(2 * (t + u) + 1) / 4][(2 * (t + u) + 1) % 4]};
            }
#pragma unroll
            for (int u = 0; u < 2; ++u)
              acc[cs][t + u] = mfma_k32v<F16 || PVF>(av[u], u32x4{ph[cs][0], ph[cs][1], ph[cs][2], ph[cs][3]},
                                                    acc[cs][t + u]);
            if constexpr (!PVF) {
#pragma unroll
              for (int u = 0; u < 2; ++u)
                acc[cs][t + u] = mfma_k32v<F16>(av[u], u32x4{pl[cs][0], pl[cs][1], pl[cs][2], pl[cs][3]}, acc[cs][t + u]);
            }
          }
          if constexpr (PVF) {   // the normaliser: all-ones rows times the probabilities
            constexpr uint32_t kOnes = 0x3C003C00u;   // f16 1.0, twice
            lacc[cs] = mfma_k32v<true>(u32x4{kOnes, kOnes, kOnes, kOnes},
                                       u32x4{ph[cs][0], ph[cs][1], ph[cs][2], ph[cs][3]}, lacc[cs]);
          }
        };
        // QK of the next pair, both blocks' chains interleaved.
        f32x4 snew[NB][CS];
        auto qk_next = [&]() {
#pragma unroll
          for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int cs = 0; cs < CS; ++cs) snew[b][cs] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int st = 0; st < DPL / 8; ++st) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
              const u32x4 kq = b ? kn_b[st] : kn_a[st];
              const uint32_t av[4] = {kq[0], kq[1], kq[2], kq[3]};
#pragma unroll
              for (int cs = 0; cs < CS; ++cs) {
                snew[b][cs] = mfma_k32<F16>(av, &qhi[cs][4 * st], snew[b][cs]);
                if constexpr (QSPLIT) snew[b][cs] = mfma_k32<F16>(av, &qlo[cs][4 * st], snew[b][cs]);
              }
            }
          }
        };
        ring_head(p, va, vb, std::true_type{}, [&]() {
          probs(0);
          qk_next();
#pragma unroll
          for (int cs = 1; cs < CS; ++cs) {
            probs(cs);
            mfma_phase(true);   // (the previous set's PV MFMAs, interleaved with this set's softmax)
            pv(cs - 1);
            mfma_phase(false);
          }
          if constexpr (!kOneMax) lane_max(snew, lmx);
          mfma_phase(true);   // the last set's PV MFMAs run back to back: ahead of the other wave's VALU
          pv(CS - 1);
          mfma_phase(false);
          constexpr int kQkMfma = NB * (DPL / 8) * CS * (QSPLIT ? 2 : 1);
          constexpr int kPvMfma = PVF ? NT + 1 : 2 * NT;
          __builtin_amdgcn_sched_group_barrier(0x002, PKV_PREFILL_ILV_LEAD, 0);
          if constexpr (CONV) {   // the late LDS reads (second V half, table entry, rewrite) before the last 4 QK MFMAs
            interleave_mfma<kQkMfma - PKV_PREFILL_LATE_QK, PKV_PREFILL_ILV_QK>();
            __builtin_amdgcn_sched_group_barrier(0x100, VQ + 3, 0);
            interleave_mfma<PKV_PREFILL_LATE_QK, PKV_PREFILL_ILV_QK>();
          } else {
            interleave_mfma<kQkMfma, PKV_PREFILL_ILV_QK>();
          }
          if constexpr (CS > 1) interleave_mfma<kPvMfma * (CS - 1), PKV_PREFILL_ILV_PV>();
          interleave_mfma<kPvMfma, PKV_PREFILL_ILV_PVL>();
        });
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int cs = 0; cs < CS; ++cs) sacc[b][cs] = snew[b][cs];
      };
      // The rest (pairs across some column's causal limit, and the chunk's
      // last pair): masked softmax and PV of pair p, then QK of pair p + 1
      // (after the last pair, of the reloaded last pair: discarded).
      auto any_step = [&](int p) {
        Pair P;
        f32x4 kscale[NB] = {};
        ring_head(p, P.va, P.vb, std::true_type{}, [&]() {
          softmax_pv(P, sacc, kscale, 2 * p, 2 * p + 1 < n, kAny, pvf);
          mfma_phase(true);
          qk(kn_a, sacc[0]);
          qk(kn_b, sacc[1]);
          mfma_phase(false);
        });
      };
      // pairs p with both blocks below the wave's causal limits: (c0 + 2p + 2) * 16 <= all_visible
      const int p_full = min(npairs, max(0, (all_visible / kBlockSize - c0) / 2));
      const int p_pipe = min(p_full, npairs - 1);   // the pipelined step needs a next pair
      int p = 0;
#pragma unroll 1
      for (; p < p_pipe; ++p) pipe_step(p);
#pragma unroll 1
      for (; p < npairs; ++p) any_step(p);
      __builtin_amdgcn_s_waitcnt(0x0F70);   // the padding copies too
      __syncthreads();                 // s_tab and the ring are rewritten by the next chunk
    }
  };
  if constexpr (PV16) {
    stage_pass(std::true_type{});
    bool fin = true;
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) {
      fin &= __builtin_isfinite(l_run[cs]) & __builtin_isfinite(lacc[cs][0]);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) fin &= __builtin_isfinite(acc[cs][t][e]);
    }
    if (__builtin_amdgcn_ballot_w64(!fin) != 0ull) s_redo = 1;
    __syncthreads();
    if (s_redo) {
#pragma unroll
      for (int cs = 0; cs < CS; ++cs) {
        m_run[cs] = -INFINITY;
        l_run[cs] = 0.f;
        lacc[cs] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[cs][t] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      bad = !seq_ok;
      stage_pass(std::false_type{});
    }
  } else {
    stage_pass(std::false_type{});
  }
  } else {
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
    // One pair of blocks in flight: the next pair's K loads are issued as soon
    // as the QK MFMAs have consumed K, its V loads once PV has consumed V.
    Pair P;
    f32x4 sacc[NB][CS];
    f32x4 kscale[NB] = {};
    int i = 0;
    if (n > 0) {
      load_k(P, kA, 0);
      load_v(P, kA, 0);
    }
    if (n > 1) {
      load_k(P, kB, 1);
      load_v(P, kB, 1);
    }
    // Steady state: the next pair exists, so loads are unconditional, and the
    // step's blocks end at least 32 keys before the wave's last block: inside
    // the context.  First the pairs below every column's causal limit, then
    // (at most a few) pairs that cross some column's limit.
    // The pairs every column sees whole are software-pipelined: the next
    // pair's QK MFMAs are issued before this pair's softmax, so the matrix
    // pipe has independent work while the VALU computes the exponentials.
    if (i + 3 < n && (c0 + i + 2) * kBlockSize <= all_visible) {
      qk_step(P, sacc, kscale, i, true, true);            // QK of pair i; K of pair i + 2 requested
#pragma unroll 1
      for (; i + 5 < n && (c0 + i + 4) * kBlockSize <= all_visible; i += 2) {
        f32x4 s_next[NB][CS];
        f32x4 k_next[NB] = {};
        qk_step(P, s_next, k_next, i + 2, true, true);    // QK of pair i + 2; K of pair i + 4 requested
        softmax_pv(P, sacc, kscale, i, true, kFull, std::false_type{});      // pair i with its V
        load_v(P, kA, i + 2);
        load_v(P, kB, i + 3);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          kscale[b] = k_next[b];
#pragma unroll
          for (int cs = 0; cs < CS; ++cs) sacc[b][cs] = s_next[b][cs];
        }
      }
      softmax_pv(P, sacc, kscale, i, true, kFull, std::false_type{});
      load_v(P, kA, i + 2);
      load_v(P, kB, i + 3);
      i += 2;
    }
#pragma unroll 1
    for (; i + 3 < n; i += 2) {
      qk_step(P, sacc, kscale, i, true, true);
      softmax_pv(P, sacc, kscale, i, true, kCausal, std::false_type{});
      load_v(P, kA, i + 2);
      load_v(P, kB, i + 3);
    }
    const int rem = n - i;        // 0..3 blocks left; P holds blocks i, i + 1 where they exist
    if (rem >= 2) {
      qk_step(P, sacc, kscale, i, true, false);
      softmax_pv(P, sacc, kscale, i, true, kAny, std::false_type{});
    }
    if (rem % 2) {                // one block left over: paired with an absent one
      if (rem == 3) {
        load_k(P, kA, i + 2);
        load_v(P, kA, i + 2);
      }
      clear_b(P);
      const int il = rem == 3 ? i + 2 : i;
      qk_step(P, sacc, kscale, il, false, false);
      softmax_pv(P, sacc, kscale, il, false, kAny, std::false_type{});
    }
    __builtin_amdgcn_wave_barrier();   // the next chunk rewrites this wave's s_tab
  }
  }

  const bool out_vec = (reinterpret_cast<uintptr_t>(a.out) & (a.out_dtype == DT_F32 ? 15 : 7)) == 0;
#pragma unroll
  for (int cs = 0; cs < CS; ++cs) {
    float l = row_sum4(l_run[cs]) + lacc[cs][0];
    if (bad) l = __builtin_nanf("");
    const float vbias = BIAS ? kInt8Bias * row_sum4(p_run[cs]) : 0.f;   // biased V operands
    if (!wave_live || !col_ok[cs]) continue;
    const size_t orow = ((size_t)(q0 + tok[cs]) * hq + head) * D;
    const float inv = 1.f / l;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f32x4 o = acc[cs][t];
      if constexpr (BIAS) o -= vbias;
      if constexpr (CH) o *= *reinterpret_cast<const f32x4*>(a.v_scale + (size_t)kvh * D + 16 * t + 4 * j);
      o *= inv;
      const size_t oi = orow + 16 * t + 4 * j;   // 4 consecutive dims: one 8- or 16-byte store when aligned
      if (out_vec) {
        if (a.out_dtype == DT_F32) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + oi) = o;
        } else {
          const bool bf = a.out_dtype == DT_BF16;
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = bf ? f32_to_bf16_rne(o[e]) : f32_to_f16_bits(o[e]);
          *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + oi) = u32x2{w[0] | (w[1] << 16), w[2] | (w[3] << 16)};
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) store_out(a.out, oi + e, a.out_dtype, o[e]);
      }
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
