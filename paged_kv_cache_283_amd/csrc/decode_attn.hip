// Paged single-token decode attention for gfx950 (CDNA4).
//
// What is computed (page "长上下文优化：注意力稀疏化与 KV Cache 管理",
// plumephp.com/llm-long-context-optimization: the MHA/GQA/MQA table and the
// Flash sketch; page "KV Cache 与 PagedAttention：显存复用与长上下文推理",
// plumephp.com/ai-kv-cache-paged-attention, "三大运行时组件": decode reads the
// KV cache block by block through the block table):
//   out[s][h] = sum_p softmax_p(scale * q[s][h] . K[p][h/G]) * V[p][h/G]
// over the kept positions p of sequence s (geometry.hpp), plus, on request,
// the H2O per-position mass (H2OEviction.update_scores in the first page):
// the probabilities averaged over all query heads, added into a score row.
//
// How, on gfx950:
//  * One persistent launch of single-wave workgroups, as many as the GPU holds.
//    The attended blocks of the whole batch are cut into equal ranges; a wave
//    streams its range for one KV head through a software pipeline and writes
//    the output of every sequence it covers whole, or a partial softmax state
//    for a sequence cut at a range boundary.  A second kernel merges those
//    partials by log-sum-exp.  Equal ranges keep every wave busy for the same
//    time whatever the mix of context lengths.
//  * Per 16-token block and wave, QK^T is one 16x16 MFMA tile: A = the block's
//    K tile (row = token; the pool stores K in 16-byte chunks of 16 token rows,
//    so every load instruction reads 1 KiB of contiguous memory straight into
//    operand registers), B = the GQA group's query rows (column = query head; the G <= 16
//    rows of a group live in registers for the whole segment).  The
//    accumulator gives lane (c, j) the logits of head c for tokens 4j..4j+3.
//  * PV is a second MFMA per 16 head-dims: A = the dim-major V tile (lane
//    (d, j) holds tokens 4j..4j+3 of dim d; V is stored in 16-byte chunks that
//    give each lane this for 16 / (4 bytes per element) tiles at once), B =
//    the probabilities exactly as the QK accumulator left them in registers,
//    so no LDS round trip or transpose sits between the two products.  The
//    output accumulator again puts head c in lane column c, next to its
//    running max and sum, so the online-softmax rescale is lane-local.
//  * Probabilities are split into a high and a low 16-bit part and fed as two
//    MFMAs, keeping ~16 mantissa bits.  8-bit codes convert to bf16 operands
//    exactly: E4M3 with the hardware converter, INT8 as code + 128 (the bias
//    is taken out of the sums).  Per-token scales multiply the logit (K) and
//    the probability (V); static per-channel scales multiply q once per
//    segment (K) and the output once at the end (V).
//  * Logits are kept in base 2 (scale * log2 e folded in) and exponentiated
//    with v_exp_f32.
#include <hip/hip_ext.h>

#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "device_common.hpp"
#include "geometry.hpp"
#include "kv_codec.hpp"
#include "launch.hpp"
#include "mfma_ops.hpp"

namespace pkv {

// Slack (base-2 units) the running max may lag behind before accumulators are rescaled.
constexpr float kRescaleSlack = 8.f;

// Build-time tuning knobs (defaults are the measured choice).
#ifndef PKV_ATTN_PIPE
#define PKV_ATTN_PIPE 3              // K/V register buffers per wave (2 or 3): blocks in flight = PIPE - 1
#endif
#ifndef PKV_ATTN_NT_LOADS
#define PKV_ATTN_NT_LOADS 1          // 1: K/V tiles loaded with the non-temporal hint (read once)
#endif
#ifndef PKV_ATTN_WAVES_PER_CU
#define PKV_ATTN_WAVES_PER_CU 4      // waves launched per CU, one per SIMD (0: as many as fit)
#endif
#ifndef PKV_ATTN_WAVES_PER_CU_FP8
#define PKV_ATTN_WAVES_PER_CU_FP8 8  // the same for 8-bit (FP8, INT8) pools (two per SIMD)
#endif
#ifndef PKV_ATTN_HEAD_FAST
#define PKV_ATTN_HEAD_FAST 0         // 16-bit and f32 pools -- 1: workgroup id = range * KV heads + head; 0: head-major
#endif
#ifndef PKV_ATTN_HEAD_FAST_8BIT
#define PKV_ATTN_HEAD_FAST_8BIT 1    // the same for 8-bit pools
#endif
#ifndef PKV_ATTN_PAIR_8BIT
#define PKV_ATTN_PAIR_8BIT 1         // per-token 8-bit pools: KV head pairs of a range on one XCD
#endif
#ifndef PKV_ATTN_ODD_SHARE
#define PKV_ATTN_ODD_SHARE 880       // per mille: odd-numbered range length relative to even (head-major only)
#endif

template <typename T>
__device__ __forceinline__ T load_stream(const T* p) {
#if PKV_ATTN_NT_LOADS
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

// The workgroup is one wave: LDS written by some lanes is read by others after
// this (LDS-only fences, so outstanding global stores are not waited for).
__device__ __forceinline__ void lds_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Floats of the per-wave LDS window for H2O logits: 32 KiB with one wave per
// SIMD (16-bit and f32 pools; a typical range fits, so chunks rarely drain),
// 8 KiB with two (8-bit pools).  Compacting instances keep 32 KiB for every
// format (half of it holds the destination tile images), which leaves room
// for one workgroup per SIMD.
__host__ __device__ constexpr int stash_floats(int kvt, bool cmp = false) {
  return is_code8(kvt) && !cmp ? 2048 : 8192;
}

// Table entries staged in LDS per chunk of a segment.
constexpr int kTabBlocks = 1024;

// Partial-output slot of a segment starting at attended block vb of its
// sequence: 0 for the first segment, vb / kPartBlocks + 1 for one starting at a
// range cut.  Cuts are at least kPartBlocks apart, so slots are distinct; the
// largest is ceil(blocks / kPartBlocks).
__device__ __forceinline__ int partial_slot(int vb) { return vb == 0 ? 0 : vb / kPartBlocks + 1; }

// Attended blocks of a sequence of length L (0 for an unusable length).
__device__ __forceinline__ int attended_blocks(const AttnArgs& a, int L) {
  const int len_cap = min(a.max_context_len, a.table_stride * kBlockSize);
  return (L < 1 || L > len_cap) ? 0 : keep_geometry(L, a.num_sinks, a.window).n_virtual;
}

// One wave attends the GQA group of KV head kvh of sequence s over attended
// blocks [seg_vb0, seg_vb1) and writes the normalised output (the segment is the
// whole sequence) or a partial (running max, exp-sum, unnormalised output) in
// slot partial_slot(seg_vb0).  CMP (16-bit pools, no sinks or window): the
// keep map masks the evicted tokens out and the kept ones are stored, from the
// operand registers, into the destination blocks (the compaction the
// eviction policy asks for, without a second read of the cache).
template <int KVT, int QT, int D, bool CMP>
__device__ __forceinline__ void wave_segment(const AttnArgs& a, int* s_tab, uint32_t* s_new, float* s_stash, int s,
                                             int kvh, int L, int seg_vb0, int seg_vb1) {
  using KT = KvType<KVT>;
  constexpr int EB = KT::kBytes;
  constexpr bool OP32 = KT::kOp32;
  constexpr bool F16 = KT::kOpF16;
  constexpr int DPL = D / 4;              // QK contraction dims held per lane
  constexpr int KW = DPL * EB / 4;        // K words per lane per block
  constexpr int NT = D / 16;              // 16-dim output tiles
  constexpr int VW = EB;                  // V words per lane per tile (4 tokens)
  constexpr bool CH = is_channel_scaled(KVT);   // static per-channel scales, folded into q and the output
  constexpr bool BIAS = code_biased<KVT>();      // INT8 operands are biased codes
  // INT8 K enters QK as f16 code + 1152 (one v_perm_b32 per two codes), so the
  // QK operands are f16; q is prescaled by 2^e into f16's range.
  constexpr bool KF16 = code_set(KVT) == DT_INT8 && is_code8(KVT);
  constexpr bool QF16 = F16 || KF16;            // QK operand type
  constexpr bool QSAME = (!OP32) && (QT == (QF16 ? DT_F16 : DT_BF16)) && !CH;
  // bf16 queries against INT8's f16 K operands: after the power-of-two
  // prescale every bf16 value of magnitude >= 2^-17 (8 significant bits) is an
  // f16 value exactly, and smaller ones round at f16's subnormal spacing in the
  // low half too, so the low half adds nothing and one MFMA per step does.
  constexpr bool QEXACT = KF16 && QT == DT_BF16 && !CH;
  constexpr bool QSPLIT = (!OP32) && !QSAME && !QEXACT;
  constexpr int QW = OP32 ? 1 : DPL / 2;  // 16-bit operand words of q per lane

  const int hq = a.num_q_heads;
  const int group = hq / a.num_kv_heads;
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;                // MFMA row/column inside a 16x16 tile
  const int j = lane >> 4;                // which 4-token / 1/4-of-dims slice
  const KeepGeom geo = keep_geometry(L, a.num_sinks, a.window);
  const bool whole = seg_vb0 == 0 && seg_vb1 == geo.n_virtual;
  const int keep_lo = a.window > 0 ? L - a.window : 0;   // p >= keep_lo is kept
  const int sinks = a.window > 0 ? a.num_sinks : 0;      // p < sinks is kept

  // ---- the group's query rows as the QK B operand (column c = query head) ----
  const int head = kvh * group + c;
  const bool head_ok = c < group;
  uint32_t qhi[QW];
  uint32_t qlo[QSPLIT ? QW : 1];
  float qf[OP32 ? DPL : 1];
  int q_exp = 0;                          // q operands carry q * 2^q_exp (INT8 K only)
  {
    // Lane (c, j) holds, for QK step st, the same head-dims the K chunks of row
    // group j carry in that step (qk_dim), so A and B agree on the contraction.
    const size_t qrow = ((size_t)s * hq + (head_ok ? head : 0)) * D;
    if constexpr (OP32) {
#pragma unroll
      for (int st = 0; st < DPL; ++st)
        qf[st] = head_ok ? load_q_elem<QT>(a.q, qrow + qk_dim_f32(st, j)) : 0.f;
    } else if constexpr (QSAME) {
      const uint16_t* qh = reinterpret_cast<const uint16_t*>(a.q) + qrow;
#pragma unroll
      for (int st = 0; st < QW / 4; ++st) {
        const u32x4 v = head_ok ? *reinterpret_cast<const u32x4*>(qh + qk_dim16<KVT>(st, j)) : u32x4{0, 0, 0, 0};
        qhi[4 * st + 0] = v[0]; qhi[4 * st + 1] = v[1]; qhi[4 * st + 2] = v[2]; qhi[4 * st + 3] = v[3];
      }
    } else {
      float qv[2 * QW];
#pragma unroll
      for (int st = 0; st < QW / 4; ++st) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int d0 = qk_dim16<KVT>(st, j) + 2 * w;
          float f0 = head_ok ? load_q_elem<QT>(a.q, qrow + d0) : 0.f;
          float f1 = head_ok ? load_q_elem<QT>(a.q, qrow + d0 + 1) : 0.f;
          if constexpr (CH) {   // q . (code * s) = (q * s) . code, with q * s carried as hi + lo
            f0 *= a.k_scale[(size_t)kvh * D + d0];
            f1 *= a.k_scale[(size_t)kvh * D + d0 + 1];
          }
          qv[2 * (4 * st + w)] = f0;
          qv[2 * (4 * st + w) + 1] = f1;
        }
      }
      if constexpr (KF16) {
        // 2^e with the head's largest |q| in [2^14, 2^15): exact, inside f16's range
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < 2 * QW; ++i) m = fmaxf(m, fabsf(qv[i]));
        m = row_max4(m);
        if (m > 0.f && m < INFINITY) {
          const int ex = (int)((__float_as_uint(m) >> 23) & 0xffu) - 127;
          q_exp = min(max(14 - ex, -60), 60);
        }
#pragma unroll
        for (int i = 0; i < 2 * QW; ++i) qv[i] = ldexpf(qv[i], q_exp);
      }
#pragma unroll
      for (int w = 0; w < QW; ++w) {
        const float f0 = qv[2 * w], f1 = qv[2 * w + 1];
        const uint32_t h0 = to_op16<QF16>(f0), h1 = to_op16<QF16>(f1);
        const uint32_t l0 = to_op16<QF16>(f0 - from_op16<QF16>(h0));
        const uint32_t l1 = to_op16<QF16>(f1 - from_op16<QF16>(h1));
        qhi[w] = h0 | (h1 << 16);
        if constexpr (QSPLIT) qlo[w] = l0 | (l1 << 16);
      }
    }
  }
  // Logit factor: the softmax scale in base 2, times 2^-e for prescaled q.
  const float lscale = a.scale_log2 * ldexpf(1.f, -q_exp);
  // Biased K operands add bias * (sum of head c's q operand values) to every logit.
  float qbias = 0.f;
  if constexpr (BIAS) {
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < QW; ++w) {
      sum += from_op16<QF16>(qhi[w] & 0xffffu) + from_op16<QF16>(qhi[w] >> 16);
      if constexpr (QSPLIT) sum += from_op16<QF16>(qlo[w] & 0xffffu) + from_op16<QF16>(qlo[w] >> 16);
    }
    qbias = (KF16 ? kInt8BiasF16 : kInt8Bias) * row_sum4(sum);
  }

  float m_run = -INFINITY;   // reference max of this head's base-2 logits (same in all 4 rows)
  float l_run = 0.f;         // this lane's share of the exp-sum
  float p_run = 0.f;         // biased V operands: this lane's share of the sum of P operand values
  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  bool bad = false;

  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_pool);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v_pool);
  const int32_t* trow = a.block_tables + (size_t)s * a.table_stride;

  // ---- decode append fused in: the segment that ends the sequence loads the
  // new token's K and V source rows (position L - 1, offset o_new of the last
  // attended block) together with its first table chunk and puts the stored
  // form in LDS next to the staged entries -- the rows themselves for 16-bit
  // and f32 pools, the codes (and the per-token scales in registers) for FP8
  // pools, quantised exactly as the write kernels do; the last block's
  // operands get them patched in, so the products see exactly the bits the
  // pool will hold.  The rows are stored into their slot when the wave has
  // finished all its segments (append_stores): stores share the load counter,
  // so a store issued here would hold up the wave's next tile waits until it
  // completes.  8-bit pools take the source in q's dtype; INT8 instances with
  // f32 queries are built without this code (fused_append_built) and their
  // pools already hold the token.
  constexpr bool C8 = is_code8(KVT);
  constexpr bool kFuse = fused_append_built(KVT, QT);
  constexpr int SEB = C8 ? (QT == DT_F32 ? 4 : 2) : EB;   // source element bytes
  constexpr int NWS = D * SEB / 4;        // words of one source row
  constexpr int NWL = (NWS + kWave - 1) / kWave;
  constexpr int NW = D * EB / 4;          // words of one stored row in LDS
  const bool fuse = kFuse && a.k_new != nullptr && seg_vb1 == geo.n_virtual;
  const int o_new = (L - 1) & (kBlockSize - 1);
  const int vb_new = geo.n_virtual - 1;
  uint32_t rk[NWL], rv[NWL];
  float ks_new = 0.f, vs_new = 0.f;       // the new token's per-token scales (per-token 8-bit formats)
  auto fused_load = [&]() {
    if constexpr (!kFuse) return;
    const size_t row = ((size_t)s * a.num_kv_heads + kvh) * NWS;
    const uint32_t* kr = reinterpret_cast<const uint32_t*>(a.k_new) + row;
    const uint32_t* vr = reinterpret_cast<const uint32_t*>(a.v_new) + row;
#pragma unroll
    for (int u = 0; u < NWL; ++u) {
      const int k = min(lane + kWave * u, NWS - 1);
      rk[u] = kr[k];
      rv[u] = vr[k];
    }
  };
  // Once the first chunk's entries are staged (the same wait covers these loads).
  auto fused_stage = [&]() {
    if constexpr (!kFuse) {
    } else if constexpr (!C8) {
#pragma unroll
      for (int u = 0; u < NWL; ++u) {
        const int k = lane + kWave * u;
        if (k < NW) {
          s_new[k] = rk[u];
          s_new[NW + k] = rv[u];
        }
      }
    } else {
      constexpr int EPW = 4 / SEB;        // source elements per word
      auto elem = [](uint32_t w, int i) { return SEB == 4 ? w : (w >> (16 * i)) & 0xffffu; };
      if constexpr (is_quantised(KVT)) {
        float km = 0.f, vm = 0.f;
#pragma unroll
        for (int u = 0; u < NWL; ++u) {
          if (lane + kWave * u < NWS) {
#pragma unroll
            for (int i = 0; i < EPW; ++i) {
              km = fmaxf(km, fabsf(raw_to_f32<QT>(elem(rk[u], i))));
              vm = fmaxf(vm, fabsf(raw_to_f32<QT>(elem(rv[u], i))));
            }
          }
        }
        ks_new = __fdiv_rn(wave_max(km), max_code8<KVT>());
        vs_new = __fdiv_rn(wave_max(vm), max_code8<KVT>());
      }
      uint8_t* sb = reinterpret_cast<uint8_t*>(s_new);
#pragma unroll
      for (int u = 0; u < NWL; ++u) {
        const int k = lane + kWave * u;
        if (k < NWS) {
#pragma unroll
          for (int i = 0; i < EPW; ++i) {
            const int d = k * EPW + i;
            const float kc = CH ? a.k_scale[(size_t)kvh * D + d] : ks_new;
            const float vc = CH ? a.v_scale[(size_t)kvh * D + d] : vs_new;
            sb[d] = (uint8_t)stored_code<QT, KVT>(elem(rk[u], i), kc);
            sb[D + d] = (uint8_t)stored_code<QT, KVT>(elem(rv[u], i), vc);
          }
        }
      }
    }
  };
  static_assert(!CMP || EB <= 2, "compaction is built for 16-bit and 8-bit pools");
  struct Regs {
    uint32_t k[KW];
    uint32_t v[NT][VW];
    f32x4 ks, vs;
    bool ok;
    int km, kd0, kd1, krank;   // CMP: keep-map entry of the block
  };

  int c0 = seg_vb0;     // first block of the current table chunk (s_tab[i] = entry of block c0 + i)

  auto load = [&](Regs& r, int i) {
    const int phys = __builtin_amdgcn_readfirstlane(s_tab[i]);
    r.ok = phys >= 0 && phys < a.num_blocks;
    // An entry outside the pool reads block 0 instead (in bounds) and marks the
    // result bad; no branch around the loads keeps the wait counts exact.
    const size_t tile = (size_t)(r.ok ? phys : 0) * a.num_kv_heads + kvh;
    // K tile [D/X][16][X]: load u gives lane (c, j) chunk 4u + j of token row c,
    // and the 64 lanes of one load read 1 KiB of contiguous memory.
    const uint8_t* kt = kbase + tile * (size_t)(kBlockSize * D * EB);
#pragma unroll
    for (int w = 0; w < KW / 4; ++w) {
      const u32x4 v = load_stream(reinterpret_cast<const u32x4*>(kt + ((size_t)(4 * w + j) * kBlockSize + c) * 16));
      r.k[4 * w + 0] = v[0]; r.k[4 * w + 1] = v[1]; r.k[4 * w + 2] = v[2]; r.k[4 * w + 3] = v[3];
    }
    // V tile in 16-byte chunks: load g gives lane (c, j) tokens 4j..4j+3 of
    // dims 16 t + c for the Y = 4 / EB tiles t = g Y .. g Y + Y - 1, which is
    // words [4 g, 4 g + 4) of r.v in [tile][word] order; 1 KiB per load.
    const uint8_t* vt = vbase + tile * (size_t)(kBlockSize * D * EB);
    uint32_t* vw = &r.v[0][0];
#pragma unroll
    for (int g = 0; g < NT * VW / 4; ++g) {
      const u32x4 v = load_stream(reinterpret_cast<const u32x4*>(vt + ((size_t)(g * 16 + c) * 4 + j) * 16));
      vw[4 * g + 0] = v[0]; vw[4 * g + 1] = v[1]; vw[4 * g + 2] = v[2]; vw[4 * g + 3] = v[3];
    }
    if constexpr (is_quantised(KVT)) {
      r.ks = *reinterpret_cast<const f32x4*>(a.k_scale + tile * kBlockSize + 4 * j);
      r.vs = *reinterpret_cast<const f32x4*>(a.v_scale + tile * kBlockSize + 4 * j);
    }
    if constexpr (CMP) {   // attended block == logical block (no sinks or window)
      const KeepMapEntry m = a.keep_map[(size_t)s * a.map_stride + c0 + i];
      r.km = m.w0;
      r.kd0 = m.dst0;
      r.kd1 = m.dst1;
      r.krank = m.rank;
    }
  };

  // CMP: the kept tokens pass through LDS images of their destination tiles
  // (the end of the logit window's space), destination tile T of the
  // sequence in image T % 2, laid out as the pool's tile (K, V, then for
  // per-token 8-bit formats the tile's 16 K and 16 V scales), and a tile goes
  // out in whole 16-byte chunks once this wave has written its last slot.
  // The segment's first and last tiles may be shared with the waves of the
  // neighbouring segments: of those only this wave's slots are stored (K
  // pieces of 16 bytes, single V elements, single scales).
  constexpr int kTileB = kBlockSize * D * EB;
  constexpr bool kScl = is_quantised(KVT);
  constexpr int kImgB = 2 * kTileB + (kScl ? 2 * kBlockSize * 4 : 0);   // one image
  constexpr int kVY = 4 / EB;                  // tiles (16 dims apart) per V chunk
  constexpr int kVE = 16 / EB;                 // elements per V chunk
  // the two images take the window's last 2 kImgB bytes; the H2O logit
  // window keeps the rest
  constexpr int kImgFloats = CMP ? 2 * kImgB / 4 : 0;
  static_assert(2 * kImgFloats <= stash_floats(KVT, CMP), "the tile images leave half the logit window");
  uint8_t* cimg = reinterpret_cast<uint8_t*>(s_stash + (stash_floats(KVT, CMP) - kImgFloats));
  using VE = typename std::conditional<EB == 2, uint16_t, uint8_t>::type;
  int c_first = -1;            // rank (destination position) of the segment's first kept token
  int c_end = 0;               // one past the last rank written
  int c_blk[2] = {-1, -1};     // destination block of the tile in each image
  auto compact_flush = [&](int T, int lo, int hi) {
    if constexpr (CMP) {
      const int blk = c_blk[T & 1];
      if (blk < 0) return;
      lds_wave_sync();
      const uint8_t* img = cimg + (T & 1) * kImgB;
      const size_t tile = (size_t)blk * a.num_kv_heads + kvh;
      uint8_t* kt = reinterpret_cast<uint8_t*>(a.k_store) + tile * kTileB;
      uint8_t* vt = reinterpret_cast<uint8_t*>(a.v_store) + tile * kTileB;
      if (lo == 0 && hi == kBlockSize) {
#pragma unroll
        for (int k = 0; k < kTileB / (kWave * 16); ++k) {
          const int off = (k * kWave + lane) * 16;
          *reinterpret_cast<u32x4*>(kt + off) = *reinterpret_cast<const u32x4*>(img + off);
          *reinterpret_cast<u32x4*>(vt + off) = *reinterpret_cast<const u32x4*>(img + kTileB + off);
        }
      } else {
        // K piece p is slot p % 16 of chunk p / 16
#pragma unroll
        for (int k = 0; k < kTileB / (kWave * 16); ++k) {
          const int p = k * kWave + lane, sl = p & 15;
          if (sl >= lo && sl < hi)
            *reinterpret_cast<u32x4*>(kt + p * 16) = *reinterpret_cast<const u32x4*>(img + p * 16);
        }
        // V element x of chunk x / kVE belongs to slot 4 (chunk % 4) + x % 4
        const VE* iv = reinterpret_cast<const VE*>(img + kTileB);
        VE* dv = reinterpret_cast<VE*>(vt);
#pragma unroll 4
        for (int k = 0; k < kTileB / (kWave * EB); ++k) {
          const int x = k * kWave + lane, sl = (((x / kVE) & 3) << 2) | (x & 3);
          if (sl >= lo && sl < hi) dv[x] = iv[x];
        }
      }
      if constexpr (kScl) {   // lanes 0-15 the K scales, 16-31 the V scales of the tile's slots
        const float* is = reinterpret_cast<const float*>(img + 2 * kTileB);
        const int sl = lane & 15;
        if (lane < 2 * kBlockSize && sl >= lo && sl < hi) {
          float* ds = lane < kBlockSize ? a.k_scale_store : a.v_scale_store;
          ds[tile * kBlockSize + sl] = is[lane];
        }
      }
    }
  };
  // Lane (c, j) holds K chunks 4w + j of token row c and the V elements of
  // tokens 4j..4j+3 for dims 16t + c (and their scales); a kept token's rank
  // is the block's first rank plus the kept tokens before it in the block.
  auto compact_put = [&](const Regs& r) {
    if constexpr (CMP) {
      const uint32_t mask = (uint32_t)r.km & 0xffffu;
      if (mask == 0u) return;
      const int r0 = r.krank;
      const int t0 = r0 >> 4;
      const int cnt = __builtin_popcount(mask);
      if (c_first < 0) c_first = r0;
      c_blk[t0 & 1] = r.kd0;
      if ((r0 & 15) + cnt > kBlockSize) c_blk[(t0 + 1) & 1] = r.kd1;
      if ((mask >> c) & 1u) {
        const int q = r0 + __builtin_popcount(mask & ((1u << c) - 1u));
        uint8_t* img = cimg + ((q >> 4) & 1) * kImgB;
#pragma unroll
        for (int w = 0; w < KW / 4; ++w)
          *reinterpret_cast<u32x4*>(img + ((4 * w + j) * kBlockSize + (q & 15)) * 16) =
              u32x4{r.k[4 * w], r.k[4 * w + 1], r.k[4 * w + 2], r.k[4 * w + 3]};
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = 4 * j + e;
        if ((mask >> tok) & 1u) {
          const int q = r0 + __builtin_popcount(mask & ((1u << tok) - 1u));
          uint8_t* img = cimg + ((q >> 4) & 1) * kImgB;
          VE* iv = reinterpret_cast<VE*>(img + kTileB);
          const int s2 = q & 15;
#pragma unroll
          for (int t = 0; t < NT; ++t)   // chunk ((t / Y) 16 + c) 4 + s2 / 4, element (t % Y) 4 + s2 % 4
            iv[(((t / kVY) * kBlockSize + c) * 4 + (s2 >> 2)) * kVE + (t % kVY) * 4 + (s2 & 3)] =
                (VE)(r.v[t][(e * EB) / 4] >> (8 * ((e * EB) % 4)));
          if constexpr (kScl) {
            if (c == 0) {
              float* is = reinterpret_cast<float*>(img + 2 * kTileB);
              is[s2] = r.ks[e];
              is[kBlockSize + s2] = r.vs[e];
            }
          }
        }
      }
      c_end = r0 + cnt;
      if (c_end >= (t0 + 1) * kBlockSize)   // tile t0 has its last slot
        compact_flush(t0, t0 == (c_first >> 4) ? (c_first & 15) : 0, kBlockSize);
    }
  };

  // H2O logits go to an LDS window of st_blocks blocks per head of the group
  // (the table chunks are cut to that length) and out to the stash in
  // coalesced 16-byte stores after each chunk: a store in every block's step
  // would make the tile waits two blocks later wait for it too (stores share
  // the load counter).
  const int st_blocks = (stash_floats(KVT, CMP) - kImgFloats) / (group * kBlockSize);
  auto stash_flush = [&](int vb0, int nb) {
    lds_wave_sync();
    const int n4 = nb * kBlockSize / 4;       // 16-byte pieces per head
    for (int idx = lane; idx < group * n4; idx += kWave) {
      const int g = idx / n4, k = idx % n4;
      *reinterpret_cast<f32x4*>(a.stash + ((size_t)s * hq + kvh * group + g) * a.nv_pad + (size_t)vb0 * kBlockSize +
                                4 * k) = *reinterpret_cast<const f32x4*>(&s_stash[g * st_blocks * kBlockSize + 4 * k]);
    }
  };

  // tail: a call that may compute the segment's last block (the pipeline's
  // steady state never does), the only place the new token is patched in.
  auto compute = [&](Regs& r, int i, auto tail) {
    bad |= !r.ok;   // outputs become NaN; the block is still computed
    const int vb = c0 + i;
    const int lb = logical_block(vb, geo.n_sink_blocks, geo.win_start);

    if constexpr (kFuse && decltype(tail)::value) {
      if (fuse && vb == vb_new) {
        // K: token row o_new is lane column c == o_new, which takes chunks
        // 4w + j of the row.  V: tokens 4j..4j+3 sit in lane row j, so o_new is
        // element o_new % 4 of every tile's word pair (16-bit) or quad (f32) in
        // lanes j == o_new / 4, which take dims 16 t + c.
        const bool krow = c == o_new;
        const bool vrow = j == (o_new >> 2);
        const int e = o_new & 3;
        uint32_t kn[KW], vn[NT];
#pragma unroll
        for (int w = 0; w < KW / 4; ++w) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(&s_new[(4 * w + j) * 4]);
          kn[4 * w + 0] = v[0]; kn[4 * w + 1] = v[1]; kn[4 * w + 2] = v[2]; kn[4 * w + 3] = v[3];
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if constexpr (EB == 1) vn[t] = reinterpret_cast<const uint8_t*>(s_new + NW)[16 * t + c];
          else if constexpr (EB == 2) vn[t] = reinterpret_cast<const uint16_t*>(s_new + NW)[16 * t + c];
          else vn[t] = s_new[NW + 16 * t + c];
        }
#pragma unroll
        for (int w = 0; w < KW; ++w) r.k[w] = krow ? kn[w] : r.k[w];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if constexpr (EB == 1) {
            r.v[t][0] = vrow ? ((r.v[t][0] & ~(0xffu << (8 * e))) | (vn[t] << (8 * e))) : r.v[t][0];
          } else if constexpr (EB == 2) {
            const uint32_t keep = (e & 1) ? 0x0000ffffu : 0xffff0000u;
            const uint32_t put = (e & 1) ? (vn[t] << 16) : vn[t];
            r.v[t][0] = (vrow && e < 2) ? ((r.v[t][0] & keep) | put) : r.v[t][0];
            r.v[t][1] = (vrow && e >= 2) ? ((r.v[t][1] & keep) | put) : r.v[t][1];
          } else {
#pragma unroll
            for (int ee = 0; ee < 4; ++ee) r.v[t][ee] = (vrow && ee == e) ? vn[t] : r.v[t][ee];
          }
        }
        if constexpr (is_quantised(KVT)) {   // lane row j holds the scales of tokens 4j..4j+3
#pragma unroll
          for (int ee = 0; ee < 4; ++ee) {
            r.ks[ee] = (vrow && ee == e) ? ks_new : r.ks[ee];
            r.vs[ee] = (vrow && ee == e) ? vs_new : r.vs[ee];
          }
        }
      }
    }

    if constexpr (CMP) {
      bad |= r.km < 0;                 // poisoned sequence
      compact_put(r);                  // (an entry outside the pool read block 0: its bytes are copied)
    }

    // ---- S = K q^T: lane (c, j) receives head c's logits of tokens 4j..4j+3
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (OP32) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) sacc = mfma_f32_k4(__uint_as_float(r.k[e]), qf[e], sacc);
    } else {
#pragma unroll
      for (int st = 0; st < DPL / 8; ++st) {
        uint32_t av[4];
        if constexpr (KF16) {
          int8x4_to_f16x4_biased(r.k[2 * st], av[0], av[1]);
          int8x4_to_f16x4_biased(r.k[2 * st + 1], av[2], av[3]);
        } else if constexpr (is_code8(KVT)) {
          code8x4_to_bf16x4<KVT>(r.k[2 * st], av[0], av[1]);
          code8x4_to_bf16x4<KVT>(r.k[2 * st + 1], av[2], av[3]);
        } else {
          av[0] = r.k[4 * st]; av[1] = r.k[4 * st + 1]; av[2] = r.k[4 * st + 2]; av[3] = r.k[4 * st + 3];
        }
        sacc = mfma_k32<QF16>(av, &qhi[4 * st], sacc);
        if constexpr (QSPLIT) sacc = mfma_k32<QF16>(av, &qlo[4 * st], sacc);
      }
    }

    // ---- logits (base 2) with the keep-set mask
    const int blk0 = lb * kBlockSize;
    const bool full = (blk0 + kBlockSize <= L) && (blk0 + kBlockSize <= sinks || blk0 >= keep_lo);
    float x[4];
    bool valid[4] = {true, true, true, true};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = (BIAS ? sacc[e] - qbias : sacc[e]) * lscale;
      if constexpr (is_quantised(KVT)) x[e] *= r.ks[e];
    }
    if constexpr (CMP) {   // evicted tokens (their V zeroed with the rest below)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        valid[e] = (r.km >> (4 * j + e)) & 1;
        x[e] = valid[e] ? x[e] : -INFINITY;
      }
    }
    if (CMP || !full) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int p = blk0 + 4 * j + e;
        if constexpr (CMP) valid[e] = valid[e] && p < L;   // (no sinks or window)
        else valid[e] = p < L && (p < sinks || p >= keep_lo);
        x[e] = valid[e] ? x[e] : -INFINITY;
      }
      // Slots outside the keep-set may hold anything (NaN included): zero their V.
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if constexpr (VW == 1) {
          const uint32_t msk = (valid[0] ? 0xffu : 0u) | (valid[1] ? 0xff00u : 0u) |
                               (valid[2] ? 0xff0000u : 0u) | (valid[3] ? 0xff000000u : 0u);
          r.v[t][0] &= msk;
        } else if constexpr (VW == 2) {
          r.v[t][0] &= (valid[0] ? 0xffffu : 0u) | (valid[1] ? 0xffff0000u : 0u);
          r.v[t][1] &= (valid[2] ? 0xffffu : 0u) | (valid[3] ? 0xffff0000u : 0u);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) r.v[t][e] = valid[e] ? r.v[t][e] : 0u;
        }
      }
    }

    // ---- online softmax with a slack: the reference max only moves (and the
    // accumulators are rescaled) when a logit exceeds it by more than
    // kRescaleSlack, so exp2 stays <= 2^kRescaleSlack and most blocks skip the
    // rescale.  Any reference gives the same normalised result.
    const float mb = row_max4(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
    const bool need = mb > m_run + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(need) != 0ull) {
      const float m_new = need ? mb : m_run;
      const float alpha = m_new == m_run ? 1.f : fast_exp2(m_run - m_new);   // 0 on the first block
      l_run *= alpha;
      if constexpr (BIAS) p_run *= alpha;
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] *= alpha;
      m_run = m_new;
    }
    const float mref = m_run == -INFINITY ? 0.f : m_run;
    float pr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pr[e] = fast_exp2(x[e] - mref);
    l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);

    if (a.stash != nullptr && head_ok)       // block i of the chunk in the LDS window
      *reinterpret_cast<f32x4*>(&s_stash[(c * st_blocks + i) * kBlockSize + 4 * j]) = f32x4{x[0], x[1], x[2], x[3]};

    // ---- probabilities as the PV B operand (V's per-token scale folded in)
    float pv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (is_quantised(KVT)) pv[e] = valid[e] ? pr[e] * r.vs[e] : 0.f;
      else pv[e] = pr[e];
    }

    // ---- O^T += V^T P^T: lane (c, j) accumulates head c, dims 16t + 4j + e
    if constexpr (OP32) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[t] = mfma_f32_k4(__uint_as_float(r.v[t][e]), pv[e], acc[t]);
      }
    } else {
      uint32_t ph[2], pl[2];
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const float f0 = pv[2 * w], f1 = pv[2 * w + 1];
        uint32_t h0, h1, l0, l1;
        if constexpr (F16) {
          h0 = f32_to_f16_bits(f0);
          h1 = f32_to_f16_bits(f1);
          l0 = f32_to_f16_bits(f0 - f16_to_f32(h0));
          l1 = f32_to_f16_bits(f1 - f16_to_f32(h1));
        } else {
          h0 = __float_as_uint(f0) >> 16;           // truncated high part, exact residual below
          h1 = __float_as_uint(f1) >> 16;
          l0 = __float_as_uint(f0 - bf16_to_f32(h0)) >> 16;
          l1 = __float_as_uint(f1 - bf16_to_f32(h1)) >> 16;
          if constexpr (BIAS) p_run += (bf16_to_f32(h0) + bf16_to_f32(l0)) + (bf16_to_f32(h1) + bf16_to_f32(l1));
        }
        ph[w] = h0 | (h1 << 16);
        pl[w] = l0 | (l1 << 16);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        uint32_t v0, v1;
        if constexpr (is_code8(KVT)) {
          code8x4_to_bf16x4<KVT>(r.v[t][0], v0, v1);
        } else {
          v0 = r.v[t][0];
          v1 = r.v[t][1];
        }
        acc[t] = mfma_k16<F16>(v0, v1, ph[0], ph[1], acc[t]);
        acc[t] = mfma_k16<F16>(v0, v1, pl[0], pl[1], acc[t]);
      }
    }
  };

  constexpr std::false_type kMid{};
  constexpr std::true_type kTail{};
  const int chunk_cap = a.stash != nullptr ? st_blocks : kTabBlocks;
  for (; c0 < seg_vb1; c0 += chunk_cap) {
    // The chunk's table entries go to LDS first: the loop reads them with LDS
    // loads, whose wait counter is separate from the K/V loads', so the
    // compiler can wait for exactly the block about to be computed.
    const int n = min(chunk_cap, seg_vb1 - c0);
    const bool first = fuse && c0 == seg_vb0;
    {
      // 512 entries per memory latency: every lane issues 8 entry loads before
      // the first is waited for (indices past the chunk reload its last entry,
      // so no load is conditional); the fused append's row loads join the
      // first round.  (16 loads per lane raised every instance by ~16 VGPRs.)
      constexpr int TU = 8;
      if (first) fused_load();
      for (int b0 = 0; b0 < n; b0 += kWave * TU) {
        int ent[TU];
#pragma unroll
        for (int u = 0; u < TU; ++u)
          ent[u] = trow[logical_block(c0 + min(b0 + lane + kWave * u, n - 1), geo.n_sink_blocks, geo.win_start)];
#pragma unroll
        for (int u = 0; u < TU; ++u) {
          const int k = b0 + lane + kWave * u;
          if (k < n) s_tab[k] = ent[u];
        }
      }
      if (first) fused_stage();
    }
    lds_wave_sync();
#if PKV_ATTN_PIPE == 2
    // Software pipeline: block i+1's loads are in flight while block i computes.
    Regs ra, rb;
    int i = 0;
    if (n > 0) load(ra, 0);
    for (; i + 2 < n; i += 2) {   // steady state: every load unconditional
      load(rb, i + 1);
      compute(ra, i, kMid);
      load(ra, i + 2);
      compute(rb, i + 1, kMid);
    }
    // at most 2 blocks left; ra holds block i
    if (i + 1 < n) load(rb, i + 1);
    if (i < n) compute(ra, i, kTail);
    if (i + 1 < n) compute(rb, i + 1, kTail);
#else
    // Software pipeline: blocks i+1 and i+2 are in flight while block i computes.
    Regs r0, r1, r2;
    int i = 0;
    if (n > 0) load(r0, 0);
    if (n > 1) load(r1, 1);
    for (; i + 4 < n; i += 3) {   // steady state: every load unconditional
      load(r2, i + 2);
      compute(r0, i, kMid);
      load(r0, i + 3);
      compute(r1, i + 1, kMid);
      load(r1, i + 4);
      compute(r2, i + 2, kMid);
    }
    // at most 4 blocks left; r0, r1 hold blocks i, i+1 where they exist
    if (i + 2 < n) load(r2, i + 2);
    if (i < n) compute(r0, i, kTail);
    if (i + 3 < n) load(r0, i + 3);
    if (i + 1 < n) compute(r1, i + 1, kTail);
    if (i + 2 < n) compute(r2, i + 2, kTail);
    if (i + 3 < n) compute(r0, i + 3, kTail);
#endif
    if (a.stash != nullptr) stash_flush(c0, n);
    lds_wave_sync();   // s_tab (and the logit window) are rewritten by the next chunk
  }

  if constexpr (CMP) {   // the open tile: this wave's slots of it
    if (c_first >= 0 && (c_end & 15) != 0) {
      const int T = (c_end - 1) >> 4;
      compact_flush(T, T == (c_first >> 4) ? (c_first & 15) : 0, c_end & 15);
    }
  }

  l_run = row_sum4(l_run);   // head c's exp-sum, in all four lanes of column c
  if (bad) l_run = __builtin_nanf("");
  if constexpr (BIAS) {      // biased V operands added kInt8Bias * sum_p P_p to every output dim
    const float vbias = kInt8Bias * row_sum4(p_run);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] -= vbias;
  }
  if (!head_ok) return;
  if constexpr (CH) {   // V's channel scales: sum_p P_p (code_p * s) = s * sum_p P_p code_p
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const f32x4 vsc = *reinterpret_cast<const f32x4*>(a.v_scale + (size_t)kvh * D + 16 * t + 4 * j);
      acc[t] *= vsc;
    }
  }
  // lane (c, j) holds head c's output dims 16 t + 4 j + e
  const size_t hs = (size_t)s * hq + head;
  if (whole) {
    const float inv = 1.f / l_run;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) store_out(a.out, hs * D + 16 * t + 4 * j + e, a.out_dtype, acc[t][e] * inv);
    }
    if (j == 0 && a.fin_ml != nullptr) {
      a.fin_ml[hs * 2 + 0] = m_run;
      a.fin_ml[hs * 2 + 1] = l_run;
    }
  } else {
    const size_t pi = hs * a.p_max + partial_slot(seg_vb0);
#pragma unroll
    for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4*>(a.part_acc + pi * D + 16 * t + 4 * j) = acc[t];
    if (j == 0) {
      a.part_ml[pi * 2 + 0] = m_run;
      a.part_ml[pi * 2 + 1] = l_run;
    }
  }
}

// The fused decode append's stores of (sequence sq, KV head h) at offset
// (L - 1) % 16 of pool block blk: the source rows' bits (16-bit and f32
// pools) or their 8-bit codes with the per-token scales, quantised exactly as
// the write kernels do.  kWaveWide: the wave's 64 lanes share the row; else
// the calling lane does it all.
template <int KVT, int QT, int D, bool kWaveWide>
__device__ __forceinline__ void append_row(const AttnArgs& a, int sq, int h, int L, int blk) {
  constexpr int EB = KvType<KVT>::kBytes;
  constexpr bool C8 = is_code8(KVT);
  constexpr int SEB = C8 ? (QT == DT_F32 ? 4 : 2) : EB;   // source element bytes
  constexpr int NWS = D * SEB / 4;
  constexpr int EPW = 4 / SEB;
  const int ln = kWaveWide ? (int)(threadIdx.x & 63) : 0;
  constexpr int step = kWaveWide ? kWave : 1;
  const int o = (L - 1) & (kBlockSize - 1);
  const size_t row = ((size_t)sq * a.num_kv_heads + h) * NWS;
  const uint32_t* kr = reinterpret_cast<const uint32_t*>(a.k_new) + row;
  const uint32_t* vr = reinterpret_cast<const uint32_t*>(a.v_new) + row;
  const size_t tile = (size_t)blk * a.num_kv_heads + h;
  uint8_t* kt = reinterpret_cast<uint8_t*>(a.k_store) + tile * (size_t)(kBlockSize * D * EB);
  uint8_t* vt = reinterpret_cast<uint8_t*>(a.v_store) + tile * (size_t)(kBlockSize * D * EB);
  if constexpr (!C8) {
    for (int k = ln; k < NWS; k += step) {   // bytes 4k..4k+3 of the row
      const uint32_t kw = kr[k], vw = vr[k];
      *reinterpret_cast<uint32_t*>(kt + ((size_t)(k / 4) * kBlockSize + o) * 16 + (k % 4) * 4) = kw;
      if constexpr (EB == 2) {
        *reinterpret_cast<uint16_t*>(vt + (size_t)v_chunk_offset<2>(o, 2 * k) * 2) = (uint16_t)vw;
        *reinterpret_cast<uint16_t*>(vt + (size_t)v_chunk_offset<2>(o, 2 * k + 1) * 2) = (uint16_t)(vw >> 16);
      } else {
        *reinterpret_cast<uint32_t*>(vt + (size_t)v_chunk_offset<4>(o, k) * 4) = vw;
      }
    }
  } else {
    auto elem = [](uint32_t w, int i) { return SEB == 4 ? w : (w >> (16 * i)) & 0xffffu; };
    float ks = 0.f, vs = 0.f;
    if constexpr (is_quantised(KVT)) {
      float km = 0.f, vm = 0.f;
      for (int k = ln; k < NWS; k += step) {
        const uint32_t kw = kr[k], vw = vr[k];
#pragma unroll
        for (int i = 0; i < EPW; ++i) {
          km = fmaxf(km, fabsf(raw_to_f32<QT>(elem(kw, i))));
          vm = fmaxf(vm, fabsf(raw_to_f32<QT>(elem(vw, i))));
        }
      }
      if constexpr (kWaveWide) {
        km = wave_max(km);
        vm = wave_max(vm);
      }
      ks = __fdiv_rn(km, max_code8<KVT>());
      vs = __fdiv_rn(vm, max_code8<KVT>());
      if (ln == 0) {
        a.k_scale_store[tile * kBlockSize + o] = ks;
        a.v_scale_store[tile * kBlockSize + o] = vs;
      }
    }
    for (int k = ln; k < NWS; k += step) {
      const uint32_t kw = kr[k], vw = vr[k];
#pragma unroll
      for (int i = 0; i < EPW; ++i) {
        const int d = k * EPW + i;
        const float kc = is_channel_scaled(KVT) ? a.k_scale[(size_t)h * D + d] : ks;
        const float vc = is_channel_scaled(KVT) ? a.v_scale[(size_t)h * D + d] : vs;
        store_elem<1>(kt + k_chunk_offset<1>(o, d), stored_code<QT, KVT>(elem(kw, i), kc));
        store_elem<1>(vt + v_chunk_offset<1>(o, d), stored_code<QT, KVT>(elem(vw, i), vc));
      }
    }
  }
}

// Pool block that takes the fused append of a sequence of length L (the
// decode append's rule: L in [1, 16 * stride] and a table entry in the pool),
// or -1.
__device__ __forceinline__ int append_block(const AttnArgs& a, int sq, int L) {
  if (L < 1 || L > a.table_stride * kBlockSize) return -1;
  const int blk = a.block_tables[(size_t)sq * a.table_stride + (L - 1) / kBlockSize];
  return (blk < 0 || blk >= a.num_blocks) ? -1 : blk;
}

// The fused decode append's stores, issued when the wave has attended all its
// segments (nothing waits for them then): the rows of KV head kvh of every
// sequence in [end_lo, end_hi] with attended blocks -- the sequences whose
// last block this wave attended.
template <int KVT, int QT, int D>
__device__ __forceinline__ void append_stores(const AttnArgs& a, int kvh, int end_lo, int end_hi) {
  for (int sq = end_lo; sq <= end_hi; ++sq) {
    const int L = a.context_lens[sq];
    if (attended_blocks(a, L) == 0) continue;   // stored in pass 1 of the kernel, if at all
    const int blk = append_block(a, sq, L);
    if (blk >= 0) append_row<KVT, QT, D, true>(a, sq, kvh, L, blk);
  }
}

// Inclusive prefix sum over the wave's 64 lanes.
__device__ __forceinline__ int wave_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

// Persistent decode attention with single-wave workgroups, as many as the GPU
// holds at once.
//
// The attended blocks of all sequences form one sequence-major list, cut into
// n_ranges ranges whose lengths alternate between pa and pb (>= kPartBlocks).
// Workgroup w takes one range for one KV head.  Workgroup ids go to the 8
// XCDs in turn: with the head-fastest order (8-bit pools) the KV heads of a
// range -- whose tiles sit side by side in the pool -- are read at the same
// time and every XCD gets the same share; with the head-major order (16-bit
// and f32 pools) range r runs on XCD r % 8 and pb < pa evens out the slower
// odd XCDs.  A range is cut at sequence boundaries into segments: a segment
// that is a whole sequence writes the output directly, the others write
// partials that attn_reduce_kernel merges.  Cuts inside a sequence are range
// starts, at least kPartBlocks apart, so partial slots (partial_slot) are
// distinct.
template <int KVT, int QT, int D, bool CMP>
__global__ void __launch_bounds__(64) attn_wave_kernel(const AttnArgs a) {
  __shared__ int s_tab[kTabBlocks];
  // the new token's stored K and V rows when the decode append is fused in
  __shared__ uint32_t s_new[2 * D * KvType<KVT>::kBytes / 4];
  // the H2O logit window (used only when attn_mass is requested)
  __shared__ __attribute__((aligned(16))) float s_stash[stash_floats(KVT, CMP)];
  const int hkv = a.num_kv_heads;
  const int B = a.num_seqs;
  const int lane = threadIdx.x;
  const int n_ranges = gridDim.x / hkv;
  constexpr bool kHeadFast = is_code8(KVT) ? PKV_ATTN_HEAD_FAST_8BIT : PKV_ATTN_HEAD_FAST;
  int r = kHeadFast ? blockIdx.x / hkv : blockIdx.x % n_ranges;
  int kvh = kHeadFast ? blockIdx.x % hkv : blockIdx.x / n_ranges;
  if (kHeadFast && is_quantised(KVT) && PKV_ATTN_PAIR_8BIT && hkv % 2 == 0 && gridDim.x % 16 == 0) {
    // Heads 2i and 2i+1 of one range on one XCD, 8 ids apart (dispatched
    // together): their per-token scale rows share 128-byte lines.
    const int x = blockIdx.x % 8, k = blockIdx.x / 8;
    const int v = (k / 2) * 8 + x;          // (range, head pair), head pair fastest
    r = v / (hkv / 2);
    kvh = 2 * (v % (hkv / 2)) + k % 2;
  }

  // Pass 1: total attended blocks; workgroup 0 records the per-sequence prefix
  // and R for the merge kernel; NaN outputs for unusable lengths.
  int total = 0;
  int nva0 = 0, incl0 = 0;     // the first 64 sequences' counts, kept for pass 2
  for (int base = 0; base < B; base += kWave) {
    const int sq = base + lane;
    const int nva = sq < B ? attended_blocks(a, a.context_lens[sq]) : 0;
    const int incl = wave_scan(nva);
    if (base == 0) {
      nva0 = nva;
      incl0 = incl;
    }
    if (blockIdx.x == 0 && sq < B) a.seq_prefix[sq] = total + incl - nva;
    if (sq < B && nva == 0 && sq % (int)gridDim.x == (int)blockIdx.x) {
      for (int idx = 0; idx < a.num_q_heads * D; ++idx)
        store_out(a.out, (size_t)sq * a.num_q_heads * D + idx, a.out_dtype, __builtin_nanf(""));
      if constexpr (fused_append_built(KVT, QT)) {
        // no wave attends this sequence; its token is still stored where the
        // decode append would store it (a length beyond max_context_len)
        const int L = a.context_lens[sq];
        const int blk = a.k_new != nullptr ? append_block(a, sq, L) : -1;
        if (blk >= 0) {
          for (int h = 0; h < hkv; ++h) append_row<KVT, QT, D, false>(a, sq, h, L, blk);
        }
      }
    }
    total += __shfl(incl, kWave - 1, kWave);
  }
  // Ranges alternate between two lengths, pa (even r) and pb (odd r).  With
  // the head-major order and a range count divisible by 8, range r runs on
  // XCD r % 8 (workgroup ids are dealt to the 8 XCDs in turn), so pb < pa
  // gives the odd XCDs less work: on MI355X they stream the same blocks about
  // 8% slower than the even ones (measured per XCD with the wall clock).
  int pa, pb;
  if (!kHeadFast && PKV_ATTN_ODD_SHARE != 1000 && n_ranges % 8 == 0) {
    const long long pair = (2LL * total + n_ranges - 1) / n_ranges;     // pa + pb
    pa = (int)(pair * 1000 / (1000 + PKV_ATTN_ODD_SHARE));
    pb = (int)(pair - pa);
  } else {
    pa = pb = (int)(((long long)total + n_ranges - 1) / n_ranges);
  }
  if (pa < kPartBlocks) pa = kPartBlocks;
  if (pb < kPartBlocks) pb = kPartBlocks;
  if (blockIdx.x == 0 && lane == 0) {
    a.seq_prefix[B] = total;
    a.hdr->per = pa;
    a.hdr->per_odd = pb;
  }
  const long long u0 = (long long)(r / 2) * (pa + pb) + (r % 2) * pa;
  if (u0 >= total) return;
  const long long u1 = min(u0 + (r % 2 ? pb : pa), (long long)total);

  // Pass 2: the sequence holding block u0, and its prefix.
  int sq = -1, prefix = 0, run = 0;
  for (int base = 0; base < B && sq < 0; base += kWave) {
    const int q = base + lane;
    // (the first 64 come from pass 1's registers: no second load of the lengths)
    const int nva = base == 0 ? nva0 : (q < B ? attended_blocks(a, a.context_lens[q]) : 0);
    const int incl = base == 0 ? incl0 : wave_scan(nva);
    const int excl = run + incl - nva;
    const unsigned long long hit = __ballot(nva > 0 && excl <= u0 && u0 < excl + nva);
    if (hit != 0ull) {
      const int src = __ffsll((long long)hit) - 1;
      sq = base + src;
      prefix = __shfl(excl, src, kWave);
    }
    run += __shfl(incl, kWave - 1, kWave);
  }
  sq = __builtin_amdgcn_readfirstlane(sq);
  prefix = __builtin_amdgcn_readfirstlane(prefix);

  long long u = u0;
  int end_lo = B, end_hi = -1;   // sequences whose last block this wave attends
  while (u < u1) {
    const int L = a.context_lens[sq];
    const int nva = attended_blocks(a, L);
    const int vb = (int)(u - prefix);
    const int cnt = (int)min((long long)(nva - vb), u1 - u);
    wave_segment<KVT, QT, D, CMP>(a, s_tab, s_new, s_stash, sq, kvh, L, vb, vb + cnt);
    if (vb + cnt == nva) {
      end_lo = min(end_lo, sq);
      end_hi = sq;
    }
    u += cnt;
    if (u < u1) {
      // next sequence with attended blocks (one exists: u < total)
      prefix += nva;
      ++sq;
      while (attended_blocks(a, a.context_lens[sq]) == 0) ++sq;
    }
  }
  if constexpr (fused_append_built(KVT, QT)) {
    if (a.k_new != nullptr) append_stores<KVT, QT, D>(a, kvh, end_lo, end_hi);
  }
}

// The segments a sequence was cut into: block 0 and every range cut inside the
// sequence's span of the block list.  Cut k is (k / 2) P + (k odd ? pa : 0),
// P = pa + pb; n == 1 means one segment, whose wave wrote the output itself.
struct SeqCuts {
  long long k0;   // first cut after the sequence start
  int base, n, pa, P;
  __device__ long long cut(long long k) const { return (k / 2) * P + (k % 2 ? pa : 0); }
  __device__ int slot(int i) const { return i == 0 ? 0 : partial_slot((int)(cut(k0 + i - 1) - base)); }
};

__device__ __forceinline__ SeqCuts seq_cuts(const AttnArgs& a, int s, int nva) {
  SeqCuts c;
  c.pa = a.hdr->per;
  c.P = c.pa + a.hdr->per_odd;
  c.base = a.seq_prefix[s];
  c.k0 = 2LL * (c.base / c.P) + (c.base % c.P < c.pa ? 1 : 2);
  const int end = c.base + nva;
  c.n = 1;
  if (c.cut(c.k0) < end) {
    const long long e = end - 1;                    // index of the last cut before end: the range holding e
    const long long k_last = 2LL * (e / c.P) + (e % c.P < c.pa ? 0 : 1);
    c.n = (int)(k_last - c.k0 + 2);
  }
  return c;
}

// Log-sum-exp merge of one (sequence, query head): the partials of the
// segments the sequence was cut into.  A sequence that was one segment
// already has its output.  With parts == 1 one wave merges the head; with
// parts == 4 the head has a 4-wave workgroup and wave w takes segment chunks
// w, w + 4, ... (few sequences: each is cut into many segments).  Per chunk
// of 16 every lane loads its D / 64 output dims of all 16 partials and lane k
// the (max, sum) of segment k, all before the first wait (the merge is
// latency-bound); then the wave max, the weights exp2(m_k - M), and the
// weighted sums, with a running rescale past one chunk.  Up to 16 segments
// wave 0 stores the output itself; past that the four waves' (M, l, o) are
// combined through LDS, so n segments cost ceil(n / 64) round trips, not
// ceil(n / 16).
template <int D>
__device__ __forceinline__ void merge_head(const AttnArgs& a, int s, int h, int w, int lane, int parts) {
  constexpr int kChunk = 16, kParts = 4;
  constexpr int DL = D / 64;                      // output dims per lane
  using VT = typename std::conditional<DL == 2, float2, float>::type;
  __shared__ float s_o[kParts][D];
  __shared__ float s_ml[kParts][2];
  const int nva = attended_blocks(a, a.context_lens[s]);
  if (nva == 0) return;                             // NaN already written
  const SeqCuts c = seq_cuts(a, s, nva);
  if (c.n == 1) return;                             // one segment: written directly
  const int n = c.n;
  if (parts > 1 && n <= kChunk && w != 0) return;   // the whole workgroup agrees on n
  const int part = parts > 1 ? w : 0;
  const size_t hs = (size_t)s * a.num_q_heads + h;
  const float* ml = a.part_ml + hs * a.p_max * 2;
  const float* pacc = a.part_acc + hs * a.p_max * D;
  float M = -INFINITY, lsum = 0.f;
  float o[DL];
#pragma unroll
  for (int e = 0; e < DL; ++e) o[e] = 0.f;
  for (int i0 = part * kChunk; i0 < n; i0 += parts * kChunk) {
    const int cnt = min(kChunk, n - i0);
    VT v[kChunk];
#pragma unroll
    for (int k = 0; k < kChunk; ++k)   // past cnt: the last segment again (weight 0, skipped)
      v[k] = *reinterpret_cast<const VT*>(pacc + (size_t)c.slot(i0 + min(k, cnt - 1)) * D + DL * lane);
    float mi = -INFINITY, li = 0.f;
    if (lane < cnt) {
      const float2 x = *reinterpret_cast<const float2*>(ml + 2 * c.slot(i0 + lane));
      mi = x.x;
      li = x.y;
    }
    float Mc = mi;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) Mc = fmaxf(Mc, __shfl_xor(Mc, off, kWave));
    const float Mn = fmaxf(M, Mc);
    const float keep = M == -INFINITY ? 0.f : fast_exp2(M - Mn);
    const float f = mi == -INFINITY ? 0.f : fast_exp2(mi - Mn);
    float lc = f * li;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) lc += __shfl_xor(lc, off, kWave);
    lsum = lsum * keep + lc;
#pragma unroll
    for (int e = 0; e < DL; ++e) o[e] *= keep;
#pragma unroll
    for (int k = 0; k < kChunk; ++k) {
      if (k < cnt) {
        const float fk = __shfl(f, k, kWave);
        if constexpr (DL == 2) {
          o[0] += fk * v[k].x;
          o[1] += fk * v[k].y;
        } else {
          o[0] += fk * v[k];
        }
      }
    }
    M = Mn;
  }
  if (parts > 1 && n > kChunk) {   // combine the four waves' states (one without chunks: M = -inf, weight 0)
#pragma unroll
    for (int e = 0; e < DL; ++e) s_o[w][DL * lane + e] = o[e];
    if (lane == 0) {
      s_ml[w][0] = M;
      s_ml[w][1] = lsum;
    }
    __syncthreads();
    if (w != 0) return;
    float Mt = -INFINITY;
#pragma unroll
    for (int p = 0; p < kParts; ++p) Mt = fmaxf(Mt, s_ml[p][0]);
    lsum = 0.f;
#pragma unroll
    for (int e = 0; e < DL; ++e) o[e] = 0.f;
#pragma unroll
    for (int p = 0; p < kParts; ++p) {
      const float mp = s_ml[p][0];
      const float f = mp == -INFINITY ? 0.f : fast_exp2(mp - Mt);
      lsum += f * s_ml[p][1];
#pragma unroll
      for (int e = 0; e < DL; ++e) o[e] += f * s_o[p][DL * lane + e];
    }
  }
#pragma unroll
  for (int e = 0; e < DL; ++e) store_out(a.out, hs * D + DL * lane + e, a.out_dtype, o[e] / lsum);
}

// split: one query head per workgroup (grid.x = Hq), else four (one per wave).
template <int D>
__global__ void __launch_bounds__(256) attn_reduce_kernel(const AttnArgs a, int split) {
  const int w = threadIdx.x >> 6;
  const int h = split ? (int)blockIdx.x : (int)blockIdx.x * 4 + w;
  if (h >= a.num_q_heads) return;   // 4-head workgroups only: no barrier there
  merge_head<D>(a, blockIdx.y, h, w, threadIdx.x & 63, split ? 4 : 1);
}

// H2O mass of 256 attended positions of sequence s (workgroup-uniform s):
// scores[s][p] += mean over query heads of exp2(x - M_h) / l_h, kept p only,
// taken as exp2(x - (M_h + log2 l_h)): one exponential per head and no
// division (the folded offset's rounding moves the result by ~1e-6
// relative).  The heads' offsets are staged in LDS, 256 heads at a time, so
// the loop over heads issues only the (coalesced) logit loads.  A head of a
// sequence that was one segment has them from its wave; otherwise the thread
// of head h merges the segments' (max, exp-sum) pairs itself, 16 loads in
// flight at a time (as many round trips as the output merge's 16 segments per
// wave), so that the mass does not wait for the output merge.
__device__ __forceinline__ void mass_block(const AttnArgs& a, int s, int bx) {
  constexpr int kPairs = 16;
  __shared__ float s_m[256];
  const int v = bx * 256 + threadIdx.x;                  // attended (virtual) position
  const int L = a.context_lens[s];
  const int len_cap = min(a.max_context_len, a.table_stride * kBlockSize);
  if (L < 1 || L > len_cap) return;                      // the whole workgroup
  const KeepGeom geo = keep_geometry(L, a.num_sinks, a.window);
  const int p = logical_block(v / kBlockSize, geo.n_sink_blocks, geo.win_start) * kBlockSize + v % kBlockSize;
  const bool active = v < geo.n_virtual * kBlockSize && is_kept(p, L, a.num_sinks, a.window);
  const int hq = a.num_q_heads;
  const SeqCuts c = seq_cuts(a, s, geo.n_virtual);
  float sum = 0.f;
  for (int h0 = 0; h0 < hq; h0 += 256) {
    const int hn = min(256, hq - h0);
    __syncthreads();                                      // the previous heads are read
    if ((int)threadIdx.x < hn) {
      const size_t hs = (size_t)s * hq + h0 + threadIdx.x;
      float M = -INFINITY, l = 0.f;
      if (c.n == 1) {
        M = a.fin_ml[hs * 2];
        l = a.fin_ml[hs * 2 + 1];
      } else {
        const float* ml = a.part_ml + hs * a.p_max * 2;
        for (int i0 = 0; i0 < c.n; i0 += kPairs) {
          const int cnt = min(kPairs, c.n - i0);
          float2 x[kPairs];
#pragma unroll
          for (int k = 0; k < kPairs; ++k)
            x[k] = *reinterpret_cast<const float2*>(ml + 2 * c.slot(i0 + min(k, cnt - 1)));
          float Mc = -INFINITY;
#pragma unroll
          for (int k = 0; k < kPairs; ++k)
            if (k < cnt) Mc = fmaxf(Mc, x[k].x);
          const float Mn = fmaxf(M, Mc);
          float lc = 0.f;
#pragma unroll
          for (int k = 0; k < kPairs; ++k)
            if (k < cnt && x[k].x != -INFINITY) lc += fast_exp2(x[k].x - Mn) * x[k].y;
          l = (M == -INFINITY ? 0.f : l * fast_exp2(M - Mn)) + lc;
          M = Mn;
        }
      }
      s_m[threadIdx.x] = M + __builtin_amdgcn_logf(l);   // v_log_f32: log2
    }
    __syncthreads();
    if (active) {
      const float* x = a.stash + ((size_t)s * hq + h0) * a.nv_pad + v;
#pragma unroll 8
      for (int h = 0; h < hn; ++h) sum += fast_exp2(x[(size_t)h * a.nv_pad] - s_m[h]);
    }
  }
  if (!active) return;
  if (a.keep_map == nullptr) {
    a.attn_mass[(size_t)s * a.mass_stride + p] += sum / (float)hq;
  } else {
    // compacting call: a kept position's score moves to its rank in the
    // compacted row, with this step's mass added; evicted ones are dropped
    const KeepMapEntry m = a.keep_map[(size_t)s * a.map_stride + p / kBlockSize];
    const uint32_t mask = (uint32_t)m.w0 & 0xffffu;
    const int t = p % kBlockSize;
    if (m.w0 >= 0 && ((mask >> t) & 1u)) {
      const int rank = m.rank + __builtin_popcount(mask & ((1u << t) - 1u));
      if (rank < a.mass_stride)
        a.attn_mass[(size_t)s * a.mass_stride + rank] = a.mass_src[(size_t)s * a.mass_src_stride + p] + sum / (float)hq;
    }
  }
}

// The H2O step's tail in one launch: the first rx workgroups of row s merge
// the output as attn_reduce_kernel does; the rest add the mass of 256
// positions each.  Neither reads what the other writes.
template <int D>
__global__ void __launch_bounds__(256) attn_merge_mass_kernel(const AttnArgs a, int split) {
  const int rx = split ? a.num_q_heads : (a.num_q_heads + 3) / 4;
  if ((int)blockIdx.x < rx) {
    const int w = threadIdx.x >> 6;
    const int h = split ? (int)blockIdx.x : (int)blockIdx.x * 4 + w;
    if (h < a.num_q_heads) merge_head<D>(a, blockIdx.y, h, w, threadIdx.x & 63, split ? 4 : 1);
  } else {
    mass_block(a, blockIdx.y, blockIdx.x - rx);
  }
}

namespace {

// Single-wave workgroups launched: per CU, as many as fit (or the build-time
// count), times the CU count; cached per device.
template <int KVT, int QT, int D, bool CMP>
int resident_waves() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_wave_kernel<KVT, QT, D, CMP>, kWave, 0) != hipSuccess)
    return 0;
  if (per_cu < 1) per_cu = 1;
  const int want = is_code8(KVT) ? PKV_ATTN_WAVES_PER_CU_FP8 : PKV_ATTN_WAVES_PER_CU;
  if (want > 0 && want < per_cu) per_cu = want;
  const int n = cus * per_cu;
  cache[dev] = n;
  return n;
}

template <int KVT, int QT, int D, bool CMP = false>
hipError_t launch_partition(const AttnArgs& a, hipStream_t st, hipEvent_t ev_begin, hipEvent_t ev_end) {
  const int waves = resident_waves<KVT, QT, D, CMP>();
  if (waves <= 0) return hipErrorInvalidDevice;
  const int n_ranges = waves / a.num_kv_heads > 0 ? waves / a.num_kv_heads : 1;
  // With timing events the dispatch stamps them itself (start and end of this
  // kernel), so no marker packets enter the stream between launches.
  if (ev_begin && ev_end)
    hipExtLaunchKernelGGL((attn_wave_kernel<KVT, QT, D, CMP>), dim3(n_ranges * a.num_kv_heads), dim3(kWave), 0, st,
                          ev_begin, ev_end, 0, a);
  else
    hipLaunchKernelGGL((attn_wave_kernel<KVT, QT, D, CMP>), dim3(n_ranges * a.num_kv_heads), dim3(kWave), 0, st, a);
  return hipGetLastError();
}

template <int KVT, int QT>
hipError_t dispatch_d(const AttnArgs& a, int d, hipStream_t st, hipEvent_t eb, hipEvent_t ee) {
  return d == 64 ? launch_partition<KVT, QT, 64>(a, st, eb, ee) : launch_partition<KVT, QT, 128>(a, st, eb, ee);
}

// Compacting calls: 16-bit pools with queries of the pool's dtype, 8-bit
// pools with bf16 or f16 queries.
template <int KVT, int QT>
hipError_t dispatch_compact(const AttnArgs& a, int d, hipStream_t st, hipEvent_t eb, hipEvent_t ee) {
  return d == 64 ? launch_partition<KVT, QT, 64, true>(a, st, eb, ee)
                 : launch_partition<KVT, QT, 128, true>(a, st, eb, ee);
}
template <int KVT>
hipError_t dispatch_compact8(const AttnArgs& a, int q_dtype, int d, hipStream_t st, hipEvent_t eb, hipEvent_t ee) {
  return q_dtype == DT_BF16 ? dispatch_compact<KVT, DT_BF16>(a, d, st, eb, ee)
                            : dispatch_compact<KVT, DT_F16>(a, d, st, eb, ee);
}

template <int KVT>
hipError_t dispatch_q(const AttnArgs& a, int q_dtype, int d, hipStream_t st, hipEvent_t eb, hipEvent_t ee) {
  switch (q_dtype) {
    case DT_F32: return dispatch_d<KVT, DT_F32>(a, d, st, eb, ee);
    case DT_BF16: return dispatch_d<KVT, DT_BF16>(a, d, st, eb, ee);
    default: return dispatch_d<KVT, DT_F16>(a, d, st, eb, ee);
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// Workspace of paged_decode_attn_noalloc: a fixed device array instead of a
// caller buffer, for callers that cannot allocate.  Each GPU the library runs
// on holds its own copy until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol):
// the device address comes from hipGetSymbolAddress, looked up once per device
// with that device current, and that pointer is what the kernels receive.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void** ptr) {
  static std::mutex mu;
  static std::map<int, void*> by_device;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto it = by_device.find(dev);
  if (it == by_device.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) return hipErrorInvalidSymbol;
    it = by_device.emplace(dev, p).first;
  }
  *ptr = it->second;
  return hipSuccess;
}

WorkspaceLayout attn_workspace_layout(int num_seqs, int num_q_heads, int head_dim, int max_context_len,
                                      int num_sinks, int window, bool want_mass) {
  WorkspaceLayout w{};
  const int nv = max_virtual_blocks(max_context_len, num_sinks, window);
  w.p_max = num_partitions(nv) + 1;   // partial_slot() is at most ceil(blocks / kPartBlocks)
  w.nv_pad = nv * kBlockSize;
  const size_t bh = (size_t)num_seqs * num_q_heads;
  size_t off = 0;
  w.acc_off = off;
  off = align256(off + bh * w.p_max * head_dim * sizeof(float));
  w.ml_off = off;
  off = align256(off + bh * w.p_max * 2 * sizeof(float));
  w.hdr_off = off;
  off = align256(off + sizeof(StreamHdr));
  w.prefix_off = off;
  off = align256(off + ((size_t)num_seqs + 1) * sizeof(int));
  if (want_mass) {
    w.stash_off = off;
    off = align256(off + bh * w.nv_pad * sizeof(float));
    w.fin_off = off;
    off = align256(off + bh * 2 * sizeof(float));
  }
  w.total = off;
  return w;
}

hipError_t launch_decode_attn(const AttnArgs& a, int kv_dtype, int q_dtype, int head_dim,
                              hipStream_t st, hipEvent_t ev_begin, hipEvent_t ev_end) {
  if (a.num_seqs == 0) return hipSuccess;
  hipError_t err;
  if (a.keep_map != nullptr) {   // validated: 16-bit pool with q of its dtype, or 8-bit pool with 16-bit q
    switch (kv_dtype) {
      case DT_BF16: err = dispatch_compact<DT_BF16, DT_BF16>(a, head_dim, st, ev_begin, ev_end); break;
      case DT_F16: err = dispatch_compact<DT_F16, DT_F16>(a, head_dim, st, ev_begin, ev_end); break;
      case DT_FP8: err = dispatch_compact8<DT_FP8>(a, q_dtype, head_dim, st, ev_begin, ev_end); break;
      case DT_INT8: err = dispatch_compact8<DT_INT8>(a, q_dtype, head_dim, st, ev_begin, ev_end); break;
      case DT_FP8_CH: err = dispatch_compact8<DT_FP8_CH>(a, q_dtype, head_dim, st, ev_begin, ev_end); break;
      default: err = dispatch_compact8<DT_INT8_CH>(a, q_dtype, head_dim, st, ev_begin, ev_end); break;
    }
  } else switch (kv_dtype) {
    case DT_F32: err = dispatch_q<DT_F32>(a, q_dtype, head_dim, st, ev_begin, ev_end); break;
    case DT_BF16: err = dispatch_q<DT_BF16>(a, q_dtype, head_dim, st, ev_begin, ev_end); break;
    case DT_F16: err = dispatch_q<DT_F16>(a, q_dtype, head_dim, st, ev_begin, ev_end); break;
    case DT_FP8: err = dispatch_q<DT_FP8>(a, q_dtype, head_dim, st, ev_begin, ev_end); break;
    case DT_INT8: err = dispatch_q<DT_INT8>(a, q_dtype, head_dim, st, ev_begin, ev_end); break;
    case DT_FP8_CH: err = dispatch_q<DT_FP8_CH>(a, q_dtype, head_dim, st, ev_begin, ev_end); break;
    default: err = dispatch_q<DT_INT8_CH>(a, q_dtype, head_dim, st, ev_begin, ev_end); break;
  }
  if (err != hipSuccess) return err;
  // Few sequences share the ranges: each is cut into many segments, and a
  // head's merge gets four waves.  Otherwise four heads share a workgroup
  // (measured: one head per workgroup costs ~1.5 us more at 64 sequences).
  const int split = a.num_seqs <= 8;
  const int rx = split ? a.num_q_heads : (a.num_q_heads + 3) / 4;
  if (a.attn_mass != nullptr) {
    dim3 grid(rx + (a.nv_pad + 255) / 256, a.num_seqs);
    if (head_dim == 64) hipLaunchKernelGGL((attn_merge_mass_kernel<64>), grid, dim3(256), 0, st, a, split);
    else hipLaunchKernelGGL((attn_merge_mass_kernel<128>), grid, dim3(256), 0, st, a, split);
  } else {
    dim3 grid(rx, a.num_seqs);
    if (head_dim == 64) hipLaunchKernelGGL((attn_reduce_kernel<64>), grid, dim3(256), 0, st, a, split);
    else hipLaunchKernelGGL((attn_reduce_kernel<128>), grid, dim3(256), 0, st, a, split);
  }
  return hipGetLastError();
}

}  // namespace pkv
