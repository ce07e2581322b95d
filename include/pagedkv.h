/*
 * pagedkv.h -- C ABI of the gfx950 (MI355X) paged KV-cache decode library.
 *
 * Pages this interface follows (cited by title and section throughout):
 *   [LC] "长上下文优化：注意力稀疏化与 KV Cache 管理"
 *        https://www.plumephp.com/llm-long-context-optimization/
 *   [PA] "KV Cache 与 PagedAttention：显存复用与长上下文推理"
 *        https://www.plumephp.com/ai-kv-cache-paged-attention/
 *   [SO] "系统优化"
 *        https://www.threethreeliu.top/projects/knowledge-inference-optimization-memory-9b32e2e927
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every array argument is a DEVICE pointer (HBM of the current HIP device)
 *    unless its comment says "host".  Arrays are dense and row-major.
 *  - The caller owns all memory.  The library never allocates or frees device
 *    memory; scratch space is a caller-provided workspace sized by a query call.
 *    The one exception is paged_decode_attn_noalloc, whose workspace is a fixed
 *    device array of the library (64 MiB per GPU, held until the process ends).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *    call only enqueues work and returns; nothing synchronises implicitly.
 *  - Return value: a pkv_status.  Scalar arguments and pointer presence are
 *    validated on the host BEFORE any HIP call, so a bad argument never reaches
 *    the GPU.  pkv_last_error() gives a thread-local message for the last
 *    non-OK status.  The library never throws and never aborts.
 *  - Device-resident indices (block tables, slot mappings, context lengths,
 *    block pairs) cannot be checked on the host.  Kernels bound-check each one
 *    they use and never touch memory outside the arrays described here; what an
 *    out-of-range value does to the result is stated per call.
 *
 * KV pool layout (one pool per layer; block_size is 16, [PA] "PagedAttention 的设计")
 * ---------------------------------------------------------------------------------
 *   k_pool  [num_blocks][num_kv_heads][head_dim/X][16][X]   K tile in 16-byte chunks:
 *           X = 16 / element bytes (8 for BF16/F16, 16 for FP8, 4 for F32); element
 *           (token o, dim d) of a tile is at [d / X][o][d % X]
 *   v_pool  [num_blocks][num_kv_heads][head_dim/(16Y)][16][4][Y][4]   V tile in 16-byte
 *           chunks: Y = 4 / element bytes (2 for BF16/F16, 4 for FP8, 1 for F32);
 *           element (token o, dim d), t = d / 16, is at [t / Y][d % 16][o / 4][t % Y][o % 4]
 *           (each chunk: 4 consecutive tokens of Y dims that are 16 apart)
 *   k_scale, v_scale  float [num_blocks][num_kv_heads][16]   (PKV_FP8_E4M3 and PKV_INT8: per token)
 *                     float [num_kv_heads][head_dim]         (the _CHANNEL formats: per channel)
 * A token at logical position p of a sequence lives in physical block
 * table[p / 16] at offset p % 16 ([PA] "物理布局示意", [LC] block-table sketch);
 * its flat slot is block * 16 + offset.  With FP8 or INT8 the stored value is
 * decode(code) * scale, one scale per (token, KV head) for K and one for V
 * ([PA] "量化原理": INT8 or FP8 halve the KV bytes; per-token scaling).  The
 * _CHANNEL formats store the same codes with one static scale per (KV head,
 * channel) instead ([PA] "量化原理": per-channel scaling): the value of
 * element (token, h, d) is decode(code) * scale[h][d].  The caller owns and
 * fills these arrays (e.g. from calibration); scales must be positive and
 * finite, and they live outside the pool: block copy, compaction and swap
 * move codes only.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_EINVAL = 1,        /* an argument is out of its documented range or a pointer is NULL */
  PKV_EUNSUPPORTED = 2,  /* valid in principle, not built: head_dim, group size, dtype combination */
  PKV_EWORKSPACE = 3,    /* workspace_bytes smaller than the query call asks for */
  PKV_EDEVICE = 4        /* a HIP launch or runtime call failed; see pkv_last_error() */
} pkv_status;

typedef enum {
  PKV_F32 = 0,
  PKV_BF16 = 1,
  PKV_F16 = 2,
  PKV_FP8_E4M3 = 3,      /* OCP E4M3FN: bias 7, max 448, no infinities, 0x7F/0xFF = NaN */
  PKV_INT8 = 4,          /* two's-complement int8 codes in [-127, 127] */
  PKV_FP8_E4M3_CHANNEL = 5,  /* E4M3FN codes, static per-(KV head, channel) scales */
  PKV_INT8_CHANNEL = 6       /* int8 codes, static per-(KV head, channel) scales */
} pkv_dtype;

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* pkv_last_error(void);

/* Library version, e.g. "pagedkv 0.1.0 gfx950". Host string, never NULL. */
const char* pkv_version(void);

/*
 * paged_decode_slots -- slot of each sequence's newest token (decode step).
 *
 * The token being decoded sits at position context_lens[s] - 1; its slot is
 * block_tables[s][(len-1)/16] * 16 + (len-1) % 16 ([PA] "PagedAttention 的设计":
 * the block table maps logical block to physical block).
 *   block_tables  int32 [num_seqs][block_table_stride]
 *   context_lens  int32 [num_seqs], length INCLUDING the new token
 *   slot_mapping  int64 [num_seqs] out; -1 where the length is < 1, exceeds
 *                 block_table_stride*16, or the table entry is not in [0, num_blocks)
 */
int paged_decode_slots(const int32_t* block_tables, int block_table_stride,
                       const int32_t* context_lens, int num_seqs, int num_blocks,
                       int block_size, int64_t* slot_mapping, void* stream);

/*
 * paged_token_slots -- slots of arbitrary (sequence, position) tokens, e.g. a
 * prefill or a chunk of one: slot = block_tables[seq][pos/16] * 16 + pos % 16
 * ([PA] "物理布局示意").
 *   seq_ids, positions  int32 [num_tokens]
 *   slot_mapping        int64 [num_tokens] out; -1 where seq_id is outside
 *                       [0, num_seqs), pos is outside [0, block_table_stride*16),
 *                       or the table entry is not in [0, num_blocks)
 */
int paged_token_slots(const int32_t* block_tables, int block_table_stride, int num_seqs,
                      const int32_t* seq_ids, const int32_t* positions, int num_tokens,
                      int num_blocks, int block_size, int64_t* slot_mapping, void* stream);

/*
 * paged_kv_write -- store new tokens' K and V into the paged pools.
 *
 * [PA] "PagedAttention 的设计" / [LC] StreamingKVCache.append: a new token's K and V
 * for every KV head go to the slot the block table assigns it.  For FP8 pools
 * ([PA] "量化原理") each (token, KV head) row of head_dim values is quantised with
 *     scale = absmax / 448        (IEEE fp32 division, correctly rounded)
 *     code  = E4M3FN(x / scale)   (fp32 division; round to nearest, ties to even,
 *                                  saturating to +-448; absmax 0 -> scale 0, codes 0)
 * and for INT8 pools with
 *     scale = absmax / 127,  code = clamp(rint(x / scale), -127, 127)
 *                                 (fp32 division; nearest integer, ties to even)
 * and the scale is stored beside the codes.  The _CHANNEL formats store
 *     code  = E4M3FN(x / scale[h][d])  or  clamp(rint(x / scale[h][d]), -127, 127)
 *                                 (fp32 division) and leave the scales alone.
 *   k_new, v_new   [num_tokens][num_kv_heads][head_dim] of src_dtype; these and the
 *                  pools 16-byte aligned (PKV_EINVAL otherwise)
 *   kv_dtype       PKV_F32/BF16/F16 require src_dtype == kv_dtype (bytes are copied);
 *                  the 8-bit formats take src_dtype F32, BF16 or F16 (finite values)
 *   k_scale, v_scale   required for the 8-bit formats (written for per-token
 *                  formats, read for _CHANNEL ones), ignored otherwise
 *   slot_mapping   int64 [num_tokens]; a slot < 0 or >= num_blocks*16 skips the token
 * num_tokens * num_kv_heads must stay <= 2^28 (PKV_EINVAL otherwise).
 * Two tokens with the same slot race (one of them wins).
 */
int paged_kv_write(const void* k_new, const void* v_new, int src_dtype,
                   void* k_pool, void* v_pool, float* k_scale, float* v_scale, int kv_dtype,
                   const int64_t* slot_mapping, int num_tokens, int num_blocks,
                   int num_kv_heads, int head_dim, int block_size, void* stream);

/*
 * paged_kv_append -- the decode step's cache write in one call: for every
 * sequence s, the new token (k_new[s], v_new[s]) goes to logical position
 * context_lens[s] - 1 through block_tables[s] ([PA] "PagedAttention 的设计": the
 * token lands in block table[p / 16] at offset p % 16).  Same stores, FP8
 * quantisation, dtype and alignment rules as paged_kv_write with the slots that
 * paged_decode_slots computes; a sequence whose slot would be -1 there (length
 * outside [1, 16 * stride], table entry outside [0, num_blocks)) is skipped.
 *   k_new, v_new   [num_seqs][num_kv_heads][head_dim] of src_dtype
 *   block_tables   int32 [num_seqs][block_table_stride]; context_lens int32 [num_seqs]
 * num_seqs * num_kv_heads must stay <= 2^26 (PKV_EINVAL otherwise).
 */
int paged_kv_append(const void* k_new, const void* v_new, int src_dtype,
                    void* k_pool, void* v_pool, float* k_scale, float* v_scale, int kv_dtype,
                    const int32_t* block_tables, int block_table_stride, const int32_t* context_lens,
                    int num_seqs, int num_blocks, int num_kv_heads, int head_dim, int block_size,
                    void* stream);

/*
 * paged_decode_attn_workspace_size -- bytes of workspace paged_decode_attn needs.
 * Pass the same num_seqs, num_q_heads, head_dim, max_context_len, num_sinks,
 * window and (attn_mass != NULL) as the attention call.  Returns 0 for
 * arguments the attention call would reject.
 */
size_t paged_decode_attn_workspace_size(int num_seqs, int num_q_heads, int head_dim,
                                        int max_context_len, int num_sinks, int window,
                                        int want_mass);

/*
 * paged_decode_attn -- single-token GQA decode attention over the paged pools.
 *
 * For sequence s of length L = context_lens[s] and query head h (KV head
 * h / G, G = num_q_heads / num_kv_heads, [LC] MHA/GQA/MQA table):
 *     z_p   = scale * dot(q[s][h], K[p])          for kept positions p
 *     out   = sum_p softmax(z)_p * V[p]
 * K[p], V[p] are read block by block through block_tables ([PA] "三大运行时组件":
 * decode loads KV per block).  Kept positions ([LC] StreamingKVCache, [SO] 4.1):
 *     window <= 0 : all p < L
 *     window  > 0 : p < num_sinks  or  p >= L - window
 * Blocks holding no kept position are not read, so their table entries may be
 * anything (e.g. -1).
 *
 *   out            [num_seqs][num_q_heads][head_dim] of out_dtype (F32/BF16/F16)
 *   q              [num_seqs][num_q_heads][head_dim] of q_dtype (F32/BF16/F16)
 *   kv_dtype       F32, BF16, F16, or an 8-bit format (then k_scale/v_scale are required;
 *                  _CHANNEL scales are folded into q and the output, not applied per key)
 *   block_tables   int32 [num_seqs][block_table_stride], stride >= ceil(max_context_len/16)
 *   context_lens   int32 [num_seqs], 1 <= L <= max_context_len (host value)
 *   num_q_heads / num_kv_heads in 1..16; head_dim 64 or 128; block_size 16
 *   attn_mass      NULL, or float [num_seqs][attn_mass_stride] (stride >= max_context_len):
 *                  for every kept position, += the H2O mass of this step
 *                  ([LC] H2OEviction.update_scores): the attention probability
 *                  averaged over all num_q_heads heads.  Other entries are untouched.
 *   workspace      >= paged_decode_attn_workspace_size(...) bytes, 256-byte aligned; any
 *                  contents (never zeroed by the caller); calls sharing one workspace
 *                  must not overlap in time
 * num_seqs * (blocks one sequence of max_context_len attends) must stay <= 2^30
 * (PKV_EUNSUPPORTED otherwise).
 * Out-of-range device values never make the kernels touch memory outside the
 * arrays above.  A sequence whose length is outside
 * [1, min(max_context_len, 16*block_table_stride)] gets NaN in every output
 * element and its attn_mass row is left alone; a sequence that needs a table
 * entry outside [0, num_blocks) gets NaN outputs and NaN added to its kept
 * attn_mass entries.
 */
int paged_decode_attn(void* out, int out_dtype,
                      const void* q, int q_dtype,
                      const void* k_pool, const void* v_pool,
                      const float* k_scale, const float* v_scale, int kv_dtype,
                      const int32_t* block_tables, int block_table_stride,
                      const int32_t* context_lens, int max_context_len,
                      int num_seqs, int num_blocks, int num_q_heads, int num_kv_heads,
                      int head_dim, int block_size, float scale,
                      int num_sinks, int window,
                      float* attn_mass, int attn_mass_stride,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_decode_attn_noalloc -- paged_decode_attn without a workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, serving loops that must not call hipMalloc, harnesses that forbid
 * it.  The call allocates nothing; its workspace is a fixed array of 64 MiB
 * in device memory that the library holds on every GPU it runs on until the
 * process ends (its address is looked up once per device, at the first call
 * with that device current).
 *   Arguments, results and error behaviour: those of paged_decode_attn, minus
 *   workspace and workspace_bytes.  A call whose paged_decode_attn workspace
 *   (paged_decode_attn_workspace_size with the same arguments) exceeds 64 MiB
 *   returns PKV_EWORKSPACE before anything is enqueued; e.g. without
 *   attn_mass 64 sequences x 32 query heads x head_dim 128 fit up to
 *   max_context_len 15872, and one sequence of 32 heads up to 10^6 tokens.
 *   All calls on one GPU share that GPU's array: two calls that overlap in
 *   time on one GPU (other streams, other host threads) race and give
 *   undefined results; calls ordered on one stream are safe.  Nothing in the
 *   array needs to start at zero, so what an earlier call left there is never
 *   read.
 */
int paged_decode_attn_noalloc(void* out, int out_dtype,
                              const void* q, int q_dtype,
                              const void* k_pool, const void* v_pool,
                              const float* k_scale, const float* v_scale, int kv_dtype,
                              const int32_t* block_tables, int block_table_stride,
                              const int32_t* context_lens, int max_context_len,
                              int num_seqs, int num_blocks, int num_q_heads, int num_kv_heads,
                              int head_dim, int block_size, float scale,
                              int num_sinks, int window,
                              float* attn_mass, int attn_mass_stride, void* stream);

/*
 * paged_decode_append_attn -- one decode step of one layer: paged_kv_append of
 * the new token of every sequence, then paged_decode_attn over the cache that
 * now holds it ([LC] StreamingKVCache: append, then attend; [PA]
 * "PagedAttention 的设计": the token lands in block table[p / 16] at offset
 * p % 16, p = context_lens[s] - 1).  The pools and the outputs end up exactly
 * as after those two calls with the same arguments, and every argument follows
 * their rules (k_new, v_new [num_seqs][num_kv_heads][head_dim] of src_dtype,
 * 16-byte aligned; the workspace is paged_decode_attn's).
 *   F32/BF16/F16 pools, and 8-bit pools whose src_dtype equals q_dtype (for
 *     INT8 pools a 16-bit q_dtype): one attention launch.  The wave that attends a sequence's last block takes
 *     the new K/V row from k_new/v_new (quantised there for 8-bit pools, with
 *     the write's arithmetic) into that block's operands and stores it into
 *     the pool slot after its last segment, so attention does not wait for
 *     the store.  A sequence whose last table entry lies outside
 *     [0, num_blocks) gets NaN outputs and no store.
 *   INT8 pools with f32 queries, and 8-bit pools with another src_dtype: the
 *     append kernel (which quantises the row) and then the attention kernel,
 *     on the stream.
 * Validation of every argument happens before anything is enqueued.
 */
int paged_decode_append_attn(void* out, int out_dtype,
                             const void* q, int q_dtype,
                             const void* k_new, const void* v_new, int src_dtype,
                             void* k_pool, void* v_pool, float* k_scale, float* v_scale, int kv_dtype,
                             const int32_t* block_tables, int block_table_stride,
                             const int32_t* context_lens, int max_context_len,
                             int num_seqs, int num_blocks, int num_q_heads, int num_kv_heads,
                             int head_dim, int block_size, float scale,
                             int num_sinks, int window,
                             float* attn_mass, int attn_mass_stride,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_decode_attn_compact -- a decode step that also applies an eviction
 * keep-set: attention over the kept tokens only, and the kept tokens moved to
 * fresh blocks in the same pass over the cache ([SO] 4.2 evict_tokens: the
 * cache restricted to the kept indices; [LC] H2OEviction: select the heavy
 * hitters, then decode on the reduced cache).  A separate kv_compact has to
 * read nearly every source tile again (a token's K row is 16-byte pieces
 * spread over its tile and its V elements are interleaved with those of its
 * block's other tokens); this call stores the kept tokens from the operand
 * registers of the attention that reads those tiles anyway.
 *
 * For sequence s with n = keep_count[s] and L = context_lens[s]:
 *   k_new, v_new NULL: the step attends positions keep_idx[s][0..n) of
 *     block_tables[s] (n >= 1; n == 0 gives NaN), and the token at
 *     keep_idx[s][i] is copied (K and V, all KV heads) to logical position i
 *     of dst_tables[s];
 *   k_new, v_new given ([num_seqs][num_kv_heads][head_dim] in q's dtype,
 *     16-byte aligned): position L - 1 holds the step's new token, stored
 *     there (quantised for 8-bit pools) as paged_decode_append_attn stores
 *     it; the step attends the
 *     listed positions (all < L - 1) and the new token, which is also copied,
 *     to logical position n.
 *   out = sum_t softmax_t(scale * q . K[t]) * V[t] over those tokens, t in
 *   keep order; the sequence then holds n (+1) tokens in dst_tables[s], the
 *   same bytes (codes and per-token scales for 8-bit pools) kv_compact and
 *   the append would give, and the host releases its source blocks.
 *   kv_dtype     BF16 or F16 with q_dtype == kv_dtype, or an 8-bit format (per-token
 *                or per-channel FP8 / INT8, k_scale / v_scale as for paged_decode_attn)
 *                with q_dtype BF16 or F16; PKV_EUNSUPPORTED otherwise
 *   keep_idx     int32 [num_seqs][keep_stride], strictly ascending per
 *                sequence; keep_count int32 [num_seqs]
 *   dst_tables   int32 [num_seqs][dst_stride], fresh blocks (no slot written
 *                here may be a source slot of this call); entries outside
 *                [0, num_blocks) skip the tokens that fall in them
 *   attn_mass    NULL, or the H2O score rows after the step, float
 *                [num_seqs][attn_mass_stride] (stride >= max_context_len): entry i
 *                (i < n, and n for the new token) becomes attn_mass_src[s][p] + this
 *                step's mass of p ([LC] H2OEviction.update_scores over the kept
 *                tokens), p the source position of the token moved to i; other
 *                entries are untouched.  attn_mass_src: the score rows before the
 *                step, float [num_seqs][attn_mass_src_stride] (stride >=
 *                max_context_len), a different array (PKV_EINVAL otherwise).
 *   workspace    >= paged_decode_attn_compact_workspace_size(..., attn_mass != NULL)
 *                bytes, 256-byte aligned
 * Other arguments: paged_decode_attn's (no sinks or window).  A
 * sequence whose count is outside [0, min(keep_stride, L - (k_new ? 1 : 0))],
 * or whose kept tokens do not fit dst_tables[s], gets NaN outputs and no
 * copies (the new token is still stored at L - 1).  A keep list that is not
 * ascending gives unspecified outputs and destination contents, written only
 * to blocks listed in dst_tables[s].  Validation of every argument happens
 * before anything is enqueued.
 */
size_t paged_decode_attn_compact_workspace_size(int num_seqs, int num_q_heads, int head_dim,
                                                int max_context_len, int want_mass);
int paged_decode_attn_compact(void* out, int out_dtype,
                              const void* q, int q_dtype,
                              const void* k_new, const void* v_new,
                              void* k_pool, void* v_pool, float* k_scale, float* v_scale, int kv_dtype,
                              const int32_t* block_tables, int block_table_stride,
                              const int32_t* context_lens, int max_context_len,
                              const int32_t* keep_idx, int keep_stride, const int32_t* keep_count,
                              const int32_t* dst_tables, int dst_stride,
                              int num_seqs, int num_blocks, int num_q_heads, int num_kv_heads,
                              int head_dim, int block_size, float scale,
                              const float* attn_mass_src, int attn_mass_src_stride,
                              float* attn_mass, int attn_mass_stride,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_prefill_attn -- causal multi-query attention over the paged cache: the
 * chunked prefill of a long prompt ([SO] 4.5 "Chunked Prefill") or the
 * continuation of a request whose prefix came from the prefix cache ([PA]
 * "共享场景的价值": a hit skips the prefill of the shared part; [SO] 4.5
 * "分页 KV Cache + 前缀缓存").
 *
 * Sequence s owns query rows [query_start[s], query_start[s+1]) of q and out;
 * with n = query_start[s+1] - query_start[s] and L = context_lens[s], these are
 * its last n positions, whose K/V are already in the cache (write them first,
 * e.g. paged_token_slots + paged_kv_write).  Row i (position p = L - n + i) and
 * query head h (KV head h / G) attend to positions 0..p:
 *     out = sum_{t <= p} softmax_t(scale * q . K[t]) * V[t]
 *   q, out         [num_tokens][num_q_heads][head_dim]; q_dtype / out_dtype F32, BF16, F16
 *   query_start    int32 [num_seqs + 1], non-decreasing, query_start[num_seqs] <= num_tokens
 *   context_lens   int32 [num_seqs], n <= L <= max_context_len
 *   max_query_len  >= every n (sizes the grid)
 *   G = num_q_heads / num_kv_heads in {1, 2, 4, 8, 16}; head_dim 64 or 128
 * No sinks/window here and no workspace.  A sequence whose rows fall outside
 * [0, num_tokens) is skipped; one with L < n, L > max_context_len or L >
 * 16 * stride, or that needs a table entry outside [0, num_blocks), gets NaN
 * in its rows.  Rows not owned by any sequence are left untouched.
 * Precision: over BF16/F16 pools the probabilities enter the P.V product as
 * f16 values (relative rounding <= 2^-11) against V in f16 (BF16 V converted
 * exactly over f16's normal range); a workgroup whose inputs leave f16's range
 * (|V| > 65504, a logit far above its chunk's first block pair) computes again
 * with ~16-bit probabilities and bf16 V, so any finite input is covered.  The
 * other pools use ~16-bit probabilities throughout.
 */
int paged_prefill_attn(void* out, int out_dtype, const void* q, int q_dtype,
                       const void* k_pool, const void* v_pool,
                       const float* k_scale, const float* v_scale, int kv_dtype,
                       const int32_t* block_tables, int block_table_stride,
                       const int32_t* context_lens, const int32_t* query_start,
                       int num_tokens, int max_context_len, int max_query_len,
                       int num_seqs, int num_blocks, int num_q_heads, int num_kv_heads,
                       int head_dim, int block_size, float scale, void* stream);

/*
 * kv_swap -- move whole blocks between the pool and a pinned host arena ([PA]
 * "三大运行时组件": the block allocator can swap blocks out to CPU RAM; [SO] 4.5
 * "CPU Offloading": inactive requests' KV waits in CPU memory and comes back
 * when needed).
 *
 * For each pair {block, slot} of block_slot_pairs: to_host = 1 copies pool
 * block `block` (K and V tiles of every KV head, and for the per-token FP8/INT8
 * formats both scale rows) to host slot `slot`; to_host = 0 copies slot `slot` back into pool
 * block `block`.  The host arena mirrors the pool layout:
 *   host_k, host_v             [host_slots][num_kv_heads][tile] (same tile bytes as the pool)
 *   host_k_scale, host_v_scale float [host_slots][num_kv_heads][16] (per-token FP8/INT8 only)
 * and must be pinned, device-accessible memory (hipHostMalloc, or torch
 * pin_memory), which the kernel reads or writes directly.
 *   block_slot_pairs  int32 [num_pairs][2], device memory
 * A pair whose block or slot is out of range is skipped.  Pairs that name the
 * same block or slot twice race.  The copy is ordered on `stream`: host code
 * may touch the arena only after synchronising with it.
 */
int kv_swap(void* k_pool, void* v_pool, float* k_scale, float* v_scale, int kv_dtype,
            void* host_k, void* host_v, float* host_k_scale, float* host_v_scale,
            const int32_t* block_slot_pairs, int num_pairs, int num_blocks, int host_slots,
            int num_kv_heads, int head_dim, int block_size, int to_host, void* stream);

/*
 * kv_block_copy -- whole-block copies, the data half of copy-on-write.
 *
 * [PA] "三大运行时组件" and its copy_on_write snippet: before a sequence writes
 * into a physical block that other sequences still share (refcount > 1), the
 * block is copied to a private one.  Refcounts and table edits are host-side;
 * this call copies K, V and (per-token FP8/INT8) both scale tiles of every KV head.
 *   block_pairs   int32 [num_pairs][2] = {src, dst}; a pair with an index outside
 *                 [0, num_blocks) or src == dst is skipped.  Pairs run concurrently:
 *                 a dst that is also another pair's src or dst races.
 */
int kv_block_copy(void* k_pool, void* v_pool, float* k_scale, float* v_scale, int kv_dtype,
                  const int32_t* block_pairs, int num_pairs, int num_blocks,
                  int num_kv_heads, int head_dim, int block_size, void* stream);

/*
 * h2o_select -- H2O keep-set per sequence ([LC] H2OEviction.select).
 *
 * For L = kv_lens[s]:
 *   L <= budget : keep positions 0..L-1
 *   otherwise   : keep the last `recent` positions plus the (budget - recent)
 *                 highest scores among positions [0, L - recent); equal scores
 *                 go to the lower position, NaN ranks below every number,
 *                 -0.0 equals +0.0.
 * Output in ascending position order.
 *   scores      float [num_seqs][scores_stride], stride >= max_kv_len
 *   kv_lens     int32 [num_seqs], 1 <= L <= max_kv_len
 *   keep_idx    int32 [num_seqs][budget] out, -1 after the kept positions
 *   keep_count  int32 [num_seqs] out (-1 for a length outside [1, max_kv_len])
 *   0 <= recent <= budget, budget >= 1
 */
int h2o_select(const float* scores, int scores_stride, const int32_t* kv_lens,
               int num_seqs, int max_kv_len, int budget, int recent,
               int32_t* keep_idx, int32_t* keep_count, void* stream);

/* Candidate sets of kv_keep_select. */
typedef enum {
  PKV_CAND_REST = 0,  /* positions that are not forced ([LC] H2OEviction.select) */
  PKV_CAND_ALL = 1    /* every position ([PA] 组合 should_cache; [SO] 4.2 evict_tokens) */
} pkv_candidates;

/*
 * kv_keep_select -- keep-set of an eviction rule per sequence.
 *
 * For L = kv_lens[s]:
 *   forced(p) = p < num_sinks  or  p >= L - recent
 *   C         = PKV_CAND_REST: the positions of [0, L) that are not forced
 *               PKV_CAND_ALL : all of [0, L)
 *   heavy set = the `heavy` highest scores[s][p] over p in C (all of C if it is
 *               smaller); equal scores go to the lower position, NaN ranks
 *               below every number, -0.0 equals +0.0
 *   kept      = forced positions united with the heavy set
 * The three rules of the pages are instances: H2OEviction.select
 * ([LC]; = h2o_select) is (0, recent, budget - recent, REST); should_cache ([PA]
 * 组合: sinks 4, window 256, 512 in total) is (4, 256, 252, ALL), whose heavy set
 * may overlap the forced positions; evict_tokens ([SO] 4.2) is (0, 0, budget, ALL).
 *   scores      float [num_seqs][scores_stride], stride >= max_kv_len
 *   kv_lens     int32 [num_seqs], 1 <= L <= max_kv_len
 *   keep_idx    int32 [num_seqs][keep_stride] out: kept positions ascending, then -1;
 *               keep_stride >= min(num_sinks + recent + heavy, max_kv_len)
 *   keep_count  int32 [num_seqs] out (-1 for a length outside [1, max_kv_len])
 */
int kv_keep_select(const float* scores, int scores_stride, const int32_t* kv_lens,
                   int num_seqs, int max_kv_len, int num_sinks, int recent, int heavy,
                   int candidates, int32_t* keep_idx, int keep_stride, int32_t* keep_count,
                   void* stream);

/*
 * kv_compact -- apply a keep-set: move each sequence's kept tokens to a dense
 * prefix of fresh blocks ([SO] 4.2 evict_tokens returns the cache restricted to
 * the kept indices; [LC] StreamingKVCache drops the middle of the cache).
 *
 * For sequence s and i < n = keep_count[s]: the token at logical position
 * keep_idx[s][i] of src_tables[s] is copied -- K, V and, for per-token FP8/INT8, both scales,
 * all KV heads -- to logical position i of dst_tables[s].  The sequence then
 * holds n tokens in ceil(n / 16) destination blocks; the host releases the
 * source blocks (BlockManager.compact).
 *   src_tables, dst_tables  int32 [num_seqs][src_stride], [num_seqs][dst_stride]
 *   keep_idx     int32 [num_seqs][keep_stride]; keep_count int32 [num_seqs];
 *                ceil(keep_stride / 16) * num_kv_heads <= 2^24 (PKV_EINVAL otherwise)
 * Destination slots must not be source slots of a token copied in the same call
 * (use fresh blocks); otherwise the result is undefined.  Slots of the last
 * destination block beyond n are left as they were.  A sequence whose count is
 * outside [0, min(keep_stride, 16 * dst_stride)] is skipped; a kept position
 * outside [0, 16 * src_stride) or whose source table entry is outside
 * [0, num_blocks) writes NaN bytes (0xFF; NaN scales) for that token; a
 * destination entry outside [0, num_blocks) skips that block.
 */
int kv_compact(void* k_pool, void* v_pool, float* k_scale, float* v_scale, int kv_dtype,
               const int32_t* src_tables, int src_stride, const int32_t* dst_tables, int dst_stride,
               const int32_t* keep_idx, int keep_stride, const int32_t* keep_count,
               int num_seqs, int num_blocks, int num_kv_heads, int head_dim, int block_size,
               void* stream);

/* ---- measurement helpers (not part of the decode path) ------------------ */

/*
 * Kernel timing for benchmarks.  Between pkv_timing_begin(capacity) and
 * pkv_timing_end(), each paged_decode_attn call has its main attention
 * kernel's dispatch stamp a HIP event pair with that kernel's own start and
 * end (no separate event packets on the stream), up to `capacity` calls.
 * pkv_timing_end waits for the last event, writes the elapsed milliseconds of
 * each recorded launch to ms_out (host, capacity floats), returns the count
 * (or -1 on error).  Not thread-safe: one timing session per process.
 */
int pkv_timing_begin(int capacity);
int pkv_timing_end(float* ms_out, int capacity);

/*
 * Streaming probes for roofline denominators: read `bytes` (multiple of 16)
 * from src and fold them into sink[0..1023] (float, written), or copy bytes
 * from src to dst.  Grid-stride kernels with 16-byte accesses.
 */
int pkv_probe_read(const void* src, size_t bytes, float* sink, void* stream);
int pkv_probe_copy(void* dst, const void* src, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
