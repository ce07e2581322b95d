// C ABI of the paged KV-cache library (declared in include/pagedkv.h).
// Validates every scalar argument and pointer on the host before any HIP call,
// then hands off to the launchers in launch.hpp.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <string>
#include <utility>
#include <vector>

#include "pagedkv.h"
#include "geometry.hpp"
#include "launch.hpp"

namespace {

thread_local std::string g_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return status;
}

int ok() {
  g_error.clear();
  return PKV_OK;
}

int device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(PKV_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool valid_kv_dtype(int d) { return d >= PKV_F32 && d <= PKV_INT8_CHANNEL; }
// Per-token scales stored per block.
bool quantised_kv(int d) { return d == PKV_FP8_E4M3 || d == PKV_INT8; }
// Static per-(KV head, channel) scales.
bool channel_kv(int d) { return d == PKV_FP8_E4M3_CHANNEL || d == PKV_INT8_CHANNEL; }
// 8-bit codes of either kind: any float source is quantised.
bool code8_kv(int d) { return quantised_kv(d) || channel_kv(d); }
bool valid_float_dtype(int d) { return d >= PKV_F32 && d <= PKV_F16; }

struct Timing {
  bool active = false;
  int used = 0;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev;
};
Timing g_timing;

// Shared checks of the attention geometry; returns PKV_OK or a status with g_error set.
int check_attn_shape(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int max_context_len,
                     int num_sinks) {
  if (num_seqs < 0 || num_seqs > 65535) return fail(PKV_EINVAL, "num_seqs %d outside [0, 65535]", num_seqs);
  if (num_q_heads < 1 || num_kv_heads < 1) return fail(PKV_EINVAL, "head counts must be >= 1");
  if (num_q_heads % num_kv_heads != 0)
    return fail(PKV_EINVAL, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads, num_kv_heads);
  if (num_q_heads / num_kv_heads > 16)
    return fail(PKV_EUNSUPPORTED, "query heads per KV head %d > 16", num_q_heads / num_kv_heads);
  if (num_kv_heads > 65535) return fail(PKV_EINVAL, "num_kv_heads %d too large", num_kv_heads);
  if (head_dim != 64 && head_dim != 128) return fail(PKV_EUNSUPPORTED, "head_dim %d (built: 64, 128)", head_dim);
  if (max_context_len < 1) return fail(PKV_EINVAL, "max_context_len %d < 1", max_context_len);
  if (max_context_len > (1 << 30)) return fail(PKV_EINVAL, "max_context_len %d too large", max_context_len);
  if (num_sinks < 0 || num_sinks > (1 << 30)) return fail(PKV_EINVAL, "num_sinks %d outside [0, 2^30]", num_sinks);
  return PKV_OK;
}

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_error.c_str(); }

const char* pkv_version(void) { return "pagedkv 0.1.0 gfx950"; }

int paged_decode_slots(const int32_t* block_tables, int block_table_stride, const int32_t* context_lens,
                       int num_seqs, int num_blocks, int block_size, int64_t* slot_mapping, void* stream) {
  if (block_size != pkv::kBlockSize) return fail(PKV_EUNSUPPORTED, "block_size %d (built: 16)", block_size);
  if (num_seqs < 0) return fail(PKV_EINVAL, "num_seqs %d < 0", num_seqs);
  if (num_seqs == 0) return ok();
  if (!block_tables || !context_lens || !slot_mapping) return fail(PKV_EINVAL, "NULL array argument");
  if (block_table_stride < 1) return fail(PKV_EINVAL, "block_table_stride %d < 1", block_table_stride);
  if (block_table_stride > (1 << 26)) return fail(PKV_EINVAL, "block_table_stride %d too large", block_table_stride);
  if (num_blocks < 1) return fail(PKV_EINVAL, "num_blocks %d < 1", num_blocks);
  return device_status(pkv::launch_decode_slots(block_tables, block_table_stride, context_lens, num_seqs, num_blocks,
                                                slot_mapping, (hipStream_t)stream),
                       "paged_decode_slots");
}

int paged_token_slots(const int32_t* block_tables, int block_table_stride, int num_seqs, const int32_t* seq_ids,
                      const int32_t* positions, int num_tokens, int num_blocks, int block_size, int64_t* slot_mapping,
                      void* stream) {
  if (block_size != pkv::kBlockSize) return fail(PKV_EUNSUPPORTED, "block_size %d (built: 16)", block_size);
  if (num_tokens < 0) return fail(PKV_EINVAL, "num_tokens %d < 0", num_tokens);
  if (num_seqs < 0) return fail(PKV_EINVAL, "num_seqs %d < 0", num_seqs);
  if (num_tokens == 0) return ok();
  if (!block_tables || !seq_ids || !positions || !slot_mapping) return fail(PKV_EINVAL, "NULL array argument");
  if (block_table_stride < 1 || block_table_stride > (1 << 26))
    return fail(PKV_EINVAL, "block_table_stride %d outside [1, 2^26]", block_table_stride);
  if (num_blocks < 1) return fail(PKV_EINVAL, "num_blocks %d < 1", num_blocks);
  return device_status(pkv::launch_token_slots(block_tables, block_table_stride, num_seqs, seq_ids, positions,
                                               num_tokens, num_blocks, slot_mapping, (hipStream_t)stream),
                       "paged_token_slots");
}

int paged_kv_write(const void* k_new, const void* v_new, int src_dtype, void* k_pool, void* v_pool, float* k_scale,
                   float* v_scale, int kv_dtype, const int64_t* slot_mapping, int num_tokens, int num_blocks,
                   int num_kv_heads, int head_dim, int block_size, void* stream) {
  if (block_size != pkv::kBlockSize) return fail(PKV_EUNSUPPORTED, "block_size %d (built: 16)", block_size);
  if (head_dim != 64 && head_dim != 128) return fail(PKV_EUNSUPPORTED, "head_dim %d (built: 64, 128)", head_dim);
  if (!valid_kv_dtype(kv_dtype)) return fail(PKV_EINVAL, "kv_dtype %d", kv_dtype);
  if (!valid_float_dtype(src_dtype)) return fail(PKV_EINVAL, "src_dtype %d", src_dtype);
  if (!code8_kv(kv_dtype) && src_dtype != kv_dtype)
    return fail(PKV_EUNSUPPORTED, "a non-quantised pool takes source of its own dtype (src %d, kv %d)", src_dtype, kv_dtype);
  if (num_tokens < 0) return fail(PKV_EINVAL, "num_tokens %d < 0", num_tokens);
  if (num_kv_heads < 1 || num_kv_heads > 65535) return fail(PKV_EINVAL, "num_kv_heads %d outside [1, 65535]", num_kv_heads);
  if (num_blocks < 1) return fail(PKV_EINVAL, "num_blocks %d < 1", num_blocks);
  if ((long long)num_tokens * num_kv_heads > (1LL << 28))   // 16 threads per row in one grid dimension
    return fail(PKV_EINVAL, "num_tokens * num_kv_heads %lld > 2^28", (long long)num_tokens * num_kv_heads);
  if (num_tokens == 0) return ok();
  if (!k_new || !v_new || !k_pool || !v_pool || !slot_mapping) return fail(PKV_EINVAL, "NULL array argument");
  if ((uintptr_t)k_new % 16 || (uintptr_t)v_new % 16 || (uintptr_t)k_pool % 16 || (uintptr_t)v_pool % 16)
    return fail(PKV_EINVAL, "k_new, v_new and the pools must be 16-byte aligned");
  if (code8_kv(kv_dtype) && (!k_scale || !v_scale)) return fail(PKV_EINVAL, "FP8/INT8 pools need k_scale and v_scale");
  return device_status(pkv::launch_kv_write(k_new, v_new, src_dtype, k_pool, v_pool, k_scale, v_scale, kv_dtype,
                                            slot_mapping, num_tokens, num_blocks, num_kv_heads, head_dim,
                                            (hipStream_t)stream),
                       "paged_kv_write");
}

int paged_kv_append(const void* k_new, const void* v_new, int src_dtype, void* k_pool, void* v_pool, float* k_scale,
                    float* v_scale, int kv_dtype, const int32_t* block_tables, int block_table_stride,
                    const int32_t* context_lens, int num_seqs, int num_blocks, int num_kv_heads, int head_dim,
                    int block_size, void* stream) {
  if (block_size != pkv::kBlockSize) return fail(PKV_EUNSUPPORTED, "block_size %d (built: 16)", block_size);
  if (head_dim != 64 && head_dim != 128) return fail(PKV_EUNSUPPORTED, "head_dim %d (built: 64, 128)", head_dim);
  if (!valid_kv_dtype(kv_dtype)) return fail(PKV_EINVAL, "kv_dtype %d", kv_dtype);
  if (!valid_float_dtype(src_dtype)) return fail(PKV_EINVAL, "src_dtype %d", src_dtype);
  if (!code8_kv(kv_dtype) && src_dtype != kv_dtype)
    return fail(PKV_EUNSUPPORTED, "a non-quantised pool takes source of its own dtype (src %d, kv %d)", src_dtype, kv_dtype);
  if (num_seqs < 0) return fail(PKV_EINVAL, "num_seqs %d < 0", num_seqs);
  if (num_kv_heads < 1 || num_kv_heads > 65535) return fail(PKV_EINVAL, "num_kv_heads %d outside [1, 65535]", num_kv_heads);
  if (num_blocks < 1) return fail(PKV_EINVAL, "num_blocks %d < 1", num_blocks);
  if (block_table_stride < 1 || block_table_stride > (1 << 26))
    return fail(PKV_EINVAL, "block_table_stride %d outside [1, 2^26]", block_table_stride);
  if ((long long)num_seqs * num_kv_heads > (1LL << 26))   // 64 threads per row in one grid dimension
    return fail(PKV_EINVAL, "num_seqs * num_kv_heads %lld > 2^26", (long long)num_seqs * num_kv_heads);
  if (num_seqs == 0) return ok();
  if (!k_new || !v_new || !k_pool || !v_pool || !block_tables || !context_lens)
    return fail(PKV_EINVAL, "NULL array argument");
  if ((uintptr_t)k_new % 16 || (uintptr_t)v_new % 16 || (uintptr_t)k_pool % 16 || (uintptr_t)v_pool % 16)
    return fail(PKV_EINVAL, "k_new, v_new and the pools must be 16-byte aligned");
  if (code8_kv(kv_dtype) && (!k_scale || !v_scale)) return fail(PKV_EINVAL, "FP8/INT8 pools need k_scale and v_scale");
  return device_status(pkv::launch_kv_append(k_new, v_new, src_dtype, k_pool, v_pool, k_scale, v_scale, kv_dtype,
                                             block_tables, block_table_stride, context_lens, num_seqs, num_blocks,
                                             num_kv_heads, head_dim, (hipStream_t)stream),
                       "paged_kv_append");
}

size_t paged_decode_attn_workspace_size(int num_seqs, int num_q_heads, int head_dim, int max_context_len,
                                        int num_sinks, int window, int want_mass) {
  if (num_seqs < 0 || num_q_heads < 1 || (head_dim != 64 && head_dim != 128) || max_context_len < 1 ||
      max_context_len > (1 << 30) || num_sinks < 0 || num_sinks > (1 << 30) || window > (1 << 30))
    return 0;
  return pkv::attn_workspace_layout(num_seqs, num_q_heads, head_dim, max_context_len, num_sinks, window,
                                    want_mass != 0)
      .total;
}

// Workspace of paged_decode_attn_compact: the attention call's (no sinks or
// window), then the keep map at the next 256-byte boundary.
static size_t compact_map_offset(int num_seqs, int num_q_heads, int head_dim, int max_context_len, bool want_mass) {
  return (pkv::attn_workspace_layout(num_seqs, num_q_heads, head_dim, max_context_len, 0, 0, want_mass).total +
          255) & ~(size_t)255;
}

size_t paged_decode_attn_compact_workspace_size(int num_seqs, int num_q_heads, int head_dim, int max_context_len,
                                                int want_mass) {
  if (num_seqs < 0 || num_q_heads < 1 || (head_dim != 64 && head_dim != 128) || max_context_len < 1 ||
      max_context_len > (1 << 30))
    return 0;
  const size_t map_stride = ((size_t)max_context_len + 15) / 16;
  return compact_map_offset(num_seqs, num_q_heads, head_dim, max_context_len, want_mass != 0) +
         (size_t)num_seqs * map_stride * sizeof(pkv::KeepMapEntry);
}

// Points a call's workspace views into `workspace`, laid out as `lay`.
static void bind_workspace(pkv::AttnArgs& a, const pkv::WorkspaceLayout& lay, void* workspace) {
  char* ws = reinterpret_cast<char*>(workspace);
  a.part_acc = reinterpret_cast<float*>(ws + lay.acc_off);
  a.part_ml = reinterpret_cast<float*>(ws + lay.ml_off);
  a.hdr = reinterpret_cast<pkv::StreamHdr*>(ws + lay.hdr_off);
  a.seq_prefix = reinterpret_cast<int*>(ws + lay.prefix_off);
  a.stash = a.attn_mass ? reinterpret_cast<float*>(ws + lay.stash_off) : nullptr;
  a.fin_ml = a.attn_mass ? reinterpret_cast<float*>(ws + lay.fin_off) : nullptr;
}

// Validates the arguments of a decode-attention call and fills `a`; no HIP
// call.  num_seqs == 0 leaves a.num_seqs = 0 (nothing to launch).
// static_workspace: the workspace is the library's fixed one of workspace_bytes
// (bound later by the caller); only its size is checked here.
static int prepare_decode_attn(pkv::AttnArgs& a, void* out, int out_dtype, const void* q, int q_dtype,
                               const void* k_pool, const void* v_pool, const float* k_scale, const float* v_scale,
                               int kv_dtype, const int32_t* block_tables, int block_table_stride,
                               const int32_t* context_lens, int max_context_len, int num_seqs, int num_blocks,
                               int num_q_heads, int num_kv_heads, int head_dim, int block_size, float scale,
                               int num_sinks, int window, float* attn_mass, int attn_mass_stride, void* workspace,
                               size_t workspace_bytes, bool static_workspace = false,
                               pkv::WorkspaceLayout* layout = nullptr) {
  a = pkv::AttnArgs{};
  if (block_size != pkv::kBlockSize) return fail(PKV_EUNSUPPORTED, "block_size %d (built: 16)", block_size);
  int st = check_attn_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, num_sinks);
  if (st != PKV_OK) return st;
  if (!valid_kv_dtype(kv_dtype)) return fail(PKV_EINVAL, "kv_dtype %d", kv_dtype);
  if (!valid_float_dtype(q_dtype)) return fail(PKV_EINVAL, "q_dtype %d", q_dtype);
  if (!valid_float_dtype(out_dtype)) return fail(PKV_EINVAL, "out_dtype %d", out_dtype);
  if (!isfinite(scale)) return fail(PKV_EINVAL, "scale is not finite");
  if (window > (1 << 30)) return fail(PKV_EINVAL, "window %d too large", window);
  if (block_table_stride > (1 << 26)) return fail(PKV_EINVAL, "block_table_stride %d too large", block_table_stride);
  if (num_blocks < 1) return fail(PKV_EINVAL, "num_blocks %d < 1", num_blocks);
  if (block_table_stride < (max_context_len + 15) / 16)
    return fail(PKV_EINVAL, "block_table_stride %d < ceil(max_context_len / 16) = %d", block_table_stride,
                (max_context_len + 15) / 16);
  if ((long long)num_seqs * pkv::max_virtual_blocks(max_context_len, num_sinks, window) > (1LL << 30))
    return fail(PKV_EUNSUPPORTED, "num_seqs %d x attended blocks of max_context_len %d exceeds 2^30", num_seqs,
                max_context_len);
  if (attn_mass != nullptr && attn_mass_stride < max_context_len)
    return fail(PKV_EINVAL, "attn_mass_stride %d < max_context_len %d", attn_mass_stride, max_context_len);
  if (num_seqs == 0) return ok();
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens)
    return fail(PKV_EINVAL, "NULL array argument");
  if (code8_kv(kv_dtype) && (!k_scale || !v_scale)) return fail(PKV_EINVAL, "FP8/INT8 pools need k_scale and v_scale");
  const pkv::WorkspaceLayout lay = pkv::attn_workspace_layout(num_seqs, num_q_heads, head_dim, max_context_len,
                                                              num_sinks, window, attn_mass != nullptr);
  if (lay.p_max > 65535)
    return fail(PKV_EUNSUPPORTED, "max_context_len %d needs %d partial slots (> 65535)", max_context_len, lay.p_max);
  if (static_workspace) {
    if (lay.total > workspace_bytes)
      return fail(PKV_EWORKSPACE, "this call needs %zu bytes of workspace; the fixed workspace of "
                  "paged_decode_attn_noalloc holds %zu (use paged_decode_attn with a caller workspace)",
                  lay.total, workspace_bytes);
  } else {
    if (workspace_bytes < lay.total)
      return fail(PKV_EWORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, lay.total);
    if (lay.total > 0 && !workspace) return fail(PKV_EINVAL, "NULL workspace");
    if (((uintptr_t)workspace & 255u) != 0) return fail(PKV_EINVAL, "workspace is not 256-byte aligned");
  }
  if ((uintptr_t)q % 16 || (uintptr_t)k_pool % 16 || (uintptr_t)v_pool % 16 ||
      (k_scale && (uintptr_t)k_scale % 16) || (v_scale && (uintptr_t)v_scale % 16))
    return fail(PKV_EINVAL, "q, pools and scales must be 16-byte aligned");

  a.out = out;
  a.out_dtype = out_dtype;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_tables = block_tables;
  a.table_stride = block_table_stride;
  a.context_lens = context_lens;
  a.max_context_len = max_context_len;
  a.num_seqs = num_seqs;
  a.num_blocks = num_blocks;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.num_sinks = num_sinks;
  a.window = window;
  a.attn_mass = attn_mass;
  a.mass_stride = attn_mass_stride;
  a.p_max = lay.p_max;
  a.nv_pad = lay.nv_pad;
  if (layout) *layout = lay;
  if (!static_workspace) bind_workspace(a, lay, workspace);
  return ok();
}

static int launch_prepared_attn(const pkv::AttnArgs& a, int kv_dtype, int q_dtype, int head_dim, void* stream,
                                const char* what) {
  if (a.num_seqs == 0) return ok();
  hipEvent_t eb = nullptr, ee = nullptr;
  if (g_timing.active && g_timing.used < (int)g_timing.ev.size()) {
    eb = g_timing.ev[g_timing.used].first;
    ee = g_timing.ev[g_timing.used].second;
    ++g_timing.used;
  }
  return device_status(pkv::launch_decode_attn(a, kv_dtype, q_dtype, head_dim, (hipStream_t)stream, eb, ee), what);
}

int paged_decode_attn(void* out, int out_dtype, const void* q, int q_dtype, const void* k_pool, const void* v_pool,
                      const float* k_scale, const float* v_scale, int kv_dtype, const int32_t* block_tables,
                      int block_table_stride, const int32_t* context_lens, int max_context_len, int num_seqs,
                      int num_blocks, int num_q_heads, int num_kv_heads, int head_dim, int block_size, float scale,
                      int num_sinks, int window, float* attn_mass, int attn_mass_stride, void* workspace,
                      size_t workspace_bytes, void* stream) {
  pkv::AttnArgs a;
  const int st = prepare_decode_attn(a, out, out_dtype, q, q_dtype, k_pool, v_pool, k_scale, v_scale, kv_dtype,
                                     block_tables, block_table_stride, context_lens, max_context_len, num_seqs,
                                     num_blocks, num_q_heads, num_kv_heads, head_dim, block_size, scale, num_sinks,
                                     window, attn_mass, attn_mass_stride, workspace, workspace_bytes);
  if (st != PKV_OK) return st;
  return launch_prepared_attn(a, kv_dtype, q_dtype, head_dim, stream, "paged_decode_attn");
}

int paged_decode_attn_noalloc(void* out, int out_dtype, const void* q, int q_dtype, const void* k_pool,
                              const void* v_pool, const float* k_scale, const float* v_scale, int kv_dtype,
                              const int32_t* block_tables, int block_table_stride, const int32_t* context_lens,
                              int max_context_len, int num_seqs, int num_blocks, int num_q_heads, int num_kv_heads,
                              int head_dim, int block_size, float scale, int num_sinks, int window, float* attn_mass,
                              int attn_mass_stride, void* stream) {
  // Every argument is checked against a workspace of the fixed size first
  // (the size limit included), before any HIP call.
  pkv::AttnArgs a;
  pkv::WorkspaceLayout lay{};
  const int st = prepare_decode_attn(a, out, out_dtype, q, q_dtype, k_pool, v_pool, k_scale, v_scale, kv_dtype,
                                     block_tables, block_table_stride, context_lens, max_context_len, num_seqs,
                                     num_blocks, num_q_heads, num_kv_heads, head_dim, block_size, scale, num_sinks,
                                     window, attn_mass, attn_mass_stride, nullptr, pkv::kStaticScratchBytes,
                                     /*static_workspace=*/true, &lay);
  if (st != PKV_OK) return st;
  if (a.num_seqs == 0) return ok();
  void* ws = nullptr;
  const int dst = device_status(pkv::static_scratch(&ws), "paged_decode_attn_noalloc: scratch lookup");
  if (dst != PKV_OK) return dst;
  bind_workspace(a, lay, ws);
  return launch_prepared_attn(a, kv_dtype, q_dtype, head_dim, stream, "paged_decode_attn_noalloc");
}

int paged_decode_append_attn(void* out, int out_dtype, const void* q, int q_dtype, const void* k_new,
                             const void* v_new, int src_dtype, void* k_pool, void* v_pool, float* k_scale,
                             float* v_scale, int kv_dtype, const int32_t* block_tables, int block_table_stride,
                             const int32_t* context_lens, int max_context_len, int num_seqs, int num_blocks,
                             int num_q_heads, int num_kv_heads, int head_dim, int block_size, float scale,
                             int num_sinks, int window, float* attn_mass, int attn_mass_stride, void* workspace,
                             size_t workspace_bytes, void* stream) {
  pkv::AttnArgs a;
  int st = prepare_decode_attn(a, out, out_dtype, q, q_dtype, k_pool, v_pool, k_scale, v_scale, kv_dtype,
                               block_tables, block_table_stride, context_lens, max_context_len, num_seqs, num_blocks,
                               num_q_heads, num_kv_heads, head_dim, block_size, scale, num_sinks, window, attn_mass,
                               attn_mass_stride, workspace, workspace_bytes);
  if (st != PKV_OK) return st;
  if (!valid_float_dtype(src_dtype)) return fail(PKV_EINVAL, "src_dtype %d", src_dtype);
  if (!code8_kv(kv_dtype) && src_dtype != kv_dtype)
    return fail(PKV_EUNSUPPORTED, "a non-quantised pool takes source of its own dtype (src %d, kv %d)", src_dtype, kv_dtype);
  if ((long long)num_seqs * num_kv_heads > (1LL << 26))   // the append kernel's limit (INT8 pools)
    return fail(PKV_EINVAL, "num_seqs * num_kv_heads %lld > 2^26", (long long)num_seqs * num_kv_heads);
  if (num_seqs == 0) return ok();
  if (!k_new || !v_new) return fail(PKV_EINVAL, "NULL array argument");
  if ((uintptr_t)k_new % 16 || (uintptr_t)v_new % 16)
    return fail(PKV_EINVAL, "k_new and v_new must be 16-byte aligned");
  if (!pkv::fused_append_built(kv_dtype, q_dtype) || (code8_kv(kv_dtype) && src_dtype != q_dtype)) {
    // INT8 pools with f32 queries, and 8-bit pools fed from a dtype other than
    // q's: the append kernel quantises the token first; the attention kernel
    // then reads it from the pool.
    st = device_status(pkv::launch_kv_append(k_new, v_new, src_dtype, k_pool, v_pool, k_scale, v_scale, kv_dtype,
                                             block_tables, block_table_stride, context_lens, num_seqs, num_blocks,
                                             num_kv_heads, head_dim, (hipStream_t)stream),
                       "paged_decode_append_attn");
    if (st != PKV_OK) return st;
  } else {
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_store = k_pool;
    a.v_store = v_pool;
    a.k_scale_store = k_scale;
    a.v_scale_store = v_scale;
  }
  return launch_prepared_attn(a, kv_dtype, q_dtype, head_dim, stream, "paged_decode_append_attn");
}

int paged_decode_attn_compact(void* out, int out_dtype, const void* q, int q_dtype, const void* k_new,
                              const void* v_new, void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                              int kv_dtype,
                              const int32_t* block_tables, int block_table_stride, const int32_t* context_lens,
                              int max_context_len, const int32_t* keep_idx, int keep_stride,
                              const int32_t* keep_count, const int32_t* dst_tables, int dst_stride, int num_seqs,
                              int num_blocks, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                              float scale, const float* attn_mass_src, int attn_mass_src_stride, float* attn_mass,
                              int attn_mass_stride, void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_kv_dtype(kv_dtype) || kv_dtype == PKV_F32)
    return fail(PKV_EUNSUPPORTED, "kv_dtype %d (compaction is built for 16-bit and 8-bit pools)", kv_dtype);
  if (code8_kv(kv_dtype) ? (q_dtype != PKV_BF16 && q_dtype != PKV_F16) : q_dtype != kv_dtype)
    return fail(PKV_EUNSUPPORTED, "q_dtype %d (built: the pool's dtype for 16-bit pools, bf16 or f16 for 8-bit)",
                q_dtype);
  if ((k_new == nullptr) != (v_new == nullptr)) return fail(PKV_EINVAL, "k_new and v_new must both be given or NULL");
  if (keep_stride < 0 || keep_stride > (1 << 30)) return fail(PKV_EINVAL, "keep_stride %d outside [0, 2^30]", keep_stride);
  if (dst_stride < 1 || dst_stride > (1 << 26)) return fail(PKV_EINVAL, "dst_stride %d outside [1, 2^26]", dst_stride);
  const bool mass = attn_mass != nullptr;
  if (mass) {
    if (!attn_mass_src) return fail(PKV_EINVAL, "attn_mass needs attn_mass_src (the source score rows)");
    if (attn_mass_src == attn_mass) return fail(PKV_EINVAL, "attn_mass_src and attn_mass must be different arrays");
    if (attn_mass_src_stride < max_context_len)
      return fail(PKV_EINVAL, "attn_mass_src_stride %d < max_context_len %d", attn_mass_src_stride, max_context_len);
  }
  const size_t need = paged_decode_attn_compact_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len, mass);
  if (workspace_bytes < need) return fail(PKV_EWORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  pkv::AttnArgs a;
  int st = prepare_decode_attn(a, out, out_dtype, q, q_dtype, k_pool, v_pool, k_scale, v_scale, kv_dtype,
                               block_tables, block_table_stride, context_lens, max_context_len, num_seqs, num_blocks,
                               num_q_heads, num_kv_heads, head_dim, block_size, scale, 0, 0, attn_mass,
                               attn_mass_stride, workspace, workspace_bytes);
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return ok();
  if (!keep_idx || !keep_count || !dst_tables) return fail(PKV_EINVAL, "NULL array argument");
  if (k_new && ((uintptr_t)k_new % 16 || (uintptr_t)v_new % 16))
    return fail(PKV_EINVAL, "k_new and v_new must be 16-byte aligned");
  const int map_stride = (max_context_len + 15) / 16;
  auto* map = reinterpret_cast<pkv::KeepMapEntry*>(
      reinterpret_cast<char*>(workspace) + compact_map_offset(num_seqs, num_q_heads, head_dim, max_context_len, mass));
  st = device_status(pkv::launch_keep_map(keep_idx, keep_stride, keep_count, context_lens, max_context_len, dst_tables,
                                          dst_stride, num_blocks, num_seqs, map_stride, k_new != nullptr ? 1 : 0, map,
                                          (hipStream_t)stream),
                     "paged_decode_attn_compact");
  if (st != PKV_OK) return st;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_store = k_pool;
  a.v_store = v_pool;
  a.k_scale_store = k_scale;
  a.v_scale_store = v_scale;
  a.keep_map = map;
  a.map_stride = map_stride;
  a.mass_src = attn_mass_src;
  a.mass_src_stride = attn_mass_src_stride;
  return launch_prepared_attn(a, kv_dtype, q_dtype, head_dim, stream, "paged_decode_attn_compact");
}

int paged_prefill_attn(void* out, int out_dtype, const void* q, int q_dtype, const void* k_pool, const void* v_pool,
                       const float* k_scale, const float* v_scale, int kv_dtype, const int32_t* block_tables,
                       int block_table_stride, const int32_t* context_lens, const int32_t* query_start,
                       int num_tokens, int max_context_len, int max_query_len, int num_seqs, int num_blocks,
                       int num_q_heads, int num_kv_heads, int head_dim, int block_size, float scale, void* stream) {
  if (block_size != pkv::kBlockSize) return fail(PKV_EUNSUPPORTED, "block_size %d (built: 16)", block_size);
  if (head_dim != 64 && head_dim != 128) return fail(PKV_EUNSUPPORTED, "head_dim %d (built: 64, 128)", head_dim);
  if (num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads)
    return fail(PKV_EINVAL, "num_q_heads %d is not a positive multiple of num_kv_heads %d", num_q_heads, num_kv_heads);
  const int g = num_q_heads / num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16)
    return fail(PKV_EUNSUPPORTED, "%d query heads per KV head (built: 1, 2, 4, 8, 16)", g);
  if (!valid_kv_dtype(kv_dtype)) return fail(PKV_EINVAL, "kv_dtype %d", kv_dtype);
  if (!valid_float_dtype(q_dtype)) return fail(PKV_EINVAL, "q_dtype %d", q_dtype);
  if (!valid_float_dtype(out_dtype)) return fail(PKV_EINVAL, "out_dtype %d", out_dtype);
  if (!isfinite(scale)) return fail(PKV_EINVAL, "scale is not finite");
  if (num_seqs < 0 || num_seqs > 65535) return fail(PKV_EINVAL, "num_seqs %d outside [0, 65535]", num_seqs);
  if (num_tokens < 0) return fail(PKV_EINVAL, "num_tokens %d < 0", num_tokens);
  if (max_context_len < 1 || max_context_len > (1 << 30))
    return fail(PKV_EINVAL, "max_context_len %d outside [1, 2^30]", max_context_len);
  if (max_query_len < 1 || max_query_len > max_context_len)
    return fail(PKV_EINVAL, "max_query_len %d outside [1, max_context_len]", max_query_len);
  if (num_blocks < 1) return fail(PKV_EINVAL, "num_blocks %d < 1", num_blocks);
  if (block_table_stride < (max_context_len + 15) / 16 || block_table_stride > (1 << 26))
    return fail(PKV_EINVAL, "block_table_stride %d < ceil(max_context_len / 16) (or > 2^26)", block_table_stride);
  const long long tiles = (max_query_len + 4LL * (16 / g) - 1) / (4LL * (16 / g));
  if (tiles * num_seqs * num_kv_heads > (1LL << 31) - 1) return fail(PKV_EINVAL, "grid too large");
  if (num_seqs == 0 || num_tokens == 0) return ok();
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens || !query_start)
    return fail(PKV_EINVAL, "NULL array argument");
  if (code8_kv(kv_dtype) && (!k_scale || !v_scale)) return fail(PKV_EINVAL, "FP8/INT8 pools need k_scale and v_scale");
  if ((uintptr_t)q % 16 || (uintptr_t)k_pool % 16 || (uintptr_t)v_pool % 16 ||
      (k_scale && (uintptr_t)k_scale % 16) || (v_scale && (uintptr_t)v_scale % 16))
    return fail(PKV_EINVAL, "q, pools and scales must be 16-byte aligned");
  pkv::PrefillArgs a{};
  a.out = out;
  a.out_dtype = out_dtype;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_tables = block_tables;
  a.table_stride = block_table_stride;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.num_tokens = num_tokens;
  a.max_context_len = max_context_len;
  a.num_seqs = num_seqs;
  a.num_blocks = num_blocks;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.tiles_per_pair = (int)tiles;
  return device_status(pkv::launch_prefill_attn(a, kv_dtype, q_dtype, head_dim, max_query_len, (hipStream_t)stream),
                       "paged_prefill_attn");
}

int kv_swap(void* k_pool, void* v_pool, float* k_scale, float* v_scale, int kv_dtype, void* host_k, void* host_v,
            float* host_k_scale, float* host_v_scale, const int32_t* block_slot_pairs, int num_pairs, int num_blocks,
            int host_slots, int num_kv_heads, int head_dim, int block_size, int to_host, void* stream) {
  if (block_size != pkv::kBlockSize) return fail(PKV_EUNSUPPORTED, "block_size %d (built: 16)", block_size);
  if (head_dim != 64 && head_dim != 128) return fail(PKV_EUNSUPPORTED, "head_dim %d (built: 64, 128)", head_dim);
  if (!valid_kv_dtype(kv_dtype)) return fail(PKV_EINVAL, "kv_dtype %d", kv_dtype);
  if (to_host != 0 && to_host != 1) return fail(PKV_EINVAL, "to_host %d is neither 0 nor 1", to_host);
  if (num_pairs < 0 || num_pairs > (1 << 24)) return fail(PKV_EINVAL, "num_pairs %d outside [0, 2^24]", num_pairs);
  if (num_blocks < 1 || host_slots < 1 || num_kv_heads < 1)
    return fail(PKV_EINVAL, "num_blocks, host_slots and num_kv_heads must be >= 1");
  if (num_pairs == 0) return ok();
  if (!k_pool || !v_pool || !host_k || !host_v || !block_slot_pairs) return fail(PKV_EINVAL, "NULL array argument");
  if (quantised_kv(kv_dtype) && (!k_scale || !v_scale || !host_k_scale || !host_v_scale))
    return fail(PKV_EINVAL, "FP8/INT8 pools need device and host scales");
  if ((uintptr_t)k_pool % 16 || (uintptr_t)v_pool % 16 || (uintptr_t)host_k % 16 || (uintptr_t)host_v % 16)
    return fail(PKV_EINVAL, "pools and host arenas must be 16-byte aligned");
  return device_status(pkv::launch_kv_swap(k_pool, v_pool, k_scale, v_scale, kv_dtype, host_k, host_v, host_k_scale,
                                           host_v_scale, block_slot_pairs, num_pairs, num_blocks, host_slots,
                                           num_kv_heads, head_dim, to_host, (hipStream_t)stream),
                       "kv_swap");
}

int kv_block_copy(void* k_pool, void* v_pool, float* k_scale, float* v_scale, int kv_dtype, const int32_t* block_pairs,
                  int num_pairs, int num_blocks, int num_kv_heads, int head_dim, int block_size, void* stream) {
  if (block_size != pkv::kBlockSize) return fail(PKV_EUNSUPPORTED, "block_size %d (built: 16)", block_size);
  if (head_dim != 64 && head_dim != 128) return fail(PKV_EUNSUPPORTED, "head_dim %d (built: 64, 128)", head_dim);
  if (!valid_kv_dtype(kv_dtype)) return fail(PKV_EINVAL, "kv_dtype %d", kv_dtype);
  if (num_pairs < 0 || num_pairs > 65535) return fail(PKV_EINVAL, "num_pairs %d outside [0, 65535]", num_pairs);
  if (num_blocks < 1 || num_kv_heads < 1) return fail(PKV_EINVAL, "num_blocks and num_kv_heads must be >= 1");
  if (num_pairs == 0) return ok();
  if (!k_pool || !v_pool || !block_pairs) return fail(PKV_EINVAL, "NULL array argument");
  if (quantised_kv(kv_dtype) && (!k_scale || !v_scale))
    return fail(PKV_EINVAL, "FP8/INT8 pools with per-token scales need k_scale and v_scale");
  if ((uintptr_t)k_pool % 16 || (uintptr_t)v_pool % 16) return fail(PKV_EINVAL, "pools must be 16-byte aligned");
  return device_status(pkv::launch_block_copy(k_pool, v_pool, k_scale, v_scale, kv_dtype, block_pairs, num_pairs,
                                              num_blocks, num_kv_heads, head_dim, (hipStream_t)stream),
                       "kv_block_copy");
}

int h2o_select(const float* scores, int scores_stride, const int32_t* kv_lens, int num_seqs, int max_kv_len,
               int budget, int recent, int32_t* keep_idx, int32_t* keep_count, void* stream) {
  if (num_seqs < 0) return fail(PKV_EINVAL, "num_seqs %d < 0", num_seqs);
  if (budget < 1) return fail(PKV_EINVAL, "budget %d < 1", budget);
  if (recent < 0 || recent > budget) return fail(PKV_EINVAL, "recent %d outside [0, budget=%d]", recent, budget);
  if (max_kv_len < 1) return fail(PKV_EINVAL, "max_kv_len %d < 1", max_kv_len);
  if (scores_stride < max_kv_len) return fail(PKV_EINVAL, "scores_stride %d < max_kv_len %d", scores_stride, max_kv_len);
  if (num_seqs == 0) return ok();
  if (!scores || !kv_lens || !keep_idx || !keep_count) return fail(PKV_EINVAL, "NULL array argument");
  if (num_seqs > (1 << 30)) return fail(PKV_EINVAL, "num_seqs too large");
  return device_status(pkv::launch_keep_select(scores, scores_stride, kv_lens, num_seqs, max_kv_len, 0, recent,
                                               budget - recent, PKV_CAND_REST, keep_idx, budget, keep_count,
                                               (hipStream_t)stream),
                       "h2o_select");
}

int kv_keep_select(const float* scores, int scores_stride, const int32_t* kv_lens, int num_seqs, int max_kv_len,
                   int num_sinks, int recent, int heavy, int candidates, int32_t* keep_idx, int keep_stride,
                   int32_t* keep_count, void* stream) {
  if (num_seqs < 0 || num_seqs > (1 << 30)) return fail(PKV_EINVAL, "num_seqs %d outside [0, 2^30]", num_seqs);
  if (num_sinks < 0 || recent < 0 || heavy < 0)
    return fail(PKV_EINVAL, "num_sinks %d, recent %d, heavy %d must be >= 0", num_sinks, recent, heavy);
  if (candidates != PKV_CAND_REST && candidates != PKV_CAND_ALL) return fail(PKV_EINVAL, "candidates %d", candidates);
  if (max_kv_len < 1 || max_kv_len > (1 << 30)) return fail(PKV_EINVAL, "max_kv_len %d outside [1, 2^30]", max_kv_len);
  if (scores_stride < max_kv_len) return fail(PKV_EINVAL, "scores_stride %d < max_kv_len %d", scores_stride, max_kv_len);
  const long long most = (long long)num_sinks + recent + heavy;
  const long long need = most < max_kv_len ? most : max_kv_len;
  if (keep_stride < need || keep_stride < 1 || keep_stride > (1 << 30))
    return fail(PKV_EINVAL, "keep_stride %d < min(num_sinks + recent + heavy, max_kv_len) = %lld (or > 2^30)",
                keep_stride, need);
  if (num_seqs == 0) return ok();
  if (!scores || !kv_lens || !keep_idx || !keep_count) return fail(PKV_EINVAL, "NULL array argument");
  return device_status(pkv::launch_keep_select(scores, scores_stride, kv_lens, num_seqs, max_kv_len, num_sinks, recent,
                                               heavy, candidates, keep_idx, keep_stride, keep_count,
                                               (hipStream_t)stream),
                       "kv_keep_select");
}

int kv_compact(void* k_pool, void* v_pool, float* k_scale, float* v_scale, int kv_dtype, const int32_t* src_tables,
               int src_stride, const int32_t* dst_tables, int dst_stride, const int32_t* keep_idx, int keep_stride,
               const int32_t* keep_count, int num_seqs, int num_blocks, int num_kv_heads, int head_dim,
               int block_size, void* stream) {
  if (block_size != pkv::kBlockSize) return fail(PKV_EUNSUPPORTED, "block_size %d (built: 16)", block_size);
  if (head_dim != 64 && head_dim != 128) return fail(PKV_EUNSUPPORTED, "head_dim %d (built: 64, 128)", head_dim);
  if (!valid_kv_dtype(kv_dtype)) return fail(PKV_EINVAL, "kv_dtype %d", kv_dtype);
  if (num_seqs < 0 || num_seqs > 65535) return fail(PKV_EINVAL, "num_seqs %d outside [0, 65535]", num_seqs);
  if (num_kv_heads < 1 || num_kv_heads > 65535) return fail(PKV_EINVAL, "num_kv_heads %d outside [1, 65535]", num_kv_heads);
  if (num_blocks < 1) return fail(PKV_EINVAL, "num_blocks %d < 1", num_blocks);
  if (src_stride < 1 || src_stride > (1 << 26) || dst_stride < 1 || dst_stride > (1 << 26))
    return fail(PKV_EINVAL, "table strides %d, %d outside [1, 2^26]", src_stride, dst_stride);
  if (keep_stride < 0 || keep_stride > (1 << 30)) return fail(PKV_EINVAL, "keep_stride %d outside [0, 2^30]", keep_stride);
  if ((long long)((keep_stride + 15) / 16) * num_kv_heads > (1LL << 24))   // 256 threads each in one grid dimension
    return fail(PKV_EINVAL, "ceil(keep_stride / 16) * num_kv_heads > 2^24");
  if (num_seqs == 0 || keep_stride == 0) return ok();
  if (!k_pool || !v_pool || !src_tables || !dst_tables || !keep_idx || !keep_count)
    return fail(PKV_EINVAL, "NULL array argument");
  if (quantised_kv(kv_dtype) && (!k_scale || !v_scale))
    return fail(PKV_EINVAL, "FP8/INT8 pools with per-token scales need k_scale and v_scale");
  if ((uintptr_t)k_pool % 16 || (uintptr_t)v_pool % 16) return fail(PKV_EINVAL, "pools must be 16-byte aligned");
  return device_status(pkv::launch_kv_compact(k_pool, v_pool, k_scale, v_scale, kv_dtype, src_tables, src_stride,
                                              dst_tables, dst_stride, keep_idx, keep_stride, keep_count, num_seqs,
                                              num_blocks, num_kv_heads, head_dim, (hipStream_t)stream),
                       "kv_compact");
}

int pkv_timing_begin(int capacity) {
  if (capacity < 1 || capacity > 100000) return fail(PKV_EINVAL, "capacity %d outside [1, 100000]", capacity);
  if (g_timing.active) return fail(PKV_EINVAL, "a timing session is already open");
  g_timing.ev.clear();
  for (int i = 0; i < capacity; ++i) {
    hipEvent_t a = nullptr, b = nullptr;
    hipError_t e = hipEventCreate(&a);
    if (e == hipSuccess) e = hipEventCreate(&b);
    if (e != hipSuccess) {
      for (auto& p : g_timing.ev) {
        (void)hipEventDestroy(p.first);
        (void)hipEventDestroy(p.second);
      }
      g_timing.ev.clear();
      return device_status(e, "hipEventCreate");
    }
    g_timing.ev.emplace_back(a, b);
  }
  g_timing.used = 0;
  g_timing.active = true;
  return ok();
}

int pkv_timing_end(float* ms_out, int capacity) {
  if (!g_timing.active) {
    fail(PKV_EINVAL, "no timing session open");
    return -1;
  }
  g_timing.active = false;
  int n = g_timing.used;
  hipError_t e = hipSuccess;
  if (n > 0) e = hipEventSynchronize(g_timing.ev[n - 1].second);
  for (int i = 0; i < n && e == hipSuccess; ++i) {
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, g_timing.ev[i].first, g_timing.ev[i].second);
    if (ms_out && i < capacity) ms_out[i] = ms;
  }
  for (auto& p : g_timing.ev) {
    (void)hipEventDestroy(p.first);
    (void)hipEventDestroy(p.second);
  }
  g_timing.ev.clear();
  g_timing.used = 0;
  if (e != hipSuccess) {
    device_status(e, "pkv_timing_end");
    return -1;
  }
  ok();
  return n < capacity ? n : capacity;
}

int pkv_probe_read(const void* src, size_t bytes, float* sink, void* stream) {
  if (bytes % 16) return fail(PKV_EINVAL, "bytes must be a multiple of 16");
  if (bytes == 0) return ok();
  if (!src || !sink) return fail(PKV_EINVAL, "NULL array argument");
  return device_status(pkv::launch_probe_read(src, bytes, sink, (hipStream_t)stream), "pkv_probe_read");
}

int pkv_probe_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (bytes % 16) return fail(PKV_EINVAL, "bytes must be a multiple of 16");
  if (bytes == 0) return ok();
  if (!src || !dst) return fail(PKV_EINVAL, "NULL array argument");
  return device_status(pkv::launch_probe_copy(dst, src, bytes, (hipStream_t)stream), "pkv_probe_copy");
}

}  // extern "C"
