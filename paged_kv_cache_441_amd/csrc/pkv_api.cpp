// The extern "C" surface of libpagedkv: argument checks, workspace layout and
// kernel dispatch.  Every check runs before anything is enqueued; no entry point
// allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/pagedkv.h"
#include "pkv_launch.hpp"

namespace {

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int log2_exact(int64_t x) {
  int s = 0;
  while ((int64_t{1} << s) < x) ++s;
  return s;
}

size_t elem_bytes(int32_t t) { return t == PKV_FP8_E4M3 ? 1 : t == PKV_BF16 ? 2 : 4; }

// Device buffers of rows (caches, queries, keys, values, outputs, workspaces) are
// moved in 16-byte pieces, int32 arrays element by element.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Arithmetic types (queries, outputs, the inputs of a quantised write).
bool valid_dtype(int32_t t) { return t == PKV_F32 || t == PKV_BF16; }
// Types a cache may hold (bit copies).
bool valid_storage(int32_t t) { return valid_dtype(t) || t == PKV_FP8_E4M3; }

// A launch holds at most 2^32 - 1 threads per grid dimension; the per-token and
// per-pair launches put up to 256 threads per item in x.
constexpr int64_t kMaxItems256 = int64_t{UINT32_MAX} / 256;

// A cache scale: positive and finite.
bool valid_scale(float x) { return std::isfinite(x) && x > 0.f; }

// Multiplication of non-negative sizes with an overflow check against a limit.
bool mul_ok(int64_t a, int64_t b, int64_t limit, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > limit / a) return false;
  *out = a * b;
  return true;
}

struct AttnShape {
  bool balanced = false;    // PKV_PARTITION_BALANCED: equal shares of the tile list per workgroup
  int64_t max_parts = 0;
  int partition = 0;
  int64_t recs = 0;         // partial-result records (one per row of head_dim + 2 floats)
  size_t plan_bytes = 0;    // the work plan at the start of the workspace
  size_t ws_bytes = 0;      // plan + partition records
};

// Shape checks common to every attention entry point; fills the derived sizes.
pkv_status check_attention_shape(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                 int32_t block_size, int32_t max_blocks_per_seq,
                                 int32_t partition_size, AttnShape* s) {
  if (num_seqs < 0 || num_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      max_blocks_per_seq <= 0 || partition_size < PKV_PARTITION_BALANCED)
    return PKV_ERR_INVALID_ARG;
  if (!is_pow2(block_size) || block_size > 1024) return PKV_ERR_INVALID_ARG;
  int64_t max_ctx = 0;
  if (!mul_ok(max_blocks_per_seq, block_size, INT32_MAX, &max_ctx)) return PKV_ERR_INVALID_ARG;
  // launches put at most 256 threads per (sequence, query head) row in x
  int64_t rows = 0;
  if (!mul_ok(num_seqs, num_heads, int64_t{UINT32_MAX} / 256, &rows)) return PKV_ERR_UNSUPPORTED;
  int64_t recs = 0, t = 0;
  if (partition_size == PKV_PARTITION_BALANCED) {
    // Balanced: one record row per (segment label, head); labels < max workgroups + seqs.
    s->balanced = true;
    s->partition = 0;
    s->max_parts = 1;
    int64_t tiles = 0;
    if (!mul_ok(num_seqs, (max_ctx + pkv::kTileTokens - 1) / pkv::kTileTokens + pkv::kSeqCost,
                INT32_MAX / 2, &tiles))
      return PKV_ERR_UNSUPPORTED;   // the tile list is indexed with int32
    if (!mul_ok(int64_t{num_seqs} + pkv::kMaxStreamWgs, num_heads, INT64_MAX / 8, &recs))
      return PKV_ERR_INVALID_ARG;
    s->plan_bytes = pkv::tile_plan_bytes(num_seqs);
  } else {
    const int P = partition_size == PKV_PARTITION_DEFAULT ? PKV_DEFAULT_PARTITION_TOKENS
                                                          : partition_size;
    if (P % block_size != 0 || P % 16 != 0) return PKV_ERR_INVALID_ARG;
    s->partition = P;
    s->max_parts = (max_ctx + P - 1) / P;
    if (!mul_ok(num_seqs, num_heads, INT64_MAX / 8, &t) ||
        !mul_ok(t, s->max_parts, INT64_MAX / 8, &recs))
      return PKV_ERR_INVALID_ARG;
    int64_t items = 0;
    if (!mul_ok(num_seqs, s->max_parts, INT32_MAX, &items)) return PKV_ERR_UNSUPPORTED;
    s->plan_bytes = pkv::plan_bytes(num_seqs, s->max_parts);
  }
  int64_t bytes = 0;
  if (!mul_ok(recs, int64_t{head_dim} + 2, INT64_MAX / 8, &bytes)) return PKV_ERR_INVALID_ARG;
  s->recs = recs;
  s->ws_bytes = s->plan_bytes + static_cast<size_t>(bytes) * 4;
  return PKV_OK;
}

void set_workspace(pkv::AttentionArgs* a, void* workspace, size_t plan_bytes, int64_t recs) {
  char* ws = static_cast<char*>(workspace);
  a->plan_count = ws ? reinterpret_cast<int*>(ws) : nullptr;
  a->plan_items = ws ? reinterpret_cast<int4*>(ws + 256) : nullptr;
  a->tile_hdr = ws ? reinterpret_cast<int*>(ws) : nullptr;
  a->tile_cum = ws ? reinterpret_cast<int*>(ws + 256) : nullptr;
  float* f = ws ? reinterpret_cast<float*>(ws + plan_bytes) : nullptr;
  a->ws_m = f;
  a->ws_l = f ? f + recs : nullptr;
  a->ws_o = f ? f + 2 * recs : nullptr;
}

pkv_status fill_attention_args(void* out, const void* query, const void* key_cache,
                               const void* value_cache, const int32_t* block_tables,
                               const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                               int32_t partition_size, int32_t kv_dtype, int32_t out_dtype,
                               void* workspace, size_t workspace_bytes, bool need_inputs,
                               pkv::AttentionArgs* a, float k_scale = 1.f,
                               float v_scale = 1.f) {
  AttnShape s;
  pkv_status st = check_attention_shape(num_seqs, num_heads, head_dim, block_size,
                                        max_blocks_per_seq, partition_size, &s);
  if (st != PKV_OK) return st;
  const bool fp8 = kv_dtype == PKV_FP8_E4M3;
  if (!(valid_dtype(kv_dtype) || fp8) || !valid_dtype(out_dtype)) return PKV_ERR_INVALID_ARG;
  if (fp8) {
    if (!valid_scale(k_scale) || !valid_scale(v_scale) ||
        !std::isfinite(static_cast<float>(static_cast<double>(scale) * k_scale * 1.4426950408889634)))
      return PKV_ERR_INVALID_ARG;   // the score factor must stay a finite fp32
    if (!s.balanced) return PKV_ERR_UNSUPPORTED;   // E4M3 caches use the balanced split
    if (need_inputs && head_dim == 64 && num_kv_heads % 2 != 0)
      return PKV_ERR_UNSUPPORTED;                  // a staged row spans at least 128 bytes
  }
  if (need_inputs) {
    if (num_kv_heads <= 0 || num_heads % num_kv_heads != 0) return PKV_ERR_INVALID_ARG;
    if (num_blocks <= 0 || num_blocks > INT32_MAX || !std::isfinite(scale))
      return PKV_ERR_INVALID_ARG;   // block ids are int32
    int64_t pool = 0;
    if (!mul_ok(num_blocks, block_size, INT64_MAX / 4096, &pool) ||
        !mul_ok(pool, int64_t{num_kv_heads} * head_dim, INT64_MAX / 8, &pool))
      return PKV_ERR_INVALID_ARG;
  }
  if (num_seqs > 0) {
    if (!out || !context_lens) return PKV_ERR_INVALID_ARG;
    if (need_inputs && (!query || !key_cache || !value_cache || !block_tables))
      return PKV_ERR_INVALID_ARG;
    if (!aligned16(out) || !aligned4(context_lens) || !aligned16(workspace) ||
        (need_inputs && (!aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache) ||
                         !aligned4(block_tables))))
      return PKV_ERR_INVALID_ARG;
  }
  if (need_inputs) {
    const int G = num_heads / num_kv_heads;
    if (!(G == 1 || G == 2 || G == 4 || G == 8)) return PKV_ERR_UNSUPPORTED;
  }
  if (!(head_dim == 64 || head_dim == 128)) return PKV_ERR_UNSUPPORTED;
  if (!(block_size == 16 || block_size == 32)) return PKV_ERR_UNSUPPORTED;
  if (num_seqs > 0 && (!workspace || workspace_bytes < s.ws_bytes)) return PKV_ERR_WORKSPACE;
  if (!s.balanced) {
    // A launch holds at most 2^32 - 1 threads per grid dimension.  Fixed partitions put
    // one workgroup per (sequence, partition) in x: up to 512 threads (eight kv heads
    // of a group) in the streaming kernel, 256 per kv head in the per-head kernel.
    const int64_t per_item = std::max<int64_t>(512, 256 * int64_t{num_kv_heads > 0 ? num_kv_heads : 1});
    int64_t threads = 0;
    if (!mul_ok(s.max_parts * num_seqs, per_item, int64_t{UINT32_MAX}, &threads))
      return PKV_ERR_UNSUPPORTED;
  }

  a->out = out;
  a->query = query;
  a->key_cache = key_cache;
  a->value_cache = value_cache;
  a->block_tables = block_tables;
  a->context_lens = context_lens;
  a->num_seqs = num_seqs;
  a->num_heads = num_heads;
  a->num_kv_heads = num_kv_heads;
  a->head_dim = head_dim;
  a->block_shift = log2_exact(block_size);
  a->max_blocks_per_seq = max_blocks_per_seq;
  a->num_blocks = num_blocks;
  // scale * log2(e), and the key cache's scale for E4M3 codes
  a->scale_log2 = static_cast<float>(static_cast<double>(scale) * (fp8 ? k_scale : 1.f) *
                                     1.4426950408889634);
  a->partition_size = s.partition;
  a->max_parts = static_cast<int>(s.max_parts);
  a->kv_bf16 = kv_dtype == PKV_BF16;
  a->kv_fp8 = fp8;
  a->v_scale = fp8 ? v_scale : 1.f;
  a->out_bf16 = out_dtype == PKV_BF16;
  a->balanced = s.balanced;
  a->per_head = false;
  set_workspace(a, workspace, s.plan_bytes, s.recs);
  return PKV_OK;
}

pkv_status hip_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

// The three stages of a decode call on one stream.
pkv_status run_decode(const pkv::AttentionArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  pkv_status st = hip_status(pkv::launch_attention_plan(a, s));
  if (st != PKV_OK) return st;
  st = hip_status(pkv::launch_attention_partition(a, s));
  if (st != PKV_OK) return st;
  if (a.balanced || a.max_parts > 1) st = hip_status(pkv::launch_attention_reduce(a, s));
  return st;
}

}  // namespace

extern "C" {

int32_t pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_status_string(int32_t status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument (null pointer, bad size or shape)";
    case PKV_ERR_UNSUPPORTED: return "unsupported combination (head_dim, block_size, GQA group or dtype)";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_HIP: return "HIP runtime error at launch";
    case PKV_ERR_NO_BLOCKS: return "no free block left in the pool";
    case PKV_ERR_SCRATCH_LIMIT:
      return "the call needs more device scratch than the library's fixed buffer holds";
    default: return "unknown status";
  }
}

pkv_status pkv_slot_mapping(const int32_t* block_tables, const int32_t* context_lens,
                            int32_t* slot_mapping, int32_t num_seqs, int32_t max_blocks_per_seq,
                            int32_t block_size, int64_t num_blocks, void* stream) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || num_blocks <= 0) return PKV_ERR_INVALID_ARG;
  if (!is_pow2(block_size) || block_size > 1024) return PKV_ERR_INVALID_ARG;
  int64_t t = 0;
  if (!mul_ok(max_blocks_per_seq, block_size, INT32_MAX, &t) ||
      !mul_ok(num_blocks, block_size, INT32_MAX, &t))
    return PKV_ERR_INVALID_ARG;   // slots are int32
  if (num_seqs == 0) return PKV_OK;
  if (!block_tables || !context_lens || !slot_mapping) return PKV_ERR_INVALID_ARG;
  if (!aligned4(block_tables) || !aligned4(context_lens) || !aligned4(slot_mapping))
    return PKV_ERR_INVALID_ARG;
  return hip_status(pkv::launch_slot_mapping(block_tables, context_lens, slot_mapping, num_seqs,
                                             max_blocks_per_seq, log2_exact(block_size),
                                             num_blocks, static_cast<hipStream_t>(stream)));
}

pkv_status pkv_kv_cache_write(const void* key, const void* value, void* key_cache,
                              void* value_cache, const int32_t* slot_mapping, int32_t num_tokens,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int64_t num_blocks, pkv_dtype kv_dtype, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PKV_ERR_INVALID_ARG;
  if (!valid_storage(kv_dtype)) return PKV_ERR_INVALID_ARG;
  int64_t row = 0, slots = 0;
  if (!mul_ok(int64_t{num_kv_heads} * head_dim, elem_bytes(kv_dtype), INT32_MAX / 2, &row))
    return PKV_ERR_INVALID_ARG;
  if (!mul_ok(num_blocks, block_size, INT64_MAX / 4096, &slots)) return PKV_ERR_INVALID_ARG;
  int64_t cache_bytes = 0;
  if (!mul_ok(slots, row, INT64_MAX / 2, &cache_bytes)) return PKV_ERR_INVALID_ARG;
  if (row % 16 != 0 || num_tokens > kMaxItems256) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping) return PKV_ERR_INVALID_ARG;
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache) ||
      !aligned4(slot_mapping))
    return PKV_ERR_INVALID_ARG;
  return hip_status(pkv::launch_cache_write(key, value, key_cache, value_cache, slot_mapping,
                                            num_tokens, static_cast<int>(row), slots,
                                            static_cast<hipStream_t>(stream)));
}

pkv_status pkv_kv_cache_write_fp8(const void* key, const void* value, void* key_cache,
                                  void* value_cache, const int32_t* slot_mapping,
                                  int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int64_t num_blocks, pkv_dtype in_dtype,
                                  float k_scale, float v_scale, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PKV_ERR_INVALID_ARG;
  if (!valid_dtype(in_dtype) || !valid_scale(k_scale) || !valid_scale(v_scale))
    return PKV_ERR_INVALID_ARG;
  int64_t row = 0, slots = 0, cache_bytes = 0;   // row: elements = cache bytes
  if (!mul_ok(num_kv_heads, head_dim, INT32_MAX / 8, &row) ||
      !mul_ok(num_blocks, block_size, INT64_MAX / 4096, &slots) ||
      !mul_ok(slots, row, INT64_MAX / 2, &cache_bytes))
    return PKV_ERR_INVALID_ARG;
  if (row % 16 != 0 || num_tokens > kMaxItems256) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping) return PKV_ERR_INVALID_ARG;
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache) ||
      !aligned4(slot_mapping))
    return PKV_ERR_INVALID_ARG;
  return hip_status(pkv::launch_cache_write_fp8(key, value, key_cache, value_cache, slot_mapping,
                                                num_tokens, static_cast<int>(row), slots,
                                                in_dtype == PKV_BF16, k_scale, v_scale,
                                                static_cast<hipStream_t>(stream)));
}

pkv_status pkv_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs,
                           int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int64_t num_blocks, pkv_dtype kv_dtype,
                           void* stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PKV_ERR_INVALID_ARG;
  if (!valid_storage(kv_dtype)) return PKV_ERR_INVALID_ARG;
  int64_t row = 0, block = 0, cache_bytes = 0;
  if (!mul_ok(int64_t{num_kv_heads} * head_dim, elem_bytes(kv_dtype), INT32_MAX / 2, &row) ||
      !mul_ok(row, block_size, INT32_MAX / 2, &block) ||
      !mul_ok(block, num_blocks, INT64_MAX / 2, &cache_bytes))
    return PKV_ERR_INVALID_ARG;
  if (block % 16 != 0 || num_pairs > kMaxItems256) return PKV_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PKV_OK;
  if (!key_cache || !value_cache || !pairs) return PKV_ERR_INVALID_ARG;
  if (!aligned16(key_cache) || !aligned16(value_cache) || !aligned4(pairs))
    return PKV_ERR_INVALID_ARG;
  return hip_status(pkv::launch_copy_blocks(key_cache, value_cache, pairs, num_pairs, block,
                                            num_blocks, static_cast<hipStream_t>(stream)));
}

size_t pkv_paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                           int32_t block_size, int32_t max_blocks_per_seq,
                                           int32_t partition_size) {
  AttnShape s;
  if (check_attention_shape(num_seqs, num_heads, head_dim, block_size, max_blocks_per_seq,
                            partition_size, &s) != PKV_OK)
    return 0;
  return s.ws_bytes;
}

}  // extern "C"

namespace {

// pkv_decode_prologue and its E4M3 form: quant 0 copies the rows of the cache's own
// type (kv_dtype), quant != 0 stores the E4M3 codes of in_dtype rows.
pkv_status prologue(const int32_t* block_tables, const int32_t* context_lens, const void* key,
                    const void* value, void* key_cache, void* value_cache,
                    int32_t* slot_mapping, int32_t num_seqs, int32_t max_blocks_per_seq,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int64_t num_blocks, int32_t kv_dtype, bool quant, int32_t in_dtype,
                    float k_scale, float v_scale, int32_t partition_size, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0)
    return PKV_ERR_INVALID_ARG;
  if (!valid_storage(kv_dtype)) return PKV_ERR_INVALID_ARG;
  if (quant && (!valid_dtype(in_dtype) || !valid_scale(k_scale) || !valid_scale(v_scale)))
    return PKV_ERR_INVALID_ARG;
  AttnShape s;
  pkv_status st = check_attention_shape(num_seqs, 1, 64, block_size, max_blocks_per_seq,
                                        partition_size, &s);
  if (st != PKV_OK) return st;
  int64_t t = 0, row = 0, cache_bytes = 0;
  if (!mul_ok(num_blocks, block_size, INT32_MAX, &t)) return PKV_ERR_INVALID_ARG;  // int32 slots
  if (!mul_ok(int64_t{num_kv_heads} * head_dim, elem_bytes(kv_dtype), INT32_MAX / 2, &row) ||
      !mul_ok(t, row, INT64_MAX / 2, &cache_bytes))
    return PKV_ERR_INVALID_ARG;
  if (row % 16 != 0 || num_seqs >= kMaxItems256) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PKV_OK;
  if (!block_tables || !context_lens || !key || !value || !key_cache || !value_cache ||
      !slot_mapping)
    return PKV_ERR_INVALID_ARG;
  if (!aligned4(block_tables) || !aligned4(context_lens) || !aligned16(key) || !aligned16(value) ||
      !aligned16(key_cache) || !aligned16(value_cache) || !aligned4(slot_mapping) ||
      !aligned16(workspace))
    return PKV_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < s.plan_bytes) return PKV_ERR_WORKSPACE;
  pkv::AttentionArgs a{};
  set_workspace(&a, workspace, s.plan_bytes, 0);
  const int q = !quant ? 0 : in_dtype == PKV_BF16 ? 2 : 1;
  return hip_status(pkv::launch_decode_prologue(
      block_tables, context_lens, key, value, key_cache, value_cache, slot_mapping, num_seqs,
      max_blocks_per_seq, log2_exact(block_size), num_blocks, static_cast<int>(row), s.partition,
      a.plan_items, a.plan_count, s.balanced, a.tile_cum, a.tile_hdr, q, k_scale, v_scale,
      static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

pkv_status pkv_decode_prologue(const int32_t* block_tables, const int32_t* context_lens,
                               const void* key, const void* value, void* key_cache,
                               void* value_cache, int32_t* slot_mapping, int32_t num_seqs,
                               int32_t max_blocks_per_seq, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int64_t num_blocks, pkv_dtype kv_dtype,
                               int32_t partition_size, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return prologue(block_tables, context_lens, key, value, key_cache, value_cache, slot_mapping,
                  num_seqs, max_blocks_per_seq, num_kv_heads, head_dim, block_size, num_blocks,
                  kv_dtype, false, kv_dtype, 1.f, 1.f, partition_size, workspace,
                  workspace_bytes, stream);
}

pkv_status pkv_decode_prologue_fp8(const int32_t* block_tables, const int32_t* context_lens,
                                   const void* key, const void* value, void* key_cache,
                                   void* value_cache, int32_t* slot_mapping, int32_t num_seqs,
                                   int32_t max_blocks_per_seq, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                   pkv_dtype in_dtype, float k_scale, float v_scale,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return prologue(block_tables, context_lens, key, value, key_cache, value_cache, slot_mapping,
                  num_seqs, max_blocks_per_seq, num_kv_heads, head_dim, block_size, num_blocks,
                  PKV_FP8_E4M3, true, in_dtype, k_scale, v_scale, PKV_PARTITION_BALANCED,
                  workspace, workspace_bytes, stream);
}

pkv_status pkv_paged_attention_plan(const int32_t* context_lens, int32_t num_seqs,
                                    int32_t block_size, int32_t max_blocks_per_seq,
                                    int32_t partition_size, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  AttnShape s;
  pkv_status st = check_attention_shape(num_seqs, 1, 64, block_size, max_blocks_per_seq,
                                        partition_size, &s);
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return PKV_OK;
  if (!context_lens || !aligned4(context_lens) || !aligned16(workspace)) return PKV_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < s.plan_bytes) return PKV_ERR_WORKSPACE;
  pkv::AttentionArgs a{};
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.block_shift = log2_exact(block_size);
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.partition_size = s.partition;
  a.max_parts = static_cast<int>(s.max_parts);
  a.balanced = s.balanced;
  set_workspace(&a, workspace, s.plan_bytes, 0);
  return hip_status(pkv::launch_attention_plan(a, static_cast<hipStream_t>(stream)));
}

pkv_status pkv_paged_attention_partition(void* out, const void* query, const void* key_cache,
                                         const void* value_cache, const int32_t* block_tables,
                                         const int32_t* context_lens, int32_t num_seqs,
                                         int32_t num_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t block_size,
                                         int32_t max_blocks_per_seq, int64_t num_blocks,
                                         float scale, int32_t partition_size,
                                         pkv_dtype kv_dtype, pkv_dtype out_dtype,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  if (kv_dtype == PKV_FP8_E4M3) return PKV_ERR_INVALID_ARG;   // the _fp8 entry carries scales
  pkv::AttentionArgs a{};
  pkv_status st = fill_attention_args(out, query, key_cache, value_cache, block_tables,
                                      context_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                                      block_size, max_blocks_per_seq, num_blocks, scale,
                                      partition_size, kv_dtype, out_dtype, workspace,
                                      workspace_bytes, true, &a);
  if (st != PKV_OK || num_seqs == 0) return st;
  return hip_status(pkv::launch_attention_partition(a, static_cast<hipStream_t>(stream)));
}

pkv_status pkv_paged_attention_reduce(void* out, const int32_t* context_lens, int32_t num_seqs,
                                      int32_t num_heads, int32_t head_dim, int32_t block_size,
                                      int32_t max_blocks_per_seq, int32_t partition_size,
                                      pkv_dtype out_dtype, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  pkv::AttentionArgs a{};
  pkv_status st = fill_attention_args(out, nullptr, nullptr, nullptr, nullptr, context_lens,
                                      num_seqs, num_heads, 0, head_dim, block_size,
                                      max_blocks_per_seq, 0, 1.0f, partition_size, PKV_F32,
                                      out_dtype, workspace, workspace_bytes, false, &a);
  if (st != PKV_OK || num_seqs == 0) return st;
  return hip_status(pkv::launch_attention_reduce(a, static_cast<hipStream_t>(stream)));
}

pkv_status pkv_paged_attention_decode(void* out, const void* query, const void* key_cache,
                                      const void* value_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t max_blocks_per_seq,
                                      int64_t num_blocks, float scale, int32_t partition_size,
                                      pkv_dtype kv_dtype, pkv_dtype out_dtype, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (kv_dtype == PKV_FP8_E4M3) return PKV_ERR_INVALID_ARG;   // the _fp8 entry carries scales
  pkv::AttentionArgs a{};
  pkv_status st = fill_attention_args(out, query, key_cache, value_cache, block_tables,
                                      context_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                                      block_size, max_blocks_per_seq, num_blocks, scale,
                                      partition_size, kv_dtype, out_dtype, workspace,
                                      workspace_bytes, true, &a);
  if (st != PKV_OK || num_seqs == 0) return st;
  return run_decode(a, stream);
}

pkv_status pkv_paged_attention_partition_per_head(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int64_t num_blocks, float scale, int32_t partition_size,
    pkv_dtype kv_dtype, pkv_dtype out_dtype, void* workspace, size_t workspace_bytes,
    void* stream) {
  if (kv_dtype == PKV_FP8_E4M3 || partition_size == PKV_PARTITION_BALANCED)
    return PKV_ERR_INVALID_ARG;
  pkv::AttentionArgs a{};
  pkv_status st = fill_attention_args(out, query, key_cache, value_cache, block_tables,
                                      context_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                                      block_size, max_blocks_per_seq, num_blocks, scale,
                                      partition_size, kv_dtype, out_dtype, workspace,
                                      workspace_bytes, true, &a);
  if (st != PKV_OK || num_seqs == 0) return st;
  a.per_head = true;
  return hip_status(pkv::launch_attention_partition(a, static_cast<hipStream_t>(stream)));
}

pkv_status pkv_paged_attention_decode_per_head(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int64_t num_blocks, float scale, int32_t partition_size,
    pkv_dtype kv_dtype, pkv_dtype out_dtype, void* workspace, size_t workspace_bytes,
    void* stream) {
  if (kv_dtype == PKV_FP8_E4M3 || partition_size == PKV_PARTITION_BALANCED)
    return PKV_ERR_INVALID_ARG;
  pkv::AttentionArgs a{};
  pkv_status st = fill_attention_args(out, query, key_cache, value_cache, block_tables,
                                      context_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                                      block_size, max_blocks_per_seq, num_blocks, scale,
                                      partition_size, kv_dtype, out_dtype, workspace,
                                      workspace_bytes, true, &a);
  if (st != PKV_OK || num_seqs == 0) return st;
  a.per_head = true;
  return run_decode(a, stream);
}

}  // extern "C"

// ---- the entry point that allocates nothing ------------------------------------------

// The device scratch of pkv_paged_attention_decode_noalloc: one copy per GPU, held from
// the first use on that GPU until the process ends.  Host code never passes `scratch`
// itself to a kernel (on the host it is only a stand-in for the symbol); it uses the
// address hipGetSymbolAddress returned for the device, kept in scratch_ptr below.
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

// The scratch address on the device of `stream` (the current device for the null
// stream), looked up once per device with that device current.
pkv_status device_scratch(void* stream, void** out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev)
                        : hipGetDevice(&dev);
  if (e != hipSuccess) return PKV_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return PKV_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return PKV_ERR_HIP;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return PKV_ERR_HIP;
    if (e != hipSuccess || !p) return PKV_ERR_HIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_paged_attention_decode_noalloc(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int64_t num_blocks, float scale, int32_t partition_size,
    pkv_dtype kv_dtype, pkv_dtype out_dtype, void* stream) {
  if (kv_dtype == PKV_FP8_E4M3) return PKV_ERR_INVALID_ARG;   // the _fp8 entry carries scales
  AttnShape s;
  pkv_status st = check_attention_shape(num_seqs, num_heads, head_dim, block_size,
                                        max_blocks_per_seq, partition_size, &s);
  if (st != PKV_OK) return st;
  if (s.ws_bytes > PKV_NOALLOC_SCRATCH_BYTES) return PKV_ERR_SCRATCH_LIMIT;
  // every other argument check, with a stand-in workspace that is never dereferenced
  pkv::AttentionArgs a{};
  static char stand_in;
  st = fill_attention_args(out, query, key_cache, value_cache, block_tables, context_lens,
                           num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                           max_blocks_per_seq, num_blocks, scale, partition_size, kv_dtype,
                           out_dtype, &stand_in, s.ws_bytes, true, &a);
  if (st != PKV_OK || num_seqs == 0) return st;
  void* ws = nullptr;
  st = device_scratch(stream, &ws);
  if (st != PKV_OK) return st;
  set_workspace(&a, ws, s.plan_bytes, s.recs);
  return run_decode(a, stream);
}

pkv_status pkv_paged_attention_partition_fp8(void* out, const void* query,
                                             const void* key_cache, const void* value_cache,
                                             const int32_t* block_tables,
                                             const int32_t* context_lens, int32_t num_seqs,
                                             int32_t num_heads, int32_t num_kv_heads,
                                             int32_t head_dim, int32_t block_size,
                                             int32_t max_blocks_per_seq, int64_t num_blocks,
                                             float scale, float k_scale, float v_scale,
                                             pkv_dtype out_dtype, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  pkv::AttentionArgs a{};
  pkv_status st = fill_attention_args(out, query, key_cache, value_cache, block_tables,
                                      context_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                                      block_size, max_blocks_per_seq, num_blocks, scale,
                                      PKV_PARTITION_BALANCED, PKV_FP8_E4M3, out_dtype, workspace,
                                      workspace_bytes, true, &a, k_scale, v_scale);
  if (st != PKV_OK || num_seqs == 0) return st;
  return hip_status(pkv::launch_attention_partition(a, static_cast<hipStream_t>(stream)));
}

pkv_status pkv_paged_attention_decode_fp8(void* out, const void* query, const void* key_cache,
                                          const void* value_cache, const int32_t* block_tables,
                                          const int32_t* context_lens, int32_t num_seqs,
                                          int32_t num_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t block_size,
                                          int32_t max_blocks_per_seq, int64_t num_blocks,
                                          float scale, float k_scale, float v_scale,
                                          pkv_dtype out_dtype, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  pkv::AttentionArgs a{};
  pkv_status st = fill_attention_args(out, query, key_cache, value_cache, block_tables,
                                      context_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                                      block_size, max_blocks_per_seq, num_blocks, scale,
                                      PKV_PARTITION_BALANCED, PKV_FP8_E4M3, out_dtype, workspace,
                                      workspace_bytes, true, &a, k_scale, v_scale);
  if (st != PKV_OK || num_seqs == 0) return st;
  return run_decode(a, stream);
}

}  // extern "C"

// ---- multi-token steps ----------------------------------------------------------------

namespace {

struct MultiShape {
  int rows = 16;            // rows per unit: 32 when sequences average more than 16 rows
  int64_t max_units = 0;
  int64_t recs = 0;
  size_t plan_bytes = 0;
  size_t ws_bytes = 0;
};

pkv_status check_multi_shape(int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t max_blocks_per_seq, MultiShape* m) {
  if (num_seqs < 0 || num_tokens < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || max_blocks_per_seq <= 0 || num_heads % num_kv_heads != 0)
    return PKV_ERR_INVALID_ARG;
  if (!is_pow2(block_size) || block_size > 1024) return PKV_ERR_INVALID_ARG;
  int64_t max_ctx = 0;
  if (!mul_ok(max_blocks_per_seq, block_size, INT32_MAX / 2, &max_ctx)) return PKV_ERR_INVALID_ARG;
  const int G = num_heads / num_kv_heads;
  if (!(G == 1 || G == 2 || G == 4 || G == 8)) return PKV_ERR_UNSUPPORTED;
  // rows per unit from the average rows per sequence: one MFMA row block, two, or
  // (long prompts, head_dim 128) kMqRowWaves waves sharing one kv head
  const int64_t rows_total = int64_t{num_tokens} * G;
  if (head_dim == 128 && rows_total >= int64_t{pkv::kMqRowUnit} * num_seqs)
    m->rows = pkv::kMqRowUnit;
  else if (rows_total > int64_t{pkv::kMqRows} * num_seqs)
    m->rows = 2 * pkv::kMqRows;
  else
    m->rows = pkv::kMqRows;
  const int64_t tpb = m->rows / G;
  m->max_units = (int64_t{num_tokens} + tpb - 1) / tpb + num_seqs;
  // list positions are int32: units x (tiles of the longest context + 1)
  int64_t pos = 0;
  if (!mul_ok(m->max_units, (max_ctx + pkv::kTileTokens - 1) / pkv::kTileTokens + pkv::kSeqCost,
              INT32_MAX / 2, &pos))
    return PKV_ERR_UNSUPPORTED;
  if (!mul_ok(m->max_units + pkv::kMaxStreamWgs, int64_t{num_kv_heads} * m->rows,
              INT64_MAX / 1024, &m->recs))
    return PKV_ERR_INVALID_ARG;
  if (head_dim == 128 && m->rows == pkv::kMqRowUnit) {
    // such a batch may take the 256-row prefill units (bf16 caches): kPfMaxPieces records
    // of kMqPrefillUnit rows per (unit, kv head) item, the items' counters and the schedule
    int64_t items = 0, need = 0;
    const int64_t units = (int64_t{num_tokens} * G + pkv::kMqPrefillUnit - 1) / pkv::kMqPrefillUnit +
                          num_seqs;
    if (!mul_ok(units, num_kv_heads, INT64_MAX / 1024, &items) ||
        !mul_ok(items, pkv::prefill_words_per_item(), INT64_MAX / 1024, &need))
      return PKV_ERR_INVALID_ARG;
    need += num_seqs + 64;
    if (need > m->recs) m->recs = need;
  }
  m->plan_bytes = pkv::multi_plan_bytes(num_seqs, m->max_units);
  int64_t bytes = 0;
  if (!mul_ok(m->recs, int64_t{head_dim} + 2, INT64_MAX / 8, &bytes)) return PKV_ERR_INVALID_ARG;
  m->ws_bytes = m->plan_bytes + static_cast<size_t>(bytes) * 4;
  return PKV_OK;
}

void set_multi_workspace(pkv::AttentionArgs* a, void* workspace, const MultiShape& m,
                         int32_t num_seqs) {
  auto r256 = [](int64_t b) { return (b + 255) / 256 * 256; };
  char* ws = static_cast<char*>(workspace);
  a->tile_hdr = reinterpret_cast<int*>(ws);
  a->tile_cum = reinterpret_cast<int*>(ws + 256);
  a->unit_seq = reinterpret_cast<int*>(ws + 256 + r256((m.max_units + 1) * 4));
  a->seq_unit = reinterpret_cast<int*>(ws + 256 + r256((m.max_units + 1) * 4) +
                                        r256(m.max_units * 4));
  a->max_units = static_cast<int>(m.max_units);
  a->unit_rows = m.rows;
  float* f = reinterpret_cast<float*>(ws + m.plan_bytes);
  a->ws_m = f;
  a->ws_l = f + m.recs;
  a->ws_o = f + 2 * m.recs;
  (void)num_seqs;
}

}  // namespace

extern "C" {

pkv_status pkv_slot_mapping_multi_query(const int32_t* block_tables, const int32_t* context_lens,
                                        const int32_t* query_start_loc, int32_t* slot_mapping,
                                        int32_t num_seqs, int32_t num_tokens,
                                        int32_t max_blocks_per_seq, int32_t block_size,
                                        int64_t num_blocks, void* stream) {
  if (num_seqs < 0 || num_tokens < 0 || max_blocks_per_seq <= 0 || num_blocks <= 0)
    return PKV_ERR_INVALID_ARG;
  if (!is_pow2(block_size) || block_size > 1024) return PKV_ERR_INVALID_ARG;
  int64_t t = 0;
  if (!mul_ok(max_blocks_per_seq, block_size, INT32_MAX / 2, &t) ||
      !mul_ok(num_blocks, block_size, INT32_MAX, &t))
    return PKV_ERR_INVALID_ARG;   // slots are int32
  if (num_tokens == 0) return PKV_OK;
  if (num_seqs == 0) return PKV_ERR_INVALID_ARG;   // tokens need a sequence
  if (!block_tables || !context_lens || !query_start_loc || !slot_mapping)
    return PKV_ERR_INVALID_ARG;
  if (!aligned4(block_tables) || !aligned4(context_lens) || !aligned4(query_start_loc) ||
      !aligned4(slot_mapping))
    return PKV_ERR_INVALID_ARG;
  return hip_status(pkv::launch_slot_mapping_multi(
      block_tables, context_lens, query_start_loc, slot_mapping, num_seqs, num_tokens,
      max_blocks_per_seq, log2_exact(block_size), num_blocks, static_cast<hipStream_t>(stream)));
}

size_t pkv_paged_attention_multi_query_workspace_bytes(int32_t num_seqs, int32_t num_tokens,
                                                       int32_t num_heads, int32_t num_kv_heads,
                                                       int32_t head_dim, int32_t block_size,
                                                       int32_t max_blocks_per_seq) {
  MultiShape m;
  if (check_multi_shape(num_seqs, num_tokens, num_heads, num_kv_heads, head_dim, block_size,
                        max_blocks_per_seq, &m) != PKV_OK)
    return 0;
  return m.ws_bytes;
}

pkv_status pkv_paged_attention_multi_query(void* out, const void* query, const void* key_cache,
                                           const void* value_cache, const int32_t* block_tables,
                                           const int32_t* context_lens,
                                           const int32_t* query_start_loc, int32_t num_seqs,
                                           int32_t num_tokens, int32_t num_heads,
                                           int32_t num_kv_heads, int32_t head_dim,
                                           int32_t block_size, int32_t max_blocks_per_seq,
                                           int64_t num_blocks, float scale, pkv_dtype kv_dtype,
                                           pkv_dtype out_dtype, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  MultiShape m;
  pkv_status st = check_multi_shape(num_seqs, num_tokens, num_heads, num_kv_heads, head_dim,
                                    block_size, max_blocks_per_seq, &m);
  if (st != PKV_OK) return st;
  if (!valid_dtype(kv_dtype) || !valid_dtype(out_dtype)) return PKV_ERR_INVALID_ARG;
  if (num_blocks <= 0 || num_blocks > INT32_MAX || !std::isfinite(scale))
    return PKV_ERR_INVALID_ARG;
  int64_t pool = 0, rows = 0;
  if (!mul_ok(num_blocks, block_size, INT64_MAX / 4096, &pool) ||
      !mul_ok(pool, int64_t{num_kv_heads} * head_dim, INT64_MAX / 8, &pool))
    return PKV_ERR_INVALID_ARG;
  // query and output offsets are 32-bit in the kernels
  if (!mul_ok(num_tokens, int64_t{num_heads} * head_dim * elem_bytes(kv_dtype), INT32_MAX, &rows))
    return PKV_ERR_UNSUPPORTED;
  if (!(head_dim == 64 || head_dim == 128)) return PKV_ERR_UNSUPPORTED;
  if (!(block_size == 16 || block_size == 32)) return PKV_ERR_UNSUPPORTED;
  // grids: the merge runs max_units * num_kv_heads + num_tokens workgroups of 256
  // threads, the prefill units at most max_units * num_kv_heads (rounded up to 8) of 512
  const int64_t unit_items = m.max_units * num_kv_heads;
  if (unit_items + num_tokens > kMaxItems256 || (unit_items + 8) > int64_t{UINT32_MAX} / 512)
    return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (num_seqs == 0) return PKV_ERR_INVALID_ARG;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens ||
      !query_start_loc)
    return PKV_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache) ||
      !aligned4(block_tables) || !aligned4(context_lens) || !aligned4(query_start_loc) ||
      !aligned16(workspace))
    return PKV_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < m.ws_bytes) return PKV_ERR_WORKSPACE;
  pkv::AttentionArgs a{};
  a.out = out;
  a.query = query;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start_loc = query_start_loc;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_shift = log2_exact(block_size);
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  a.kv_bf16 = kv_dtype == PKV_BF16;
  a.out_bf16 = out_dtype == PKV_BF16;
  a.v_scale = 1.f;
  set_multi_workspace(&a, workspace, m, num_seqs);
  pkv::select_multi_mode(&a);
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = hip_status(pkv::launch_multi_plan(a, s));
  if (st != PKV_OK) return st;
  st = hip_status(pkv::launch_attention_multi(a, s));
  if (st != PKV_OK) return st;
  return hip_status(pkv::launch_attention_multi_reduce(a, s));
}

}  // extern "C"
