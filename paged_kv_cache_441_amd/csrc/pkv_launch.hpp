// Host-side launchers of the libpagedkv kernels.  Arguments are checked by the
// C ABI layer (pkv_api.cpp) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

hipError_t launch_slot_mapping(const int32_t* block_tables, const int32_t* context_lens,
                               int32_t* slot_mapping, int num_seqs, int max_blocks_per_seq,
                               int block_shift, int64_t num_blocks, hipStream_t stream);

hipError_t launch_cache_write(const void* key, const void* value, void* key_cache,
                              void* value_cache, const int32_t* slot_mapping, int num_tokens,
                              int row_bytes, int64_t num_slots, hipStream_t stream);

hipError_t launch_decode_prologue(const int32_t* block_tables, const int32_t* context_lens,
                                  const void* key, const void* value, void* key_cache,
                                  void* value_cache, int32_t* slot_mapping, int num_seqs,
                                  int max_blocks_per_seq, int block_shift, int64_t num_blocks,
                                  int row_bytes, int partition_size, int4* plan_items,
                                  int* plan_count, hipStream_t stream);

struct AttentionArgs {
  void* out;
  const void* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int head_dim;
  int block_shift;          // log2(block_size)
  int max_blocks_per_seq;
  int64_t num_blocks;
  float scale_log2;         // scale * log2(e): scores live in the base-2 exponent domain
  int partition_size;
  int max_parts;            // ceil(max_blocks_per_seq * block_size / partition_size)
  bool kv_bf16;
  bool out_bf16;
  int* plan_count;          // number of work items in the plan
  int4* plan_items;         // [num_seqs * max_parts] (seq, partition, context length, partitions)
  float* ws_m;              // [num_seqs][num_heads][max_parts]
  float* ws_l;              // [num_seqs][num_heads][max_parts]
  float* ws_o;              // [num_seqs][num_heads][max_parts][head_dim]
};

// Workspace layout, in bytes from its start (all offsets 256-byte aligned):
//   plan: count (int32) at 0, items (int4) at 256;
//   then m, l and o records of the partitions (fp32).
size_t plan_bytes(int64_t num_seqs, int64_t max_parts);

hipError_t launch_attention_plan(const AttentionArgs& a, hipStream_t stream);
hipError_t launch_attention_partition(const AttentionArgs& a, hipStream_t stream);
hipError_t launch_attention_reduce(const AttentionArgs& a, hipStream_t stream);

}  // namespace pkv
