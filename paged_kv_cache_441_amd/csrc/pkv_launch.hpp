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

// E4M3 cache rows from fp32 or bfloat16 inputs divided by k_scale / v_scale.
hipError_t launch_cache_write_fp8(const void* key, const void* value, void* key_cache,
                                  void* value_cache, const int32_t* slot_mapping, int num_tokens,
                                  int row_elems, int64_t num_slots, bool in_bf16, float k_scale,
                                  float v_scale, hipStream_t stream);

// Builds the fixed-partition plan (plan_items, plan_count) or, when balanced, the
// tile plan (tile_cum, tile_hdr).  quant: 0 copies the new rows, 1 and 2 store the
// E4M3 codes of fp32 or bfloat16 rows (row_bytes are then the cache row's bytes).
hipError_t launch_decode_prologue(const int32_t* block_tables, const int32_t* context_lens,
                                  const void* key, const void* value, void* key_cache,
                                  void* value_cache, int32_t* slot_mapping, int num_seqs,
                                  int max_blocks_per_seq, int block_shift, int64_t num_blocks,
                                  int row_bytes, int partition_size, int4* plan_items,
                                  int* plan_count, bool balanced, int* tile_cum, int* tile_hdr,
                                  int quant, float k_scale, float v_scale, hipStream_t stream);

hipError_t launch_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs,
                              int num_pairs, int64_t block_bytes, int64_t num_blocks,
                              hipStream_t stream);

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
  bool kv_fp8;              // E4M3 caches (queries bfloat16); scale_log2 includes k_scale
  bool out_bf16;
  float v_scale;            // E4M3 caches: multiplies the value rows
  int* plan_count;          // number of work items in the plan
  int4* plan_items;         // [num_seqs * max_parts] (seq, partition, context length, partitions)
  float* ws_m;              // [num_seqs][num_heads][max_parts]
  float* ws_l;              // [num_seqs][num_heads][max_parts]
  float* ws_o;              // [num_seqs][num_heads][max_parts][head_dim]
  // Balanced mode (PKV_PARTITION_BALANCED): the tile plan, and the partial results of the
  // segments, one record row per (segment label, query head).
  bool balanced;
  // Fixed partitions in the per-head layout (one workgroup per kv head, partition and
  // sequence, loads through the caches) instead of the streaming kernel.
  bool per_head;
  int* tile_hdr;            // [0] total tiles, [1] workgroups per kv-head group
  int* tile_cum;            // [num_seqs + 1] tiles before each sequence
  // Multi-token steps: the flat token batch and the units of the work list (a unit is
  // one sequence's block of unit_rows (new token, query head) rows of one kv head).
  const int32_t* query_start_loc;   // [num_seqs + 1]
  int num_tokens;
  int unit_rows;            // 16, 32, kMqRowUnit or kMqPrefillUnit rows per unit
  int max_units;            // capacity of the unit arrays
  int grid_wgs;             // prefill units: workgroups of the launch (a multiple of 8)
  int* unit_seq;            // [max_units] sequence of each unit
  int* seq_unit;            // [num_seqs + 1] first unit of each sequence
};

// Multi-token steps: rows of one MFMA row block of (token, head) rows; a unit is one
// or two of them.
constexpr int kMqRows = 16;
// Multi-token steps with long prompts: waves of a workgroup that share one kv head,
// each taking kMqRowRB row blocks (a unit of kMqRowUnit rows).
constexpr int kMqRowWaves = 4;
#ifndef PKV_MULTI_ROW_RB
#define PKV_MULTI_ROW_RB 2
#endif
constexpr int kMqRowRB = PKV_MULTI_ROW_RB;   // row blocks per wave in that mode
constexpr int kMqRowUnit = kMqRowWaves * 16 * kMqRowRB;
// Long prompts with bf16 caches and 128-element heads: units of this many rows, one
// workgroup each over the unit's whole causal context (no split), when such units
// fill the GPU at least once.
constexpr int kMqPrefillUnit = 256;
// Prefill units split each (unit, kv head) item's context into up to kPfMaxPieces
// pieces, which write (m, l, o) records of their rows; the last one merges them.
// Workspace words per item in each of the m and l arrays: kPfMaxPieces records' rows,
// and two words of schedule (m array: per-XCD prefix sums and the plan's scan, at most
// one word per item each) or one counter (l array); the caller adds the ranked
// sequences and a little slack.
constexpr int kPfMaxPieces = 4;
constexpr int64_t prefill_words_per_item() { return kPfMaxPieces * kMqPrefillUnit + 2; }

// Balanced mode: at most this many workgroups per kv-head group, so segment labels
// (workgroup + sequence) stay below kMaxStreamWgs + num_seqs.
constexpr int kMaxStreamWgs = 1024;
// Balanced mode: tokens per tile of the tile list.
#ifndef PKV_TILE_TOKENS
#define PKV_TILE_TOKENS 16
#endif
constexpr int kTileTokens = PKV_TILE_TOKENS;
// Balanced mode: list positions charged per sequence on top of its tiles (the cost
// of starting and closing a sequence, in tiles).
#ifndef PKV_SEQ_COST
#define PKV_SEQ_COST 1
#endif
constexpr int kSeqCost = PKV_SEQ_COST;

// Workspace layout, in bytes from its start (all offsets 256-byte aligned):
//   plan: count (int32) at 0, items (int4) at 256;
//   then m, l and o records of the partitions (fp32).
size_t plan_bytes(int64_t num_seqs, int64_t max_parts);
// Balanced mode: header (256 bytes) and the tile prefix sums.
size_t tile_plan_bytes(int64_t num_seqs);

hipError_t launch_attention_plan(const AttentionArgs& a, hipStream_t stream);
hipError_t launch_attention_partition(const AttentionArgs& a, hipStream_t stream);
// Balanced mode: the tile plan, the streaming partition stage (whole token rows
// staged through LDS, equal shares of the tile list per workgroup) and its merge.
hipError_t launch_tile_plan(const AttentionArgs& a, hipStream_t stream);
hipError_t launch_attention_stream(const AttentionArgs& a, hipStream_t stream);
// Fixed partitions through the streaming kernel: one workgroup per plan item.
hipError_t launch_attention_stream_fixed(const AttentionArgs& a, hipStream_t stream);
hipError_t launch_attention_stream_reduce(const AttentionArgs& a, hipStream_t stream);
hipError_t launch_attention_reduce(const AttentionArgs& a, hipStream_t stream);

// Multi-token steps (several new tokens per sequence, causal within the step).
hipError_t launch_slot_mapping_multi(const int32_t* block_tables, const int32_t* context_lens,
                                     const int32_t* query_start_loc, int32_t* slot_mapping,
                                     int num_seqs, int num_tokens, int max_blocks_per_seq,
                                     int block_shift, int64_t num_blocks, hipStream_t stream);
// Workspace of a multi-token step: plan header (256 B), then the unit plan arrays,
// each rounded up to 256 bytes; the records follow.
size_t multi_plan_bytes(int64_t num_seqs, int64_t max_units);
// Picks the unit shape for the arguments (possibly the prefill units), before the plan.
void select_multi_mode(AttentionArgs* a);
hipError_t launch_multi_plan(const AttentionArgs& a, hipStream_t stream);
hipError_t launch_attention_multi(const AttentionArgs& a, hipStream_t stream);
hipError_t launch_attention_multi_reduce(const AttentionArgs& a, hipStream_t stream);

}  // namespace pkv
