// Slot mapping and the cache write (reshape_and_cache) for gfx950.
//
// A token at 0-based position pos of a sequence lies in logical block
// pos / block_size at offset pos % block_size; its cache slot is
// physical_block * block_size + offset (page "vllm源码剖析", section 一.3, the
// worked example of a token's offset).  With the cache viewed as
// [num_blocks * block_size][num_kv_heads][head_dim] (same page, section 一.2 on
// the reshaped cache), a token's K (or V) for all heads is one contiguous row at
// slot * num_kv_heads * head_dim, so the write is a row copy per token.
#include "pkv_device.hpp"
#include "pkv_launch.hpp"
#include "pkv_plan.hpp"

namespace pkv {

// Slot of sequence i's new token, or -1 for an invalid length or block id.
__device__ __forceinline__ int32_t slot_of(const int32_t* __restrict__ block_tables,
                                           const int32_t* __restrict__ context_lens, int i,
                                           int max_blocks_per_seq, int block_shift,
                                           int64_t num_blocks) {
  const int ctx = context_lens[i];
  const int block_size = 1 << block_shift;
  if (ctx < 1 || ctx > max_blocks_per_seq * block_size) return -1;
  const int pos = ctx - 1;
  const int logical = pos >> block_shift;
  const int offset = pos & (block_size - 1);
  const int32_t physical = block_tables[(int64_t)i * max_blocks_per_seq + logical];
  if (physical < 0 || (int64_t)physical >= num_blocks) return -1;
  return physical * block_size + offset;
}

__global__ __launch_bounds__(256) void slot_mapping_kernel(
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    int32_t* __restrict__ slot_mapping, int num_seqs, int max_blocks_per_seq,
    int block_shift, int64_t num_blocks) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= num_seqs) return;
  slot_mapping[i] = slot_of(block_tables, context_lens, i, max_blocks_per_seq, block_shift,
                            num_blocks);
}

// One workgroup per token: copy the token's K row and V row (num_kv_heads*head_dim
// elements each, a multiple of 16 bytes) in 16-byte pieces.
__global__ __launch_bounds__(256) void cache_write_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value,
    uint4* __restrict__ key_cache, uint4* __restrict__ value_cache,
    const int32_t* __restrict__ slot_mapping, int chunks_per_row, int64_t num_slots) {
  const int t = blockIdx.x;
  const int32_t slot = slot_mapping[t];
  if (slot < 0 || (int64_t)slot >= num_slots) return;
  const int64_t src = (int64_t)t * chunks_per_row;
  const int64_t dst = (int64_t)slot * chunks_per_row;
  for (int c = threadIdx.x; c < 2 * chunks_per_row; c += blockDim.x) {
    if (c < chunks_per_row) {
      key_cache[dst + c] = key[src + c];
    } else {
      value_cache[dst + c - chunks_per_row] = value[src + c - chunks_per_row];
    }
  }
}

// The input words behind cache piece g of a row (16 bytes of cache): one chunk for a
// bit copy (quant 0), four fp32 chunks (quant 1) or two bfloat16 chunks (quant 2).
__device__ __forceinline__ void load_piece(const void* src, int64_t g, int quant,
                                           uint4 (&w)[4]) {
  const uint4* p = static_cast<const uint4*>(src);
  if (quant == 0) {
    w[0] = p[g];
  } else if (quant == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = p[4 * g + i];
  } else {
    w[0] = p[2 * g];
    w[1] = p[2 * g + 1];
  }
}

// The cache piece for loaded input words: the words themselves (quant 0), else the
// E4M3 codes of x / scale (the quotient rounded to fp32, then to E4M3) for their 16
// elements.
__device__ __forceinline__ uint4 encode_piece(const uint4 (&w)[4], int quant, float scale) {
  if (quant == 0) return w[0];
  float x[16];
  if (quant == 2) {
    unpack_chunk<BF16>(w[0], x);
    unpack_chunk<BF16>(w[1], x + 8);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) unpack_chunk<F32>(w[i], x + 4 * i);
  }
  uint32_t c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[i] = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) c[i] |= e4m3_encode(__fdiv_rn(x[4 * i + j], scale)) << (8 * j);
  }
  return make_uint4(c[0], c[1], c[2], c[3]);
}

// Token t's K and V rows into cache slot `slot`, each cache row `chunks` 16-byte
// chunks: a bit copy (quant 0) or the E4M3 codes of fp32 (quant 1) or bfloat16
// (quant 2) inputs.  The workgroup's threads share the 2 * chunks pieces.
__device__ __forceinline__ void store_token(const void* key, const void* value, void* key_cache,
                                            void* value_cache, int64_t t, int64_t slot,
                                            int chunks, int quant, float k_scale, float v_scale) {
  const int64_t src = t * chunks, dst = slot * chunks;
  for (int c = threadIdx.x; c < 2 * chunks; c += blockDim.x) {
    const bool is_k = c < chunks;
    const int64_t cc = is_k ? c : c - chunks;
    uint4 w[4];
    load_piece(is_k ? key : value, src + cc, quant, w);
    static_cast<uint4*>(is_k ? key_cache : value_cache)[dst + cc] =
        encode_piece(w, quant, is_k ? k_scale : v_scale);
  }
}

// One workgroup per token: the E4M3 codes of the token's K and V rows.
__global__ __launch_bounds__(256) void cache_write_fp8_kernel(
    const void* __restrict__ key, const void* __restrict__ value, void* __restrict__ key_cache,
    void* __restrict__ value_cache, const int32_t* __restrict__ slot_mapping, int chunks_per_row,
    int64_t num_slots, int quant, float k_scale, float v_scale) {
  const int t = blockIdx.x;
  const int32_t slot = slot_mapping[t];
  if (slot < 0 || (int64_t)slot >= num_slots) return;
  store_token(key, value, key_cache, value_cache, t, slot, chunks_per_row, quant, k_scale,
              v_scale);
}

// The decode step's prologue in one launch: workgroup 0 builds the attention plan
// while workgroup 1 + i computes sequence i's slot and stores its new K/V rows.
constexpr int kPrologueThreads = 256;

__global__ __launch_bounds__(kPrologueThreads) void decode_prologue_kernel(
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    const void* __restrict__ key, const void* __restrict__ value, void* __restrict__ key_cache,
    void* __restrict__ value_cache, int32_t* __restrict__ slot_mapping, int num_seqs,
    int max_blocks_per_seq, int block_shift, int64_t num_blocks, int chunks_per_row,
    int partition_size, int4* __restrict__ plan_items, int* __restrict__ plan_count,
    bool balanced, int* __restrict__ tile_cum, int* __restrict__ tile_hdr, int quant,
    float k_scale, float v_scale) {
  if (blockIdx.x == 0) {
    if (balanced)
      build_tile_plan<kPrologueThreads>(context_lens, num_seqs, max_blocks_per_seq << block_shift,
                                        tile_cum, tile_hdr);
    else
      build_plan<kPrologueThreads>(context_lens, num_seqs, partition_size,
                                   max_blocks_per_seq << block_shift, plan_items, plan_count);
    return;
  }
  const int t = blockIdx.x - 1;
  const int chunks = chunks_per_row;
  if (2 * chunks > kPrologueThreads) {
    const int32_t slot = slot_of(block_tables, context_lens, t, max_blocks_per_seq, block_shift,
                                 num_blocks);
    if (threadIdx.x == 0) slot_mapping[t] = slot;
    if (slot < 0) return;
    store_token(key, value, key_cache, value_cache, t, slot, chunks, quant, k_scale, v_scale);
    return;
  }
  // Both rows fit one pass: each thread loads its input piece before the slot is
  // known (the input does not depend on it), so these loads are in flight during the
  // two dependent reads of the slot computation.
  const int c = threadIdx.x;
  const bool live = c < 2 * chunks;
  const bool is_k = c < chunks;
  const int64_t cc = is_k ? c : c - chunks;
  uint4 w[4];
  if (live) load_piece(is_k ? key : value, (int64_t)t * chunks + cc, quant, w);
  const int32_t slot = slot_of(block_tables, context_lens, t, max_blocks_per_seq, block_shift,
                               num_blocks);
  if (threadIdx.x == 0) slot_mapping[t] = slot;
  if (slot < 0 || !live) return;
  static_cast<uint4*>(is_k ? key_cache : value_cache)[(int64_t)slot * chunks + cc] =
      encode_piece(w, quant, is_k ? k_scale : v_scale);
}

hipError_t launch_decode_prologue(const int32_t* block_tables, const int32_t* context_lens,
                                  const void* key, const void* value, void* key_cache,
                                  void* value_cache, int32_t* slot_mapping, int num_seqs,
                                  int max_blocks_per_seq, int block_shift, int64_t num_blocks,
                                  int row_bytes, int partition_size, int4* plan_items,
                                  int* plan_count, bool balanced, int* tile_cum, int* tile_hdr,
                                  int quant, float k_scale, float v_scale, hipStream_t stream) {
  hipLaunchKernelGGL(decode_prologue_kernel, dim3(num_seqs + 1), dim3(kPrologueThreads), 0, stream,
                     block_tables, context_lens, key, value, key_cache, value_cache, slot_mapping,
                     num_seqs, max_blocks_per_seq, block_shift, num_blocks, row_bytes / 16,
                     partition_size, plan_items, plan_count, balanced, tile_cum, tile_hdr, quant,
                     k_scale, v_scale);
  return hipGetLastError();
}

hipError_t launch_slot_mapping(const int32_t* block_tables, const int32_t* context_lens,
                               int32_t* slot_mapping, int num_seqs, int max_blocks_per_seq,
                               int block_shift, int64_t num_blocks, hipStream_t stream) {
  const int threads = 256;
  const int grid = (num_seqs + threads - 1) / threads;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(grid), dim3(threads), 0, stream, block_tables,
                     context_lens, slot_mapping, num_seqs, max_blocks_per_seq, block_shift,
                     num_blocks);
  return hipGetLastError();
}

hipError_t launch_cache_write(const void* key, const void* value, void* key_cache,
                              void* value_cache, const int32_t* slot_mapping, int num_tokens,
                              int row_bytes, int64_t num_slots, hipStream_t stream) {
  const int chunks = row_bytes / 16;
  const int threads = chunks * 2 >= 256 ? 256 : ((chunks * 2 + 63) / 64) * 64;
  hipLaunchKernelGGL(cache_write_kernel, dim3(num_tokens), dim3(threads), 0, stream,
                     static_cast<const uint4*>(key), static_cast<const uint4*>(value),
                     static_cast<uint4*>(key_cache), static_cast<uint4*>(value_cache),
                     slot_mapping, chunks, num_slots);
  return hipGetLastError();
}

hipError_t launch_cache_write_fp8(const void* key, const void* value, void* key_cache,
                                  void* value_cache, const int32_t* slot_mapping, int num_tokens,
                                  int row_elems, int64_t num_slots, bool in_bf16, float k_scale,
                                  float v_scale, hipStream_t stream) {
  const int chunks = row_elems / 16;
  const int threads = chunks * 2 >= 256 ? 256 : ((chunks * 2 + 63) / 64) * 64;
  hipLaunchKernelGGL(cache_write_fp8_kernel, dim3(num_tokens), dim3(threads), 0, stream, key,
                     value, key_cache, value_cache, slot_mapping, chunks, num_slots,
                     in_bf16 ? 2 : 1, k_scale, v_scale);
  return hipGetLastError();
}

// ---- block copies (copy-on-write) -------------------------------------------------
// For every (src, dst) pair, block dst of both caches becomes a copy of block src.
// Workgroup (p, c) copies chunk c (kCopyChunk bytes) of pair p's blocks: every lane
// loads all of its 16-byte pieces of both caches before it stores any.  Pairs with
// an id outside the pool are skipped.  Pairs run in parallel: the caller's contract
// is that no dst repeats and no dst is also a src.
//
// The pieces are native 4 x u32 vectors, and the loads are never conditional: a piece
// past the block's end (only in a block whose size is not a multiple of kCopyChunk)
// re-reads the block's last piece and is not stored.  With conditional loads into an
// array of the struct-typed uint4, the compiler moved the array to LDS and scratch
// memory, and the scratch round trip cost half as much HBM traffic again as the copy.
// The stores are non-temporal: the copied blocks are not read again by this launch,
// and on MI355X (4096 random 32 KiB block pairs of both caches) this took a launch
// from 115 to 85 us.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kCopyThreads = 256;
constexpr int kCopyPer = 4;                            // pieces per lane per cache
constexpr int kCopyChunk = kCopyThreads * kCopyPer * 16;

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    u32x4* __restrict__ key_cache, u32x4* __restrict__ value_cache,
    const int32_t* __restrict__ pairs, int64_t block_chunks, int64_t num_blocks) {
  const int p = blockIdx.x;
  const int32_t src = pairs[2 * p];
  const int32_t dst = pairs[2 * p + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const int64_t c0 = (int64_t)blockIdx.y * (kCopyChunk / 16) + threadIdx.x;
  const int64_t s = (int64_t)src * block_chunks, d = (int64_t)dst * block_chunks;
  u32x4 k[kCopyPer], v[kCopyPer];
#pragma unroll
  for (int i = 0; i < kCopyPer; ++i) {
    const int64_t c = min(c0 + i * kCopyThreads, block_chunks - 1);
    k[i] = key_cache[s + c];
    v[i] = value_cache[s + c];
  }
#pragma unroll
  for (int i = 0; i < kCopyPer; ++i) {
    const int64_t c = c0 + i * kCopyThreads;
    if (c < block_chunks) {
      __builtin_nontemporal_store(k[i], key_cache + d + c);
      __builtin_nontemporal_store(v[i], value_cache + d + c);
    }
  }
}

hipError_t launch_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs,
                              int num_pairs, int64_t block_bytes, int64_t num_blocks,
                              hipStream_t stream) {
  const dim3 grid((unsigned)num_pairs, (unsigned)((block_bytes + kCopyChunk - 1) / kCopyChunk));
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kCopyThreads), 0, stream,
                     static_cast<u32x4*>(key_cache), static_cast<u32x4*>(value_cache), pairs,
                     block_bytes / 16, num_blocks);
  return hipGetLastError();
}

}  // namespace pkv
