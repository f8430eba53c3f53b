/*
 * pagedkv.h -- C ABI of libpagedkv.so: the PagedAttention decode step on AMD
 * Instinct MI355X (gfx950).
 *
 * The decode step of a batch of sequences, each with one new token:
 *   1. pkv_slot_mapping            -- where each new token goes in the paged cache;
 *   2. pkv_kv_cache_write          -- scatter the new tokens' K/V rows there
 *                                     (reshape_and_cache);
 *   3. pkv_paged_attention_decode  -- attention of each sequence's query over its
 *                                     whole paged context, split into pieces that
 *                                     are merged by log-sum-exp (= the plan, the
 *                                     partition and the reduce stages below).
 *
 * Two ways to split the contexts, chosen by partition_size:
 *  - partition_size P > 0 (fixed partitions): sequence i is cut into partitions of
 *    P tokens; one workgroup per (sequence, partition) and group of kv heads, which
 *    streams whole token rows of its heads through LDS; longest partitions first.
 *    partition_size PKV_PARTITION_DEFAULT (0) means P = PKV_DEFAULT_PARTITION_TOKENS
 *    (512).  A sequence's result depends only on its own data and P.
 *  - partition_size PKV_PARTITION_BALANCED (-1): the (sequence, 16-token tile) pairs
 *    of the whole batch, plus one position per sequence for its fixed cost, form one
 *    list that is cut into equal contiguous shares, one per workgroup of a grid the
 *    GPU holds at once; each workgroup streams whole token rows of its kv-head group
 *    through LDS.  Where the pieces of a sequence end therefore depends on the
 *    whole batch (and on the GPU's compute-unit count), so a sequence's result
 *    may differ between batches in the last bits of fp32; for one batch on one
 *    GPU it is deterministic.  It is the faster split when context lengths vary
 *    widely.
 * Other negative values are PKV_ERR_INVALID_ARG.
 *
 * Cache layout (both key_cache and value_cache), row-major, no padding:
 *     [num_blocks][block_size][num_kv_heads][head_dim]
 * Viewed with the first two dimensions merged, every cache "slot"
 * (= physical_block * block_size + offset) is one token's contiguous row of
 * num_kv_heads * head_dim elements.  (Page "vllm源码剖析", section 一.2, the
 * paragraph on why the cache is reshaped: [num_blocks, block_size, num_kv_heads,
 * head_size] with the first two dimensions merged so that a token's data is
 * contiguous.)
 *
 * Conventions shared by every entry point:
 *  - Pointers named as device buffers are device (HBM) addresses owned by the
 *    caller; the library never allocates, frees or retains them.  Its only global
 *    state is per-device facts looked up once (the compute-unit count, the address of
 *    pkv_paged_attention_decode_noalloc's scratch array); the entry points are
 *    reentrant, with the overlap rule of that scratch array stated at its entry.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Work is
 *    only enqueued on it; no call synchronises the host.  Ordering (write before
 *    attention) is the caller's, by using one stream.
 *  - Integer tensors are int32, row-major.  Element types are pkv_dtype.
 *  - Alignment: buffers of rows (caches, queries, keys, values, outputs, workspaces,
 *    block-pair lists excepted) start on 16-byte boundaries, int32 arrays on 4-byte
 *    ones; a misaligned pointer is PKV_ERR_INVALID_ARG.
 *  - Errors come back as a pkv_status, never as an abort or exception.  Every
 *    argument check happens before any GPU work is enqueued, so a call that
 *    returns an error other than PKV_ERR_HIP has touched nothing.
 *  - A sequence's context length counts its new token: the new token sits at
 *    0-based position context_len - 1.
 */
#ifndef PAGEDKV_H_
#define PAGEDKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 7   /* 7: multi-token workspace sized for context pieces */

/* partition_size values with a name (see above) */
#define PKV_PARTITION_DEFAULT 0            /* fixed partitions of 512 tokens */
#define PKV_DEFAULT_PARTITION_TOKENS 512
#define PKV_PARTITION_BALANCED (-1)        /* the balanced split */

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,  /* null pointer, non-positive size, inconsistent shapes */
  PKV_ERR_UNSUPPORTED = 2,  /* a valid combination the library has no kernel for */
  PKV_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
  PKV_ERR_HIP = 4,          /* the HIP runtime reported an error at launch */
  PKV_ERR_NO_BLOCKS = 5,    /* the block pool has no free block left */
  PKV_ERR_SCRATCH_LIMIT = 6 /* more scratch than the no-alloc entry point's fixed buffer */
} pkv_status;

typedef enum {
  PKV_F32 = 0,      /* IEEE binary32 */
  PKV_BF16 = 1,     /* bfloat16 (top 16 bits of a binary32) */
  PKV_FP8_E4M3 = 2, /* OCP 8-bit float E4M3 (cache storage only; see the FP8 section) */
  /* Not types: these two make every int32 value a value of pkv_dtype, so that an
   * unknown code passed by a caller is rejected (PKV_ERR_INVALID_ARG) rather than
   * being an out-of-range enumeration value. */
  PKV_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  PKV_DTYPE_RANGE_MAX_ = 2147483647
} pkv_dtype;

/* PKV_ABI_VERSION of the loaded library. */
int32_t pkv_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* pkv_status_string(int32_t status);

/*
 * pkv_slot_mapping -- slot of each sequence's new token.
 *
 * Defines: position pos = context_lens[i] - 1 lies in logical block
 * pos / block_size at offset pos % block_size; the block table maps the logical
 * block to a physical one and
 *     slot_mapping[i] = block_tables[i][pos / block_size] * block_size + pos % block_size.
 * (Page "vllm源码剖析", section 一.3, the worked example of a token's offset:
 * block size 4, tokens 1-4 in block 0 and 5-8 in block 1, offset by the modulus.)
 *
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq], physical block ids
 *   context_lens  device int32 [num_seqs]
 *   slot_mapping  device int32 [num_seqs], written
 *   num_blocks    pool size; used to recognise invalid ids
 *
 * A sequence whose context length is outside [1, max_blocks_per_seq*block_size],
 * or whose target block id is outside [0, num_blocks), gets slot -1 (which
 * pkv_kv_cache_write skips).  num_seqs == 0 is a no-op.
 * block_size must be a power of two in [1, 1024].
 */
pkv_status pkv_slot_mapping(const int32_t* block_tables, const int32_t* context_lens,
                            int32_t* slot_mapping, int32_t num_seqs,
                            int32_t max_blocks_per_seq, int32_t block_size,
                            int64_t num_blocks, void* stream);

/*
 * pkv_kv_cache_write -- reshape_and_cache: store each new token's K and V rows.
 *
 * For every token t with 0 <= slot_mapping[t] < num_blocks*block_size:
 *     key_cache  [slot / block_size][slot % block_size][:][:] = key  [t][:][:]
 *     value_cache[slot / block_size][slot % block_size][:][:] = value[t][:][:]
 * as a bit copy.  Tokens with a negative slot are padding and are skipped; slots
 * at or past the end of the pool are skipped as well (never written).  Two tokens
 * with the same slot are a caller error (which one lands is unspecified).
 * (Page "vllm源码剖析", section 一.2 on the reshaped cache; page "vLLM
 * PagedAttention 原理与源码深度解析", section 3.3, writing a token into the
 * sequence's last block.)
 *
 *   key, value              device [num_tokens][num_kv_heads][head_dim], kv_dtype
 *   key_cache, value_cache  device [num_blocks][block_size][num_kv_heads][head_dim]
 *   slot_mapping            device int32 [num_tokens]
 *
 * Any head_dim with num_kv_heads*head_dim*sizeof(kv_dtype) a multiple of 16 bytes
 * is accepted; kv_dtype may be PKV_FP8_E4M3 (codes copied as they are).
 * num_tokens == 0 is a no-op.
 */
pkv_status pkv_kv_cache_write(const void* key, const void* value, void* key_cache,
                              void* value_cache, const int32_t* slot_mapping,
                              int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int64_t num_blocks, pkv_dtype kv_dtype,
                              void* stream);

/*
 * ---- The block pool (host) and block copies (device) -----------------------------
 *
 * The pool owns the ids 0 .. num_blocks-1 of the physical KV blocks: a first-in
 * first-out list of free ids and a reference count per block.  (Page
 * "vllm源码分析：我是如何一步步读懂PagedAttention核心实现的？", 第一讲, the
 * BlockAllocator: allocation takes the first free id and sets its count to 1, an
 * empty list is an error, a block goes back to the end of the list when its count
 * drops to 0; page "读一个真实 serving 系统 · vLLM 架构巡礼": sequences that share a
 * prefix point at the same blocks, the shared count is above one, and a shared block
 * is copied before it is changed.)  The pool lives in host memory, owned by the
 * library between create and destroy; it is not thread-safe (callers serialise the
 * calls on one pool).  Block tables passed to it are host int32 arrays owned by the
 * caller.
 *
 * pkv_block_pool_allocate   takes one free block (count 1); PKV_ERR_NO_BLOCKS if none.
 * pkv_block_pool_release    drops one reference to each listed block (a block may be
 *                           listed several times); blocks reaching 0 go back to the
 *                           free list in list order.  INVALID_ARG, with nothing
 *                           changed, if an id is out of range or would drop below 0.
 * pkv_block_pool_fork       adds one reference to each listed block: a forked
 *                           sequence's table is a copy of its parent's (the caller
 *                           copies it).  INVALID_ARG, nothing changed, for an id out
 *                           of range or not in use.
 * pkv_block_pool_num_free   free blocks (-1 for a null pool).
 * pkv_block_pool_ref_count  a block's count (-1 for a bad id or a null pool).
 *
 * pkv_block_pool_append_slots -- the slot of each sequence's next token, in sequence
 * order.  Sequence i has num_tokens[i] tokens and the table
 * tables[i*table_capacity .. +table_lens[i]) (ceil(num_tokens[i] / block_size) ids).
 * Its next token, at position n = num_tokens[i]:
 *   - n % block_size == 0: a new block is allocated and appended to the table;
 *   - otherwise it goes into the last block; if that block is shared (count > 1) a
 *     fresh block is allocated, the pair (old, fresh) is appended to `copies`
 *     (int32 [num_seqs][2], host), one reference to the old block is dropped and the
 *     fresh block replaces it in the table.
 * slots[i] = table[n / block_size] * block_size + n % block_size.  (Page "vLLM
 * PagedAttention 原理与源码深度解析", sections 3.3 and 5.2: a full last block means a new
 * block; the page's sketch writes into the old block after allocating a new one,
 * while here the token goes to the block that holds its position.)  The copies must
 * be done (pkv_copy_blocks) before the new tokens are written.  *done receives the
 * number of sequences handled; on PKV_ERR_NO_BLOCKS or INVALID_ARG the sequences
 * before *done have been updated and the rest have not.
 *
 * pkv_copy_blocks -- for each (src, dst) in pairs (device int32 [num_pairs][2]), block
 * dst of key_cache and value_cache becomes a bitwise copy of block src.  Pairs run
 * in parallel: no dst may repeat or also be a src (copy-on-write pairs from one
 * pkv_block_pool_append_slots call satisfy this).  Pairs with an id outside
 * [0, num_blocks) are skipped.
 */
typedef struct pkv_block_pool pkv_block_pool;

pkv_status pkv_block_pool_create(int32_t num_blocks, pkv_block_pool** pool);
void pkv_block_pool_destroy(pkv_block_pool* pool);
int32_t pkv_block_pool_num_free(const pkv_block_pool* pool);
int32_t pkv_block_pool_ref_count(const pkv_block_pool* pool, int32_t block);
pkv_status pkv_block_pool_allocate(pkv_block_pool* pool, int32_t* block);
pkv_status pkv_block_pool_release(pkv_block_pool* pool, const int32_t* blocks, int32_t n);
pkv_status pkv_block_pool_fork(pkv_block_pool* pool, const int32_t* blocks, int32_t n);
pkv_status pkv_block_pool_append_slots(pkv_block_pool* pool, int32_t* tables,
                                       int32_t* table_lens, int32_t table_capacity,
                                       const int32_t* num_tokens, int32_t num_seqs,
                                       int32_t block_size, int32_t* slots, int32_t* copies,
                                       int32_t* num_copies, int32_t* done);

/*
 * ---- Prefix caching on the pool (host) ---------------------------------------------
 *
 * Full blocks of a sequence can be entered into a hash-to-block map and reused by
 * later requests that start with the same tokens.  (Page "vllm源码剖析", the BlockPool
 * paragraphs: a logical block's hash is computed from its token content and its
 * predecessor's hash, cached_block_hash_to_block maps it to the block, a hit only
 * raises the block's count, and a block whose count reaches 0 rejoins the free queue
 * with its hash, which is cleared when the block is handed out again; page "读一个真实
 * serving 系统 · vLLM 架构巡礼", section 2: _block_hash and touch().)  Choices the pages
 * leave open: the hash is 64-bit FNV-1a over the parent hash (8 bytes, little-endian,
 * 0 for the first block) followed by the block's token ids (int32, 4 bytes each,
 * little-endian); a hit also compares the stored tokens and parent hash, so a hash
 * collision never shares a block.  Token arrays are host int32 arrays owned by the
 * caller; only full blocks (num_tokens / block_size of them) take part.  The first
 * call fixes the pool's block size; a later call with another one is INVALID_ARG.
 *
 * pkv_prefix_block_hashes       hashes[j] (host uint64) of every full block j.
 * pkv_block_pool_match_prefix   the longest run of leading full blocks found in the
 *                               map (at most max_blocks), written to blocks (host
 *                               int32); each gets one more reference and, if it was
 *                               free, leaves the free list.
 * pkv_block_pool_register_prefix  enters the full blocks of a sequence whose K/V are
 *                               stored in table[0 .. num_tokens / block_size) (blocks
 *                               in use); a block already cached, or a hash already
 *                               mapped to another block, is left as it is.
 *                               INVALID_ARG, nothing changed, for a block not in use.
 * pkv_block_pool_num_cached     hashes in the map (-1 for a null pool).
 * pkv_block_pool_allocate (and append_slots) take the front of the free list as
 * before; a cached block taken there leaves the map.
 */
pkv_status pkv_prefix_block_hashes(const int32_t* tokens, int32_t num_tokens,
                                   int32_t block_size, uint64_t* hashes);
int32_t pkv_block_pool_num_cached(const pkv_block_pool* pool);
pkv_status pkv_block_pool_match_prefix(pkv_block_pool* pool, const int32_t* tokens,
                                       int32_t num_tokens, int32_t block_size,
                                       int32_t* blocks, int32_t max_blocks, int32_t* num_hit);
pkv_status pkv_block_pool_register_prefix(pkv_block_pool* pool, const int32_t* tokens,
                                          int32_t num_tokens, int32_t block_size,
                                          const int32_t* table, int32_t table_len,
                                          int32_t* num_registered);

pkv_status pkv_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs,
                           int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int64_t num_blocks, pkv_dtype kv_dtype,
                           void* stream);

/*
 * ---- FP8 (E4M3) caches -------------------------------------------------------------
 *
 * A KV cache of 8-bit floats (page "vLLM PagedAttention 原理与源码深度解析", section
 * 8.4, names an fp8 KV cache as a serving option; the pages fix neither the format
 * nor the scaling, so these are this library's choices):
 *  - format: OCP E4M3 -- sign, 4 exponent bits biased by 7, 3 mantissa bits; no
 *    infinities; S.1111.111 is NaN; the largest finite magnitude is 448; exponent
 *    field 0 holds the subnormals m * 2^-9;
 *  - one fp32 scale per cache (k_scale, v_scale, positive and finite): the cache
 *    element e stands for decode(e) * scale;
 *  - writing x stores E4M3(x / scale): the quotient rounded to fp32, then to the
 *    nearest E4M3 value with ties to the even code; magnitudes of 448 and beyond
 *    saturate to +-448 and NaN is stored as 0x7F.
 * The cache layout is the one above with one byte per element.
 *
 * pkv_kv_cache_write_fp8 -- pkv_kv_cache_write storing the codes of fp32 or bf16
 * (in_dtype) rows; num_kv_heads*head_dim must be a multiple of 16.
 *
 * pkv_decode_prologue_fp8 -- pkv_decode_prologue storing codes as above; it builds
 * the balanced-split plan (partition_size PKV_PARTITION_BALANCED).
 *
 * pkv_paged_attention_decode_fp8 -- pkv_paged_attention_decode over E4M3 caches:
 * scores scale * k_scale * <q, decode(k_t)>, output sum_t p_t v_scale decode(v_t) /
 * sum_t p_t.  Decoding is exact (every E4M3 value is a bfloat16); queries are bf16;
 * accumulation is fp32.  Always the balanced split: the workspace is
 * pkv_paged_attention_workspace_bytes(..., PKV_PARTITION_BALANCED), and the staged
 * form is pkv_paged_attention_plan and pkv_paged_attention_reduce with partition_size
 * PKV_PARTITION_BALANCED around pkv_paged_attention_partition_fp8.  Supported: head_dim 64 (with an even
 * num_kv_heads) or 128, block_size 16 or 32, num_heads / num_kv_heads in {1, 2, 4,
 * 8}, out_dtype PKV_F32 or PKV_BF16.  The device-side contract (NaN rows for a bad
 * context length or block id) is that of pkv_paged_attention_decode.  The unscaled
 * attention entry points reject PKV_FP8_E4M3 with PKV_ERR_INVALID_ARG.
 */
pkv_status pkv_kv_cache_write_fp8(const void* key, const void* value, void* key_cache,
                                  void* value_cache, const int32_t* slot_mapping,
                                  int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int64_t num_blocks, pkv_dtype in_dtype,
                                  float k_scale, float v_scale, void* stream);

pkv_status pkv_decode_prologue_fp8(const int32_t* block_tables, const int32_t* context_lens,
                                   const void* key, const void* value, void* key_cache,
                                   void* value_cache, int32_t* slot_mapping, int32_t num_seqs,
                                   int32_t max_blocks_per_seq, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                   pkv_dtype in_dtype, float k_scale, float v_scale,
                                   void* workspace, size_t workspace_bytes, void* stream);

pkv_status pkv_paged_attention_decode_fp8(void* out, const void* query, const void* key_cache,
                                          const void* value_cache, const int32_t* block_tables,
                                          const int32_t* context_lens, int32_t num_seqs,
                                          int32_t num_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t block_size,
                                          int32_t max_blocks_per_seq, int64_t num_blocks,
                                          float scale, float k_scale, float v_scale,
                                          pkv_dtype out_dtype, void* workspace,
                                          size_t workspace_bytes, void* stream);

pkv_status pkv_paged_attention_partition_fp8(void* out, const void* query,
                                             const void* key_cache, const void* value_cache,
                                             const int32_t* block_tables,
                                             const int32_t* context_lens, int32_t num_seqs,
                                             int32_t num_heads, int32_t num_kv_heads,
                                             int32_t head_dim, int32_t block_size,
                                             int32_t max_blocks_per_seq, int64_t num_blocks,
                                             float scale, float k_scale, float v_scale,
                                             pkv_dtype out_dtype, void* workspace,
                                             size_t workspace_bytes, void* stream);

/*
 * ---- Steps with several new tokens per sequence -------------------------------------
 *
 * Chunked prefill and the verification of speculated tokens hand each sequence a
 * number of new tokens in one step.  (Page "读一个真实 serving 系统 · vLLM 架构巡礼",
 * section 3: the scheduler has no separate prefill and decode phases, every request
 * just gets new tokens; page "vLLM PagedAttention 原理与源码深度解析", sections 8.1 and
 * 8.2: a long prompt is cut into chunks, a draft model proposes 5 tokens for the main
 * model to verify; page "vllm源码剖析", section 一.3: the requests' tokens are packed
 * into one flat batch with a start and a length each.)  The pages print no kernel for
 * this step; the reading here:
 *
 *   query_start_loc  device int32 [num_seqs + 1]: sequence i owns the new tokens
 *                    query_start_loc[i] .. query_start_loc[i+1] - 1 of the flat batch
 *                    (non-decreasing from 0 to num_tokens);
 *   context_lens     device int32 [num_seqs]: every token of sequence i after the step,
 *                    its new ones included, so new token j sits at position
 *                    p = context_lens[i] - q_len_i + j;
 *   new token j attends to positions 0 .. p of its sequence (causal within the step):
 *     out[t][h] = sum_{u <= p} softmax_u(scale * <q_{t,h}, k_u>) v_u,
 *   with kv head h / (num_heads / num_kv_heads).  One new token per sequence is a
 *   decode step.
 *
 * pkv_slot_mapping_multi_query -- slot_mapping[t] (device int32 [num_tokens]) of every
 * new token: block_tables[i][p / block_size] * block_size + p % block_size, or -1 for a
 * sequence whose new tokens do not fit (q_len > context_len, a context past its table,
 * a range outside the flat batch) or a block id outside [0, num_blocks).  The rows
 * are then stored with pkv_kv_cache_write(key, value, ..., slot_mapping, num_tokens,
 * ...), key/value being [num_tokens][num_kv_heads][head_dim].
 *
 * pkv_paged_attention_multi_query -- out [num_tokens][num_heads][head_dim] (out_dtype)
 * from query [num_tokens][num_heads][head_dim] (kv_dtype) over the paged caches, the
 * new tokens' rows already written.  Accumulation fp32; scores and probabilities fp32
 * throughout (no reduced-precision P).  Supported: kv_dtype PKV_F32 or PKV_BF16,
 * head_dim 64 or 128, block_size 16 or 32, num_heads / num_kv_heads in {1, 2, 4, 8},
 * num_tokens * num_heads * head_dim * sizeof(kv_dtype) below 2^31.
 * Work split.  Rows are (new token, query head) pairs; the rows of one sequence and kv
 * head are cut into units of R rows (R / G consecutive new tokens with the
 * G = num_heads / num_kv_heads query heads of the kv head).  With A = num_tokens * G /
 * num_seqs the average rows per sequence: R = 16 when A <= 16; R = 128 when head_dim
 * is 128 and A >= 128; R = 32 otherwise.  Units and their tiles are split over the
 * GPU in equal shares and the pieces merged by log-sum-exp, except that with bf16
 * caches, head_dim 128 and R = 128, units of 256 rows are used when they give at least
 * one (unit, kv head) item per compute unit (the environment variable
 * PKV_PREFILL_MIN_ITEMS, read at each call, sets another threshold): each item's causal
 * context is then cut into pieces (two on an even batch, up to four for the units of a
 * history much longer than the rest), computed by different workgroups and merged by
 * log-sum-exp in a fixed order by whichever finishes last.  Where the pieces fall
 * depends on the whole batch and the GPU, so results may differ between batches in
 * the last bits of fp32; for one batch on one GPU they are deterministic.
 * Workspace: pkv_paged_attention_multi_query_workspace_bytes() bytes, no
 * initialisation needed.  With U = ceil(num_tokens / (R / G)) + num_seqs, it holds a
 * 256-byte header, the unit plan (U + 1, U and num_seqs + 1 int32, each rounded up to
 * 256 bytes) and N records of (head_dim + 2) fp32: N = (1024 + U) * num_kv_heads * R,
 * or, when the 256-row units may be taken (head_dim 128, R = 128), at least
 * 1026 * U' * num_kv_heads + num_seqs + 64 with U' = ceil(num_tokens * G / 256) +
 * num_seqs (four records per item, the items' counters and the schedule).
 * PKV_ERR_UNSUPPORTED when U * num_kv_heads + num_tokens exceeds 2^32 / 256 - 1.
 * Device-side contract: rows of a sequence that does not fit
 * (as for the slot mapping), or that lists a block id outside [0, num_blocks) within
 * its context, are NaN; a query_start_loc that is not a non-decreasing cut of the
 * flat batch may make every row NaN; nothing outside the listed blocks and the flat
 * batch is read.  num_tokens == 0 is a no-op.
 */
pkv_status pkv_slot_mapping_multi_query(const int32_t* block_tables, const int32_t* context_lens,
                                        const int32_t* query_start_loc, int32_t* slot_mapping,
                                        int32_t num_seqs, int32_t num_tokens,
                                        int32_t max_blocks_per_seq, int32_t block_size,
                                        int64_t num_blocks, void* stream);

size_t pkv_paged_attention_multi_query_workspace_bytes(int32_t num_seqs, int32_t num_tokens,
                                                       int32_t num_heads, int32_t num_kv_heads,
                                                       int32_t head_dim, int32_t block_size,
                                                       int32_t max_blocks_per_seq);

pkv_status pkv_paged_attention_multi_query(void* out, const void* query, const void* key_cache,
                                           const void* value_cache, const int32_t* block_tables,
                                           const int32_t* context_lens,
                                           const int32_t* query_start_loc, int32_t num_seqs,
                                           int32_t num_tokens, int32_t num_heads,
                                           int32_t num_kv_heads, int32_t head_dim,
                                           int32_t block_size, int32_t max_blocks_per_seq,
                                           int64_t num_blocks, float scale, pkv_dtype kv_dtype,
                                           pkv_dtype out_dtype, void* workspace,
                                           size_t workspace_bytes, void* stream);

/*
 * pkv_decode_prologue -- the steps of a decode step that come before attention,
 * in one launch: pkv_slot_mapping for every sequence (written to slot_mapping),
 * pkv_kv_cache_write of every sequence's new token (key/value row t belongs to
 * sequence t) at that slot, and pkv_paged_attention_plan into the workspace.
 * The results are bit-identical to the three separate calls.  A model with
 * several layers calls it for its first layer and reuses slot_mapping and the
 * plan for the others (pkv_kv_cache_write + the partition and reduce stages).
 *
 *   key, value    device [num_seqs][num_kv_heads][head_dim], kv_dtype
 *   slot_mapping  device int32 [num_seqs], written
 *   workspace     at least the plan part of pkv_paged_attention_workspace_bytes()
 *
 * Arguments are checked as for the three separate calls.
 */
pkv_status pkv_decode_prologue(const int32_t* block_tables, const int32_t* context_lens,
                               const void* key, const void* value, void* key_cache,
                               void* value_cache, int32_t* slot_mapping, int32_t num_seqs,
                               int32_t max_blocks_per_seq, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int64_t num_blocks, pkv_dtype kv_dtype,
                               int32_t partition_size, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Bytes of device workspace pkv_paged_attention_decode needs (0 for invalid
 * arguments).  With fixed partitions of P tokens and
 * NP = ceil(max_blocks_per_seq*block_size / P), the workspace holds
 *   - the work plan: 256 bytes, then one 16-byte item per (sequence, partition),
 *     rounded up to 256 bytes:  256 + roundup256(num_seqs * NP * 16);
 *   - one (max, sum, partial output) fp32 record per (sequence, query head,
 *     partition):  num_seqs * num_heads * NP * (head_dim + 2) * 4.
 * With the balanced split (PKV_PARTITION_BALANCED) it holds
 *   - the tile plan: 256 bytes of header, then num_seqs + 1 int32 prefix sums,
 *     rounded up to 256 bytes:  256 + roundup256((num_seqs + 1) * 4);
 *   - one record per (segment label, query head), labels below 1024 + num_seqs:
 *     (1024 + num_seqs) * num_heads * (head_dim + 2) * 4.
 * Its contents need no initialisation and are scratch between calls.
 */
size_t pkv_paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                           int32_t head_dim, int32_t block_size,
                                           int32_t max_blocks_per_seq, int32_t partition_size);

/*
 * pkv_paged_attention_decode -- one query token per sequence attends to its
 * whole paged context.
 *
 * For sequence i, query head h, kv head g = h / (num_heads / num_kv_heads), and
 * context rows k_t, v_t (t < ctx = context_lens[i]) read through the block table
 * (row t is row t % block_size of physical block block_tables[i][t / block_size]):
 *     s_t = scale * <q_{i,h}, k_t>,   p_t = exp(s_t - max_u s_u),
 *     out[i][h] = sum_t p_t v_t / sum_t p_t.
 * (Page "vllm源码分析：我是如何一步步读懂PagedAttention核心实现的？", 第三讲: the
 * logical-to-physical block indirection, then the usual softmax and weighted
 * sum; page "vLLM PagedAttention 原理与源码深度解析", section 5.3: gather K/V
 * through block_tables up to context_lens, scores divided by sqrt(head_dim),
 * softmax, weighted sum of V.  The max subtraction and the partition merge below
 * are not printed on the pages; they leave the result unchanged.)
 *
 * Contexts are split into pieces (fixed partitions of P = partition_size tokens,
 * 512 for PKV_PARTITION_DEFAULT, or the segments of the balanced split for
 * PKV_PARTITION_BALANCED), each giving
 * (m_k, l_k, o_k); the pieces are merged in order as
 *     M = max m_k,  w_k = l_k exp(m_k - M),  out = sum w_k o_k / sum w_k.
 * A sequence in a single piece is written directly.
 *
 *   out           device [num_seqs][num_heads][head_dim], out_dtype (written)
 *   query         device [num_seqs][num_heads][head_dim], kv_dtype
 *   key_cache, value_cache  device caches as above, kv_dtype
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq]; entries at or past
 *                 ceil(ctx/block_size) are never read
 *   context_lens  device int32 [num_seqs], 1 <= ctx <= max_blocks_per_seq*block_size
 *   scale         multiplies q.k (1/sqrt(head_dim) for standard attention)
 *   partition_size  P in tokens, a multiple of block_size and of 16;
 *                 PKV_PARTITION_DEFAULT (0) for 512; PKV_PARTITION_BALANCED (-1) for
 *                 the balanced split
 *   workspace     device buffer of at least pkv_paged_attention_workspace_bytes()
 *
 * Supported: kv_dtype in {PKV_F32, PKV_BF16}; out_dtype in {PKV_F32, PKV_BF16}
 * (bf16 output is the fp32 result rounded to nearest even); head_dim in {64, 128};
 * block_size in {16, 32}; num_heads / num_kv_heads in {1, 2, 4, 8}.  Other
 * combinations return PKV_ERR_UNSUPPORTED.  Accumulation is fp32.
 *
 * Device-side contract: a sequence whose context length is out of range, or that
 * lists a block id outside [0, num_blocks) within its context, gets NaN in every
 * element of its output rows; no memory outside the listed blocks is read.
 * num_seqs == 0 is a no-op.
 */
pkv_status pkv_paged_attention_decode(void* out, const void* query, const void* key_cache,
                                      const void* value_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t max_blocks_per_seq,
                                      int64_t num_blocks, float scale, int32_t partition_size,
                                      pkv_dtype kv_dtype, pkv_dtype out_dtype, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * The three stages of pkv_paged_attention_decode, for callers that want to place,
 * reuse or time them separately.  Called in this order on one stream with the
 * same arguments and workspace they produce exactly what
 * pkv_paged_attention_decode produces.
 *
 * pkv_paged_attention_plan writes the work plan into the start of the workspace.
 * Fixed partitions: one item per (sequence, partition) that holds tokens -- whole
 * partitions first, then the partial last partitions from largest to smallest --
 * so that the partition stage hands the longest work out first.  Balanced split:
 * the prefix sums of the sequences' list positions (ceil(ctx / 16) + 1 for a valid
 * context, 0 otherwise) and their total.  It reads only context_lens; a plan stays
 * valid for as long as context_lens, block_size, max_blocks_per_seq,
 * partition_size and num_seqs are unchanged (for example for every layer of one
 * decode step).  It needs workspace_bytes of at least the plan part described
 * above.
 *
 * pkv_paged_attention_partition runs the planned work: it writes sequences that
 * fit in one piece straight to `out` and the records of the others to the
 * workspace.  Fixed partitions: it checks the plan's items against num_seqs and
 * the partition count, so a stale plan yields wrong numbers, never an access
 * outside the buffers.  Balanced split: a stale plan likewise yields wrong numbers
 * (tiles past a table row count as invalid blocks), never an access outside the
 * buffers.
 *
 * pkv_paged_attention_reduce merges the records of the sequences split into
 * several pieces into `out`, in piece order.  With the balanced split it also
 * writes the NaN rows of sequences with an invalid context length, so it must
 * follow every partition stage there.
 */
pkv_status pkv_paged_attention_plan(const int32_t* context_lens, int32_t num_seqs,
                                    int32_t block_size, int32_t max_blocks_per_seq,
                                    int32_t partition_size, void* workspace,
                                    size_t workspace_bytes, void* stream);

pkv_status pkv_paged_attention_partition(void* out, const void* query, const void* key_cache,
                                         const void* value_cache, const int32_t* block_tables,
                                         const int32_t* context_lens, int32_t num_seqs,
                                         int32_t num_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t block_size,
                                         int32_t max_blocks_per_seq, int64_t num_blocks,
                                         float scale, int32_t partition_size,
                                         pkv_dtype kv_dtype, pkv_dtype out_dtype,
                                         void* workspace, size_t workspace_bytes, void* stream);

pkv_status pkv_paged_attention_reduce(void* out, const int32_t* context_lens, int32_t num_seqs,
                                      int32_t num_heads, int32_t head_dim, int32_t block_size,
                                      int32_t max_blocks_per_seq, int32_t partition_size,
                                      pkv_dtype out_dtype, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * pkv_paged_attention_decode_noalloc -- pkv_paged_attention_decode for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments minus the workspace, same kernels,
 * same results (bit for bit, for the same partition_size).
 *
 * The workspace lives instead in a fixed device array inside the library, one per GPU,
 * of PKV_NOALLOC_SCRATCH_BYTES (64 MiB); it is set up on the first call on a GPU (the
 * GPU of `stream`, or the current one for the null stream) and held until the process
 * ends.  A call whose workspace (pkv_paged_attention_workspace_bytes of the same
 * arguments) would exceed it returns PKV_ERR_SCRATCH_LIMIT before any GPU work; the
 * balanced split needs (1024 + num_seqs) * num_heads * (head_dim + 2) * 4 bytes plus
 * its plan, e.g. 256 sequences of 32 heads of 128 fit.  The call allocates and frees
 * nothing.  Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (on different streams, or from different host threads without ordering) race
 * and may produce wrong results; calls ordered on one stream are safe.  The array's
 * contents need no clearing between calls.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (64u << 20)

pkv_status pkv_paged_attention_decode_noalloc(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int64_t num_blocks, float scale, int32_t partition_size,
    pkv_dtype kv_dtype, pkv_dtype out_dtype, void* stream);

/*
 * The per-head layout of fixed partitions, for batches whose sequences share prefix
 * blocks.  (Page "读一个真实 serving 系统 · vLLM 架构巡礼", section 2: requests with a
 * common prefix point at the same physical blocks; page "vllm源码剖析", the BlockPool
 * paragraphs: a cached block is handed to every request that matches it.)  The
 * library cannot tell from its arguments that tables share blocks; the caller, who
 * holds the reference counts, can.
 *
 * pkv_paged_attention_partition_per_head is pkv_paged_attention_partition with one
 * 4-wave workgroup per (kv head, partition, sequence) instead of one per (partition,
 * sequence) and group of kv heads, reading keys and values through the caches (the
 * streaming kernel's copies bypass them).  The workgroups of sequences that share a
 * block then run side by side and the block is fetched from HBM about once.  Same
 * arguments, same workspace and plan (pkv_paged_attention_plan, then
 * pkv_paged_attention_reduce), same results to fp32 rounding; fixed partitions only:
 * partition_size PKV_PARTITION_BALANCED is PKV_ERR_INVALID_ARG.  Caches of PKV_F32 or
 * PKV_BF16.
 *
 * pkv_paged_attention_decode_per_head is pkv_paged_attention_decode (plan, this
 * partition stage, reduce) in that layout.
 */
pkv_status pkv_paged_attention_partition_per_head(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int64_t num_blocks, float scale, int32_t partition_size,
    pkv_dtype kv_dtype, pkv_dtype out_dtype, void* workspace, size_t workspace_bytes,
    void* stream);

pkv_status pkv_paged_attention_decode_per_head(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int64_t num_blocks, float scale, int32_t partition_size,
    pkv_dtype kv_dtype, pkv_dtype out_dtype, void* workspace, size_t workspace_bytes,
    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H_ */
