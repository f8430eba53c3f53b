// PagedAttention decode for gfx950: a partition kernel and a log-sum-exp reduce.
//
// What is computed (page "vllm源码分析：我是如何一步步读懂PagedAttention核心实现的？",
// 第三讲, and page "vLLM PagedAttention 原理与源码深度解析", section 5.3): for each
// sequence and query head, the context rows of K and V are found through the
// block table (logical block -> physical block), scores are the scaled dot
// products of the query with every key of the context, a softmax turns them into
// weights, and the output is the weighted sum of the values.  The max subtraction
// and the split into partitions merged by log-sum-exp leave that result unchanged
// and are this design's, not the pages'.
//
// Work decomposition.  One workgroup of four wave64s per (kv head, context
// partition, sequence).  A partition of P tokens is cut into 16-token tiles; wave w
// takes tiles w, w+4, w+8, ..., a few at a time.  For every tile:
//   * Q.K^T on the matrix cores for GQA groups of four or eight heads: one 16x16
//     MFMA output holds the scores of the group (zero-padded to 16 rows) against 16
//     tokens.  Each lane feeds the MFMA a 16-byte piece of one key row straight from
//     HBM, so a tile's keys are read once, in 64-byte runs per row and instruction.
//     Groups of one or two heads take the same pieces into dot products on the VALU
//     (each lane a quarter of the dims, the quarters added by lane-row swaps).
//   * softmax on the VALU with a running (per wave) maximum in the base-2 exponent
//     domain; row maxima and sums use DPP within 16-lane rows.
//   * P.V on the VALU: 16-byte pieces of value rows, fp32 fused multiply-adds, the
//     probabilities broadcast from LDS.
// At the end the four waves merge their (max, sum, partial output) through LDS.
// A sequence with one partition writes its output directly; otherwise the
// partition's (m, l, o/l) goes to the workspace and the reduce kernel merges the
// partitions in index order.  No atomics: the result does not depend on timing.
#include <math.h>

#include "pkv_device.hpp"
#include "pkv_launch.hpp"
#include "pkv_plan.hpp"
#include "pkv_stream.hpp"
#include "pkv_tile.hpp"

namespace pkv {

// Word 3 of a raw buffer descriptor on gfx9-family parts: 32-bit data format,
// no swizzle, no index stride.
constexpr int kBufferFlags = 0x00020000;

// Build-time tuning knobs (defaults: the measured best on MI355X).
#ifndef PKV_WAVES_PER_EU
#define PKV_WAVES_PER_EU 1         // occupancy floor handed to the register allocator
#endif

size_t plan_bytes(int64_t num_seqs, int64_t max_parts) {
  return 256 + ((size_t)(num_seqs * max_parts) * sizeof(int4) + 255) / 256 * 256;
}

// The standalone plan stage: one workgroup.
__global__ __launch_bounds__(kPlanThreads) void paged_attention_plan_kernel(AttentionArgs a) {
  build_plan<kPlanThreads>(a.context_lens, a.num_seqs, a.partition_size,
                           a.max_blocks_per_seq << a.block_shift, a.plan_items, a.plan_count);
}

// The loads of one 16-token tile, in flight while the previous tile is computed.
template <int QKC, int STEPS>
struct TileLoads {
  uint4 k[QKC];     // key chunks in MFMA B-operand order
  uint4 v[STEPS];   // value chunks, one per wave load of RPS rows
  int ntok;         // live tokens of the tile; 0 = no tile (past the end, or a bad block)
};

template <typename T, int D, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(PKV_WAVES_PER_EU)))
void paged_attention_partition_kernel(AttentionArgs a) {
  using Geo = Geometry<T, D, G>;
  constexpr int EPL = Geo::kEPL;
  constexpr int NCH = Geo::kChunksPerRow;
  constexpr int QKC = Geo::kQkChunks;
  constexpr int RPS = Geo::kRowsPerStep;
  constexpr int STEPS = Geo::kSteps;
  constexpr int EB = T::kElemBytes;

  __shared__ float p_lds[4][16][G];     // per wave: probabilities of its current tile
  __shared__ float red_o[4][G][D];
  __shared__ float red_m[4][G];
  __shared__ float red_l[4][G];
  __shared__ int red_bad[4];

  const int lane = threadIdx.x & (kWave - 1);
  // The wave index is the same in every lane; saying so lets everything derived
  // from it (tile numbers, block ids, block base addresses) live in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int Hkv = a.num_kv_heads;
  const int H = Hkv * G;
  // Workgroup -> (plan item, kv head); heads vary fastest.  Items are checked so
  // that a stale plan can give wrong numbers but never an out-of-range access.
  const int g = blockIdx.x % Hkv;
  const int idx = blockIdx.x / Hkv;
  const int count = min(*a.plan_count, a.num_seqs * a.max_parts);
  if (idx >= count) return;
  const int4 item = a.plan_items[idx];
  const int seq = item.x;
  const int part = item.y;
  const int ctx = item.z;
  if (seq < 0 || seq >= a.num_seqs || part < 0 || part >= a.max_parts) return;

  const int max_ctx = a.max_blocks_per_seq << a.block_shift;
  if (ctx < 1 || ctx > max_ctx) {
    // Invalid context length: the sequence's rows become NaN (written once).
    if (part == 0) {
      for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x)
        store_out(a.out, ((int64_t)seq * H + g * G) * D + idx, __builtin_nanf(""), a.out_bf16);
    }
    return;
  }
  const int p_start = part * a.partition_size;
  if (p_start >= ctx) return;
  const int p_end = min(p_start + a.partition_size, ctx);
  const int nparts = (ctx + a.partition_size - 1) / a.partition_size;
  const int ntiles = (p_end - p_start + 15) >> 4;

  const int quarter = lane >> 4;   // MFMA operand k-group / output row group
  const int col = lane & 15;       // MFMA A row (head) and B column (token)
  const int rg = lane / NCH;       // value row within a wave load
  const int li = lane % NCH;       // 16-byte chunk within a value row

  // Query rows of this kv head's group, as the MFMA A operand (rows >= G are zero).
  // Groups of one or two heads would fill one or two of its 16 rows: their scores are
  // dot products on the VALU, with every head's chunks 4c + quarter of the query in qv.
  constexpr bool kValuQK = G <= 2;
  uint4 qa[kValuQK ? 1 : QKC];
  uint4 qv[kValuQK ? G : 1][kValuQK ? QKC : 1];
  if constexpr (kValuQK) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const char* qrow = static_cast<const char*>(a.query) + ((int64_t)seq * H + g * G + h) * D * EB;
#pragma unroll
      for (int c = 0; c < QKC; ++c) qv[h][c] = load16(qrow, (4 * c + quarter) * 16);
    }
  } else {
    const char* qrow = static_cast<const char*>(a.query) +
                       ((int64_t)seq * H + g * G + (col < G ? col : 0)) * D * EB;
#pragma unroll
    for (int c = 0; c < QKC; ++c)
      qa[c] = col < G ? load16(qrow, (4 * c + quarter) * 16) : make_uint4(0, 0, 0, 0);
  }

  // Byte offsets: the block base is the same for the whole wave (a scalar), the
  // per-lane part fits in 32 bits.
  const uint32_t row_bytes = (uint32_t)Hkv * D * EB;   // between consecutive tokens of a block
  const uint32_t k_lane = col * row_bytes + quarter * 16;
  const uint32_t v_lane = rg * row_bytes + li * 16;
  const int32_t* bt_row = a.block_tables + (int64_t)seq * a.max_blocks_per_seq;
  const int bs_mask = (1 << a.block_shift) - 1;
  const int64_t head_bytes = (int64_t)g * D * EB;
  const int num_blocks = (int)a.num_blocks;               // the ABI keeps it below 2^31
  const int tile_span = (int)(15 * row_bytes + D * EB);   // bytes of one head's 16 rows
  const char* kcache = static_cast<const char*>(a.key_cache);
  const char* vcache = static_cast<const char*>(a.value_cache);
  const float kNegInf = -__builtin_inff();

  float m_run[G];
  float acc[G][EPL];
  float l_lane[4];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = kNegInf;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) l_lane[j] = 0.f;
  int bad = 0;

  using Loads = TileLoads<QKC, STEPS>;

  // Issue the key and value loads of tile ``tile`` (wave-uniform decisions only).
  // The loads themselves are unconditional, so the compiler can count them and
  // wait for exactly the tile being computed while the next one is in flight: a
  // tile that does not exist (past the partition's end, or a bad block id) reads
  // pool block 0 instead, which is always in bounds and, shared by every
  // workgroup, stays in cache.
  //
  // Loads go through raw buffer descriptors built per tile in scalar registers:
  // base = the tile's first row of this head, range = the 16 rows of the head.
  // Lane offsets stay 32-bit, no 64-bit address arithmetic lands in vector
  // registers, and the hardware returns zeros for anything past the range.
  auto issue = [&](Loads& r, int tile) {
    int ntok = 0;
    int64_t off = 0;
    if (tile < ntiles) {
      const int tok0 = p_start + 16 * tile;
      const int32_t blk = bt_row[tok0 >> a.block_shift];
      if (blk < 0 || blk >= num_blocks) {
        bad = 1;
      } else {
        ntok = min(16, p_end - tok0);
        off = (((int64_t)blk << a.block_shift) + (tok0 & bs_mask)) * row_bytes + head_bytes;
      }
    }
    r.ntok = ntok;
    const auto kd = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kcache + off), 0,
                                                      tile_span, kBufferFlags);
    const auto vd = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vcache + off), 0,
                                                      tile_span, kBufferFlags);
#pragma unroll
    for (int c = 0; c < QKC; ++c)
      r.k[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                             kd, k_lane + c * 64, 0, 0));
    // keys before values in every copy of this code, so the wait counts agree
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
      r.v[s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                             vd, v_lane, s * RPS * row_bytes, 0));
  };

  // Scores, running maximum, probabilities and P.V for one loaded tile.
  auto compute = [&](const Loads& r) {
    if (r.ntok == 0) return;
    floatx4 s4;
    if constexpr (kValuQK) {
      // the lane's chunks of token col's key against each head's query, the four
      // quarters' sums added; element j holds head j % G, as the MFMA rows would
      float sh[G];
#pragma unroll
      for (int h = 0; h < G; ++h) sh[h] = sum_xor32(sum_xor16(lane_dot<T, QKC>(qv[h], r.k)));
#pragma unroll
      for (int j = 0; j < 4; ++j) s4[j] = sh[j % G];
    } else {
      s4 = tile_scores<T, QKC>(qa, r.k);
    }
    const bool live = col < r.ntok;
    float sc[4], gmax[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sc[j] = live ? s4[j] * a.scale_log2 : kNegInf;
      gmax[j] = row16_max(sc[j]);
    }
    float alpha[G];
    bool rescale = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float gm = readlane(gmax[h & 3], 16 * (h >> 2));
      const float mn = fmaxf(m_run[h], gm);
      alpha[h] = fast_exp2(m_run[h] - mn);
      rescale |= m_run[h] != mn;
      m_run[h] = mn;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float mrow, arow;
      if constexpr (G <= 4) {
        mrow = j < G ? m_run[j < G ? j : 0] : 0.f;
        arow = j < G ? alpha[j < G ? j : 0] : 1.f;
      } else {
        mrow = quarter == 0 ? m_run[j] : m_run[(4 + j) % G];
        arow = quarter == 0 ? alpha[j] : alpha[(4 + j) % G];
      }
      sc[j] = fast_exp2(sc[j] - mrow);
      l_lane[j] = l_lane[j] * arow + sc[j];
    }
    if (rescale) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha[h];
    }
    if (quarter < Geo::kQuarters) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * quarter + j < G) p_lds[wave][col][(4 * quarter + j) % G] = sc[j];
    }
    __builtin_amdgcn_wave_barrier();
    const bool full = r.ntok == 16;
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      const int n = s * RPS + rg;
      float pv[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pv[h] = p_lds[wave][n][h];
      float v[EPL];
      unpack_chunk<T>(r.v[s], v);
      if (!full && n >= r.ntok) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) v[e] = 0.f;   // rows past the context may hold NaN
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pv[h], v[e], acc[h][e]);
    }
    __builtin_amdgcn_wave_barrier();
  };

  // Wave w takes tiles w, w+4, w+8, ...; the next tile's loads are issued before
  // the current tile is computed (two register sets used in turn).
  Loads A, B;
  int t = wave;
  issue(A, t);
  while (t < ntiles) {
    issue(B, t + 4);
    compute(A);
    t += 4;
    if (t >= ntiles) break;
    issue(A, t + 4);
    compute(B);
    t += 4;
  }

  // ---- merge the four waves ---------------------------------------------------
#pragma unroll
  for (int off = NCH; off < kWave; off <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] += __shfl_xor(acc[h][e], off);
#pragma unroll
  for (int j = 0; j < 4; ++j) l_lane[j] = row16_sum(l_lane[j]);
  if (lane < NCH) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) red_o[wave][h][li * EPL + e] = acc[h][e];
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float lw = readlane(l_lane[h & 3], 16 * (h >> 2));
    if (lane == 0) {
      red_m[wave][h] = m_run[h];
      red_l[wave][h] = lw;
    }
  }
  if (lane == 0) red_bad[wave] = bad;
  __syncthreads();

  const bool any_bad = red_bad[0] | red_bad[1] | red_bad[2] | red_bad[3];
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int h = idx / D;
    const int d = idx % D;
    float M = red_m[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, red_m[w][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = fast_exp2(red_m[w][h] - M);   // waves without tiles: exp2(-inf) = 0
      L = fmaf(red_l[w][h], f, L);
      O = fmaf(red_o[w][h][d], f, O);
    }
    const float res = any_bad ? __builtin_nanf("") : O / L;
    const int64_t row = (int64_t)seq * H + g * G + h;
    if (nparts == 1) {
      store_out(a.out, row * D + d, res, a.out_bf16);
    } else {
      const int64_t rec = row * a.max_parts + part;
      a.ws_o[rec * D + d] = res;
      if (d == 0) {
        a.ws_m[rec] = M;
        a.ws_l[rec] = L;
      }
    }
  }
}

// ---- partition merge --------------------------------------------------------------
// For every multi-partition (sequence, head) row: M = max m_k, w_k = l_k 2^(m_k - M),
// out = sum w_k o_k / sum w_k.  Lanes read 16-byte pieces of the partial outputs.
// Each lane group keeps its own running (max, sum, weighted output) over a fixed
// subset of the partitions; the groups are then merged in a fixed order, so the
// result does not depend on timing.

// Few partitions per row: one wave per row, four rows per workgroup, one round of
// loads, no barriers.
constexpr int kNarrowMaxParts = 16;

template <int D>
__global__ __launch_bounds__(256) void paged_attention_reduce_narrow_kernel(AttentionArgs a) {
  constexpr int LPR = D / 4;             // lanes per record (float4 each)
  constexpr int KGW = kWave / LPR;       // records per wave load
  constexpr int NK = kNarrowMaxParts / KGW;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (row >= (int64_t)a.num_seqs * a.num_heads) return;
  const int seq = (int)(row / a.num_heads);
  const int ctx = a.context_lens[seq];
  const int max_ctx = a.max_blocks_per_seq << a.block_shift;
  if (ctx < 1 || ctx > max_ctx) return;
  const int nparts = (ctx + a.partition_size - 1) / a.partition_size;
  if (nparts <= 1) return;
  const int kg = lane / LPR;
  const int lr = lane % LPR;
  const int64_t rec0 = row * a.max_parts;
  float m[NK], l[NK];
  float4 o[NK];
  bool live[NK];
#pragma unroll
  for (int u = 0; u < NK; ++u) {
    const int k = kg + u * KGW;
    live[u] = k < nparts;
    m[u] = live[u] ? a.ws_m[rec0 + k] : 0.f;
    l[u] = live[u] ? a.ws_l[rec0 + k] : 0.f;
    o[u] = live[u] ? reinterpret_cast<const float4*>(a.ws_o + (rec0 + k) * D)[lr]
                   : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  Running r{-__builtin_inff(), 0.f, make_float4(0.f, 0.f, 0.f, 0.f)};
  accumulate(r, m, l, o, live);
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
    Running s;
    s.m = __shfl_xor(r.m, off);
    s.l = __shfl_xor(r.l, off);
    s.o.x = __shfl_xor(r.o.x, off);
    s.o.y = __shfl_xor(r.o.y, off);
    s.o.z = __shfl_xor(r.o.z, off);
    s.o.w = __shfl_xor(r.o.w, off);
    // both lanes of a pair merge the same two values in the same order
    if (lane & off) { const Running t = r; r = s; s = t; }
    merge_into(r, s);
  }
  if (kg == 0) store_row4(a, row * D + lr * 4, r);
}

// Many partitions per row (long contexts): one workgroup per row, KG lane groups
// each streaming every KG-th partition four at a time, merged through LDS.
template <int D>
__global__ __launch_bounds__(256) void paged_attention_reduce_wide_kernel(AttentionArgs a) {
  constexpr int kThreads = 256;
  constexpr int LPR = D / 4;
  constexpr int KG = kThreads / LPR;
  constexpr int kUnroll = 4;
  __shared__ float4 red_o[KG][LPR];
  __shared__ float red_m[KG];
  __shared__ float red_l[KG];
  const int64_t row = blockIdx.x;
  const int seq = (int)(row / a.num_heads);
  const int ctx = a.context_lens[seq];
  const int max_ctx = a.max_blocks_per_seq << a.block_shift;
  if (ctx < 1 || ctx > max_ctx) return;
  const int nparts = (ctx + a.partition_size - 1) / a.partition_size;
  if (nparts <= 1) return;
  const int kg = threadIdx.x / LPR;
  const int lr = threadIdx.x % LPR;
  const int64_t rec0 = row * a.max_parts;
  Running r{-__builtin_inff(), 0.f, make_float4(0.f, 0.f, 0.f, 0.f)};
  for (int k0 = kg; k0 < nparts; k0 += KG * kUnroll) {
    float m[kUnroll], l[kUnroll];
    float4 o[kUnroll];
    bool live[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int k = k0 + u * KG;
      live[u] = k < nparts;
      m[u] = live[u] ? a.ws_m[rec0 + k] : 0.f;
      l[u] = live[u] ? a.ws_l[rec0 + k] : 0.f;
      o[u] = live[u] ? reinterpret_cast<const float4*>(a.ws_o + (rec0 + k) * D)[lr]
                     : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    accumulate(r, m, l, o, live);
  }
  red_o[kg][lr] = r.o;
  if (lr == 0) {
    red_m[kg] = r.m;
    red_l[kg] = r.l;
  }
  __syncthreads();
  if (threadIdx.x < LPR) {
    Running t{red_m[0], red_l[0], red_o[0][threadIdx.x]};
#pragma unroll
    for (int q = 1; q < KG; ++q) merge_into(t, Running{red_m[q], red_l[q], red_o[q][threadIdx.x]});
    store_row4(a, row * D + threadIdx.x * 4, t);
  }
}

// ---- dispatch ------------------------------------------------------------------

hipError_t launch_attention_plan(const AttentionArgs& a, hipStream_t stream) {
  if (a.balanced) return launch_tile_plan(a, stream);
  hipLaunchKernelGGL(paged_attention_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_partition_g(const AttentionArgs& a, hipStream_t stream) {
  const int G = a.num_heads / a.num_kv_heads;
  const dim3 grid((unsigned)((int64_t)a.num_kv_heads * a.max_parts * a.num_seqs));
  const dim3 block(256);
  switch (G) {
    case 1: hipLaunchKernelGGL((paged_attention_partition_kernel<T, D, 1>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((paged_attention_partition_kernel<T, D, 2>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((paged_attention_partition_kernel<T, D, 4>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((paged_attention_partition_kernel<T, D, 8>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Fixed partitions run in the streaming kernel (whole token rows of a kv-head group
// through LDS, copies past the caches) unless the caller asks for the per-head
// layout above, which reads through the caches and suits batches sharing prefix blocks.
hipError_t launch_attention_partition(const AttentionArgs& a, hipStream_t stream) {
  if (a.balanced) return launch_attention_stream(a, stream);
  if (!a.per_head) return launch_attention_stream_fixed(a, stream);
  if (a.kv_bf16) {
    if (a.head_dim == 64) return launch_partition_g<BF16, 64>(a, stream);
    if (a.head_dim == 128) return launch_partition_g<BF16, 128>(a, stream);
  } else if (!a.kv_fp8) {
    if (a.head_dim == 64) return launch_partition_g<F32, 64>(a, stream);
    if (a.head_dim == 128) return launch_partition_g<F32, 128>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attention_reduce(const AttentionArgs& a, hipStream_t stream) {
  if (a.balanced) return launch_attention_stream_reduce(a, stream);
  const int64_t rows = (int64_t)a.num_heads * a.num_seqs;
  const bool narrow = a.max_parts <= kNarrowMaxParts;
  if (a.head_dim == 64) {
    if (narrow)
      hipLaunchKernelGGL(paged_attention_reduce_narrow_kernel<64>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(paged_attention_reduce_wide_kernel<64>, dim3((unsigned)rows), dim3(256), 0, stream, a);
  } else if (a.head_dim == 128) {
    if (narrow)
      hipLaunchKernelGGL(paged_attention_reduce_narrow_kernel<128>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(paged_attention_reduce_wide_kernel<128>, dim3((unsigned)rows), dim3(256), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
