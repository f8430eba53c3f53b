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
//   * Q.K^T on the matrix cores: one 16x16 MFMA output holds the scores of up to 16
//     query heads (the kv head's GQA group, zero-padded) against 16 tokens.  Each
//     lane feeds the MFMA a 16-byte piece of one key row straight from HBM, so a
//     tile's keys are read once, in 64-byte runs per row and instruction.
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

namespace pkv {

template <typename T, int D, int G>
struct Geometry {
  static constexpr int kEPL = T::kPerChunk;                 // elements per 16-byte chunk
  static constexpr int kChunksPerRow = D * T::kElemBytes / 16;
  static constexpr int kQkChunks = kChunksPerRow / 4;      // chunks per lane for one tile's keys
  static constexpr int kRowsPerStep = kWave / kChunksPerRow;  // value rows per wave load
  static constexpr int kSteps = 16 / kRowsPerStep;           // wave loads per tile of values
  static constexpr int kQuarters = (G + 3) / 4;             // MFMA output quarters with real heads
  static_assert(kChunksPerRow % 4 == 0 && kChunksPerRow <= kWave, "row shape");
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "GQA group");
};

// Scores of one 16-token tile: lane l receives S[head 4*(l/16)+j][token l%16], j<4.
template <typename T, int QKC>
__device__ __forceinline__ floatx4 tile_scores(const uint4 (&q)[QKC], const uint4 (&k)[QKC]);

template <>
__device__ __forceinline__ floatx4 tile_scores<BF16, 4>(const uint4 (&q)[4], const uint4 (&k)[4]) {
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, q[c]),
                                                  __builtin_bit_cast(bf16x8, k[c]), acc, 0, 0, 0);
  return acc;
}

template <>
__device__ __forceinline__ floatx4 tile_scores<BF16, 2>(const uint4 (&q)[2], const uint4 (&k)[2]) {
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 2; ++c)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, q[c]),
                                                  __builtin_bit_cast(bf16x8, k[c]), acc, 0, 0, 0);
  return acc;
}

template <int QKC>
__device__ __forceinline__ floatx4 tile_scores_f32(const uint4 (&q)[QKC], const uint4 (&k)[QKC]) {
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < QKC; ++c) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(q[c].x), __uint_as_float(k[c].x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(q[c].y), __uint_as_float(k[c].y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(q[c].z), __uint_as_float(k[c].z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(q[c].w), __uint_as_float(k[c].w), acc, 0, 0, 0);
  }
  return acc;
}

template <>
__device__ __forceinline__ floatx4 tile_scores<F32, 4>(const uint4 (&q)[4], const uint4 (&k)[4]) {
  return tile_scores_f32<4>(q, k);
}
template <>
__device__ __forceinline__ floatx4 tile_scores<F32, 8>(const uint4 (&q)[8], const uint4 (&k)[8]) {
  return tile_scores_f32<8>(q, k);
}

__device__ __forceinline__ uint4 load16(const void* base, int64_t byte_off) {
  return *reinterpret_cast<const uint4*>(static_cast<const char*>(base) + byte_off);
}

__device__ __forceinline__ void store_out(void* out, int64_t idx, float v, bool out_bf16) {
  if (out_bf16)
    static_cast<uint16_t*>(out)[idx] = f32_to_bf16_rne(v);
  else
    static_cast<float*>(out)[idx] = v;
}

template <typename T, int D, int G, int TPG>
__global__ __launch_bounds__(256) void paged_attention_partition_kernel(AttentionArgs a) {
  using Geo = Geometry<T, D, G>;
  constexpr int EPL = Geo::kEPL;
  constexpr int NCH = Geo::kChunksPerRow;
  constexpr int QKC = Geo::kQkChunks;
  constexpr int RPS = Geo::kRowsPerStep;
  constexpr int STEPS = Geo::kSteps;
  constexpr int EB = T::kElemBytes;

  __shared__ float p_lds[4][TPG][16][G];
  __shared__ float red_o[4][G][D];
  __shared__ float red_m[4][G];
  __shared__ float red_l[4][G];
  __shared__ int red_bad[4];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int Hkv = a.num_kv_heads;
  const int H = Hkv * G;
  const int g = blockIdx.x % Hkv;
  const int rest = blockIdx.x / Hkv;
  const int part = rest % a.max_parts;
  const int seq = rest / a.max_parts;

  const int ctx = a.context_lens[seq];
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
  uint4 qa[QKC];
  {
    const char* qrow = static_cast<const char*>(a.query) +
                       ((int64_t)seq * H + g * G + (col < G ? col : 0)) * D * EB;
#pragma unroll
    for (int c = 0; c < QKC; ++c)
      qa[c] = col < G ? load16(qrow, (4 * c + quarter) * 16) : make_uint4(0, 0, 0, 0);
  }

  const int64_t row_bytes = (int64_t)Hkv * D * EB;  // between consecutive tokens of a block
  const int32_t* bt_row = a.block_tables + (int64_t)seq * a.max_blocks_per_seq;
  const int bs_mask = (1 << a.block_shift) - 1;
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

  for (int t0 = wave; t0 < ntiles; t0 += 4 * TPG) {
    int64_t base[TPG];
    int ntok[TPG];
    bool tv[TPG];
#pragma unroll
    for (int i = 0; i < TPG; ++i) {
      const int tile = t0 + 4 * i;
      const int tok0 = p_start + 16 * tile;
      tv[i] = tile < ntiles;
      ntok[i] = tv[i] ? min(16, p_end - tok0) : 0;
      int32_t blk = tv[i] ? bt_row[tok0 >> a.block_shift] : 0;
      if (tv[i] && (blk < 0 || (int64_t)blk >= a.num_blocks)) {
        bad = 1;
        tv[i] = false;
        ntok[i] = 0;
      }
      base[i] = (((int64_t)blk << a.block_shift) + (tok0 & bs_mask)) * row_bytes + (int64_t)g * D * EB;
    }

    uint4 kr[TPG][QKC];
    uint4 vr[TPG][STEPS];
#pragma unroll
    for (int i = 0; i < TPG; ++i) {
      if (tv[i]) {
#pragma unroll
        for (int c = 0; c < QKC; ++c)
          kr[i][c] = load16(a.key_cache, base[i] + col * row_bytes + (4 * c + quarter) * 16);
      }
    }
#pragma unroll
    for (int i = 0; i < TPG; ++i) {
      if (tv[i]) {
#pragma unroll
        for (int s = 0; s < STEPS; ++s)
          vr[i][s] = load16(a.value_cache, base[i] + (s * RPS + rg) * row_bytes + li * 16);
      }
    }

    // ---- scores ---------------------------------------------------------------
    float sc[TPG][4];
#pragma unroll
    for (int i = 0; i < TPG; ++i) {
      floatx4 r = {0.f, 0.f, 0.f, 0.f};
      if (tv[i]) r = tile_scores<T, QKC>(qa, kr[i]);
      const bool live = col < ntok[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[i][j] = live ? r[j] * a.scale_log2 : kNegInf;
    }

    // ---- running maximum, probabilities ---------------------------------------
    float gmax[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float x = sc[0][j];
#pragma unroll
      for (int i = 1; i < TPG; ++i) x = fmaxf(x, sc[i][j]);
      gmax[j] = row16_max(x);
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
    float mrow[4], arow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (G <= 4) {
        mrow[j] = j < G ? m_run[j < G ? j : 0] : 0.f;
        arow[j] = j < G ? alpha[j < G ? j : 0] : 1.f;
      } else {
        mrow[j] = quarter == 0 ? m_run[j] : m_run[(4 + j) % G];
        arow[j] = quarter == 0 ? alpha[j] : alpha[(4 + j) % G];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float lsum = 0.f;
#pragma unroll
      for (int i = 0; i < TPG; ++i) {
        sc[i][j] = fast_exp2(sc[i][j] - mrow[j]);
        lsum += sc[i][j];
      }
      l_lane[j] = l_lane[j] * arow[j] + lsum;
    }
    if (rescale) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha[h];
    }
    if (quarter < Geo::kQuarters) {
#pragma unroll
      for (int i = 0; i < TPG; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (4 * quarter + j < G) p_lds[wave][i][col][(4 * quarter + j) % G] = sc[i][j];
    }
    __builtin_amdgcn_wave_barrier();

    // ---- P.V ----------------------------------------------------------------------
#pragma unroll
    for (int i = 0; i < TPG; ++i) {
      if (!tv[i]) continue;
      const bool full = ntok[i] == 16;
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        const int n = s * RPS + rg;
        float pv[G];
#pragma unroll
        for (int h = 0; h < G; ++h) pv[h] = p_lds[wave][i][n][h];
        float v[EPL];
        unpack_chunk<T>(vr[i][s], v);
        if (!full && n >= ntok[i]) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) v[e] = 0.f;   // rows past the context may hold NaN
        }
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pv[h], v[e], acc[h][e]);
      }
    }
    __builtin_amdgcn_wave_barrier();
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

// Merge the partition records of every multi-partition (sequence, head), in
// partition order: M = max m_k, w_k = l_k * 2^(m_k - M), out = sum w_k o_k / sum w_k.
template <int D>
__global__ __launch_bounds__(D) void paged_attention_reduce_kernel(AttentionArgs a) {
  const int h = blockIdx.x % a.num_heads;
  const int seq = blockIdx.x / a.num_heads;
  const int d = threadIdx.x;
  const int ctx = a.context_lens[seq];
  const int max_ctx = a.max_blocks_per_seq << a.block_shift;
  if (ctx < 1 || ctx > max_ctx) return;
  const int nparts = (ctx + a.partition_size - 1) / a.partition_size;
  if (nparts <= 1) return;
  const int64_t row = (int64_t)seq * a.num_heads + h;
  const int64_t rec0 = row * a.max_parts;
  float M = -__builtin_inff();
  for (int k = 0; k < nparts; ++k) M = fmaxf(M, a.ws_m[rec0 + k]);
  float num = 0.f, den = 0.f;
  for (int k = 0; k < nparts; ++k) {
    const float w = a.ws_l[rec0 + k] * fast_exp2(a.ws_m[rec0 + k] - M);
    num = fmaf(w, a.ws_o[(rec0 + k) * D + d], num);
    den += w;
  }
  store_out(a.out, row * D + d, num / den, a.out_bf16);
}

// ---- dispatch ------------------------------------------------------------------

constexpr int kTilesPerGroup = 2;

template <typename T, int D>
static hipError_t launch_partition_g(const AttentionArgs& a, hipStream_t stream) {
  const int G = a.num_heads / a.num_kv_heads;
  const dim3 grid((unsigned)((int64_t)a.num_kv_heads * a.max_parts * a.num_seqs));
  const dim3 block(256);
  switch (G) {
    case 1: hipLaunchKernelGGL((paged_attention_partition_kernel<T, D, 1, kTilesPerGroup>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((paged_attention_partition_kernel<T, D, 2, kTilesPerGroup>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((paged_attention_partition_kernel<T, D, 4, kTilesPerGroup>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((paged_attention_partition_kernel<T, D, 8, kTilesPerGroup>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention_partition(const AttentionArgs& a, hipStream_t stream) {
  if (a.kv_bf16) {
    if (a.head_dim == 64) return launch_partition_g<BF16, 64>(a, stream);
    if (a.head_dim == 128) return launch_partition_g<BF16, 128>(a, stream);
  } else {
    if (a.head_dim == 64) return launch_partition_g<F32, 64>(a, stream);
    if (a.head_dim == 128) return launch_partition_g<F32, 128>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attention_reduce(const AttentionArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)a.num_heads * a.num_seqs));
  if (a.head_dim == 64)
    hipLaunchKernelGGL(paged_attention_reduce_kernel<64>, grid, dim3(64), 0, stream, a);
  else if (a.head_dim == 128)
    hipLaunchKernelGGL(paged_attention_reduce_kernel<128>, grid, dim3(128), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
