// Per-tile device pieces shared by the paged-attention kernels of libpagedkv:
// the tile geometry, the Q.K^T scores of one 16-token tile on the matrix cores,
// and output stores.
#pragma once

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

// One lane's part of a query-key dot product on the VALU: its QKC 16-byte chunks of
// one head's query against the same dims of a key row, bfloat16 pairs by v_dot2 (the
// products are exact in fp32) or fp32 FMAs; two partial sums for a shorter chain.
// For GQA groups of one or two heads, where a 16-row matrix instruction would hold
// one or two real rows.
template <typename T, int QKC>
__device__ __forceinline__ float lane_dot(const uint4 (&q)[QKC], const uint4 (&k)[QKC]) {
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int c = 0; c < QKC; ++c) {
    if constexpr (T::kElemBytes == 4) {
      s0 = fmaf(__uint_as_float(q[c].x), __uint_as_float(k[c].x), s0);
      s1 = fmaf(__uint_as_float(q[c].y), __uint_as_float(k[c].y), s1);
      s0 = fmaf(__uint_as_float(q[c].z), __uint_as_float(k[c].z), s0);
      s1 = fmaf(__uint_as_float(q[c].w), __uint_as_float(k[c].w), s1);
    } else {
      s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q[c].x),
                                          __builtin_bit_cast(bf16x2, k[c].x), s0, false);
      s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q[c].y),
                                          __builtin_bit_cast(bf16x2, k[c].y), s1, false);
      s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q[c].z),
                                          __builtin_bit_cast(bf16x2, k[c].z), s0, false);
      s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q[c].w),
                                          __builtin_bit_cast(bf16x2, k[c].w), s1, false);
    }
  }
  return s0 + s1;
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

// ---- log-sum-exp merge of partial results -----------------------------------------
// A partial result over part of a context is (m, l, o): the maximum score (base-2
// exponent domain), the sum of 2^(s - m) and the normalised output o.  Two such
// results merge into the one over both parts.
struct Running {
  float m;     // running maximum (base-2 exponent domain); -inf when empty
  float l;     // sum of weights relative to m
  float4 o;    // weighted partial outputs relative to m
};

__device__ __forceinline__ float rel_scale(float m_old, float m_new) {
  return m_old == -__builtin_inff() ? 0.f : fast_exp2(m_old - m_new);
}

__device__ __forceinline__ void merge_into(Running& r, const Running& s) {
  const float mn = fmaxf(r.m, s.m);
  const float fr = rel_scale(r.m, mn), fs = rel_scale(s.m, mn);
  r.l = r.l * fr + s.l * fs;
  r.o.x = r.o.x * fr + s.o.x * fs;
  r.o.y = r.o.y * fr + s.o.y * fs;
  r.o.z = r.o.z * fr + s.o.z * fs;
  r.o.w = r.o.w * fr + s.o.w * fs;
  r.m = mn;
}

template <int N>
__device__ __forceinline__ void accumulate(Running& r, const float (&m)[N], const float (&l)[N],
                                           const float4 (&o)[N], const bool (&live)[N]) {
  float mb = r.m;
#pragma unroll
  for (int u = 0; u < N; ++u) mb = live[u] ? fmaxf(mb, m[u]) : mb;
  const float f = rel_scale(r.m, mb);
  r.l *= f;
  r.o.x *= f; r.o.y *= f; r.o.z *= f; r.o.w *= f;
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const float w = live[u] ? l[u] * fast_exp2(m[u] - mb) : 0.f;
    r.l += w;
    r.o.x = fmaf(w, o[u].x, r.o.x);
    r.o.y = fmaf(w, o[u].y, r.o.y);
    r.o.z = fmaf(w, o[u].z, r.o.z);
    r.o.w = fmaf(w, o[u].w, r.o.w);
  }
  r.m = mb;
}

// Four consecutive outputs from idx (a multiple of 4) in one store.
__device__ __forceinline__ void store_row4(const AttentionArgs& a, int64_t idx, const Running& r) {
  const float x = r.o.x / r.l, y = r.o.y / r.l, z = r.o.z / r.l, w = r.o.w / r.l;
  if (a.out_bf16) {
    const uint2 v = make_uint2(f32_to_bf16_rne(x) | (uint32_t)f32_to_bf16_rne(y) << 16,
                               f32_to_bf16_rne(z) | (uint32_t)f32_to_bf16_rne(w) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + idx) = v;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(a.out) + idx) = make_float4(x, y, z, w);
  }
}

}  // namespace pkv
