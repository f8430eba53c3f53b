// Device-side helpers shared by the gfx950 kernels of libpagedkv: element types,
// bfloat16 conversion, wave64 DPP reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Storage tags.  A 16-byte "chunk" is the unit every lane loads.
struct F32 {
  using storage = float;
  static constexpr int kElemBytes = 4;
  static constexpr int kPerChunk = 4;
};
struct BF16 {
  using storage = uint16_t;
  static constexpr int kElemBytes = 2;
  static constexpr int kPerChunk = 8;
};

// An 8-bit float cache (OCP E4M3: sign, 4 exponent bits biased by 7, 3 mantissa
// bits, no infinities, S.1111.111 the NaN, 448 the largest finite value).  Queries
// beside such a cache are bfloat16.
struct FP8 {
  using storage = uint8_t;
  static constexpr int kElemBytes = 1;
  static constexpr int kPerChunk = 16;
};

typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// E4M3 code of x, rounded to the nearest value with ties to the even code; finite
// magnitudes of 448 and beyond (and infinities) give +-448, NaN gives 0x7F.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;                  // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;          // |x| >= 448
  if (a < 0x3c800000u)                                // |x| < 2^-6: codes m * 2^-9
    return sign | static_cast<uint32_t>(__builtin_rintf(__uint_as_float(a) * 512.f));
  // normal: move the exponent bias from 127 to 7, then round the 23 mantissa bits
  // to 3, ties to even (a carry out of the mantissa raises the exponent)
  uint32_t b = a - (120u << 23);
  b += 0x7ffffu + ((b >> 20) & 1u);
  return sign | (b >> 20);
}

// Four E4M3 codes (one 32-bit word, lowest byte first) to fp32 or bfloat16; every
// E4M3 value is exact in both.
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float* v) {
  const floatx2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  const floatx2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  v[0] = lo[0]; v[1] = lo[1]; v[2] = hi[0]; v[3] = hi[1];
}
__device__ __forceinline__ uint2 e4m3x4_to_bf16(uint32_t w) {
  const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, false);
  const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, true);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// bfloat16 -> fp32 is exact: the 16 bits are the top half of the fp32 pattern.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bfloat16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Unpack one 16-byte chunk into fp32 values.
template <typename T>
__device__ __forceinline__ void unpack_chunk(const uint4& c, float* v);

template <>
__device__ __forceinline__ void unpack_chunk<F32>(const uint4& c, float* v) {
  v[0] = __uint_as_float(c.x);
  v[1] = __uint_as_float(c.y);
  v[2] = __uint_as_float(c.z);
  v[3] = __uint_as_float(c.w);
}

template <>
__device__ __forceinline__ void unpack_chunk<BF16>(const uint4& c, float* v) {
  v[0] = bf16_lo(c.x); v[1] = bf16_hi(c.x);
  v[2] = bf16_lo(c.y); v[3] = bf16_hi(c.y);
  v[4] = bf16_lo(c.z); v[5] = bf16_hi(c.z);
  v[6] = bf16_lo(c.w); v[7] = bf16_hi(c.w);
}

// ---- DPP within one 16-lane row of a wave64 -------------------------------------
// Control codes of the gfx9 data-parallel-primitive lane selectors.
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowMirror = 0x140;   // lane r <- lane 15-r
constexpr int kDppRowHalfMirror = 0x141;  // lane r <- lane 7-r within each half-row

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}

// After these four steps every lane of a 16-lane row holds the row's result.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<kDppRowMirror>(x));
  x = fmaxf(x, dpp<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp<kDppQuadXor2>(x));
  x = fmaxf(x, dpp<kDppQuadXor1>(x));
  return x;
}

// Order-preserving integer keys of floats (any value but NaN): a signed integer
// compare of the keys orders the floats, so maxima can use the integer max, which
// needs no NaN canonicalisation and fuses with DPP lane moves.
__device__ __forceinline__ int float_key(float x) {
  const int b = __float_as_int(x);
  return b ^ ((b >> 31) & 0x7fffffff);
}
__device__ __forceinline__ float key_float(int k) {
  return __int_as_float(k ^ ((k >> 31) & 0x7fffffff));
}

template <int kCtrl>
__device__ __forceinline__ int dpp_i(int x) {
  // all rows and banks enabled, so bound_ctrl never applies; it lets the move fuse
  // into the instruction that consumes it
  return __builtin_amdgcn_mov_dpp(x, kCtrl, 0xF, 0xF, true);
}

// Maximum of the keys over the first N lanes (N = 8 or 16) of every 16-lane row;
// lanes 0..N-1 of each row receive it.
template <int N>
__device__ __forceinline__ int row_max_key(int k) {
  static_assert(N == 8 || N == 16, "row span");
  if constexpr (N == 16) k = max(k, dpp_i<kDppRowMirror>(k));
  k = max(k, dpp_i<kDppRowHalfMirror>(k));
  k = max(k, dpp_i<kDppQuadXor2>(k));
  k = max(k, dpp_i<kDppQuadXor1>(k));
  return k;
}

__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<kDppRowMirror>(x);
  x += dpp<kDppRowHalfMirror>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppQuadXor1>(x);
  return x;
}

__device__ __forceinline__ float readlane(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pkv
