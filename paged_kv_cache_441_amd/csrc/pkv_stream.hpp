// Pieces shared by the streaming attention kernels of libpagedkv (decode and
// multi-token steps): direct-to-LDS tile copies with explicit waits, the LDS image of
// a tile, and the equal shares of a work list.
#pragma once

#include <atomic>

#include "pkv_device.hpp"
#include "pkv_launch.hpp"

namespace pkv {

// Reads through the constant address space become scalar loads when the address is
// wave-uniform; used for data no kernel of this launch writes (tables, lengths, the
// tile plan), so their waits do not hold up the tile copies in flight.
typedef const int32_t __attribute__((address_space(4))) cint32;

// A workgroup barrier with no memory fence: the fence of __syncthreads would wait
// for every outstanding copy, including the ones meant to stay in flight.  The
// memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void bare_barrier() { asm volatile("s_barrier" ::: "memory"); }

// One direct-to-LDS copy: lane i's 16 bytes at base + off (base wave-uniform) land at
// LDS byte lds + 16 i.  Written as assembly so that the compiler, which cannot tell
// the ring's buffers apart once more than a few copies are in flight, adds no wait
// for it before LDS reads; the kernel waits for the copies itself (s_waitcnt vmcnt)
// before the barrier that hands a tile to the readers.
// Cache policy of a copy.  kStream sets the non-temporal bit: for KV tiles that a
// launch reads once, streaming them past the caches raised the decode kernel's rate
// on MI355X from 5.7 to 6.4 TB/s (Llama-3-8B-shaped batch); sc0/sc1 scope bits made
// no difference.
enum class Cpol { kDefault, kStream };
template <Cpol P = Cpol::kDefault>
__device__ __forceinline__ void dma16(const char* base, uint32_t off, uint32_t lds) {
  if constexpr (P == Cpol::kStream)
    asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
  else
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
}

// Reductions of x over lanes l and l ^ 16, or l and l ^ 32, by gfx950's lane-row swaps
// (no LDS round trip): swapping a register with itself hands each lane, in its two
// results, its own value and its partner's, so max and sum need no select.
__device__ __forceinline__ float max_xor16(float x) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// An empty statement with side effects: the block holding it stays a real branch,
// instead of being executed on every path and selected away (the compiler does that
// to short blocks), for rare paths such as a rescale or a partial tile.
__device__ __forceinline__ void keep_branch() { asm volatile(""); }

// Waits until at most N of this wave's copies are outstanding; copies retire in
// order, so every copy issued before the last N has landed in LDS.
template <int N>
__device__ __forceinline__ void wait_copies() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// s_waitcnt immediate for vmcnt(0) with the other counters unconstrained (gfx9
// layout: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).  Unlike the
// assembly waits above, the compiler sees this one.
constexpr int kWaitVmcnt0 = (0x7 << 4) | (0xf << 8);

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(__attribute__((address_space(3))) const void*)p;
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <typename T, int D, int HW, int TOK>
struct Stage;

// The LDS image of one tile: TOK token rows of HW heads, copied by NW waves (NW = HW
// when each wave owns a head, more when several waves share one head's rows).
template <typename T, int D, int HW, int TOK, int NW>
struct StageW {
  static constexpr int kRowBytes = HW * D * T::kElemBytes;   // one token row of the HW heads
  static constexpr int kSlots = kRowBytes / 16;               // 16-byte slots per row
  static constexpr int kSwz = kSlots >= 16 ? 15 : kSlots - 1;
  // The XOR pattern of row r.  E4M3 rows are read as 8-byte value pieces, 16 lanes
  // per row and two rows (r, r ^ 1) per 32-lane half of a read: their patterns differ
  // in the top bit, so the two rows' 128 bytes land in different bank halves.
  static __device__ __forceinline__ int swz(int r) {
    if constexpr (T::kElemBytes == 1)
      return ((r & 1) ? (kSwz + 1) >> 1 : 0) | ((r & kSwz) >> 1);
    else
      return r & kSwz;
  }
  static constexpr int kTileBytes = TOK * kRowBytes;          // per cache
  static constexpr int kTileSlots = kTileBytes / 16;
  static constexpr int kCopies = kTileBytes / (NW * 1024);    // 1 KiB copies per wave and cache
  static_assert(kTileBytes % (NW * 1024) == 0, "a tile splits into 1 KiB wave copies");
  static_assert(kSlots >= 8, "rows of at least 128 bytes");
};

template <typename T, int D, int HW, int TOK>
struct Stage : StageW<T, D, HW, TOK, HW> {};

// Workgroups are handed to the 8 XCDs of an MI355X round-robin (workgroup i to XCD
// i % 8), and each XCD has its own L2.  This gives the workgroups of one XCD
// consecutive share indices (XCD x takes shares [x * n / 8, (x + 1) * n / 8)), so
// that neighbouring shares, which read the same sequence's tiles at about the same
// time when a sequence spans many units, meet in one L2.  Identity when the grid is
// not a multiple of 8.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_local_share(int block, int nwg) {
  if (nwg % kXcds != 0) return block;
  return (block % kXcds) * (nwg / kXcds) + block / kXcds;
}

// floor(n / d) for 0 <= n and 0 < d < 2^31: 32-bit division when n fits (the common
// case; a 64-bit division is a long instruction sequence on the GPU).
__device__ __forceinline__ int64_t div_floor(int64_t n, int d) {
  if (n <= 0xffffffffll) return (int64_t)((uint32_t)n / (uint32_t)d);
  return n / d;
}

// Share w of the tile list is [floor(w * total / nwg), floor((w + 1) * total / nwg)).
// The share holding tile j:
__device__ __forceinline__ int share_of(int64_t j, int nwg, int total) {
  return (int)div_floor((j + 1) * nwg - 1, total);
}

// Shares are empty when there are more workgroups than tiles.
__device__ __forceinline__ bool share_nonempty(int w, int nwg, int total) {
  return div_floor((int64_t)w * total, nwg) < div_floor((int64_t)(w + 1) * total, nwg);
}

// Compute units of the current device, looked up once per device.
inline int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace pkv
