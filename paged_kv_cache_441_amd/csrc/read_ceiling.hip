// Read-bandwidth ceilings for the benchmark (libpkv_ceiling.so; not part of the
// libpagedkv ABI).  Two load-only kernels give the rates that the decode kernel's
// memory traffic can be compared with in the same process:
//
//  - pkv_ceiling_block_read: whole KV blocks of both caches, in the order of a list of
//    physical block ids (the blocks a decode batch references, in table order), each
//    block read as contiguous 16-byte non-temporal loads.  This is the decode kernel's
//    access pattern without its compute: the same bytes, the same placement in the
//    pool, the same cache policy.
//  - pkv_ceiling_linear_read: one contiguous buffer streamed with 16-byte
//    non-temporal loads, eight in flight per lane.
//
// Both fold what they load into one 16-byte value per thread, written to `sink`, so
// the loads cannot be dropped.  Every load is in bounds: block ids are checked on
// the host against the pool, and the block loop reads exactly block_bytes per block.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// Workgroup w reads blocks w, w + gridDim.x, ...; a block's bytes of both caches
// are spread over the workgroup's lanes, loads of one round issued before any is used.
__global__ __launch_bounds__(kThreads) void block_read_kernel(
    const u32x4* __restrict__ kc, const u32x4* __restrict__ vc, const int32_t* __restrict__ ids,
    int n_blocks, int64_t block_vecs, u32x4* __restrict__ sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int j = blockIdx.x; j < n_blocks; j += gridDim.x) {
    const int64_t base = (int64_t)ids[j] * block_vecs;
    for (int64_t i = threadIdx.x; i < block_vecs; i += 4 * kThreads) {
      u32x4 v[8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t e = i + (int64_t)u * kThreads;
        const int64_t c = e < block_vecs ? e : block_vecs - 1;   // clamp: stays in the block
        v[2 * u] = __builtin_nontemporal_load(kc + base + c);
        v[2 * u + 1] = __builtin_nontemporal_load(vc + base + c);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc ^= v[u];
    }
  }
  sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

__global__ __launch_bounds__(kThreads) void linear_read_kernel(const u32x4* __restrict__ in,
                                                               int64_t n,
                                                               u32x4* __restrict__ sink) {
  const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int64_t i = tid;
  for (; i + 7 * stride < n; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(in + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  for (; i < n; i += stride) acc ^= in[i];
  sink[tid] = acc;
}

}  // namespace

extern "C" {

// sink: device buffer of grid * 256 * 16 bytes.  Returns a hipError_t value.
int pkv_ceiling_block_read(const void* key_cache, const void* value_cache,
                           const int32_t* block_ids, int32_t n_blocks, int64_t block_bytes,
                           int32_t grid, void* sink, void* stream) {
  if (!key_cache || !value_cache || !block_ids || !sink || n_blocks <= 0 || grid <= 0 ||
      block_bytes <= 0 || block_bytes % 16 != 0)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(block_read_kernel, dim3(grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(key_cache),
                     static_cast<const u32x4*>(value_cache), block_ids, n_blocks,
                     block_bytes / 16, static_cast<u32x4*>(sink));
  return hipGetLastError();
}

// sink: device buffer of grid * 256 * 16 bytes; bytes a multiple of 16.
int pkv_ceiling_linear_read(const void* buf, int64_t bytes, int32_t grid, void* sink,
                            void* stream) {
  if (!buf || !sink || bytes <= 0 || bytes % 16 != 0 || grid <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(linear_read_kernel, dim3(grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf),
                     bytes / 16, static_cast<u32x4*>(sink));
  return hipGetLastError();
}

}  // extern "C"
