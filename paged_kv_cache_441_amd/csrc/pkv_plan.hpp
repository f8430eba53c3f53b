// The attention work plan (device side), shared by the standalone plan kernel and
// the fused decode prologue.
#pragma once

#include "pkv_device.hpp"
#include "pkv_launch.hpp"

namespace pkv {

// ---- work plan -------------------------------------------------------------------
// The partition kernel's grid is sized for the longest context the block tables
// allow, so most of its workgroups may find nothing to do, and the hardware hands
// out workgroups in index order.  The plan lists the real (sequence, partition)
// work items so that workgroup k takes item k / num_kv_heads: every whole
// partition first, then the partial last partitions, longest first (eight size
// classes), then nothing.  Dispatching the longest items first keeps the end of
// the kernel from waiting on a few long ones, and the idle workgroups all sit at
// the end of the grid where they cost almost nothing.  A sequence with an invalid
// context length gets one item, whose workgroups write its NaN output.
constexpr int kPlanThreads = 1024;   // threads of the standalone plan kernel
constexpr int kPlanClasses = 8;
constexpr int kPlanCats = 1 + kPlanClasses;   // whole partitions, then the size classes

// Work items of sequence i in category k (0: whole partitions, 1 + c: a partial
// last partition of size class c).
struct PlanCounts {
  int n[kPlanCats];
};

__device__ __forceinline__ PlanCounts plan_counts(int ctx, bool exists, int P, int max_ctx) {
  PlanCounts c;
#pragma unroll
  for (int k = 0; k < kPlanCats; ++k) c.n[k] = 0;
  if (!exists) return c;
  const bool valid = ctx >= 1 && ctx <= max_ctx;
  c.n[0] = valid ? ctx / P : 1;
  const int rem = valid ? ctx % P : 0;
  if (rem > 0) {
    const int cls = (int)(((int64_t)(P - rem) * kPlanClasses) / P);
#pragma unroll
    for (int k = 0; k < kPlanClasses; ++k) c.n[1 + k] = cls == k;
  }
  return c;
}

// Exclusive prefix sums of all categories over the workgroup at once; tot
// receives the workgroup totals.
template <int NT>
__device__ __forceinline__ PlanCounts plan_scan(const PlanCounts& x, int (*lds)[kPlanCats],
                                                PlanCounts* tot) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  PlanCounts inc = x;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
#pragma unroll
    for (int k = 0; k < kPlanCats; ++k) {
      const int y = __shfl_up(inc.n[k], off);
      if (lane >= off) inc.n[k] += y;
    }
  }
  if (lane == kWave - 1) {
#pragma unroll
    for (int k = 0; k < kPlanCats; ++k) lds[wave][k] = inc.n[k];
  }
  __syncthreads();
  PlanCounts ex;
#pragma unroll
  for (int k = 0; k < kPlanCats; ++k) {
    int before = 0, all = 0;
    for (int w = 0; w < NT / kWave; ++w) {
      const int t = lds[w][k];
      before += w < wave ? t : 0;
      all += t;
    }
    ex.n[k] = before + inc.n[k] - x.n[k];
    tot->n[k] = all;
  }
  __syncthreads();
  return ex;
}

// Builds the plan with the NT threads of the calling workgroup (every thread must
// call it).  Items go to items[0 .. *count).
template <int NT>
__device__ void build_plan(const int32_t* __restrict__ context_lens, int num_seqs, int P,
                           int max_ctx, int4* __restrict__ items, int* __restrict__ count) {
  __shared__ int lds[NT / kWave][kPlanCats];
  const bool one_chunk = num_seqs <= NT;
  int base[kPlanCats], carry[kPlanCats];
#pragma unroll
  for (int k = 0; k < kPlanCats; ++k) carry[k] = 0;
  if (!one_chunk) {
    // totals first, so that every category's items start after all earlier ones
    PlanCounts tot_all{};
    for (int c0 = 0; c0 < num_seqs; c0 += NT) {
      const int i = c0 + threadIdx.x;
      const PlanCounts x = plan_counts(i < num_seqs ? context_lens[i] : 0, i < num_seqs,
                                       P, max_ctx);
      PlanCounts t;
      plan_scan<NT>(x, lds, &t);
#pragma unroll
      for (int k = 0; k < kPlanCats; ++k) tot_all.n[k] += t.n[k];
    }
    int acc = 0;
#pragma unroll
    for (int k = 0; k < kPlanCats; ++k) {
      base[k] = acc;
      acc += tot_all.n[k];
    }
  }
  int total = 0;
  for (int c0 = 0; c0 < num_seqs; c0 += NT) {
    const int i = c0 + threadIdx.x;
    const int ctx = i < num_seqs ? context_lens[i] : 0;
    const PlanCounts x = plan_counts(ctx, i < num_seqs, P, max_ctx);
    PlanCounts t;
    const PlanCounts ex = plan_scan<NT>(x, lds, &t);
    if (one_chunk) {
      int acc = 0;
#pragma unroll
      for (int k = 0; k < kPlanCats; ++k) {
        base[k] = acc;
        acc += t.n[k];
      }
    }
    const bool valid = ctx >= 1 && ctx <= max_ctx;
    const int nparts = valid ? (ctx + P - 1) / P : 1;
    const int pos0 = base[0] + carry[0] + ex.n[0];
    for (int p = 0; p < x.n[0]; ++p) items[pos0 + p] = make_int4(i, p, ctx, nparts);
#pragma unroll
    for (int k = 1; k < kPlanCats; ++k)
      if (x.n[k]) items[base[k] + carry[k] + ex.n[k]] = make_int4(i, x.n[0], ctx, nparts);
#pragma unroll
    for (int k = 0; k < kPlanCats; ++k) {
      carry[k] += t.n[k];
      total += t.n[k];
    }
  }
  if (threadIdx.x == 0) *count = total;
}

// ---- tile plan (balanced split) -------------------------------------------------------
// In the balanced mode the attention work is the ordered list of all (sequence,
// tile) pairs, a tile being kTileTokens consecutive tokens of one sequence, each
// sequence's tiles preceded by kSeqCost positions that stand for its fixed cost;
// the partition stage cuts the list into equal contiguous shares, one per
// workgroup.  The plan is the exclusive prefix sum of the positions: cum[i]
// positions precede sequence i (i = 0..num_seqs), and hdr[0] = cum[num_seqs] is
// the total.  A sequence with an invalid context length has no positions.
// (kTileTokens, kSeqCost: pkv_launch.hpp.)

template <int NT>
__device__ void build_tile_plan(const int32_t* __restrict__ context_lens, int num_seqs,
                                int max_ctx, int* __restrict__ cum, int* __restrict__ hdr) {
  __shared__ int lds[NT / kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  int carry = 0;
  for (int c0 = 0; c0 < num_seqs; c0 += NT) {
    const int i = c0 + threadIdx.x;
    const int ctx = i < num_seqs ? context_lens[i] : 0;
    const int x =
        (ctx >= 1 && ctx <= max_ctx) ? (ctx + kTileTokens - 1) / kTileTokens + kSeqCost : 0;
    int inc = x;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(inc, off);
      if (lane >= off) inc += y;
    }
    if (lane == kWave - 1) lds[wave] = inc;
    __syncthreads();
    int before = 0, total = 0;
    for (int w = 0; w < NT / kWave; ++w) {
      const int t = lds[w];
      before += w < wave ? t : 0;
      total += t;
    }
    if (i < num_seqs) cum[i] = carry + before + inc - x;
    carry += total;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    cum[num_seqs] = carry;
    hdr[0] = carry;
  }
}

}  // namespace pkv
