// Paged attention for steps that hand each sequence several new tokens: a chunk of a
// long prompt, or the tokens a draft model proposed, to be verified.
//
// What is computed (page "读一个真实 serving 系统 · vLLM 架构巡礼", section 3: one
// scheduler for all steps, each request getting some new tokens; page "vLLM
// PagedAttention 原理与源码深度解析", sections 8.1 and 8.2, chunked prefill and
// speculative decoding; page "vllm源码剖析", section 一.3, the requests packed into one
// flat token batch with a start and a length each): sequence i's new tokens are
// query_start_loc[i] .. query_start_loc[i+1] - 1 of the flat batch; context_lens[i]
// counts them, so new token j sits at position p = ctx - q_len + j, and it attends
// to positions 0 .. p of its sequence.  A step with one new token per sequence is a
// decode step.
//
// Work split.  Rows are (new token, query head) pairs; the rows of one sequence and
// kv head are cut into units of 16 or 32 rows (R / G consecutive new tokens with the
// G query heads of the kv head each), one or two MFMA operands.  A unit
// reads the tiles of its sequence up to its last token's position.  As in the
// balanced decode split, all (unit, tile) pairs form one list, each unit preceded
// by kSeqCost positions, and a one-round grid takes equal shares of it; the run of
// one unit inside a share is a segment, written directly when it is the whole unit
// and as records under the label w + unit otherwise, merged afterwards in share order.
//
// Per tile (16 tokens of the HW kv heads of the workgroup, staged whole through LDS
// with direct-to-LDS copies as in the decode stream kernel):
//  - S^T = K . Q^T on the matrix cores: the key tile is the A operand and the unit's
//    16 query rows the B operand, so lane (row n, quarter q) receives row n's scores
//    for tokens 4q .. 4q + 3.  Those four values are already the lane's part of the
//    P operand of P.V, so no transpose through LDS is needed.
//  - causal mask (token t visible to a row at position p when t <= p), online
//    softmax per row in the base-2 domain with the lazy rebase of the decode kernel;
//    row maxima and sums across the four lanes of a row by lane shuffles.
//  - P.V on the matrix cores.  Each lane reads D / 16 consecutive value columns of a
//    token row in one LDS read, one column per output block, so the value tile needs
//    no transpose either (output block e holds columns e, e + D/16, ...; undone at
//    the store).  bf16 caches: P split into bf16 hi + lo parts, together exact to
//    about 2^-17 of p (a single bf16 P could move outputs by up to ~5e-3), on the
//    full-rate v_mfma_f32_16x16x32_bf16: lane quarter q supplies the hi and then the
//    lo parts of tokens 4q .. 4q + 3 as its eight k values (A), and the same tokens'
//    value rows twice (B, packed from four token rows); fp32 caches:
//    v_mfma_f32_16x16x4_f32 with fp32 P, k-step s taking token 4q + s from lane
//    quarter q.
//  - A unit is one or two MFMA row blocks (16 or 32 rows: two when the sequences
//    average more than 16 rows), so up to 32 rows share one pass over the tiles.
#include "pkv_device.hpp"
#include "pkv_launch.hpp"
#include "pkv_stream.hpp"
#include "pkv_tile.hpp"

#include <cstdlib>
#include <type_traits>

namespace pkv {

// ---- slot mapping of every new token ---------------------------------------------

// Sequence owning flat token t: the last i with query_start_loc[i] <= t (binary search
// over num_seqs + 1 entries; the caller checks the answer).
__device__ __forceinline__ int owner_of(const int32_t* __restrict__ qsl, int num_seqs, int t) {
  int lo = 0, hi = num_seqs;   // qsl[lo] <= t is assumed for lo = 0
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (qsl[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// Whether sequence i is a well-formed part of the step: its tokens lie inside the
// flat batch, there is at least one, and its context holds them and fits its table.
__device__ __forceinline__ bool seq_valid(int q0, int q1, int ctx, int num_tokens, int max_ctx) {
  return q0 >= 0 && q1 > q0 && q1 <= num_tokens && ctx >= q1 - q0 && ctx <= max_ctx;
}

__global__ __launch_bounds__(256) void slot_mapping_multi_kernel(
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    const int32_t* __restrict__ qsl, int32_t* __restrict__ slot_mapping, int num_seqs,
    int num_tokens, int max_blocks_per_seq, int block_shift, int64_t num_blocks) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= num_tokens) return;
  const int i = owner_of(qsl, num_seqs, t);
  const int q0 = qsl[i], q1 = qsl[i + 1], ctx = context_lens[i];
  int32_t slot = -1;
  if (seq_valid(q0, q1, ctx, num_tokens, max_blocks_per_seq << block_shift) && t >= q0 &&
      t < q1) {
    const int pos = ctx - (q1 - q0) + (t - q0);
    const int32_t phys = block_tables[(int64_t)i * max_blocks_per_seq + (pos >> block_shift)];
    if (phys >= 0 && (int64_t)phys < num_blocks)
      slot = (phys << block_shift) + (pos & ((1 << block_shift) - 1));
  }
  slot_mapping[t] = slot;
}

hipError_t launch_slot_mapping_multi(const int32_t* block_tables, const int32_t* context_lens,
                                     const int32_t* query_start_loc, int32_t* slot_mapping,
                                     int num_seqs, int num_tokens, int max_blocks_per_seq,
                                     int block_shift, int64_t num_blocks, hipStream_t stream) {
  const int grid = (num_tokens + 255) / 256;
  hipLaunchKernelGGL(slot_mapping_multi_kernel, dim3(grid), dim3(256), 0, stream, block_tables,
                     context_lens, query_start_loc, slot_mapping, num_seqs, num_tokens,
                     max_blocks_per_seq, block_shift, num_blocks);
  return hipGetLastError();
}

// ---- the unit plan ---------------------------------------------------------------
// hdr[0]: positions of the list; hdr[1]: workgroups per kv-head group (written by the
// attention kernel); hdr[2]: units.  seq_unit[i]: first unit of sequence i (units of
// invalid sequences: none); unit_seq[u]: the sequence of unit u; cum[u]: positions
// before unit u.  If the units would exceed the workspace (possible only when
// query_start_loc is not a non-decreasing cut of the flat batch), the plan has none
// and every output row is NaN.

constexpr int kMqPlanThreads = 1024;

size_t multi_plan_bytes(int64_t num_seqs, int64_t max_units) {
  auto r256 = [](int64_t b) { return (size_t)((b + 255) / 256 * 256); };
  return 256 + r256((max_units + 1) * 4) + r256(max_units * 4) + r256((num_seqs + 1) * 4);
}

// Exclusive prefix sum over the workgroup of x(k) for k < n into out[k]; returns the
// total.  NT threads; every thread calls it.
template <int NT, typename F>
__device__ int block_scan(int n, F x_of, int* __restrict__ out) {
  __shared__ int part[NT / kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  int carry = 0;
  for (int c0 = 0; c0 < n; c0 += NT) {
    const int k = c0 + threadIdx.x;
    const int x = k < n ? x_of(k) : 0;
    int inc = x;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(inc, off);
      if (lane >= off) inc += y;
    }
    if (lane == kWave - 1) part[wave] = inc;
    __syncthreads();
    int before = 0, total = 0;
    for (int v = 0; v < NT / kWave; ++v) {
      const int t = part[v];
      before += v < wave ? t : 0;
      total += t;
    }
    if (k < n) out[k] = carry + before + inc - x;
    carry += total;
    __syncthreads();
  }
  return carry;
}

// ---- prefill schedule ------------------------------------------------------------------
// Prefill units (kMqPrefillUnit rows over the unit's whole causal context) are split
// into pieces along the context, so that long histories no longer set the kernel's
// time; the piece that finishes last merges them.  With P the batch's tiles per
// workgroup (rounded up), an item of n tiles takes k = clamp(round(2 n / P), 1,
// kPfMaxPieces) pieces: two on an even batch (about two pieces per workgroup), up to
// kPfMaxPieces for the items of a history much longer than the rest, and one (no
// record, no merge) for items much shorter.  The pieces are
// dealt to the XCDs by (sequence, kv head) group, group k to XCD k % kXcds with the
// groups ranked by context length (longest first): the units of one group share their
// tiles in one L2, and every XCD gets a similar mix.  Within an XCD the groups' pieces
// form one list, largest first (a group's units last to first, an item's pieces in
// order); the XCD's workgroups take it in snake order (round r: workgroup j takes
// position rW + j, or rW + W - 1 - j on odd rounds), which pairs large pieces with
// small ones.
//
// Workspace (words; NI = max_units * num_kv_heads items, NG = num_seqs * num_kv_heads
// groups, J = ceil(NG / kXcds), K = kPfMaxPieces):
//   m array: the records' m values [K NI * kMqPrefillUnit], then the per-XCD prefix sums
//            of pieces over its groups [kXcds][J + 1], then the ranked sequences [B],
//            then the plan's scan [kXcds J + 1];
//   l array: the records' l values [K NI * kMqPrefillUnit], then one counter per item;
//   o array: the records' rows [K NI * kMqPrefillUnit][head_dim].
// Record of piece h of item i, row r: (K i + h) * kMqPrefillUnit + r.  The tile target
// P is tile_hdr[4].
constexpr int kPfTok = 32;   // tokens per tile of the prefill kernel

struct PrefillLayout {
  int NI, NG, J;
  int* xcum;    // [kXcds][J + 1]
  int* order;   // [num_seqs]: sequence of each rank
  int* scan;    // [kXcds J + 1]: the plan's scan, XCD-major
  int* ctr;     // [NI]
  __device__ explicit PrefillLayout(const AttentionArgs& a) {
    NI = a.max_units * a.num_kv_heads;
    NG = a.num_seqs * a.num_kv_heads;
    J = (NG + kXcds - 1) / kXcds;
    xcum = reinterpret_cast<int*>(a.ws_m + (int64_t)kPfMaxPieces * NI * kMqPrefillUnit);
    order = xcum + kXcds * (J + 1);
    scan = order + a.num_seqs;
    ctr = reinterpret_cast<int*>(a.ws_l + (int64_t)kPfMaxPieces * NI * kMqPrefillUnit);
  }
};

// Tiles of the causal context of unit `unit` of a sequence (tpb new tokens per unit).
__device__ __forceinline__ int pf_unit_tiles(int ctx, int qlen, int unit, int tpb) {
  const int j1 = min(qlen, (unit + 1) * tpb);
  return (ctx - qlen + j1 + kPfTok - 1) / kPfTok;
}
// Pieces of an item of n tiles, P the tile target: 2 n / P rounded to the nearest (32-bit
// arithmetic: n is below 2^26 tiles, P below 2^30).
__device__ __forceinline__ int pf_pieces(int n, int P) {
  const uint32_t k = (4u * (uint32_t)n + (uint32_t)P) / (2u * (uint32_t)P);
  return min(kPfMaxPieces, max(1, (int)k));
}

// Sequences are ranked only up to this many (beyond, they keep their index order).
constexpr int kPfRankMax = 1024;

__device__ void build_prefill_schedule(const AttentionArgs& a, int U) {
  const int B = a.num_seqs, Hkv = a.num_kv_heads;
  const int tpb = kMqPrefillUnit / (a.num_heads / Hkv);
  const PrefillLayout L(a);
  for (int i = threadIdx.x; i < U * Hkv; i += kMqPlanThreads) L.ctr[i] = 0;
  // One pass over the sequences: the rank key (context length; -1 for a sequence
  // without units, ranked last) and the tiles of its units, summed for the tile target
  // (all items' tiles over the launch's workgroups).  Up to kPfRankMax sequences, their
  // lengths, rank and pieces are kept in LDS.
  const bool small = B <= kPfRankMax;
  __shared__ int key[kPfRankMax], qlen_s[kPfRankMax], pcs_s[kPfRankMax], ord_s[kPfRankMax];
  __shared__ unsigned long long tiles_all;
  if (threadIdx.x == 0) tiles_all = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < B; i += kMqPlanThreads) {
    const int nun = a.seq_unit[i + 1] - a.seq_unit[i];
    const int ctx = a.context_lens[i];
    const int qlen = a.query_start_loc[i + 1] - a.query_start_loc[i];
    unsigned long long t = 0;
    for (int u = 0; u < nun; ++u) t += pf_unit_tiles(ctx, qlen, u, tpb);
    if (t) atomicAdd(&tiles_all, t);
    if (small) {
      key[i] = nun > 0 ? ctx : -1;
      qlen_s[i] = nun > 0 ? qlen : 0;
    }
  }
  __syncthreads();
  const int64_t all = (int64_t)tiles_all * Hkv;
  const int P = (int)min((int64_t)1 << 30, max((int64_t)1, (all + a.grid_wgs - 1) / a.grid_wgs));
  if (threadIdx.x == 0) a.tile_hdr[4] = P;
  // pieces of sequence i's units (every kv head's group of it has as many)
  auto seq_pieces = [&](int i, int ctx, int qlen) {
    const int nun = (qlen + tpb - 1) / tpb;
    int n = 0;
    for (int u = 0; u < nun; ++u) n += pf_pieces(pf_unit_tiles(ctx, qlen, u, tpb), P);
    return n;
  };
  // rank: longest first (ties by index)
  if (small) {
    for (int i = threadIdx.x; i < B; i += kMqPlanThreads) {
      const int ki = key[i];
      int r = 0;
      for (int j = 0; j < B; ++j) {
        const int kj = key[j];
        r += kj > ki || (kj == ki && j < i);
      }
      L.order[r] = i;
      ord_s[r] = i;
      pcs_s[i] = ki < 0 ? 0 : seq_pieces(i, ki, qlen_s[i]);
    }
  } else {
    for (int i = threadIdx.x; i < B; i += kMqPlanThreads) L.order[i] = i;
  }
  __syncthreads();
  // per XCD x: exclusive prefix sums over its groups k = kXcds j + x (rank k / Hkv, kv
  // head k % Hkv) of their pieces; entry J is the XCD's total.  One scan over
  // t = x J + j (XCD-major), then each XCD's sums less its first.
  const int J = L.J;
  auto pieces_of = [&](int t) {
    const int k = kXcds * (t % J) + t / J;
    if (k >= L.NG) return 0;
    if (small) return pcs_s[ord_s[k / Hkv]];
    const int i = k / Hkv;   // index order beyond kPfRankMax sequences
    const int nun = a.seq_unit[i + 1] - a.seq_unit[i];
    if (nun == 0) return 0;
    return seq_pieces(i, a.context_lens[i], a.query_start_loc[i + 1] - a.query_start_loc[i]);
  };
  const int tot = block_scan<kMqPlanThreads>(kXcds * J, pieces_of, L.scan);
  if (threadIdx.x == 0) L.scan[kXcds * J] = tot;
  __syncthreads();
  for (int t = threadIdx.x; t < kXcds * (J + 1); t += kMqPlanThreads) {
    const int x = t / (J + 1), j = t % (J + 1);
    L.xcum[t] = L.scan[x * J + j] - L.scan[x * J];
  }
}

__global__ __launch_bounds__(kMqPlanThreads) void multi_plan_kernel(AttentionArgs a) {
  const int B = a.num_seqs;
  const int G = a.num_heads / a.num_kv_heads;
  const int tpb = a.unit_rows / G;   // new tokens per unit
  const int max_ctx = a.max_blocks_per_seq << a.block_shift;
  const int32_t* qsl = a.query_start_loc;
  auto units_of = [&](int i) {
    const int q0 = qsl[i], q1 = qsl[i + 1];
    return seq_valid(q0, q1, a.context_lens[i], a.num_tokens, max_ctx) ? (q1 - q0 + tpb - 1) / tpb
                                                                       : 0;
  };
  int U = block_scan<kMqPlanThreads>(B, units_of, a.seq_unit);
  const bool fits = U <= a.max_units;
  if (!fits) U = 0;
  if (threadIdx.x == 0) a.seq_unit[B] = U;
  __syncthreads();
  if (!fits) {
    for (int i = threadIdx.x; i < B; i += kMqPlanThreads) a.seq_unit[i] = 0;
  } else {
    for (int i = threadIdx.x; i < B; i += kMqPlanThreads) {
      const int n = units_of(i), u0 = a.seq_unit[i];
      for (int k = 0; k < n; ++k) a.unit_seq[u0 + k] = i;
    }
  }
  __syncthreads();
  if (a.unit_rows == kMqPrefillUnit) {
    if (threadIdx.x == 0) a.tile_hdr[2] = U;
    build_prefill_schedule(a, U);
    return;
  }
  // positions of unit u: the tiles up to its last token's position, plus kSeqCost
  auto positions_of = [&](int u) {
    const int i = a.unit_seq[u];
    const int q0 = qsl[i], qlen = qsl[i + 1] - q0;
    const int j_end = min(qlen, (u - a.seq_unit[i] + 1) * tpb);
    const int last = a.context_lens[i] - qlen + j_end;   // positions 0 .. last - 1
    return (last + kTileTokens - 1) / kTileTokens + kSeqCost;
  };
  const int total = block_scan<kMqPlanThreads>(U, positions_of, a.tile_cum);
  if (threadIdx.x == 0) {
    a.tile_cum[U] = total;
    a.tile_hdr[0] = total;
    a.tile_hdr[2] = U;
  }
}

hipError_t launch_multi_plan(const AttentionArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(multi_plan_kernel, dim3(1), dim3(kMqPlanThreads), 0, stream, a);
  return hipGetLastError();
}

// ---- the attention kernel ----------------------------------------------------------

// Cache policy of the KV tile copies.  In head mode a sequence's tiles are mostly read
// by one unit, and streaming them past the caches (non-temporal) helps: 412 -> 381 us
// for 5 speculated tokens on the Llama-3-8B-shaped batch (MI355X).  In row mode the
// units of a long prompt re-read its tiles while the caches still hold them, and the
// default policy is kept (865 us against 885 us non-temporal for 512-token chunks).
template <int HW, int NW>
constexpr Cpol multi_kv_cpol() { return HW == NW ? Cpol::kStream : Cpol::kDefault; }

// NW waves per workgroup.  NW == HW: each wave owns one of the HW kv heads of the
// staged rows and a unit is RB row blocks.  HW == 1 < NW: the waves share one kv
// head's rows and each takes RB of the unit's NW * RB row blocks, so one pass over
// the tiles serves NW * RB * 16 rows (long prompts).
// Waves per SIMD the register budget must allow.  bf16 row mode: three (168
// registers; the few values that no longer fit wait in scratch for the end of a
// segment).  Measured on MI355X, 4 prompts' 512-token chunks: 617 us at two waves per
// SIMD, 563 us at three, 1.32 ms at four (spills inside the tile loop).
#ifndef PKV_MULTI_ROW_WPE
#define PKV_MULTI_ROW_WPE 3
#endif
template <typename T, int D, int HW, int NW>
constexpr int multi_wpe() {
  return HW == 1 && NW > 1 && D == 128 && std::is_same<T, BF16>::value ? PKV_MULTI_ROW_WPE : 1;
}

template <typename T, int D, int G, int HW, int RB, int NW, int NBUF>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(multi_wpe<T, D, HW, NW>())))
void paged_attention_multi_kernel(AttentionArgs a) {
  constexpr int TOK = kTileTokens;
  constexpr bool kRowWaves = NW != HW;      // waves split the rows of one head
  static_assert(!kRowWaves || HW == 1, "row-split waves share a single head");
  using St = StageW<T, D, HW, TOK, NW>;
  constexpr int EB = T::kElemBytes;
  constexpr int NCH = D * EB / 16;          // 16-byte chunks of a head's row
  constexpr int QKC = D * EB / 64;          // key / query chunks per lane = MFMAs per tile
  constexpr int ROWS = kRowWaves ? NW * 16 * RB : 16 * RB;   // rows per unit
  constexpr int TPB = ROWS / G;             // new tokens per unit
  constexpr int CPL = D / 16;               // value columns per lane per k-step
  constexpr int L = 2 * St::kCopies;        // tile copies per wave per step
  constexpr int QROW = D * EB;              // bytes of one query row
  constexpr int NS = St::kTileSlots;
  static_assert(TOK == 16, "tile rows");

  // NBUF tiles rotate through one ring; the copies are assembly the compiler does not
  // track, so one array indexed at run time costs no extra waits
  // (slot s: the key tile at ring[s], the value tile at ring[s] + NS)
  __shared__ uint4 ring[NBUF][2 * NS];
  static_assert(NBUF >= 2 && NBUF <= 8, "ring depth");

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int nwg = gridDim.x;
  const int w = xcd_local_share(blockIdx.x, nwg);
  const int hg = blockIdx.y;
  const int Hkv = a.num_kv_heads;
  const int H = Hkv * G;
  const int hw_idx = kRowWaves ? 0 : wave;  // this wave's head within the staged rows
  const int g = hg * HW + hw_idx;           // this wave's kv head
  const int row0 = kRowWaves ? wave * 16 * RB : 0;   // this wave's first row of the unit

  cint32* cum = (cint32*)a.tile_cum;
  cint32* ctx_of = (cint32*)a.context_lens;
  cint32* tables = (cint32*)a.block_tables;
  cint32* qsl = (cint32*)a.query_start_loc;
  cint32* unit_seq = (cint32*)a.unit_seq;
  cint32* seq_unit = (cint32*)a.seq_unit;
  const int total = ((cint32*)a.tile_hdr)[0];
  const int U = ((cint32*)a.tile_hdr)[2];
  if (w == 0 && hg == 0 && threadIdx.x == 0) a.tile_hdr[1] = nwg;
  const int64_t start = (int64_t)w * total / nwg;
  const int64_t end = (int64_t)(w + 1) * total / nwg;
  if (start >= end) return;

  // the unit holding position `start` (64-way search over cum[0 .. U])
  int lo = 0, len = U + 1;
  while (len > 1) {
    const int step = (len + kWave - 1) / kWave;
    const int i = lo + lane * step;
    const bool ok = i < lo + len && a.tile_cum[i] <= start;
    const int k = __builtin_amdgcn_readfirstlane(__popcll(__ballot(ok)));
    const int nlo = lo + (k - 1) * step;
    len = min(step, lo + len - nlo);
    lo = nlo;
  }
  const int unit0 = lo;

  const int quarter = lane >> 4;
  const int col = lane & 15;                // MFMA row of the key tile / column of Q^T

  const int64_t row_stride = (int64_t)Hkv * D * EB;
  uint32_t copy_off[St::kCopies];
#pragma unroll
  for (int i = 0; i < St::kCopies; ++i) {
    const int s = (i * NW + wave) * kWave + lane;
    const int r = s / St::kSlots;
    const int p = s % St::kSlots;
    copy_off[i] = (uint32_t)(r * row_stride) + (uint32_t)((p ^ St::swz(r)) * 16);
  }
  const char* kcache = static_cast<const char*>(a.key_cache) + (int64_t)hg * St::kRowBytes;
  const char* vcache = static_cast<const char*>(a.value_cache) + (int64_t)hg * St::kRowBytes;
  const int shift = a.block_shift;
  const int bs_mask = (1 << shift) - 1;
  const int MB = a.max_blocks_per_seq;
  const int max_ctx = MB << shift;
  const int num_blocks = (int)a.num_blocks;
  const float kNegInf = -__builtin_inff();

  struct Cursor {
    int u, t, nt, stop;
  };
  // Moves a cursor to the next unit that starts in this share, or invalidates it
  // (every unit has at least one tile).  Cursors are values, kept wave-uniform.
  auto next_unit = [&](Cursor c) -> Cursor {
    const int u = uniform(c.u) + 1;
    const int cs = uniform(cum[u]);
    c.u = u;
    c.t = 0;
    if (u >= U || cs + kSeqCost >= end) {
      c.nt = c.stop = 0;
      return c;
    }
    c.nt = uniform(cum[u + 1] - cs - kSeqCost);
    c.stop = uniform(min(c.nt, (int)(end - cs - kSeqCost)));
    return c;
  };
  auto first_cursor = [&]() -> Cursor {
    const int cs = cum[unit0];
    Cursor c;
    c.u = unit0;
    c.nt = uniform(cum[unit0 + 1] - cs - kSeqCost);
    c.t = uniform(max(0, (int)(start - cs - kSeqCost)));
    c.stop = uniform(min(c.nt, (int)(end - cs - kSeqCost)));
    if (c.t >= c.stop) c = next_unit(c);
    return c;
  };

  // ---- issue side ----
  Cursor ic = first_cursor();
  unsigned bad_pipe = 0;
  auto issue = [&](uint4* kb, uint4* vb) {
    int64_t base = 0;
    bad_pipe <<= 1;
    if (ic.t < ic.stop) {
      const int tok0 = uniform(ic.t * TOK);
      const int seq = uniform(unit_seq[uniform(ic.u)]);
      const int32_t blk =
          uniform(tok0 < max_ctx ? tables[(int64_t)seq * MB + (tok0 >> shift)] : -1);
      if (blk >= 0 && blk < num_blocks)
        base = (((int64_t)blk << shift) + (tok0 & bs_mask)) * row_stride;
      else
        bad_pipe |= 1u;
      if (++ic.t == ic.stop) ic = next_unit(ic);
    }
    const uint32_t kd = lds_addr(kb) + wave * 1024;
    const uint32_t vd = lds_addr(vb) + wave * 1024;
    const char* kbase = kcache + base;
    const char* vbase = vcache + base;
#pragma unroll
    for (int i = 0; i < St::kCopies; ++i) dma16<multi_kv_cpol<HW, NW>()>(kbase, copy_off[i], kd + i * NW * 1024);
#pragma unroll
    for (int i = 0; i < St::kCopies; ++i) dma16<multi_kv_cpol<HW, NW>()>(vbase, copy_off[i], vd + i * NW * 1024);
  };

  // ---- compute side ----
  Cursor cc = first_cursor();
  if (cc.t >= cc.stop) return;

  // the unit under the compute cursor
  int uq0 = 0, uqlen = 0, uctx = 0, uj0 = 0;
  auto unit_info = [&]() {
    const int useq = uniform(unit_seq[cc.u]);
    uq0 = uniform(qsl[useq]);
    uqlen = uniform(qsl[useq + 1] - uq0);
    uctx = uniform(ctx_of[useq]);
    uj0 = uniform((cc.u - seq_unit[useq]) * TPB);
  };
  bool seg_from_zero = cc.t == 0;
  int seg_bad = 0;

  // The unit's rows as the B operand of Q.K^T: row r (block r / 16, lane column
  // r % 16) is new token j0 + r / G (a row past the sequence's last new token repeats
  // the unit's first one and is never stored) with query head g * G + r % G.  Loaded
  // once per unit with ordinary loads and waited for at once, which also waits for
  // the tile copies in flight: one drain per unit.
  uint4 qa[RB][QKC];
  auto load_query = [&]() {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = row0 + rb * 16 + col;
      const int jq = uj0 + r / G < uqlen ? uj0 + r / G : uj0;
      const char* row = static_cast<const char*>(a.query) +
                        ((int64_t)(uq0 + jq) * H + g * G + r % G) * QROW;
#pragma unroll
      for (int c = 0; c < QKC; ++c)
        qa[rb][c] = *reinterpret_cast<const uint4*>(row + (4 * c + quarter) * 16);
    }
    // a wait the compiler sees (all vector memory, the copies in flight included), so
    // that it places none of its own for these loads inside the tile loop
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  };

  float m_run[RB];      // running maximum of the lane's row of each block (base-2)
  float l_lane[RB];     // the lane's share of that row's sum
  floatx4 acc[RB][CPL]; // rows 16 rb + 4 quarter + j, columns col * CPL + e of block e
  auto reset = [&]() {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      m_run[rb] = kNegInf;
      l_lane[rb] = 0.f;
#pragma unroll
      for (int e = 0; e < CPL; ++e) acc[rb][e] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    seg_bad = 0;
  };

  auto compute = [&](const uint4* kb, const uint4* vb, bool bad) {
    constexpr float kRebase = 8.f;
    const int tok0 = cc.t * TOK;
    seg_bad |= bad;
    uint4 kk[QKC];
#pragma unroll
    for (int c = 0; c < QKC; ++c)
      kk[c] = kb[col * St::kSlots + ((hw_idx * NCH + 4 * c + quarter) ^ St::swz(col))];
    // A tile that ends at or before the first position any row of this wave sees
    // needs no causal mask (a wave-uniform test).
    const bool unmasked = tok0 + TOK - 1 <= uctx - uqlen + min(uj0 + row0 / G, uqlen - 1);
    float p[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const floatx4 s4 = tile_scores<T, QKC>(kk, qa[rb]);   // S^T: row col, tokens 4q + j
      float sc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[j] = s4[j] * a.scale_log2;
      if (!unmasked) {
        keep_branch();
        const int jrow = min(uj0 + (row0 + rb * 16 + col) / G, uqlen - 1);
        const int prow = uctx - uqlen + jrow;                // last position the row sees
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (tok0 + 4 * quarter + j > prow) sc[j] = kNegInf;
      }
      float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      mx = max_xor32(max_xor16(mx));
      const bool up = mx > m_run[rb] + kRebase;
      if (__ballot(up)) {
        keep_branch();
        const float alpha = up ? fast_exp2(m_run[rb] - mx) : 1.f;   // 0 when m_run is -inf
        m_run[rb] = up ? mx : m_run[rb];
        l_lane[rb] *= alpha;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float aj = __shfl(alpha, 4 * quarter + j);
#pragma unroll
          for (int e = 0; e < CPL; ++e) acc[rb][e][j] *= aj;
        }
      }
      const float mref = m_run[rb] == kNegInf ? 0.f : m_run[rb];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[rb][j] = fast_exp2(sc[j] - mref);   // 0 for masked tokens
        l_lane[rb] += p[rb][j];
      }
    }
    const bool full = tok0 + TOK <= uctx;
    if constexpr (std::is_same<T, BF16>::value) {
      // P.V on bf16 matrix instructions (16x16x32): lane quarter q supplies the hi and
      // the lo terms of tokens 4q .. 4q + 3 of its row (A) and those tokens' value
      // columns twice (B, packed from four token rows).  Together hi + lo are exact to
      // about 2^-17 of p, so the products keep fp32-level accuracy.
      uint32_t w[4][CPL / 2];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int vr = 4 * quarter + s;
        if constexpr (CPL == 8) {
          const uint4 c = vb[vr * St::kSlots + ((hw_idx * NCH + col) ^ St::swz(vr))];
          w[s][0] = c.x; w[s][1] = c.y; w[s][2] = c.z; w[s][3] = c.w;
        } else {
          static_assert(CPL == 4, "value piece");
          const int slot = (hw_idx * NCH + (col >> 1)) ^ St::swz(vr);
          const uint2 c = reinterpret_cast<const uint2*>(vb)[2 * (vr * St::kSlots + slot) + (col & 1)];
          w[s][0] = c.x; w[s][1] = c.y;
        }
      }
      if (!full) {   // rows past the context may hold NaN
        keep_branch();
#pragma unroll
        for (int s = 0; s < 4; ++s)
          if (tok0 + 4 * quarter + s >= uctx)
#pragma unroll
            for (int d = 0; d < CPL / 2; ++d) w[s][d] = 0u;
      }
      uint2 bv[CPL];   // block e: column col * CPL + e of tokens 4q .. 4q + 3
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        // even e: the low bf16 of two rows' words, odd e: the high ones
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const int d = e >> 1;
        bv[e].x = __builtin_amdgcn_perm(w[1][d], w[0][d], sel);
        bv[e].y = __builtin_amdgcn_perm(w[3][d], w[2][d], sel);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const floatx2 p01 = {p[rb][0], p[rb][1]}, p23 = {p[rb][2], p[rb][3]};
        const bf16x2 h01 = __builtin_convertvector(p01, bf16x2);
        const bf16x2 h23 = __builtin_convertvector(p23, bf16x2);
        const floatx2 r01 = p01 - __builtin_convertvector(h01, floatx2);
        const floatx2 r23 = p23 - __builtin_convertvector(h23, floatx2);
        const bf16x2 l01 = __builtin_convertvector(r01, bf16x2);
        const bf16x2 l23 = __builtin_convertvector(r23, bf16x2);
        const bf16x8 ahl = {h01[0], h01[1], h23[0], h23[1], l01[0], l01[1], l23[0], l23[1]};
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          const bf16x8 b = __builtin_bit_cast(bf16x8, make_uint4(bv[e].x, bv[e].y, bv[e].x, bv[e].y));
          acc[rb][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahl, b, acc[rb][e], 0, 0, 0);
        }
      }
      return;
    }
    // fp32 caches: P.V on fp32 matrix instructions; k-step s takes token 4q + s of lane
    // quarter q; the value row is read once for all row blocks
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int vr = 4 * quarter + s;
      float v[CPL];
      if constexpr (CPL * EB == 16) {
        unpack_chunk<T>(vb[vr * St::kSlots + ((hw_idx * NCH + col) ^ St::swz(vr))], v);
      } else if constexpr (CPL * EB == 32) {
        unpack_chunk<T>(vb[vr * St::kSlots + ((hw_idx * NCH + 2 * col) ^ St::swz(vr))], v);
        unpack_chunk<T>(vb[vr * St::kSlots + ((hw_idx * NCH + 2 * col + 1) ^ St::swz(vr))],
                        v + CPL / 2);
      } else {
        static_assert(CPL * EB == 8, "value piece");
        const int slot = (hw_idx * NCH + (col >> 1)) ^ St::swz(vr);
        const uint2 c8 = reinterpret_cast<const uint2*>(vb)[2 * (vr * St::kSlots + slot) + (col & 1)];
        v[0] = bf16_lo(c8.x); v[1] = bf16_hi(c8.x);
        v[2] = bf16_lo(c8.y); v[3] = bf16_hi(c8.y);
      }
      if (!full && tok0 + vr >= uctx) {
#pragma unroll
        for (int e = 0; e < CPL; ++e) v[e] = 0.f;   // rows past the context may hold NaN
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int e = 0; e < CPL; ++e)
          acc[rb][e] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[rb][s], v[e], acc[rb][e], 0, 0, 0);
    }
  };

  // End of a segment: sums across the four lanes of each row, normalise, store rows
  // 16 rb + 4 quarter + j (output or record).
  auto finish = [&](bool whole) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float l_row = sum_xor32(sum_xor16(l_lane[rb]));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = row0 + rb * 16 + 4 * quarter + j;
        const float lr = __shfl(l_row, 4 * quarter + j);
        const float mr = __shfl(m_run[rb], 4 * quarter + j);
        const int jq = uj0 + r / G;
        if (jq >= uqlen) continue;
        const float inv = seg_bad ? __builtin_nanf("") : (lr > 0.f ? 1.f / lr : 0.f);
        float o[CPL];
#pragma unroll
        for (int e = 0; e < CPL; ++e) o[e] = acc[rb][e][j] * inv;
        if (whole) {
          const int64_t orow = ((int64_t)(uq0 + jq) * H + g * G + r % G) * D + col * CPL;
          if (a.out_bf16) {
            uint16_t* dst = static_cast<uint16_t*>(a.out) + orow;
#pragma unroll
            for (int e = 0; e < CPL; e += 4) {
              uint2 v;
              v.x = f32_to_bf16_rne(o[e]) | (uint32_t)f32_to_bf16_rne(o[e + 1]) << 16;
              v.y = f32_to_bf16_rne(o[e + 2]) | (uint32_t)f32_to_bf16_rne(o[e + 3]) << 16;
              *reinterpret_cast<uint2*>(dst + e) = v;
            }
          } else {
            // non-temporal: the next tile's wait also waits for these stores, and they
            // complete sooner when streamed past the caches (5 speculated tokens per
            // sequence, Llama-3-8B-shaped batch: 344 -> 332 us per call on MI355X)
            float* dst = static_cast<float*>(a.out) + orow;
#pragma unroll
            for (int e = 0; e < CPL; e += 4) {
              const floatx4 v = {o[e], o[e + 1], o[e + 2], o[e + 3]};
              __builtin_nontemporal_store(v, reinterpret_cast<floatx4*>(dst + e));
            }
          }
        } else {
          const int64_t rec = (((int64_t)w + cc.u) * Hkv + g) * ROWS + r;
          float* dst = a.ws_o + rec * D + col * CPL;
#pragma unroll
          for (int e = 0; e < CPL; e += 4) {
            const floatx4 v = {o[e], o[e + 1], o[e + 2], o[e + 3]};
            __builtin_nontemporal_store(v, reinterpret_cast<floatx4*>(dst + e));
          }
          if (col == 0) {
            a.ws_m[rec] = mr;
            a.ws_l[rec] = seg_bad ? __builtin_nanf("") : lr;
          }
        }
      }
    }
  };

  reset();
  unit_info();
  load_query();

  // Tile j sits in ring slot j % NBUF.  Per step: issue tile j + NBUF - 1 into the
  // slot of tile j - 1 (released by the previous step's last barrier), wait for this
  // wave's copies of tile j (the NBUF - 1 later tiles stay in flight), barrier (every
  // wave's copies of tile j have landed), compute tile j, barrier (every wave is done
  // with its slot).  Issuing before the wait keeps NBUF - 1 tiles in flight during
  // the wait, not NBUF - 2.
#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i) issue(ring[i], ring[i] + NS);
  for (int j = 0;; ++j) {
    if (cc.t >= cc.stop) break;
    const int fill = (j + NBUF - 1) % NBUF;
    issue(ring[fill], ring[fill] + NS);
    wait_copies<(NBUF - 1) * L>();
    bare_barrier();
    compute(ring[j % NBUF], ring[j % NBUF] + NS, (bad_pipe >> (NBUF - 1)) & 1u);
    bare_barrier();
    if (cc.t == cc.stop - 1) {
      finish(seg_from_zero && cc.stop == cc.nt);
      reset();
      cc = next_unit(cc);
      seg_from_zero = true;
      if (cc.t < cc.stop) {
        unit_info();
        load_query();
      }
    } else {
      ++cc.t;
    }
  }
  wait_copies<0>();
}

// ---- long prompts with bf16 caches: 256-row units in two context pieces ----------------
// Chunked prefill hands a few sequences many new tokens each.  There the work is the
// matrix products, and what costs is re-reading a sequence's context for every unit
// of its rows.  This mode:
//  - makes units of 256 rows (kPfWaves waves of two 16-row MFMA blocks sharing one kv
//    head's staged tiles); each (unit, kv head) item's causal context is cut into two
//    halves, the pieces, computed by one workgroup each and merged by the later one
//    (the prefill schedule above), so that a few long histories no longer set the time;
//  - deals the pieces of one (sequence, kv head) to one XCD, where its units run side
//    by side reading the same tiles at about the same time: L2 serves the repeats;
//  - runs one workgroup per compute unit, each taking its XCD's pieces in snake order;
//  - stages 32-token tiles, so that P.V runs on the full-rate v_mfma_f32_16x16x32_bf16
//    with k = the lane's four tokens of each 16-token half: the lane's own eight
//    probabilities form its A operand (as hi and lo bf16 parts, two instructions),
//    and transposed LDS reads give its B operand, the matching eight value rows' entries
//    of one dim (no byte permutes);
//  - stages each piece's record through the ring at the end, so that its stores write
//    whole rows.
// Rows of a sequence whose context lists a block id outside the pool are all NaN
// (each piece checks the whole table row first).
constexpr int kPfWaves = kMqPrefillUnit / 32;   // 8 waves, 32 rows each
#ifndef PKV_PREFILL_NBUF
#define PKV_PREFILL_NBUF 4
#endif
constexpr int kPfNbuf = PKV_PREFILL_NBUF;        // tiles in the ring

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Maxima of raw scores as the hardware instructions alone.  fmaxf on values the
// compiler cannot prove canonical (matrix results, lane swaps) gets a canonicalising
// move per operand first: 12 of the tile's vector instructions per wave.  A NaN score
// reaches its exponential, and so its row's output, either way.
__device__ __forceinline__ float hw_max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float hw_max(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

template <int G>
__global__ __launch_bounds__(kPfWaves * kWave) __attribute__((amdgpu_waves_per_eu(2)))
void paged_attention_prefill_kernel(AttentionArgs a) {
  constexpr int D = 128;
  constexpr int RB = 2;                     // 16-row MFMA blocks per wave
  constexpr int ROWB = D * 2;               // bytes of one head's bf16 row
  constexpr int SLOTS = ROWB / 16;          // 16-byte slots per row
  constexpr int TSLOTS = kPfTok * SLOTS;    // slots per tile and cache
  constexpr int TPB = kMqPrefillUnit / G;   // new tokens per unit
  constexpr int CPL = D / 16;               // value columns per lane = output blocks
  static_assert(kPfTok * ROWB == kPfWaves * 1024, "one 1 KiB copy per wave, cache and tile");
  __shared__ uint4 kring[kPfNbuf][TSLOTS], vring[kPfNbuf][TSLOTS];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform(threadIdx.x / kWave);
  const int quarter = lane >> 4;
  const int col = lane & 15;
  const int Hkv = a.num_kv_heads;
  const int H = Hkv * G;
  __shared__ int merge_flag;
  const PrefillLayout PL(a);
  cint32* seq_unit = (cint32*)a.seq_unit;
  cint32* order = (cint32*)PL.order;
  // this workgroup's XCD (workgroup b runs on XCD b % 8) and its place among the W there
  const int W = gridDim.x / kXcds;
  const int xcd = blockIdx.x % kXcds, jw = blockIdx.x / kXcds;
  cint32* xc = (cint32*)PL.xcum + xcd * (PL.J + 1);
  const int nx = xc[PL.J];
  const int P = ((cint32*)a.tile_hdr)[4];   // the schedule's tile target
  for (int rnd = 0;; ++rnd) {
    const int pos = rnd * W + ((rnd & 1) ? W - 1 - jw : jw);   // snake order
    if (pos >= nx) break;
    // the group holding list position pos: the last glo < J with xc[glo] <= pos
    int glo = 0, ghi = PL.J;
    while (ghi - glo > 1) {
      const int mid = (glo + ghi) >> 1;
      if (xc[mid] <= pos) glo = mid; else ghi = mid;
    }
    const int grp = kXcds * glo + xcd;
    const int seq = order[grp / Hkv];
    const int g = grp % Hkv;
    const int u0 = seq_unit[seq];
    const int nun = seq_unit[seq + 1] - u0;   // > 0 for a group with pieces
    cint32* qsl = (cint32*)a.query_start_loc;
    const int q0 = qsl[seq];
    const int qlen = qsl[seq + 1] - q0;
    const int ctx = ((cint32*)a.context_lens)[seq];
    // the group's units last to first (largest first), each an item of npc pieces
    int in_grp = pos - xc[glo];
    int unit = nun - 1, ntiles = 0, npc = 1;
    for (;; --unit) {
      ntiles = pf_unit_tiles(ctx, qlen, unit, TPB);
      npc = pf_pieces(ntiles, P);
      if (in_grp < npc || unit == 0) break;
      in_grp -= npc;
    }
    // (the plan counted the same pieces; the clamp keeps a record inside its item's
    // kPfMaxPieces even if it had not)
    const int piece = min(in_grp, npc - 1);
    const int item = u0 * Hkv + g * nun + unit;
    const int j0 = unit * TPB;                 // first new token of the unit
    const int j1 = min(qlen, j0 + TPB);
    const int base_pos = ctx - qlen;          // position of new token 0
    // this piece's tiles
    const int t_lo = ntiles * piece / npc;        // below 2^28: 32-bit arithmetic
    const int t_hi = ntiles * (piece + 1) / npc;
    __syncthreads();   // the previous piece is done with the ring and merge_flag

    const int shift = a.block_shift;
    const int bs_mask = (1 << shift) - 1;
    const int MB = a.max_blocks_per_seq;
    const int num_blocks = (int)a.num_blocks;
    const int32_t* table = a.block_tables + (int64_t)seq * MB;

    // every block of the context must be in the pool (the lane index through an empty
    // asm keeps the lane's address part from being hoisted out of the piece loop)
    int bl = lane;
    asm volatile("" : "+v"(bl));
    bool bad_lane = false;
    for (int b = bl; b < ((ctx + bs_mask) >> shift); b += kWave) {
      const int32_t id = table[b];
      bad_lane |= id < 0 || id >= num_blocks;
    }
    const bool seq_bad = __ballot(bad_lane) != 0;

    // this wave's rows: r = 32 wave + 16 rb + col is new token j0 + r / G with query head
    // g G + r % G (a row past the last new token repeats token j0 and is not stored)
    const int wrow0 = wave * 16 * RB;
    const int wj_lo = j0 + wrow0 / G;
    const int wj_hi = min(j0 + (wrow0 + 16 * RB - 1) / G, qlen - 1);
    const bool wave_live = wj_lo < qlen;
    const int wpos_lo = base_pos + min(wj_lo, qlen - 1);   // positions the wave's rows see
    const int wpos_hi = base_pos + wj_hi;
    const int wtiles = wave_live ? wpos_hi / kPfTok + 1 : 0;
    const int w_end = min(wtiles, t_hi);      // the wave's tiles in this piece: [t_lo, w_end)

    // queries; for a negative scale the query's sign bits are flipped (exact) so that
    // the scale is positive and a row's largest raw score is its largest scaled one
    // (a zero scale becomes the smallest normal float: every 2^(s * scale) is then 1 as
    // for zero, and a masked -inf score stays -inf instead of turning NaN)
    const float scale = fmaxf(fabsf(a.scale_log2), 1.17549435e-38f);
    const uint32_t qflip = a.scale_log2 < 0.f ? 0x80008000u : 0u;
    uint4 qa[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = wrow0 + rb * 16 + col;
      const int jq = j0 + r / G < qlen ? j0 + r / G : j0;
      const char* row = static_cast<const char*>(a.query) +
                        ((int64_t)(q0 + jq) * H + g * G + r % G) * ROWB;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint4 v = *reinterpret_cast<const uint4*>(row + (4 * c + quarter) * 16);
        v.x ^= qflip; v.y ^= qflip; v.z ^= qflip; v.w ^= qflip;
        qa[rb][c] = v;
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

    // copies: wave w brings rows 4w .. 4w + 3 of each tile, lane l row 4w + l / 16, its
    // 16-byte piece l % 16 stored at slot (l % 16) ^ row (rows are 16 slots)
    const int64_t row_stride = (int64_t)Hkv * ROWB;
    const int crow = 4 * wave + quarter;
    const uint32_t copy_off = (uint32_t)(quarter * row_stride) + (uint32_t)(((col ^ crow) & 15) * 16);
    const char* kcache = static_cast<const char*>(a.key_cache) + g * ROWB;
    const char* vcache = static_cast<const char*>(a.value_cache) + g * ROWB;
    auto issue = [&](int tt, int slot) {
      int64_t off = 0;                        // rows past the context: the pool's first rows
      const int t0 = tt * kPfTok + 4 * wave;
      if (tt < t_hi && t0 < ctx) {
        const int32_t blk = uniform(((cint32*)table)[t0 >> shift]);
        if (blk >= 0 && blk < num_blocks) off = (((int64_t)blk << shift) + (t0 & bs_mask)) * row_stride;
      }
      dma16<Cpol::kDefault>(kcache + off, copy_off, lds_addr(kring[slot]) + wave * 1024);
      dma16<Cpol::kDefault>(vcache + off, copy_off, lds_addr(vring[slot]) + wave * 1024);
    };

    const float kNegInf = -__builtin_inff();
    float m_run[RB], l_lane[RB];
    floatx4 acc[RB][CPL];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      m_run[rb] = kNegInf;
      l_lane[rb] = 0.f;
#pragma unroll
      for (int e = 0; e < CPL; ++e) acc[rb][e] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    // S^T = K . Q^T of a tile's two 16-token halves (raw, unscaled): lane (quarter q,
    // column n) gets row n's scores of tokens 16 h + 4 q + i in s[rb][4 h + i]
    auto scores = [&](const uint4* kb, float (&sv)[RB][8]) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint4 kk[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) kk[c] = kb[(16 * h + col) * SLOTS + ((4 * c + quarter) ^ col)];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const floatx4 s4 = tile_scores<BF16, 4>(kk, qa[rb]);
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[rb][4 * h + i] = s4[i];
        }
      }
    };
    // the causal edge: tokens past a row's position get -inf (a branch taken on the last
    // tiles of the wave's rows only)
    auto mask_edge = [&](int tt, float (&sv)[RB][8]) {
      const int tok0 = tt * kPfTok;
      if (tok0 + kPfTok - 1 > wpos_lo) {
        keep_branch();
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int prow = base_pos + min(j0 + (wrow0 + rb * 16 + col) / G, qlen - 1);
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if (tok0 + 16 * (k >> 2) + 4 * quarter + (k & 3) > prow) sv[rb][k] = kNegInf;
        }
      }
    };
    // the running maxima after a tile (base-2 domain; raw scores, positive scale): a row
    // takes a new maximum only when it exceeds the old one by more than 2^8, and then
    // its earlier terms are scaled by alpha; returns whether any row of the wave rose
    auto maxima = [&](const float (&sv)[RB][8], float (&mnew)[RB], float (&alpha)[RB]) {
      constexpr float kRebase = 8.f;
      bool rise = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float a3 = hw_max3(sv[rb][0], sv[rb][1], sv[rb][2]);
        const float b3 = hw_max3(sv[rb][3], sv[rb][4], sv[rb][5]);
        const float c3 = hw_max3(sv[rb][6], sv[rb][7], a3);
        float mx = hw_max(b3, c3);
        auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = hw_max(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
        auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = hw_max(__uint_as_float(s32[0]), __uint_as_float(s32[1])) * scale;
        const bool up = mx > m_run[rb] + kRebase;
        mnew[rb] = up ? mx : m_run[rb];
        alpha[rb] = up ? fast_exp2(m_run[rb] - mx) : 1.f;   // 0 when m_run is -inf
        rise |= up;
      }
      return __ballot(rise) != 0;
    };
    // probabilities of a tile relative to mnew, as bf16 hi + lo parts (together exact
    // to about 2^-17 of p), and their sums per lane
    auto probs = [&](const float (&sv)[RB][8], const float (&mnew)[RB], bf16x8 (&ph)[RB],
                     bf16x8 (&pl)[RB], float (&lsum)[RB]) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float nref = mnew[rb] == kNegInf ? 0.f : -mnew[rb];
        float p[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          p[k] = fast_exp2(fmaf(sv[rb][k], scale, nref));   // 0 for masked tokens
          lsum[rb] += p[k];
        }
        // lo = p - hi as one bf16 dot product per value, (hi0, hi1) . (-1, 0) + p0: the
        // products are exact and so is the difference, which fp32 holds.  The pair
        // (-1, 0) is 0x0000bf80; it is moved into a scalar register here because the
        // compiler would otherwise encode it as the inline constant -1.0, which the
        // instruction reads as 0xbf800000, i.e. (0, -1).
        uint32_t kneg0;
        asm("s_mov_b32 %0, 0xbf80" : "=s"(kneg0));
        const bf16x2 neg0 = __builtin_bit_cast(bf16x2, kneg0);
        const bf16x2 neg1 = __builtin_bit_cast(bf16x2, 0xbf800000u);
#pragma unroll
        for (int k = 0; k < 8; k += 2) {
          const floatx2 pp = {p[k], p[k + 1]};
          const bf16x2 h2 = __builtin_convertvector(pp, bf16x2);
          const floatx2 rr = {__builtin_amdgcn_fdot2_f32_bf16(h2, neg0, p[k], false),
                              __builtin_amdgcn_fdot2_f32_bf16(h2, neg1, p[k + 1], false)};
          const bf16x2 l2 = __builtin_convertvector(rr, bf16x2);
          ph[rb][k] = h2[0]; ph[rb][k + 1] = h2[1];
          pl[rb][k] = l2[0]; pl[rb][k + 1] = l2[1];
        }
      }
    };
    // Value operand of output block e, dims 16 e .. 16 e + 15 (lane column n: dim
    // 16 e + n), over the lane's eight k slots: tokens 16 h + 4 quarter + i of the tile
    // (h < 2, i < 4), the order of the probabilities in ph / pl.  Two transposed LDS
    // reads per block (ds_read_b64_tr_b16): within each 16-lane quarter, lane 4 i + m
    // addresses the 8 bytes of token 16 h + 4 quarter + i's row that hold dims
    // 16 e + 4 m .. 16 e + 4 m + 3, and the read hands lane n the bf16 of dim 16 e + n
    // from each of the four rows, in k order.  Slot j of row r is stored at j ^ (r & 15),
    // so the lane's byte offset is tr_base + 32 (e ^ tr_x) for h = 0, 16 rows further
    // for h = 1.
    const int tr_row = 4 * quarter + (col >> 2);
    const int tr_m = col & 3;
    const uint32_t tr_base = (uint32_t)(tr_row * ROWB + ((((tr_m >> 1) ^ tr_row) & 1) << 4) +
                                        ((tr_m & 1) << 3));
    const uint32_t tr_x = (uint32_t)((tr_row & 15) >> 1);
    auto read_v = [&](int tt, const uint4* vb, int hv, bf16x8 (&bv)[4], bool zero_tail) {
      const uint32_t base = lds_addr(vb) + tr_base;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t o = base + (((uint32_t)(4 * hv + k) ^ tr_x) << 5);
        const lds_s16x4* p0 = reinterpret_cast<const lds_s16x4*>((size_t)o);
        const lds_s16x4* p1 = reinterpret_cast<const lds_s16x4*>((size_t)(o + 16 * ROWB));
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_s16x4*>(p0));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_s16x4*>(p1));
        const s16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        bv[k] = __builtin_bit_cast(bf16x8, both);
      }
      if (zero_tail && tt * kPfTok + kPfTok > ctx) {
        // rows past the context may hold NaN: zero the lane's k slots of those tokens
        keep_branch();
        uint32_t mk[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const int t0 = tt * kPfTok + 16 * (d >> 1) + 4 * quarter + 2 * (d & 1);
          mk[d] = (t0 < ctx ? 0xffffu : 0u) | (t0 + 1 < ctx ? 0xffff0000u : 0u);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint4 u = __builtin_bit_cast(uint4, bv[k]);
          u.x &= mk[0]; u.y &= mk[1]; u.z &= mk[2]; u.w &= mk[3];
          bv[k] = __builtin_bit_cast(bf16x8, u);
        }
      }
    };
    // acc += P . V for output blocks 4 hv .. 4 hv + 3 on v_mfma_f32_16x16x32_bf16 (hi and
    // lo parts of P)
    auto pv = [&](const bf16x8 (&bv)[4], int hv, const bf16x8 (&ph)[RB], const bf16x8 (&pl)[RB]) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int e = 4 * hv + k;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          acc[rb][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph[rb], bv[k], acc[rb][e], 0, 0, 0);
          acc[rb][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl[rb], bv[k], acc[rb][e], 0, 0, 0);
        }
      }
    };
    auto rescale = [&](const float (&alpha)[RB]) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ai = __shfl(alpha[rb], 4 * quarter + i);
#pragma unroll
          for (int e = 0; e < CPL; ++e) acc[rb][e][i] *= ai;
        }
    };

    // The tile loop over the piece's tiles [t_lo, t_hi), pipelined one tile deep.  Step t
    // (tile t sits in ring slot (t - t_lo) % kPfNbuf) starts with the scores of tile t in
    // registers, masked, and the running maxima already raised for them.  It waits for
    // this wave's copies of tile t + 1, passes one barrier (every wave's copies of tile
    // t + 1 have landed; every wave is done with step t - 1 and so with tile t - 1),
    // issues tile t + kPfNbuf - 1 into tile t - 1's slot, and then runs one block of
    // straight-line work: the scores of tile t + 1 on the matrix cores beside the
    // probabilities of tile t on the vector unit, then P.V of tile t on the matrix cores
    // beside the maxima of tile t + 1.  The block asks the compiler for that interleave
    // (scheduling groups of one matrix instruction and a few vector ones); the compiled
    // loop keeps the score products together all the same, and the order written out with
    // scheduling fences ran slower than the compiler's.  A rise of a row maximum for tile
    // t + 1 rescales the accumulators after P.V of tile t (a rare branch).  The wave's
    // last steps take a general path with the conditions.
    static_assert(kPfNbuf >= 4, "tiles t and t + 1 stay staged while t + 2 lands");
    constexpr int kAhead = (kPfNbuf - 3) * 2;   // copies of later tiles left in flight
#pragma unroll
    for (int i = 0; i < kPfNbuf - 1; ++i) issue(t_lo + i, i);
    float sA[RB][8], sB[RB][8];
    wait_copies<kAhead + 2>();                  // tile t_lo
    bare_barrier();
    if (w_end > t_lo) {
      scores(kring[0], sA);
      mask_edge(t_lo, sA);
      float mnew[RB], alpha[RB];
      maxima(sA, mnew, alpha);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) m_run[rb] = mnew[rb];
    }

    auto step = [&](int lt, float (&s_cur)[RB][8], float (&s_nxt)[RB][8]) {
      const int tt = t_lo + lt;                 // tile tt sits in ring slot lt % kPfNbuf
      wait_copies<kAhead>();                    // tile tt + 1
      bare_barrier();
      issue(tt + kPfNbuf - 1, (lt + kPfNbuf - 1) % kPfNbuf);
      float mnew[RB], alpha[RB], lsum[RB] = {0.f, 0.f};
      bf16x8 ph[RB], pl[RB];
      bool rise = false;
      if (tt + 1 < w_end) {
        // tile tt is not the wave's last, so its value rows are all inside the context
        auto block = [&](bool edge) {
          bf16x8 w0[4], w1[4];
          scores(kring[(lt + 1) % kPfNbuf], s_nxt);
          read_v(tt, vring[lt % kPfNbuf], 0, w0, false);
          probs(s_cur, m_run, ph, pl, lsum);
          if (edge) {
            const int tok0 = (tt + 1) * kPfTok;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
              const int prow = base_pos + min(j0 + (wrow0 + rb * 16 + col) / G, qlen - 1);
#pragma unroll
              for (int k = 0; k < 8; ++k)
                if (tok0 + 16 * (k >> 2) + 4 * quarter + (k & 3) > prow) s_nxt[rb][k] = kNegInf;
            }
          }
          pv(w0, 0, ph, pl);
          read_v(tt, vring[lt % kPfNbuf], 1, w1, false);
          pv(w1, 1, ph, pl);
          rise = maxima(s_nxt, mnew, alpha);
          __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);   // keys and the first values
#pragma unroll
          for (int i = 0; i < 16; ++i) {                        // scores beside probabilities
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x402, 5, 0);
          }
#pragma unroll
          for (int i = 0; i < 32; ++i) {                        // P.V beside the maxima
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x402, 2, 0);
          }
        };
        block((tt + 1) * kPfTok + kPfTok - 1 > wpos_lo);
      } else {
        if (tt < w_end) {
          bf16x8 w0[4], w1[4];
          read_v(tt, vring[lt % kPfNbuf], 0, w0, true);
          probs(s_cur, m_run, ph, pl, lsum);
          pv(w0, 0, ph, pl);
          read_v(tt, vring[lt % kPfNbuf], 1, w1, true);
          pv(w1, 1, ph, pl);
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) alpha[rb] = 1.f;
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) l_lane[rb] += lsum[rb];
      if (rise) {
        keep_branch();
        rescale(alpha);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) l_lane[rb] *= alpha[rb];
      }
      if (tt + 1 < w_end) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) m_run[rb] = mnew[rb];
      }
    };
    for (int lt = 0; t_lo + lt < t_hi; lt += 2) {
      step(lt, sA, sB);
      if (t_lo + lt + 1 >= t_hi) break;
      step(lt + 1, sB, sA);
    }
    wait_copies<0>();
    bare_barrier();   // every wave is done with the ring, which now stages the record

    // Rows 16 rb + 4 quarter + i of the wave, each normalised by its own sum (summed
    // across the four lanes of the row), are written to the wave's 8 KiB of the ring as
    // [row][dim] (lane n holds dims 16 e + n) and read back 16 contiguous bytes per lane,
    // so that every store covers whole rows: the output rows of an item of one piece,
    // else the piece's record (with m and l per row; a row without tokens in this piece
    // has l = 0, m = -inf and o = 0).
    const bool direct = npc == 1;
    const int64_t rec0 = ((int64_t)item * kPfMaxPieces + piece) * kMqPrefillUnit;
    // (the lane index through an empty asm: the addresses below are then formed here, per
    // piece, instead of being hoisted out of the piece loop and held in registers)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int rq = ln >> 4, rc = ln & 15;
    if (wave_live) {
      float* stage = reinterpret_cast<float*>(wave < 4 ? &kring[0][0] : &vring[0][0]) + (wave & 3) * 16 * D;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float l_row = sum_xor32(sum_xor16(l_lane[rb]));   // row 16 rb + col
        if (!direct && rq == 0) {
          a.ws_m[rec0 + wrow0 + rb * 16 + rc] = m_run[rb];
          a.ws_l[rec0 + wrow0 + rb * 16 + rc] = l_row;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lr = __shfl(l_row, 4 * rq + i);
          const float inv = direct ? (seq_bad ? __builtin_nanf("") : 1.f / lr) : (lr > 0.f ? 1.f / lr : 0.f);
#pragma unroll
          for (int e = 0; e < CPL; ++e) stage[(4 * rq + i) * D + 16 * e + rc] = acc[rb][e][i] * inv;
        }
        // (a wave's LDS accesses complete in order: the reads see these writes, and the next
        // block's writes come after these reads)
        if (!direct) {
#pragma unroll
          for (int k = 0; k < 16 * (D / 4) / kWave; ++k) {
            const int c = k * kWave + ln;
            const int i = c / (D / 4), ch = c % (D / 4);
            const floatx4 v = *reinterpret_cast<const floatx4*>(stage + i * D + ch * 4);
            *reinterpret_cast<floatx4*>(a.ws_o + (rec0 + wrow0 + rb * 16 + i) * D + ch * 4) = v;
          }
        } else if (a.out_bf16) {
#pragma unroll
          for (int k = 0; k < 16 * (D / 8) / kWave; ++k) {
            const int c = k * kWave + ln;
            const int i = c / (D / 8), ch = c % (D / 8);
            const floatx4 x = *reinterpret_cast<const floatx4*>(stage + i * D + ch * 8);
            const floatx4 y = *reinterpret_cast<const floatx4*>(stage + i * D + ch * 8 + 4);
            const int r = wrow0 + rb * 16 + i;
            const int jq = j0 + r / G;
            if (jq < qlen) {
              uint4 v;
              v.x = f32_to_bf16_rne(x[0]) | (uint32_t)f32_to_bf16_rne(x[1]) << 16;
              v.y = f32_to_bf16_rne(x[2]) | (uint32_t)f32_to_bf16_rne(x[3]) << 16;
              v.z = f32_to_bf16_rne(y[0]) | (uint32_t)f32_to_bf16_rne(y[1]) << 16;
              v.w = f32_to_bf16_rne(y[2]) | (uint32_t)f32_to_bf16_rne(y[3]) << 16;
              *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) +
                                        ((int64_t)(q0 + jq) * H + g * G + r % G) * D + ch * 8) = v;
            }
          }
        } else {
#pragma unroll
          for (int k = 0; k < 16 * (D / 4) / kWave; ++k) {
            const int c = k * kWave + ln;
            const int i = c / (D / 4), ch = c % (D / 4);
            const floatx4 v = *reinterpret_cast<const floatx4*>(stage + i * D + ch * 4);
            const int r = wrow0 + rb * 16 + i;
            const int jq = j0 + r / G;
            if (jq < qlen)
              *reinterpret_cast<floatx4*>(static_cast<float*>(a.out) +
                                          ((int64_t)(q0 + jq) * H + g * G + r % G) * D + ch * 4) = v;
          }
        }
      }
    }
    if (direct) continue;

    // Count the piece in: the records are released at agent scope before the count, and
    // the piece that counts last acquires the others' and merges them.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (threadIdx.x == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const int prev = __hip_atomic_fetch_add(PL.ctr + item, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      merge_flag = prev == npc - 1;
      if (prev == npc - 1) {
        // cleared for a later launch on the same plan
        __hip_atomic_store(PL.ctr + item, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      }
    }
    __syncthreads();
    if (merge_flag) {
      // Output rows of the unit's real rows: the records merged in piece order (so that
      // the result does not depend on which piece came last), NI4 row pieces of 4 dims
      // per thread and round.
      constexpr int C4 = D / 4;
      constexpr int NI4 = 4;
      constexpr int NT = kPfWaves * kWave;
      static_assert(kMqPrefillUnit * C4 % (NT * NI4) == 0, "whole rounds of row pieces");
      const int64_t rb0 = (int64_t)item * kPfMaxPieces * kMqPrefillUnit;   // piece h at + h * rows
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
#pragma unroll 1
      for (int c0 = tid; c0 < kMqPrefillUnit * C4; c0 += NT * NI4) {
        float mx[NI4], wsum[NI4];
        floatx4 osum[NI4];
#pragma unroll
        for (int u = 0; u < NI4; ++u) {
          mx[u] = -__builtin_inff();
          wsum[u] = 0.f;
          osum[u] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
        for (int h = 0; h < npc; ++h) {
#pragma unroll
          for (int u = 0; u < NI4; ++u)
            mx[u] = fmaxf(mx[u], a.ws_m[rb0 + h * kMqPrefillUnit + (c0 + u * NT) / C4]);
        }
        for (int h = 0; h < npc; ++h) {
          float m[NI4], l[NI4];
          floatx4 o[NI4];
#pragma unroll
          for (int u = 0; u < NI4; ++u) {
            const int64_t x = rb0 + h * kMqPrefillUnit + (c0 + u * NT) / C4;
            m[u] = a.ws_m[x];
            l[u] = a.ws_l[x];
            o[u] = *reinterpret_cast<const floatx4*>(a.ws_o + x * D + ((c0 + u * NT) % C4) * 4);
          }
#pragma unroll
          for (int u = 0; u < NI4; ++u) {
            const float w = l[u] * rel_scale(m[u], mx[u]);
            wsum[u] += w;
#pragma unroll
            for (int e = 0; e < 4; ++e) osum[u][e] = fmaf(w, o[u][e], osum[u][e]);
          }
        }
#pragma unroll
        for (int u = 0; u < NI4; ++u) {
          const int r = (c0 + u * NT) / C4, ch = (c0 + u * NT) % C4;
          const int jq = j0 + r / G;
          if (jq >= qlen) continue;
          const float inv = seq_bad ? __builtin_nanf("") : 1.f / wsum[u];
          float res[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) res[e] = osum[u][e] * inv;
          const int64_t o = ((int64_t)(q0 + jq) * H + g * G + r % G) * D + ch * 4;
          if (a.out_bf16) {
            const uint2 v = make_uint2(f32_to_bf16_rne(res[0]) | (uint32_t)f32_to_bf16_rne(res[1]) << 16,
                                       f32_to_bf16_rne(res[2]) | (uint32_t)f32_to_bf16_rne(res[3]) << 16);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + o) = v;
          } else {
            *reinterpret_cast<floatx4*>(static_cast<float*>(a.out) + o) =
                floatx4{res[0], res[1], res[2], res[3]};
          }
        }
      }
    }
  }   // pieces
}

template <int G>
static hipError_t launch_prefill_g(const AttentionArgs& a, hipStream_t stream) {
  // a.grid_wgs workgroups (one per compute unit, a multiple of the XCD count; the plan's
  // tile target is per workgroup), each taking its XCD's pieces in snake order
  if (a.grid_wgs < kXcds || a.grid_wgs % kXcds != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(paged_attention_prefill_kernel<G>, dim3((unsigned)a.grid_wgs),
                     dim3(kPfWaves * kWave), 0, stream, a);
  return hipGetLastError();
}

static hipError_t launch_prefill(const AttentionArgs& a, hipStream_t stream) {
  switch (a.num_heads / a.num_kv_heads) {
    case 1: return launch_prefill_g<1>(a, stream);
    case 2: return launch_prefill_g<2>(a, stream);
    case 4: return launch_prefill_g<4>(a, stream);
    case 8: return launch_prefill_g<8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

// ---- merge of the segments ----------------------------------------------------------
// Two kinds of workgroups.  The first max_units * Hkv take one (unit, kv head) each:
// a unit inside one share was written by the attention kernel and its workgroup
// exits; otherwise the workgroup folds the unit's records of that kv head, share by
// share in share order, and writes the rows.  The unit's records of one kv head and
// label are contiguous rows, so the loads are whole rows, and the unit, its sequence
// and its shares come from a few independent loads (no search).  The last
// num_tokens workgroups take one new token each and give NaN rows to the tokens that
// belong to no valid sequence (or to every token, when the plan has no units).
template <int D>
__global__ __launch_bounds__(256) void paged_attention_multi_reduce_kernel(AttentionArgs a) {
  constexpr int C4 = D / 4;              // float4 pieces of a row
  constexpr int KS = 2;                  // shares whose records are loaded together
  constexpr int NI = 2;                  // items per thread whose records are loaded together
  const int H = a.num_heads;
  const int Hkv = a.num_kv_heads;
  const int G = H / Hkv;
  const int rows = a.unit_rows;
  cint32* hdr = (cint32*)a.tile_hdr;
  cint32* qsl = (cint32*)a.query_start_loc;
  // prefill units merge their own pieces: only the NaN rows are left to write
  const int64_t unit_wgs = a.unit_rows == kMqPrefillUnit ? 0 : (int64_t)a.max_units * Hkv;
  if ((int64_t)blockIdx.x >= unit_wgs) {
    const int t = (int)((int64_t)blockIdx.x - unit_wgs);
    // the sequence holding token t: the last i with qsl[i] <= t (64-way search)
    int lo = 0, len = a.num_seqs + 1;
    const int lane = threadIdx.x & (kWave - 1);
    while (len > 1) {
      const int step = (len + kWave - 1) / kWave;
      const int i = lo + lane * step;
      const bool ok = i < lo + len && qsl[i] <= t;
      const int k = __builtin_amdgcn_readfirstlane(__popcll(__ballot(ok)));
      const int nlo = lo + (max(k, 1) - 1) * step;
      len = min(step, lo + len - nlo);
      lo = nlo;
    }
    const int i = lo;
    const int q0 = qsl[i], q1 = qsl[i + 1];
    const int max_ctx = a.max_blocks_per_seq << a.block_shift;
    const bool valid = hdr[2] > 0 && t >= q0 && t < q1 &&
                       seq_valid(q0, q1, ((cint32*)a.context_lens)[i], a.num_tokens, max_ctx);
    if (valid) return;
    const float nan = __builtin_nanf("");
    for (int k = threadIdx.x; k < H * C4; k += 256)
      store_row4(a, ((int64_t)t * H) * D + k * 4, Running{0.f, 1.f, make_float4(nan, nan, nan, nan)});
    return;
  }
  const int u = blockIdx.x / Hkv;
  const int g = blockIdx.x % Hkv;
  const int U = hdr[2];
  if (u >= U) return;
  const int c0 = ((cint32*)a.tile_cum)[u], c1 = ((cint32*)a.tile_cum)[u + 1];
  const int seq = ((cint32*)a.unit_seq)[u];
  const int total = hdr[0];
  const int nwg = hdr[1];
  const int w0 = share_of((int64_t)c0 + kSeqCost, nwg, total);
  const int w1 = share_of((int64_t)c1 - 1, nwg, total);
  if (w0 == w1) return;
  const int q0 = qsl[seq];
  const int qlen = qsl[seq + 1] - q0;
  const int uj0 = (u - ((cint32*)a.seq_unit)[seq]) * (rows / G);
  const int nrows = min(rows, (qlen - uj0) * G);          // the unit's real rows
  const int64_t lab_stride = (int64_t)Hkv * rows;           // between labels L and L + 1
  const int64_t base = ((int64_t)u * Hkv + g) * rows;        // record row 0 under label 0
  // Each thread merges NI (row, float4) items of the unit; the records of all NI items
  // and KS shares are loaded before any is merged, so one round of loads covers a unit
  // split over at most KS shares.
  const int items = nrows * C4;
  for (int k0 = threadIdx.x; k0 < items; k0 += 256 * NI) {
    Running acc[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) acc[i] = Running{-__builtin_inff(), 0.f, make_float4(0.f, 0.f, 0.f, 0.f)};
    for (int wb = w0; wb <= w1; wb += KS) {
      float l[NI][KS], m[NI][KS];
      floatx4 o[NI][KS];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int k = min(k0 + 256 * i, items - 1);   // past the unit's items: a repeat
        const int r = k / C4, c = k % C4;
#pragma unroll
        for (int q = 0; q < KS; ++q) {
          const int ww = min(wb + q, w1);
          const int64_t rec = base + (int64_t)ww * lab_stride + r;
          l[i][q] = a.ws_l[rec];
          m[i][q] = a.ws_m[rec];
          o[i][q] = reinterpret_cast<const floatx4*>(a.ws_o + rec * D)[c];
        }
      }
      // Records of segments in which a row saw no token have l = 0 (and m = -inf);
      // they weigh nothing.  A NaN l marks bad data and is kept.  Empty shares wrote
      // no record.
#pragma unroll
      for (int q = 0; q < KS; ++q) {
        const int ww = wb + q;
        if (ww > w1 || !share_nonempty(ww, nwg, total)) continue;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          if (!(l[i][q] > 0.f) && !(l[i][q] != l[i][q])) continue;
          const float lq = l[i][q];
          const Running sg{m[i][q], lq, make_float4(o[i][q][0] * lq, o[i][q][1] * lq,
                                                   o[i][q][2] * lq, o[i][q][3] * lq)};
          merge_into(acc[i], sg);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int k = k0 + 256 * i;
      if (k >= items) break;
      const int r = k / C4, c = k % C4;
      const int jq = uj0 + r / G;
      store_row4(a, ((int64_t)(q0 + jq) * H + g * G + r % G) * D + c * 4, acc[i]);
    }
  }
}

void select_multi_mode(AttentionArgs* a) {
  // bf16 caches with 128-element heads whose rows would take the row-split mode take
  // the 256-row prefill units instead when those fill the GPU at least once (at least
  // one (unit, kv head) item per compute unit; PKV_PREFILL_MIN_ITEMS sets another
  // threshold, 0 to always take them)
  if (a->unit_rows != kMqRowUnit || !a->kv_bf16 || a->head_dim != 128) return;
  const int G = a->num_heads / a->num_kv_heads;
  const int64_t tpb = kMqPrefillUnit / G;
  const int64_t units = ((int64_t)a->num_tokens + tpb - 1) / tpb;
  int64_t min_items = device_cus();
  if (const char* env = getenv("PKV_PREFILL_MIN_ITEMS")) min_items = atoll(env);
  if (units * a->num_kv_heads < min_items) return;
  a->unit_rows = kMqPrefillUnit;
  a->max_units = (int)(units + a->num_seqs);   // within the arrays sized for row-split units
  // one workgroup per compute unit, a multiple of the XCD count
  a->grid_wgs = max(kXcds, device_cus() / kXcds * kXcds);
}

hipError_t launch_attention_multi_reduce(const AttentionArgs& a, hipStream_t stream) {
  const int64_t wgs =
      (a.unit_rows == kMqPrefillUnit ? 0 : (int64_t)a.max_units * a.num_kv_heads) + a.num_tokens;
  if (wgs > INT32_MAX) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)wgs);
  if (a.head_dim == 64)
    hipLaunchKernelGGL(paged_attention_multi_reduce_kernel<64>, grid, dim3(256), 0, stream, a);
  else if (a.head_dim == 128)
    hipLaunchKernelGGL(paged_attention_multi_reduce_kernel<128>, grid, dim3(256), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---- dispatch ------------------------------------------------------------------

template <typename T, int D, int G, int HW, int RB, int NW, int NBUF = 2>
static hipError_t launch_multi_rb(const AttentionArgs& a, hipStream_t stream) {
  auto kernel = paged_attention_multi_kernel<T, D, G, HW, RB, NW, NBUF>;
  static const int per_cu = [&] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, NW * kWave, 0) != hipSuccess)
      n = 1;
    return n > 0 ? n : 1;
  }();
  const int cus = device_cus();
  if (cus <= 0) return hipErrorInvalidDevice;
  const int hgroups = a.num_kv_heads / HW;
  const int nwg = max(1, min(kMaxStreamWgs, per_cu * cus / hgroups));
  hipLaunchKernelGGL(kernel, dim3(nwg, hgroups), dim3(NW * kWave), 0, stream, a);
  return hipGetLastError();
}

// Ring depth of the head mode (one wave per kv head of the workgroup).
#ifndef PKV_MULTI_HEAD_NBUF
#define PKV_MULTI_HEAD_NBUF 2
#endif

template <typename T, int D, int G, int HW>
static hipError_t launch_multi_shape(const AttentionArgs& a, hipStream_t stream) {
  constexpr int NB = PKV_MULTI_HEAD_NBUF;
  return a.unit_rows == 32 ? launch_multi_rb<T, D, G, HW, 2, HW, NB>(a, stream)
                           : launch_multi_rb<T, D, G, HW, 1, HW, NB>(a, stream);
}

// Ring depth of the row-split mode: its tiles are one head's rows (a quarter or less
// of a whole-row tile), so more of them are kept in flight.
#ifndef PKV_MULTI_ROW_NBUF
#define PKV_MULTI_ROW_NBUF 2
#endif

#ifndef PKV_MULTI_MAX_ROW
#define PKV_MULTI_MAX_ROW 2048
#endif

// Heads per workgroup: the largest of 8, 4, 2, 1 dividing the kv heads with a token
// row of the group within PKV_MULTI_MAX_ROW bytes and at least 128 bytes.  Whole 2 KiB
// rows (8 bf16 heads of 128) with one workgroup per compute unit: 310 us per launch
// for 5 speculated tokens per sequence on the Llama-3-8B-shaped batch, against 320 us
// with 1 KiB rows and two workgroups per unit (MI355X).
template <typename T, int D, int G>
static hipError_t launch_multi_hw(const AttentionArgs& a, hipStream_t stream) {
  constexpr int kRow = D * T::kElemBytes;
  // long prompts: four waves share one kv head's rows, 128 rows per unit
  if constexpr (16 * kRow % (kMqRowWaves * 1024) == 0)
    if (a.unit_rows == kMqRowUnit)
      return launch_multi_rb<T, D, G, 1, kMqRowRB, kMqRowWaves, PKV_MULTI_ROW_NBUF>(a, stream);
  if constexpr (8 * kRow <= PKV_MULTI_MAX_ROW)
    if (a.num_kv_heads % 8 == 0) return launch_multi_shape<T, D, G, 8>(a, stream);
  if constexpr (4 * kRow <= PKV_MULTI_MAX_ROW)
    if (a.num_kv_heads % 4 == 0) return launch_multi_shape<T, D, G, 4>(a, stream);
  if constexpr (2 * kRow <= PKV_MULTI_MAX_ROW)
    if (a.num_kv_heads % 2 == 0) return launch_multi_shape<T, D, G, 2>(a, stream);
  return launch_multi_shape<T, D, G, 1>(a, stream);
}

template <typename T, int D>
static hipError_t launch_multi_g(const AttentionArgs& a, hipStream_t stream) {
  switch (a.num_heads / a.num_kv_heads) {
    case 1: return launch_multi_hw<T, D, 1>(a, stream);
    case 2: return launch_multi_hw<T, D, 2>(a, stream);
    case 4: return launch_multi_hw<T, D, 4>(a, stream);
    case 8: return launch_multi_hw<T, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attention_multi(const AttentionArgs& a, hipStream_t stream) {
  if (a.unit_rows == kMqPrefillUnit) return launch_prefill(a, stream);
  if (a.kv_bf16) {
    if (a.head_dim == 64) return launch_multi_g<BF16, 64>(a, stream);
    if (a.head_dim == 128) return launch_multi_g<BF16, 128>(a, stream);
  } else {
    if (a.head_dim == 64) return launch_multi_g<F32, 64>(a, stream);
    if (a.head_dim == 128) return launch_multi_g<F32, 128>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
