// PagedAttention decode, balanced mode: a streaming partition stage and its merge.
//
// What is computed is the same as in paged_attention.hip (page "vllm源码分析：我是
// 如何一步步读懂PagedAttention核心实现的？", 第三讲, and page "vLLM PagedAttention 原理与
// 源码深度解析", section 5.3): per sequence and query head, scaled dot products with
// the context's keys found through the block table, a softmax, the weighted sum of
// the values.  Splitting a context into pieces merged by log-sum-exp leaves the
// result unchanged; where the pieces fall is this design's choice.
//
// Work split.  All (sequence, tile) pairs, a tile being 16 consecutive tokens of one
// sequence, form one ordered list; each sequence's tiles are preceded by kSeqCost
// positions that stand for the fixed cost of starting and closing a sequence, so
// that shares crossing many short sequences get fewer tiles (the tile plan holds
// the prefix sums).  The grid has as many workgroups per kv-head group as the GPU
// holds at once, and workgroup w takes the w-th of that many equal contiguous
// shares of the list.  It streams
// through its share without a break: the copies of the next tile are in flight
// while a tile is computed, also across sequence boundaries, and every workgroup
// ends at about the same time.  The run of one sequence inside one share is a
// segment.  A segment that is a whole sequence writes its output directly; the
// others write their (m, l, o) record under the label w + sequence (labels grow
// along the list, so they are unique), and the merge kernel combines a sequence's
// records in share order.
//
// How the bytes move.  One wave per kv head of the workgroup's group of HW heads.
// A tile is the 16 token rows of the HW heads' keys and values, HW*D*elem bytes per
// row, which the heads of one block row hold contiguously (the whole 2 KiB row of
// a Llama-3-8B-shaped cache).  The workgroup copies it from HBM straight into LDS
// with 16-byte direct-to-LDS loads, each wave instruction covering 1 KiB of
// consecutive bytes, so every token row is fetched whole and at once.  On MI355X
// this reads the batch's blocks at up to 6.2 TB/s, against 5.5-5.9 TB/s when each
// head's 256-byte pieces are read by a workgroup of their own.
//
// LDS image of a tile: row r at r*ROW bytes; its 16-byte slots are XOR-swizzled
// (slot j of the row is stored at j ^ (r & 15)), so that sixteen lanes reading the
// same slot of sixteen rows (the MFMA key operand) or sixteen slots of one row (the
// value reads) hit sixteen different bank groups.  The swizzle is done on the
// global side: each lane fetches the global slot that belongs in its LDS slot.
//
// NBUF tiles rotate through distinct LDS buffers.  Per tile: issue the copies of
// the tile NBUF - 1 ahead, wait for this wave's copies of the tile, barrier, compute
// the tile from LDS: Q.K^T on the matrix cores (the GQA group of the wave's head as
// the A operand; groups of one or two heads as dot products on the VALU), online
// softmax in the base-2 exponent domain, P.V on the matrix cores (bf16 and E4M3 caches,
// 128-element heads, groups of four or eight) or on the VALU in fp32; barrier.  While
// a wave waits for a tile, the tiles after it are already in flight.  No atomics:
// results do not depend on timing.
#include "pkv_device.hpp"
#include "pkv_launch.hpp"
#include "pkv_plan.hpp"
#include "pkv_stream.hpp"
#include "pkv_tile.hpp"

#include <type_traits>

namespace pkv {

// Segment-end stores (outputs and records), non-temporal when NT: each is written once
// while the tile copies stream, and the merge reads the records back from memory.  With
// bf16 caches that took the Llama-3-8B-shaped batch from 260.1-261.8 to 255.7-257.4 us
// and the long-context batch in 512-token partitions from 434-435 to 410 us; with E4M3
// caches it cost 1-2 us, so they keep ordinary stores.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <bool NT, typename V>
__device__ __forceinline__ void st_seg(V* p, V v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}
template <bool NT>
__device__ __forceinline__ void st_seg4(float* p, float x, float y, float z, float w) {
  st_seg<NT>(reinterpret_cast<floatx4*>(p), floatx4{x, y, z, w});
}


#ifndef PKV_STREAM_NBUF
#define PKV_STREAM_NBUF 2
#endif
// E4M3 caches: a tile is half the bytes, and the per-tile compute no longer hides
// under its copies with one workgroup per compute unit; two workgroups of 8 waves
// share one when the registers allow it (WPE: waves per SIMD the register budget
// must allow; measured on MI355X, Llama-3-8B-shaped batch: 192 us with one
// workgroup per CU, 178 us with two; a third or fourth ring buffer did not help).
#ifndef PKV_STREAM_NBUF_FP8
#define PKV_STREAM_NBUF_FP8 2
#endif
#ifndef PKV_STREAM_WPE_FP8
#define PKV_STREAM_WPE_FP8 4
#endif

// KV tiles are copied non-temporal (streamed past the caches) unless built with
// PKV_STREAM_KV_NT=0.
#ifndef PKV_STREAM_KV_NT
#define PKV_STREAM_KV_NT 1
#endif
constexpr Cpol kKvCpol = PKV_STREAM_KV_NT ? Cpol::kStream : Cpol::kDefault;

template <typename T>
constexpr int stream_nbuf() { return T::kElemBytes == 1 ? PKV_STREAM_NBUF_FP8 : PKV_STREAM_NBUF; }
// GQA groups of 8 need more registers than a 4-wave-per-SIMD budget holds
template <typename T, int G>
constexpr int stream_wpe() { return T::kElemBytes == 1 && G <= 4 ? PKV_STREAM_WPE_FP8 : 1; }

// Cache policy of the KV tile copies in fixed-partition mode (1: non-temporal, as in the
// balanced split).
#ifndef PKV_STREAM_FIXED_NT
#define PKV_STREAM_FIXED_NT 1
#endif

// FIXED: fixed partitions of a.partition_size tokens instead of the balanced split.
// Workgroup w then takes work item w of the fixed plan (sequence, partition, context
// length, partitions), streams that partition's tiles in the same way, and writes the
// output (a sequence of one partition) or the partition's record in the layout the
// fixed-partition merge reads: (sequence * H + head) * max_parts + partition.
template <typename T, int D, int G, int HW, int NBUF, bool FIXED>
__global__ __launch_bounds__(HW * kWave) __attribute__((amdgpu_waves_per_eu(stream_wpe<T, G>())))
void paged_attention_stream_kernel(AttentionArgs a) {
  constexpr Cpol kPol = FIXED && !PKV_STREAM_FIXED_NT ? Cpol::kDefault : kKvCpol;
  constexpr int TOK = kTileTokens;
  using St = Stage<T, D, HW, TOK>;
  constexpr bool kF8 = T::kElemBytes == 1;  // E4M3 caches, bfloat16 queries
  constexpr bool kNtSeg = !kF8;              // non-temporal segment-end stores
  using QT = typename std::conditional<kF8, BF16, T>::type;   // query and MFMA operand type
  constexpr int EB = T::kElemBytes;
  constexpr int QEB = QT::kElemBytes;
  constexpr int NCH = D * EB / 16;          // 16-byte chunks of one head's cache row
  constexpr int QKC = D * QEB / 64;         // query chunks per lane = MFMAs per tile
  constexpr int KCH = kF8 ? D / 64 : QKC;   // 16-byte key chunks a lane reads per tile
  constexpr int PB = kF8 ? 8 : 16;          // bytes of one lane's piece of a value row
  constexpr int EPL = PB / EB;              // value elements per piece
  constexpr int NPC = D * EB / PB;          // pieces per head's value row
  constexpr int RPS = kWave / NPC;          // value rows per wave read
  constexpr int STEPS = TOK / RPS;
  constexpr int kQuarters = (G + 3) / 4;    // MFMA output quarters holding real heads
  // GQA groups of four or eight heads: Q.K^T on the matrix cores, and P.V too with bf16
  // and E4M3 caches and D = 128 (fp32 caches and D = 64 use fp32 FMAs on the VALU).
  // Groups of one or two heads would fill one or two of a matrix instruction's 16
  // rows: their dot products and P.V run on the VALU.
  constexpr bool kValuQK = G <= 2;
  constexpr bool kMfmaPV = (kF8 || std::is_same<T, BF16>::value) && D == 128 && !kValuQK;
  static_assert(NCH % 4 == 0 || kF8, "row shape");
  constexpr int L = 2 * St::kCopies;        // copy instructions per wave per tile
  constexpr int NS = St::kTileSlots;
  static_assert(TOK % RPS == 0 && TOK <= 16, "tile rows");
  static_assert(NBUF >= 2 && NBUF <= 4, "buffers");

  // Distinct objects per buffer, so that reads of one buffer are never made to wait
  // for copies into another.
  __shared__ uint4 kb0[NS], vb0[NS], kb1[NS], vb1[NS];
  __shared__ uint4 kb2[NBUF > 2 ? NS : 1], vb2[NBUF > 2 ? NS : 1];
  __shared__ uint4 kb3[NBUF > 3 ? NS : 1], vb3[NBUF > 3 ? NS : 1];
  // probabilities of the tile: [token][head], or [head][token] for the matrix P.V
  __shared__ float p_lds[HW][kMfmaPV ? G : 16][kMfmaPV ? 16 : G];
  // the query rows of each wave's GQA group, copied in like the tiles
  constexpr int QB = G * D * QEB;
  __shared__ uint4 q_lds[HW][QB / 16];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int nwg = gridDim.x;                // workgroups per kv-head group
  const int w = blockIdx.x;
  const int hg = blockIdx.y;
  const int B = a.num_seqs;
  const int H = a.num_kv_heads * G;
  const int g = hg * HW + wave;             // this wave's kv head

  cint32* cum = (cint32*)a.tile_cum;
  cint32* ctx_of = (cint32*)a.context_lens;
  cint32* tables = (cint32*)a.block_tables;
  int64_t start = 0, end = 0;
  int seq0 = 0;
  int fx_p = 0, fx_ctx = 0;   // fixed partitions: the item's partition and context length
  if constexpr (FIXED) {
    // Items are checked, so that a stale plan gives wrong numbers but never an
    // out-of-range access.
    cint32* items = (cint32*)a.plan_items;
    const int count = min(((cint32*)a.plan_count)[0], B * a.max_parts);
    if (w >= count) return;
    seq0 = items[4 * w];
    fx_p = items[4 * w + 1];
    fx_ctx = items[4 * w + 2];
    if (seq0 < 0 || seq0 >= B || fx_p < 0 || fx_p >= a.max_parts) return;
    if (fx_ctx < 1 || fx_ctx > (a.max_blocks_per_seq << a.block_shift)) {
      // invalid context length: NaN rows, written by the item of partition 0
      if (fx_p == 0)
        for (int i = lane; i < G * D; i += kWave)
          store_out(a.out, ((int64_t)seq0 * H + g * G) * D + i, __builtin_nanf(""), a.out_bf16);
      return;
    }
    if ((int64_t)fx_p * a.partition_size >= fx_ctx) return;
  } else {
    const int total = ((cint32*)a.tile_hdr)[0];
    if (w == 0 && hg == 0 && threadIdx.x == 0) a.tile_hdr[1] = nwg;   // for the merge
    start = (int64_t)w * total / nwg;
    end = (int64_t)(w + 1) * total / nwg;
    if (start >= end) return;

    // The sequence holding position `start`: the last i in [0, B] with cum[i] <=
    // start (sequences without tiles share their cum value with the next one).  A
    // 64-way search, one vector load per round.
    int lo = 0, len = B + 1;
    while (len > 1) {
      const int step = (len + kWave - 1) / kWave;
      const int i = lo + lane * step;
      const bool ok = i < lo + len && a.tile_cum[i] <= start;
      const int k = __builtin_amdgcn_readfirstlane(__popcll(__ballot(ok)));
      const int nlo = lo + (k - 1) * step;
      len = min(step, lo + len - nlo);
      lo = nlo;
    }
    seq0 = lo;
  }

  const int quarter = lane >> 4;   // MFMA operand k-group / output row group
  const int col = lane & 15;       // MFMA A row (head) and B column (token)
  const int rg = lane / NPC;       // value row within a step
  const int li = lane % NPC;       // piece within a head's value row

  // Copy geometry.  Copy instruction i of this wave fills LDS slots
  // [(i*HW + wave)*64, +64) of the tile image; this lane's slot is row r, slot p,
  // and it fetches the global slot p ^ (r & swz) of that row.
  const int64_t row_stride = (int64_t)a.num_kv_heads * D * EB;   // between tokens of a block
  uint32_t copy_off[St::kCopies];
#pragma unroll
  for (int i = 0; i < St::kCopies; ++i) {
    const int s = (i * HW + wave) * kWave + lane;
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
  const int num_blocks = (int)a.num_blocks;               // the ABI keeps it below 2^31
  const float kNegInf = -__builtin_inff();

  // A cursor over the real tiles of this share: sequence s, tile t, tiles of the
  // sequence nt, and stop, the end of the share's part of the sequence (t < stop
  // while the cursor is valid).  Sequence i's real tile t sits at position
  // cum[i] + kSeqCost + t of the list.
  struct Cursor {
    int s, t, nt, stop;
  };
  // Moves c to the next sequence with real tiles in this share, or invalidates it.
  // The cursor is wave-uniform; readfirstlane keeps it in scalar registers, so the
  // plan is read with scalar loads whose waits leave the copies in flight alone.
  auto next_seq = [&](Cursor& c) {
    if constexpr (FIXED) {   // one partition per workgroup
      c.s = B;
      c.t = c.stop = 0;
      return;
    }
    int s = uniform(c.s);
    int cs = cum[s + 1];
    for (;;) {
      ++s;
      if (s >= B || cs + kSeqCost >= end) {
        c.s = s;
        c.t = c.stop = 0;
        return;
      }
      const int cn = uniform(cum[s + 1]);
      if (cn > cs) {
        c.s = s;
        c.t = 0;
        c.nt = cn - cs - kSeqCost;
        c.stop = uniform(min(c.nt, (int)(end - cs - kSeqCost)));
        return;
      }
      cs = cn;
    }
  };
  auto first_cursor = [&](Cursor& c) {
    if constexpr (FIXED) {
      const int tp = a.partition_size / TOK;   // a multiple of 16 tokens
      c.s = seq0;
      c.nt = uniform((fx_ctx + TOK - 1) / TOK);
      c.t = uniform(fx_p * tp);
      c.stop = uniform(min(c.nt, c.t + tp));
      return;
    }
    const int cs = cum[seq0];
    c.s = seq0;
    c.nt = uniform(cum[seq0 + 1] - cs - kSeqCost);
    c.t = uniform(max(0, (int)(start - cs - kSeqCost)));
    c.stop = uniform(min(c.nt, (int)(end - cs - kSeqCost)));
    if (c.t >= c.stop) next_seq(c);
  };
  auto advance = [&](Cursor& c) {
    if (++c.t == c.stop) next_seq(c);
  };

  // ---- issue side: the copies of the next tile of the share ----------------------
  Cursor ic;
  first_cursor(ic);
  // Copies of the tile under the issue cursor into (kb, vb), then advance.  Past the
  // share's end, or behind an invalid block id, pool block 0 is copied instead:
  // always in bounds, and the copy count per tile stays fixed, which the wait counts
  // rely on.  bad_pipe bit k: the tile issued k issues ago sat behind an invalid
  // block id.
  unsigned bad_pipe = 0;
  auto issue = [&](uint4* kb, uint4* vb) {
    int64_t base = 0;
    bad_pipe <<= 1;
    if (ic.t < ic.stop) {
      const int tok0 = uniform(ic.t * TOK);
      // a tile past the table (possible only with a stale plan) counts as invalid
      const int32_t blk =
          uniform(tok0 < max_ctx ? tables[(int64_t)uniform(ic.s) * MB + (tok0 >> shift)] : -1);
      if (blk >= 0 && blk < num_blocks)
        base = (((int64_t)blk << shift) + (tok0 & bs_mask)) * row_stride;
      else
        bad_pipe |= 1u;
      advance(ic);
    }
    const uint32_t kd = lds_addr(kb) + wave * 1024;
    const uint32_t vd = lds_addr(vb) + wave * 1024;
    const char* kbase = kcache + base;
    const char* vbase = vcache + base;
#pragma unroll
    for (int i = 0; i < St::kCopies; ++i) dma16<kPol>(kbase, copy_off[i], kd + i * HW * 1024);
#pragma unroll
    for (int i = 0; i < St::kCopies; ++i) dma16<kPol>(vbase, copy_off[i], vd + i * HW * 1024);
  };

  // ---- compute side ------------------------------------------------------------------
  Cursor cc;
  first_cursor(cc);
  if (cc.t >= cc.stop) return;           // only sequence overheads in this share
  int cctx = ctx_of[cc.s];
  bool seg_from_zero = cc.t == 0;        // the segment began at the sequence's first tile
  int seg_bad = 0;

  // Query rows of this kv head's group as the MFMA A operand.  A new sequence's G
  // rows (contiguous in the query) are copied into q_lds with the tiles' copies, and
  // read into registers at its first tile; row m of the operand holds query head
  // m % G (the rows past G repeat real ones and their scores are never used).
  // MFMA c takes the k-range [32c, 32c + 32) of the products (8c and 16c for fp32,
  // in its steps of 4) in row chunks 4c + quarter.  With an E4M3 cache a lane instead
  // takes the contiguous query chunks QKC * quarter + c, matching the contiguous key
  // bytes it reads; a dot product may sum its terms in any order.
  uint4 qa[kValuQK ? 1 : QKC];
  bool q_fresh = false;   // a query copy was issued after the last step's copies
  auto load_query = [&](int s) {
    q_fresh = true;
    const char* src =
        static_cast<const char*>(a.query) + ((int64_t)s * H + g * G) * (D * QEB);
#pragma unroll
    for (int i = 0; i < (QB + 1023) / 1024; ++i) {
      if (QB >= (i + 1) * 1024 || lane * 16 < QB - i * 1024)
        dma16(src, (uint32_t)((i * kWave + lane) * 16), lds_addr(q_lds[wave]) + i * 1024);
    }
  };
  // (VALU scores read the query from q_lds at every tile instead: it stays there until
  // the sequence's last tile is done)
  auto read_query = [&]() {
    if constexpr (!kValuQK) {
      const uint4* q = q_lds[wave] + (col % G) * (D * QEB / 16);
#pragma unroll
      for (int c = 0; c < QKC; ++c) qa[c] = q[kF8 ? QKC * quarter + c : 4 * c + quarter];
    }
  };

  float m_run[G];
  float acc[G][EPL];
  // matrix P.V: acc8[e] holds head 4 quarter + j (rows past G are padding), value
  // column col * 8 + e
  floatx4 acc8[8];
  float l_lane[4];
  auto reset = [&]() {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m_run[h] = kNegInf;
      if constexpr (!kMfmaPV) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
      }
    }
    if constexpr (kMfmaPV) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc8[e] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) l_lane[j] = 0.f;
    seg_bad = 0;
  };

  // Scores, probabilities and P.V for the current tile.  The probabilities are
  // taken relative to a reference m_run per head that is raised only when a
  // tile's maximum exceeds it by more than 2^kRebase (then the accumulators are
  // rescaled); in between they stay below 2^kRebase.  Any reference gives the same
  // normalised result; this one keeps the rescaling off almost every tile.
  auto compute = [&](const uint4* kb, const uint4* vb, bool bad) {
    constexpr float kRebase = 8.f;
    const int tok0 = cc.t * TOK;
    const int ntok = min(TOK, cctx - tok0);
    const bool full = ntok == TOK;
    seg_bad |= bad;
    // key operand: this lane's column is token kr of the tile (columns past TOK
    // repeat rows; they are masked out below)
    const int kr = col & (TOK - 1);
    uint4 kk[QKC];
    if constexpr (kF8) {
      // 16 codes per chunk -> two bfloat16 operands (exact)
#pragma unroll
      for (int j = 0; j < KCH; ++j) {
        const uint4 c8 = kb[kr * St::kSlots + ((wave * NCH + KCH * quarter + j) ^ St::swz(kr))];
        const uint2 b0 = e4m3x4_to_bf16(c8.x), b1 = e4m3x4_to_bf16(c8.y);
        const uint2 b2 = e4m3x4_to_bf16(c8.z), b3 = e4m3x4_to_bf16(c8.w);
        kk[2 * j] = make_uint4(b0.x, b0.y, b1.x, b1.y);
        kk[2 * j + 1] = make_uint4(b2.x, b2.y, b3.x, b3.y);
      }
    } else {
#pragma unroll
      for (int c = 0; c < QKC; ++c)
        kk[c] = kb[kr * St::kSlots + ((wave * NCH + 4 * c + quarter) ^ St::swz(kr))];
    }
    floatx4 s4;
    if constexpr (kValuQK) {
      // lane (quarter, col): its chunks of token col's key against each head's query,
      // then the four quarters' sums added (every quarter ends with the same value);
      // element j holds head j % G, as the matrix instruction's rows would
      float sh[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        uint4 qc[QKC];   // head h's chunks of the lane's dims (the key chunks it holds)
#pragma unroll
        for (int c = 0; c < QKC; ++c)
          qc[c] = q_lds[wave][h * (D * QEB / 16) + (kF8 ? QKC * quarter + c : 4 * c + quarter)];
        sh[h] = sum_xor32(sum_xor16(lane_dot<QT, QKC>(qc, kk)));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) s4[j] = sh[j % G];
    } else {
      s4 = tile_scores<QT, QKC>(qa, kk);
    }
    float sc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sc[j] = s4[j] * a.scale_log2;
    if (TOK < 16 || !full) {
      // columns past the context (and past TOK) take no weight: a branch taken on a
      // sequence's last tile only
      keep_branch();
      const bool live = col < ntok;
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[j] = live ? sc[j] : kNegInf;
    }
    // the tile's maximum key of head h, read from lane hlane(h) of gkey[hreg(h)]
    int gkey[4];
    if constexpr (kValuQK || !kF8) {
      // one 16-lane reduction per register: head j (kValuQK: every quarter holds the same
      // scores), else head 4 r + j in quarter r of sc[j]
#pragma unroll
      for (int j = 0; j < (kValuQK ? G : 4); ++j) gkey[j] = row_max_key<TOK>(float_key(sc[j]));
    } else {
      // E4M3 caches: head 4 r + j sits in quarter r of sc[j].  Two half-wave swaps and
      // one row swap transpose the 16-lane rows against the four registers, putting head
      // 4 r + q in quarter q of one register, so that one 16-lane reduction serves four
      // heads (fewer vector instructions; on bf16 caches the one longer dependent chain
      // made the kernel 1.5 us slower, so they keep four reductions)
      const auto a02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(sc[0]),
                                                        __float_as_uint(sc[2]), false, false);
      const auto a13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(sc[1]),
                                                        __float_as_uint(sc[3]), false, false);
      const auto t = __builtin_amdgcn_permlane16_swap(a02[0], a13[0], false, false);
      gkey[0] = row_max_key<TOK>(float_key(__uint_as_float(t[0])));
      if constexpr (kQuarters > 1) gkey[1] = row_max_key<TOK>(float_key(__uint_as_float(t[1])));
    }
    auto hreg = [](int h) { return kValuQK ? h : !kF8 ? (h & 3) : h >> 2; };
    auto hlane = [](int h) { return kValuQK ? 0 : !kF8 ? 16 * (h >> 2) : 16 * (h & 3); };
    float alpha[G];
    bool rebase = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float gm = key_float(__builtin_amdgcn_readlane(gkey[hreg(h)], hlane(h)));
      const bool up = gm > m_run[h] + kRebase;   // uniform across the wave
      const float mn = up ? gm : m_run[h];
      alpha[h] = up ? fast_exp2(m_run[h] - mn) : 1.f;
      rebase |= up;
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
      l_lane[j] = fmaf(l_lane[j], arow, sc[j]);   // arow is 1 unless the row rebased
    }
    if (rebase) {
      if constexpr (kMfmaPV) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float aj = (G > 4 && quarter == 1) ? alpha[(4 + j) % G] : alpha[j % G];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc8[e][j] *= aj;
        }
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha[h];
      }
    }
    if (quarter < kQuarters) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * quarter + j < G) {
          if constexpr (kMfmaPV)
            p_lds[wave][(4 * quarter + j) % G][col] = sc[j];
          else
            p_lds[wave][col][(4 * quarter + j) % G] = sc[j];
        }
    }
    __builtin_amdgcn_wave_barrier();
    if constexpr (kMfmaPV) {
      // P.V on bf16 matrix instructions.  A: P with the wave's heads as rows (row col,
      // real for col < G) and tokens 4 quarter .. 4 quarter + 3 as k; B: the same
      // tokens' value columns col * 8 + e for output block e, packed from four token
      // rows (a column permutation, undone at the store).  P is split into hi + lo
      // bf16 terms, together exact to about 2^-17 of p; E4M3 values are exact in bf16.
      // rows col >= G read head col % G's probabilities: finite values whose products
      // land in padding rows of the accumulators, which are never stored
      const floatx4 pa = *reinterpret_cast<const floatx4*>(&p_lds[wave][col % G][4 * quarter]);
      const floatx2 p01 = {pa[0], pa[1]}, p23 = {pa[2], pa[3]};
      const bf16x2 h01 = __builtin_convertvector(p01, bf16x2);
      const bf16x2 h23 = __builtin_convertvector(p23, bf16x2);
      // lo = p - hi as one bf16 dot product per value, (hi0, hi1) . (-1, 0) + p0 and
      // (hi0, hi1) . (0, -1) + p1: the products and the difference are exact in fp32.
      // The pair (-1, 0) is the word 0x0000bf80; it is set in a scalar register because
      // the compiler would encode it as the inline constant -1.0, i.e. 0xbf800000.
      uint32_t kneg0;
      asm("s_mov_b32 %0, 0xbf80" : "=s"(kneg0));
      const bf16x2 neg0 = __builtin_bit_cast(bf16x2, kneg0);
      const bf16x2 neg1 = __builtin_bit_cast(bf16x2, 0xbf800000u);
      const floatx2 r01 = {__builtin_amdgcn_fdot2_f32_bf16(h01, neg0, pa[0], false),
                           __builtin_amdgcn_fdot2_f32_bf16(h01, neg1, pa[1], false)};
      const floatx2 r23 = {__builtin_amdgcn_fdot2_f32_bf16(h23, neg0, pa[2], false),
                           __builtin_amdgcn_fdot2_f32_bf16(h23, neg1, pa[3], false)};
      const bf16x2 l01 = __builtin_convertvector(r01, bf16x2);
      const bf16x2 l23 = __builtin_convertvector(r23, bf16x2);
      const bf16x4 ahi = __builtin_bit_cast(
          bf16x4, make_uint2(__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)));
      const bf16x4 alo = __builtin_bit_cast(
          bf16x4, make_uint2(__builtin_bit_cast(uint32_t, l01), __builtin_bit_cast(uint32_t, l23)));
      if constexpr (kF8) {
        // E4M3 caches, whose kernel runs four waves per SIMD, keep two k = 16 products,
        // which need fewer registers.  cw[s]: the codes of token 4 quarter + s, value
        // columns col * 8 .. col * 8 + 7 (4 per word)
        uint32_t cw[4][2];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int n = 4 * quarter + s;
          const int slot = (wave * NCH + (col >> 1)) ^ St::swz(n);
          const uint2 c8 = reinterpret_cast<const uint2*>(vb)[2 * (n * St::kSlots + slot) + (col & 1)];
          cw[s][0] = c8.x;
          cw[s][1] = c8.y;
        }
        if (!full) {
          // rows past the context may hold NaN codes: zero them (a sequence's last tile)
          keep_branch();
#pragma unroll
          for (int s = 0; s < 4; ++s)
            if (4 * quarter + s >= ntok) cw[s][0] = cw[s][1] = 0u;
        }
        // column pair k (columns 2k, 2k + 1): one byte permute per token pair puts the
        // pair's codes side by side (t0 2k, t1 2k, t0 2k+1, t1 2k+1); each half of that
        // word converts to one column's bf16 pair of those tokens
        uint32_t xw[4][2];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t sel = (k & 1) ? 0x07030602u : 0x05010400u;
          xw[k][0] = __builtin_amdgcn_perm(cw[1][k >> 1], cw[0][k >> 1], sel);
          xw[k][1] = __builtin_amdgcn_perm(cw[3][k >> 1], cw[2][k >> 1], sel);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t x01 = xw[e >> 1][0], x23 = xw[e >> 1][1];
          const bf16x2 c01 = (e & 1) ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x01, 1.f, true)
                                     : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x01, 1.f, false);
          const bf16x2 c23 = (e & 1) ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x23, 1.f, true)
                                     : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x23, 1.f, false);
          const bf16x4 b = {c01[0], c01[1], c23[0], c23[1]};
          acc8[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahi, b, acc8[e], 0, 0, 0);
          acc8[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(alo, b, acc8[e], 0, 0, 0);
        }
      } else {
        // bf16 caches: one k = 32 operand, the lane's four hi terms then its four lo
        // terms, against its four value rows twice (the order of k is free)
        const bf16x8 ahl = {h01[0], h01[1], h23[0], h23[1], l01[0], l01[1], l23[0], l23[1]};
        uint32_t wv[4][4];   // token 4 quarter + s: value columns col * 8 .. col * 8 + 7
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int n = 4 * quarter + s;
          const uint4 c = vb[n * St::kSlots + ((wave * NCH + col) ^ St::swz(n))];
          wv[s][0] = c.x; wv[s][1] = c.y; wv[s][2] = c.z; wv[s][3] = c.w;
        }
        if (!full) {
          // rows past the context may hold NaN: zero them (a sequence's last tile only)
          keep_branch();
#pragma unroll
          for (int s = 0; s < 4; ++s)
            if (4 * quarter + s >= ntok) wv[s][0] = wv[s][1] = wv[s][2] = wv[s][3] = 0u;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // column col * 8 + e: the low bf16 of word e / 2 for even e, else the high
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          const uint32_t bx = __builtin_amdgcn_perm(wv[1][e >> 1], wv[0][e >> 1], sel);
          const uint32_t by = __builtin_amdgcn_perm(wv[3][e >> 1], wv[2][e >> 1], sel);
          const bf16x8 b = __builtin_bit_cast(bf16x8, make_uint4(bx, by, bx, by));
          acc8[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahl, b, acc8[e], 0, 0, 0);
        }
      }
      __builtin_amdgcn_wave_barrier();
      return;
    }
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      const int n = s * RPS + rg;
      float pv[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pv[h] = p_lds[wave][n][h];
      float v[EPL];
      if constexpr (kF8) {
        const int slot = (wave * NCH + (li >> 1)) ^ St::swz(n);
        const uint2 c8 = reinterpret_cast<const uint2*>(vb)[2 * (n * St::kSlots + slot) + (li & 1)];
        e4m3x4_to_f32(c8.x, v);
        e4m3x4_to_f32(c8.y, v + 4);
      } else {
        unpack_chunk<T>(vb[n * St::kSlots + ((wave * NCH + li) ^ St::swz(n))], v);
      }
      if (!full && n >= ntok) {
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

  // The record of head h of this wave's group for the current segment: label
  // w + sequence in the balanced split, the fixed plan's layout with fixed partitions.
  auto rec_of = [&](int h) -> int64_t {
    if constexpr (FIXED)
      return ((int64_t)cc.s * H + g * G + h) * a.max_parts + fx_p;
    else
      return ((int64_t)w + cc.s) * H + g * G + h;
  };

  // End of a segment: fold the row groups, normalise, store (the output itself for
  // a whole sequence, else the segment's record), 16 bytes at a time.
  auto finish = [&](bool whole) {
    if constexpr (kMfmaPV) {
#pragma unroll
      for (int j = 0; j < 4; ++j) l_lane[j] = row16_sum(l_lane[j]);
      float l_head[G];
#pragma unroll
      for (int h = 0; h < G; ++h) l_head[h] = readlane(l_lane[h & 3], 16 * (h >> 2));
      if (quarter >= kQuarters) return;   // padding rows
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int h = 4 * quarter + j;
        if (h >= G) continue;
        const float lh = (G > 4 && quarter == 1) ? l_head[(4 + j) % G] : l_head[j % G];
        const float mh = (G > 4 && quarter == 1) ? m_run[(4 + j) % G] : m_run[j % G];
        const float inv = (kF8 ? a.v_scale : 1.f) / lh;
        float res[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) res[e] = seg_bad ? __builtin_nanf("") : acc8[e][j] * inv;
        if (whole) {
          const int64_t orow = ((int64_t)cc.s * H + g * G + h) * D + col * 8;
          if (a.out_bf16) {
            const u32x4 v = {
                f32_to_bf16_rne(res[0]) | (uint32_t)f32_to_bf16_rne(res[1]) << 16,
                f32_to_bf16_rne(res[2]) | (uint32_t)f32_to_bf16_rne(res[3]) << 16,
                f32_to_bf16_rne(res[4]) | (uint32_t)f32_to_bf16_rne(res[5]) << 16,
                f32_to_bf16_rne(res[6]) | (uint32_t)f32_to_bf16_rne(res[7]) << 16};
            st_seg<kNtSeg>(reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.out) + orow), v);
          } else {
            float* o = static_cast<float*>(a.out) + orow;
            st_seg4<kNtSeg>(o, res[0], res[1], res[2], res[3]);
            st_seg4<kNtSeg>(o + 4, res[4], res[5], res[6], res[7]);
          }
        } else {
          const int64_t rec = rec_of(h);
          float* o = a.ws_o + rec * D + col * 8;
          st_seg4<kNtSeg>(o, res[0], res[1], res[2], res[3]);
          st_seg4<kNtSeg>(o + 4, res[4], res[5], res[6], res[7]);
          if (col == 0) {
            a.ws_m[rec] = mh;
            a.ws_l[rec] = lh;
          }
        }
      }
      return;
    }
#pragma unroll
    for (int off = NPC; off < kWave; off <<= 1)
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] += __shfl_xor(acc[h][e], off);
#pragma unroll
    for (int j = 0; j < 4; ++j) l_lane[j] = row16_sum(l_lane[j]);
    float l_head[G];
#pragma unroll
    for (int h = 0; h < G; ++h) l_head[h] = readlane(l_lane[h & 3], 16 * (h >> 2));
    if (lane >= NPC) return;
    float res[G][EPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float inv = (kF8 ? a.v_scale : 1.f) / l_head[h];
#pragma unroll
      for (int e = 0; e < EPL; ++e) res[h][e] = seg_bad ? __builtin_nanf("") : acc[h][e] * inv;
    }
    if (whole) {
      const int64_t row0 = (int64_t)cc.s * H + g * G;
      if (a.out_bf16) {
        uint16_t* o = static_cast<uint16_t*>(a.out) + row0 * D + li * EPL;
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < EPL; e += 4) {
            const u32x2 v = {
                f32_to_bf16_rne(res[h][e]) | (uint32_t)f32_to_bf16_rne(res[h][e + 1]) << 16,
                f32_to_bf16_rne(res[h][e + 2]) | (uint32_t)f32_to_bf16_rne(res[h][e + 3]) << 16};
            st_seg<kNtSeg>(reinterpret_cast<u32x2*>(o + h * D + e), v);
          }
      } else {
        float* o = static_cast<float*>(a.out) + row0 * D + li * EPL;
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < EPL; e += 4)
            st_seg4<kNtSeg>(o + h * D + e, res[h][e], res[h][e + 1], res[h][e + 2],
                            res[h][e + 3]);
      }
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float* o = a.ws_o + rec_of(h) * D + li * EPL;
#pragma unroll
        for (int e = 0; e < EPL; e += 4)
          st_seg4<kNtSeg>(o + e, res[h][e], res[h][e + 1], res[h][e + 2], res[h][e + 3]);
      }
      if (lane < G) {
        // lane h < G writes head h's (m, l); m_run and l_head are uniform
        float mh = m_run[0], lh = l_head[0];
#pragma unroll
        for (int h = 1; h < G; ++h) {
          mh = lane == h ? m_run[h] : mh;
          lh = lane == h ? l_head[h] : lh;
        }
        a.ws_m[rec_of(lane)] = mh;
        a.ws_l[rec_of(lane)] = lh;
      }
    }
  };

  reset();
  load_query(cc.s);

  // One step of the ring: issue the copies of the tile NBUF - 1 ahead into the
  // buffer freed at the end of the previous step, wait for this wave's copies of
  // tile j and its query loads (the later tiles stay in flight), barrier (every
  // wave's copies of tile j have landed), compute tile j, barrier (every wave is
  // done reading its buffer), close the segment where it ends.  The copies and the
  // query loads are invisible to the compiler, so these are the only waits.
#define PKV_STREAM_STEP(KB, VB, KF, VF)                                   \
  if (cc.t >= cc.stop) break;                                             \
  issue(KF, VF);                                                          \
  if (NBUF > 2 && q_fresh) {                                              \
    /* a new query's copy is newer than the previous steps' copies */     \
    wait_copies<L>();                                                     \
  } else {                                                                \
    wait_copies<(NBUF - 1) * L>();                                        \
  }                                                                       \
  bare_barrier();                                                         \
  if (q_fresh) {                                                          \
    read_query();                                                         \
    q_fresh = false;                                                      \
  }                                                                       \
  compute(KB, VB, (bad_pipe >> (NBUF - 1)) & 1u);                         \
  bare_barrier();                                                         \
  if (cc.t == cc.stop - 1) {                                              \
    /* the share's part of this sequence ends with this tile */           \
    finish(seg_from_zero && cc.stop == cc.nt);                            \
    reset();                                                              \
    next_seq(cc);                                                         \
    seg_from_zero = true;                                                 \
    if (cc.t < cc.stop) {                                                 \
      cctx = ctx_of[cc.s];                                                \
      load_query(cc.s);                                                   \
    }                                                                     \
  } else {                                                                \
    ++cc.t;                                                               \
  }

  if constexpr (NBUF == 2) {
    issue(kb0, vb0);
    for (;;) {
      PKV_STREAM_STEP(kb0, vb0, kb1, vb1)
      PKV_STREAM_STEP(kb1, vb1, kb0, vb0)
    }
  } else if constexpr (NBUF == 3) {
    issue(kb0, vb0);
    issue(kb1, vb1);
    for (;;) {
      PKV_STREAM_STEP(kb0, vb0, kb2, vb2)
      PKV_STREAM_STEP(kb1, vb1, kb0, vb0)
      PKV_STREAM_STEP(kb2, vb2, kb1, vb1)
    }
  } else {
    issue(kb0, vb0);
    issue(kb1, vb1);
    issue(kb2, vb2);
    for (;;) {
      PKV_STREAM_STEP(kb0, vb0, kb3, vb3)
      PKV_STREAM_STEP(kb1, vb1, kb0, vb0)
      PKV_STREAM_STEP(kb2, vb2, kb1, vb1)
      PKV_STREAM_STEP(kb3, vb3, kb2, vb2)
    }
  }
#undef PKV_STREAM_STEP
  // the ring's last copies (of block 0) land before the wave ends
  wait_copies<0>();
}


// ---- tile plan ---------------------------------------------------------------------

__global__ __launch_bounds__(kPlanThreads) void tile_plan_kernel(AttentionArgs a) {
  build_tile_plan<kPlanThreads>(a.context_lens, a.num_seqs, a.max_blocks_per_seq << a.block_shift,
                                a.tile_cum, a.tile_hdr);
}

size_t tile_plan_bytes(int64_t num_seqs) {
  return 256 + ((size_t)(num_seqs + 1) * sizeof(int) + 255) / 256 * 256;
}

hipError_t launch_tile_plan(const AttentionArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(tile_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a);
  return hipGetLastError();
}

// ---- merge of the segments ------------------------------------------------------------
// One wave per (sequence, query head) row.  Sequences without tiles (an invalid
// context length: the plan gives them no positions) get NaN rows; a sequence inside one share was written by the
// partition stage; otherwise its records, labels w + sequence for the non-empty
// shares w it spans, are merged in share order.  Lane groups take every KGW-th record, U at a
// time; the groups are combined in a fixed order, so the result does not depend on
// timing.
template <int D>
__global__ __launch_bounds__(256) void paged_attention_stream_reduce_kernel(AttentionArgs a) {
  constexpr int LPR = D / 4;             // lanes per record (float4 each)
  constexpr int KGW = kWave / LPR;       // records per wave round
  constexpr int U = 4;                   // rounds in flight
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (row >= (int64_t)a.num_seqs * a.num_heads) return;
  const int H = a.num_heads;
  const int seq = (int)(row / H);
  const int qh = (int)(row % H);
  const int kg = lane / LPR;
  const int lr = lane % LPR;
  // One round of independent loads: the plan says which sequences have tiles (a
  // valid context length) and where they sit.
  const int c0 = a.tile_cum[seq];
  const int c1 = a.tile_cum[seq + 1];
  const int total = a.tile_hdr[0];
  const int nwg = a.tile_hdr[1];
  if (c1 == c0) {
    if (kg == 0) {
      const float nan = __builtin_nanf("");
      store_row4(a, row * D + lr * 4, Running{0.f, 1.f, make_float4(nan, nan, nan, nan)});
    }
    return;
  }
  // shares holding the sequence's first and last real tiles
  const int w0 = share_of((int64_t)c0 + kSeqCost, nwg, total);
  const int w1 = share_of((int64_t)c1 - 1, nwg, total);
  if (w0 == w1) return;
  Running r{-__builtin_inff(), 0.f, make_float4(0.f, 0.f, 0.f, 0.f)};
  for (int w = w0 + kg; w <= w1; w += KGW * U) {
    float m[U], l[U];
    float4 o[U];
    bool live[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ww = w + u * KGW;
      live[u] = ww <= w1 && share_nonempty(ww, nwg, total);   // empty shares wrote nothing
      const int64_t rec = ((int64_t)ww + seq) * H + qh;
      m[u] = live[u] ? a.ws_m[rec] : 0.f;
      l[u] = live[u] ? a.ws_l[rec] : 0.f;
      o[u] = live[u] ? reinterpret_cast<const float4*>(a.ws_o + rec * D)[lr]
                     : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    accumulate(r, m, l, o, live);
  }
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

hipError_t launch_attention_stream_reduce(const AttentionArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.num_heads * a.num_seqs;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (a.head_dim == 64)
    hipLaunchKernelGGL(paged_attention_stream_reduce_kernel<64>, grid, dim3(256), 0, stream, a);
  else if (a.head_dim == 128)
    hipLaunchKernelGGL(paged_attention_stream_reduce_kernel<128>, grid, dim3(256), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---- dispatch ------------------------------------------------------------------

template <typename T, int D, int G, int HW, bool FIXED>
static hipError_t launch_stream_shape(const AttentionArgs& a, hipStream_t stream) {
  auto kernel = paged_attention_stream_kernel<T, D, G, HW, stream_nbuf<T>(), FIXED>;
  const int hgroups = a.num_kv_heads / HW;
  if constexpr (FIXED) {
    // one workgroup per possible plan item; those past the plan's count exit at once
    const int64_t items = (int64_t)a.num_seqs * a.max_parts;
    hipLaunchKernelGGL(kernel, dim3((unsigned)items, hgroups), dim3(HW * kWave), 0, stream, a);
    return hipGetLastError();
  }
  // Workgroups one compute unit holds at once, from the kernel's own resource use.
  static const int per_cu = [&] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, HW * kWave, 0) != hipSuccess)
      n = 1;
    return n > 0 ? n : 1;
  }();
  const int cus = device_cus();
  if (cus <= 0) return hipErrorInvalidDevice;
  const int nwg = max(1, min(kMaxStreamWgs, per_cu * cus / hgroups));
  hipLaunchKernelGGL(kernel, dim3(nwg, hgroups), dim3(HW * kWave), 0, stream, a);
  return hipGetLastError();
}

#ifndef PKV_STREAM_MAX_ROW
#define PKV_STREAM_MAX_ROW 2048
#endif

// Heads per workgroup: the largest of 8, 4, 2, 1 that divides the kv heads and keeps
// a token row of the group within PKV_STREAM_MAX_ROW bytes (and at 128 bytes or
// more: 64-element E4M3 heads pair up).
template <typename T, int D, int G, bool FIXED>
static hipError_t launch_stream_hw(const AttentionArgs& a, hipStream_t stream) {
  constexpr int kRow = D * T::kElemBytes;
  if constexpr (8 * kRow <= PKV_STREAM_MAX_ROW)
    if (a.num_kv_heads % 8 == 0) return launch_stream_shape<T, D, G, 8, FIXED>(a, stream);
  if constexpr (4 * kRow <= PKV_STREAM_MAX_ROW)
    if (a.num_kv_heads % 4 == 0) return launch_stream_shape<T, D, G, 4, FIXED>(a, stream);
  // a tile row spans at least 128 bytes
  if (a.num_kv_heads % 2 == 0) return launch_stream_shape<T, D, G, 2, FIXED>(a, stream);
  if constexpr (kRow >= 128)
    return launch_stream_shape<T, D, G, 1, FIXED>(a, stream);
  else
    return hipErrorInvalidValue;
}

template <typename T, int D, bool FIXED = false>
static hipError_t launch_stream_g(const AttentionArgs& a, hipStream_t stream) {
  switch (a.num_heads / a.num_kv_heads) {
    case 1: return launch_stream_hw<T, D, 1, FIXED>(a, stream);
    case 2: return launch_stream_hw<T, D, 2, FIXED>(a, stream);
    case 4: return launch_stream_hw<T, D, 4, FIXED>(a, stream);
    case 8: return launch_stream_hw<T, D, 8, FIXED>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attention_stream(const AttentionArgs& a, hipStream_t stream) {
  if (a.kv_fp8) {
    if (a.head_dim == 64) return launch_stream_g<FP8, 64>(a, stream);
    if (a.head_dim == 128) return launch_stream_g<FP8, 128>(a, stream);
  } else if (a.kv_bf16) {
    if (a.head_dim == 64) return launch_stream_g<BF16, 64>(a, stream);
    if (a.head_dim == 128) return launch_stream_g<BF16, 128>(a, stream);
  } else {
    if (a.head_dim == 64) return launch_stream_g<F32, 64>(a, stream);
    if (a.head_dim == 128) return launch_stream_g<F32, 128>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attention_stream_fixed(const AttentionArgs& a, hipStream_t stream) {
  if (a.kv_bf16) {
    if (a.head_dim == 64) return launch_stream_g<BF16, 64, true>(a, stream);
    if (a.head_dim == 128) return launch_stream_g<BF16, 128, true>(a, stream);
  } else if (!a.kv_fp8) {
    if (a.head_dim == 64) return launch_stream_g<F32, 64, true>(a, stream);
    if (a.head_dim == 128) return launch_stream_g<F32, 128, true>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
