// Paged attention for several new tokens per sequence, for gfx950 (CDNA4).
//
// The last n_b tokens of sequence b -- a prefill chunk ("vLLM 核心概念", section
// "Chunked Prefill"; "PagedAttention 实战", section "Chunked Prefill：长 prompt 不要一次吃
// 完全部预算") or the draft tokens of a speculative verify ("vLLM 核心概念", section
// "推测解码（Speculative Decoding）") -- have their K/V in the cache already and are
// the queries; query i, at position ctx_b - n_b + i, attends over cached positions
// 0 .. ctx_b - n_b + i.
//
//   chunk_attn_kernel   one workgroup per (sequence, KV head, 1-3 tiles of 16 query
//                       columns, key partition); a column is one (new token, query
//                       head of the KV head's group) pair, so a tile holds 16 / G
//                       tokens of G heads
//   chunk_wide_kernel   the same for launches with at least 128 columns per
//                       (sequence, KV head): one workgroup per 128 columns
//   chunk_merge_kernel  log-sum-exp merge of the key partitions ("PagedAttention
//                       实战", section "2026 年的新变化": sequence split)
//
// chunk_attn_kernel: the matrix-core mapping is the decode kernel's with the 16
// query heads of a KV head replaced by 16 columns: S^T = K.Q^T (16 tokens x 16
// columns) with v_mfma_f32_16x16x32, then out^T += V^T.P^T with
// v_mfma_f32_16x16x16, whose B operand is the S^T register layout.  Lane l owns
// column l % 16, so the causal mask, the online softmax and the rescale are
// lane-local.  The 4 waves split a partition's blocks (every 4th) and combine in
// LDS.  Every K/V tile a workgroup reads serves its 16-48 columns, which suits a
// few new tokens per sequence (speculative verify) but makes long chunks L2-bound.
// When its launch gives each workgroup slot only a few items, its workgroups take
// the sequences longest first (a counting sort over classes of context length),
// so the longest items do not start last.
//
// chunk_wide_kernel: each wave owns 32 columns (two groups of 16) and all four
// waves walk the same keys, two blocks (32 tokens) per stage, so a K/V tile
// read from L2 serves 128 columns.  Each stage goes through LDS (double
// buffered): K as stored, V interleaved as [token quad][dim][block][4 tokens].
// Both products use v_mfma_f32_16x16x32: S^T of the two blocks is computed per
// block, and out^T += V^T.P^T takes all 32 tokens at once, with lane l's eight
// P values (tokens 4g..4g+3 of each block, g = l / 16, from the two S^T tiles)
// as its B operand and the interleaved V rows as A.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "pa_device.h"
#include "pa_internal.h"

namespace {

using namespace pa_dev;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kCols = 16;                       // query columns per workgroup
constexpr float kLazyMax = 8.f;                 // log2 headroom before the reference max moves
constexpr int kMinPartTokens = 1024;            // key partitions: 1024 .. 4096 tokens
constexpr int kMaxPartTokens = 4096;

struct ChunkArgs {
  const uint16_t* q;            // [total][H][D]
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* q_starts;      // [B + 1], or NULL: sequence b's one query is row b
  const int32_t* block_tables;  // [B][max_blocks]
  const int32_t* ctx_lens;      // [B]
  uint16_t* out;                // [total][H][D]
  const float* k_scales;        // FP8 pools: per-KV-head scales of K and V, else unused
  const float* v_scales;
  float2* ws_ml;                // [total][H][P] (max in log2 units, sum), when P > 1
  float* ws_acc;                // [total][H][P][D] unnormalised output
  int32_t num_seqs, total, num_heads, num_kv_heads, group;
  int32_t max_blocks, max_ctx, num_blocks;
  int32_t col_tiles;            // column groups per (sequence, KV head) in the grid
  int32_t parts;                // key partitions per column group in the grid (P)
  int32_t part_blocks;          // blocks per key partition when P > 1
  int32_t ordered;              // narrow kernel: take the sequences longest first
  float scale_log2;             // scale * log2(e)
};

// Position of the work: every (sequence, KV head) group goes to XCD group % 8 (the
// XCDs take workgroup ids round-robin) and its items -- partition-major, then
// column tile -- run back to back there, so the tiles reading one partition's
// blocks share that XCD's L2.
struct ChunkItem {
  int32_t b, kvh, tile, part;
};
__device__ __forceinline__ bool chunk_item(const ChunkArgs& a, int32_t parts, ChunkItem* it) {
  const int32_t per_group = a.col_tiles * parts;
  const int32_t x = blockIdx.x & 7;
  const int32_t k = blockIdx.x >> 3;
  const int32_t gi = x + 8 * (k / per_group);
  if (gi >= a.num_seqs * a.num_kv_heads) return false;
  const int32_t r = k - (k / per_group) * per_group;
  it->part = r / a.col_tiles;
  it->tile = r - it->part * a.col_tiles;
  it->b = gi / a.num_kv_heads;
  it->kvh = gi - it->b * a.num_kv_heads;
  return true;
}

// Largest-first order of the sequences: a counting sort over 16 classes of context
// length (in steps of 1/16 of the longest), from the longest class down, ascending
// sequence index within a class.  Long items start first and short ones fill the
// tail; in the order the sequences come, a long one may start last and set the
// launch's length.  A length outside [1, max_ctx] is class 0 (its rows become NaN).
constexpr int kOrderClasses = 16;
constexpr int kOrderChunks = 4;          // context lengths kept in registers: 4 x 64
__device__ __forceinline__ int32_t order_class(int32_t ctx, int32_t max_ctx) {
  if (ctx < 1 || ctx > max_ctx) return 0;
  return static_cast<int32_t>(static_cast<int64_t>(ctx) * kOrderClasses /
                              (static_cast<int64_t>(max_ctx) + 1));
}
// Lane of the k-th (from 0) set bit of mask.
__device__ __forceinline__ int32_t kth_lane(uint64_t mask, int32_t k, int32_t lane) {
  const bool mine = ((mask >> lane) & 1) && __popcll(mask & ((1ull << lane) - 1)) == k;
  return __ffsll(static_cast<unsigned long long>(__ballot(mine))) - 1;
}
__device__ __forceinline__ void load_order_chunk(const ChunkArgs& a, int32_t c0, int32_t lane,
                                                 int32_t cl[kOrderChunks]) {
#pragma unroll
  for (int u = 0; u < kOrderChunks; ++u) {
    const int32_t i = c0 + 64 * u + lane;
    cl[u] = i < a.num_seqs ? order_class(a.ctx_lens[i], a.max_ctx) : -1;
  }
}
// Sequence of rank r (0 <= r < num_seqs) in that order; every lane gets it.
__device__ int32_t seq_of_rank(const ChunkArgs& a, int32_t r, int32_t lane) {
  constexpr int32_t kGroup = 64 * kOrderChunks;
  int32_t cl0[kOrderChunks];             // the first group, kept for the second pass
  int32_t cnt = 0;                       // lane c: sequences of class c
  for (int32_t c0 = 0; c0 < a.num_seqs; c0 += kGroup) {
    int32_t cl[kOrderChunks];
    load_order_chunk(a, c0, lane, cl);
    if (c0 == 0) {
#pragma unroll
      for (int u = 0; u < kOrderChunks; ++u) cl0[u] = cl[u];
    }
#pragma unroll
    for (int u = 0; u < kOrderChunks; ++u) {
      if (c0 + 64 * u >= a.num_seqs) break;     // no sequence in this or later chunks
#pragma unroll 1
      for (int32_t c = 0; c < kOrderClasses; ++c) {
        const int32_t nc = __popcll(__ballot(cl[u] == c));
        cnt += lane == c ? nc : 0;
      }
    }
  }
  int32_t cls = 0, k = r;
  for (int32_t c = kOrderClasses - 1; c >= 0; --c) {
    const int32_t cc = __builtin_amdgcn_readlane(cnt, c);
    if (k < cc) {
      cls = c;
      break;
    }
    k -= cc;
  }
  for (int32_t c0 = 0; c0 < a.num_seqs; c0 += kGroup) {
    int32_t cl[kOrderChunks];
    if (c0 == 0) {
#pragma unroll
      for (int u = 0; u < kOrderChunks; ++u) cl[u] = cl0[u];
    } else {
      load_order_chunk(a, c0, lane, cl);
    }
#pragma unroll
    for (int u = 0; u < kOrderChunks; ++u) {
      const uint64_t m = __ballot(cl[u] == cls);
      const int32_t pc = __popcll(m);
      if (k < pc) return c0 + 64 * u + kth_lane(m, k, lane);
      k -= pc;
    }
  }
  return -1;    // not reached: the classes count every sequence
}
// chunk_item with the groups taken in largest-first order of their sequences: group
// rank g = (sequence rank) * Hkv + KV head, placed on XCD g % 8 as above.  The
// order costs every workgroup two passes over the lengths, so the launch asks for
// it (a.ordered) only when the slots get few items each; many items per slot
// balance by themselves.
__device__ __forceinline__ bool chunk_item_ordered(const ChunkArgs& a, int32_t lane,
                                                   ChunkItem* it) {
  if (!a.ordered) return chunk_item(a, a.parts, it);
  const int32_t per_group = a.col_tiles * a.parts;
  const int32_t x = blockIdx.x & 7;
  const int32_t k = blockIdx.x >> 3;
  const int32_t g = x + 8 * (k / per_group);
  if (g >= a.num_seqs * a.num_kv_heads) return false;
  const int32_t r = k - (k / per_group) * per_group;
  it->part = r / a.col_tiles;
  it->tile = r - it->part * a.col_tiles;
  const int32_t srank = g / a.num_kv_heads;
  it->kvh = g - srank * a.num_kv_heads;
  it->b = seq_of_rank(a, srank, lane);
  return it->b >= 0;
}

// The sequence's rows and the tile's columns.  Returns false when nothing may be
// written (rows outside [0, total]) or the tile holds no column.
struct ChunkSeq {
  int32_t qs, n, ctx, cols, pmax;
  bool bad;   // context length outside [1, max_ctx], or more new tokens than cached ones
};
template <int kTileCols = kCols>
__device__ __forceinline__ bool chunk_seq(const ChunkArgs& a, const ChunkItem& it, ChunkSeq* s) {
  // no q_starts: one query per sequence, row b (decode with wide query groups)
  const int32_t qs = a.q_starts ? a.q_starts[it.b] : it.b;
  const int32_t qe = a.q_starts ? a.q_starts[it.b + 1] : it.b + 1;
  if (qs < 0 || qe < qs || qe > a.total) return false;
  s->qs = qs;
  s->n = qe - qs;
  s->ctx = a.ctx_lens[it.b];
  s->cols = s->n * a.group;
  if (it.tile * kTileCols >= s->cols) return false;
  s->bad = s->ctx < 1 || s->ctx > a.max_ctx || s->n > s->ctx;
  const int32_t last_col = min(it.tile * kTileCols + kTileCols - 1, s->cols - 1);
  s->pmax = s->ctx - s->n + last_col / a.group;   // furthest position a tile column sees
  return true;
}

// NT column tiles of 16 per workgroup (NT * 16 columns): every K/V tile a wave
// loads serves all of them, so a launch with up to 48 columns per (sequence, KV
// head) reads each tile once.  Three tiles at head dim 128 keep their q fragments
// in LDS (the registers hold the accumulators and two blocks of K/V).  kStream:
// each tile is read by one workgroup only, so the loads are non-temporal.
template <class E, int D, int NT, bool kStream, bool kFp8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(NT * D > 192 ? 2 : 3)))
void chunk_attn_kernel(ChunkArgs a) {
  constexpr int KK = D / 32;
  constexpr int LW = kFp8 ? KK / 2 : KK;   // 16-byte loads per lane per tile (FP8: half)
  constexpr int64_t kTileBytes = static_cast<int64_t>(kBlock) * D * (kFp8 ? 1 : 2);
  constexpr int MT = D / 16;
  constexpr int kLdsStride = D + 4;
  constexpr bool kQLds = NT * D > 256;
  __shared__ u32x4 s_q[kQLds ? NT * KK * 64 : 1];
  __shared__ float s_m[NT][kWaves][kCols];
  __shared__ float s_l[NT][kWaves][kCols];
  __shared__ __attribute__((aligned(16))) float s_acc[kWaves][kCols * kLdsStride];
  __shared__ int s_bad;

  ChunkItem it;
  if (!chunk_item_ordered(a, threadIdx.x & 63, &it)) return;
  ChunkSeq sq;
  if (!chunk_seq<NT * kCols>(a, it, &sq)) return;
  const int32_t b = __builtin_amdgcn_readfirstlane(it.b);
  const int32_t kvh = __builtin_amdgcn_readfirstlane(it.kvh);
  const int32_t part = __builtin_amdgcn_readfirstlane(it.part);
  const int32_t col0 = __builtin_amdgcn_readfirstlane(it.tile) * (NT * kCols);
  const int32_t ctx = __builtin_amdgcn_readfirstlane(sq.ctx);
  const int32_t pmax = __builtin_amdgcn_readfirstlane(sq.pmax);
  const int32_t G = a.group;
  const int32_t H = a.num_heads;

  const int32_t tid = threadIdx.x;
  const int32_t w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t lane = tid & 63;
  const int32_t n = lane & 15;       // column of this lane within each 16-column tile
  const int32_t g4 = lane >> 4;      // token quad within a block

  // Blocks the workgroup reads: 0 .. pmax / 16, in partitions of part_blocks -- or
  // all in one, with the outputs written directly, when the launch has a single
  // partition or the sequence's whole context fits one.
  const bool direct = a.parts == 1 || (!sq.bad && ctx <= a.part_blocks * kBlock);
  const int32_t nblk_t = sq.bad ? 1 : pmax / kBlock + 1;
  const int32_t pblocks = direct ? nblk_t : a.part_blocks;
  if (part * pblocks >= nblk_t) return;

  if (sq.bad) {
    // NaN in every row of the columns (once: partition 0 writes it, the merge keeps it)
    for (int32_t i = tid; i < NT * kCols * D; i += kThreads) {
      const int32_t c = col0 + i / D;
      if (c < sq.cols) {
        const int64_t row = static_cast<int64_t>(sq.qs + c / G) * H + kvh * G + c % G;
        a.out[row * D + i % D] = E::kNaN;
      }
    }
    return;
  }

  // The wave's blocks: first, first + 4, ... below jend.  The ids of the first run
  // of 64 are requested before the q fragments (whose LDS store ends in a barrier).
  const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_blocks;
  const int32_t jbeg = part * pblocks;
  const int32_t jend = min(nblk_t, jbeg + pblocks);
  const int32_t first = jbeg + w;
  const int32_t nw = first < jend ? (jend - first + kWaves - 1) / kWaves : 0;
  int32_t ids0 = 0;
  if (lane < min(64, nw)) ids0 = bt[first + kWaves * lane];

  // FP8 pools: the K scale folds into the score scale, the V scale into the output.
  // The running max is taken on raw scores and then scaled, which needs a scale
  // > 0: the sign of a negative one is moved into q (its sign bits flipped).
  const float scale_signed = kFp8 ? a.scale_log2 * a.k_scales[kvh] : a.scale_log2;
  const uint32_t q_flip = scale_signed < 0.f ? 0x80008000u : 0u;
  // A zero scale would turn a masked score (-inf) into NaN: 1e-30 leaves every
  // exponent rounding to the same value and a masked one at -inf.
  const float score_scale = fmaxf(fabsf(scale_signed), 1e-30f);
  const float out_scale = kFp8 ? a.v_scales[kvh] : 1.f;
  // keys up to the workgroup's first column's position are seen by every column
  const int32_t pmin = ctx - sq.n + col0 / G;

  // This lane's column in tile t: token ti of the chunk, head gh of the group,
  // position pos[t].  Padding columns load zero q and mask nothing.
  int32_t pos[NT];
  u32x4 qf[kQLds ? 1 : NT][KK];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int32_t col = col0 + t * kCols + n;
    const bool col_ok = col < sq.cols;
    const int32_t ti = col_ok ? col / G : 0;
    const int32_t gh = col_ok ? col - ti * G : 0;
    pos[t] = col_ok ? ctx - sq.n + ti : pmax;
    const int64_t q_row = (static_cast<int64_t>(sq.qs + ti) * H + kvh * G + gh) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if constexpr (kQLds) {
        // wave w stores the fragments (t, kk) with (t * KK + kk) % 4 == w
        if ((t * KK + kk) % kWaves == w)
          s_q[(t * KK + kk) * 64 + lane] =
              col_ok ? load16(a.q + q_row + 32 * kk + 8 * g4) ^ q_flip : u32x4{0, 0, 0, 0};
      } else {
        qf[t][kk] = col_ok ? load16(a.q + q_row + 32 * kk + 8 * g4) ^ q_flip : u32x4{0, 0, 0, 0};
      }
    }
  }
  if constexpr (kQLds) __syncthreads();

  const int64_t head_off_b = static_cast<int64_t>(kvh) * kTileBytes;
  const int64_t blk_stride_b = static_cast<int64_t>(a.num_kv_heads) * kTileBytes;

  // Running max, unnormalised output and column sums of P per tile; the sums come
  // from the matrix cores (P^T times a tile of ones: every row of lsum holds the
  // column's sum), which keeps a conversion and an add per score off the vector ALU.
  bool bad_blk = false;
  float m_run[NT];
  f32x4 acc[NT][MT], lsum[NT];
  const u16x4 ones = __builtin_bit_cast(u16x4, uint2{E::kOne2, E::kOne2});
  const u32x4 ones4 = {E::kOne2, E::kOne2, E::kOne2, E::kOne2};
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    m_run[t] = -INFINITY;
    lsum[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[t][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // FP8 pools take the wave's blocks in pairs (four code buffers; below), except
  // three tiles at three waves per SIMD, whose registers that does not fit
  constexpr bool kPairs = kFp8 && (NT < 3 || NT * D > 192);
  u32x4 kb[kPairs ? 4 : 2][LW], vb[kPairs ? 4 : 2][LW];   // 16-bit: the operands; FP8: codes
  // The wave's blocks go in runs of up to 64: lane i holds the id of the run's i-th.
  int32_t ids = 0, i0 = 0, cnt = 0;

  // Bounded buffer loads as in the decode pass; a step past the run's last block
  // has an empty range and reads nothing.  With several column groups per
  // (sequence, KV head) each tile is read by all of them, so it goes through the
  // caches; with one (kStream) it is read once.
  auto load_block = [&](int buf, int32_t i) {
    const int32_t phys = __builtin_amdgcn_readlane(ids, min(i, cnt - 1));
    const int32_t bytes = i < cnt ? static_cast<int32_t>(kTileBytes) : 0;
    const auto kr = tile_rsrc(reinterpret_cast<const char*>(a.k_cache) + phys * blk_stride_b + head_off_b, bytes);
    const auto vr = tile_rsrc(reinterpret_cast<const char*>(a.v_cache) + phys * blk_stride_b + head_off_b, bytes);
    if constexpr (kFp8) {
      // the decode pass's FP8 operand loads: K dims 64pp + 8g4 .. +7 and 64pp + 32 +
      // 8g4 .. +7 of token n; V dims (64qq + 2n, +1) and (64qq + 32 + 2n, +1) of
      // tokens 4g4 .. +3
#pragma unroll
      for (int pp = 0; pp < LW; ++pp) kb[buf][pp] = load_tile<kStream>(kr, ((pp * 16 + n) * 4 + g4) * 16);
#pragma unroll
      for (int qq = 0; qq < LW; ++qq)
        vb[buf][qq] = load_tile<kStream>(vr, ((g4 * (D / 64) + qq) * 16 + n) * 16);
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) kb[buf][kk] = load_tile<kStream>(kr, (kk * 64 + lane) * 16);
#pragma unroll
      for (int j2 = 0; j2 < KK; ++j2)
        vb[buf][j2] = load_tile<kStream>(vr, ((g4 * D) + 32 * j2 + 2 * n) * 8);
    }
  };

  auto compute_block = [&](int buf, int32_t i) {
    // the block's operands: the loaded registers, or the FP8 codes widened exactly
    u32x4 K[KK], V[KK];
#pragma unroll
    for (int t = 0; t < LW; ++t) {
      if constexpr (kFp8) {
        K[2 * t] = widen_fp8<E>(kb[buf][t][0], kb[buf][t][1]);
        K[2 * t + 1] = widen_fp8<E>(kb[buf][t][2], kb[buf][t][3]);
        V[2 * t] = widen_fp8<E>(vb[buf][t][0], vb[buf][t][1]);
        V[2 * t + 1] = widen_fp8<E>(vb[buf][t][2], vb[buf][t][3]);
      } else {
        K[t] = kb[buf][t];
        V[t] = vb[buf][t];
      }
    }
    f32x4 s[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        u32x4 qv;
        if constexpr (kQLds)
          qv = s_q[(t * KK + kk) * 64 + lane];
        else
          qv = qf[t][kk];
        s[t] = E::mfma_qk(K[kk], qv, s[t]);
      }
    }
    const int32_t t0 = (first + kWaves * (i0 + i)) * kBlock; // position of the block's token 0
    const int32_t valid = i < cnt ? ctx - t0 : 0;            // tokens of the block in context
    if (valid < kBlock) {
      // positions past the context may hold anything (NaN included): zero their V
#pragma unroll
      for (int j2 = 0; j2 < KK; ++j2) {
        u16x8 vv = __builtin_bit_cast(u16x8, V[j2]);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (4 * g4 + (e & 3) >= valid) vv[e] = 0;
        V[j2] = __builtin_bit_cast(u32x4, vv);
      }
    }
    // the causal mask matters only for a block reaching past the first column's
    // position (and for the padding steps past the wave's last block)
    const bool diag = i >= cnt || t0 + kBlock - 1 > pmin;
    const float c = score_scale;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      // raw scores; the running max m_run is kept in scaled log2 units
      float sv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[r] = s[t][r];
      if (diag) {
        const int32_t seen = i < cnt ? pos[t] - t0 : -1;      // this column sees tokens 0 .. seen
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * g4 + r > seen) sv[r] = -INFINITY;
      }
      const float bmax = col_max4_raw(max3_raw(max3_raw(sv[0], sv[1], sv[2]), sv[3], sv[3]));
      // The reference max moves only when a score passes it by more than kLazyMax
      // (log2 units; c >= 0, so the max commutes with the scale), so P <= 2^kLazyMax
      // and most blocks skip the rescale.
      const float m_new = bmax * c > m_run[t] + kLazyMax ? bmax * c : m_run[t];
      // a column may have seen nothing yet: exponentiate against a finite stand-in
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[t] - m_use);
      m_run[t] = m_new;
      // P in 16 bits, two scores per word
      const u16x4 pb = __builtin_bit_cast(
          u16x4, uint2{E::pack2(fast_exp2(__builtin_fmaf(sv[0], c, -m_use)),
                                fast_exp2(__builtin_fmaf(sv[1], c, -m_use))),
                       E::pack2(fast_exp2(__builtin_fmaf(sv[2], c, -m_use)),
                                fast_exp2(__builtin_fmaf(sv[3], c, -m_use)))});
      if (__ballot(alpha != 1.f) != 0) {              // the reference moved somewhere
#pragma unroll
        for (int j = 0; j < MT; ++j) acc[t][j] *= alpha;
        lsum[t] *= alpha;
      }
#pragma unroll
      for (int j2 = 0; j2 < KK; ++j2) {
        const u16x8 vv = __builtin_bit_cast(u16x8, V[j2]);
        const u16x4 lo = {vv[0], vv[1], vv[2], vv[3]};
        const u16x4 hi = {vv[4], vv[5], vv[6], vv[7]};
        acc[t][2 * j2] = E::mfma_pv(lo, pb, acc[t][2 * j2]);
        acc[t][2 * j2 + 1] = E::mfma_pv(hi, pb, acc[t][2 * j2 + 1]);
      }
      lsum[t] = E::mfma_pv(ones, pb, lsum[t]);
    }
  };

  // FP8 pools: blocks i and i + 1 of the wave (buffers b0, b0 + 1) in one step.  The
  // codes of the two blocks widen straight into the operands of the 32-token matrix
  // instruction (a 16-byte operand holds 4 tokens of each), so P.V takes half the
  // matrix instructions of two 16-token steps, and the pair shares one maximum, one
  // rescale and one column-sum instruction.  Positions past the context get zero
  // codes (they may hold anything, NaN codes included).
  auto compute_pair = [&](int b0, int32_t i) {
    int32_t t0[2], valid[2];
    uint32_t keep[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      t0[h] = (first + kWaves * (i0 + i + h)) * kBlock;
      valid[h] = i + h < cnt ? ctx - t0[h] : 0;
      // code byte e of a word is token 4 g4 + e
      const int32_t nv = min(max(valid[h] - 4 * g4, 0), 4);
      keep[h] = nv >= 4 ? 0xffffffffu : (1u << (8 * nv)) - 1u;
    }
    // scores: each q fragment serves both blocks
    u32x4 K[2][KK];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int t = 0; t < LW; ++t) {
        K[h][2 * t] = widen_fp8<E>(kb[b0 + h][t][0], kb[b0 + h][t][1]);
        K[h][2 * t + 1] = widen_fp8<E>(kb[b0 + h][t][2], kb[b0 + h][t][3]);
      }
    f32x4 s[NT][2];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      s[t][0] = s[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        u32x4 qv;
        if constexpr (kQLds)
          qv = s_q[(t * KK + kk) * 64 + lane];
        else
          qv = qf[t][kk];
        s[t][0] = E::mfma_qk(K[0][kk], qv, s[t][0]);
        s[t][1] = E::mfma_qk(K[1][kk], qv, s[t][1]);
      }
    }
    // softmax of every tile first (its scores become the 4-word P operand), so the
    // widened V operands below are not live beside the scores
    __builtin_amdgcn_sched_barrier(0);
    const bool diag = i + 1 >= cnt || t0[1] + kBlock - 1 > pmin;
    const float c = score_scale;
    u32x4 pw[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float sv[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) sv[r] = s[t][r >> 2][r & 3];
      if (diag) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int32_t seen = i + h < cnt ? pos[t] - t0[h] : -1;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (4 * g4 + r > seen) sv[4 * h + r] = -INFINITY;
        }
      }
      const float bmax = col_max4_raw(max3_raw(max3_raw(sv[0], sv[1], sv[2]),
                                               max3_raw(sv[3], sv[4], sv[5]),
                                               max3_raw(sv[6], sv[7], sv[7])));
      const float m_new = bmax * c > m_run[t] + kLazyMax ? bmax * c : m_run[t];
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[t] - m_use);
      m_run[t] = m_new;
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2)
        pw[t][w2] = E::pack2(fast_exp2(__builtin_fmaf(sv[2 * w2], c, -m_use)),
                             fast_exp2(__builtin_fmaf(sv[2 * w2 + 1], c, -m_use)));
      if (__ballot(alpha != 1.f) != 0) {
#pragma unroll
        for (int j = 0; j < MT; ++j) acc[t][j] *= alpha;
        lsum[t] *= alpha;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // P.V: operand (j2, par) holds dims 64 qq + 32 hf + 2 n + par (j2 = 2 qq + hf) of the
    // 4 tokens 4 g4 .. + 3 of block i, then the same 4 of block i + 1
#pragma unroll
    for (int qq = 0; qq < LW; ++qq)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int par = 0; par < 2; ++par) {
          const u32x4 v2 = widen_fp8<E>(vb[b0][qq][2 * hf + par] & keep[0],
                                        vb[b0 + 1][qq][2 * hf + par] & keep[1]);
#pragma unroll
          for (int t = 0; t < NT; ++t)
            acc[t][2 * (2 * qq + hf) + par] = E::mfma_qk(v2, pw[t], acc[t][2 * (2 * qq + hf) + par]);
        }
#pragma unroll
    for (int t = 0; t < NT; ++t) lsum[t] = E::mfma_qk(ones4, pw[t], lsum[t]);
  };

  for (i0 = 0; i0 < nw; i0 += 64) {
    cnt = min(64, nw - i0);
    if (i0 == 0) {
      ids = ids0;
    } else {
      ids = 0;
      if (lane < cnt) ids = bt[first + kWaves * (i0 + lane)];
    }
    const bool id_bad = lane < cnt && (ids < 0 || ids >= a.num_blocks);
    if (id_bad) ids = 0;
    bad_blk = bad_blk || __ballot(id_bad) != 0;
    if constexpr (kPairs) {
      load_block(0, 0);
      load_block(1, 1);
      for (int32_t i = 0; i < cnt; i += 4) {
        load_block(2, i + 2);
        load_block(3, i + 3);
        __builtin_amdgcn_sched_barrier(0);
        compute_pair(0, i);
        load_block(0, i + 4);
        load_block(1, i + 5);
        __builtin_amdgcn_sched_barrier(0);
        compute_pair(2, i + 2);
      }
    } else {
      load_block(0, 0);
      for (int32_t i = 0; i < cnt; i += 2) {
        load_block(1, i + 1);
        __builtin_amdgcn_sched_barrier(0);
        compute_block(0, i);
        load_block(0, i + 2);
        __builtin_amdgcn_sched_barrier(0);
        compute_block(1, i + 1);
      }
    }
  }

  // ---- combine the four waves in LDS, one 16-column tile at a time ----
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (g4 == 0) {
      s_m[t][w][n] = m_run[t];
      s_l[t][w][n] = lsum[t][0];
    }
  }
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (bad_blk) s_bad = 1;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t > 0) __syncthreads();   // the previous tile's reads of s_acc are done
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, s_m[t][v][n]);
    const float wscale = fast_exp2(m_run[t] - (M == -INFINITY ? 0.f : M)) * out_scale;
    {
      float* row = &s_acc[w][n * kLdsStride];
#pragma unroll
      for (int j2 = 0; j2 < KK; ++j2) {
        const f32x4 e = acc[t][2 * j2] * wscale;
        const f32x4 o = acc[t][2 * j2 + 1] * wscale;
        float* dst = row + 32 * j2 + 8 * g4;
        *reinterpret_cast<f32x4*>(dst) = f32x4{e[0], o[0], e[1], o[1]};
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{e[2], o[2], e[3], o[3]};
      }
    }
    __syncthreads();
    const bool poisoned = s_bad != 0;

    // each thread finishes 4 consecutive dims of one column
    for (int32_t i4 = tid; i4 < kCols * (D / 4); i4 += kThreads) {
      const int32_t c = i4 / (D / 4);
      const int32_t d = (i4 - c * (D / 4)) * 4;
      const int32_t gc = col0 + t * kCols + c;
      if (gc >= sq.cols) continue;
      float Mc = -INFINITY;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) Mc = fmaxf(Mc, s_m[t][v][c]);
      const float Mu = Mc == -INFINITY ? 0.f : Mc;
      float L = 0.f;
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        L += s_l[t][v][c] * fast_exp2(s_m[t][v][c] - Mu);
        o += *reinterpret_cast<const f32x4*>(&s_acc[v][c * kLdsStride + d]);
      }
      const int64_t hrow = static_cast<int64_t>(sq.qs + gc / G) * H + kvh * G + gc % G;
      if (direct) {
        u16x4 ov;
        if (poisoned) {
          ov = u16x4{E::kNaN, E::kNaN, E::kNaN, E::kNaN};
        } else {
          const float inv = 1.f / L;
#pragma unroll
          for (int r = 0; r < 4; ++r) ov[r] = E::from_float(o[r] * inv);
        }
        *reinterpret_cast<u16x4*>(a.out + hrow * D + d) = ov;
      } else {
        const int64_t st = hrow * a.parts + part;
        if (poisoned) o = f32x4{NAN, NAN, NAN, NAN};
        *reinterpret_cast<f32x4*>(a.ws_acc + st * D + d) = o;
        if (d == 0) a.ws_ml[st] = poisoned ? float2{0.f, NAN} : float2{Mc, L};
      }
    }
  }
}

constexpr int kWideGroups = 2;                  // groups of 16 columns per wave
constexpr int kWaveCols = 16 * kWideGroups;
constexpr int kWideCols = kWaves * kWaveCols;   // columns per workgroup of the wide kernel

template <class E, int D, bool kFp8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWideGroups > 2 ? 1 : 2)))
void chunk_wide_kernel(ChunkArgs a) {
  constexpr int NG = kWideGroups;
  constexpr int KK = D / 32;                 // 32-dim steps of q.K^T
  constexpr int MT = D / 16;                 // 16-dim tiles of the output
  constexpr int kTileElems = kBlock * D;     // one block's K (or V) tile
  constexpr int kTileBytes = kTileElems * (kFp8 ? 1 : 2);
  // 16-byte pieces of a stage's K per thread (FP8: 16 codes a piece; at head dim 64
  // only the first two waves hold one)
  constexpr int kKChunks = kFp8 ? 1 : 2 * kTileElems / 8 / kThreads;
  constexpr int kKPieces8 = 2 * kTileElems / 16;              // FP8 K pieces of a stage
  constexpr int kVPairs = 2 * D;             // (token quad, dim pair) pieces of a stage's V
  constexpr int kVPieces8 = kTileElems / 16; // FP8 V pieces of one block
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2][2 * kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[2][2 * kTileElems];

  ChunkItem it;
  if (!chunk_item(a, a.parts, &it)) return;
  ChunkSeq sq;
  if (!chunk_seq<kWideCols>(a, it, &sq)) return;
  const int32_t b = __builtin_amdgcn_readfirstlane(it.b);
  const int32_t kvh = __builtin_amdgcn_readfirstlane(it.kvh);
  const int32_t part = __builtin_amdgcn_readfirstlane(it.part);
  const int32_t tile = __builtin_amdgcn_readfirstlane(it.tile);
  const int32_t ctx = __builtin_amdgcn_readfirstlane(sq.ctx);
  const int32_t pmax = __builtin_amdgcn_readfirstlane(sq.pmax);
  const int32_t G = a.group;
  const int32_t H = a.num_heads;

  const int32_t tid = threadIdx.x;
  const int32_t w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t lane = tid & 63;
  const int32_t n = lane & 15;
  const int32_t g4 = lane >> 4;

  const bool direct = a.parts == 1 || (!sq.bad && ctx <= a.part_blocks * kBlock);
  const int32_t nblk_t = sq.bad ? 1 : pmax / kBlock + 1;
  const int32_t pblocks = direct ? nblk_t : a.part_blocks;
  if (part * pblocks >= nblk_t) return;

  if (sq.bad) {
    for (int32_t i = tid; i < kWideCols * D; i += kThreads) {
      const int32_t c = tile * kWideCols + i / D;
      if (c < sq.cols) {
        const int64_t row = static_cast<int64_t>(sq.qs + c / G) * H + kvh * G + c % G;
        a.out[row * D + i % D] = E::kNaN;
      }
    }
    return;
  }

  // position of the tile's first column: keys up to it are seen by every column
  const int32_t pmin = ctx - sq.n + (tile * kWideCols) / G;
  // FP8 pools: the K scale folds into the score scale, the V scale into the output.
  // The running max is taken on raw scores and then scaled, which needs a scale
  // > 0: the sign of a negative one is moved into q (its sign bits flipped).
  const float scale_signed = kFp8 ? a.scale_log2 * a.k_scales[kvh] : a.scale_log2;
  const uint32_t q_flip = scale_signed < 0.f ? 0x80008000u : 0u;
  // A zero scale would turn a masked score (-inf) into NaN: 1e-30 leaves every
  // exponent rounding to the same value and a masked one at -inf.
  const float score_scale = fmaxf(fabsf(scale_signed), 1e-30f);
  const float out_scale = kFp8 ? a.v_scales[kvh] : 1.f;
  // the lane's columns (one per group of 16)
  int32_t pos[NG];
  bool col_ok[NG];
  int64_t hrow[NG];
  u32x4 qf[NG][KK];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int32_t col = tile * kWideCols + w * kWaveCols + gi * 16 + n;
    col_ok[gi] = col < sq.cols;
    const int32_t ti = col_ok[gi] ? col / G : 0;
    const int32_t gh = col_ok[gi] ? col - ti * G : 0;
    pos[gi] = col_ok[gi] ? ctx - sq.n + ti : pmax;        // padding columns: zero q
    hrow[gi] = static_cast<int64_t>(sq.qs + ti) * H + kvh * G + gh;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[gi][kk] = col_ok[gi] ? load16(a.q + hrow[gi] * D + 32 * kk + 8 * g4) ^ q_flip : u32x4{0, 0, 0, 0};
  }

  const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_blocks;
  const int32_t jbeg = part * pblocks;
  const int32_t jend = min(nblk_t, jbeg + pblocks);
  const int32_t nstage = (jend - jbeg + 1) / 2;
  const int64_t head_off_b = static_cast<int64_t>(kvh) * kTileBytes;
  const int64_t blk_stride_b = static_cast<int64_t>(a.num_kv_heads) * kTileBytes;
  const char* kc = reinterpret_cast<const char*>(a.k_cache);
  const char* vc = reinterpret_cast<const char*>(a.v_cache);

  // block ids in runs of 64: lane i holds the id of block jbeg + 64 r + i
  int32_t ids = 0;
  bool bad_blk = false;
  auto load_ids = [&](int32_t r) {
    const int32_t j = jbeg + 64 * r + lane;
    int32_t v = j < jend ? bt[j] : 0;
    const bool bad = j < jend && (v < 0 || v >= a.num_blocks);
    if (bad) v = 0;
    bad_blk = bad_blk || __ballot(bad) != 0;
    ids = v;
  };

  // a stage's K and V, global -> registers -> LDS; two register sets, so the loads
  // of a stage are issued two stages before it is computed
  using KRegs = u32x4[kKChunks];
  using VRegs = u32x4[2];
  // Issued for every step, also past the last stage: the empty ranges of stages
  // that do not exist read nothing, and no load sits behind a branch (which would
  // make the compiler copy -- and so wait for -- the loaded registers).
  auto stage_load = [&](int32_t st, KRegs& kst, VRegs& vst) {
    const int32_t j0 = jbeg + 2 * st;
    const int32_t l0 = (2 * st) & 63;                        // index within the id run
    const int32_t p0 = __builtin_amdgcn_readlane(ids, l0);
    const int32_t p1 = __builtin_amdgcn_readlane(ids, l0 + 1);
    const int32_t bytes0 = j0 < jend ? kTileBytes : 0;
    const int32_t bytes1 = j0 + 1 < jend ? kTileBytes : 0;
    const int32_t wp = __builtin_amdgcn_readfirstlane(w * 64);
    if constexpr (kFp8) {
      // K: FP8 piece tid % (kKPieces8 / 2) of block tid / (kKPieces8 / 2); V: FP8 piece
      // tid < kVPieces8 of both blocks.  Waves past the pieces read empty ranges.
      const bool second = wp >= kKPieces8 / 2;
      const int32_t kbytes = wp < kKPieces8 ? (second ? bytes1 : bytes0) : 0;
      const auto kr = tile_rsrc(kc + (second ? p1 : p0) * blk_stride_b + head_off_b, kbytes);
      kst[0] = load_tile<false>(kr, (tid % (kKPieces8 / 2)) * 16);
      const int32_t vb = wp < kVPieces8 ? 1 : 0;
      const auto v0 = tile_rsrc(vc + p0 * blk_stride_b + head_off_b, bytes0 * vb);
      const auto v1 = tile_rsrc(vc + p1 * blk_stride_b + head_off_b, bytes1 * vb);
      vst[0] = load_tile<false>(v0, tid * 16);
      vst[1] = load_tile<false>(v1, tid * 16);
    } else {
#pragma unroll
      for (int c = 0; c < kKChunks; ++c) {
        // the wave's 64 pieces all lie in one block's tile (a tile is 128 or 256 pieces)
        const int32_t wpiece = __builtin_amdgcn_readfirstlane(w * 64 + c * kThreads);
        const bool second = wpiece >= kTileElems / 8;
        const auto kr = tile_rsrc(kc + (second ? p1 : p0) * blk_stride_b + head_off_b,
                                  second ? bytes1 : bytes0);
        kst[c] = load_tile<false>(kr, ((tid + c * kThreads) % (kTileElems / 8)) * 16);
      }
      // V: pieces tid < 2 D of both blocks (whole waves: 2 D is a multiple of 64); the
      // other waves read an empty range
      const int32_t vb = wp < kVPairs ? 1 : 0;
      const auto v0 = tile_rsrc(vc + p0 * blk_stride_b + head_off_b, bytes0 * vb);
      const auto v1 = tile_rsrc(vc + p1 * blk_stride_b + head_off_b, bytes1 * vb);
      vst[0] = load_tile<false>(v0, tid * 16);
      vst[1] = load_tile<false>(v1, tid * 16);
    }
  };
  // (token quad tq, dims d and d + 1, 4 tokens each) of the stage's two blocks into the
  // interleaved V layout, positions past the context zeroed (they may hold anything,
  // NaN included)
  auto store_v = [&](int32_t st, int buf, int32_t tq, int32_t d, u16x8 x0, u16x8 x1) {
    const int32_t t0 = (jbeg + 2 * st) * kBlock + 4 * tq;   // position of the quad's token 0
    if ((jbeg + 2 * st + 2) * kBlock > ctx) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (t0 + (e & 3) >= ctx) x0[e] = 0;
        if (t0 + kBlock + (e & 3) >= ctx) x1[e] = 0;
      }
    }
    const u16x8 lo = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    const u16x8 hi = {x0[4], x0[5], x0[6], x0[7], x1[4], x1[5], x1[6], x1[7]};
    uint16_t* dst = &s_v[buf][(tq * D + d) * 8];
    *reinterpret_cast<u16x8*>(dst) = lo;
    *reinterpret_cast<u16x8*>(dst + 8) = hi;
  };
  auto stage_store = [&](int32_t st, int buf, const KRegs& kst, const VRegs& vst) {
    if constexpr (kFp8) {
      // K piece: dims 64pp + 8g8 .. +7 and 64pp + 32 + 8g8 .. +7 of token n8, widened
      // exactly and stored where the 16-bit layout keeps them
      if (tid < kKPieces8) {
        const int32_t blk = tid / (kKPieces8 / 2);
        const int32_t p8 = tid - blk * (kKPieces8 / 2);
        const int32_t g8 = p8 & 3, n8 = (p8 >> 2) & 15, pp = p8 >> 6;
        uint16_t* kt = &s_k[buf][blk * kTileElems];
        *reinterpret_cast<u32x4*>(kt + ((8 * pp + g8) * 16 + n8) * 8) =
            widen_fp8<E>(kst[0][0], kst[0][1]);
        *reinterpret_cast<u32x4*>(kt + ((8 * pp + 4 + g8) * 16 + n8) * 8) =
            widen_fp8<E>(kst[0][2], kst[0][3]);
      }
      // V piece: dims (64qq + 2n, +1) and (64qq + 32 + 2n, +1) of token quad tq
      if (tid < kVPieces8) {
        const int32_t nv = tid & 15, qq = (tid >> 4) % (D / 64), tq = (tid >> 4) / (D / 64);
#pragma unroll
        for (int h = 0; h < 2; ++h)
          store_v(st, buf, tq, 64 * qq + 32 * h + 2 * nv,
                  __builtin_bit_cast(u16x8, widen_fp8<E>(vst[0][2 * h], vst[0][2 * h + 1])),
                  __builtin_bit_cast(u16x8, widen_fp8<E>(vst[1][2 * h], vst[1][2 * h + 1])));
      }
    } else {
#pragma unroll
      for (int c = 0; c < kKChunks; ++c)
        *reinterpret_cast<u32x4*>(&s_k[buf][(tid + c * kThreads) * 8]) = kst[c];
      if (tid < kVPairs) {
        // piece tid holds token quad tq, dims d and d + 1, 4 tokens each, of one block
        const int32_t tq = tid / (D / 2);
        store_v(st, buf, tq, 2 * (tid - tq * (D / 2)), __builtin_bit_cast(u16x8, vst[0]),
                __builtin_bit_cast(u16x8, vst[1]));
      }
    }
  };

  // Running max per column, the unnormalised output, and the column sums of P: those
  // come from the matrix cores too, as P^T times a tile of ones (every row of lsum
  // holds the column's sum), which moves a conversion and an add per score off the
  // vector ALU, the unit this kernel waits on.
  float m_run[NG];
  f32x4 acc[NG][MT], lsum[NG];
  const u32x4 ones = {E::kOne2, E::kOne2, E::kOne2, E::kOne2};
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    m_run[gi] = -INFINITY;
    lsum[gi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[gi][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto compute = [&](int32_t st, int buf) {
    f32x4 sc[NG][2];   // [group][block]
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) sc[gi][0] = sc[gi][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // all K operands first, then independent accumulation chains per 32-dim step
    u32x4 kf[2][KK];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        kf[blk][kk] =
            *reinterpret_cast<const u32x4*>(&s_k[buf][blk * kTileElems + (kk * 64 + lane) * 8]);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) sc[gi][blk] = E::mfma_qk(kf[blk][kk], qf[gi][kk], sc[gi][blk]);
    // V operands, read while the softmax runs
    u32x4 vf[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
      vf[t] = *reinterpret_cast<const u32x4*>(&s_v[buf][(g4 * D + 16 * t + n) * 8]);
    const int32_t t0 = (jbeg + 2 * st) * kBlock;   // position of the stage's first key
    // a stage wholly at or before the tile's first position needs no causal mask
    const bool diag = t0 + 2 * kBlock - 1 > pmin;
    const float c = score_scale;
    u32x4 pf[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      // raw scores; the running max m_run is kept in scaled log2 units
      float sv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[e] = e < 4 ? sc[gi][0][e] : sc[gi][1][e - 4];
      if (diag) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int32_t key = t0 + (e < 4 ? 4 * g4 + e : kBlock + 4 * g4 + e - 4);
          if (key > pos[gi]) sv[e] = -INFINITY;
        }
      }
      float bmax = max3_raw(max3_raw(sv[0], sv[1], sv[2]), max3_raw(sv[3], sv[4], sv[5]),
                            max3_raw(sv[6], sv[7], sv[7]));
      bmax = col_max4_raw(bmax);
      // The reference max moves only when a score exceeds it by more than 2^8 (c >= 0:
      // the max commutes with the scale).  Exponents stay <= 8, so P <= 256, which the
      // 16-bit P and the float32 sums hold at full relative precision, and most stages
      // skip the rescale of the accumulators.  The normalisation and the partition
      // merge are exact for any reference.
      const float m_new = bmax * c > m_run[gi] + kLazyMax ? bmax * c : m_run[gi];
      // a column may have seen nothing yet: exponentiate against a finite stand-in
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[gi] - m_use);
      m_run[gi] = m_new;
      // P in 16 bits, two scores per operand word
      u32x4 pw;
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2)
        pw[w2] = E::pack2(fast_exp2(__builtin_fmaf(sv[2 * w2], c, -m_use)),
                          fast_exp2(__builtin_fmaf(sv[2 * w2 + 1], c, -m_use)));
      if (__ballot(alpha != 1.f) != 0) {              // the running max moved somewhere
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[gi][t] *= alpha;
        lsum[gi] *= alpha;
      }
      pf[gi] = pw;
    }
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) acc[gi][t] = E::mfma_qk(vf[t], pf[gi], acc[gi][t]);
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) lsum[gi] = E::mfma_qk(ones, pf[gi], lsum[gi]);
  };

  // free: the set that receives stage st + 2; held: the set holding stage st + 1
  auto step = [&](int32_t st, KRegs& k_free, VRegs& v_free, const KRegs& k_held,
                  const VRegs& v_held) {
    if ((2 * (st + 2)) % 64 == 0) load_ids((2 * (st + 2)) / 64);
    stage_load(st + 2, k_free, v_free);
    compute(st, st & 1);
    stage_store(st + 1, (st + 1) & 1, k_held, v_held);   // past the end: never read
    __syncthreads();
  };
  u32x4 kA[kKChunks], vA[2], kB[kKChunks], vB[2];
  load_ids(0);
  stage_load(0, kA, vA);
  stage_load(1, kB, vB);
  stage_store(0, 0, kA, vA);
  __syncthreads();
  for (int32_t st = 0; st < nstage; st += 2) {
    step(st, kA, vA, kB, vB);
    if (st + 1 < nstage) step(st + 1, kB, vB, kA, vA);
  }

  // ---- outputs: lane l holds dims 16 t + 4 g4 .. + 3 of its columns ----
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const float L = lsum[gi][0];
    if (!col_ok[gi]) continue;
    if (direct) {
      const float inv = out_scale / L;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        u16x4 ov;
#pragma unroll
        for (int r = 0; r < 4; ++r) ov[r] = bad_blk ? E::kNaN : E::from_float(acc[gi][t][r] * inv);
        *reinterpret_cast<u16x4*>(a.out + hrow[gi] * D + 16 * t + 4 * g4) = ov;
      }
    } else {
      const int64_t st = hrow[gi] * a.parts + part;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const f32x4 o = bad_blk ? f32x4{NAN, NAN, NAN, NAN} : acc[gi][t] * out_scale;
        *reinterpret_cast<f32x4*>(a.ws_acc + st * D + 16 * t + 4 * g4) = o;
      }
      if (g4 == 0) a.ws_ml[st] = bad_blk ? float2{0.f, NAN} : float2{m_run[gi], L};
    }
  }
}

// One workgroup per (sequence, KV head, column tile) of the sequences whose context
// spans several partitions, 4 dims of one column per thread: M = max_p m_p, out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p over
// the partitions a column's own position reaches (later ones hold nothing for it),
// in partition order.
template <class E, int D>
__global__ __launch_bounds__(kThreads) void chunk_merge_kernel(ChunkArgs a) {
  ChunkItem it;
  if (!chunk_item(a, 1, &it)) return;
  ChunkSeq sq;
  if (!chunk_seq(a, it, &sq)) return;
  if (sq.bad) return;                       // the attention pass wrote NaN
  const int32_t part_tokens = a.part_blocks * kBlock;
  if (sq.ctx <= part_tokens) return;        // one partition: written directly
  const int32_t G = a.group;
  const int32_t H = a.num_heads;
  for (int32_t i4 = threadIdx.x; i4 < kCols * (D / 4); i4 += kThreads) {
    const int32_t c = i4 / (D / 4);
    const int32_t d = (i4 - c * (D / 4)) * 4;
    const int32_t gc = it.tile * kCols + c;
    if (gc >= sq.cols) continue;
    const int32_t pos = sq.ctx - sq.n + gc / G;
    const int32_t np = pos / part_tokens + 1;
    const int64_t hrow = static_cast<int64_t>(sq.qs + gc / G) * H + it.kvh * G + gc % G;
    const int64_t st0 = hrow * a.parts;
    float M = -INFINITY;
    for (int32_t p = 0; p < np; ++p) M = fmaxf(M, a.ws_ml[st0 + p].x);
    float L = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    for (int32_t p = 0; p < np; ++p) {
      const float2 ml = a.ws_ml[st0 + p];
      const float wgt = fast_exp2(ml.x - M);
      L += wgt * ml.y;
      o += wgt * *reinterpret_cast<const f32x4*>(a.ws_acc + (st0 + p) * D + d);
    }
    const float inv = 1.f / L;
    u16x4 ov;
#pragma unroll
    for (int r = 0; r < 4; ++r) ov[r] = E::from_float(o[r] * inv);
    *reinterpret_cast<u16x4*>(a.out + hrow * D + d) = ov;
  }
}

// The launch plan.  Launches with at least 128 columns per (sequence, KV head)
// use the wide kernel; narrower ones the narrow kernel with up to three 16-column
// tiles per workgroup.
// Key partitions: one when the column groups alone give every workgroup slot
// enough items (eight for the narrow kernel, two for the wide one); else the
// longest of 4096, 2048 and 1024 tokens for which even the longest possible item
// list (every sequence at the longest context) gives every slot two items, so
// long contexts with few new tokens still spread over the device while each item
// stays long enough to amortise its start-up.
constexpr int kMaxNarrowTiles = 3;
struct ChunkPlan {
  bool wide;
  int32_t nt;           // 16-column tiles per workgroup of the narrow kernel
  int32_t tiles;        // column groups of the attention launch
  int32_t merge_tiles;  // 16-column tiles of the merge launch
  int32_t parts;
  int32_t part_blocks;
  bool ordered;         // narrow kernel, at most kOrderedItemsPerSlot items per slot
};
constexpr int64_t kOrderedItemsPerSlot = 4;
constexpr int32_t kMaxOrderedSeqs = 1024;
ChunkPlan chunk_plan(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t max_q_len, int32_t max_ctx) {
  ChunkPlan p;
  const int64_t cols = static_cast<int64_t>(max_q_len) * (num_heads / num_kv_heads);
  p.wide = cols >= kWideCols;
  p.merge_tiles = static_cast<int32_t>((cols + kCols - 1) / kCols);
  p.nt = p.wide ? 1 : std::min(p.merge_tiles, kMaxNarrowTiles);
  p.tiles = p.wide ? static_cast<int32_t>((cols + kWideCols - 1) / kWideCols)
                   : (p.merge_tiles + p.nt - 1) / p.nt;
  const int64_t items = static_cast<int64_t>(num_seqs) * num_kv_heads * p.tiles;
  // workgroups per compute unit: the wide kernel and the multi-tile narrow one at
  // head dim 128 run two, the others three or more
  const int64_t per_cu = p.wide ? (kWideGroups > 2 ? 1 : 2) : p.nt * head_dim > 192 ? 2 : 3;
  const int64_t slots = per_cu * static_cast<int64_t>(pa::device_cus());
  p.part_blocks = kMinPartTokens / kBlock;
  if (items >= (p.wide ? 1 : 8) * slots) {
    p.parts = 1;
  } else {
    for (int32_t pt = kMaxPartTokens; pt > kMinPartTokens; pt /= 2)
      if (items * ((max_ctx + pt - 1) / pt) >= 2 * slots) {
        p.part_blocks = pt / kBlock;
        break;
      }
    const int32_t part_tokens = p.part_blocks * kBlock;
    p.parts = (max_ctx + part_tokens - 1) / part_tokens;
  }
  p.ordered = !p.wide && num_seqs <= kMaxOrderedSeqs &&
              items * p.parts <= kOrderedItemsPerSlot * slots;
  return p;
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// e0 / e1 (optional): events that take the start of the attention kernel and the end of
// the call's last kernel, attached to the dispatches.
template <class E, int D, bool kStream, bool kFp8>
void launch_narrow(const ChunkArgs& a, int32_t nt, dim3 grid, hipStream_t s, hipEvent_t e0,
                   hipEvent_t e1) {
  if (nt == 1)
    hipExtLaunchKernelGGL(chunk_attn_kernel<E, D, 1, kStream, kFp8>, grid, dim3(kThreads), 0, s,
                          e0, e1, 0, a);
  else if (nt == 2)
    hipExtLaunchKernelGGL(chunk_attn_kernel<E, D, 2, kStream, kFp8>, grid, dim3(kThreads), 0, s,
                          e0, e1, 0, a);
  else
    hipExtLaunchKernelGGL(chunk_attn_kernel<E, D, 3, kStream, kFp8>, grid, dim3(kThreads), 0, s,
                          e0, e1, 0, a);
}

template <class E, int D, bool kFp8>
void launch_chunk_d(const ChunkArgs& a, const ChunkPlan& p, int64_t groups8, bool stream,
                    hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const dim3 grid(static_cast<uint32_t>(groups8 * p.tiles * p.parts));
  hipEvent_t e1_attn = p.parts > 1 ? nullptr : e1;   // with a merge, it takes the end
  if (p.wide)
    hipExtLaunchKernelGGL(chunk_wide_kernel<E, D, kFp8>, grid, dim3(kThreads), 0, s, e0, e1_attn,
                          0, a);
  else if (stream)
    launch_narrow<E, D, true, kFp8>(a, p.nt, grid, s, e0, e1_attn);
  else
    launch_narrow<E, D, false, kFp8>(a, p.nt, grid, s, e0, e1_attn);
  if (p.parts > 1) {
    ChunkArgs m = a;                     // the merge works in 16-column tiles
    m.col_tiles = p.merge_tiles;
    hipExtLaunchKernelGGL(chunk_merge_kernel<E, D>,
                          dim3(static_cast<uint32_t>(groups8 * p.merge_tiles)), dim3(kThreads), 0,
                          s, nullptr, e1, 0, m);
  }
}

template <class E>
void launch_chunk(const ChunkArgs& a, const ChunkPlan& p, int64_t groups8, int d, bool fp8,
                  bool stream, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (d == 64) {
    if (fp8)
      launch_chunk_d<E, 64, true>(a, p, groups8, stream, s, e0, e1);
    else
      launch_chunk_d<E, 64, false>(a, p, groups8, stream, s, e0, e1);
  } else {
    if (fp8)
      launch_chunk_d<E, 128, true>(a, p, groups8, stream, s, e0, e1);
    else
      launch_chunk_d<E, 128, false>(a, p, groups8, stream, s, e0, e1);
  }
}

}  // namespace

namespace pa {

// pa_chunk_attention's checks and launches; q_starts NULL means one query per
// sequence, row b (the caller has checked that this is what it wants).
pa_status chunk_run(const char* fn, const pa_cache* cache, const void* q, const int32_t* q_starts,
                    int32_t num_seqs, int32_t total_q, int32_t max_q_len, int32_t num_heads,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t max_context_len, float scale, void* out,
                    void* workspace, size_t workspace_bytes, void* ev_begin, void* ev_end,
                    void* stream) {
  pa_status st = pa::check_cache(cache, fn);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || total_q < 0)
    return pa::fail(PA_ERR_INVALID_ARG, "%s: num_seqs %d, total_q %d", fn, num_seqs, total_q);
  if (num_seqs == 0 || total_q == 0) return PA_OK;
  if (num_heads <= 0 || num_heads % cache->num_kv_heads)
    return pa::fail(PA_ERR_INVALID_ARG, "%s: num_heads %d not a multiple of num_kv_heads %d", fn,
                    num_heads, cache->num_kv_heads);
  if (max_q_len < 1 || max_context_len < 1)
    return pa::fail(PA_ERR_INVALID_ARG, "%s: max_q_len %d, max_context_len %d", fn, max_q_len,
                    max_context_len);
  if (max_blocks_per_seq < 1 || static_cast<int64_t>(max_blocks_per_seq) * kBlock < max_context_len)
    return pa::fail(PA_ERR_INVALID_ARG, "%s: max_blocks_per_seq %d cannot hold %d tokens", fn,
                    max_blocks_per_seq, max_context_len);
  if (!q || !block_tables || !context_lens || !out || !pa::aligned16(q) ||
      !pa::aligned16(out))
    return pa::fail(PA_ERR_INVALID_ARG, "%s: NULL pointer or q / out not 16-byte aligned", fn);
  if (!std::isfinite(scale)) return pa::fail(PA_ERR_INVALID_ARG, "%s: scale is not finite", fn);
  const int32_t G = num_heads / cache->num_kv_heads;
  const ChunkPlan plan = chunk_plan(num_seqs, num_heads, cache->num_kv_heads, cache->head_dim,
                                    max_q_len, max_context_len);
  const int32_t P = plan.parts;
  const int64_t groups = static_cast<int64_t>(num_seqs) * cache->num_kv_heads;
  const int64_t groups8 = 8 * ((groups + 7) / 8);
  const int64_t grid = groups8 * plan.tiles * P;
  if (grid > INT32_MAX || groups8 * plan.merge_tiles > INT32_MAX ||
      static_cast<int64_t>(total_q) * num_heads * P > INT32_MAX)
    return pa::fail(PA_ERR_UNSUPPORTED, "%s: launch too large", fn);
  const size_t need = pa_chunk_workspace_size(num_seqs, num_heads, cache->num_kv_heads,
                                              cache->head_dim, total_q, max_q_len, max_context_len);
  if (need > 0 && (!workspace || workspace_bytes < need || !pa::aligned16(workspace)))
    return pa::fail(PA_ERR_WORKSPACE, "%s: workspace %zu bytes, %zu needed", fn, workspace_bytes,
                    need);
  ChunkArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint16_t*>(cache->k_cache);
  a.v_cache = static_cast<const uint16_t*>(cache->v_cache);
  a.k_scales = cache->k_scales;
  a.v_scales = cache->v_scales;
  a.q_starts = q_starts;
  a.block_tables = block_tables;
  a.ctx_lens = context_lens;
  a.out = static_cast<uint16_t*>(out);
  const int64_t rows = static_cast<int64_t>(total_q) * num_heads * P;
  a.ws_ml = P > 1 ? static_cast<float2*>(workspace) : nullptr;
  a.ws_acc = P > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                              round256(static_cast<size_t>(rows) * sizeof(float2)))
                   : nullptr;
  a.num_seqs = num_seqs;
  a.total = total_q;
  a.num_heads = num_heads;
  a.num_kv_heads = cache->num_kv_heads;
  a.group = G;
  a.max_blocks = max_blocks_per_seq;
  a.max_ctx = max_context_len;
  a.num_blocks = cache->num_blocks;
  a.col_tiles = plan.tiles;
  a.parts = P;
  a.part_blocks = plan.part_blocks;
  a.ordered = plan.ordered ? 1 : 0;
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // one column group per (sequence, KV head) reads each tile once, unless blocks
  // are shared between sequences
  const bool once = plan.tiles == 1 && !(cache->flags & PA_CACHE_SHARED_BLOCKS);
  const bool fp8 = (cache->flags & PA_CACHE_FP8) != 0;
  const auto e0 = static_cast<hipEvent_t>(ev_begin), e1 = static_cast<hipEvent_t>(ev_end);
  if (cache->dtype == PA_F16)
    launch_chunk<F16>(a, plan, groups8, cache->head_dim, fp8, once, s, e0, e1);
  else
    launch_chunk<BF16>(a, plan, groups8, cache->head_dim, fp8, once, s, e0, e1);
  return pa::launch_status(fn);
}

pa_status chunk_decode(const char* fn, const pa_cache* cache, const void* q, int32_t num_seqs,
                       int32_t num_heads, const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* context_lens, int32_t max_context_len, float scale,
                       void* out, void* workspace, size_t workspace_bytes, void* ev_begin,
                       void* ev_end, void* stream) {
  return chunk_run(fn, cache, q, nullptr, num_seqs, num_seqs, 1, num_heads, block_tables,
                   max_blocks_per_seq, context_lens, max_context_len, scale, out, workspace,
                   workspace_bytes, ev_begin, ev_end, stream);
}

}  // namespace pa

extern "C" {

size_t pa_chunk_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t total_q, int32_t max_q_len,
                               int32_t max_context_len) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads ||
      head_dim <= 0 || total_q <= 0 || max_q_len <= 0 || max_context_len <= 0)
    return 0;
  const int32_t P =
      chunk_plan(num_seqs, num_heads, num_kv_heads, head_dim, max_q_len, max_context_len).parts;
  if (P <= 1) return 0;
  const int64_t rows = static_cast<int64_t>(total_q) * num_heads * P;
  return round256(static_cast<size_t>(rows) * sizeof(float2)) +
         static_cast<size_t>(rows) * head_dim * sizeof(float);
}

pa_status pa_chunk_attention(const pa_cache* cache, const void* q, const int32_t* q_starts,
                             int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                             int32_t num_heads, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* context_lens,
                             int32_t max_context_len, float scale, void* out, void* workspace,
                             size_t workspace_bytes, void* attn_begin, void* attn_end,
                             void* stream) {
  pa::clear_error();
  if (!q_starts && num_seqs > 0 && total_q > 0)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_chunk_attention: q_starts is NULL");
  return pa::chunk_run("pa_chunk_attention", cache, q, q_starts, num_seqs, total_q, max_q_len,
                       num_heads, block_tables, max_blocks_per_seq, context_lens, max_context_len,
                       scale, out, workspace, workspace_bytes, attn_begin, attn_end, stream);
}

}  // extern "C"
