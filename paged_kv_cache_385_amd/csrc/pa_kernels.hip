// Paged KV-cache kernels for gfx950 (CDNA4) and their C-ABI entry points.
//
//   cache_write_kernel   slot-mapped store of new tokens' K/V ("vLLM 核心概念",
//                        sections "为什么需要 KV Cache？" and "按需分配")
//   block_copy_kernel    whole-block copies: copy-on-write ("理解 vLLM PagedAttention",
//                        section 六) and swapping to and from host pools ("vLLM 核心概念",
//                        section 内存层次结构)
//   decode_attn_kernel   single-query attention over a block-paged context
//                        ("PagedAttention 实战", section "Decode：逐 token 生成输出";
//                        "vLLM 核心概念", section "逻辑视图与物理视图分离")
//   decode_merge_kernel  log-sum-exp merge of context partitions ("PagedAttention 实战",
//                        section "2026 年的新变化": sequence split)
//
// Layout of the pools (see pa.h): K [NB][Hkv][D/8][16][8], V [NB][Hkv][4][D][4].
// With that layout one (block, head) tile is 16*D contiguous elements and each
// wave reads it with one 16-byte load per lane per 1 KiB; every loaded vector is
// already a matrix-core operand:
//   q.K^T : v_mfma_f32_16x16x32_{f16,bf16}, A = K tile (16 tokens x 32 dims),
//           B = q^T (32 dims x 16 query heads of one KV-head group, zero-padded),
//           C = S^T (16 tokens x 16 heads); lane l holds tokens 4(l/16)..+3 of head l%16.
//   P.V   : v_mfma_f32_16x16x16_{f16,bf16}, A = V^T (16 dims x 16 tokens),
//           B = P^T (16 tokens x 16 heads) -- exactly the S^T register layout, so the
//           softmax output feeds the second product without any data movement,
//           C = out^T; lane l accumulates head l%16, so the online-softmax rescale
//           is lane-local.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstdint>
#include <vector>

#include "pa_device.h"
#include "pa_internal.h"
#include "pa_timeline.h"

#ifdef PA_TIMELINE
// Records of the decode kernel's workgroups (instrumented build only; layout in
// pa_timeline.h).  TL_STAMP reads the constant 100 MHz counter.
__device__ uint64_t g_timeline[PA_TIMELINE_MAX_WORKGROUPS * PA_TIMELINE_WORDS];
#define TL_STAMP(v) v = __builtin_amdgcn_s_memrealtime()
#else
#define TL_STAMP(v) ((void)0)
#endif

namespace {

using namespace pa_dev;

constexpr int kPartTokens = PA_PARTITION_TOKENS;            // shortest partition (512)
constexpr int kMaxPartTokens = 8 * PA_PARTITION_TOKENS;     // longest partition (4096)
constexpr int kWaves = 4;                                   // waves per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kMaxParts = 1024;                             // longest context / 512
#ifndef PA_SIZE_CLASSES
#define PA_SIZE_CLASSES 4
#endif
constexpr int kClasses = PA_SIZE_CLASSES;                   // size classes of last partitions
// pa_cache_write calls with at least this many tokens take the whole-block kernel
#ifndef PA_BULK_WRITE_TOKENS
#define PA_BULK_WRITE_TOKENS 64
#endif
constexpr int kBulkTokens = PA_BULK_WRITE_TOKENS;
static_assert(kClasses >= 1 && kClasses <= 64, "one lane per size class");

// ---- cache write -----------------------------------------------------------------
// One thread per (token, KV head, 8-dim chunk): a 16-byte K store, eight 2-byte V stores.
template <int D>
__global__ __launch_bounds__(256) void cache_write_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int64_t* __restrict__ slots, uint16_t* __restrict__ k_cache,
    uint16_t* __restrict__ v_cache, int32_t num_tokens, int32_t hkv, int64_t num_slots) {
  constexpr int kChunks = D / 8;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per_token = static_cast<int64_t>(hkv) * kChunks;
  if (idx >= static_cast<int64_t>(num_tokens) * per_token) return;
  const int64_t t = idx / per_token;
  const int32_t rem = static_cast<int32_t>(idx - t * per_token);
  const int32_t h = rem / kChunks;
  const int32_t c = rem - h * kChunks;
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot >> 4;
  const int32_t off = static_cast<int32_t>(slot & 15);
  const int64_t src = (t * hkv + h) * D + 8 * c;
  const int64_t tile = (blk * hkv + h) * (kBlock * D);
  store16(k_cache + tile + (static_cast<int64_t>(c) * kBlock + off) * 8, load16(k + src));
  const u16x8 vv = __builtin_bit_cast(u16x8, load16(v + src));
  uint16_t* vdst = v_cache + tile + (static_cast<int64_t>(off >> 2) * D + 8 * c) * 4 + (off & 3);
#pragma unroll
  for (int i = 0; i < 8; ++i) vdst[4 * i] = vv[i];
}

// Bulk form: one workgroup of 2*D threads per (16 consecutive tokens of the input,
// KV head).  A whole block is a run of 16 consecutive input tokens whose slots are
// 16j .. 16j + 15 in order (what a prefill or an admission stores, wherever the
// run starts in the input); at most one such run starts within any 16 tokens.  The
// workgroup writes the run that starts among its tokens, if any, as the block's K
// and V tiles of that head front to back, 16 bytes per thread each:
//   thread i, K: dims 8(i/16) .. +7 of token i%16 of the run, one 16-byte load;
//   thread i, V: dims 2m, 2m+1 of tokens 4(i/(D/2)) .. +3, m = i % (D/2): four
//   4-byte loads, one per token, each a contiguous run across the wave.
// Its tokens outside any whole block (partial blocks, slots out of order, skipped
// or out-of-range slots) are stored one element group at a time, as
// cache_write_kernel does; its tokens inside a run that started in the previous
// group are left to that group's workgroup.
template <int D>
__global__ __launch_bounds__(2 * D) void cache_write_bulk_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int64_t* __restrict__ slots, uint16_t* __restrict__ k_cache,
    uint16_t* __restrict__ v_cache, int32_t num_tokens, int32_t hkv, int64_t num_slots) {
  constexpr int kThreadsB = 2 * D;
  constexpr int kChunks = D / 8;
  constexpr int kWin = 3 * kBlock - 1;           // tokens g0 - 15 .. g0 + 31
  static_assert(kThreadsB >= 64 && kBlock * kChunks <= kThreadsB, "one element group per thread");
  __shared__ int64_t s_slot[kWin];
  __shared__ int32_t s_prev, s_start;
  const int32_t i = threadIdx.x;
  const int32_t h = blockIdx.y;
  const int64_t g0 = static_cast<int64_t>(blockIdx.x) * kBlock;
  for (int32_t j = i; j < kWin; j += kThreadsB) {
    const int64_t t = g0 - (kBlock - 1) + j;
    s_slot[j] = t >= 0 && t < num_tokens ? slots[t] : -1;
  }
  __syncthreads();
  if (i < 64) {
    // lane j < 31: does a whole block start at token g0 - 15 + j?
    bool start = false;
    if (i < 2 * kBlock - 1) {
      const int64_t s0 = s_slot[i];
      start = s0 >= 0 && (s0 & (kBlock - 1)) == 0 && s0 + kBlock <= num_slots;
      for (int j = 1; j < kBlock && start; ++j) start = s_slot[i + j] == s0 + j;
    }
    const uint64_t m = __ballot(start);
    if (i == 0) {
      const uint64_t prev = m & ((1ull << (kBlock - 1)) - 1);   // starts before g0
      const uint64_t cur = m >> (kBlock - 1);                   // starts at g0 .. g0 + 15
      s_prev = prev ? __ffsll(static_cast<unsigned long long>(prev)) : 0;   // tokens covered
      s_start = cur ? __ffsll(static_cast<unsigned long long>(cur)) - 1 : -1;
    }
  }
  __syncthreads();
  const int32_t covered_prev = s_prev, start = s_start;
  const int64_t row = static_cast<int64_t>(hkv) * D;            // elements per input token
  if (start >= 0) {
    const int64_t t0 = g0 + start;
    const int64_t tile = ((s_slot[kBlock - 1 + start] >> 4) * hkv + h) * (kBlock * D);
    const int32_t kt = i & 15, kc = i >> 4;
    store16(k_cache + tile + 8 * i, load16(k + (t0 + kt) * row + h * D + 8 * kc));
    const int32_t quad = i / (D / 2), m = i % (D / 2);
    const uint16_t* vs = v + (t0 + 4 * quad) * row + h * D + 2 * m;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = *reinterpret_cast<const uint32_t*>(vs + j * row);
    // [dim 2m][token 4quad .. +3], then [dim 2m + 1][...]
    const u32x4 out = {(w[0] & 0xffffu) | (w[1] << 16), (w[2] & 0xffffu) | (w[3] << 16),
                       (w[0] >> 16) | (w[1] & 0xffff0000u), (w[2] >> 16) | (w[3] & 0xffff0000u)};
    store16(v_cache + tile + 8 * i, out);
  }
  // the group's other tokens, one (token, 8-dim chunk) per thread
  if (i >= kBlock * kChunks) return;
  const int32_t r = i / kChunks;                 // token g0 + r
  const int32_t c = i % kChunks;
  if (r < covered_prev || (start >= 0 && r >= start)) return;
  const int64_t t = g0 + r;
  if (t >= num_tokens) return;
  const int64_t slot = s_slot[kBlock - 1 + r];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot >> 4;
  const int32_t off = static_cast<int32_t>(slot & 15);
  const int64_t src = t * row + h * D + 8 * c;
  const int64_t tile = (blk * hkv + h) * (kBlock * D);
  store16(k_cache + tile + (static_cast<int64_t>(c) * kBlock + off) * 8, load16(k + src));
  const u16x8 vv = __builtin_bit_cast(u16x8, load16(v + src));
  uint16_t* vdst = v_cache + tile + (static_cast<int64_t>(off >> 2) * D + 8 * c) * 4 + (off & 3);
#pragma unroll
  for (int e = 0; e < 8; ++e) vdst[4 * e] = vv[e];
}

// FP8 pools: the same thread map; the 8 dims of a thread are 8 consecutive bytes
// of the K tile (one 8-byte store) and 8 scattered bytes of the V tile.
template <class E, int D>
__global__ __launch_bounds__(256) void cache_write8_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int64_t* __restrict__ slots, uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
    const float* __restrict__ k_scales, const float* __restrict__ v_scales, int32_t num_tokens,
    int32_t hkv, int64_t num_slots) {
  constexpr int kChunks = D / 8;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per_token = static_cast<int64_t>(hkv) * kChunks;
  if (idx >= static_cast<int64_t>(num_tokens) * per_token) return;
  const int64_t t = idx / per_token;
  const int32_t rem = static_cast<int32_t>(idx - t * per_token);
  const int32_t h = rem / kChunks;
  const int32_t c = rem - h * kChunks;
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot >> 4;
  const int32_t off = static_cast<int32_t>(slot & 15);
  const int64_t src = (t * hkv + h) * D + 8 * c;
  const int64_t tile = (blk * hkv + h) * (kBlock * D);
  const float ks = k_scales[h], vs = v_scales[h];
  const u16x8 kv = __builtin_bit_cast(u16x8, load16(k + src));
  const u16x8 vv = __builtin_bit_cast(u16x8, load16(v + src));
  // K: dims 8c .. 8c+7 = group c / 8 of 64, quad c % 4, half (c % 8) / 4
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    lo |= fp8_code(E::to_float(kv[e]), ks) << (8 * e);
    hi |= fp8_code(E::to_float(kv[e + 4]), ks) << (8 * e);
  }
  const int64_t kb = (((static_cast<int64_t>(c / 8) * kBlock + off) * 4 + c % 4) * 2 + (c % 8) / 4) * 8;
  *reinterpret_cast<uint2*>(k_cache + tile + kb) = uint2{lo, hi};
  // V: dim d = 8c + e sits at [t/4][d/64][(d%32)/2][(d%64)/32][d%2][t%4]
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int32_t d = 8 * c + e;
    const int64_t vb = ((((static_cast<int64_t>(off >> 2) * (D / 64) + d / 64) * 16 + (d % 32) / 2) * 2 +
                         (d % 64) / 32) * 2 + (d & 1)) * 4 + (off & 3);
    v_cache[tile + vb] = static_cast<uint8_t>(fp8_code(E::to_float(vv[e]), vs));
  }
}

// ---- block copy ------------------------------------------------------------------
// grid.y = pair, grid.x strides over the 16-byte vectors of one block in both pools.
// Whole-block copies from one pool pair to another (the same pools for
// copy-on-write, device and host pools for swapping): workgroup column y copies
// pair y, 16 bytes of K and of V per thread per step.
__global__ __launch_bounds__(256) void block_copy_kernel(
    const int32_t* __restrict__ pairs, const u32x4* src_k, const u32x4* src_v, u32x4* dst_k,
    u32x4* dst_v, int64_t vecs_per_block, int32_t src_blocks, int32_t dst_blocks) {
  const int32_t src = pairs[2 * blockIdx.y];
  const int32_t dst = pairs[2 * blockIdx.y + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const u32x4* ks = src_k + src * vecs_per_block;
  const u32x4* vs = src_v + src * vecs_per_block;
  u32x4* kd = dst_k + dst * vecs_per_block;
  u32x4* vd = dst_v + dst * vecs_per_block;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < vecs_per_block;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const u32x4 a = ks[i];
    const u32x4 b = vs[i];
    kd[i] = a;
    vd[i] = b;
  }
}

// ---- decode: attention pass --------------------------------------------------------
struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;
  const int32_t* ctx_lens;
  uint16_t* out;
  uint16_t* k_dst;             // the pools again, for the fused store of the new tokens
  uint16_t* v_dst;
  const uint16_t* k_new;       // [B][Hkv][D] new tokens, or NULL: no fused store
  const uint16_t* v_new;
  const int64_t* new_slots;    // [B]
  const float* k_scales;       // FP8 pools: [Hkv] scales of K and of V
  const float* v_scales;
  int32_t* counters; // [B][Hkv] partitions finished, or NULL: the merge is a separate launch
  int32_t* claim;    // list positions handed out so far, or NULL: workgroup i takes position i
  int32_t claim_base; // workgroups below this id take their id as position (the first round)
  float2* ws_ml;     // [B][H][P] (max in log2 units, sum)
  float* ws_acc;     // [B][H][P][D] unnormalised output
  int32_t num_seqs, num_heads, num_kv_heads, group;
  int32_t max_blocks, max_ctx, num_blocks, max_parts;
  int32_t part_blocks;  // blocks per partition (32 .. 256)
  int32_t part_shift;   // log2(part_blocks)
  int32_t head_groups;  // work items per (sequence, partition): num_kv_heads >> heads_shift
  int32_t heads_shift;  // log2 of the KV heads one item covers (0, 1 or 2)
  float scale_log2;     // scale * log2(e)
};

// Stores and loads of partition states that another workgroup of the same launch
// reads: agent-scope relaxed atomics, which stay coherent across the XCDs' L2
// caches without any cache-wide write-back or invalidation (agent-scope fences
// do both and made the pass several times slower).
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this thread's stores are performed (vmcnt counts stores on gfx9).
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ int32_t wave_sum_i(int32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ int32_t wave_incl_scan_i(int32_t x, int32_t lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}
// Lane holding the k-th (0-based) set bit of `mask`.
__device__ __forceinline__ int32_t kth_set_lane(uint64_t mask, int32_t k, int32_t lane) {
  const bool mine = ((mask >> lane) & 1) && __popcll(mask & ((1ull << lane) - 1)) == k;
  return __ffsll(static_cast<unsigned long long>(__ballot(mine))) - 1;
}

// How a sequence splits into work items: `nfull` partitions of 2^pbs blocks,
// then at most one shorter partition whose size class (0 .. kClasses - 1, in
// steps of 1/kClasses of a partition) is `cls`, or -1 when there is none.  A context length outside
// [1, max_ctx] is one item of class 0 (its workgroup writes NaN); a lane past
// the last sequence (live == false) has no items.
__device__ __forceinline__ void seq_items(int32_t ctx, bool live, int32_t max_ctx, int32_t pbs,
                                          int32_t* nfull, int32_t* cls) {
  if (!live) {
    *nfull = 0;
    *cls = -1;
    return;
  }
  if (ctx < 1 || ctx > max_ctx) {
    *nfull = 0;
    *cls = 0;
    return;
  }
  const int32_t nblk = (ctx + kBlock - 1) / kBlock;
  *nfull = nblk >> pbs;
  const int32_t rem = nblk & ((1 << pbs) - 1);
  *cls = rem ? (kClasses * rem) >> pbs : -1;
}

// Context lengths are read kPlanChunks x 64 at a time: all loads of a group are
// in flight together, and for up to 256 sequences the second pass reuses them.
constexpr int kPlanChunks = 4;
__device__ __forceinline__ void load_ctx_group(const DecodeArgs& a, int32_t c0, int32_t lane,
                                               int32_t cv[kPlanChunks]) {
#pragma unroll
  for (int k = 0; k < kPlanChunks; ++k) {
    const int32_t i = c0 + 64 * k + lane;
    cv[k] = i < a.num_seqs ? a.ctx_lens[i] : 0;
  }
}

// Work item of this workgroup.  Every partition of every sequence and group of
// 2^heads_shift KV heads is one item (*okvh returns the group); the list holds the
// full partitions first, ordered (KV head group, sequence, partition), then the
// last, shorter partitions from the largest size class to the smallest, ordered
// (KV head group, sequence) within a class -- big items start
// first so the short ones fill the tail.  Workgroup i takes list position i: the
// 8 XCDs take workgroup ids in turn, so each XCD gets every 8th item of the
// size-ordered list and about an eighth of the bytes.  (Giving each XCD 8
// consecutive positions of every 64 instead left half of them 10% more bytes on
// the 70B-shaped layer, and its pass ended with the slowest.)  Returns false for a workgroup
// beyond the list (the launch is sized for the longest possible list).  Every
// lane of every wave computes the same answer from the context lengths; the
// item's context length comes back in *octx.
template <class PosFn>
__device__ bool plan_item(const DecodeArgs& a, int32_t lane, PosFn list_position, int32_t* ob,
                          int32_t* okvh, int32_t* op, int32_t* octx) {
  const int32_t B = a.num_seqs, pbs = a.part_shift, hkv = a.head_groups;
  constexpr int32_t kGroup = 64 * kPlanChunks;
  int32_t cv0[kPlanChunks];            // the first group, kept for the second pass
  load_ctx_group(a, 0, lane, cv0);
  int32_t nfull_tot = 0, n_part = 0;
  int32_t cnt = 0;                     // lane c: sequences whose last partition has class c
  for (int32_t c0 = 0; c0 < B; c0 += kGroup) {
    int32_t cv[kPlanChunks];
    if (c0 == 0) {
#pragma unroll
      for (int k = 0; k < kPlanChunks; ++k) cv[k] = cv0[k];
    } else {
      load_ctx_group(a, c0, lane, cv);
    }
#pragma unroll
    for (int k = 0; k < kPlanChunks; ++k) {
      int32_t nf, cl;
      seq_items(cv[k], c0 + 64 * k + lane < B, a.max_ctx, pbs, &nf, &cl);
      nfull_tot += wave_sum_i(nf);
      n_part += __popcll(__ballot(cl >= 0));
#pragma unroll 1
      for (int32_t c = 0; c < kClasses; ++c) {
        const int32_t nc = __popcll(__ballot(cl == c));
        cnt += lane == c ? nc : 0;
      }
    }
  }
  const int32_t n_full = nfull_tot * hkv;
  const int32_t n_items = n_full + n_part * hkv;
  const int32_t i = list_position();
  if (i >= n_items) return false;

  // Second pass: find the item's sequence.  In the full-partition part the
  // target is the j-th full partition in sequence order; in the class part, the
  // k-th sequence of class cls.
  const bool full = i < n_full;
  int32_t kvh, j = 0, cls = -1, k = 0;
  if (full) {
    kvh = i / nfull_tot;
    j = i - kvh * nfull_tot;
  } else {
    // classes from the largest down; r indexes into class cls
    int32_t r = i - n_full;
    int32_t ccount = 0;
    for (int32_t c = kClasses - 1; c >= 0; --c) {
      const int32_t cc = __builtin_amdgcn_readlane(cnt, c);
      if (r < cc * hkv) {
        cls = c;
        ccount = cc;
        break;
      }
      r -= cc * hkv;
    }
    kvh = r / ccount;
    k = r - kvh * ccount;
  }
  int32_t base = 0;
  for (int32_t c0 = 0; c0 < B; c0 += kGroup) {
    int32_t cv[kPlanChunks];
    if (c0 == 0) {
#pragma unroll
      for (int u = 0; u < kPlanChunks; ++u) cv[u] = cv0[u];
    } else {
      load_ctx_group(a, c0, lane, cv);
    }
#pragma unroll
    for (int u = 0; u < kPlanChunks; ++u) {
      int32_t nf, cl;
      seq_items(cv[u], c0 + 64 * u + lane < B, a.max_ctx, pbs, &nf, &cl);
      uint64_t hit;
      int32_t part = 0;
      if (full) {
        const int32_t incl = base + wave_incl_scan_i(nf, lane);
        hit = __ballot(incl - nf <= j && j < incl);
        if (hit) {
          const int32_t l = __ffsll(static_cast<unsigned long long>(hit)) - 1;
          part = j - (__shfl(incl, l) - __shfl(nf, l));
        }
        base = __shfl(incl, 63);
      } else {
        const uint64_t m = __ballot(cl == cls);
        const int32_t pc = __popcll(m);
        hit = 0;
        if (k < pc) {
          hit = 1ull << kth_set_lane(m, k, lane);
          part = __shfl(nf, __ffsll(static_cast<unsigned long long>(hit)) - 1);
        }
        k -= pc;
      }
      if (hit) {
        const int32_t l = __ffsll(static_cast<unsigned long long>(hit)) - 1;
        *ob = c0 + 64 * u + l;
        *okvh = kvh;
        *op = part;
        *octx = __shfl(cv[u], l);
        return true;
      }
    }
  }
  return false;     // not reached
}

// Registers for three waves per SIMD: 162-163 at head dim 128 on 16-bit pools, 130-132 on
// FP8 pools (no spills), and 34 KB of LDS per workgroup.  Held to 128 registers (four
// waves), the FP8 form spills and its steps took 84 against 81 us.  On 16-bit pools at
// head dim 128 the launch pads LDS so that two workgroups share a CU (launch_attn_t).
template <class E, int D, bool kStream, bool kFp8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3)))
void decode_attn_kernel(DecodeArgs a) {
  constexpr int KK = D / 32;        // 16x16x32 steps for q.K^T; also 16-byte V loads per lane
  constexpr int LW = kFp8 ? KK / 2 : KK;   // 16-byte loads per lane per tile (FP8: half)
  constexpr int64_t kTileBytes = static_cast<int64_t>(kBlock) * D * (kFp8 ? 1 : 2);
  constexpr int MT = D / 16;        // output tiles of 16 dims
  constexpr int kLdsStride = D + 4; // floats per head row in LDS (staggers banks)
  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];
  __shared__ __attribute__((aligned(16))) float s_acc[kWaves][16 * kLdsStride];

  const int32_t tid = threadIdx.x;
  const int32_t w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t lane = tid & 63;
  [[maybe_unused]] uint64_t t_entry = 0, t_plan = 0, t_first = 0, t_loop = 0;
  TL_STAMP(t_entry);
  // The workgroup's place in the item list.  The first round (ids below claim_base, one
  // per workgroup slot of the device) takes its id; a later workgroup, with a claim
  // counter, takes the next unclaimed place after them, so that whichever slot frees
  // first (on whichever XCD) takes the next-largest item.  The claim is issued before
  // the plan's loads and waited for after them; the workgroup that takes the last place
  // resets the counter.
  __shared__ int32_t s_pos;
  const int32_t base = a.claim_base;
  const bool claims = a.claim != nullptr && static_cast<int32_t>(blockIdx.x) >= base;
  int32_t claimed = 0;
  if (claims && tid == 0)
    claimed = __hip_atomic_fetch_add(a.claim, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  auto list_position = [&]() -> int32_t {
    if (!claims) return static_cast<int32_t>(blockIdx.x);
    if (tid == 0) {
      s_pos = base + claimed;
      if (claimed == static_cast<int32_t>(gridDim.x) - base - 1)
        __hip_atomic_store(a.claim, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    return s_pos;
  };
  int32_t b, kg, p, ctx;
  if (!plan_item(a, lane, list_position, &b, &kg, &p, &ctx)) return;
  TL_STAMP(t_plan);
  b = __builtin_amdgcn_readfirstlane(b);
  kg = __builtin_amdgcn_readfirstlane(kg);
  p = __builtin_amdgcn_readfirstlane(p);
  ctx = __builtin_amdgcn_readfirstlane(ctx);
  const int32_t G = a.group;
  const int32_t PB = a.part_blocks;
  // The item covers KV heads kg * hpi .. + hpi - 1; each has wph = 4 / hpi waves, and
  // this wave works on head kvh with the other waves of that head.
  const int32_t hsh = a.heads_shift;
  const int32_t hpi = 1 << hsh;           // KV heads of the item
  const int32_t wsh = 2 - hsh;            // log2(waves per head)
  const int32_t wph = 1 << wsh;
  const int32_t hl = w >> wsh;            // this wave's head within the item
  const int32_t wi = w & (wph - 1);       // this wave among its head's waves
  const int32_t kvh = kg * hpi + hl;

  if (b >= a.num_seqs || kg >= a.head_groups) return;   // cannot happen; keeps every read in bounds
  const bool bad_ctx = ctx < 1 || ctx > a.max_ctx;
  const int32_t nparts = bad_ctx ? 1 : (ctx + PB * kBlock - 1) / (PB * kBlock);
  if (p < 0 || p >= nparts) return;
  const int32_t n = lane & 15;       // query head within the group (MFMA column)
  const int32_t g4 = lane >> 4;      // token quad within a block (MFMA row group)
  const int32_t rows = hpi * G;      // output rows of the item: heads kg * hpi * G .. + rows - 1
  const int64_t item_row0 = (static_cast<int64_t>(b) * a.num_heads + kg * rows) * D;
  const int64_t q_row0 = (static_cast<int64_t>(b) * a.num_heads + kvh * G) * D;   // this wave's

  if (bad_ctx) {
    for (int32_t i = tid; i < rows * D; i += kThreads) a.out[item_row0 + i] = E::kNaN;
    return;
  }
  const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_blocks;

  // q fragments: B operand of q.K^T, dims 32kk + 8*g4 .. +7 of head n (zero for n >= G)
  u32x4 qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    qf[kk] = (n < G) ? load16(a.q + q_row0 + static_cast<int64_t>(n) * D + 32 * kk + 8 * g4)
                     : u32x4{0, 0, 0, 0};
  }

  // This wave's blocks are first, first + wph, ... below jend (at most PB / wph of them).
  const int32_t nblk = (ctx + kBlock - 1) / kBlock;
  const int32_t jend = min(nblk, (p + 1) * PB);
  const int32_t first = p * PB + wi;
  const int32_t nw = first < jend ? (jend - first + wph - 1) >> wsh : 0;
  const int64_t tile_elems = static_cast<int64_t>(kBlock) * D;
  const int64_t head_off = static_cast<int64_t>(kvh) * tile_elems;
  const int64_t blk_stride = static_cast<int64_t>(a.num_kv_heads) * tile_elems;
  const int64_t head_off_b = static_cast<int64_t>(kvh) * kTileBytes;
  const int64_t blk_stride_b = static_cast<int64_t>(a.num_kv_heads) * kTileBytes;
  // FP8 pools: the scales fold into the score (K) and the output (V)
  const float score_scale = kFp8 ? a.scale_log2 * a.k_scales[kvh] : a.scale_log2;

  // All of the wave's block ids in one load: lane i holds the id of its i-th block,
  // so no table read sits between two tile loads.
  int32_t ids = 0;
  if (lane < nw) ids = bt[first + wph * lane];
  const bool id_bad = lane < nw && (ids < 0 || ids >= a.num_blocks);
  if (id_bad) ids = 0;

  // Fused store of the step's new token (pa_decode_fused).  The sequence's last
  // position sits in its last block, the st_i-th block of one wave of the last
  // partition's workgroup.  That wave loads the token's K and V
  // fragments alongside q, puts them into the loaded tile in registers (the
  // cache still holds the old bytes there when the tile is read) and stores them
  // into the cache from the same registers and addresses.  No other workgroup
  // reads that position.  A slot that is not the sequence's last position is not
  // written and poisons the sequence's output; a negative slot stores nothing.
  // The fragments wait in the wave's (not yet used) LDS combine area.  FP8 pools:
  // the fragments are quantised (the codes of the cache write) before they wait,
  // and the codes are put into the loaded code tiles.
  bool st_on = false, slot_bad = false;
  int32_t st_i = -1, st_off = 0;
  u32x4* st_k = reinterpret_cast<u32x4*>(&s_acc[w][0]) + lane * KK;          // [64][KK]
  uint32_t* st_v = reinterpret_cast<uint32_t*>(&s_acc[w][0]) + 64 * 4 * KK + lane * KK;
  u32x4 kpatch[KK];
  uint32_t vpatch[KK];
  if (a.new_slots != nullptr && p == nparts - 1) {
    const int64_t slot = a.new_slots[b];
    const int32_t jl = nblk - 1 - p * PB;       // last block, within the partition
    if (slot >= 0 && (jl & (wph - 1)) == wi) {
      st_i = jl >> wsh;
      st_off = (ctx - 1) % kBlock;
      const int32_t phys = __builtin_amdgcn_readlane(ids, st_i);
      const bool phys_bad = __builtin_amdgcn_readlane(id_bad ? 1 : 0, st_i) != 0;
      st_on = !phys_bad && slot == static_cast<int64_t>(phys) * kBlock + st_off;
      slot_bad = !st_on;
      const int64_t src = (static_cast<int64_t>(b) * a.num_kv_heads + kvh) * D;
      if (st_on && n == st_off) {
        if constexpr (kFp8) {
          // the lane's K codes: dims 64pp + 8g4 .. +7, then 64pp + 32 + 8g4 .. +7
#pragma unroll
          for (int pp = 0; pp < LW; ++pp) {
            kpatch[2 * pp] = load16(a.k_new + src + 64 * pp + 8 * g4);
            kpatch[2 * pp + 1] = load16(a.k_new + src + 64 * pp + 32 + 8 * g4);
          }
        } else {
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) kpatch[kk] = load16(a.k_new + src + 32 * kk + 8 * g4);
        }
      }
      if (st_on && g4 == (st_off >> 2)) {
        if constexpr (kFp8) {
          // the lane's V codes: dims (64qq + 2n, +1), then (64qq + 32 + 2n, +1)
#pragma unroll
          for (int qq = 0; qq < LW; ++qq) {
            vpatch[2 * qq] = *reinterpret_cast<const uint32_t*>(a.v_new + src + 64 * qq + 2 * n);
            vpatch[2 * qq + 1] = *reinterpret_cast<const uint32_t*>(a.v_new + src + 64 * qq + 32 + 2 * n);
          }
        } else {
#pragma unroll
          for (int j2 = 0; j2 < KK; ++j2)
            vpatch[j2] = *reinterpret_cast<const uint32_t*>(a.v_new + src + 32 * j2 + 2 * n);
        }
      }
    }
  }
  const bool bad_blk = __ballot(id_bad) != 0 || slot_bad;
  // FP8: the codes of two 16-bit values (a word) and of two words, low byte first
  auto code2 = [](uint32_t x, float sc) {
    return fp8_code(E::to_float(static_cast<uint16_t>(x & 0xffff)), sc) |
           fp8_code(E::to_float(static_cast<uint16_t>(x >> 16)), sc) << 8;
  };
  auto code4 = [&](uint32_t x, uint32_t y, float sc) { return code2(x, sc) | code2(y, sc) << 16; };
  auto stash_patch = [&]() {   // after the first tile loads are issued
    if (st_on && n == st_off) {
      if constexpr (kFp8) {
        const float ks = a.k_scales[kvh];
#pragma unroll
        for (int pp = 0; pp < LW; ++pp)
          st_k[pp] = u32x4{code4(kpatch[2 * pp][0], kpatch[2 * pp][1], ks),
                           code4(kpatch[2 * pp][2], kpatch[2 * pp][3], ks),
                           code4(kpatch[2 * pp + 1][0], kpatch[2 * pp + 1][1], ks),
                           code4(kpatch[2 * pp + 1][2], kpatch[2 * pp + 1][3], ks)};
      } else {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) st_k[kk] = kpatch[kk];
      }
    }
    if (st_on && g4 == (st_off >> 2)) {
      if constexpr (kFp8) {
        // codes of dims (2n, 2n + 1) of both halves: the (half, parity) order of a word
        const float vs = a.v_scales[kvh];
#pragma unroll
        for (int qq = 0; qq < LW; ++qq) st_v[qq] = code4(vpatch[2 * qq], vpatch[2 * qq + 1], vs);
      } else {
#pragma unroll
        for (int j2 = 0; j2 < KK; ++j2) st_v[j2] = vpatch[j2];
      }
    }
  };

  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x4 acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 kb[2][LW], vb[2][LW];     // 16-bit pools: the operands themselves; FP8: raw codes

  // Tiles are read with buffer loads whose resource covers exactly the tile; a
  // step past the wave's last block (i >= nw) gets an empty range, so its loads
  // return zeros without touching memory and the loop needs no branch.
  auto load_block = [&](int buf, int32_t i) {
    const int32_t phys = __builtin_amdgcn_readlane(ids, min(i, nw - 1));
    const int32_t bytes = i < nw ? static_cast<int32_t>(kTileBytes) : 0;
    const auto kr = tile_rsrc(reinterpret_cast<const char*>(a.k_cache) + phys * blk_stride_b + head_off_b, bytes);
    const auto vr = tile_rsrc(reinterpret_cast<const char*>(a.v_cache) + phys * blk_stride_b + head_off_b, bytes);
    if constexpr (kFp8) {
      // K: dims 64pp + 8g4 .. +7 and 64pp + 32 + 8g4 .. +7 of token n; V: dims
      // (64qq + 2n, +1) and (64qq + 32 + 2n, +1) of tokens 4g4 .. +3
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

  // Block i of the wave; i >= nw is a padding step whose positions are all masked,
  // which leaves m_run, l_run and acc unchanged (m_run is finite by then).
  auto compute_block = [&](int buf, int32_t i) {
    if (kFp8 && st_on && i == st_i) {
      const int32_t phys = __builtin_amdgcn_readlane(ids, i);
      char* kt8 = reinterpret_cast<char*>(a.k_dst) + phys * blk_stride_b + head_off_b;
      char* vt8 = reinterpret_cast<char*>(a.v_dst) + phys * blk_stride_b + head_off_b;
      if (n == st_off) {          // K codes of token st_off: 16 dims per lane per step
#pragma unroll
        for (int pp = 0; pp < LW; ++pp) {
          kb[buf][pp] = st_k[pp];
          *reinterpret_cast<u32x4*>(kt8 + ((pp * 16 + n) * 4 + g4) * 16) = kb[buf][pp];
        }
      }
      if (g4 == (st_off >> 2)) {  // V: byte st_off % 4 of each (half, parity) word
        const int32_t e = st_off & 3;
#pragma unroll
        for (int qq = 0; qq < LW; ++qq) {
          const uint32_t c = st_v[qq];
          u32x4 wv = vb[buf][qq];
          char* vd = vt8 + ((g4 * (D / 64) + qq) * 16 + n) * 16 + e;
#pragma unroll
          for (int hp = 0; hp < 4; ++hp) {
            const uint32_t code = (c >> (8 * hp)) & 0xffu;
            wv[hp] = (wv[hp] & ~(0xffu << (8 * e))) | (code << (8 * e));
            vd[4 * hp] = static_cast<char>(code);
          }
          vb[buf][qq] = wv;
        }
      }
    }
    if (!kFp8 && st_on && i == st_i) {
      const int32_t phys = __builtin_amdgcn_readlane(ids, i);
      uint16_t* kt = a.k_dst + phys * blk_stride + head_off;
      uint16_t* vt = a.v_dst + phys * blk_stride + head_off;
      if (n == st_off) {          // K row st_off: 8 dims per lane per step
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          kb[buf][kk] = st_k[kk];
          store16(kt + (kk * 64 + lane) * 8, kb[buf][kk]);
        }
      }
      if (g4 == (st_off >> 2)) {  // V column st_off: dims 2n, 2n + 1 per lane per step
        const int32_t e = st_off & 3;
#pragma unroll
        for (int j2 = 0; j2 < KK; ++j2) {
          u16x8 vv = __builtin_bit_cast(u16x8, vb[buf][j2]);
          const uint32_t pv = st_v[j2];
          vv[e] = static_cast<uint16_t>(pv & 0xffff);
          vv[e + 4] = static_cast<uint16_t>(pv >> 16);
          vb[buf][j2] = __builtin_bit_cast(u32x4, vv);
          uint16_t* vd = vt + ((g4 * D) + 32 * j2 + 2 * n) * 4 + e;
          vd[0] = vv[e];
          vd[4] = vv[e + 4];
        }
      }
    }
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
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) s = E::mfma_qk(K[kk], qf[kk], s);
    const int32_t valid = i < nw ? ctx - (first + wph * i) * kBlock : 0;   // tokens in context
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[r] = s[r] * score_scale;
      if (valid < kBlock && 4 * g4 + r >= valid) sv[r] = -INFINITY;
    }
    float bmax = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    const float m_new = fmaxf(m_run, bmax);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    u16x4 pb;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pb[r] = E::from_float(fast_exp2(sv[r] - m_new));
      psum += E::to_float(pb[r]);
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[i] *= alpha;
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
#pragma unroll
    for (int j2 = 0; j2 < KK; ++j2) {
      const u16x8 vv = __builtin_bit_cast(u16x8, V[j2]);
      const u16x4 lo = {vv[0], vv[1], vv[2], vv[3]};
      const u16x4 hi = {vv[4], vv[5], vv[6], vv[7]};
      acc[2 * j2] = E::mfma_pv(lo, pb, acc[2 * j2]);
      acc[2 * j2 + 1] = E::mfma_pv(hi, pb, acc[2 * j2 + 1]);
    }
  };

  // Two register buffers; every step issues the next block's loads before it
  // computes the current one.  The loads are unconditional (the index is clamped
  // to the last block, which then comes from L2) so the wait before each compute
  // covers exactly the older buffer.
  // The scheduling barriers keep the compiler from sinking a prefetch below the
  // first wait of the compute that follows it.
  if (nw > 0) {
    load_block(0, 0);
    stash_patch();
    for (int32_t i = 0; i < nw; i += 2) {
      load_block(1, i + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute_block(0, i);
#ifdef PA_TIMELINE
      if (i == 0) TL_STAMP(t_first);
#endif
      load_block(0, i + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute_block(1, i + 1);
    }
  }
  TL_STAMP(t_loop);

  // ---- combine the four waves of the workgroup in LDS ----
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (g4 == 0) {
    s_m[w][n] = m_run;
    s_l[w][n] = l_run;
  }
  // any wave that met an out-of-range block id poisons the whole result
  __shared__ int s_bad;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (bad_blk) s_bad = 1;
  // the waves of this wave's head
  float M = -INFINITY;
  for (int u = hl * wph; u < (hl + 1) * wph; ++u) M = fmaxf(M, s_m[u][n]);
  const float wscale = fast_exp2(m_run - M);   // 0 for a wave that saw no block
  if (n < G) {
    float* row = &s_acc[w][n * kLdsStride];
#pragma unroll
    for (int j2 = 0; j2 < KK; ++j2) {
      const f32x4 e = acc[2 * j2] * wscale;
      const f32x4 o = acc[2 * j2 + 1] * wscale;
      float* dst = row + 32 * j2 + 8 * g4;
      *reinterpret_cast<f32x4*>(dst) = f32x4{e[0], o[0], e[1], o[1]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{e[2], o[2], e[3], o[3]};
    }
  }
  __syncthreads();
  const bool poisoned = s_bad != 0;

  // each thread finishes 4 consecutive dims of one query head of the item: row hr is
  // column hh of the item's head h2, whose waves are h2 * wph .. + wph - 1
  for (int32_t i4 = tid; i4 < rows * (D / 4); i4 += kThreads) {
    const int32_t hr = i4 / (D / 4);
    const int32_t d = (i4 - hr * (D / 4)) * 4;
    const int32_t h2 = hr / G;
    const int32_t hh = hr - h2 * G;
    const int32_t u0 = h2 * wph;
    float Mh = -INFINITY;
    for (int u = u0; u < u0 + wph; ++u) Mh = fmaxf(Mh, s_m[u][hh]);
    float L = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    for (int u = u0; u < u0 + wph; ++u) {
      L += s_l[u][hh] * fast_exp2(s_m[u][hh] - Mh);
      o += *reinterpret_cast<const f32x4*>(&s_acc[u][hh * kLdsStride + d]);
    }
    if (kFp8) o *= a.v_scales[kg * hpi + h2];   // V codes stand for code * v_scale
    const int64_t row = item_row0 + static_cast<int64_t>(hr) * D;
    if (nparts == 1) {
      u16x4 ov;
      if (poisoned) {
        ov = u16x4{E::kNaN, E::kNaN, E::kNaN, E::kNaN};
      } else {
        const float inv = 1.f / L;
#pragma unroll
        for (int r = 0; r < 4; ++r) ov[r] = E::from_float(o[r] * inv);
      }
      *reinterpret_cast<u16x4*>(a.out + row + d) = ov;
    } else {
      const int64_t st = (static_cast<int64_t>(b) * a.num_heads + kg * rows + hr) * a.max_parts + p;
      if (poisoned) o = f32x4{NAN, NAN, NAN, NAN};
      const float2 ml = poisoned ? float2{0.f, NAN} : float2{Mh, L};
      if (a.counters) {
        // read by another workgroup of this launch: device-coherent stores
#pragma unroll
        for (int r = 0; r < 4; ++r) store_coherent(a.ws_acc + st * D + d + r, o[r]);
        if (d == 0) {
          store_coherent(&a.ws_ml[st].x, ml.x);
          store_coherent(&a.ws_ml[st].y, ml.y);
        }
      } else {
        *reinterpret_cast<f32x4*>(a.ws_acc + st * D + d) = o;
        if (d == 0) a.ws_ml[st] = ml;
      }
    }
  }
#ifdef PA_TIMELINE
  if (tid == 0 && blockIdx.x < PA_TIMELINE_MAX_WORKGROUPS) {
    uint64_t t_out;
    TL_STAMP(t_out);
    const uint32_t xcc = __builtin_amdgcn_s_getreg(0x1814);   // XCC_ID, bits 3:0
    const uint32_t hw = __builtin_amdgcn_s_getreg(0xf804);    // HW_ID, all 32 bits
    uint64_t* r = g_timeline + static_cast<uint64_t>(blockIdx.x) * PA_TIMELINE_WORDS;
    r[0] = t_entry;
    r[1] = t_plan;
    r[2] = t_first;
    r[3] = t_loop;
    r[4] = t_out;
    r[5] = (static_cast<uint64_t>(b) << 32) | static_cast<uint32_t>(p);
    r[6] = (static_cast<uint64_t>(kg) << 32) | (static_cast<uint32_t>(nw) << 16) |
           static_cast<uint32_t>(jend - p * PB);
    r[7] = (static_cast<uint64_t>(xcc) << 32) | hw;
  }
#endif
  if (nparts == 1 || a.counters == nullptr) return;

  // Fused merge: the last of the sequence's partitions (for these KV heads) to
  // finish combines all of them.  Its partial stores are complete (waited for)
  // before the count is raised, and the merging workgroup reads the states with
  // device-coherent loads after it has seen the count reach nparts - 1.
  __shared__ int32_t s_ticket;
  wait_stores();
  __syncthreads();
  int32_t* counter = a.counters + static_cast<int64_t>(b) * a.head_groups + kg;
  if (tid == 0) s_ticket = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (s_ticket != nparts - 1) return;
  for (int32_t i4 = tid; i4 < rows * (D / 4); i4 += kThreads) {
    const int32_t hr = i4 / (D / 4);
    const int32_t d = (i4 - hr * (D / 4)) * 4;
    const int64_t st0 = (static_cast<int64_t>(b) * a.num_heads + kg * rows + hr) * a.max_parts;
    float M = -INFINITY;
    for (int32_t u = 0; u < nparts; ++u) M = fmaxf(M, load_coherent(&a.ws_ml[st0 + u].x));
    float L = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    for (int32_t u = 0; u < nparts; ++u) {
      const float wgt = fast_exp2(load_coherent(&a.ws_ml[st0 + u].x) - M);
      L += wgt * load_coherent(&a.ws_ml[st0 + u].y);
      const float* src = a.ws_acc + (st0 + u) * D + d;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] += wgt * load_coherent(src + r);
    }
    const float inv = 1.f / L;
    u16x4 ov;
#pragma unroll
    for (int r = 0; r < 4; ++r) ov[r] = E::from_float(o[r] * inv);
    *reinterpret_cast<u16x4*>(a.out + item_row0 + static_cast<int64_t>(hr) * D + d) = ov;
  }
  if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- decode: log-sum-exp merge -----------------------------------------------------
struct MergeArgs {
  const int32_t* ctx_lens;
  uint16_t* out;
  const float2* ws_ml;
  const float* ws_acc;
  int32_t num_seqs, num_heads, max_ctx, max_parts, part_tokens;
};

// One wave per (sequence, query head): M = max_p m_p, w_p = 2^(m_p - M),
// out = sum_p w_p acc_p / sum_p w_p l_p.  Lane l owns D/64 consecutive dims; the
// partitions are visited in index order, so the result does not depend on timing.
template <class E, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(MergeArgs a) {
  constexpr int V = D / 64;              // floats per lane
  const int32_t row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.num_seqs * a.num_heads) return;
  const int32_t lane = threadIdx.x & 63;
  const int32_t b = row / a.num_heads;
  const int32_t ctx = a.ctx_lens[b];
  if (ctx < 1 || ctx > a.max_ctx) return;                 // attention pass wrote NaN
  const int32_t nparts = (ctx + a.part_tokens - 1) / a.part_tokens;
  if (nparts <= 1) return;                                // attention pass wrote out
  const int64_t st0 = static_cast<int64_t>(row) * a.max_parts;
  const float2* ml = a.ws_ml + st0;

  // Every lane forms M and L itself, in partition order: the same arithmetic, in
  // the same order, as the merge inside the attention pass, so both give the
  // same bits.
  float M = -INFINITY;
  for (int32_t i = 0; i < nparts; ++i) M = fmaxf(M, ml[i].x);
  float L = 0.f;
  for (int32_t i = 0; i < nparts; ++i) {
    const float2 v = ml[i];
    L += fast_exp2(v.x - M) * v.y;
  }

  float o[V];
#pragma unroll
  for (int e = 0; e < V; ++e) o[e] = 0.f;
  const float* acc = a.ws_acc + st0 * D + lane * V;
  for (int32_t c = 0; c < nparts; c += 64) {
    const int32_t cnt = min(64, nparts - c);
    const float wl = lane < cnt ? fast_exp2(ml[c + lane].x - M) : 0.f;
    int32_t i = 0;
    for (; i + 4 <= cnt; i += 4) {
      float t[4][V];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < V; ++e) t[u][e] = acc[static_cast<int64_t>(c + i + u) * D + e];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float wgt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                        __builtin_bit_cast(int32_t, wl), i + u));
#pragma unroll
        for (int e = 0; e < V; ++e) o[e] += wgt * t[u][e];
      }
    }
    for (; i < cnt; ++i) {
      const float wgt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                      __builtin_bit_cast(int32_t, wl), i));
#pragma unroll
      for (int e = 0; e < V; ++e) o[e] += wgt * acc[static_cast<int64_t>(c + i) * D + e];
    }
  }
  const float inv = 1.f / L;
  uint16_t* dst = a.out + static_cast<int64_t>(row) * D + lane * V;
#pragma unroll
  for (int e = 0; e < V; ++e) dst[e] = E::from_float(o[e] * inv);
}

}  // namespace

namespace pa {

size_t decode_counter_bytes(int64_t num_seqs, int64_t num_heads) {
  return ((static_cast<size_t>(num_seqs) * num_heads + 1) * sizeof(int32_t) + 255) & ~size_t(255);
}

// Compute units of the current device (queried once per device).
int32_t device_cus() {
  static std::atomic<int32_t> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int32_t n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    n = v;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// ---- host-side helpers -------------------------------------------------------------
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

pa_status check_cache(const pa_cache* c, const char* fn) {
  if (!c) return pa::fail(PA_ERR_INVALID_ARG, "%s: cache is NULL", fn);
  if (!c->k_cache || !c->v_cache) return pa::fail(PA_ERR_INVALID_ARG, "%s: cache pointers are NULL", fn);
  if (!aligned16(c->k_cache) || !aligned16(c->v_cache))
    return pa::fail(PA_ERR_INVALID_ARG, "%s: cache pointers must be 16-byte aligned", fn);
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0)
    return pa::fail(PA_ERR_INVALID_ARG, "%s: num_blocks %d, num_kv_heads %d", fn, c->num_blocks, c->num_kv_heads);
  if (c->block_size != kBlock)
    return pa::fail(PA_ERR_UNSUPPORTED, "%s: block_size %d (only 16)", fn, c->block_size);
  if (c->head_dim != 64 && c->head_dim != 128)
    return pa::fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d (64 or 128)", fn, c->head_dim);
  if (c->dtype != PA_F16 && c->dtype != PA_BF16)
    return pa::fail(PA_ERR_UNSUPPORTED, "%s: dtype %d", fn, c->dtype);
  if (c->flags & ~(PA_CACHE_SHARED_BLOCKS | PA_CACHE_FP8))
    return pa::fail(PA_ERR_INVALID_ARG, "%s: unknown cache flags 0x%x", fn, c->flags);
  if ((c->flags & PA_CACHE_FP8) &&
      (!c->k_scales || !c->v_scales || (reinterpret_cast<uintptr_t>(c->k_scales) & 3u) ||
       (reinterpret_cast<uintptr_t>(c->v_scales) & 3u)))
    return pa::fail(PA_ERR_INVALID_ARG, "%s: FP8 pools need aligned k_scales and v_scales", fn);
  return PA_OK;
}

pa_status launch_status(const char* fn) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pa::fail(PA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  return PA_OK;
}

}  // namespace pa

namespace {

using pa::aligned16;
using pa::check_cache;
using pa::launch_status;
using pa::device_cus;


int32_t parts_for(int32_t max_ctx, int32_t part_tokens) {
  return (max_ctx + part_tokens - 1) / part_tokens;
}


// Partition length of one launch: the longest of 4096, 2048 and 1024 tokens for
// which even the longest possible item list gives every workgroup slot of the
// device (counted as three per compute unit, as the registers allow; 16-bit pools at
// head dim 128 run two, for which the count asks a little more) two items, else 512
// tokens.  A longer item
// spends less of its time on start-up and combine per byte it reads; two items
// per slot keep enough of them for the largest-first order to balance the slots.
int32_t part_tokens_for(int32_t num_seqs, int32_t num_kv_heads, int32_t max_ctx) {
  const int64_t slots = 3 * static_cast<int64_t>(device_cus());
  for (int32_t pt = kMaxPartTokens; pt > kPartTokens; pt /= 2) {
    const int64_t items = static_cast<int64_t>(num_seqs) * num_kv_heads * parts_for(max_ctx, pt);
    if (items >= 2 * slots) return pt;
  }
  return kPartTokens;
}

// log2 of the KV heads one decode item covers: 1 (two heads, two waves each) when
// each KV head serves one query head, the pools are 16-bit and B * Hkv / 2 *
// (partitions at 4096 tokens) items still give every workgroup slot (three per
// compute unit) 4/3 of one; else 0.  Measured on the 7B-shaped layer: 217.5 against
// 223 us; four heads per item, and two on FP8 pools, were slower.  The kernel takes
// shifts up to 2.  PA_HEADS_PER_ITEM=1 in the environment keeps one KV head per item
// (read once).
int32_t heads_shift_for(int32_t num_seqs, int32_t num_kv_heads, int32_t group, bool fp8,
                        int32_t max_ctx) {
  static const bool off = [] {
    const char* e = std::getenv("PA_HEADS_PER_ITEM");
    return e && e[0] == '1';
  }();
  if (off || group != 1 || fp8 || num_kv_heads % 2) return 0;
  const int64_t slots = 3 * static_cast<int64_t>(device_cus());
  const int64_t items = static_cast<int64_t>(num_seqs) * (num_kv_heads >> 1) *
                        parts_for(max_ctx, kMaxPartTokens);
  return 3 * items >= 4 * slots ? 1 : 0;
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }
size_t ws_ml_bytes(int64_t rows) { return round256(static_cast<size_t>(rows) * sizeof(float2)); }
// Workspace: counters int32[B][H] and the claim counter (zero between calls) |
// (max, sum) float2[rows] | acc float[rows][D]
size_t ws_counter_bytes(int64_t num_seqs, int64_t num_heads) {
  return pa::decode_counter_bytes(num_seqs, num_heads);
}
// The merge runs inside the attention pass when a sequence has at most this many partitions.
constexpr int32_t kMaxFusedParts = 8;

// PA_FUSED_MERGE=0 in the environment keeps the merge a separate launch (read once).
bool fused_merge_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("PA_FUSED_MERGE");
    return !(e && e[0] == '0');
  }();
  return on;
}

struct DecodeSetup {
  DecodeArgs args;
  int64_t grid;
  bool shared_blocks;   // read K/V through the caches
  bool fp8;             // the pools hold E4M3 codes
  bool wide_group;      // more than 16 query heads per KV head: the chunk kernels
};

// A partition length the caller may fix: 0 (chosen per launch) or 512 .. 4096 tokens,
// a power of two.
bool valid_part_tokens(int32_t pt) {
  return pt == 0 || (pt >= kPartTokens && pt <= kMaxPartTokens && (pt & (pt - 1)) == 0);
}

pa_status prepare_decode(const char* fn, const pa_cache* cache, const void* q, int32_t num_seqs,
                         int32_t num_heads, const int32_t* block_tables, int32_t max_blocks,
                         const int32_t* ctx_lens, int32_t max_ctx, float scale, void* out,
                         void* workspace, size_t workspace_bytes, bool need_q, DecodeSetup* su,
                         int32_t part_tokens = 0) {
  pa_status st = check_cache(cache, fn);
  if (st != PA_OK) return st;
  if (num_seqs < 0) return pa::fail(PA_ERR_INVALID_ARG, "%s: num_seqs %d", fn, num_seqs);
  if (num_heads <= 0 || num_heads % cache->num_kv_heads)
    return pa::fail(PA_ERR_INVALID_ARG, "%s: num_heads %d not a multiple of num_kv_heads %d", fn,
                    num_heads, cache->num_kv_heads);
  const int32_t G = num_heads / cache->num_kv_heads;
  su->wide_group = G > 16;
  if (max_ctx < 1) return pa::fail(PA_ERR_INVALID_ARG, "%s: max_context_len %d", fn, max_ctx);
  if (need_q) {
    if (max_blocks < 1 || static_cast<int64_t>(max_blocks) * kBlock < max_ctx)
      return pa::fail(PA_ERR_INVALID_ARG, "%s: max_blocks_per_seq %d cannot hold %d tokens", fn,
                      max_blocks, max_ctx);
    if (num_seqs > 0 && (!q || !block_tables || !aligned16(q)))
      return pa::fail(PA_ERR_INVALID_ARG, "%s: q / block_tables NULL or q misaligned", fn);
    if (!std::isfinite(scale)) return pa::fail(PA_ERR_INVALID_ARG, "%s: scale is not finite", fn);
  }
  if (num_seqs > 0 && (!ctx_lens || !out || !aligned16(out)))
    return pa::fail(PA_ERR_INVALID_ARG, "%s: context_lens / out NULL or out misaligned", fn);
  if (parts_for(max_ctx, kPartTokens) > kMaxParts)
    return pa::fail(PA_ERR_UNSUPPORTED, "%s: max_context_len %d too long", fn, max_ctx);
  if (!valid_part_tokens(part_tokens))
    return pa::fail(PA_ERR_INVALID_ARG, "%s: partition_tokens %d (0, or a power of two in 512 .. 4096)",
                    fn, part_tokens);
  // One query head per KV head (MHA): an item covers 2 KV heads of a sequence while
  // that still leaves every workgroup slot about 4/3 of an item, so fewer items pay
  // the start-up of one.
  const int32_t hsh = heads_shift_for(num_seqs, cache->num_kv_heads, G,
                                      (cache->flags & PA_CACHE_FP8) != 0, max_ctx);
  const int32_t groups = cache->num_kv_heads >> hsh;
  const int32_t PT = part_tokens ? part_tokens : part_tokens_for(num_seqs, groups, max_ctx);
  const int32_t P = parts_for(max_ctx, PT);
  // The workspace is sized for 512-token partitions; a launch with longer ones uses a prefix.
  const size_t need = P > 1 ? pa_decode_workspace_size(num_seqs, num_heads, cache->head_dim, max_ctx) : 0;
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return pa::fail(PA_ERR_WORKSPACE, "%s: workspace %zu bytes, %zu needed", fn, workspace_bytes, need);
  const int64_t grid = static_cast<int64_t>(P) * groups * num_seqs;
  if (grid > INT32_MAX) return pa::fail(PA_ERR_UNSUPPORTED, "%s: grid too large", fn);
  DecodeArgs& a = su->args;
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint16_t*>(cache->k_cache);
  a.v_cache = static_cast<const uint16_t*>(cache->v_cache);
  a.block_tables = block_tables;
  a.ctx_lens = ctx_lens;
  a.out = static_cast<uint16_t*>(out);
  const int64_t rows = static_cast<int64_t>(num_seqs) * num_heads * P;
  a.k_dst = static_cast<uint16_t*>(cache->k_cache);
  a.v_dst = static_cast<uint16_t*>(cache->v_cache);
  a.k_new = nullptr;
  a.v_new = nullptr;
  a.new_slots = nullptr;
  a.counters = nullptr;
  // the claim counter follows the merge counters ([B][H] words) in the counter region
  a.claim = workspace && workspace_bytes >= ws_counter_bytes(num_seqs, num_heads)
                ? static_cast<int32_t*>(workspace) + static_cast<int64_t>(num_seqs) * num_heads
                : nullptr;
  // workgroup slots of the device: two per CU on 16-bit pools at head dim 128, else three
  const bool pad = (cache->flags & PA_CACHE_FP8) == 0 && cache->head_dim == 128;
  a.claim_base = (pad ? 2 : 3) * device_cus();
  char* wsb = static_cast<char*>(workspace) + ws_counter_bytes(num_seqs, num_heads);
  a.ws_ml = need ? reinterpret_cast<float2*>(wsb) : nullptr;
  a.ws_acc = need ? reinterpret_cast<float*>(wsb + ws_ml_bytes(rows)) : nullptr;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = cache->num_kv_heads;
  a.group = G;
  a.max_blocks = max_blocks;
  a.max_ctx = max_ctx;
  a.num_blocks = cache->num_blocks;
  a.max_parts = P;
  a.part_blocks = PT / kBlock;
  a.part_shift = __builtin_ctz(static_cast<unsigned>(PT / kBlock));
  a.head_groups = groups;
  a.heads_shift = hsh;
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  a.k_scales = cache->k_scales;
  a.v_scales = cache->v_scales;
  su->grid = grid;
  su->shared_blocks = (cache->flags & PA_CACHE_SHARED_BLOCKS) != 0;
  su->fp8 = (cache->flags & PA_CACHE_FP8) != 0;
  return PA_OK;
}

// The attention launch.  Events given (hipEvent_t, may be NULL) are attached to the
// dispatch itself: they take the kernel's own start and end times, without the queue
// time around it that events recorded before and after the launch would include.
// On 16-bit pools at head dim 128 the launch reserves kOccupancyPadLds bytes of LDS it
// never uses, so that two workgroups share a compute unit instead of three.  A CU serves
// its workgroups' loads about oldest first, so the third mostly waits for its first tile
// while holding a slot; with two, the 70B-shaped layer's pass is ~1.3 % shorter and its
// step ~2 % (three alternating runs), the others even.  FP8 pools, whose waves stream half
// the bytes per tile, keep three (two were 7 % slower).
constexpr uint32_t kOccupancyPadLds = 24 * 1024;

template <class E, bool kStream, bool kFp8>
void launch_attn_t(const DecodeSetup& su, int d, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (d == 64)
    hipExtLaunchKernelGGL(decode_attn_kernel<E, 64, kStream, kFp8>, dim3(su.grid), dim3(kThreads),
                          0, s, e0, e1, 0, su.args);
  else
    hipExtLaunchKernelGGL(decode_attn_kernel<E, 128, kStream, kFp8>, dim3(su.grid), dim3(kThreads),
                          kFp8 ? 0u : kOccupancyPadLds, s, e0, e1, 0, su.args);
}

template <class E>
void launch_attn(const DecodeSetup& su, int d, hipStream_t s, hipEvent_t e0 = nullptr,
                 hipEvent_t e1 = nullptr) {
  if (su.fp8) {
    if (su.shared_blocks)
      launch_attn_t<E, false, true>(su, d, s, e0, e1);
    else
      launch_attn_t<E, true, true>(su, d, s, e0, e1);
  } else {
    if (su.shared_blocks)
      launch_attn_t<E, false, false>(su, d, s, e0, e1);
    else
      launch_attn_t<E, true, false>(su, d, s, e0, e1);
  }
}

// The separate merge launch; a stop event given (hipEvent_t, may be NULL) takes the
// merge kernel's own end time.
template <class E>
void launch_merge(const MergeArgs& m, int64_t grid, int d, hipStream_t s, hipEvent_t e1 = nullptr) {
  if (d == 64)
    hipExtLaunchKernelGGL(decode_merge_kernel<E, 64>, dim3(grid), dim3(256), 0, s, nullptr, e1, 0, m);
  else
    hipExtLaunchKernelGGL(decode_merge_kernel<E, 128>, dim3(grid), dim3(256), 0, s, nullptr, e1, 0, m);
}

template <class E>
void launch_write8_t(const pa_cache* c, const uint16_t* k, const uint16_t* v, const int64_t* slots,
                     int32_t n, int64_t num_slots, int64_t grid, hipStream_t s) {
  auto kc = static_cast<uint8_t*>(c->k_cache);
  auto vc = static_cast<uint8_t*>(c->v_cache);
  if (c->head_dim == 64)
    cache_write8_kernel<E, 64><<<dim3(grid), dim3(256), 0, s>>>(k, v, slots, kc, vc, c->k_scales,
                                                                c->v_scales, n, c->num_kv_heads, num_slots);
  else
    cache_write8_kernel<E, 128><<<dim3(grid), dim3(256), 0, s>>>(k, v, slots, kc, vc, c->k_scales,
                                                                 c->v_scales, n, c->num_kv_heads, num_slots);
}

// The quantising store of new tokens into FP8 pools (grid: one thread per 8 dims).
void launch_write8(const pa_cache* c, const uint16_t* k, const uint16_t* v, const int64_t* slots,
                   int32_t n, int64_t num_slots, int64_t grid, hipStream_t s) {
  if (c->dtype == PA_F16)
    launch_write8_t<F16>(c, k, v, slots, n, num_slots, grid, s);
  else
    launch_write8_t<BF16>(c, k, v, slots, n, num_slots, grid, s);
}

}  // namespace

namespace pa {

pa_status decode_check(const pa_cache* cache, const void* q, int32_t num_seqs, int32_t num_heads,
                       int32_t max_blocks_per_seq, int32_t max_ctx, float scale, void* out,
                       void* workspace, size_t workspace_bytes) {
  DecodeSetup su;
  const int32_t dummy_table = 0, dummy_ctx = 0;
  pa_status st = prepare_decode("pa_decode", cache, q, num_seqs, num_heads, &dummy_table,
                                max_blocks_per_seq, &dummy_ctx, max_ctx, scale, out, workspace,
                                workspace_bytes, true, &su);
  if (st != PA_OK) return st;
  const size_t need = pa_decode_workspace_size(num_seqs, num_heads, cache->head_dim, max_ctx);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return pa::fail(PA_ERR_WORKSPACE, "pa_decode: workspace %zu bytes, %zu needed for contexts up to %d",
                    workspace_bytes, need, max_ctx);
  return PA_OK;
}

// Every decode entry point: optional fused store of the new tokens (k_new != NULL),
// the attention pass (between the optional events), and the merge -- inside the
// attention pass when fuse_merge and every sequence has at most kMaxFusedParts
// partitions, else as a second launch.  merge == false stops after the attention
// pass (the partition states stay in the workspace).
pa_status decode_run(const char* fn, const pa_cache* cache, const void* q, int32_t num_seqs,
                     int32_t num_heads, const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t max_context_len, float scale, void* out,
                     void* workspace, size_t workspace_bytes, const void* k_new, const void* v_new,
                     const int64_t* slot_mapping, bool merge, bool fuse_merge,
                     int32_t part_tokens, void* ev_begin, void* ev_end, void* stream) {
  pa::clear_error();
  DecodeSetup su;
  pa_status st = prepare_decode(fn, cache, q, num_seqs, num_heads, block_tables, max_blocks_per_seq,
                                context_lens, max_context_len, scale, out, workspace,
                                workspace_bytes, true, &su, part_tokens);
  if (st != PA_OK || num_seqs == 0) return st;
  if (part_tokens && su.wide_group)
    return pa::fail(PA_ERR_UNSUPPORTED, "%s: a fixed partition length needs at most 16 query heads "
                    "per KV head", fn);
  if (k_new) {
    if (!v_new || !slot_mapping || !aligned16(k_new) || !aligned16(v_new) ||
        (reinterpret_cast<uintptr_t>(slot_mapping) & 7u))
      return pa::fail(PA_ERR_INVALID_ARG, "%s: k_new / v_new / slot_mapping NULL or misaligned", fn);
    if (su.fp8 && su.wide_group) {
      // the several-token kernels do not store: the quantising store is its own launch
      const int64_t grid = (static_cast<int64_t>(num_seqs) * cache->num_kv_heads *
                            (cache->head_dim / 8) + 255) / 256;
      launch_write8(cache, static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                    slot_mapping, num_seqs, static_cast<int64_t>(cache->num_blocks) * kBlock, grid,
                    static_cast<hipStream_t>(stream));
      st = launch_status(fn);
      if (st != PA_OK) return st;
    } else {
      su.args.k_new = static_cast<const uint16_t*>(k_new);
      su.args.v_new = static_cast<const uint16_t*>(v_new);
      su.args.new_slots = slot_mapping;
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (su.wide_group) {
    // More than 16 query heads per KV head do not fit one matrix-core tile of the
    // decode pass: the several-token kernels run with one query per sequence, their
    // partition states past the workspace counters.  A 16-bit store of new tokens is
    // then its own launch first (the slots are stored as given).
    if (k_new && !su.fp8) {
      st = pa_cache_write(cache, k_new, v_new, slot_mapping, num_seqs, stream);
      if (st != PA_OK) return st;
    }
    const size_t cb = ws_counter_bytes(num_seqs, num_heads);
    void* ws = workspace && workspace_bytes > cb ? static_cast<char*>(workspace) + cb : nullptr;
    const size_t wsb = ws ? workspace_bytes - cb : 0;
    return chunk_decode(fn, cache, q, num_seqs, num_heads, block_tables, max_blocks_per_seq,
                        context_lens, max_context_len, scale, out, ws, wsb, ev_begin, ev_end,
                        stream);
  }
  const int32_t P = su.args.max_parts;
  if (merge && fuse_merge && P > 1 && P <= kMaxFusedParts && fused_merge_enabled())
    su.args.counters = static_cast<int32_t*>(workspace);
  // The events, if any, take the attention kernel's own start and the end of the
  // last kernel of the pass: the attention kernel, or the separate merge after it.
  const bool separate_merge = merge && P > 1 && !su.args.counters;
  const hipEvent_t e0 = static_cast<hipEvent_t>(ev_begin), e1 = static_cast<hipEvent_t>(ev_end);
  if (cache->dtype == PA_F16)
    launch_attn<F16>(su, cache->head_dim, s, e0, separate_merge ? nullptr : e1);
  else
    launch_attn<BF16>(su, cache->head_dim, s, e0, separate_merge ? nullptr : e1);
  st = launch_status(fn);
  if (st != PA_OK || !separate_merge) return st;
  MergeArgs m;
  m.ctx_lens = context_lens;
  m.out = static_cast<uint16_t*>(out);
  m.ws_ml = su.args.ws_ml;
  m.ws_acc = su.args.ws_acc;
  m.num_seqs = num_seqs;
  m.num_heads = num_heads;
  m.max_ctx = max_context_len;
  m.max_parts = P;
  m.part_tokens = su.args.part_blocks * kBlock;
  const int64_t grid = (static_cast<int64_t>(num_seqs) * num_heads + 3) / 4;
  if (cache->dtype == PA_F16)
    launch_merge<F16>(m, grid, cache->head_dim, s, e1);
  else
    launch_merge<BF16>(m, grid, cache->head_dim, s, e1);
  return launch_status(fn);
}

}  // namespace pa

extern "C" {

pa_status pa_cache_write(const pa_cache* cache, const void* k, const void* v,
                         const int64_t* slot_mapping, int32_t num_tokens, void* stream) {
  pa::clear_error();
  pa_status st = check_cache(cache, "pa_cache_write");
  if (st != PA_OK) return st;
  if (num_tokens < 0) return pa::fail(PA_ERR_INVALID_ARG, "pa_cache_write: num_tokens %d", num_tokens);
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !aligned16(k) || !aligned16(v) ||
      (reinterpret_cast<uintptr_t>(slot_mapping) & 7u))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_cache_write: k / v / slot_mapping NULL or misaligned");
  const int D = cache->head_dim;
  const int64_t threads = static_cast<int64_t>(num_tokens) * cache->num_kv_heads * (D / 8);
  const int64_t grid = (threads + 255) / 256;
  if (grid > INT32_MAX) return pa::fail(PA_ERR_UNSUPPORTED, "pa_cache_write: too many tokens");
  const int64_t num_slots = static_cast<int64_t>(cache->num_blocks) * kBlock;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto kp = static_cast<const uint16_t*>(k);
  auto vp = static_cast<const uint16_t*>(v);
  if (cache->flags & PA_CACHE_FP8) {
    launch_write8(cache, kp, vp, slot_mapping, num_tokens, num_slots, grid, s);
    return launch_status("pa_cache_write");
  }
  auto kc = static_cast<uint16_t*>(cache->k_cache);
  auto vc = static_cast<uint16_t*>(cache->v_cache);
  if (num_tokens >= kBulkTokens && cache->num_kv_heads <= 65535) {
    // many tokens (a prefill, an admission): whole blocks are written tile by tile
    const dim3 g(static_cast<uint32_t>((num_tokens + kBlock - 1) / kBlock),
                 static_cast<uint32_t>(cache->num_kv_heads));
    if (D == 64)
      cache_write_bulk_kernel<64><<<g, dim3(128), 0, s>>>(kp, vp, slot_mapping, kc, vc, num_tokens,
                                                          cache->num_kv_heads, num_slots);
    else
      cache_write_bulk_kernel<128><<<g, dim3(256), 0, s>>>(kp, vp, slot_mapping, kc, vc, num_tokens,
                                                           cache->num_kv_heads, num_slots);
    return launch_status("pa_cache_write");
  }
  if (D == 64)
    cache_write_kernel<64><<<dim3(grid), dim3(256), 0, s>>>(kp, vp, slot_mapping, kc, vc, num_tokens,
                                                           cache->num_kv_heads, num_slots);
  else
    cache_write_kernel<128><<<dim3(grid), dim3(256), 0, s>>>(kp, vp, slot_mapping, kc, vc, num_tokens,
                                                            cache->num_kv_heads, num_slots);
  return launch_status("pa_cache_write");
}

pa_status pa_copy_blocks(const pa_cache* cache, const int32_t* pairs, const int32_t* pairs_host,
                         int32_t num_pairs, void* stream) {
  pa::clear_error();
  pa_status st = check_cache(cache, "pa_copy_blocks");
  if (st != PA_OK) return st;
  if (num_pairs < 0) return pa::fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: num_pairs %d", num_pairs);
  if (num_pairs == 0) return PA_OK;
  if (!pairs) return pa::fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: pairs is NULL");
  if (num_pairs > 65535) return pa::fail(PA_ERR_UNSUPPORTED, "pa_copy_blocks: more than 65535 pairs");
  if (pairs_host) {
    // destinations distinct, none also a source, all ids in range
    const int32_t nb = cache->num_blocks;
    std::vector<uint8_t> role(nb, 0);   // bit 0: source, bit 1: destination
    for (int32_t i = 0; i < num_pairs; ++i) {
      const int32_t s = pairs_host[2 * i], d = pairs_host[2 * i + 1];
      if (s < 0 || s >= nb || d < 0 || d >= nb)
        return pa::fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: pair %d (%d, %d) out of range", i, s, d);
      if (role[d] & 2) return pa::fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: destination %d repeated", d);
      role[s] |= 1;
      role[d] |= 2;
    }
    for (int32_t b = 0; b < nb; ++b)
      if (role[b] == 3) return pa::fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: block %d is source and destination", b);
  }
  const int64_t elem = (cache->flags & PA_CACHE_FP8) ? 1 : 2;
  const int64_t vecs = static_cast<int64_t>(cache->num_kv_heads) * kBlock * cache->head_dim * elem / 16;
  const int64_t gx = std::min<int64_t>((vecs + 255) / 256, 64);
  block_copy_kernel<<<dim3(gx, num_pairs), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
      pairs, static_cast<const u32x4*>(cache->k_cache), static_cast<const u32x4*>(cache->v_cache),
      static_cast<u32x4*>(cache->k_cache), static_cast<u32x4*>(cache->v_cache), vecs,
      cache->num_blocks, cache->num_blocks);
  return launch_status("pa_copy_blocks");
}

pa_status pa_swap_blocks(const pa_cache* device, const pa_cache* host, int32_t direction,
                         const int32_t* pairs, const int32_t* pairs_host, int32_t num_pairs,
                         void* stream) {
  const char* fn = "pa_swap_blocks";
  pa::clear_error();
  pa_status st = check_cache(device, fn);
  if (st != PA_OK) return st;
  st = check_cache(host, fn);
  if (st != PA_OK) return st;
  if (device->num_kv_heads != host->num_kv_heads || device->head_dim != host->head_dim ||
      device->dtype != host->dtype || ((device->flags ^ host->flags) & PA_CACHE_FP8))
    return pa::fail(PA_ERR_INVALID_ARG, "%s: device and host pools differ in layout", fn);
  if (direction != PA_SWAP_OUT && direction != PA_SWAP_IN)
    return pa::fail(PA_ERR_INVALID_ARG, "%s: direction %d", fn, direction);
  if (num_pairs < 0) return pa::fail(PA_ERR_INVALID_ARG, "%s: num_pairs %d", fn, num_pairs);
  if (num_pairs == 0) return PA_OK;
  if (!pairs) return pa::fail(PA_ERR_INVALID_ARG, "%s: pairs is NULL", fn);
  if (num_pairs > 65535) return pa::fail(PA_ERR_UNSUPPORTED, "%s: more than 65535 pairs", fn);
  const pa_cache* src = direction == PA_SWAP_OUT ? device : host;
  const pa_cache* dst = direction == PA_SWAP_OUT ? host : device;
  if (pairs_host) {
    std::vector<uint8_t> taken(dst->num_blocks, 0);
    for (int32_t i = 0; i < num_pairs; ++i) {
      const int32_t s = pairs_host[2 * i], d = pairs_host[2 * i + 1];
      if (s < 0 || s >= src->num_blocks || d < 0 || d >= dst->num_blocks)
        return pa::fail(PA_ERR_INVALID_ARG, "%s: pair %d (%d, %d) out of range", fn, i, s, d);
      if (taken[d]) return pa::fail(PA_ERR_INVALID_ARG, "%s: destination %d repeated", fn, d);
      taken[d] = 1;
    }
  }
  const int64_t elem = (device->flags & PA_CACHE_FP8) ? 1 : 2;
  const int64_t vecs = static_cast<int64_t>(device->num_kv_heads) * kBlock * device->head_dim * elem / 16;
  const int64_t gx = std::min<int64_t>((vecs + 255) / 256, 64);
  block_copy_kernel<<<dim3(gx, num_pairs), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
      pairs, static_cast<const u32x4*>(src->k_cache), static_cast<const u32x4*>(src->v_cache),
      static_cast<u32x4*>(dst->k_cache), static_cast<u32x4*>(dst->v_cache), vecs, src->num_blocks,
      dst->num_blocks);
  return launch_status(fn);
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                int32_t max_context_len) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || max_context_len <= kPartTokens) return 0;
  const int64_t P = parts_for(max_context_len, kPartTokens);
  const int64_t rows = static_cast<int64_t>(num_seqs) * num_heads * P;
  return ws_counter_bytes(num_seqs, num_heads) + ws_ml_bytes(rows) +
         static_cast<size_t>(rows) * head_dim * sizeof(float);
}

pa_status pa_decode_attention(const pa_cache* cache, const void* q, int32_t num_seqs,
                              int32_t num_heads, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* context_lens,
                              int32_t max_context_len, float scale, void* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return pa::decode_run("pa_decode_attention", cache, q, num_seqs, num_heads, block_tables,
                        max_blocks_per_seq, context_lens, max_context_len, scale, out, workspace,
                        workspace_bytes, nullptr, nullptr, nullptr, false, false, 0, nullptr,
                        nullptr, stream);
}

pa_status pa_decode_merge(const pa_cache* cache, int32_t num_seqs, int32_t num_heads,
                          const int32_t* context_lens, int32_t max_context_len, void* out,
                          void* workspace, size_t workspace_bytes, void* stream) {
  pa::clear_error();
  DecodeSetup su;
  pa_status st = prepare_decode("pa_decode_merge", cache, nullptr, num_seqs, num_heads, nullptr, 0,
                                context_lens, max_context_len, 1.f, out, workspace,
                                workspace_bytes, false, &su);
  // wide query groups: pa_decode_attention has merged already
  if (st != PA_OK || num_seqs == 0 || su.args.max_parts <= 1 || su.wide_group) return st;
  MergeArgs m;
  m.ctx_lens = context_lens;
  m.out = static_cast<uint16_t*>(out);
  m.ws_ml = su.args.ws_ml;
  m.ws_acc = su.args.ws_acc;
  m.num_seqs = num_seqs;
  m.num_heads = num_heads;
  m.max_ctx = max_context_len;
  m.max_parts = su.args.max_parts;
  m.part_tokens = su.args.part_blocks * kBlock;
  const int64_t grid = (static_cast<int64_t>(num_seqs) * num_heads + 3) / 4;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (cache->dtype == PA_F16)
    launch_merge<F16>(m, grid, cache->head_dim, s);
  else
    launch_merge<BF16>(m, grid, cache->head_dim, s);
  return launch_status("pa_decode_merge");
}

pa_status pa_decode(const pa_cache* cache, const void* q, int32_t num_seqs, int32_t num_heads,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t max_context_len, float scale, void* out,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return pa::decode_run("pa_decode", cache, q, num_seqs, num_heads, block_tables,
                        max_blocks_per_seq, context_lens, max_context_len, scale, out, workspace,
                        workspace_bytes, nullptr, nullptr, nullptr, true, true, 0, nullptr,
                        nullptr, stream);
}

pa_status pa_decode_partitioned(const pa_cache* cache, const void* q, int32_t num_seqs,
                                int32_t num_heads, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* context_lens,
                                int32_t max_context_len, float scale, int32_t partition_tokens,
                                void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return pa::decode_run("pa_decode_partitioned", cache, q, num_seqs, num_heads, block_tables,
                        max_blocks_per_seq, context_lens, max_context_len, scale, out, workspace,
                        workspace_bytes, nullptr, nullptr, nullptr, true, true, partition_tokens,
                        nullptr, nullptr, stream);
}

pa_status pa_decode_fused(const pa_cache* cache, const void* k_new, const void* v_new,
                          const int64_t* slot_mapping, const void* q, int32_t num_seqs,
                          int32_t num_heads, const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t max_context_len, float scale,
                          void* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!k_new) return pa::fail(PA_ERR_INVALID_ARG, "pa_decode_fused: k_new is NULL");
  return pa::decode_run("pa_decode_fused", cache, q, num_seqs, num_heads, block_tables,
                        max_blocks_per_seq, context_lens, max_context_len, scale, out, workspace,
                        workspace_bytes, k_new, v_new, slot_mapping, true, true, 0, nullptr,
                        nullptr, stream);
}

// ---- timeline of the decode kernel (instrumented build) ---------------------------
pa_status pa_timeline_clear(void* stream) {
  pa::clear_error();
#ifdef PA_TIMELINE
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(g_timeline)) != hipSuccess || !ptr)
    return pa::fail(PA_ERR_HIP, "pa_timeline_clear: no device address for the records");
  if (hipMemsetAsync(ptr, 0, sizeof(g_timeline), static_cast<hipStream_t>(stream)) != hipSuccess)
    return pa::fail(PA_ERR_HIP, "pa_timeline_clear: hipMemsetAsync failed");
  return PA_OK;
#else
  (void)stream;
  return pa::fail(PA_ERR_UNSUPPORTED, "pa_timeline_clear: library built without PA_TIMELINE");
#endif
}

pa_status pa_timeline_read(uint64_t* host, int32_t num_workgroups) {
  pa::clear_error();
  if (!host || num_workgroups < 1 || num_workgroups > PA_TIMELINE_MAX_WORKGROUPS)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_timeline_read: host NULL or num_workgroups %d (1 .. %d)",
                    num_workgroups, PA_TIMELINE_MAX_WORKGROUPS);
#ifdef PA_TIMELINE
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(g_timeline)) != hipSuccess || !ptr)
    return pa::fail(PA_ERR_HIP, "pa_timeline_read: no device address for the records");
  if (hipDeviceSynchronize() != hipSuccess ||
      hipMemcpy(host, ptr, sizeof(uint64_t) * PA_TIMELINE_WORDS * num_workgroups,
                hipMemcpyDeviceToHost) != hipSuccess)
    return pa::fail(PA_ERR_HIP, "pa_timeline_read: copy failed");
  return PA_OK;
#else
  return pa::fail(PA_ERR_UNSUPPORTED, "pa_timeline_read: library built without PA_TIMELINE");
#endif
}

}  // extern "C"
