// Grouped decode: single-query attention for a batch in which groups of sequences
// share the leading blocks of their block tables (samples or beams forked from one
// prompt: "理解 vLLM PagedAttention", section 六; "vLLM 核心概念", section "内存共享").
//
// Each work item is (group, KV head, partition of the group's block list).  The
// list holds the group's shared blocks, then each member's own blocks.  The query
// heads of all the group's sequences for that KV head are the columns of the
// matrix-core tile (at most 16), so a shared block is read once and scored against
// every member's queries; a member's own block is scored against all columns with
// the other members' columns masked.  Per column the online softmax runs as in the
// single-sequence kernel; a column whose member has no token in a partition keeps
// an empty state (max -inf, sum 0), which the log-sum-exp merge weighs as zero.
// The partitions of a (group, KV head) are merged by the last of them to finish.
//
// The work plan (which sequences, how many shared blocks, the item order) comes
// from pa_group_plan on the host; context lengths are the plan's.

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
constexpr int kMaxColumns = 16;
constexpr int kHeader = 8, kGroupInts = 8, kMemberInts = 4;

struct GroupArgs {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;
  const int32_t* plan;          // device copy of the plan
  uint16_t* out;
  const float* k_scales;        // FP8 pools: [Hkv] scales of K and of V
  const float* v_scales;
  int32_t* counters;            // [groups][Hkv] partitions finished
  float2* ws_ml;                // [B][H][max_parts] (max in log2 units, sum)
  float* ws_acc;                // [B][H][max_parts][D] unnormalised output
  int32_t num_heads, num_kv_heads, group, max_blocks, num_blocks;
  int32_t part_blocks, max_parts, members_off, items_off;
  float scale_log2;
};

__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <class E, int D, bool kStream, bool kFp8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3)))
void decode_group_kernel(GroupArgs a) {
  constexpr int KK = D / 32;
  constexpr int LW = kFp8 ? KK / 2 : KK;
  constexpr int64_t kTileBytes = static_cast<int64_t>(kBlock) * D * (kFp8 ? 1 : 2);
  constexpr int MT = D / 16;
  constexpr int kLdsStride = D + 4;
  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];
  __shared__ __attribute__((aligned(16))) float s_acc[kWaves][16 * kLdsStride];
  __shared__ int32_t s_mem[kMaxColumns][kMemberInts];   // (sequence, private offset, blocks, context)
  __shared__ int s_bad;
  __shared__ int32_t s_ticket;

  const int32_t tid = threadIdx.x;
  const int32_t w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t lane = tid & 63;
  const int32_t n = lane & 15;       // column of the tile: (member n / G, query head n % G)
  const int32_t g4 = lane >> 4;
  const int32_t hkv = a.num_kv_heads;
  const int32_t G = a.group;
  const int32_t PB = a.part_blocks;
  const int32_t pair = a.plan[a.items_off + blockIdx.x / hkv];
  const int32_t kvh = blockIdx.x % hkv;
  const int32_t gi = pair >> 12, p = pair & 4095;
  const int32_t* gr = a.plan + kHeader + kGroupInts * gi;
  const int32_t mfirst = gr[0], nm = gr[1], ns = gr[2], L = gr[3], parts = gr[4], ctx_max = gr[5];
  const int32_t cols = nm * G;
  if (nm < 1 || cols > kMaxColumns || p >= parts) return;   // cannot happen for a plan's items
  if (tid < nm * kMemberInts)
    s_mem[tid / kMemberInts][tid % kMemberInts] = a.plan[a.members_off + kMemberInts * mfirst + tid];
  __syncthreads();

  const bool col_on = n < cols;
  const int32_t mn = col_on ? n / G : 0;                  // this lane's column's member
  const int32_t col_seq = s_mem[mn][0];
  const int32_t col_ctx = col_on ? s_mem[mn][3] : 0;
  const int32_t col_head = kvh * G + (n - mn * G);
  u32x4 qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    qf[kk] = col_on ? load16(a.q + (static_cast<int64_t>(col_seq) * a.num_heads + col_head) * D +
                             32 * kk + 8 * g4)
                    : u32x4{0, 0, 0, 0};
  }

  // This wave's blocks are list positions first, first + 4, ... below jend.  Lane i
  // holds the i-th one's member (-1: shared by all), its index in that member's
  // table, and its physical id.
  const int32_t jend = min(L, (p + 1) * PB);
  const int32_t first = p * PB + w;
  const int32_t nw = first < jend ? (jend - first + kWaves - 1) / kWaves : 0;
  int32_t bmem = -1, bj = 0, ids = 0;
  if (lane < nw) {
    const int32_t k = first + kWaves * lane;
    int32_t seq = s_mem[0][0];
    if (k < ns) {
      bj = k;
    } else {
      const int32_t r = k - ns;
      int32_t m = 0;
      while (m + 1 < nm && s_mem[m + 1][1] <= r) ++m;   // private offsets ascend
      bmem = m;
      bj = ns + (r - s_mem[m][1]);
      seq = s_mem[m][0];
    }
    ids = a.block_tables[static_cast<int64_t>(seq) * a.max_blocks + bj];
  }
  const bool id_bad = lane < nw && (ids < 0 || ids >= a.num_blocks);
  if (id_bad) ids = 0;
  const bool bad_blk = __ballot(id_bad) != 0;

  const int64_t head_off_b = static_cast<int64_t>(kvh) * kTileBytes;
  const int64_t blk_stride_b = static_cast<int64_t>(hkv) * kTileBytes;
  const float score_scale = kFp8 ? a.scale_log2 * a.k_scales[kvh] : a.scale_log2;

  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x4 acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 kb[2][LW], vb[2][LW];

  // one unconditional load per step: an empty range past the wave's last block
  auto load_block = [&](int buf, int32_t i) {
    const int32_t phys = __builtin_amdgcn_readlane(ids, min(i, nw - 1));
    const int32_t bytes = i < nw ? static_cast<int32_t>(kTileBytes) : 0;
    const auto kr = tile_rsrc(reinterpret_cast<const char*>(a.k_cache) + phys * blk_stride_b + head_off_b, bytes);
    const auto vr = tile_rsrc(reinterpret_cast<const char*>(a.v_cache) + phys * blk_stride_b + head_off_b, bytes);
    if constexpr (kFp8) {
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

  // Block i of the wave (i >= nw: a padding step, every position masked).  Column n
  // sees the block's tokens below its member's context when the block is shared or
  // its member's own; a column that has seen no token yet exponentiates against a
  // finite stand-in, so a fully masked block adds nothing.
  auto compute_block = [&](int buf, int32_t i) {
    const bool real = i < nw;
    const int32_t bm = __builtin_amdgcn_readlane(bmem, min(i, 63));
    const int32_t jb = __builtin_amdgcn_readlane(bj, min(i, 63));
    const int32_t base = jb * kBlock;
    const int32_t col_valid = real && col_on && (bm < 0 || bm == mn) ? col_ctx - base : 0;
    const int32_t owner_ctx = bm < 0 ? ctx_max : __builtin_amdgcn_readlane(col_ctx, max(bm, 0) * G);
    const int32_t vmax = real ? owner_ctx - base : 0;    // rows past it may hold anything
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
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[r] = 4 * g4 + r < col_valid ? s[r] * score_scale : -INFINITY;
    float bmax = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    const float m_new = fmaxf(m_run, bmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    u16x4 pb;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pb[r] = E::from_float(fast_exp2(sv[r] - m_use));
      psum += E::to_float(pb[r]);
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int i2 = 0; i2 < MT; ++i2) acc[i2] *= alpha;
    if (vmax < kBlock) {
#pragma unroll
      for (int j2 = 0; j2 < KK; ++j2) {
        u16x8 vv = __builtin_bit_cast(u16x8, V[j2]);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (4 * g4 + (e & 3) >= vmax) vv[e] = 0;
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

  if (nw > 0) {
    load_block(0, 0);
    for (int32_t i = 0; i < nw; i += 2) {
      load_block(1, i + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute_block(0, i);
      load_block(0, i + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute_block(1, i + 1);
    }
  }

  // ---- combine the four waves in LDS ----
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (g4 == 0) {
    s_m[w][n] = m_run;
    s_l[w][n] = l_run;
  }
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (bad_blk) s_bad = 1;
  float M = -INFINITY;
#pragma unroll
  for (int u = 0; u < kWaves; ++u) M = fmaxf(M, s_m[u][n]);
  const float wscale = fast_exp2(m_run - (M == -INFINITY ? 0.f : M));   // 0 for a wave that saw nothing
  if (col_on) {
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

  // each thread finishes 4 consecutive dims of one column
  auto column_row = [&](int32_t c) {
    const int32_t m = c / G;
    return static_cast<int64_t>(s_mem[m][0]) * a.num_heads + kvh * G + (c - m * G);
  };
  for (int32_t i4 = tid; i4 < cols * (D / 4); i4 += kThreads) {
    const int32_t c = i4 / (D / 4);
    const int32_t d = (i4 - c * (D / 4)) * 4;
    float Mh = -INFINITY;
#pragma unroll
    for (int u = 0; u < kWaves; ++u) Mh = fmaxf(Mh, s_m[u][c]);
    const float Mu = Mh == -INFINITY ? 0.f : Mh;
    float Lh = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kWaves; ++u) {
      Lh += s_l[u][c] * fast_exp2(s_m[u][c] - Mu);
      o += *reinterpret_cast<const f32x4*>(&s_acc[u][c * kLdsStride + d]);
    }
    if (kFp8) o *= a.v_scales[kvh];
    const int64_t hrow = column_row(c);
    if (parts == 1) {
      u16x4 ov;
      if (poisoned) {
        ov = u16x4{E::kNaN, E::kNaN, E::kNaN, E::kNaN};
      } else {
        const float inv = 1.f / Lh;
#pragma unroll
        for (int r = 0; r < 4; ++r) ov[r] = E::from_float(o[r] * inv);
      }
      *reinterpret_cast<u16x4*>(a.out + hrow * D + d) = ov;
    } else {
      const int64_t st = hrow * a.max_parts + p;
      if (poisoned) o = f32x4{NAN, NAN, NAN, NAN};
      const float2 ml = poisoned ? float2{0.f, NAN} : float2{Mh, Lh};
#pragma unroll
      for (int r = 0; r < 4; ++r) store_coherent(a.ws_acc + st * D + d + r, o[r]);
      if (d == 0) {
        store_coherent(&a.ws_ml[st].x, ml.x);
        store_coherent(&a.ws_ml[st].y, ml.y);
      }
    }
  }
  if (parts == 1) return;

  // the last of the (group, KV head)'s partitions to finish merges them all
  wait_stores();
  __syncthreads();
  int32_t* counter = a.counters + static_cast<int64_t>(gi) * hkv + kvh;
  if (tid == 0) s_ticket = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (s_ticket != parts - 1) return;
  for (int32_t i4 = tid; i4 < cols * (D / 4); i4 += kThreads) {
    const int32_t c = i4 / (D / 4);
    const int32_t d = (i4 - c * (D / 4)) * 4;
    const int64_t hrow = column_row(c);
    const int64_t st0 = hrow * a.max_parts;
    float Mx = -INFINITY;
    for (int32_t u = 0; u < parts; ++u) Mx = fmaxf(Mx, load_coherent(&a.ws_ml[st0 + u].x));
    float Lx = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    for (int32_t u = 0; u < parts; ++u) {
      const float wgt = fast_exp2(load_coherent(&a.ws_ml[st0 + u].x) - Mx);
      Lx += wgt * load_coherent(&a.ws_ml[st0 + u].y);
      const float* src = a.ws_acc + (st0 + u) * D + d;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] += wgt * load_coherent(src + r);
    }
    const float inv = 1.f / Lx;
    u16x4 ov;
#pragma unroll
    for (int r = 0; r < 4; ++r) ov[r] = E::from_float(o[r] * inv);
    *reinterpret_cast<u16x4*>(a.out + hrow * D + d) = ov;
  }
  if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class E, bool kStream, bool kFp8>
void launch_t(const GroupArgs& g, int64_t grid, int d, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (d == 64)
    hipExtLaunchKernelGGL(decode_group_kernel<E, 64, kStream, kFp8>, dim3(grid), dim3(kThreads), 0, s,
                          e0, e1, 0, g);
  else
    hipExtLaunchKernelGGL(decode_group_kernel<E, 128, kStream, kFp8>, dim3(grid), dim3(kThreads), 0, s,
                          e0, e1, 0, g);
}

template <class E>
void launch(const GroupArgs& g, int64_t grid, int d, bool fp8, hipStream_t s, hipEvent_t e0,
            hipEvent_t e1) {
  if (fp8) launch_t<E, true, true>(g, grid, d, s, e0, e1);
  else launch_t<E, true, false>(g, grid, d, s, e0, e1);
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

namespace pa {

pa_status decode_grouped_run(const char* fn, const pa_cache* cache, const void* q, int32_t num_seqs,
                             int32_t num_heads, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, int32_t max_context_len,
                             const int32_t* plan, const int32_t* plan_host, float scale, void* out,
                             void* workspace, size_t workspace_bytes, void* ev_begin, void* ev_end,
                             void* stream) {
  pa_status st = check_cache(cache, fn);
  if (st != PA_OK) return st;
  if (num_seqs <= 0 || num_heads <= 0 || num_heads % cache->num_kv_heads)
    return fail(PA_ERR_INVALID_ARG, "%s: num_seqs %d, num_heads %d", fn, num_seqs, num_heads);
  const int32_t G = num_heads / cache->num_kv_heads;
  if (!q || !out || !block_tables || !plan || !plan_host || !aligned16(q) || !aligned16(out))
    return fail(PA_ERR_INVALID_ARG, "%s: NULL or misaligned argument", fn);
  if (max_blocks_per_seq < 1 || static_cast<int64_t>(max_blocks_per_seq) * kBlock < max_context_len ||
      max_context_len < 1)
    return fail(PA_ERR_INVALID_ARG, "%s: max_blocks_per_seq %d, max_context_len %d", fn,
                max_blocks_per_seq, max_context_len);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "%s: scale is not finite", fn);
  const int32_t ng = plan_host[0], pairs = plan_host[1], pb = plan_host[2], max_parts = plan_host[3];
  if (plan_host[4] != num_seqs || ng < 1 || ng > num_seqs || pairs < 1 ||
      (pb != 32 && pb != 64 && pb != 128 && pb != 256) || max_parts < 1 ||
      max_parts > (max_context_len + 511) / 512)
    return fail(PA_ERR_INVALID_ARG, "%s: the plan does not fit this call (groups %d, items %d, "
                "partition %d, partitions %d, sequences %d)", fn, ng, pairs, pb, max_parts, plan_host[4]);
  if (static_cast<int64_t>(pairs) * cache->num_kv_heads > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "%s: grid too large", fn);
  // Every index the kernel derives from the plan stays inside the tables, the
  // workspace and the output only if the plan is self-consistent: check it all.
  const int32_t* members = plan_host + kHeader + kGroupInts * ng;
  const int32_t* items = members + kMemberInts * num_seqs;
  for (int32_t g = 0; g < ng; ++g) {
    const int32_t* r = plan_host + kHeader + kGroupInts * g;
    const int32_t first = r[0], nm = r[1], ns = r[2], L = r[3], parts = r[4];
    if (nm < 1 || nm * G > kMaxColumns || first < 0 || first > num_seqs - nm || ns < 0 ||
        parts < 1 || parts > max_parts || L < 1 || static_cast<int64_t>(parts) * pb < L ||
        static_cast<int64_t>(parts - 1) * pb >= L)
      return fail(PA_ERR_INVALID_ARG, "%s: plan group %d is malformed", fn, g);
    int64_t list = ns;
    int32_t ctx_max = 0;
    for (int32_t k = 0; k < nm; ++k) {
      const int32_t* m = members + kMemberInts * (first + k);
      const int32_t seq = m[0], off = m[1], nblk = m[2], ctx = m[3];
      if (seq < 0 || seq >= num_seqs || ctx < 1 || ctx > max_context_len ||
          nblk != (ctx + kBlock - 1) / kBlock || nblk < ns || off != list - ns)
        return fail(PA_ERR_INVALID_ARG, "%s: plan member %d of group %d is malformed", fn, k, g);
      list += nblk - ns;
      ctx_max = std::max(ctx_max, ctx);
    }
    if (list != L || ctx_max != r[5])
      return fail(PA_ERR_INVALID_ARG, "%s: plan group %d lists %lld blocks, says %d", fn, g,
                  static_cast<long long>(list), L);
  }
  for (int32_t i = 0; i < pairs; ++i) {
    const int32_t gi = items[i] >> 12, p = items[i] & 4095;
    if (items[i] < 0 || gi >= ng || p >= plan_host[kHeader + kGroupInts * gi + 4])
      return fail(PA_ERR_INVALID_ARG, "%s: plan item %d is malformed", fn, i);
  }
  const int64_t rows = static_cast<int64_t>(num_seqs) * num_heads * max_parts;
  const size_t counters = pa::decode_counter_bytes(num_seqs, num_heads);
  const size_t need = max_parts > 1 ? counters + round256(rows * sizeof(float2)) + rows * cache->head_dim * sizeof(float) : 0;
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(PA_ERR_WORKSPACE, "%s: workspace %zu bytes, %zu needed", fn, workspace_bytes, need);
  GroupArgs g;
  g.q = static_cast<const uint16_t*>(q);
  g.k_cache = static_cast<const uint16_t*>(cache->k_cache);
  g.v_cache = static_cast<const uint16_t*>(cache->v_cache);
  g.block_tables = block_tables;
  g.plan = plan;
  g.out = static_cast<uint16_t*>(out);
  g.k_scales = cache->k_scales;
  g.v_scales = cache->v_scales;
  char* ws = static_cast<char*>(workspace);
  g.counters = need ? reinterpret_cast<int32_t*>(ws) : nullptr;
  g.ws_ml = need ? reinterpret_cast<float2*>(ws + counters) : nullptr;
  g.ws_acc = need ? reinterpret_cast<float*>(ws + counters + round256(rows * sizeof(float2))) : nullptr;
  g.num_heads = num_heads;
  g.num_kv_heads = cache->num_kv_heads;
  g.group = G;
  g.max_blocks = max_blocks_per_seq;
  g.num_blocks = cache->num_blocks;
  g.part_blocks = pb;
  g.max_parts = max_parts;
  g.members_off = kHeader + kGroupInts * ng;
  g.items_off = g.members_off + kMemberInts * num_seqs;
  g.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  const bool fp8 = (cache->flags & PA_CACHE_FP8) != 0;
  // Within a group every block is read by one item only; a prefix that several groups
  // share (a family wider than one tile) is read by items that seldom run on one XCD
  // at once.  The loads stream (non-temporal): measured faster for every plan tried.
  const int64_t grid = static_cast<int64_t>(pairs) * cache->num_kv_heads;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipEvent_t e0 = static_cast<hipEvent_t>(ev_begin), e1 = static_cast<hipEvent_t>(ev_end);
  if (cache->dtype == PA_F16)
    launch<F16>(g, grid, cache->head_dim, fp8, s, e0, e1);
  else
    launch<BF16>(g, grid, cache->head_dim, fp8, s, e0, e1);
  return launch_status(fn);
}

}  // namespace pa

extern "C" {

pa_status pa_decode_grouped(const pa_cache* cache, const void* q, int32_t num_seqs,
                            int32_t num_heads, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, int32_t max_context_len,
                            const int32_t* plan, const int32_t* plan_host, float scale, void* out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  pa::clear_error();
  return pa::decode_grouped_run("pa_decode_grouped", cache, q, num_seqs, num_heads, block_tables,
                                max_blocks_per_seq, max_context_len, plan, plan_host, scale, out,
                                workspace, workspace_bytes, nullptr, nullptr, stream);
}

}  // extern "C"
