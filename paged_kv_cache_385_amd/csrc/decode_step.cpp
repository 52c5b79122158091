// One decode step of a batch of sequences, host work and device work in one call.
//
// The order is the one a decode step needs ("vLLM 核心概念", section "为什么需要
// KV Cache？": the new token's K/V is cached, then attention reads all cached
// tokens; "理解 vLLM PagedAttention", section 六: a sequence that diverges from a
// shared block gets its private copy before it writes):
//   1. host: the block manager reserves every sequence's next slot, reporting
//      copy-on-write pairs, and packs tables and lengths into the staging buffer;
//   2. one host-to-device copy of the staging buffer -- on the caller's stream,
//      or on a copy stream (the copy of step i + 1 runs while step i's kernels
//      still run; the host, or on an idle stream the stream, waits for it) --
//      or none: with no device staging buffer the kernels read the pinned one
//      in place;
//   3. pa_copy_blocks for the pairs (two 16-token tiles per copied block of a
//      32-token manager), then pa_decode_fused (the new tokens'
//      store and the decode in one attention pass, then the merge) -- all on
//      the caller's stream.  When the manager holds shared blocks and grouping
//      the batch by shared prefix saves enough block reads (pa_group_plan, run on
//      the packed tables, its plan staged and uploaded with them), the new
//      tokens are stored by pa_cache_write and pa_decode_grouped attends.

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdlib>

#include "pa_internal.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

struct StagingLayout {
  size_t slots, ctx, tables, pairs, plan, plan_bytes, total;
};

StagingLayout layout(int32_t n, int32_t max_blocks) {
  StagingLayout l;
  l.slots = 0;
  l.ctx = l.slots + align_up(sizeof(int64_t) * static_cast<size_t>(n));
  l.tables = l.ctx + align_up(sizeof(int32_t) * static_cast<size_t>(n));
  l.pairs = l.tables + align_up(sizeof(int32_t) * static_cast<size_t>(n) * max_blocks);
  // up to two tile copies per sequence (a 32-token block is two 16-token tiles)
  l.plan = l.pairs + align_up(sizeof(int32_t) * 4 * static_cast<size_t>(n));
  // a grouped-decode plan for the longest context the tables can hold
  l.plan_bytes = align_up(pa_group_plan_bytes(n, max_blocks * PA_BLOCK_SIZE));
  l.total = l.plan + l.plan_bytes;
  return l;
}

// PA_GROUPED_DECODE=0 in the environment: steps never take the grouped decode (read once).
bool grouped_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("PA_GROUPED_DECODE");
    return !(e && e[0] == '0');
  }();
  return on;
}

// PA_STEP_STREAM_WAIT=1 in the environment: a step with a copy stream makes its stream
// wait for the copy instead of the host.
bool stream_wait_forced() {
  static const bool on = [] {
    const char* e = std::getenv("PA_STEP_STREAM_WAIT");
    return e && e[0] == '1';
  }();
  return on;
}

}  // namespace

extern "C" {

size_t pa_decode_step_staging_bytes(int32_t num_seqs, int32_t max_blocks_per_seq) {
  if (num_seqs <= 0 || max_blocks_per_seq <= 0) return 0;
  return layout(num_seqs, max_blocks_per_seq).total;
}

pa_status pa_decode_step(pa_bm* bm, const pa_cache* cache, int32_t num_seqs, const int64_t* seq_ids,
                         const void* k_new, const void* v_new, const void* q, int32_t num_heads,
                         float scale, void* out, void* workspace, size_t workspace_bytes,
                         void* staging_host, void* staging_dev, size_t staging_bytes,
                         int32_t max_blocks_per_seq, void* attn_begin, void* attn_end,
                         pa_step_info* info, void* copy_stream, void* copy_event, void* stream) {
  pa::clear_error();
  if (!bm || !cache || num_seqs <= 0 || !seq_ids || !k_new || !v_new || !q || !out ||
      !staging_host || max_blocks_per_seq <= 0)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_decode_step: bad arguments");
  const bool zero_copy = staging_dev == nullptr;
  if (copy_stream && (zero_copy || !copy_event))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_decode_step: a copy stream needs staging_dev and copy_event");
  const StagingLayout l = layout(num_seqs, max_blocks_per_seq);
  if (staging_bytes < l.total)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_decode_step: staging %zu bytes, %zu needed",
                    staging_bytes, l.total);
  if (reinterpret_cast<uintptr_t>(staging_host) % kAlign || reinterpret_cast<uintptr_t>(staging_dev) % kAlign)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_decode_step: staging buffers must be 256-byte aligned");
  if (reinterpret_cast<uintptr_t>(k_new) % 16 || reinterpret_cast<uintptr_t>(v_new) % 16)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_decode_step: k_new / v_new must be 16-byte aligned");
  const int64_t max_tokens = static_cast<int64_t>(max_blocks_per_seq) * PA_BLOCK_SIZE;
  if (max_tokens > INT32_MAX)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_decode_step: max_blocks_per_seq %d too large", max_blocks_per_seq);
  // Everything the device calls check, against the longest context the packing allows,
  // before the block manager changes.
  pa_status st = pa::decode_check(cache, q, num_seqs, num_heads, max_blocks_per_seq,
                                  static_cast<int32_t>(max_tokens), scale, out, workspace,
                                  workspace_bytes);
  if (st != PA_OK) return st;

  char* hb = static_cast<char*>(staging_host);
  char* db = static_cast<char*>(staging_dev);
  auto* slots_h = reinterpret_cast<int64_t*>(hb + l.slots);
  auto* ctx_h = reinterpret_cast<int32_t*>(hb + l.ctx);
  auto* tables_h = reinterpret_cast<int32_t*>(hb + l.tables);
  auto* pairs_h = reinterpret_cast<int32_t*>(hb + l.pairs);
  int32_t n_cow = 0, max_ctx = 0;
  st = pa_bm_step(bm, num_seqs, seq_ids, slots_h, pairs_h, num_seqs, &n_cow, tables_h,
                  max_blocks_per_seq, ctx_h, &max_ctx);
  if (st != PA_OK) return st;
  // pairs of manager blocks -> pairs of pool tiles (two per 32-token block), in place;
  // the staging area holds two tile pairs per sequence
  st = pa_bm_tile_pairs(bm, pairs_h, n_cow, pairs_h, 2 * num_seqs, &n_cow);
  if (st != PA_OK) return st;
  // Blocks shared by several sequences of the manager: the batch may decode as groups
  // that read each shared block once (pa_decode_grouped), when the plan says it saves
  // enough.  A plan that cannot be made leaves the ordinary decode.
  auto* plan_h = reinterpret_cast<int32_t*>(hb + l.plan);
  int32_t plan_ints = 0;
  if (grouped_enabled() && pa::bm_shared_blocks(bm) > 0 &&
      pa_group_plan(tables_h, num_seqs, max_blocks_per_seq, ctx_h, max_ctx, num_heads,
                    cache->num_kv_heads, 2 * pa::device_cus(), plan_h, l.plan_bytes,
                    &plan_ints) != PA_OK)
    plan_ints = 0;
  if (info) {
    info->num_cow = n_cow;
    info->max_context_len = max_ctx;
    info->grouped = plan_ints > 0 ? 1 : 0;
    info->host_waited = 0;
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (zero_copy) {
    // the kernels read the pinned staging buffer in place, over the host link
    void* dp = nullptr;
    if (hipHostGetDevicePointer(&dp, staging_host, 0) != hipSuccess || !dp)
      return pa::fail(PA_ERR_HIP, "pa_decode_step: staging_host is not pinned, mapped host memory");
    db = static_cast<char*>(dp);
  } else {
    const size_t upload = plan_ints ? l.plan + sizeof(int32_t) * plan_ints
                          : n_cow    ? l.pairs + sizeof(int32_t) * 2 * n_cow
                                     : l.pairs;
    hipStream_t cs = copy_stream ? static_cast<hipStream_t>(copy_stream) : s;
    if (hipMemcpyAsync(db, hb, upload, hipMemcpyHostToDevice, cs) != hipSuccess)
      return pa::fail(PA_ERR_HIP, "pa_decode_step: hipMemcpyAsync failed");
    if (copy_stream) {
      hipEvent_t ev = static_cast<hipEvent_t>(copy_event);
      // The host waits for the copy, and the kernels are queued with nothing before
      // them on `stream`.  A cross-stream wait is a barrier packet, and asking whether
      // `stream` is still busy (hipStreamQuery) puts a marker behind its last kernel;
      // either one delays the next kernel by about 5 us on gfx950 even when nothing
      // is left to wait for.  In a loop of steps the copy ends long before the
      // previous step's kernels do, so the host's wait costs the device nothing.
      const bool host_wait = !stream_wait_forced();
      if (hipEventRecord(ev, cs) != hipSuccess ||
          (host_wait ? hipEventSynchronize(ev) : hipStreamWaitEvent(s, ev, 0)) != hipSuccess)
        return pa::fail(PA_ERR_HIP, "pa_decode_step: copy-stream event failed");
      if (info) info->host_waited = host_wait ? 1 : 0;
    }
  }
  if (n_cow) {
    st = pa_copy_blocks(cache, reinterpret_cast<const int32_t*>(db + l.pairs), pairs_h, n_cow, stream);
    if (st != PA_OK) return st;
  }
  // blocks shared by several sequences are read through the caches
  pa_cache c = *cache;
  if (pa::bm_shared_blocks(bm) > 0) c.flags |= PA_CACHE_SHARED_BLOCKS;
  if (plan_ints) {
    // grouped: the new tokens are stored by their own launch, then the groups attend
    st = pa_cache_write(cache, k_new, v_new, reinterpret_cast<const int64_t*>(db + l.slots), num_seqs,
                        stream);
    if (st != PA_OK) return st;
    return pa::decode_grouped_run("pa_decode_step", &c, q, num_seqs, num_heads,
                                  reinterpret_cast<const int32_t*>(db + l.tables), max_blocks_per_seq,
                                  max_ctx, reinterpret_cast<const int32_t*>(db + l.plan), plan_h, scale,
                                  out, workspace, workspace_bytes, attn_begin, attn_end, stream);
  }
  return pa::decode_run("pa_decode_step", &c, q, num_seqs, num_heads,
                        reinterpret_cast<const int32_t*>(db + l.tables), max_blocks_per_seq,
                        reinterpret_cast<const int32_t*>(db + l.ctx), max_ctx, scale, out, workspace,
                        workspace_bytes, k_new, v_new, reinterpret_cast<const int64_t*>(db + l.slots),
                        true, true, 0, attn_begin, attn_end, stream);
}

}  // extern "C"
