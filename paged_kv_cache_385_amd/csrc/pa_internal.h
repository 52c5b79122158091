// Internal helpers shared by the library's translation units (host side).
#pragma once

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "../../include/pa.h"

namespace pa {

// Records a formatted detail for pa_last_error() and returns `st`.
pa_status fail(pa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Checks of a cache descriptor shared by every entry point (fn names the caller).
pa_status check_cache(const pa_cache* c, const char* fn);
// PA_ERR_HIP with the runtime's message if the last launch failed.
pa_status launch_status(const char* fn);
bool aligned16(const void* p);
// Compute units of the current device (queried once per device).
int32_t device_cus();

// Blocks of the manager whose reference count is above one (kept up to date).
int64_t bm_shared_blocks(const pa_bm* bm);
// 16-token pool tiles per block of the manager (1, or 2 for 32-token blocks).
int32_t bm_tiles_per_block(const pa_bm* bm);

// Argument checks of pa_decode for a call whose context lengths are at most
// max_ctx, with a workspace of at least pa_decode_workspace_size(..., max_ctx)
// bytes; enqueues nothing.
// Bytes of a decode workspace's leading counter region: the merge counters int32[B][H]
// and the claim counter after them, all zero between calls.
size_t decode_counter_bytes(int64_t num_seqs, int64_t num_heads);
pa_status decode_check(const pa_cache* cache, const void* q, int32_t num_seqs, int32_t num_heads,
                       int32_t max_blocks_per_seq, int32_t max_ctx, float scale, void* out,
                       void* workspace, size_t workspace_bytes);

// Every decode entry point: the optional fused store of new tokens (k_new != NULL),
// the attention pass between the optional events ev_begin / ev_end (hipEvent_t),
// then, if merge, the log-sum-exp merge (inside the attention pass when
// fuse_merge allows and the partitions are few, else a second launch).
// part_tokens fixes the partition length (512 .. 4096, a power of two); 0 lets
// the launch choose it from the batch shape and the device.
pa_status decode_run(const char* fn, const pa_cache* cache, const void* q, int32_t num_seqs,
                     int32_t num_heads, const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t max_context_len, float scale, void* out,
                     void* workspace, size_t workspace_bytes, const void* k_new, const void* v_new,
                     const int64_t* slot_mapping, bool merge, bool fuse_merge,
                     int32_t part_tokens, void* ev_begin, void* ev_end, void* stream);

// pa_decode_grouped with the optional events (hipEvent_t) attached to the kernel's
// dispatch: its own start and end.
pa_status decode_grouped_run(const char* fn, const pa_cache* cache, const void* q, int32_t num_seqs,
                             int32_t num_heads, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, int32_t max_context_len,
                             const int32_t* plan, const int32_t* plan_host, float scale, void* out,
                             void* workspace, size_t workspace_bytes, void* ev_begin, void* ev_end,
                             void* stream);

// Decode with more than 16 query heads per KV head: pa_chunk_attention's kernels
// with one query per sequence (q and out [num_seqs][num_heads][head_dim]), the
// key-partition states in `workspace` (pa_chunk_workspace_size bytes for
// total_q = num_seqs, max_q_len = 1, which pa_decode_workspace_size covers past
// its counters).  Checks and launches as pa_chunk_attention.
pa_status chunk_decode(const char* fn, const pa_cache* cache, const void* q, int32_t num_seqs,
                       int32_t num_heads, const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* context_lens, int32_t max_context_len, float scale,
                       void* out, void* workspace, size_t workspace_bytes, void* ev_begin,
                       void* ev_end, void* stream);

}  // namespace pa
