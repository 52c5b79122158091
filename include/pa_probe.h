/*
 * pa_probe.h -- streaming-read probes of libpa: a measured read ceiling for the
 * decode kernel on the device it runs on.
 *
 * Decode attention is bound by reading every cached K/V byte of the history once
 * per step ("PagedAttention 实战", section "Decode：逐 token 生成输出"; "理解 vLLM
 * PagedAttention", section 七: longer contexts read more).  These calls read the
 * same kind of bytes with no computation, so the rate they reach is what the
 * memory system gives that access pattern: a second denominator beside the
 * nominal HBM peak.  They are measurement tools; the decode path never calls them.
 *
 * Both calls enqueue one kernel on `stream` (a hipStream_t), read every given
 * byte exactly once with 16-byte non-temporal loads, and write nothing except,
 * never in practice, one word to `sink` (device, 4 bytes): a value folded from
 * the data is stored only if it equals a fixed constant, which keeps every load
 * alive.  Arguments are checked on the host before the launch; a rejected call
 * enqueues nothing and returns PA_ERR_INVALID_ARG (detail in pa_last_error()).
 * Launch failures return PA_ERR_HIP.
 */
#ifndef PA_PROBE_H
#define PA_PROBE_H

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read bytes [0, bytes) of `buf` (device, 16-byte aligned, bytes a non-zero
 * multiple of 16), front to back.  workgroups_per_cu (1 .. 64) workgroups of
 * 256 threads per compute unit stride over the buffer, four loads in flight per
 * thread. */
pa_status pa_probe_read_contiguous(const void* buf, size_t bytes, int32_t workgroups_per_cu,
                                   uint32_t* sink, void* stream);

/* Read tiles tiles[0 .. num_tiles) of a K pool and of a V pool (device, 16-byte
 * aligned, pool_bytes each): tile i is bytes [i, i + 1) x tile_bytes of both pools,
 * so a list of (block * num_kv_heads + head) ids reads the tiles a decode pass over
 * those (block, head) pairs reads, in the list's order.  tile_bytes is one (block,
 * KV head) tile of the pool, 16 tokens x head_dim x element bytes: 4096 for a
 * 16-bit pool at head_dim 128, 2048 for an FP8 pool (or a 16-bit one at head_dim
 * 64), 1024 for an FP8 pool at head_dim 64; other sizes are rejected.  `tiles` is
 * the device copy of the list, `tiles_host` the same list on the host, where every
 * id is checked against pool_bytes / tile_bytes.  Each tile is read by tile_bytes /
 * 16 lanes with one 16-byte load each, so a workgroup (256 threads) covers 4096 /
 * tile_bytes tiles of each pool per load instruction, two such steps in flight;
 * workgroups_per_cu (1 .. 64) workgroups per compute unit. */
pa_status pa_probe_read_tiles(const void* k_base, const void* v_base, size_t pool_bytes,
                              int32_t tile_bytes, const int32_t* tiles, const int32_t* tiles_host,
                              int32_t num_tiles, int32_t workgroups_per_cu, uint32_t* sink,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H */
