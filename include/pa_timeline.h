/*
 * pa_timeline.h -- per-workgroup timeline of the decode kernel: a measurement tool.
 *
 * Decode time is the time to read the cached K/V of every context token
 * ("PagedAttention 实战", section "Decode：逐 token 生成输出").  How much of a
 * pass each workgroup spends streaming, and how much in its fixed start-up (the
 * sequence's lengths, its block ids, the first tile), decides how close the pass
 * comes to that bound.  These calls expose stamps the decode kernel takes when
 * the library is compiled with PA_TIMELINE defined (libpa_timeline.so, built
 * beside libpa.so); in the ordinary build they return PA_ERR_UNSUPPORTED and
 * the kernel takes no stamps.
 *
 * Thread 0 of every workgroup of a decode_attn_kernel launch (pa_decode,
 * pa_decode_fused, pa_decode_attention, pa_decode_partitioned, pa_decode_step)
 * writes one record of PA_TIMELINE_WORDS 64-bit words at index blockIdx.x, for
 * blockIdx.x < PA_TIMELINE_MAX_WORKGROUPS (later workgroups write nothing):
 *   [0] entry        [1] item known (sequence, KV heads, partition)
 *   [2] first tile computed by wave 0 (0: that wave streamed no tile)
 *   [3] wave 0's last tile computed   [4] output or partial state written
 *   [5] sequence << 32 | partition
 *   [6] KV-head group << 32 | wave 0's tiles << 16 | tiles of the item per KV head
 *   [7] XCC id << 32 | the hardware id register (CU, SE, SIMD, wave fields)
 * Words 0-4 are readings of the 100 MHz constant counter (s_memrealtime); one
 * launch's records share its time base.  A record whose word 0 is 0 was not
 * written since the last clear.  Records are overwritten by every launch: clear,
 * run one launch, synchronize, read.
 */
#ifndef PA_TIMELINE_H
#define PA_TIMELINE_H

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

#define PA_TIMELINE_WORDS 8
#define PA_TIMELINE_MAX_WORKGROUPS 65536

/* Zero every record (on the device current at the call, enqueued on `stream`,
 * a hipStream_t). */
pa_status pa_timeline_clear(void* stream);

/* Copy records 0 .. num_workgroups - 1 (1 .. PA_TIMELINE_MAX_WORKGROUPS) into
 * `host` (num_workgroups * PA_TIMELINE_WORDS words).  Synchronous: it waits for
 * the device current at the call, so the caller need not synchronize first. */
pa_status pa_timeline_read(uint64_t* host, int32_t num_workgroups);

#ifdef __cplusplus
}
#endif

#endif /* PA_TIMELINE_H */
