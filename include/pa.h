/*
 * pa.h -- C ABI of libpa: paged KV-cache decode attention for AMD MI355X (gfx950).
 *
 * The library implements the data-parallel hot path of PagedAttention as the
 * explainer pages describe it: the K and V vectors of every cached token live
 * in fixed-size blocks (16 tokens) scattered through one physical pool and are
 * reached through a per-sequence block table ("vLLM 核心概念", sections
 * "核心概念：块（Block）" and "逻辑视图与物理视图分离"); each decode step stores the
 * new token's K/V and then attends over the whole cached history ("vLLM 核心概念",
 * section "为什么需要 KV Cache？"; "PagedAttention 实战", section
 * "Decode：逐 token 生成输出"); forked sequences share blocks and copy a block
 * only when they diverge ("理解 vLLM PagedAttention", section 六).
 *
 * Conventions for every device entry point
 *   - All tensors are caller-owned device memory (allocated by the caller, e.g.
 *     with PyTorch); the library never allocates device memory, never frees it
 *     and never synchronises.  Work is enqueued on `stream` (a hipStream_t; NULL
 *     means the default stream) and is asynchronous.
 *   - Scalar arguments and shapes are validated on the host before anything is
 *     enqueued; a rejected call enqueues nothing.  A launch failure returns
 *     PA_ERR_HIP.  The detail of the last error on the calling thread is in
 *     pa_last_error().
 *   - Device-resident indices (slots, block tables, context lengths, copy
 *     pairs) cannot be checked on the host.  The kernels check them and never
 *     touch memory outside the pools because of them: an out-of-range slot or
 *     copy pair is skipped, and a sequence whose context length or block ids
 *     are out of range gets NaN in its output rows.
 *
 * Cache layout (the pages leave it open; chosen so that every decode load is a
 * contiguous 16-byte lane load that lands directly in a matrix-core operand):
 *   K pool: [num_blocks][num_kv_heads][head_dim/8][16][8]
 *           token t, dim d of (block b, head h) at [b][h][d/8][t][d%8]
 *   V pool: [num_blocks][num_kv_heads][4][head_dim][4]
 *           token t, dim d of (block b, head h) at [b][h][t/4][d][t%4]
 *   One (block, head) tile of K or V is 16*head_dim contiguous elements; one
 *   physical block of a pool is num_kv_heads*16*head_dim contiguous elements.
 * FP8 pools (PA_CACHE_FP8): one byte per element, laid out so that one 16-byte
 * lane load holds the operands of two matrix-core steps:
 *   K pool: [num_blocks][num_kv_heads][head_dim/64][16][4][2][8]
 *           token t, dim d at [b][h][d/64][t][(d%32)/8][(d%64)/32][d%8]
 *   V pool: [num_blocks][num_kv_heads][4][head_dim/64][16][2][2][4]
 *           token t, dim d at [b][h][t/4][d/64][(d%32)/2][(d%64)/32][d%2][t%4]
 * Slot encoding: slot = physical_block * 16 + position_in_block.
 * Query-to-KV head map: query head h reads KV head h / (num_heads/num_kv_heads).
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,   /* null pointer, bad shape, misaligned buffer, bad id   */
  PA_ERR_UNSUPPORTED = 2,   /* valid but not implemented (head_dim, dtype, group)   */
  PA_ERR_OUT_OF_BLOCKS = 3, /* block manager: the free list cannot satisfy a call  */
  PA_ERR_WORKSPACE = 4,     /* workspace smaller than pa_decode_workspace_size()    */
  PA_ERR_HIP = 5,           /* a HIP runtime call failed                            */
  PA_ERR_NOT_FOUND = 6      /* block manager: unknown sequence id                   */
} pa_status;

typedef enum pa_dtype { PA_F16 = 0, PA_BF16 = 1 } pa_dtype;

/* Block size of every pool (tokens per block); the pages' default. */
#define PA_BLOCK_SIZE 16
/* Tokens of context one decode workgroup covers before partitions are merged. */
#define PA_PARTITION_TOKENS 512

/* Hint for pa_cache.flags: blocks may be referenced by several sequences of one
 * call (shared prefixes).  The decode then reads K/V through the caches so that
 * sequences sharing a block can hit on it; without the hint it streams K/V with
 * non-temporal loads, which read HBM faster when every block is read once.
 * Results are the same bits either way. */
#define PA_CACHE_SHARED_BLOCKS 1

/* pa_cache.flags: the pools hold 8-bit floating-point codes (OCP E4M3: bias 7,
 * subnormals, 448 largest, 0x7F NaN) in the FP8 layout above, one float32 scale
 * per KV head for K (k_scales) and one for V (v_scales).  A stored element is
 * E4M3(fp32(x) / fp32(scale)), rounded to nearest even, saturated at +-448, NaN
 * stored as 0x7F; it stands for decode(code) * scale.  The pages only say that
 * the KV cache can be kept quantised, FP8 among the formats ("理解 vLLM
 * PagedAttention", version matrix, row "量化"); the format, the per-head scales
 * and the rounding are this library's reading.  dtype stays the dtype of q,
 * out and of the k / v given to pa_cache_write.  The attention calls widen the
 * codes exactly to dtype and fold k_scales into the score scale and v_scales
 * into the output. */
#define PA_CACHE_FP8 2

/* A KV pool pair.  k_cache and v_cache are device pointers in the layout above,
 * 16-byte aligned, each num_blocks*num_kv_heads*16*head_dim elements of dtype
 * (of one byte with PA_CACHE_FP8).  block_size must be 16; head_dim must be 64
 * or 128; flags is a combination of PA_CACHE_SHARED_BLOCKS and PA_CACHE_FP8.
 * k_scales / v_scales: device float32[num_kv_heads], 4-byte aligned, positive
 * finite (caller's contract), required with PA_CACHE_FP8 and ignored without. */
typedef struct pa_cache {
  void* k_cache;
  void* v_cache;
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;            /* pa_dtype */
  int32_t flags;            /* PA_CACHE_* */
  const float* k_scales;    /* PA_CACHE_FP8: per-KV-head scales of K, else NULL */
  const float* v_scales;    /* PA_CACHE_FP8: per-KV-head scales of V, else NULL */
} pa_cache;

/* ---------------------------------------------------------------------------
 * pa_cache_write -- slot-mapped store of new tokens' K and V.
 * Defined by: the current token's key and value are cached so later steps
 * reuse them ("vLLM 核心概念", section "为什么需要 KV Cache？"), in the block the
 * table names for that position ("vLLM 核心概念", section "按需分配").
 *   k, v          device, [num_tokens][num_kv_heads][head_dim] packed (no padding
 *                 between tokens), cache dtype, 16-byte aligned.  FP8 pools store
 *                 their quantised codes (see PA_CACHE_FP8).
 *   slot_mapping  device, int64[num_tokens]; token i is stored at slot
 *                 slot_mapping[i].  A negative slot skips the token; a slot at or
 *                 beyond num_blocks*16 is skipped too.
 *   num_tokens    >= 0; 0 enqueues nothing.
 * Two tokens mapped to one slot in the same call: either may win.
 * Errors: PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_HIP.
 * ------------------------------------------------------------------------- */
pa_status pa_cache_write(const pa_cache* cache, const void* k, const void* v,
                         const int64_t* slot_mapping, int32_t num_tokens, void* stream);

/* ---------------------------------------------------------------------------
 * pa_copy_blocks -- copy-on-write block copy.
 * Defined by: sequences that share a prompt point at the same physical blocks
 * and a new block is taken only when later tokens diverge, as in copy-on-write
 * ("理解 vLLM PagedAttention", section 六; "PagedAttention 实战", section
 * "PagedAttention 的核心", item 3).  For every pair (src, dst) the whole K block
 * and V block dst (all heads, all 16 positions) become bit-identical copies of
 * block src.
 *   pairs       device, int32[num_pairs][2] = (src, dst).
 *   pairs_host  optional host copy of the same pairs (may be NULL).  When given,
 *               it is checked: ids in [0, num_blocks), destinations distinct, no
 *               destination also a source; a violation returns
 *               PA_ERR_INVALID_ARG and enqueues nothing.  Without it these
 *               preconditions are the caller's (the block manager's lists
 *               always satisfy them); out-of-range pairs are skipped on device.
 *   num_pairs   >= 0; 0 enqueues nothing.
 * Errors: PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_HIP.
 * ------------------------------------------------------------------------- */
pa_status pa_copy_blocks(const pa_cache* cache, const int32_t* pairs,
                         const int32_t* pairs_host, int32_t num_pairs, void* stream);

/* ---------------------------------------------------------------------------
 * pa_decode_workspace_size -- bytes of workspace pa_decode needs.
 * Long contexts are split into partitions, each covered by one workgroup, whose
 * partial softmax states (max, sum, unnormalised output; float32) are kept in
 * the workspace and merged by log-sum-exp ("PagedAttention 实战", section
 * "2026 年的新变化": sequence split).  A launch uses partitions of 4096, 2048
 * or 1024 tokens -- the longest for which even the longest possible list of
 * items gives every workgroup slot of the device (three per compute unit) two
 * of them -- else of PA_PARTITION_TOKENS (512) tokens; the size returned
 * covers every choice.  Layout: int32 counters[num_seqs * num_heads + 1]
 * (padded to 256 bytes), then the states.  The last counter hands out the
 * places of the attention pass's item list beyond the first round of
 * workgroups: a workgroup that starts later takes the next unclaimed place, so
 * the items go to whichever slots free first.  When a call is given no
 * workspace, workgroup i takes place i.
 * The counters must be zero before a workspace's first use (allocate it
 * zero-filled); every completed call leaves them zero.  Returns 0 when
 * max_context_len <= PA_PARTITION_TOKENS (no merge) and for invalid arguments.
 * ------------------------------------------------------------------------- */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                int32_t max_context_len);

/* ---------------------------------------------------------------------------
 * pa_decode -- single-query paged decode attention (attention pass, then merge).
 * Defined by: each decode step reads the cached K/V of all history tokens
 * ("PagedAttention 实战", section "Decode：逐 token 生成输出"; "理解 vLLM
 * PagedAttention", section 七) through the block table ("vLLM 核心概念", section
 * "逻辑视图与物理视图分离").  For sequence b with context n_b = context_lens[b]
 * and query head h (KV head g = h / (num_heads/num_kv_heads)):
 *     s_t = scale * <q[b,h,:], K_b[t,g,:]>,  t = 0 .. n_b-1
 *     out[b,h,:] = sum_t softmax(s)_t * V_b[t,g,:]
 * where K_b[t] is token t % 16 of block block_tables[b][t / 16].  Scores,
 * softmax and accumulation are float32; out is rounded to the cache dtype
 * (round to nearest even).  The reduction order depends only on logical token
 * positions, so the result is bit-identical for any placement of the blocks.
 *   q, out              device, [num_seqs][num_heads][head_dim], cache dtype,
 *                       16-byte aligned.
 *   block_tables        device, int32[num_seqs][max_blocks_per_seq].
 *   context_lens        device, int32[num_seqs], each in [1, max_context_len].
 *   max_context_len     host bound on every context length, <= 16*max_blocks_per_seq.
 *   num_heads           a multiple of num_kv_heads.  With more than 16 query heads
 *                       per KV head (one matrix-core tile holds 16), the call runs
 *                       the kernels of pa_chunk_attention with one query per
 *                       sequence, their key-partition states in the workspace past
 *                       its counters; pa_decode_fused then stores the new tokens in
 *                       a launch of their own (slots stored as given), and
 *                       pa_decode_attention does the whole computation, leaving
 *                       nothing to pa_decode_merge.
 *   workspace           device, >= pa_decode_workspace_size(...) bytes, 16-byte
 *                       aligned, counters zero (may be NULL when that size is 0).
 * When every sequence has at most 8 partitions the merge runs inside the
 * attention pass: the last workgroup of a (sequence, KV head) to finish, found
 * with the workspace counter, combines the partitions (one launch); otherwise
 * a second launch merges.  Calls that share a workspace must not overlap.
 * A sequence with context length outside [1, max_context_len] or a block id
 * outside [0, num_blocks) gets NaN in its output rows.
 * Errors: PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP.
 * ------------------------------------------------------------------------- */
pa_status pa_decode(const pa_cache* cache, const void* q, int32_t num_seqs, int32_t num_heads,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t max_context_len, float scale,
                    void* out, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * pa_decode_noalloc -- pa_decode without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine).  Its scratch (the merge
 * counters and the partition states pa_decode keeps in the workspace) is a
 * device array of PA_NOALLOC_SCRATCH_BYTES inside the library: each GPU the call
 * runs on holds one until the process ends, and the first call on a device looks
 * up its address there (the current device; `stream` must belong to it).
 *   - A call whose pa_decode_workspace_size(num_seqs, num_heads, head_dim,
 *     max_context_len) exceeds PA_NOALLOC_SCRATCH_BYTES returns PA_ERR_WORKSPACE
 *     and enqueues nothing.
 *   - Each call first zeroes the counters with a small kernel (no memset node),
 *     then runs pa_decode's kernels on the scratch: the same bits as pa_decode.
 *   - Every call on one GPU shares that GPU's array, which keeps the last call's
 *     contents: calls that may overlap on one GPU (other streams, other host
 *     threads) race and must be serialised by the caller.
 * Arguments and errors otherwise as pa_decode.
 * ------------------------------------------------------------------------- */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
pa_status pa_decode_noalloc(const pa_cache* cache, const void* q, int32_t num_seqs,
                            int32_t num_heads, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t max_context_len, float scale, void* out, void* stream);

/* ---------------------------------------------------------------------------
 * pa_decode_partitioned -- pa_decode with the context partition length fixed by
 * the caller.  Defined by: a long context is split into pieces that separate
 * workgroups attend over, and the pieces' results are combined by log-sum-exp
 * ("PagedAttention 实战", section "2026 年的新变化": sequence split).
 * pa_decode picks the partition length per launch from the batch shape and the
 * device's compute-unit count, and the float32 rounding of the merge depends
 * on it; a fixed length gives results that are bit-identical on any device and
 * reproduces a stated split (e.g. 512-token partitions).
 *   partition_tokens   512, 1024, 2048 or 4096 (0: chosen per launch, as pa_decode).
 * Every other argument, the workspace rule (pa_decode_workspace_size covers every
 * length) and the merge placement are as pa_decode.  More than 16 query heads per
 * KV head with a non-zero partition_tokens: PA_ERR_UNSUPPORTED.  Any other length:
 * PA_ERR_INVALID_ARG.
 * ------------------------------------------------------------------------- */
pa_status pa_decode_partitioned(const pa_cache* cache, const void* q, int32_t num_seqs,
                                int32_t num_heads, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* context_lens,
                                int32_t max_context_len, float scale, int32_t partition_tokens,
                                void* out, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Grouped decode -- pa_decode for a batch in which groups of sequences share the
 * leading blocks of their block tables: samples or beams forked from one prompt
 * point those logical blocks at the same physical blocks ("理解 vLLM
 * PagedAttention", section 六; "vLLM 核心概念", section "内存共享").  Same result as
 * pa_decode (the same formula, every sequence over its whole context; a different
 * float32 summation order, so not the same bits), but each shared block is read
 * once per group: one work item scores it against the query heads of every member
 * (at most 16 query heads per KV head in a group, i.e. 16 / G members).
 *
 * pa_group_plan (host only) finds the groups and the work items:
 *   tables           host int32[num_seqs][max_blocks_per_seq], the batch's tables.
 *   context_lens     host int32[num_seqs], each in [1, max_context_len].
 *   min_items        items (over all KV heads) to aim for when choosing the
 *                    partition length (the decode step asks for 2 per compute
 *                    unit: longer items pay their start-up fewer times).
 *   plan             host int32 buffer of plan_bytes >= pa_group_plan_bytes(...).
 *   *plan_ints       receives the plan's length in int32s, or 0 when grouping would
 *                    save less than a tenth of the block reads (use pa_decode then)
 *                    or cannot be expressed (query groups wider than 16, lists
 *                    too long for the workspace).
 * Groups: sequences whose first block is the same physical block, in sequence order,
 * cut into chunks of 16 / G; each group shares its members' longest common table
 * prefix.  A group's block list is its shared blocks, then every member's own
 * blocks; it is cut into partitions of 32..256 blocks (the longest that still gives
 * min_items items and fits the workspace's states).  Plan layout (int32): header
 * [groups, item pairs, partition blocks, max partitions, num_seqs, 0, 0, 0]; per
 * group [first member, members, shared blocks, list blocks, partitions, longest
 * context, 0, 0]; per member [sequence, offset of its own blocks in the list after
 * the shared ones, blocks, context length]; per item pair (group << 12 | partition),
 * largest first.  Errors: PA_ERR_INVALID_ARG (nothing written).
 *
 * pa_decode_grouped runs the plan: one workgroup per (item pair, KV head).
 *   plan / plan_host  the plan in device memory (a copy of plan_host) and on the host.
 *   block_tables      device copy of the tables the plan was made from; the context
 *                     lengths are the plan's.
 *   workspace         >= pa_decode_workspace_size(num_seqs, num_heads, head_dim,
 *                     max_context_len) bytes, counters zero (may be NULL when every
 *                     group has one partition); the partitions of a (group, KV
 *                     head) are merged by the last of them to finish.
 * plan_host is checked whole before the launch (every member a sequence of this
 * batch with a context in [1, max_context_len] and the matching block count, every
 * group's list length, partitions and items consistent): a plan that fails is
 * PA_ERR_INVALID_ARG.  The device copy must equal it.  A block id outside
 * [0, num_blocks) poisons its group's rows with NaN.  No cache write is fused
 * (call pa_cache_write first).  Other arguments and errors as pa_decode.
 * ------------------------------------------------------------------------- */
size_t pa_group_plan_bytes(int32_t num_seqs, int32_t max_context_len);
pa_status pa_group_plan(const int32_t* tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, int32_t max_context_len, int32_t num_heads,
                        int32_t num_kv_heads, int32_t min_items, int32_t* plan, size_t plan_bytes,
                        int32_t* plan_ints);
pa_status pa_decode_grouped(const pa_cache* cache, const void* q, int32_t num_seqs,
                            int32_t num_heads, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, int32_t max_context_len,
                            const int32_t* plan, const int32_t* plan_host, float scale, void* out,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * pa_decode_fused -- the step's cache write and its decode in one attention pass.
 * Same result as pa_cache_write(cache, k_new, v_new, slot_mapping, num_seqs)
 * followed by pa_decode(...), when token i (k_new[i], v_new[i], [Hkv][D]) is
 * the newest token of sequence i: its slot is the last context position,
 *     slot_mapping[i] == block_tables[i][(n_i - 1) / 16] * 16 + (n_i - 1) % 16,
 * which is what the block manager's append returns.  The wave that reads that
 * position puts the token into the tile it loaded and stores it to the cache
 * from there, so no separate cache-write launch runs and nothing waits for the
 * store.
 *   slot_mapping[i] < 0    the token is not stored (the cache is read as is);
 *   any other mismatch     the token is not stored and sequence i's output is NaN;
 *   invalid context length sequence i's output is NaN and its token is not stored.
 * Arguments otherwise as pa_cache_write and pa_decode.
 * ------------------------------------------------------------------------- */
pa_status pa_decode_fused(const pa_cache* cache, const void* k_new, const void* v_new,
                          const int64_t* slot_mapping, const void* q, int32_t num_seqs,
                          int32_t num_heads, const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t max_context_len, float scale,
                          void* out, void* workspace, size_t workspace_bytes, void* stream);

/* The two stages of pa_decode as separate launches, for callers that time or
 * schedule them apart.  pa_decode_attention is the attention pass: one
 * workgroup per (sequence, KV head, partition) walks its blocks with an online
 * softmax.  For a sequence with one partition it writes out[] itself;
 * otherwise it writes the partition's float32 state (max in log2 units of the
 * scaled score, sum, unnormalised output) to the workspace and never merges.
 * pa_decode_merge combines those states by log-sum-exp and writes out[] for
 * every sequence with more than one partition; it must be given the same
 * num_seqs, num_heads and max_context_len (hence the same partition length).
 * Same arguments and errors as pa_decode; pa_decode_merge is a no-op when
 * there is a single partition. */
pa_status pa_decode_attention(const pa_cache* cache, const void* q, int32_t num_seqs,
                              int32_t num_heads, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* context_lens,
                              int32_t max_context_len, float scale, void* out, void* workspace,
                              size_t workspace_bytes, void* stream);
pa_status pa_decode_merge(const pa_cache* cache, int32_t num_seqs, int32_t num_heads,
                          const int32_t* context_lens, int32_t max_context_len, void* out,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Status name; never NULL. */
const char* pa_status_string(pa_status status);
/* Detail of the last failed call on this thread ("" if none). */
const char* pa_last_error(void);

/* ===========================================================================
 * Host block manager (pure host code, no device calls; not thread-safe).
 * Defined by: blocks come from one global pool, a sequence appends blocks as it
 * grows and returns them when it ends, and several sequences may point logical
 * blocks at one physical block ("理解 vLLM PagedAttention", section 三); a block
 * is taken exactly when the last one is full, the first token included
 * ("vLLM 核心概念", section "按需分配"; "理解 vLLM PagedAttention", section 四);
 * forked sequences share blocks and copy one only on divergence (same page,
 * section 六).  Policies the pages leave open:
 *   - the free list is a LIFO stack that starts as `free_order` (NULL = 0,1,2..)
 *     and pops free_order[0] first; freed blocks are pushed on top;
 *   - freeing a sequence drops one reference per block, last logical block
 *     first, pushing each block whose count reaches zero;
 *   - an append into a shared (refcount > 1), partially filled last block
 *     takes a fresh block and reports (old, new) as a copy-on-write pair; the
 *     old block loses a reference; the last sharer writes in place;
 *   - a failing append or batch changes nothing.
 * Block size ("vLLM 核心概念", section 块大小（Block Size）的选择: smaller blocks
 * waste less memory, larger ones need fewer table entries): 16 or 32 tokens.  A
 * 32-token manager block b is the pool's two 16-token blocks (tiles) 2 b and
 * 2 b + 1, so the pool holds 2 * num_blocks tiles and the kernels are unchanged:
 * slots keep their numbering (32 b + i is tile 2 b + i / 16, position i % 16);
 * pa_bm_pack and pa_bm_step write tables in tiles (max_blocks counts tiles);
 * copy-on-write pairs from the append calls are in manager blocks, a pair (s, d)
 * meaning tile copies (2 s, 2 d) and (2 s + 1, 2 d + 1) (pa_bm_tile_pairs expands
 * them; pa_decode_step does so itself).  Prefix caching and swapping need 16-token
 * blocks.
 * ======================================================================== */
typedef struct pa_bm pa_bm;

typedef struct pa_bm_stats {
  int64_t num_blocks;
  int64_t free_blocks;
  int64_t used_blocks;      /* refcount > 0 */
  int64_t shared_blocks;    /* refcount > 1 */
  int64_t allocated_slots;  /* used_blocks * 16 */
  int64_t occupied_slots;   /* per used block, the most tokens any sharer keeps in it */
  double waste;             /* 1 - occupied/allocated (0 when nothing is allocated) */
} pa_bm_stats;

pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                       pa_bm** out);
void pa_bm_destroy(pa_bm* bm);
pa_status pa_bm_add_seq(pa_bm* bm, int64_t seq_id);
/* Reserve the slot of the next token of one sequence.  cow_src and cow_dst receive
 * -1 unless this append copied a shared block. */
pa_status pa_bm_append(pa_bm* bm, int64_t seq_id, int64_t* slot, int32_t* cow_src,
                       int32_t* cow_dst);
/* One token for each of n distinct sequences, in order, all or nothing.
 * slots: int64[n].  cow_pairs: int32[cow_cap][2]; *n_cow receives the count
 * (at most n; cow_cap >= n guarantees room, else PA_ERR_INVALID_ARG). */
pa_status pa_bm_append_batch(pa_bm* bm, int32_t n, const int64_t* seq_ids, int64_t* slots,
                             int32_t* cow_pairs, int32_t cow_cap, int32_t* n_cow);
/* count tokens appended to one sequence (a prefill), each one an append;
 * all or nothing.  slots: int64[count]; cow pairs as above (at most count). */
pa_status pa_bm_append_tokens(pa_bm* bm, int64_t seq_id, int32_t count, int64_t* slots,
                              int32_t* cow_pairs, int32_t cow_cap, int32_t* n_cow);
pa_status pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child);
pa_status pa_bm_free_seq(pa_bm* bm, int64_t seq_id);
pa_status pa_bm_seq_len(const pa_bm* bm, int64_t seq_id, int64_t* len);
/* Copy a sequence's table (logical order) to out[0..cap); *n = its length. */
pa_status pa_bm_block_table(const pa_bm* bm, int64_t seq_id, int32_t* out, int32_t cap,
                            int32_t* n);
/* Pack n sequences' tables into tables[n][max_blocks] (unused entries -1) and
 * their lengths into ctx_lens[n]. */
pa_status pa_bm_pack(const pa_bm* bm, int32_t n, const int64_t* seq_ids, int32_t* tables,
                     int32_t max_blocks, int32_t* ctx_lens);
pa_status pa_bm_refcount(const pa_bm* bm, int32_t block, int32_t* out);
/* Free blocks, next-to-pop first, into out[0..cap); *n = how many are free. */
pa_status pa_bm_free_list(const pa_bm* bm, int32_t* out, int32_t cap, int32_t* n);
pa_status pa_bm_stats_get(const pa_bm* bm, pa_bm_stats* out);
/* One decode step's host work for n distinct sequences: pa_bm_append_batch, then
 * pa_bm_pack into tables[n][max_blocks] and ctx_lens[n]; *max_ctx receives the
 * longest context.  All or nothing: fails before any change when a table would
 * outgrow max_blocks after its append. */
pa_status pa_bm_step(pa_bm* bm, int32_t n, const int64_t* seq_ids, int64_t* slots,
                     int32_t* cow_pairs, int32_t cow_cap, int32_t* n_cow, int32_t* tables,
                     int32_t max_blocks, int32_t* ctx_lens, int32_t* max_ctx);
/* Copy-on-write pairs of manager blocks (n pairs, host int32[n][2]) as the pairs of
 * pool tiles that pa_copy_blocks takes: the same pairs with 16-token blocks; with
 * 32-token blocks each pair (s, d) becomes (2 s, 2 d), (2 s + 1, 2 d + 1), in order.
 * tile_pairs (host int32[cap][2]) may be `pairs` itself (expanded in place);
 * *n_tiles receives the number of tile pairs.  PA_ERR_INVALID_ARG when cap is too
 * small (nothing written). */
pa_status pa_bm_tile_pairs(const pa_bm* bm, const int32_t* pairs, int32_t n, int32_t* tile_pairs,
                           int32_t cap, int32_t* n_tiles);

/* ---------------------------------------------------------------------------
 * Automatic prefix caching (host only).  A request whose leading tokens equal an
 * earlier request's reuses the blocks computed for them and skips their prefill
 * ("vLLM 核心概念", section 前缀缓存（Prefix Caching）, automatic matching;
 * "PagedAttention 实战", section "Prefix Caching：让相同前缀不要反复算"); the
 * system keeps block references, an index, a lifecycle and an eviction policy
 * ("理解 vLLM PagedAttention", section 六), with hit-rate statistics, tenant
 * isolation and invalidation when the model changes ("PagedAttention 实战",
 * Prefix Caching and its fifth step).  Policies the pages leave open:
 *   - the unit of reuse is a full block, identified exactly by the tenant and
 *     the whole token prefix through its last token (a block's K/V depend on
 *     every earlier token), never by its own 16 tokens alone;
 *   - a block is indexed when its 16th token id is committed, unless its prefix
 *     is already indexed (then it stays private) or it is indexed already; an
 *     indexed block is full and is never written again;
 *   - a new request matches its prompt's full blocks from the first, stopping
 *     at the first miss, at most floor((n - 1) / 16) of them, so that at least
 *     one prompt token is left to compute; each hit takes a reference;
 *   - an indexed block whose last reference goes keeps its contents and becomes
 *     evictable; other blocks return to the free stack;
 *   - allocation pops the free stack first and only then evicts the evictable
 *     block released longest ago (LRU; a freed sequence releases its tail block
 *     first, so tails are evicted before heads); eviction drops the index entry;
 *   - reset (a model change) drops every index entry and pushes the evictable
 *     blocks onto the free stack, oldest release first.
 * Capacity checks of the append calls count free and evictable blocks.
 * ------------------------------------------------------------------------- */
typedef struct pa_bm_prefix_stats {
  int64_t requests;          /* pa_bm_add_seq_cached calls */
  int64_t query_blocks;      /* full blocks they were allowed to look up */
  int64_t hit_blocks;        /* blocks they reused (hit rate = hit / query) */
  int64_t cached_blocks;     /* blocks in the index now (any refcount) */
  int64_t evictable_blocks;  /* indexed blocks with refcount 0 */
  int64_t evictions;         /* index entries dropped to hand a block out */
} pa_bm_prefix_stats;

/* Turn prefix caching on; only while no sequence is live (PA_ERR_INVALID_ARG
 * otherwise).  The calls below return PA_ERR_UNSUPPORTED until it is on. */
pa_status pa_bm_enable_prefix_cache(pa_bm* bm);
/* Create sequence seq_id for a prompt of n token ids (host int32[n]) under
 * tenant >= 0 (a prefix only matches blocks committed under the same tenant).
 * The sequence starts holding the matched blocks; *cached_tokens receives their
 * token count (a multiple of 16, < n when n > 0), and those tokens count as
 * committed.  The caller then appends (pa_bm_append_tokens) and computes the
 * other n - *cached_tokens tokens. */
pa_status pa_bm_add_seq_cached(pa_bm* bm, int64_t seq_id, int64_t tenant, const int32_t* tokens,
                               int32_t n, int32_t* cached_tokens);
/* Admission of n requests in one call (what a serving loop does per step): for
 * each i in order, pa_bm_add_seq_cached(seq_ids[i], tenants[i] (tenants NULL:
 * all 0), prompt i), pa_bm_append_tokens of the prompt's other tokens and
 * pa_bm_commit_tokens of their ids.  Prompt i is tokens[offsets[i] ..
 * offsets[i+1]) (offsets: int64[n + 1], non-decreasing); a later request can
 * reuse blocks an earlier one of the same call filled, so the caller stores the
 * new tokens' K/V (one pa_cache_write of all of them) before any attention
 * reads them.  cached: int32[n] reused tokens per request; slots: the new
 * tokens' slots, request after request (slot_cap >= offsets[n] - offsets[0]
 * always suffices).  *admitted receives how many requests (a prefix of the
 * list) were admitted: on PA_ERR_OUT_OF_BLOCKS request *admitted was not (its
 * matched blocks are released again) and the ones after it were not tried.
 * Argument errors are found before anything changes. */
pa_status pa_bm_admit_batch(pa_bm* bm, int32_t n, const int64_t* seq_ids, const int64_t* tenants,
                            const int32_t* tokens, const int64_t* offsets, int32_t* cached,
                            int64_t* slots, int64_t slot_cap, int32_t* admitted);
/* Token ids of a sequence's next `count` appended but uncommitted slots, in
 * order, once their K/V are written; full blocks enter the index here.  More
 * ids than uncommitted slots: PA_ERR_INVALID_ARG, nothing changes.  pa_bm_add_seq
 * sequences commit under tenant 0; forks inherit the parent's tenant and
 * committed ids. */
pa_status pa_bm_commit_tokens(pa_bm* bm, int64_t seq_id, const int32_t* tokens, int32_t count);
/* One id for each of n distinct sequences (a decode step); all or nothing. */
pa_status pa_bm_commit_batch(pa_bm* bm, int32_t n, const int64_t* seq_ids, const int32_t* tokens);
pa_status pa_bm_prefix_cache_reset(pa_bm* bm);
pa_status pa_bm_prefix_stats_get(const pa_bm* bm, pa_bm_prefix_stats* out);
/* Evictable blocks, next to evict first, into out[0..cap); *n = how many. */
pa_status pa_bm_evictable_list(const pa_bm* bm, int32_t* out, int32_t cap, int32_t* n);
/* Indexed blocks in ascending order, into out[0..cap); *n = how many. */
pa_status pa_bm_cached_list(const pa_bm* bm, int32_t* out, int32_t cap, int32_t* n);

/* ---------------------------------------------------------------------------
 * Swapping between the device pool and a host tier (host only; the copies are
 * pa_swap_blocks).  Blocks that do not fit in GPU memory spill to CPU memory and
 * come back when needed ("vLLM 核心概念", section 内存层次结构); preemption is the
 * fallback when resources run short ("理解 vLLM PagedAttention", section 五).
 * Policies the pages leave open:
 *   - the host tier is a pool of num_host_blocks blocks of the device pool's
 *     shape, with a LIFO free stack starting as host_free_order (NULL = 0, 1, ..)
 *     and its own reference counts;
 *   - pa_bm_swap_out moves the n listed resident sequences to the host tier at
 *     once: each distinct device block they reference (order of first
 *     appearance: list order, then logical order) gets one host block, so blocks
 *     they share stay shared; pairs[i] = (device block, host block) to copy
 *     (pa_swap_blocks, PA_SWAP_OUT) before the released device blocks are
 *     written again; then the sequences drop their device references, one after
 *     the other, last logical block first; a block that a resident sequence
 *     still references keeps its device copy;
 *   - pa_bm_swap_in is the mirror image (device blocks taken as an append takes
 *     them, so cached prefix blocks may be evicted; pairs = (host block, device
 *     block), to copy with PA_SWAP_IN before the sequences are read);
 *   - both are all or nothing (PA_ERR_OUT_OF_BLOCKS when the target tier lacks
 *     blocks); pair_cap must hold the distinct blocks (the listed sequences'
 *     table lengths summed always suffice), else PA_ERR_INVALID_ARG;
 *   - a swapped-out sequence is not resident: growing, forking, committing or
 *     packing it gives PA_ERR_NOT_FOUND; pa_bm_free_seq releases its host blocks
 *     and pa_bm_seq_len still answers.
 * ------------------------------------------------------------------------- */
pa_status pa_bm_enable_swap(pa_bm* bm, int32_t num_host_blocks, const int32_t* host_free_order);
pa_status pa_bm_swap_out(pa_bm* bm, int32_t n, const int64_t* seq_ids, int32_t* pairs,
                         int32_t pair_cap, int32_t* n_pairs);
pa_status pa_bm_swap_in(pa_bm* bm, int32_t n, const int64_t* seq_ids, int32_t* pairs,
                        int32_t pair_cap, int32_t* n_pairs);
/* *out = 1 when the sequence is swapped out, 0 when resident. */
pa_status pa_bm_is_swapped(const pa_bm* bm, int64_t seq_id, int32_t* out);
/* A swapped-out sequence's host blocks, in logical order; *n = how many. */
pa_status pa_bm_host_table(const pa_bm* bm, int64_t seq_id, int32_t* out, int32_t cap, int32_t* n);
pa_status pa_bm_host_refcount(const pa_bm* bm, int32_t block, int32_t* out);
/* Free host blocks, next-to-pop first. */
pa_status pa_bm_host_free_list(const pa_bm* bm, int32_t* out, int32_t cap, int32_t* n);

/* ---------------------------------------------------------------------------
 * pa_swap_blocks -- block copies between the device pools and host pools.
 * Defined by: KV blocks move between GPU memory and CPU memory ("vLLM 核心概念",
 * section 内存层次结构).  `host` describes pools of the device pools' layout,
 * dtype, head count, head size and FP8 scales, whose k_cache / v_cache are
 * pinned host memory mapped for the device (as hipHostMalloc returns); its
 * num_blocks is the host pool's size.  For every pair the whole K and V block
 * (all heads, 16 positions) is copied: PA_SWAP_OUT copies device block
 * pairs[i][0] to host block pairs[i][1], PA_SWAP_IN host block pairs[i][0] to
 * device block pairs[i][1].  One kernel moves every pair over the host link.
 *   pairs       int32[num_pairs][2], device-readable (device or mapped memory).
 *   pairs_host  optional host copy, checked as in pa_copy_blocks (ids in range
 *               of their pools, destinations distinct); without it
 *               out-of-range pairs are skipped on the device.
 * Errors: PA_ERR_INVALID_ARG (layouts differ, bad direction or pairs),
 * PA_ERR_UNSUPPORTED (more than 65535 pairs), PA_ERR_HIP.
 * ------------------------------------------------------------------------- */
#define PA_SWAP_OUT 0
#define PA_SWAP_IN 1
pa_status pa_swap_blocks(const pa_cache* device, const pa_cache* host, int32_t direction,
                         const int32_t* pairs, const int32_t* pairs_host, int32_t num_pairs,
                         void* stream);

/* ---------------------------------------------------------------------------
 * pa_chunk_attention -- several new tokens per sequence: the last q_len_b of
 * sequence b's context_lens[b] cached tokens are queries, and query i (position
 * context_lens[b] - q_len_b + i) attends over cached positions 0 .. its own.
 * That is a prefill chunk ("vLLM 核心概念", section "Chunked Prefill";
 * "PagedAttention 实战", section "Chunked Prefill：长 prompt 不要一次吃完全部预算")
 * or the tokens of a speculative verify ("vLLM 核心概念", section "推测解码
 * （Speculative Decoding）"); with q_len 1 it is the decode of pa_decode.  The new
 * tokens' K/V must be in the cache already (pa_cache_write).
 *   q, out           device, [total_q][num_heads][head_dim], cache dtype (FP8
 *                    pools: the descriptor's dtype), 16-byte aligned; sequence b
 *                    owns rows q_starts[b] .. q_starts[b+1].
 *   q_starts         device, int32[num_seqs + 1], non-decreasing, q_starts[0] >= 0,
 *                    q_starts[num_seqs] <= total_q; every q_len at most max_q_len
 *                    (rows past max_q_len of a longer one are not written).
 *   block_tables, context_lens, max_context_len, max_blocks_per_seq: as pa_decode.
 *   workspace        device, >= pa_chunk_workspace_size(...) bytes, 16-byte aligned
 *                    (NULL when that size is 0).
 *   attn_begin, attn_end  optional hipEvent_t (NULL to skip), attached to the
 *                    dispatches: the start of the attention kernel and the end of
 *                    the call's last kernel (the merge, when there is one).
 * One workgroup per (sequence, KV head, 16-48 (token, head) columns, key
 * partition), sequences taken longest first when there are at most 48 columns
 * and the launch gives each workgroup slot at most 4 items;
 * when the column groups alone do not fill the device, keys are split
 * into partitions of 1024, 2048 or 4096 tokens (the longest that still gives
 * every workgroup slot two items).  A sequence whose context fits one partition
 * is written directly; the partition states of the others are merged by
 * log-sum-exp in a second launch ("PagedAttention 实战", section "2026 年的新变化").
 * A sequence whose rows
 * fall outside [0, total_q] is skipped (nothing written); one with a context
 * length outside [1, max_context_len] or more new tokens than cached ones gets
 * NaN rows; a block id outside [0, num_blocks) poisons (NaN) the rows of every
 * column group that reads it.
 * Errors: PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP.
 * ------------------------------------------------------------------------- */
size_t pa_chunk_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t total_q, int32_t max_q_len,
                               int32_t max_context_len);
pa_status pa_chunk_attention(const pa_cache* cache, const void* q, const int32_t* q_starts,
                             int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                             int32_t num_heads, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* context_lens,
                             int32_t max_context_len, float scale, void* out, void* workspace,
                             size_t workspace_bytes, void* attn_begin, void* attn_end,
                             void* stream);

/* ===========================================================================
 * pa_decode_step -- one whole decode step of a batch, in one call.
 * The order a decode step needs: the new token's K/V is stored before attention
 * reads every cached token ("vLLM 核心概念", section "为什么需要 KV Cache？"),
 * and a sequence about to write into a shared block first gets its own copy
 * ("理解 vLLM PagedAttention", section 六).  The call
 *   1. runs pa_bm_step for seq_ids on the host, writing slots, lengths, tables
 *      and copy-on-write pairs into staging_host (pinned host memory) in the
 *      layout below;
 *   2. enqueues one copy of that region to staging_dev (device memory) -- on
 *      `stream`, or, when copy_stream is given, on copy_stream, so the copy can
 *      run while earlier work of `stream` still runs, and records copy_event (a
 *      hipEvent_t) there.  The call then waits on the host for copy_event before
 *      it enqueues the kernels (a wait placed in `stream`, like a query of
 *      whether `stream` is busy, would cost queue time between the kernels).
 *      The host wait lasts as long as the copy and whatever copy_stream ran
 *      before it.  PA_STEP_STREAM_WAIT=1 in the environment makes `stream` wait
 *      for copy_event instead -- or, when
 *      staging_dev is NULL, nothing: the kernels read staging_host in place (it
 *      must then be pinned host memory mapped for the device, as hipHostMalloc
 *      returns);
 *   3. enqueues pa_copy_blocks (if any pair), then pa_decode_fused: the store
 *      of k_new/v_new ([num_seqs][num_kv_heads][head_dim], token i belongs to
 *      seq_ids[i]) and the decode, all on `stream`.  When the block manager
 *      holds shared blocks and pa_group_plan finds groups worth decoding
 *      together (its plan is made on the host from the packed tables and staged
 *      with them), the step enqueues pa_cache_write of the new tokens and then
 *      pa_decode_grouped instead of pa_decode_fused.
 * Staging layout (each part 256-byte aligned, both buffers 256-byte aligned and
 * at least pa_decode_step_staging_bytes() long): int64 slots[n] | int32 ctx[n] |
 * int32 tables[n][max_blocks_per_seq] | int32 pairs[2 n][2] (tile pairs) | int32
 * plan[pa_group_plan_bytes(n, 16 * max_blocks_per_seq) / 4].  staging_host must
 * not be rewritten while an earlier copy from it may still be pending, nor
 * staging_dev while kernels of an earlier step may still read it (the caller
 * alternates two buffers of each and waits on events; with copy_stream, it
 * makes copy_stream wait for the end of the step that last read staging_dev).
 * workspace: at least pa_decode_workspace_size(n, num_heads, head_dim,
 * 16 * max_blocks_per_seq) bytes.  attn_begin / attn_end: optional hipEvent_t
 * that take the start and end of the attention kernels themselves (attached to
 * their dispatches: the start of the attention kernel, the end of the last
 * launch of the pass), NULL to skip.  info (optional) receives
 * the number of copy-on-write pairs, the longest context of the step,
 * whether it decoded as groups and whether the host waited for the copy.
 * The decode reads through the caches (PA_CACHE_SHARED_BLOCKS) whenever the
 * block manager holds a block with more than one reference.
 * Every argument is checked before the block manager changes; after that only
 * PA_ERR_HIP can occur.
 * ========================================================================= */
typedef struct pa_step_info {
  int32_t num_cow;
  int32_t max_context_len;
  int32_t grouped;          /* 1: pa_decode_grouped ran, 0: pa_decode_fused */
  int32_t host_waited;      /* 1: the host waited for the copy on copy_stream */
} pa_step_info;

size_t pa_decode_step_staging_bytes(int32_t num_seqs, int32_t max_blocks_per_seq);
pa_status pa_decode_step(pa_bm* bm, const pa_cache* cache, int32_t num_seqs, const int64_t* seq_ids,
                         const void* k_new, const void* v_new, const void* q, int32_t num_heads,
                         float scale, void* out, void* workspace, size_t workspace_bytes,
                         void* staging_host, void* staging_dev, size_t staging_bytes,
                         int32_t max_blocks_per_seq, void* attn_begin, void* attn_end,
                         pa_step_info* info, void* copy_stream, void* copy_event, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
