/*
 * pa.h — C ABI of libpa: attention over a paged KV cache on MI355X (gfx950).
 *
 * Keys and values of every sequence live in fixed pages of 16 tokens.  A
 * per-sequence block table maps logical page j (tokens 16j .. 16j+15) to a
 * physical block of the pool ("第 15 章：推理引擎与部署" §15.6 "PagedAttention：
 * 分页 KV Cache"; "大模型部署.md" §2.1 item 4 "PageAttention 内存管理技术详解").
 * Attention is exact softmax(Q Kᵀ · scale) V computed with a tiled online
 * softmax ("第 15 章" §15.1 "算法详解"), over batches that mix single-token
 * decodes with causal prefill chunks ("DeepSpeed-FastGen 深度解析" §3.2,
 * Dynamic SplitFuse).
 *
 * Conventions for every entry point:
 *  - All integers are signed; sizes are element counts unless named *_bytes.
 *  - "device" pointers point to GPU memory owned by the caller; the library
 *    never allocates, frees or retains device memory.  "host" pointers point
 *    to CPU memory and are only read during the call.
 *  - Device work is enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream) and returns without synchronising.  Faults inside kernels
 *    surface at the caller's next synchronisation.
 *  - Argument errors are detected on the host before anything is enqueued;
 *    the call then returns a negative pa_status and pa_last_error() explains.
 *  - Facts only the device can see (block ids, slots, lengths read from device
 *    arrays) are checked by the kernels: an offending item is skipped (no
 *    out-of-range address is ever formed) and a PA_DEV_* bit is OR-ed into
 *    *dev_status when dev_status is not NULL.  The caller zeroes that int32
 *    before the call and reads it after synchronising.
 *
 * Pool layout (dtype T, X = 16 / sizeof(T): 4 for float32, 8 for bfloat16):
 *    k_cache  [num_blocks][num_kv_heads][head_dim / X][16][X]
 *    v_cache  [num_blocks][num_kv_heads][head_dim][16]
 *  Token o of physical block b, KV head h keeps key element e at
 *  k_cache[b][h][e / X][o][e % X] and value element e at v_cache[b][h][e][o].
 *  Each (block, head) page is one contiguous run of 16 * head_dim elements,
 *  so a 16-token page is read with fully coalesced 16-byte loads.
 *  A slot is block * 16 + offset.
 *
 * Supported: head_dim 64 or 128, block_size 16, num_q_heads a multiple of
 * num_kv_heads, dtype float32 or bfloat16 (q, caches and output share it;
 * accumulation is float32).
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
  PA_ERR_INVALID = -1,      /* bad argument (null pointer, bad size, bad id)          */
  PA_ERR_UNSUPPORTED = -2,  /* valid but not implemented (head_dim, block_size, dtype) */
  PA_ERR_NO_BLOCKS = -3,    /* allocator pool exhausted; allocator state unchanged     */
  PA_ERR_REFCOUNT = -4,     /* reference count would drop below zero                   */
  PA_ERR_NOT_FOUND = -5,    /* unknown sequence id                                     */
  PA_ERR_HIP = -6           /* the HIP runtime reported an error at launch             */
} pa_status;

typedef enum pa_dtype { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

typedef enum pa_alloc_status {
  PA_ALLOC_OK = 0,     /* enough free blocks now                        */
  PA_ALLOC_LATER = 1,  /* enough blocks exist, not enough are free now  */
  PA_ALLOC_NEVER = 2   /* the pool can never hold the request           */
} pa_alloc_status;

/* Bits OR-ed into *dev_status by kernels. */
#define PA_DEV_BAD_BLOCK 1   /* block id outside [0, num_blocks) (table entry or copy pair) */
#define PA_DEV_BAD_SLOT 2    /* slot outside [0, num_blocks * 16)                            */
#define PA_DEV_BAD_LENGTH 4  /* context length / query offsets inconsistent with the bounds  */
#define PA_DEV_BAD_POSITION 8 /* position outside [0, max_position) (rotary cache write)      */
#define PA_DEV_BAD_GROUP 16   /* a shared-prefix group failed its checks and was ignored        */

/* Message for the last failing call on this thread ("" if none).  Valid until
 * the next call into the library from the same thread. */
const char* pa_last_error(void);

/* ABI revision of this header; bumped on any incompatible change. */
int32_t pa_abi_version(void);

/* ------------------------------------------------------------------ cache write
 * pa_reshape_and_cache — store the new tokens' keys and values into the pool.
 * For every token t with slot_mapping[t] >= 0 and every KV head h:
 *   k_cache[slot/16][h][:][slot%16][:] = key[t][h][:]   (in the layout above)
 *   v_cache[slot/16][h][:][slot%16]    = value[t][h][:]
 * exact byte copies.  A negative slot marks a padding token and is skipped.
 * Slots must be distinct (overlapping writes race); a slot >= num_blocks*16
 * is skipped and flagged PA_DEV_BAD_SLOT.
 * (The new K/V enter the cache at each decode step, "【自用】AI infra相关" part
 * 一.2; slots index the KV storage directly like SGLang's out_cache_loc,
 * "大模型部署.md" §2.4 item 4.)
 *   key, value    device, [num_tokens][num_kv_heads][head_dim] of dtype
 *   k_cache, v_cache  device, pool layout above, num_blocks blocks
 *   slot_mapping  device, int64 [num_tokens]
 * PA_ERR_INVALID for num_kv_heads > 65535 (one launch dimension per head).
 */
pa_status pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                               const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               pa_dtype dtype, int32_t* dev_status, void* stream);

/* pa_rope_reshape_and_cache — the cache write with the rotary position
 * embedding applied on the way ("第 15 章：推理引擎与部署" §15.3, RoPE fused into
 * the kernels that read q and k, saving the round trip of the rotated tensors
 * through memory; "DeepSpeed-FastGen 深度解析" §6, rotary embedding fused with
 * the blocked KV layout).  For token t at position p = positions[t], with
 * c = cos_table[p], s = sin_table[p] (head_dim/2 floats each), every head row
 * x of q and of key is rotated pairwise (rotate-half form):
 *   x'[i] = x[i] c[i] - x[i + d/2] s[i],  x'[i + d/2] = x[i + d/2] c[i] + x[i] s[i]
 * in float32 (one rounded product and one fused multiply-add per element),
 * rounded to dtype.  The rotated q goes to q_out (q_out == q allowed); the
 * rotated key and the unchanged value are stored through slot_mapping[t] as
 * in pa_reshape_and_cache (negative slot: q is still rotated, nothing is
 * stored).  A position outside [0, max_position) skips the token entirely
 * (q_out row untouched) and sets PA_DEV_BAD_POSITION.
 *   q, q_out       device, [num_tokens][num_q_heads][head_dim] of dtype
 *   key, value     device, [num_tokens][num_kv_heads][head_dim] of dtype
 *   positions      device, int32 [num_tokens]
 *   cos_table, sin_table  device, float32 [max_position][head_dim / 2]
 * PA_ERR_INVALID for num_q_heads + num_kv_heads > 65535.
 */
pa_status pa_rope_reshape_and_cache(void* q_out, const void* q, const void* key, const void* value,
                                    void* k_cache, void* v_cache, const int64_t* slot_mapping,
                                    const int32_t* positions, const float* cos_table, const float* sin_table,
                                    int32_t max_position, int32_t num_tokens, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t num_blocks, int32_t head_dim,
                                    int32_t block_size, pa_dtype dtype, int32_t* dev_status, void* stream);

/* ------------------------------------------------------------------ attention
 * Workspace bytes pa_forward needs for a batch within these bounds.  The
 * workspace holds the per-call plan, work-queue counters and the partial
 * (m, l, O) states of split contexts; it needs no initialisation and its
 * content is meaningless between calls.
 */
size_t pa_forward_workspace_bytes(int32_t num_seqs, int32_t total_q_tokens, int32_t max_q_len,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_context_len, pa_dtype dtype);

/* pa_forward — paged attention over a ragged batch of sequences.
 * Sequence s owns query rows query_start_loc[s] .. query_start_loc[s+1]-1
 * (q_len rows, 0 <= q_len <= context_lens[s]) and sees context_lens[s] keys,
 * the new tokens included (write them with pa_reshape_and_cache first).
 * Row i of sequence s sits at position p = context_lens[s] - q_len + i and
 * attends keys 0..p: a decode row (q_len 1) sees the whole context, a prefill
 * chunk is causal inside itself.  Query head h reads KV head h / G with
 * G = num_q_heads / num_kv_heads ("大模型部署.md" §4.1 item 4, MQA/GQA).
 *   out[t][h][:] = Σ_j softmax_j(scale · q[t][h]·k_j) v_j      (rounded to dtype)
 * ("第7章：大模型部署实战" §2.2.2 formula; "第 15 章" §15.1).  Long contexts
 * are split into fixed key partitions processed by separate wavefronts and
 * merged exactly by log-sum-exp rescaling; partition boundaries depend only on
 * the sequence's own lengths, so a sequence's output does not depend on
 * what else is in the batch.
 *   out            device, [total_q_tokens][num_q_heads][head_dim] of dtype
 *   q              device, [total_q_tokens][num_q_heads][head_dim] of dtype
 *   k_cache, v_cache  device, pool layout above
 *   block_tables   device, int32 [num_seqs][max_blocks_per_seq]; entries past
 *                  ceil(context_len/16) are never read
 *   context_lens   device, int32 [num_seqs]
 *   query_start_loc device, int32 [num_seqs + 1], query_start_loc[0] = 0,
 *                  non-decreasing, query_start_loc[num_seqs] = total_q_tokens
 *   max_q_len, max_context_len  host-known upper bounds of the device arrays
 *                  (the launch is sized from them without reading the device)
 *   scale          softmax scale (1/sqrt(head_dim) for standard attention)
 *   workspace      device, >= pa_forward_workspace_bytes(...) bytes, 256-byte aligned
 * Output rows of sequences flagged by the device checks are not written.
 */
pa_status pa_forward(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, const int32_t* query_start_loc,
                     int32_t num_seqs, int32_t total_q_tokens, int32_t max_q_len,
                     int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                     pa_dtype dtype, void* workspace, size_t workspace_bytes,
                     int32_t* dev_status, void* stream);

/* pa_forward_shared — pa_forward for batches in which groups of decode
 * sequences share the pages of a common prefix (the samples of one prompt:
 * "大模型部署.md" §2.1 item 4 and "【自用】AI infra相关" part 二.2(1), sharing
 * between the samples of one prompt; "第 15 章" §15.6).  The result is the
 * same attention as pa_forward; what changes is the work: a shared page is
 * read once for all members of its group.  Each member's attention is split
 * at the shared length S into the shared keys, computed for all members
 * together as one MFMA tile (members x query heads of a KV head as rows),
 * and its own keys S .. L-1; the two partial softmax states are combined by
 * the log-sum-exp merge of split contexts ("第 15 章" §15.1 rescaling),
 * which is exact.
 *   groups  device, int32 [num_groups][3]: first sequence, number of members,
 *           shared keys S.  Members are the consecutive sequences first ..
 *           first + members - 1; groups are listed in increasing order and do
 *           not overlap.  A group is used only if: 2 <= members,
 *           members x (num_q_heads / num_kv_heads) <= 16, S > 0 is a multiple
 *           of 16 and at most max_context_len, every member is a single-row
 *           decode with context length >= S, and the first S/16 block-table
 *           entries of every member equal those of the first member.  Any
 *           other group is ignored (its members are attended as plain
 *           sequences, still correctly) and PA_DEV_BAD_GROUP is set.
 * Other arguments as pa_forward; workspace >= pa_forward_shared_workspace_bytes.
 * bfloat16 only, at most 8 query heads per KV head (PA_ERR_UNSUPPORTED). */
pa_status pa_forward_shared(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, const int32_t* query_start_loc,
                            const int32_t* groups, int32_t num_groups, int32_t num_seqs,
                            int32_t total_q_tokens, int32_t max_q_len, int32_t max_context_len,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t num_blocks, float scale, pa_dtype dtype,
                            void* workspace, size_t workspace_bytes, int32_t* dev_status, void* stream);
/* Workspace bytes of pa_forward_shared for these bounds and num_groups groups. */
size_t pa_forward_shared_workspace_bytes(int32_t num_seqs, int32_t num_groups, int32_t total_q_tokens,
                                         int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t max_context_len, pa_dtype dtype);

/* pa_forward_noalloc — pa_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation, with the workspace taken from a
 * static array the library holds on each GPU instead of a caller buffer.
 * Arguments as pa_forward without workspace/workspace_bytes.  The array holds
 * pa_forward_noalloc_max_workspace_bytes() bytes (64 MiB); a batch whose
 * pa_forward_workspace_bytes(...) exceeds it fails with PA_ERR_INVALID and
 * nothing is enqueued.  Nothing is allocated: the array lives in the library's
 * device data from load until the process ends, one per GPU; its device
 * address is looked up once per device (hipGetSymbolAddress, the first call
 * with that device current).  Every call on one GPU uses the same array, and
 * nothing in it needs clearing between calls (the first kernel of the pass
 * writes every counter it reads); calls that may overlap in time on one GPU
 * (other streams, other threads) race on it and must be ordered by the
 * caller.  The caller still owns and passes inputs and outputs. */
pa_status pa_forward_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, const int32_t* query_start_loc,
                             int32_t num_seqs, int32_t total_q_tokens, int32_t max_q_len,
                             int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                             pa_dtype dtype, int32_t* dev_status, void* stream);
/* Size of pa_forward_noalloc's static workspace, in bytes. */
size_t pa_forward_noalloc_max_workspace_bytes(void);

/* Measurement hook, for timing only (changes nothing that is computed).
 * pa_forward runs five stages on its stream: 0 planner, 1 VALU worker (decode
 * rows with one query head per KV head), 2 MFMA worker (GQA decode rows and
 * short prefill chunks), 3 tile worker (prefill chunks of more than 16 rows
 * per KV head), 4 log-sum-exp merge.  After this call, every pa_forward on the
 * calling thread records events[2k] before and events[2k+1] after stage k
 * (k < num_events/2) with hipEventRecord on its stream; a stage that has no
 * work records both events back to back.  events: host array of hipEvent_t
 * created by the caller, who keeps it alive; NULL entries are skipped.
 * num_events 0 (events may be NULL) turns recording off. */
pa_status pa_set_stage_events(void* const* events, int32_t num_events);

/* ------------------------------------------------------------------ copy-on-write
 * pa_copy_blocks — for each pair (src, dst) = block_pairs[2i], block_pairs[2i+1],
 * copy the whole key and value page of block src (all KV heads) onto block dst,
 * byte for byte: the private copy a sequence needs before it writes into a
 * block it shares ("大模型部署.md" §2.1 item 3 append_slots returning
 * (old, new); item 4 写时复制).  Destinations must be distinct and must not
 * be sources of other pairs.  Pairs with an id outside [0, num_blocks) are
 * skipped and flagged PA_DEV_BAD_BLOCK.
 *   block_pairs  device, int32 [num_pairs][2]
 */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs,
                         int32_t num_pairs, int32_t num_blocks, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, pa_dtype dtype,
                         int32_t* dev_status, void* stream);

/* ------------------------------------------------------------------ host allocator
 * Reference-counted physical block allocator with per-sequence block tables
 * ("大模型部署.md" §2.1 item 3, BlockSpaceManagerV1: _allocate_sequence,
 * can_allocate with watermark, append_slots with copy-on-write; "第7章" §2.3:
 * a free list popped from its end and appended to on release).  Pure host
 * code: no device memory, no HIP calls.  A handle is owned by the caller
 * (create/destroy) and is not thread-safe.  Every failing call leaves the
 * allocator unchanged.
 */
typedef struct pa_allocator pa_allocator;

/* initial_free_order: host int32 [num_blocks], a permutation of 0..num_blocks-1
 * giving the free stack bottom to top (blocks are taken from the end), or NULL
 * for 0..num_blocks-1.  watermark: fraction of the pool kept in reserve by
 * pa_alloc_can_allocate (int(watermark * num_blocks) blocks). */
pa_status pa_alloc_create(int32_t num_blocks, int32_t block_size, double watermark,
                          const int32_t* initial_free_order, pa_allocator** out);
void pa_alloc_destroy(pa_allocator* a);
/* Free blocks (with prefix caching: free stack + evictor). */
int32_t pa_alloc_num_free(const pa_allocator* a);
/* Reference count of a block, or -1 for an id outside the pool. */
int32_t pa_alloc_ref_count(const pa_allocator* a, int32_t block);
/* Admission check for a new sequence of num_tokens tokens:
 * NEVER if num_blocks - need < watermark blocks, OK if free - need >= watermark
 * blocks, else LATER (need = ceil(num_tokens / block_size)). */
pa_status pa_alloc_can_allocate(const pa_allocator* a, int32_t num_tokens, pa_alloc_status* out);

/* New sequence holding num_tokens tokens: ceil(num_tokens/block_size) blocks
 * taken in logical order, each with reference count 1.  All or nothing. */
pa_status pa_seq_create(pa_allocator* a, int64_t seq_id, int32_t num_tokens);
/* child shares every block of parent (reference counts + 1) and its length. */
pa_status pa_seq_fork(pa_allocator* a, int64_t parent_id, int64_t child_id);
/* Reserve the slot of the sequence's next token (length L -> L+1):
 *  - table one block short: take a free block;
 *  - else last block shared (count > 1): take a free block in its place, drop
 *    one reference from the old block and report (old, new) in
  *    *cow_src and *cow_dst (copy it with pa_copy_blocks before writing);
 *  - else nothing changes.
 * *slot_out = table[L/16]*16 + L%16.  *cow_src = *cow_dst = -1 without a copy. */
pa_status pa_seq_append_slot(pa_allocator* a, int64_t seq_id, int64_t* slot_out,
                             int32_t* cow_src, int32_t* cow_dst);
/* pa_seq_append_slot for n sequences in order; stops at the first failure
 * (the sequences before it keep their new slot).  slots_out: int64 [n];
 * cow_pairs_out: int32 [n][2] receives only the copies that happened, packed;
 * *num_cow_out their count. */
pa_status pa_seq_append_slots(pa_allocator* a, int32_t n, const int64_t* seq_ids,
                              int64_t* slots_out, int32_t* cow_pairs_out, int32_t* num_cow_out);
/* Slots of token positions start .. start+n-1 (must lie inside the sequence). */
pa_status pa_seq_slots(const pa_allocator* a, int64_t seq_id, int32_t start, int32_t n,
                       int64_t* slots_out);
/* Number of tokens of a sequence. */
pa_status pa_seq_num_tokens(const pa_allocator* a, int64_t seq_id, int32_t* out);
/* Copy a sequence's block table into out[0..cap); *n_out = its length
 * (PA_ERR_INVALID if cap is too small). */
pa_status pa_seq_block_table(const pa_allocator* a, int64_t seq_id, int32_t* out, int32_t cap,
                             int32_t* n_out);
/* Block tables of n sequences as rows of a [n][cap] matrix, padded with -1. */
pa_status pa_seq_block_tables(const pa_allocator* a, int32_t n, const int64_t* seq_ids,
                              int32_t* out, int32_t cap);
/* Drop the sequence: one reference less on each block in logical order;
 * blocks reaching zero return to the free stack in that order (with prefix
 * caching, a block carrying a hash goes to the evictor instead). */
pa_status pa_seq_free(pa_allocator* a, int64_t seq_id);

/* Streaming sequence (StreamingLLM, "第 15 章：推理引擎与部署" §15.4 Attention
 * Sink): the cache keeps the first num_sinks tokens and the most recent
 * `window` tokens, at most num_sinks + window, at cache positions
 * 0 .. num_sinks + window - 1.  Created with num_tokens <= num_sinks + window
 * tokens (positions 0 .. num_tokens - 1; the caller keeps a longer prompt's
 * sinks and last tokens).  pa_seq_append_slot / pa_seq_append_slots: while the
 * cache grows, as for any sequence; once it is full, the new token takes the
 * position of the oldest window token, num_sinks + (seen - num_sinks) mod
 * window, seen = tokens appended before it (a ring: attention does not depend
 * on the order of its keys), and the block holding that position is copied on
 * write first when it is shared.  pa_seq_num_tokens gives the cached tokens,
 * min(seen, num_sinks + window) — the context length to attend.  All or
 * nothing; PA_ERR_INVALID for a negative count, window <= 0 or too many
 * tokens. */
pa_status pa_seq_create_streaming(pa_allocator* a, int64_t seq_id, int32_t num_sinks, int32_t window,
                                  int32_t num_tokens);

/* ------------------------------------------------------------------ prefix caching
 * Reuse of the pages of equal prompt prefixes ("大模型部署.md" §2.1 item 3,
 * CachedBlockAllocator and LRUEvictor; "【自用】AI infra相关" part 二.4(2)).
 * Every full block of a sequence made from token ids gets a 64-bit hash of
 * the previous block's hash and its own 16 token ids (a hit also compares the
 * tokens and the parent hash, so a collision costs a miss, never a wrong
 * page).  A block whose hash is cached — in use, or released and waiting in
 * the evictor — is shared instead of allocated.  Released hashed blocks wait
 * in the evictor and still count as free: a new block comes from the free
 * stack, and only when that is empty from the evictor, which gives up the
 * block released longest ago (an allocator clock advances once per mutating
 * call), among blocks released by the same call the one whose hash covers the
 * most tokens.  Sequences made with pa_seq_create never carry hashes; those
 * made from token ids must append with pa_seq_append_tokens.
 *
 * Switch prefix caching on; the allocator must not be in use yet
 * (PA_ERR_INVALID otherwise). */
pa_status pa_alloc_enable_prefix_caching(pa_allocator* a);
/* Blocks waiting in the evictor (included in pa_alloc_num_free). */
int32_t pa_alloc_num_evictable(const pa_allocator* a);
/* New sequence from host token_ids[num_tokens]: every full block whose hash is
 * cached is shared (these are taken first, in logical order), the other
 * blocks are new (a new full block is registered under its hash).  All or
 * nothing.  *num_cached_tokens = 16 x the number of leading full blocks that
 * were shared: the prefix whose K/V the pool already holds once the sequence
 * that made those pages has written them; the caller writes tokens from there
 * on (a remainder past the last full block is always new). */
pa_status pa_seq_create_tokens(pa_allocator* a, int64_t seq_id, const int32_t* token_ids,
                               int32_t num_tokens, int32_t* num_cached_tokens);
/* pa_seq_append_slots for sequences made from token ids, with the new token of
 * each (token_ids: host int32 [n]).  When a token fills the last block and an
 * equal block is cached, the sequence switches to that block (one more
 * reference; the filled block is released, or, when it was shared, keeps its
 * other users and no copy is reported); otherwise the filled block (the copy,
 * when it was shared) is registered under its hash. */
pa_status pa_seq_append_tokens(pa_allocator* a, int32_t n, const int64_t* seq_ids, const int32_t* token_ids,
                               int64_t* slots_out, int32_t* cow_pairs_out, int32_t* num_cow_out);

/* ------------------------------------------------------------------ SplitFuse composer
 * Host-side composition of forward passes under a token budget
 * ("DeepSpeed-FastGen 深度解析" §3.1-§3.2, Dynamic SplitFuse: long prompts are
 * split over several passes, short ones fused to fill the budget exactly;
 * "第 15 章：推理引擎与部署", chunked prefill: Σ chunk tokens + number of decodes
 * <= budget).  A pass takes every running decode (one token each, in the
 * order the sequences started decoding; those past the budget wait), then
 * prompt chunks in arrival order, each min(tokens remaining, budget left),
 * until the budget is used.  A prompt decodes from the pass after the one
 * that took its last chunk.  Opaque handle, not thread-safe; every failing
 * call leaves it unchanged. */
typedef struct pa_splitfuse pa_splitfuse;
pa_status pa_sf_create(int32_t token_budget, pa_splitfuse** out);
void pa_sf_destroy(pa_splitfuse* c);
/* Queue a prompt of prompt_len (> 0) tokens; seq_id must be new. */
pa_status pa_sf_add_prompt(pa_splitfuse* c, int64_t seq_id, int32_t prompt_len);
/* Remove a sequence, queued or decoding (PA_ERR_NOT_FOUND if unknown). */
pa_status pa_sf_finish(pa_splitfuse* c, int64_t seq_id);
/* Compose the next pass into host arrays of capacity cap: row i is sequence
 * seq_ids[i] with q_lens[i] query tokens and context_lens[i] keys after the
 * pass (its earlier tokens included) — prompt chunks first, then decodes, the
 * order pa_forward's query_start_loc takes them.  *num_rows_out = rows (also
 * when cap is too small: PA_ERR_INVALID, nothing changes), *num_tokens_out =
 * Σ q_lens. */
pa_status pa_sf_step(pa_splitfuse* c, int32_t cap, int64_t* seq_ids, int32_t* q_lens, int32_t* context_lens,
                     int32_t* num_rows_out, int32_t* num_tokens_out);

/* ------------------------------------------------------------------ decode step
 * One decode step of num_seqs sequences with one new token each, driven from
 * the host allocator (parallel sampling: "大模型部署.md" §2.1 items 3-4,
 * append_slots returning the copy-on-write pairs, pages shared between the
 * samples of a prompt): pa_seq_append_slots for every sequence, then one
 * upload of the step's slots, context lengths, query starts, copy pairs and
 * block tables, pa_copy_blocks of the reported pairs, pa_reshape_and_cache of
 * the new keys and values, and pa_forward (pa_forward_shared when groups are
 * given) for one query row per sequence — all enqueued on `stream`, the
 * operations the caller would otherwise issue one by one.
 *
 * Staging layout (offsets in bytes, n = num_seqs, c = table columns):
 *   slots int64 [n] at 0; context lengths int32 [n] at 8n; query starts int32
 *   [n + 1] at 12n; copy pairs int32 [n][2] at P = 16n + 4 rounded up to a
 *   multiple of 8; block tables int32 [n][c] at P + 8n, padded with -1.
 * Bytes needed for tables of up to max_blocks_per_seq columns (0 for a
 * non-positive argument): */
size_t pa_decode_step_staging_bytes(int32_t num_seqs, int32_t max_blocks_per_seq);
/* Host half: appends one slot to each sequence (in order; with token_ids, a
 * host int32 [num_seqs] array of the new tokens, through pa_seq_append_tokens
 * for sequences made from token ids, else pa_seq_append_slots) and writes the
 * staging layout above into host_staging (host, 8-byte aligned, at least
 * pa_decode_step_staging_bytes(num_seqs, max_blocks_per_seq) bytes), with
 * c = ceil(longest context / 16) columns.  Out: *num_cow_out copy pairs,
 * *max_context_len_out, *table_cols_out = c, *used_bytes_out = bytes of the
 * layout for c columns.  Unknown sequences and a sequence whose table would
 * exceed max_blocks_per_seq fail before the allocator changes; an exhausted
 * pool fails as pa_seq_append_slots (the sequences before the failing one
 * keep their new slot). */
pa_status pa_decode_step_stage(pa_allocator* a, int32_t num_seqs, const int64_t* seq_ids,
                               const int32_t* token_ids, int32_t max_blocks_per_seq, void* host_staging, size_t staging_bytes,
                               int32_t* num_cow_out, int32_t* max_context_len_out, int32_t* table_cols_out,
                               size_t* used_bytes_out);
/* The whole step.  pa_decode_step_stage into host_staging, then hipMemcpyAsync
 * of the used bytes into dev_staging and the three launches on `stream`.
 *   seq_ids        host, int64 [num_seqs]; row i of q / new_key / new_value / out
 *                  is sequence seq_ids[i]
 *   token_ids      host, int32 [num_seqs] new tokens of sequences made from
 *                  token ids (prefix caching), or NULL
 *   q, out         device, [num_seqs][num_q_heads][head_dim] of dtype
 *   new_key, new_value  device, [num_seqs][num_kv_heads][head_dim] of dtype
 *   k_cache, v_cache    device, pool layout above, num_blocks blocks
 *   groups         device, int32 [num_groups][3] as in pa_forward_shared, or
 *                  NULL with num_groups 0 (plain pa_forward)
 *   host_staging   host, pinned (hipHostMalloc) for an asynchronous copy; it
 *                  must not be rewritten before the copy has run: give each
 *                  step in flight a region of its own, or synchronise
 *   dev_staging    device, 8-byte aligned, staging_bytes bytes (both buffers
 *                  are at least pa_decode_step_staging_bytes(num_seqs,
 *                  max_blocks_per_seq))
 *   workspace      device, 256-byte aligned, at least the workspace bytes of
 *                  pa_forward (pa_forward_shared with groups) for num_seqs
 *                  single-row sequences of up to 16 x max_blocks_per_seq keys
 * Argument errors are reported before the allocator changes; a HIP error of
 * the upload returns PA_ERR_HIP after the allocator has advanced. */
pa_status pa_decode_step(pa_allocator* a, int32_t num_seqs, const int64_t* seq_ids, const int32_t* token_ids,
                         void* out, const void* q,
                         const void* new_key, const void* new_value, void* k_cache, void* v_cache,
                         int32_t num_blocks, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         pa_dtype dtype, float scale, const int32_t* groups, int32_t num_groups,
                         int32_t max_blocks_per_seq, void* host_staging, void* dev_staging, size_t staging_bytes,
                         void* workspace, size_t workspace_bytes, int32_t* dev_status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
