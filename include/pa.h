/*
 * pa.h -- C ABI of the MI355X (gfx950) paged-attention library, libpa.so.
 *
 * Paged attention is softmax attention computed directly over a K/V cache
 * that is scattered into fixed-size physical blocks and reached through a
 * per-sequence block table (JuliaPagedAttn README, "Architecture" and
 * "Block Layout"; Pico-vLLM #5 Paged Attention, "核心数据结构和设计模式";
 * nanoserve Day 19, "What I added today").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument named as device memory must point to memory the
 *   caller allocated on the current HIP device; the library never allocates,
 *   frees or keeps a pointer after a call returns.  Host pointers (the
 *   descriptor structs themselves) are only read during the call.
 * - Work is enqueued on `stream` (NULL = the default stream) and runs
 *   asynchronously; a PA_OK return means the launch was accepted.
 *   PA_ERR_HIP carries the HIP status of the library's own launch only: an
 *   earlier failed HIP call of the caller's, left uncleared, neither fails a
 *   call here nor is cleared by one.  Faults during execution surface at the
 *   caller's next synchronisation, as for any HIP kernel.
 * - Arguments are checked on the host before anything is enqueued.  A
 *   failed check returns PA_ERR_INVALID_ARG or PA_ERR_UNSUPPORTED and
 *   enqueues nothing; pa_last_error() then describes the failed check.
 *   The contents of device arrays (tables, lengths, slots) are not read on
 *   the host; the kernels treat out-of-range entries as described per call
 *   and never access memory outside the buffers described here.
 * - Indices are 0-based.  Element types: PA_F32 is IEEE binary32, PA_BF16 is
 *   bfloat16 (the high 16 bits of a binary32).  q, out, k_new and v_new use
 *   the pool's element type.
 * - The library keeps no state between calls apart from thread-local error
 *   text and the block allocators the caller creates, so calls from several
 *   host threads are safe; one allocator must not be used by two threads at
 *   once.  Calls that write the same device memory must be ordered by the
 *   caller (one stream).
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same declaration as the HIP runtime's, so either header may come first. */
typedef struct ihipStream_t* hipStream_t;

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1,  /* null pointer, bad size, misaligned pointer ... */
  PA_ERR_UNSUPPORTED = -2,  /* valid request outside what the kernels cover  */
  PA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required    */
  PA_ERR_HIP = -4,          /* the HIP runtime refused a launch              */
  PA_ERR_NO_BLOCKS = -5     /* the block allocator has too few free blocks   */
} pa_status;

typedef enum pa_dtype {
  PA_F32 = 0,
  PA_BF16 = 1
} pa_dtype;

typedef enum pa_layout {
  /* a block is [block_size, num_kv_heads, head_dim]: the Pico-vLLM pool tensor
   * [2, num_layers, num_blocks, block_size, num_kv_heads, head_dim]
   * ("核心数据结构和设计模式", BlockManager listing) */
  PA_LAYOUT_TOKEN_MAJOR = 0,
  /* a block is [num_kv_heads, block_size, head_dim]: JuliaPagedAttn's
   * per-block K / V [head_dim, block_size, num_kv_heads] ("Block Layout"),
   * which is column-major, read in row-major order; each KV head's 16 token
   * rows of a block are one contiguous span */
  PA_LAYOUT_HEAD_MAJOR = 1
} pa_layout;

/*
 * The block pool of one attention layer.
 *
 * k_cache and v_cache (device) each hold num_blocks blocks of `dtype`; block
 * b starts block_stride elements after block b - 1 and is laid out as
 * `layout` says, densely (head_dim elements per token row of a head).
 * block_stride == 0 means dense blocks (block_size * num_kv_heads *
 * head_dim), i.e. a row-major [num_blocks, block_size, num_kv_heads,
 * head_dim] (token-major) or [num_blocks, num_kv_heads, block_size,
 * head_dim] (head-major) array.  One block table addresses both pools.
 *
 * The pages' pool variants map onto this descriptor as follows:
 *   - one layer of a multi-layer pool [2, num_layers, num_blocks, ...]:
 *     k_cache = &pool[0][layer], v_cache = &pool[1][layer], dense blocks;
 *   - JuliaPagedAttn's 5-D K_cache / V_cache (column-major [head_dim,
 *     block_size, num_kv_heads, num_blocks, num_layers]): k_cache =
 *     &K_cache[layer], v_cache = &V_cache[layer], PA_LAYOUT_HEAD_MAJOR;
 *   - K and V of a block stored together ([num_blocks, 2, block ...],
 *     "unified K/V blocks" in JuliaPagedAttn "Features"): k_cache = &pool[0][0],
 *     v_cache = &pool[0][1], block_stride = 2 * block elements.
 *
 * Both pointers must be 16-byte aligned; block_stride, if not 0, must be at
 * least the dense block size and a multiple of 16 bytes.  Slots keep their
 * meaning in every layout: slot = block * block_size + offset in the block.
 *
 * Supported: block_size 8, 16, 32, 64, 128 or 256 (JuliaPagedAttn
 * "API Reference" and Pico-vLLM's BlockManager both take the block size as
 * a parameter), head_dim 64 or 128, dtype PA_F32 or PA_BF16.  The kernels
 * walk a history in units of 16 tokens whatever the block size.
 */
typedef struct pa_kv_pool {
  void* k_cache;
  void* v_cache;
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;        /* pa_dtype */
  int32_t layout;       /* pa_layout */
  int64_t block_stride; /* elements from one block to the next; 0 = dense */
} pa_kv_pool;

/*
 * The sequences of a batch.
 *
 * block_tables (device, int32 [num_seqs, max_blocks_per_seq], row-major):
 *   physical block ids, the fixed-width form of Pico-vLLM's int32
 *   get_block_table() ("核心数据结构和设计模式").  Entry j of row s holds
 *   positions j*block_size .. (j+1)*block_size-1 of sequence s.  Entries at
 *   or past ceil(context_lens[s] / block_size) are never read.  Several rows
 *   may name the same physical block (copy-on-write sharing of a prefix,
 *   JuliaPagedAttn "Copy-on-Write").
 * context_lens (device, int32 [num_seqs]): tokens of each sequence already in
 *   the pool, counting the one written in the current step (Pico-vLLM's +1
 *   rule; JuliaPagedAttn's `context_lengths`).
 * max_context_len (host): an upper bound of context_lens used to size the
 *   launch.  Kernels use min(context_lens[s], max_context_len,
 *   max_blocks_per_seq * block_size) as the context length, so a violated
 *   bound truncates instead of reading out of bounds.
 */
typedef struct pa_seq_desc {
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;
} pa_seq_desc;

/*
 * pa_slot_mapping -- pool slot of each new token.
 *
 * Token i belongs to sequence s and is one of its q_len newest positions:
 *   without q_start_loc (NULL): num_tokens == num_seqs, token i is the last
 *     position context_lens[i]-1 of sequence i (decode);
 *   with q_start_loc (device, int32 [num_seqs+1], non-decreasing, first 0):
 *     sequence s owns tokens q_start_loc[s] .. q_start_loc[s+1]-1, q_len =
 *     q_start_loc[s+1]-q_start_loc[s], and token q_start_loc[s]+i sits at
 *     position context_lens[s] - q_len + i (prefill, or a chunk of one).
 * slot_mapping (device, int64 [num_tokens], written):
 *   block_tables[s][pos / block_size] * block_size + pos % block_size: the
 *   block and the offset of the token inside it (for a dense token-major
 *   pool, the flat row of the token in the pool viewed as [num_blocks *
 *   block_size, num_kv_heads, head_dim]; JuliaPagedAttn "Project Structure":
 *   slot mapping in the cache layout; nanoserve Day 19 "Diagram":
 *   slot_mapping).  -1 where
 *   the position is negative, at or past the context, past the table width,
 *   or the table entry is not a block of the pool.
 */
pa_status pa_slot_mapping(const pa_kv_pool* pool, const pa_seq_desc* seqs,
                          const int32_t* q_start_loc, int32_t num_tokens,
                          int64_t* slot_mapping, hipStream_t stream);

/*
 * pa_write_kv -- scatter this step's K/V rows into the pool.
 *
 * k_new, v_new (device, [num_tokens, num_kv_heads, head_dim] of the pool's
 * dtype, 16-byte aligned) are copied bit for bit into row slot_mapping[t] of
 * k_cache and v_cache (JuliaPagedAttn "API Reference": write_kv_cache!;
 * nanoserve Day 19 "What I added today": the write of this step's K/V to its
 * slots).  Slots below 0 or at or past num_blocks * block_size are skipped.
 * Two tokens with the same slot race (the caller's responsibility).
 */
pa_status pa_write_kv(const pa_kv_pool* pool, const void* k_new, const void* v_new,
                      const int64_t* slot_mapping, int32_t num_tokens,
                      hipStream_t stream);

/*
 * Copy-on-write paging (JuliaPagedAttn README, "Copy-on-Write": sequences
 * that share a prefix name the same physical blocks, whose reference count
 * is then above one; a write into such a block first allocates a new block,
 * copies the data, points the writer's table at the copy and drops one
 * reference from the shared block).
 *
 * pa_block_allocator -- host-side free list and reference counts of one
 * pool's num_blocks physical blocks.  Free ids are handed out first-in
 * first-out: 0 .. num_blocks-1 in order at first, released ids appended at
 * the back (Pico-vLLM #5 Paged Attention, "核心数据结构和设计模式",
 * BlockManager: deque of free ids, popleft / append).  Every call checks
 * its whole request first; a failed call changes nothing.  Host memory
 * only; an allocator is not thread-safe.
 */
typedef struct pa_block_allocator pa_block_allocator;

/* A new allocator with every block free; *out receives it. */
pa_status pa_allocator_create(int32_t num_blocks, pa_block_allocator** out);
void pa_allocator_destroy(pa_block_allocator* alloc);
/* Free blocks now (-1 for a null allocator). */
int32_t pa_allocator_num_free(const pa_block_allocator* alloc);
/* References held on `block` (0 = free; -1 = not a block of the pool). */
int32_t pa_allocator_refcount(const pa_block_allocator* alloc, int32_t block);

/* Take n free blocks into blocks[0..n) (host), each with one reference.
 * PA_ERR_NO_BLOCKS if fewer than n are free (the p2 allocate error). */
pa_status pa_allocator_allocate(pa_block_allocator* alloc, int32_t n, int32_t* blocks);

/* One more reference on each listed block: another table now names it
 * (JuliaPagedAttn's cow_fork!).  Every block must be allocated. */
pa_status pa_allocator_fork(pa_block_allocator* alloc, const int32_t* blocks, int32_t n);

/* Drop one reference per listing; a block whose count reaches 0 goes to
 * the back of the free list, in listing order.  A block listed k times must
 * hold at least k references. */
pa_status pa_allocator_release(pa_block_allocator* alloc, const int32_t* blocks, int32_t n);

/*
 * pa_allocator_prepare_write -- make positions [start, start+count) of one
 * sequence writable before its K/V are written there.
 *
 * table (host, int32 [width]) is the sequence's block-table row, of which
 * entries [0, *num_used) are in use.  Every touched entry that names a
 * shared block (reference count > 1) is replaced by a freshly allocated
 * block: the pair (old, new) is appended to copy_src / copy_dst (host,
 * capacity copy_cap; *num_copies receives the count) and one reference is
 * dropped from the old block.  Touched entries at or past *num_used are
 * filled with freshly allocated blocks and *num_used grows.  The caller then
 * uploads the row, runs pa_copy_blocks on the pairs and writes the K/V.
 * start must not leave a gap (start <= *num_used * block_size).
 * PA_ERR_NO_BLOCKS if the allocator cannot supply every block needed.
 */
pa_status pa_allocator_prepare_write(pa_block_allocator* alloc, int32_t* table, int32_t width,
                                     int32_t* num_used, int32_t block_size, int32_t start,
                                     int32_t count, int32_t* copy_src, int32_t* copy_dst,
                                     int32_t copy_cap, int32_t* num_copies);

/*
 * pa_append_kv -- the decode step's write in one launch: pa_slot_mapping
 * without q_start_loc (each sequence's newest position, context_lens[s] - 1)
 * fused with pa_write_kv (nanoserve Day 19, "What I added today": this
 * step's K/V written to its slot before attention reads the history).
 *
 * k_new, v_new (device, [num_seqs, num_kv_heads, head_dim] of the pool's
 * dtype, 16-byte aligned): row s goes to sequence s's slot, bit for bit.
 * slot_mapping (device, int64 [num_seqs], written; may be NULL): the slot
 * used for each sequence, -1 where it was skipped (empty context, position
 * past the table width, or a table entry that is not a block of the pool).
 * The result equals pa_slot_mapping followed by pa_write_kv.
 */
pa_status pa_append_kv(const pa_kv_pool* pool, const pa_seq_desc* seqs, const void* k_new,
                       const void* v_new, int64_t* slot_mapping, hipStream_t stream);

/*
 * pa_copy_blocks -- copy whole blocks of both pools on the device: for each
 * pair i, block src_blocks[i] of k_cache and of v_cache is copied bit for
 * bit to block dst_blocks[i] (the data move of a copy-on-write).
 * src_blocks / dst_blocks: device int32 [num_pairs]; pairs naming a block
 * outside the pool are skipped.  A destination that is also a source, or
 * listed twice, races (the caller's responsibility).  num_pairs <= 65535.
 */
pa_status pa_copy_blocks(const pa_kv_pool* pool, const int32_t* src_blocks,
                         const int32_t* dst_blocks, int32_t num_pairs, hipStream_t stream);

/*
 * pa_swap_blocks -- move whole blocks between the device pool and a pool in
 * pinned host memory (Pico-vLLM #5 Paged Attention, BlockManager swap_out:
 * a GPU block is copied into a free CPU block of the pinned CPU pool;
 * swap_in: back into a free GPU block).  Pair i copies, in both K and V,
 * device block device_blocks[i] to host block host_blocks[i]
 * (direction PA_SWAP_OUT) or host block host_blocks[i] to device block
 * device_blocks[i] (PA_SWAP_IN), bit for bit.  The caller does the
 * bookkeeping (which blocks are free; pa_block_allocator serves either pool).
 *
 * host_pool: k_cache / v_cache in pinned host memory (hipHostMalloc, or a
 * pinned torch tensor), same block_size, num_kv_heads, head_dim and dtype as
 * device_pool; the device reads or writes it directly, so one launch moves
 * the whole batch.  device_blocks / host_blocks: int32 [num_pairs] readable by
 * the device (device memory or pinned host memory).  Pairs naming a block
 * outside its pool are skipped.  The copy is asynchronous on `stream`: the
 * host pool may be read, or reused, after the stream has passed it.
 * The library owns nothing; both pools and both id arrays stay the caller's.
 *
 * Errors (nothing enqueued): PA_ERR_INVALID_ARG for a bad descriptor, pools
 * whose block shape or dtype differ, an unknown direction, a device pool that
 * is not device memory, a host pool that is not pinned host memory mapped to
 * the device at the same address (pageable memory is refused, since the
 * kernel would fault on it), or id arrays the device cannot read;
 * PA_ERR_UNSUPPORTED for num_pairs > 65535; PA_ERR_HIP if the launch fails.
 */
typedef enum pa_swap_direction {
  PA_SWAP_OUT = 0,  /* device pool -> host pool */
  PA_SWAP_IN = 1    /* host pool -> device pool */
} pa_swap_direction;

pa_status pa_swap_blocks(const pa_kv_pool* device_pool, const pa_kv_pool* host_pool,
                         const int32_t* device_blocks, const int32_t* host_blocks,
                         int32_t num_pairs, int32_t direction, hipStream_t stream);

/*
 * pa_decode_workspace_bytes -- device workspace pa_decode needs for this
 * pool, batch shape, num_q_heads and partition_size (only the pool's sizes
 * are read, not its pointers).
 *
 * 0 when the context is not split (partition_size 0 or >= the longest
 * context): the kernel then writes `out` directly.  Otherwise 256 KiB of
 * arrival counters, then 2 * V * n_rep * head_dim floats of partial outputs
 * (padded to 256 bytes), then 2 * V * n_rep * 2 floats of (max, sum), with
 * V = min(2048, ceil(num_kv_heads * num_seqs * ceil(max_context_len / 16) /
 * (partition_size / 16))) the most slices a call can use (with
 * max_context_len capped at max_blocks_per_seq * block_size).  Host only, needs
 * no device; returns 0 for invalid arguments too (pa_decode then reports
 * them).
 */
size_t pa_decode_workspace_bytes(const pa_kv_pool* pool, const pa_seq_desc* seqs,
                                 int32_t num_q_heads, int32_t partition_size);

/*
 * pa_decode -- attention of one new query row per (sequence, query head)
 * over the sequence's whole paged history.
 *
 * out[s, h, :] = sum_t softmax_t(scale * q[s,h,:] . K_s[t, h / n_rep, :])
 *                * V_s[t, h / n_rep, :]
 * with t = 0 .. context_len-1 read through block_tables and n_rep =
 * num_q_heads / num_kv_heads (GQA: the compact KV heads are repeated to the
 * query heads at read time, nanoserve Day 19 "What I learned" item 4).
 * The softmax is computed online with a running maximum and running sum
 * (JuliaPagedAttn "Online Softmax"); a context of length 0 gives zeros.
 *
 * q (device, [num_seqs, num_q_heads, head_dim]) and out (device, same shape)
 * are in the pool's dtype, 16-byte aligned; out is rounded to nearest even
 * for bf16.  Accumulation is fp32.
 *
 * partition_size: 0 (or at least the longest context) = each (sequence, KV
 * head) pair in one pass.  Otherwise a multiple of 16 that turns on
 * the split-context decode: the blocks of all pairs, laid end to end, are cut
 * into slices of at least partition_size tokens, one per workgroup that the
 * GPU holds at once.  When the non-empty contexts differ in length the
 * slices cover nine tenths of the work and the rest is cut into chunks of a
 * sixteenth of a slice (at least partition_size tokens) that the workgroups
 * take one at a time as they finish, so faster workgroups take more; with
 * equal lengths the slices cover it all.  A pair cut by slice or chunk
 * boundaries is computed in pieces, each keeping its own maximum, sum and
 * normalised output, and the workgroup that finishes its last piece merges
 * them by log-sum-exp weighting, in token order, in the same kernel.
 *
 * workspace (device, 256-byte aligned, at least pa_decode_workspace_bytes(...)
 * bytes; may be NULL when that is 0): its first 256 KiB hold one arrival
 * counter per (sequence, KV head) and, in their last 256 bytes, the
 * counters that hand out the chunks; the rest holds the pieces' results.
 * The counters must be zero before the first call that uses the workspace
 * (zero the whole buffer once when allocating it); every call leaves them
 * zero again, so one workspace serves any later batch shape.  The rest's contents
 * on entry do not matter.  Calls that share a workspace must not overlap.
 *
 * Supported: num_q_heads / num_kv_heads in {1, 2, 4, 8}; num_seqs <= 4096;
 * num_kv_heads * num_seqs * ceil(max_context_len / 16) < 2^31; split,
 * num_seqs * num_kv_heads <= 65472.
 */
pa_status pa_decode(const pa_kv_pool* pool, const pa_seq_desc* seqs, const void* q,
                    void* out, int32_t num_q_heads, float scale, int32_t partition_size,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pa_decode_step -- one decode step in one launch: pa_append_kv (this
 * step's K/V written to each sequence's newest slot) followed by pa_decode
 * (attention over the whole history, the new token included), with the same
 * results bit for bit (nanoserve Day 19, "What I added today": the step's
 * K/V written to the cache, then attention over it in place; JuliaPagedAttn
 * "API Reference": write_kv_cache! then paged_attention_cpu!).
 *
 * k_new, v_new and slot_mapping are those of pa_append_kv; q, out,
 * num_q_heads, scale, partition_size and the workspace those of pa_decode.
 * Inside the launch each new row is written to its slot once, and the
 * attention takes the new token's K and V from k_new and v_new instead of
 * reading the slot back, so no pool location is both written and read in
 * the call.  As with pa_append_kv followed by pa_decode, the written slot
 * must not be part of another sequence's context in the same call (the
 * copy-on-write rule of the block allocator guarantees it).  Errors are
 * those of both calls; nothing is launched on an error.
 */
pa_status pa_decode_step(const pa_kv_pool* pool, const pa_seq_desc* seqs, const void* k_new,
                         const void* v_new, int64_t* slot_mapping, const void* q, void* out,
                         int32_t num_q_heads, float scale, int32_t partition_size,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pa_decode_noalloc -- pa_decode without a caller workspace, for callers
 * that cannot allocate device memory around the call: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.
 *
 * Arguments and results are those of pa_decode with workspace NULL: the
 * split decode's arrival counters and partial results live instead in a
 * device array of the library's own, pa_decode_noalloc_max_bytes() bytes
 * (16.5 MiB: the largest workspace pa_decode_workspace_bytes can ask for),
 * which every GPU the library runs on holds until the process ends.  The
 * call allocates and frees nothing.  Its first call on a device looks up
 * that device's copy of the array and clears the counters with a small
 * kernel on `stream`; every call leaves them zero again.
 *
 * All calls on one GPU share that GPU's array: calls that overlap in time on
 * one GPU (other streams, other host threads) race and must be ordered by
 * the caller.  A request whose split would need more than the array holds
 * returns PA_ERR_UNSUPPORTED and enqueues nothing; other errors are those
 * of pa_decode.
 */
pa_status pa_decode_noalloc(const pa_kv_pool* pool, const pa_seq_desc* seqs, const void* q,
                            void* out, int32_t num_q_heads, float scale, int32_t partition_size,
                            hipStream_t stream);

/* Bytes of the array pa_decode_noalloc uses per GPU (host only). */
size_t pa_decode_noalloc_max_bytes(void);

/*
 * pa_decode_split_info -- how pa_decode would split this batch (host only,
 * nothing launched; needs the device the decode would run on to be current).
 *
 * host_context_lens (host, int32 [num_seqs]) is a host copy of
 * seqs->context_lens; the other arguments are those of pa_decode (q, out and
 * the workspace are not needed).  Fills *info: the workgroups of the launch;
 * slice_blocks, each workgroup's static slice in blocks (each segment of a
 * (sequence, KV head) pair priced as a fixed number of extra blocks), 0 when
 * the context is not split; chunk_blocks and units, the chunks handed out
 * after the slices (0 when none) and the slices and chunks in all; and how
 * many pieces the non-empty pairs are cut into (1 each when not split).
 * partition_size is a lower bound of the slice and the chunk, not the
 * slice itself.
 */
typedef struct pa_decode_split {
  int32_t workgroups;
  int32_t slice_blocks;  /* each workgroup's static slice */
  int32_t pairs;         /* (sequence, KV head) pairs with a non-empty context */
  int32_t max_pieces;    /* most pieces of one pair */
  float mean_pieces;     /* mean pieces per pair */
  int32_t chunk_blocks;  /* the chunks handed out after the slices (0: none) */
  int32_t units;         /* slices + chunks */
} pa_decode_split;

pa_status pa_decode_split_info(const pa_kv_pool* pool, const pa_seq_desc* seqs,
                               const int32_t* host_context_lens, int32_t num_q_heads,
                               int32_t partition_size, pa_decode_split* info);

/*
 * pa_prefill -- causal attention of every new token of every sequence over
 * its paged history, in one call (JuliaPagedAttn "Features": batched
 * prefill, all prompt positions processed in a single kernel call).
 *
 * q (device, [total_q_tokens, num_q_heads, head_dim]) and out (same shape)
 * are in the pool's dtype, 16-byte aligned.  q_start_loc (device, int32
 * [num_seqs+1]) lists each sequence's tokens as in pa_slot_mapping (its
 * entries are clamped to [0, total_q_tokens], so no row outside q and out is
 * touched); token q_start_loc[s]+i of a sequence with q_len new tokens sits
 * at position p = context_lens[s] - q_len + i and attends to positions
 * 0 .. p of its sequence (the K/V of the new tokens must already be in the
 * pool: pa_write_kv first).  A token whose position is negative (q_len
 * above the context length) sees no key and its row of out is zero.
 * max_q_len (host) bounds every q_len and sizes the launch: of a sequence
 * with more new tokens, only the newest max_q_len are computed, each at its
 * own position, and the rows of the older ones are not written.  Keys whose
 * table entry is not a block of the pool get no weight (as in pa_decode).
 *
 * Supported: PA_BF16 and PA_F32 pools, head_dim 64 or 128, num_q_heads /
 * num_kv_heads in {1, 2, 4, 8}.  QK^T and PV run on the matrix cores with
 * fp32 accumulation: bf16 pools on bf16 matrix instructions (the
 * probabilities rounded to bf16 for the PV product), fp32 pools on fp32 ones
 * (nothing rounded below fp32).
 */
pa_status pa_prefill(const pa_kv_pool* pool, const pa_seq_desc* seqs, const void* q,
                     void* out, const int32_t* q_start_loc, int32_t total_q_tokens,
                     int32_t max_q_len, int32_t num_q_heads, float scale,
                     hipStream_t stream);

/*
 * pa_read_checksum -- a plain read stream over a device buffer, to measure
 * the read bandwidth a read-once kernel such as pa_decode can reach on this
 * device (the decode's roofline is quoted against the HBM peak; this is the
 * practical ceiling beside it).  Not part of the attention path.
 *
 *   buf        device, 16-byte aligned, `bytes` bytes (a multiple of 16).
 *   words      device, [num_words] uint32 output; 1 <= num_words <= 65535.
 *              Word i is the XOR of the little-endian 32-bit words of the
 *              byte range [i*S, min((i+1)*S, bytes)), S = 16 * ceil(bytes /
 *              16 / num_words); a word whose range is empty is 0.
 * Every byte is read once with non-temporal 16-byte loads, one workgroup per
 * output word.  PA_ERR_INVALID_ARG for a null pointer, bytes not a multiple
 * of 16 or num_words out of range; PA_ERR_UNSUPPORTED if S exceeds 2 GiB.
 * bytes == 0 writes zeros to every word.
 */
pa_status pa_read_checksum(const void* buf, size_t bytes, uint32_t* words, int32_t num_words,
                           hipStream_t stream);

/* Static text naming a status code. */
const char* pa_status_string(int32_t status);

/* Thread-local text describing the last failed check or HIP error of this
 * thread ("" if none).  Valid until the next call on the same thread. */
const char* pa_last_error(void);

/* Library ABI version: (major << 16) | minor. */
int32_t pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
