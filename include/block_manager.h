/*
 * block_manager.h -- host-side KV block manager of libpa.so (C ABI).
 *
 * It produces what the device path consumes: per-sequence block tables,
 * context lengths, the slot of every new token (pa_write_kv), the block pairs
 * to copy before a write into a shared block (pa_copy_blocks) and the block
 * pairs of a swap between the device pool and a host pool (pa_swap_blocks).
 * Defined by:
 *   "How does vLLM PagedAttention manage Virtual Memory Pages to eliminate KV
 *   cache fragmentation?", section "Key Technical Innovations": a table per
 *   sequence maps its logical blocks to physical blocks anywhere in the pool
 *   (item 1); one block of block_size tokens is taken at a time as the
 *   sequence grows (item 2); parallel samples share the blocks of a common
 *   prompt, copy-on-write (item 3).  Section "Example": blocks come from the
 *   front of a free list that starts as 0, 1, ..., and a new block is taken
 *   when a token lands at position p with p % block_size == 0.
 *   "Paged Attention: OS-Inspired Memory Management for KV Caches", section
 *   "Key terms in this lesson": reference counts on shared blocks;
 *   copy-on-write gives a writer its own copy of a shared block; internal
 *   fragmentation (reported by pa_bm_stats).
 *   "PagedAttention and KV memory management", section "Key takeaways":
 *   preemption by swapping whole sequences out and back in.
 *
 * Rules where the pages leave the choice open:
 *   - Freed blocks go to the BACK of their pool's free list, in table order;
 *     allocation takes the FRONT.  Block ids are therefore deterministic.
 *   - Copy-on-write happens in pa_bm_append: a token whose position lands in
 *     a partly filled last block that other sequences also hold first moves
 *     the sequence to a fresh block; the caller must copy the old block into
 *     the new one (pa_copy_blocks) before writing the token.  The last holder
 *     of a block writes in place.
 *   - pa_bm_fork gives the child the parent's table and length; each block
 *     gains one reference.
 *   - Swap moves whole sequences between pools.  A block held by several of
 *     the listed sequences moves once (one pair) with all their references;
 *     a block also held by a sequence that is not listed is copied, and stays
 *     where it is with its remaining references.
 *   - Every call is all-or-nothing: on error nothing has changed.
 *
 * All pointers are HOST memory owned by the caller; the manager keeps none of
 * them.  A manager is not thread-safe: calls on one manager must not overlap.
 * Status codes are those of paged_attention.h plus PA_ERR_NO_ROOM (not enough
 * free blocks in the pool concerned, or a table would exceed
 * max_blocks_per_seq); pa_last_error() gives the message.
 */
#ifndef PA_BLOCK_MANAGER_H
#define PA_BLOCK_MANAGER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ERR_NO_ROOM 5

#define PA_POOL_DEVICE 0
#define PA_POOL_HOST 1

typedef struct pa_block_manager pa_block_manager;

/* Usage snapshot.  Tokens count distinct stored positions: a block shared by
 * several sequences counts once.  Internal waste = 1 - stored_tokens /
 * (blocks_used * block_size). */
typedef struct pa_bm_usage {
  int32_t num_seqs;              /* live sequences (both pools) */
  int32_t device_blocks_used;    /* blocks with a nonzero reference count */
  int32_t host_blocks_used;
  int32_t device_blocks_shared;  /* blocks with a reference count above 1 */
  int64_t device_tokens_logical; /* sum of context lengths of device sequences */
  int64_t device_tokens_stored;  /* distinct positions held in device blocks */
} pa_bm_usage;

/* New manager over a device pool of num_device_blocks and a host pool of
 * num_host_blocks (may be 0) blocks of block_size tokens.  device_free_order:
 * NULL for 0 .. num_device_blocks-1, else a permutation of those ids giving
 * the initial order of the device free list (e.g. a shuffled pool). */
int pa_bm_create(int32_t num_device_blocks, int32_t num_host_blocks, int32_t block_size,
                 int32_t max_blocks_per_seq, const int32_t* device_free_order,
                 pa_block_manager** out);
void pa_bm_destroy(pa_block_manager* bm);

/* New device sequence holding num_tokens (>= 0) prompt tokens, in
 * ceil(num_tokens / block_size) fresh blocks.  slots: NULL or [num_tokens],
 * receives the slot of each prompt position. */
int pa_bm_add(pa_block_manager* bm, int64_t seq, int32_t num_tokens, int32_t* slots);

/* One new token for each of n distinct device sequences, in order.
 *   slots    [n]  slot of each new token (block * block_size + offset)
 *   cow_src, cow_dst  [n]  the first *num_cow entries are the block pairs to
 *            copy (within the device pool) before the tokens are written.
 * Either may be NULL only if n == 0. */
int pa_bm_append(pa_block_manager* bm, const int64_t* seqs, int32_t n, int32_t* slots,
                 int32_t* cow_src, int32_t* cow_dst, int32_t* num_cow);

/* child (new id) shares parent's blocks and length. */
int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child);

/* Drop a sequence; blocks whose count reaches 0 return to their free list. */
int pa_bm_free(pa_block_manager* bm, int64_t seq);

/* Move n distinct sequences device -> host (swap_out) or host -> device
 * (swap_in).  src_blocks / dst_blocks [capacity]: the first *num_pairs entries
 * are the blocks to copy, source pool id -> destination pool id (pass them to
 * pa_swap_blocks).  capacity must cover the distinct blocks of the listed
 * sequences (PA_ERR_INVALID_ARG otherwise). */
int pa_bm_swap_out(pa_block_manager* bm, const int64_t* seqs, int32_t n, int32_t* src_blocks,
                   int32_t* dst_blocks, int32_t capacity, int32_t* num_pairs);
int pa_bm_swap_in(pa_block_manager* bm, const int64_t* seqs, int32_t n, int32_t* src_blocks,
                  int32_t* dst_blocks, int32_t capacity, int32_t* num_pairs);

/* Block tables [n, stride] (entries past a sequence's blocks are -1) and
 * context lengths [n] of n device sequences, ready for pa_decode.
 * stride >= the longest of their tables. */
int pa_bm_block_tables(const pa_block_manager* bm, const int64_t* seqs, int32_t n,
                       int32_t* tables, int32_t stride, int32_t* context_lens);

/* Groups for pa_decode_shared_prefix over the batch seqs[0..n-1] (device
 * sequences, in the order the batch lists them): maximal runs of consecutive
 * sequences whose tables start with the same block, e.g. samples forked from
 * one prompt and listed together.  group_starts [n + 1] receives the run
 * boundaries (group g = batch entries group_starts[g] .. group_starts[g+1]-1),
 * prefix_blocks [n] the number of leading whole blocks every member of the run
 * holds in common (0 for a run of one), *num_groups the number of runs. */
int pa_bm_prefix_groups(const pa_block_manager* bm, const int64_t* seqs, int32_t n,
                        int32_t* group_starts, int32_t* prefix_blocks, int32_t* num_groups);

/* One sequence: its table (NULL, or room for max_blocks_per_seq entries),
 * length, number of blocks and pool (PA_POOL_DEVICE / PA_POOL_HOST). */
int pa_bm_sequence(const pa_block_manager* bm, int64_t seq, int32_t* table, int32_t* length,
                   int32_t* num_blocks, int32_t* pool);

/* Free blocks of a pool; reference counts [pool size]; the free list in
 * allocation order (front first) [pool size], its length in *n. */
int pa_bm_num_free(const pa_block_manager* bm, int32_t pool, int32_t* n);
int pa_bm_refcounts(const pa_block_manager* bm, int32_t pool, int32_t* counts);
int pa_bm_free_list(const pa_block_manager* bm, int32_t pool, int32_t* blocks, int32_t* n);

int pa_bm_stats(const pa_block_manager* bm, pa_bm_usage* out);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCK_MANAGER_H */
