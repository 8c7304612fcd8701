/*
 * paged_attention.h -- C ABI of the MI355X (gfx950) paged decode library (libpa.so).
 *
 * Two operations on a KV cache held as fixed-size physical blocks in one pool,
 * reached through per-sequence block tables:
 *
 *   pa_write_kv  -- the slot write: each new token's K and V go into its slot
 *                   of the sequence's current block.  Defined by "How does vLLM
 *                   PagedAttention manage Virtual Memory Pages to eliminate KV
 *                   cache fragmentation?", sections "Key Technical Innovations"
 *                   (item 2: blocks of e.g. 16 tokens are taken one at a time as
 *                   generation proceeds) and "Example" (a new token is placed in
 *                   the sequence's current physical block).
 *   pa_decode    -- single-query attention for every sequence straight over the
 *                   paged pool.  Defined by "PagedAttention and KV memory
 *                   management", section "The kernel side": read the sequence's
 *                   block table, load each physical block's K and V tiles in
 *                   turn, and compute scores and weighted values without first
 *                   gathering the KV into one buffer.
 *
 * Layout (all row-major; the same on every entry point):
 *   k_cache  [num_blocks, num_kv_heads, block_size, head_dim]       kv dtype
 *   v_cache  [num_blocks, num_kv_heads, (block_size/T)*head_dim, T]  kv dtype
 *   T = 16 when 16 divides block_size, otherwise T = block_size: V is kept
 *   feature-major in sub-tiles of T tokens, so token o's feature d is
 *   v_cache[b, h, (o/T)*head_dim + d, o%T].  For block_size <= 16 this is
 *   plainly [num_blocks, num_kv_heads, head_dim, block_size].  Every 16-token
 *   piece of a (block, KV head) tile is then one contiguous span of K and one
 *   of V.
 *   A slot is physical_block * block_size + offset_in_block.
 *   Query head h reads KV head h / (num_heads / num_kv_heads).
 *   out = softmax(scale * q . K^T) . V over positions 0 .. context_len-1.
 *
 * Pointers: every array argument is DEVICE memory on the current HIP device,
 * owned by the caller.  The library allocates nothing, keeps no pointer after
 * a call returns, and never synchronises.  Each call enqueues its kernels on
 * `stream` (a hipStream_t; NULL means the null stream) and returns at once;
 * ordering between calls comes from the stream.
 *
 * Errors: argument errors are reported synchronously, before anything is
 * enqueued, as a nonzero pa_status; pa_last_error() then gives a message
 * (thread-local, valid until the next call on that thread).  A launch
 * failure is PA_ERR_LAUNCH.  No C++ exception crosses this interface.
 *
 * Device-side data (slots, block ids, context lengths) are not checked on the
 * host.  The kernels never access memory outside the arrays described by the
 * size arguments: a slot outside [0, num_blocks*block_size) is not written, a
 * block id outside [0, num_blocks) is not read (that block then contributes
 * nothing), and a context length is clamped to [0, max_blocks_per_seq *
 * block_size].  Such inputs still give an unspecified result for the affected
 * sequence.  Two tokens with the same slot in one pa_write_kv call race.
 */
#ifndef PAGED_ATTENTION_H
#define PAGED_ATTENTION_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k_cache, v_cache, k_new, v_new.  out is always fp32. */
typedef enum pa_dtype {
  PA_DTYPE_F32 = 0,   /* IEEE binary32 */
  PA_DTYPE_BF16 = 1   /* bfloat16: the top 16 bits of a binary32 */
} pa_dtype;

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, Hq % Hkv != 0, ... */
  PA_ERR_UNSUPPORTED = 2,   /* (dtype, head_dim, block_size, group size) not compiled */
  PA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required */
  PA_ERR_LAUNCH = 4         /* the HIP runtime refused a kernel launch */
} pa_status;

/*
 * Slot write.  For t in [0, num_tokens): if slot_mapping[t] >= 0, with
 * b = slot / block_size and o = slot % block_size,
 *   k_cache[b, h, o, :] = k_new[t, h, :]   and
 *   v_cache[b, h, (o/T)*head_dim + d, o%T] = v_new[t, h, d]  for every d
 * for every KV head h.  The copy moves raw element bits (NaN payloads
 * included).  A negative slot is skipped.  Slots must be distinct.
 *
 *   k_new, v_new   [num_tokens, num_kv_heads, head_dim]  kv dtype, device
 *   slot_mapping   [num_tokens] int32, device
 *   num_tokens == 0 is a successful no-op (pointers may then be NULL).
 * Supported: kv_dtype F32 or BF16, any head_dim in [1, 1024], any block_size >= 1.
 */
int pa_write_kv(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t kv_dtype,
                void* stream);

/*
 * One decode step: pa_write_kv followed by pa_decode, in one call, with the
 * same results (bit for bit) as the two calls made in that order on
 * `stream`.  The slot write and the decode planner do not depend on each
 * other, so they run in one launch; the step takes one launch less.
 * Arguments as in pa_write_kv (k_new, v_new, slot_mapping, num_tokens) and
 * pa_decode (the rest); the workspace is pa_decode's.  Argument errors are
 * reported before anything is launched.  Either part may be empty
 * (num_tokens == 0 or num_seqs == 0).
 */
int pa_decode_step(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                   const int32_t* slot_mapping, int32_t num_tokens, float* out, const void* q,
                   const int32_t* block_tables, const int32_t* context_lens, float scale,
                   int32_t block_size, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                   int32_t head_dim, int32_t max_blocks_per_seq, int32_t num_blocks,
                   int32_t kv_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Copy-on-write block copies inside one pool.  For i in [0, num_pairs):
 *   block dst_blocks[i] := block src_blocks[i]
 * in both k_cache and v_cache (all KV heads, all block_size positions; raw
 * bits).  This is the copy a writer needs before it appends into a block that
 * other sequences share ("Paged Attention: OS-Inspired Memory Management for
 * KV Caches", section "Key terms in this lesson": copy-on-write gives the
 * writer a private copy; "How does vLLM PagedAttention manage Virtual Memory
 * Pages ...", section "Key Technical Innovations", item 3).  The pairs come
 * from the block manager's pa_bm_append.
 *   src_blocks, dst_blocks  [num_pairs] int32, device (or device-visible
 *                           pinned host memory)
 * A pair with an id outside [0, num_blocks) is skipped.  Destinations must be
 * distinct and must not be sources in the same call (else the copies race).
 * num_pairs == 0 is a successful no-op.
 */
int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_blocks,
                   const int32_t* dst_blocks, int32_t num_pairs, int32_t num_blocks,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t kv_dtype,
                   void* stream);

/*
 * Block swap between two pools of the same block shape, e.g. the device pool
 * and a host pool in pinned memory (hipHostMalloc, which the device
 * addresses directly), for preemption by swapping ("PagedAttention and KV
 * memory management", section "Key takeaways").  For i in [0, num_pairs):
 *   dst pool block dst_blocks[i] := src pool block src_blocks[i]
 * in both tensors (raw bits).  The pairs come from pa_bm_swap_out (device ->
 * host) or pa_bm_swap_in (host -> device).  Pools and id arrays must be
 * addressable by the device; a pinned host pool is read or written across the
 * host link by the kernel itself (one launch for all pairs).  A pair with an
 * id outside its pool is skipped; destinations must be distinct and, when
 * both sides are the same pool, not sources of the same call.  Completion is
 * ordered by `stream`: the host must synchronise before it reads a host pool.
 */
int pa_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                   const int32_t* src_blocks, const int32_t* dst_blocks, int32_t num_pairs,
                   int32_t src_num_blocks, int32_t dst_num_blocks, int32_t num_kv_heads,
                   int32_t head_dim, int32_t block_size, int32_t kv_dtype, void* stream);

/*
 * Bytes of device workspace pa_decode needs for these shapes (an invalid
 * shape returns 0).  The workspace holds the call's work list, its counters
 * and the softmax states (max, sum, weighted sum) of context partitions that
 * are merged across workgroups.  Every call initialises what it uses: the
 * contents need no initialisation and are meaningless between calls.  Calls
 * that may run at the same time (different streams) need separate
 * workspaces; calls ordered on one stream may share one.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_blocks_per_seq,
                                 int32_t block_size, int32_t kv_dtype);

/*
 * Decode attention.  For every sequence s and query head h, with
 * L = context_lens[s] (counting the token written by this step's pa_write_kv)
 * and kv = h / (num_heads / num_kv_heads):
 *   out[s, h, :] = sum_t softmax_t(scale * q[s,h,:] . K_s[t,kv,:]) * V_s[t,kv,:],  t < L
 * where position t of sequence s lives in block block_tables[s, t / block_size]
 * at offset t % block_size.  L == 0 gives out[s, :, :] = 0.
 *
 *   out            [num_seqs, num_heads, head_dim] fp32, device (written)
 *   q              [num_seqs, num_heads, head_dim] kv dtype, device
 *   block_tables   [num_seqs, max_blocks_per_seq] int32, device; entries past
 *                  ceil(L / block_size) are never read (padding, e.g. -1)
 *   context_lens   [num_seqs] int32, device
 *   workspace      device, 256-byte aligned, at least
 *                  pa_decode_workspace_bytes(...) bytes (else PA_ERR_WORKSPACE)
 *   num_seqs == 0 is a successful no-op.
 * Compiled: head_dim in {64, 128}, block_size in {16, 32}, group size
 * num_heads / num_kv_heads in [1, 16], kv_dtype F32 or BF16.
 * The reduction order depends only on logical positions, so results are
 * bitwise reproducible and independent of where the blocks sit in the pool.
 * The call's kernels: a planner (skipped for bf16 batches of at most 64
 * sequences, which the attention kernel plans itself), the attention kernel,
 * and a merge of split sequences (when a sequence can span two partitions).
 * The environment variable PA_NUM_CUS_OVERRIDE, if set, replaces the device's
 * CU count in how the kernel shares out its work, and PA_DECODE_GRID_OVERRIDE,
 * if set to a positive number below the default, the number of workgroups of
 * the attention launch (test hooks; they change which workgroup computes
 * what, never the result).
 * After the call, pa_decode_check reports whether its kernels completed.
 */
int pa_decode(float* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, float scale,
              int32_t block_size, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
              int32_t head_dim, int32_t max_blocks_per_seq, int32_t num_blocks, int32_t kv_dtype,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode with the context split made explicit, for tests and tuning.
 * partition_tokens: tokens handled by one workgroup (a multiple of
 * block_size, or 0 for the library's choice).  flags: PA_FLAG_VECTOR_ALU
 * selects the plain vector-ALU kernel (by default both bf16 and fp32 KV use
 * the matrix-core kernel: bf16 products with fp32 sums, or fp32 products).
 * PA_FLAG_PACKED_POOL is a diagnostic for a pool that
 * holds each sequence's blocks consecutively: block j of sequence s is taken
 * to be block_tables[s, 0] + j, and only the first entry of each row is read
 * (bf16 matrix-core kernel only; else PA_ERR_UNSUPPORTED).  On such a pool it
 * gives the same bits as the ordinary path; timing the two on one packed pool
 * isolates the cost of reading the table per block ("PagedAttention and KV
 * memory management", section "Myths and failure modes": the indirection
 * costs a few percent).  The workspace must hold
 * pa_decode_workspace_bytes_ex(..., partition_tokens) bytes.
 */
#define PA_FLAG_VECTOR_ALU 1
#define PA_FLAG_PACKED_POOL 2
int pa_decode_ex(float* out, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, const int32_t* context_lens, float scale,
                 int32_t block_size, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                 int32_t head_dim, int32_t max_blocks_per_seq, int32_t num_blocks,
                 int32_t kv_dtype, void* workspace, size_t workspace_bytes,
                 int32_t partition_tokens, int32_t flags, void* stream);

size_t pa_decode_workspace_bytes_ex(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t max_blocks_per_seq,
                                    int32_t block_size, int32_t kv_dtype,
                                    int32_t partition_tokens);

/*
 * Decode attention with shared prompt prefixes.  Same result as pa_decode
 * (up to the rounding of a different reduction order), for a batch in which
 * groups of consecutive sequences -- e.g. parallel samples or beams forked
 * from one prompt -- hold the same leading physical blocks ("How does vLLM
 * PagedAttention manage Virtual Memory Pages ...", section "Key Technical
 * Innovations", item 3: copy-on-write sharing of prompt blocks; "PagedAttention
 * and KV memory management", section "Myths and failure modes": without
 * sharing, n samples multiply the prompt's KV by n).  Each shared K/V tile is
 * read once for all the group's sequences and query heads (up to 32 query
 * rows per read, with matrix-core products), instead of once per sequence.
 *
 *   group_starts   [num_groups + 1] int32, device: group g is sequences
 *                  group_starts[g] .. group_starts[g+1]-1 (non-decreasing;
 *                  sequences outside every group are decoded as usual; a
 *                  list that is not non-decreasing is ignored: the batch is
 *                  then decoded without shared prefixes, which gives the
 *                  same result; values are clamped to [0, num_seqs])
 *   prefix_blocks  [num_groups] int32, device: leading table entries that
 *                  every sequence of group g has in common.  Only whole
 *                  blocks inside every member's context are treated as
 *                  shared: the kernel uses min(prefix_blocks[g],
 *                  min over members of context_len / block_size).  They are
 *                  read through the group's first table; tables that differ
 *                  there give an unspecified result (never an out-of-bounds
 *                  access).
 *   num_groups == 0 gives plain pa_decode results.
 * Supported: kv_dtype BF16, the shapes of pa_decode, num_seqs <= 8192.  Other
 * dtypes return PA_ERR_UNSUPPORTED.  The workspace must hold
 * pa_decode_shared_prefix_workspace_bytes(...) bytes (partition_tokens as in
 * pa_decode_ex; 0 = the library's choice).
 */
int pa_decode_shared_prefix(float* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            const int32_t* group_starts, const int32_t* prefix_blocks,
                            int32_t num_groups, float scale, int32_t block_size, int32_t num_seqs,
                            int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t max_blocks_per_seq, int32_t num_blocks, int32_t kv_dtype,
                            void* workspace, size_t workspace_bytes, int32_t partition_tokens,
                            void* stream);

size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                               int32_t num_kv_heads, int32_t head_dim,
                                               int32_t max_blocks_per_seq, int32_t block_size,
                                               int32_t kv_dtype, int32_t partition_tokens);

/*
 * Completion check of the last decode call that used `workspace` (pa_decode,
 * pa_decode_ex, pa_decode_step or pa_decode_shared_prefix).  The attention
 * kernel's waves hand work to one another through the workgroup's shared
 * memory; each such wait is bounded, and a wait that does not end (a broken
 * invariant, never expected) is given up so that the kernel still ends:
 * that call's output is then incomplete.  The call records it in the int32
 * word at byte offset 80 of the workspace (set for every call: cleared by the
 * planner launch at its start, or, for a batch of at most 64 sequences that
 * the attention kernel plans itself, written by the call's last kernel from
 * a word of that kernel's own).  This call enqueues on `stream` a copy of
 * that word into *flag: 0 = every wait ended, 1 = the output of that call is
 * incomplete.
 *   workspace   the workspace the decode call used (device, 256-byte aligned,
 *               workspace_bytes >= 4224, as any decode workspace is); NULL
 *               with workspace_bytes == 0 means pa_decode_noalloc's array
 *               on the current device
 *   flag        one int32, device memory or pinned host memory (4-byte
 *               aligned); valid once `stream` has reached this point
 * Errors (reported before anything is enqueued): a null pointer or a
 * misaligned flag is PA_ERR_INVALID_ARG; a misaligned or too small workspace
 * is PA_ERR_WORKSPACE.  The call allocates nothing and does not synchronise.
 */
int pa_decode_check(const void* workspace, size_t workspace_bytes, int32_t* flag, void* stream);

/*
 * pa_decode for callers that cannot allocate or pass device memory for a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments as pa_decode without the
 * workspace, and the same result up to rounding: bit for bit whenever
 * pa_decode's own workspace for these shapes would fit in the array;
 * otherwise the context split may use longer partitions.  The workspace is
 * the library's own fixed device array of 64 MiB, one per device: the HIP
 * runtime reserves it when it loads the library's device code on that
 * device, and it is held until the process ends; the call itself allocates
 * nothing.
 * Shapes whose workspace does not fit in 64 MiB even with 8192-token
 * partitions (roughly num_seqs * num_heads * ceil(max_blocks_per_seq *
 * block_size / 8192) * (head_dim + 2) * 4 bytes) are rejected with
 * PA_ERR_WORKSPACE before anything is enqueued; other argument errors are
 * pa_decode's.  Every call on a device uses that device's one array: calls
 * that may overlap on one device (different streams, or threads) race and
 * must not be made.  pa_decode_check(NULL, 0, flag, stream) reports the
 * completion of the last such call on the current device.
 */
int pa_decode_noalloc(float* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, float scale,
                      int32_t block_size, int32_t num_seqs, int32_t num_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                      int32_t num_blocks, int32_t kv_dtype, void* stream);

/* Tokens per partition that pa_decode picks for these shapes (0 if invalid). */
int32_t pa_decode_partition_tokens(int32_t num_seqs, int32_t num_kv_heads,
                                   int32_t max_blocks_per_seq, int32_t block_size);

/*
 * Kernel timing, for benchmarks and diagnostics.  Between
 * pa_kernel_timing_begin and pa_kernel_timing_end, each of the first
 * `capacity` pa_decode / pa_decode_ex calls made on the device that was
 * current at begin records a pair of HIP events on its stream, right before
 * and right after its attention kernel (the planner and the partition merge
 * are outside the pair).  pa_kernel_timing_end waits for those events (it
 * synchronises), writes the summed elapsed milliseconds and the number of
 * timed calls, and releases the events.  Begin creates the events (host API
 * objects, no caller buffer); timing is process-wide and not nested: begin
 * while on, or end while off, is PA_ERR_INVALID_ARG.
 */
int pa_kernel_timing_begin(int32_t capacity);
int pa_kernel_timing_end(double* total_ms, int32_t* launches);

/*
 * Bandwidth probes, for the benchmark's empirical ceilings (not part of the
 * decode path).  pa_probe_read reads `bytes` (a multiple of 16) at `src`
 * once, contiguously.  pa_probe_read_tiles reads, for each listed tile index
 * t in [0, pool_tiles), the tile_bytes at k_cache + t * tile_bytes and at
 * v_cache + t * tile_bytes (tile_bytes 4096 or 8192: one (block, KV head)
 * tile of 16 or 32 tokens x 128 bf16 features); other indices are skipped.
 * Both use the decode kernel's nontemporal 16-byte loads and do no
 * arithmetic beyond folding the data into a register; `sink` (one device
 * word) is written only if that fold equals a fixed 32-bit value.
 */
int pa_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream);
int pa_probe_read_tiles(const void* k_cache, const void* v_cache, const int32_t* tiles,
                        int32_t num_tiles, int32_t tile_bytes, int64_t pool_tiles, uint32_t* sink,
                        void* stream);

/* Static description of a status code.  pa_status_str is the same function
 * under a shorter name.  Status and dtype arguments are int32_t rather than
 * the enum types above, so that their size in the ABI is fixed; their values
 * are the enumerators. */
const char* pa_status_string(int32_t status);
const char* pa_status_str(int32_t status);

/* Message for the last failing call on this thread ("" if none). */
const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTENTION_H */
