// Internal interface between the C ABI (pa_api.cpp) and the kernel launchers.
// Not installed; callers use include/paged_attention.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <hip/hip_vector_types.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Everything one decode launch needs.  Pointers are device pointers.
struct DecodeParams {
  float* out;                 // [S, Hq, D] fp32
  const void* q;              // [S, Hq, D] kv dtype
  const void* k_cache;        // [NB, Hkv, BS, D]
  const void* v_cache;        // [NB, Hkv, D, BS]
  const int32_t* tables;      // [S, max_blocks]
  const int32_t* lens;        // [S]
  float scale_log2;           // scale * log2(e): scores are kept in base-2 units
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t group;              // num_heads / num_kv_heads, 1..16
  int32_t max_blocks;         // table row length
  int32_t num_blocks;         // pool size, for the block-id range check
  int32_t part_blocks_min;    // smallest partition the planner may pick (sizes the workspace)
  int32_t part_blocks_max;    // largest partition the planner may pick
  int32_t num_parts_max;      // ceil(max_blocks / part_blocks_min): partition-state row stride
  int32_t balance;            // planner: the largest item is at most 1/balance of a
                              // workgroup's share of the work (0: always part_blocks_min;
                              // the API sets 1 for adaptive, the launcher the ratio)
  int32_t decode_grid;        // workgroups of the decode launch (set by the launcher)
  int32_t num_cus;            // compute units of the device (set by the launcher)
  int32_t lds_slots;          // LDS state slots of the matrix-core kernel (set by the launcher)
  int32_t lds_records;        // LDS output records of the matrix-core kernel (set by the launcher)
  float* ws_acc;              // [S, Hkv, num_parts_max, group, D] partition sums
  float* ws_ml;               // [S, Hkv, num_parts_max, group, 2] partition (max, sum)
  int4* ws_items;             // [S * num_parts_max] work list: (sequence, partition, length,
                              //  first block: the sequence's shared-prefix blocks, else 0)
  int2* ws_split;             // [S] (sequence, partitions) of sequences spanning several:
                              //  up to kMergeShort partitions from the front, more from the back
  int32_t* ws_ctrl;           // [kCtrlSize] control words (planner, kernels)
  // Shared prefixes (num_groups == 0: none).  Sequences group_starts[g] ..
  // group_starts[g+1]-1 share their first prefix_blocks[g] table entries.
  const int32_t* group_starts;  // [num_groups + 1]
  const int32_t* prefix_blocks; // [num_groups]
  int32_t num_groups;
  int32_t prefix_rows;          // query rows one prefix item serves (its sequences x group)
  int4* ws_pitems;              // [S * num_parts_max] prefix work list:
                                //  (first sequence, sequences, partition, prefix blocks)
  int32_t packed_pool;          // diagnostic: block j of sequence s is tables[s, 0] + j
  int32_t inline_plan;          // the attention kernel plans the batch itself (no planner
                                //  launch; set by the launcher)
};

// ws_ctrl slots written by the planner: work-list entries, chosen partition
// size in blocks, number of split sequences.
constexpr int kCtrlEntries = 0;
constexpr int kCtrlPartBlocks = 1;
constexpr int kCtrlSplits = 2;
constexpr int kCtrlPrefixItems = 3;   // entries of the prefix work list
constexpr int kCtrlPrefixPart = 4;    // blocks per prefix partition
constexpr int kCtrlLongSplits = 5;    // split sequences with more than kMergeShort partitions,
                                      // listed from the back of ws_split
constexpr int kMergeShort = 16;
// Set by the decode kernel if one of its waits on other waves of its
// workgroup did not end (a broken invariant; the output is then incomplete).
// Cleared by the planner (or set by merge_splits, below); read through
// pa_decode_check.
constexpr int kCtrlAbort = 20;
// The same for an attention kernel that plans the batch itself (no planner
// launch clears anything before it): such a wait stores kAbortMark here, and
// merge_splits, which always follows that kernel, sets kCtrlAbort to whether
// the mark is present and clears this word.
constexpr int kCtrlAbortPlanned = 21;
constexpr int32_t kAbortMark = 0x5a17ab07;
// Claim counters of the matrix-core kernel's work list, one per pool, each
// in a 128-byte line of its own; zeroed by the planner (the self-planning
// kernel claims nothing).
constexpr int kClaimPools = 32;
constexpr int kClaimStride = 32;
constexpr int kCtrlClaims = 32;
constexpr int kCtrlSize = kCtrlClaims + kClaimPools * kClaimStride;

enum class KvType { F32 = 0, BF16 = 1 };

// Status helpers shared by the C entry points: fail() stores the message for
// pa_last_error() (thread-local) and returns `code`; succeed() clears it.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int succeed();

// Arguments of one slot write (device pointers); the element loop is in
// pa_write_body.h (device code).
struct WriteArgs {
  void* k_cache;
  void* v_cache;
  const void* k_new;
  const void* v_new;
  const int32_t* slots;
  int64_t total;        // num_tokens * num_kv_heads * head_dim elements
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t v_tile;       // tokens per feature-major V sub-tile: 16 if 16 | block_size, else block_size
  int64_t num_slots;    // num_blocks * block_size
  int32_t elem_bytes;   // 2 (bf16) or 4 (fp32)
  // Shifts for head_dim, num_kv_heads, block_size and v_tile when all four
  // are powers of two and element and slot indices fit in 31 bits (narrow);
  // the index arithmetic then takes shifts and masks instead of 64-bit
  // divisions.
  int32_t narrow;
  int32_t log2_d, log2_h, log2_bs, log2_vt;
};

WriteArgs make_write_args(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                          const int32_t* slots, int32_t num_tokens, int32_t num_blocks,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          KvType type);

hipError_t launch_write_kv(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                           const int32_t* slots, int32_t num_tokens, int32_t num_blocks,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           KvType type, hipStream_t stream);

// dst block dst_ids[i] := src block src_ids[i] in both tensors (spans of
// span_bytes); pairs with an id outside its pool are skipped.
hipError_t launch_copy_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                              const int32_t* src_ids, const int32_t* dst_ids, int32_t num_pairs,
                              int32_t src_blocks, int32_t dst_blocks, int64_t span_bytes,
                              hipStream_t stream);

// Returns hipErrorInvalidValue for a (type, D, BS) combination without a kernel.
// params_bytes is sizeof(DecodeParams) as the caller was compiled: if it is
// not the size this launcher was compiled with (objects built from two
// versions of this header and linked together), nothing is launched and
// hipErrorInvalidImage is returned; the kernels would otherwise read the
// pointers at the wrong offsets.
// Non-null events are recorded on `stream` right before and right after the
// attention kernel (not the planner or the merge), for kernel timing.
// A non-null `write` is a slot write done in the planner's launch (its
// workgroups other than the planner's), so the whole step takes one launch
// less; the write and the plan are independent.
hipError_t launch_decode(const DecodeParams& p, size_t params_bytes, KvType type,
                         int32_t head_dim, int32_t block_size, bool vector_alu,
                         hipStream_t stream, hipEvent_t ev_before = nullptr,
                         hipEvent_t ev_after = nullptr, const WriteArgs* write = nullptr);

// pa_decode with the library's adaptive partition size, its smallest choice
// raised to floor_tokens (a power-of-two multiple of the default smallest):
// the workspace then needs fewer partition states.  Same checks and status
// codes as pa_decode.
int decode_with_floor(float* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, float scale,
                      int32_t block_size, int32_t num_seqs, int32_t num_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                      int32_t num_blocks, int32_t kv_dtype, void* workspace,
                      size_t workspace_bytes, int32_t floor_tokens, void* stream);

// Smallest and (in *max_tokens) largest partition the adaptive choice may take.
int32_t adaptive_partition_limits(int32_t block_size, int32_t* max_tokens);

// Device address and size of pa_decode_noalloc's scratch on the current
// device (pa_noalloc.hip); a pa_status.
int noalloc_scratch(void** ptr, size_t* bytes);

// Enqueue on `stream` a copy of the workspace's abort word (int32 at
// ws_ctrl[kCtrlAbort]) into *flag (device or pinned host memory).
hipError_t launch_copy_word(const int32_t* src, int32_t* flag, hipStream_t stream);

bool decode_supported(KvType type, int32_t head_dim, int32_t block_size, int32_t group);

// Bandwidth probes (pa_probe.hip).  bytes: a multiple of 16; tile_bytes: 4096 or 8192.
hipError_t launch_probe_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);
hipError_t launch_probe_read_tiles(const void* k_cache, const void* v_cache, const int32_t* tiles,
                                   int32_t num_tiles, int32_t tile_bytes, int64_t pool_tiles,
                                   uint32_t* sink, hipStream_t stream);

}  // namespace pa
