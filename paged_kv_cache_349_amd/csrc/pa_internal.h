// Internal interface between the C ABI (pa_api.cpp) and the kernel launchers.
// Not installed; callers use include/paged_attention.h.
#pragma once

#include <hip/hip_runtime_api.h>
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
  int32_t part_blocks;        // blocks per partition (one workgroup each)
  int32_t num_parts_max;      // ceil(max_blocks / part_blocks)
  float* ws_acc;              // [S, Hkv, num_parts_max, group, D] partition sums
  float* ws_ml;               // [S, Hkv, num_parts_max, group, 2] partition (max, sum)
};

enum class KvType { F32 = 0, BF16 = 1 };

hipError_t launch_write_kv(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                           const int32_t* slots, int32_t num_tokens, int32_t num_blocks,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           KvType type, hipStream_t stream);

// Returns hipErrorInvalidValue for a (type, D, BS) combination without a kernel.
hipError_t launch_decode(const DecodeParams& p, KvType type, int32_t head_dim,
                         int32_t block_size, bool vector_alu, hipStream_t stream);

bool decode_supported(KvType type, int32_t head_dim, int32_t block_size, int32_t group);

}  // namespace pa
