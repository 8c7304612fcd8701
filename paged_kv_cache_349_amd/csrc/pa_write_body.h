// Slot-write element loop shared by the write kernel and the fused
// write + plan kernel (device code; included by .hip sources only).
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "pa_internal.h"

namespace pa {

// Elements first, first + stride, ... of the write: one per (token, kv head,
// feature).  Reads of k_new/v_new and the K-cache writes are contiguous along
// the feature; V-cache writes stride by v_tile elements because a V sub-tile
// keeps each feature's tokens together (token o, feature d of a tile at
// ((o / v_tile) * head_dim + d) * v_tile + o % v_tile).  Raw bits are copied
// (uint16 / uint32).
// The stores are nontemporal.  With ordinary stores the partly written lines
// stayed dirty in the caches and the decode that reads the pool next ran
// 198.6 us instead of 185.2 us on the large-batch workload (kernel trace, one
// host; a decode after another decode: 185-189 us), as if those lines were
// written back while it streamed; the write itself takes 6.6 us either way.
// With power-of-two sizes and 31-bit indices (w.narrow) the index
// arithmetic is shifts and masks: the 64-bit divisions of the general loop
// cost each wave hundreds of instructions before its first load.
template <typename E>
__device__ __forceinline__ void write_elements(const WriteArgs& w, int64_t first, int64_t stride) {
  E* __restrict__ kc = (E*)w.k_cache;
  E* __restrict__ vc = (E*)w.v_cache;
  const E* __restrict__ kn = (const E*)w.k_new;
  const E* __restrict__ vn = (const E*)w.v_new;
  if (w.narrow) {
    // total and step are below 2^31, so i + step never wraps.
    const uint32_t total = (uint32_t)w.total, step = (uint32_t)min(stride, (int64_t)INT32_MAX);
    const uint32_t mask_d = (1u << w.log2_d) - 1, mask_h = (1u << w.log2_h) - 1;
    const uint32_t mask_bs = (1u << w.log2_bs) - 1, mask_vt = (1u << w.log2_vt) - 1;
    for (uint32_t i = (uint32_t)min(first, w.total); i < total; i += step) {
      const uint32_t d = i & mask_d;
      const uint32_t th = i >> w.log2_d;
      const uint32_t h = th & mask_h;
      const uint32_t t = th >> w.log2_h;
      const int32_t slot = w.slots[t];
      if (slot < 0 || slot >= w.num_slots) continue;  // padding token, or out of the pool
      const uint32_t b = (uint32_t)slot >> w.log2_bs;
      const uint32_t o = (uint32_t)slot & mask_bs;
      const int64_t tile = (int64_t)b * w.num_kv_heads + h;
      const uint32_t sub = o >> w.log2_vt;
      __builtin_nontemporal_store(kn[i], &kc[(tile * w.block_size + o) * w.head_dim + d]);
      __builtin_nontemporal_store(vn[i], &vc[tile * w.block_size * w.head_dim +
                                             ((int64_t)sub * w.head_dim + d) * w.v_tile +
                                             (o & mask_vt)]);
    }
    return;
  }
  for (int64_t i = first; i < w.total; i += stride) {
    const int32_t d = (int32_t)(i % w.head_dim);
    const int64_t th = i / w.head_dim;
    const int32_t h = (int32_t)(th % w.num_kv_heads);
    const int64_t t = th / w.num_kv_heads;
    const int64_t slot = w.slots[t];
    if (slot < 0 || slot >= w.num_slots) continue;  // padding token, or out of the pool
    const int64_t b = slot / w.block_size;
    const int32_t o = (int32_t)(slot % w.block_size);
    const int64_t tile = b * w.num_kv_heads + h;
    const int32_t sub = o / w.v_tile;
    __builtin_nontemporal_store(kn[i], &kc[(tile * w.block_size + o) * w.head_dim + d]);
    __builtin_nontemporal_store(vn[i], &vc[tile * w.block_size * w.head_dim +
                                           ((int64_t)sub * w.head_dim + d) * w.v_tile +
                                           (o - sub * w.v_tile)]);
  }
}

}  // namespace pa
