// Slot write: copy each new token's K and V into its slot of the block pool.
//
// "How does vLLM PagedAttention manage Virtual Memory Pages to eliminate KV
// cache fragmentation?", section "Key Technical Innovations" (item 2) and
// section "Example": a sequence's new token goes into its current physical
// block.  The slot (block * block_size + offset) comes from the caller.
//
// The copy is of raw element bits (uint16 for bf16, uint32 for fp32), never
// through a float register, so every bit pattern arrives unchanged.
// Bound: a few MiB per step at most; the work is one pass over k_new/v_new.
#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pa {
namespace {

// One thread per (token, kv head, feature) element.  Reads of k_new/v_new and
// the K-cache writes are contiguous along the feature; V-cache writes stride
// by block_size elements because a V tile keeps each feature's tokens together.
template <typename E>
__global__ __launch_bounds__(256) void write_kv_kernel(E* __restrict__ kc, E* __restrict__ vc,
                                                        const E* __restrict__ kn,
                                                        const E* __restrict__ vn,
                                                        const int32_t* __restrict__ slots,
                                                        int64_t total, int32_t num_kv_heads,
                                                        int32_t head_dim, int32_t block_size,
                                                        int64_t num_slots) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int32_t d = (int32_t)(i % head_dim);
    const int64_t th = i / head_dim;
    const int32_t h = (int32_t)(th % num_kv_heads);
    const int64_t t = th / num_kv_heads;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_slots) continue;  // padding token, or out of the pool
    const int64_t b = slot / block_size;
    const int32_t o = (int32_t)(slot % block_size);
    const int64_t tile = b * num_kv_heads + h;
    kc[(tile * block_size + o) * head_dim + d] = kn[i];
    vc[(tile * head_dim + d) * block_size + o] = vn[i];
  }
}

}  // namespace

hipError_t launch_write_kv(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                           const int32_t* slots, int32_t num_tokens, int32_t num_blocks,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           KvType type, hipStream_t stream) {
  const int64_t total = (int64_t)num_tokens * num_kv_heads * head_dim;
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;  // grid-stride loop covers the rest
  if (type == KvType::BF16) {
    hipLaunchKernelGGL(write_kv_kernel<uint16_t>, dim3((unsigned)blocks), dim3(threads), 0,
                       stream, (uint16_t*)k_cache, (uint16_t*)v_cache, (const uint16_t*)k_new,
                       (const uint16_t*)v_new, slots, total, num_kv_heads, head_dim, block_size,
                       num_slots);
  } else {
    hipLaunchKernelGGL(write_kv_kernel<uint32_t>, dim3((unsigned)blocks), dim3(threads), 0,
                       stream, (uint32_t*)k_cache, (uint32_t*)v_cache, (const uint32_t*)k_new,
                       (const uint32_t*)v_new, slots, total, num_kv_heads, head_dim, block_size,
                       num_slots);
  }
  return hipGetLastError();
}

}  // namespace pa
