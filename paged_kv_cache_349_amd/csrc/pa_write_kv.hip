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
// The element loop (pa_write_body.h) also runs inside the decode planner's
// launch when a whole step is issued at once (pa_decode_step).
#include <hip/hip_runtime.h>

#include "pa_internal.h"
#include "pa_write_body.h"

namespace pa {
namespace {

template <typename E>
__global__ __launch_bounds__(256) void write_kv_kernel(WriteArgs w) {
  write_elements<E>(w, (int64_t)blockIdx.x * blockDim.x + threadIdx.x,
                    (int64_t)gridDim.x * blockDim.x);
}

}  // namespace

WriteArgs make_write_args(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                          const int32_t* slots, int32_t num_tokens, int32_t num_blocks,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          KvType type) {
  WriteArgs w;
  w.k_cache = k_cache;
  w.v_cache = v_cache;
  w.k_new = k_new;
  w.v_new = v_new;
  w.slots = slots;
  w.total = (int64_t)num_tokens * num_kv_heads * head_dim;
  w.num_kv_heads = num_kv_heads;
  w.head_dim = head_dim;
  w.block_size = block_size;
  w.v_tile = block_size % 16 == 0 ? 16 : block_size;
  w.num_slots = (int64_t)num_blocks * block_size;
  w.elem_bytes = type == KvType::BF16 ? 2 : 4;
  auto log2_of = [](int64_t v) {   // -1 unless v is a power of two
    if (v <= 0 || (v & (v - 1)) != 0) return -1;
    int k = 0;
    while ((int64_t(1) << k) < v) ++k;
    return k;
  };
  w.log2_d = log2_of(head_dim);
  w.log2_h = log2_of(num_kv_heads);
  w.log2_bs = log2_of(block_size);
  w.log2_vt = log2_of(w.v_tile);
  w.narrow = w.log2_d >= 0 && w.log2_h >= 0 && w.log2_bs >= 0 && w.log2_vt >= 0 &&
             w.total <= INT32_MAX && w.num_slots <= INT32_MAX;
  return w;
}

hipError_t launch_write_kv(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                           const int32_t* slots, int32_t num_tokens, int32_t num_blocks,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           KvType type, hipStream_t stream) {
  const WriteArgs w = make_write_args(k_cache, v_cache, k_new, v_new, slots, num_tokens,
                                      num_blocks, num_kv_heads, head_dim, block_size, type);
  const int threads = 256;
  int64_t blocks = (w.total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;  // grid-stride loop covers the rest
  if (type == KvType::BF16)
    hipLaunchKernelGGL(write_kv_kernel<uint16_t>, dim3((unsigned)blocks), dim3(threads), 0,
                       stream, w);
  else
    hipLaunchKernelGGL(write_kv_kernel<uint32_t>, dim3((unsigned)blocks), dim3(threads), 0,
                       stream, w);
  return hipGetLastError();
}

}  // namespace pa
