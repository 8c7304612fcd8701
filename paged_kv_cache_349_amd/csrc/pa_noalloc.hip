// pa_decode for callers that cannot allocate: code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc.  The decode's
// workspace (work list, planner counters, partition states) is a file-scope
// device array of fixed size instead of a caller buffer.
//
// The array is one per device: each device the library runs on holds its
// copy, the driver's allocation of the code object's globals, until the
// process ends.  Host code never uses the array's name as an address (on the
// host it is only a stand-in): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current and
// kept here, and that pointer is what the kernels receive.
//
// Every call on a device shares that device's array, which keeps the last
// call's contents.  The decode planner initialises every word a call reads
// (its counters, claim counters and completion word are cleared at the start
// of each call), so nothing has to be cleared here.  Calls that overlap on
// one device (different streams, or threads) race on the array.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "paged_attention.h"
#include "pa_internal.h"

namespace {

// 64 MiB: the large-batch shape (256 sequences, 64 query heads of 128
// features, contexts up to 4.5k tokens) needs 45 MB of partition states at
// its smallest admissible partition (1024 tokens); contexts of up to 57k
// tokens fit at that batch with 8192-token partitions.
constexpr size_t kScratchBytes = size_t(64) << 20;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
std::map<int, void*> g_scratch;   // device -> address of its copy of `scratch`

}  // namespace

namespace pa {

int noalloc_scratch(void** ptr, size_t* bytes) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_mu);
  auto it = g_scratch.find(dev);
  if (it == g_scratch.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(PA_ERR_LAUNCH, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    it = g_scratch.emplace(dev, p).first;
  }
  *ptr = it->second;
  *bytes = kScratchBytes;
  return PA_OK;
}

}  // namespace pa

extern "C" int pa_decode_noalloc(float* out, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_tables,
                                 const int32_t* context_lens, float scale, int32_t block_size,
                                 int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_blocks_per_seq, int32_t num_blocks,
                                 int32_t kv_dtype, void* stream) {
  // The smallest partition whose workspace fits the scratch, in the adaptive
  // choice's own steps (the default smallest times a power of two), so the
  // partition the planner picks is unchanged whenever it is at least that.
  int32_t max_tokens = 0;
  int32_t floor_tokens = pa::adaptive_partition_limits(block_size > 0 ? block_size : 1, &max_tokens);
  size_t need = 0;
  for (;;) {
    need = pa_decode_workspace_bytes_ex(num_seqs, num_heads, num_kv_heads, head_dim,
                                        max_blocks_per_seq, block_size, kv_dtype, floor_tokens);
    if (need == 0 || need <= kScratchBytes || floor_tokens * 2 > max_tokens) break;
    floor_tokens *= 2;
  }
  if (need != 0 && need > kScratchBytes)
    return pa::fail(PA_ERR_WORKSPACE,
                    "these shapes need %zu bytes of decode workspace even with %d-token "
                    "partitions; pa_decode_noalloc has %zu (use pa_decode with a caller workspace)",
                    need, floor_tokens, kScratchBytes);
  // pa_decode's argument checks first, with no workspace: anything but the
  // missing workspace (an argument error, or an empty batch) is the answer.
  // Nothing is launched either way.
  const int dry = pa::decode_with_floor(out, q, k_cache, v_cache, block_tables, context_lens,
                                        scale, block_size, num_seqs, num_heads, num_kv_heads,
                                        head_dim, max_blocks_per_seq, num_blocks, kv_dtype,
                                        nullptr, 0, floor_tokens, stream);
  if (dry != PA_ERR_WORKSPACE) return dry;
  void* ptr = nullptr;
  size_t bytes = 0;
  const int st = pa::noalloc_scratch(&ptr, &bytes);
  if (st != PA_OK) return st;
  return pa::decode_with_floor(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                               block_size, num_seqs, num_heads, num_kv_heads, head_dim,
                               max_blocks_per_seq, num_blocks, kv_dtype, ptr, bytes, floor_tokens,
                               stream);
}
