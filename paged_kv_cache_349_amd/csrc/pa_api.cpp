// C ABI of libpa.so: argument checks, partition choice, dispatch.
// The declarations and the contract live in include/paged_attention.h.
#include "paged_attention.h"
#include "block_manager.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <utility>
#include <vector>

#include "pa_internal.h"

namespace {
thread_local char g_last_error[512];
}  // namespace

namespace pa {

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int succeed() {
  g_last_error[0] = '\0';
  return PA_OK;
}

}  // namespace pa

namespace {

using pa::fail;
int ok() { return pa::succeed(); }

constexpr double kLog2e = 1.4426950408889634;

// Partition (work item) size.  With partition_tokens == 0 the decode
// planner picks, on the device from the actual context lengths, a power-of-two
// multiple of the smallest size below, up to the largest, small enough for
// the work to spread evenly over the resident workgroups (the launcher sets
// the ratio).  The workspace is sized for the smallest.
constexpr int32_t kMinPartitionTokens = 256;
constexpr int32_t kMaxPartitionTokens = 8192;
// The planner keeps per-sequence lengths and prefix starts in LDS.
constexpr int32_t kMaxPrefixSeqs = 8192;

int32_t min_partition_tokens(int32_t block_size) {
  const int32_t t = kMinPartitionTokens < block_size ? block_size : kMinPartitionTokens;
  return t - t % block_size;
}

// Workspace regions, each 256-byte aligned: planner outputs, work list, list
// of split sequences, and (when a sequence may span several partitions) the
// partition states.  With shared prefixes: one more partition per sequence
// (the prefix is cut on its own, so the cuts may add one partition), the
// prefix work list, and partition states always (every sequence with a
// shared prefix is merged).
struct Layout {
  int32_t part_blocks = 0;
  int32_t num_parts_max = 0;
  size_t ctrl_off = 0, items_off = 0, split_off = 0, acc_off = 0, ml_off = 0, pitems_off = 0;
  size_t total = 0;
};

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

Layout workspace_layout(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                        int32_t max_blocks, int32_t block_size, int32_t partition_tokens,
                        bool prefix = false) {
  Layout l;
  l.part_blocks = partition_tokens / block_size;
  l.num_parts_max = (max_blocks + l.part_blocks - 1) / l.part_blocks + (prefix ? 1 : 0);
  size_t off = 0;
  l.ctrl_off = off;
  off += align256(pa::kCtrlSize * sizeof(int32_t));
  l.items_off = off;
  off += align256((size_t)num_seqs * l.num_parts_max * 4 * sizeof(int32_t));
  l.split_off = off;
  off += align256((size_t)num_seqs * 2 * sizeof(int32_t));
  if (l.num_parts_max > 1) {
    const size_t rows = (size_t)num_seqs * num_heads * l.num_parts_max;
    l.acc_off = off;
    off += align256(rows * head_dim * sizeof(float));
    l.ml_off = off;
    off += align256(rows * 2 * sizeof(float));
  }
  if (prefix) {
    l.pitems_off = off;
    off += align256((size_t)num_seqs * l.num_parts_max * 4 * sizeof(int32_t));
  }
  l.total = off;
  return l;
}

// Event pairs handed to the decode launcher while kernel timing is on.
struct KernelTiming {
  std::mutex mu;
  bool on = false;
  int device = -1;
  size_t used = 0;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> events;

  void release() {
    for (auto& ev : events) {
      hipEventDestroy(ev.first);
      hipEventDestroy(ev.second);
    }
    events.clear();
    used = 0;
    on = false;
  }
};

KernelTiming g_timing;

// The next unused event pair if timing is on for the current device.
std::pair<hipEvent_t, hipEvent_t> next_timing_events() {
  std::lock_guard<std::mutex> lock(g_timing.mu);
  int dev = -1;
  if (!g_timing.on || g_timing.used >= g_timing.events.size() || hipGetDevice(&dev) != hipSuccess ||
      dev != g_timing.device)
    return {nullptr, nullptr};
  return g_timing.events[g_timing.used++];
}

bool shapes_valid(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                  int32_t max_blocks, int32_t block_size) {
  return num_seqs >= 0 && num_heads > 0 && num_kv_heads > 0 && head_dim > 0 && max_blocks > 0 &&
         block_size > 0 && num_heads % num_kv_heads == 0;
}

static int decode_common(float* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens, float scale,
                         int32_t block_size, int32_t num_seqs, int32_t num_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                         int32_t num_blocks, int32_t kv_dtype, void* workspace,
                         size_t workspace_bytes, int32_t partition_tokens, int32_t flags,
                         const int32_t* group_starts, const int32_t* prefix_blocks,
                         int32_t num_groups, bool prefix, void* stream,
                         const pa::WriteArgs* write = nullptr, int32_t floor_tokens = 0) {
  if (kv_dtype != PA_DTYPE_F32 && kv_dtype != PA_DTYPE_BF16)
    return fail(PA_ERR_UNSUPPORTED, "kv_dtype=%d is neither F32 nor BF16", kv_dtype);
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs=%d < 0", num_seqs);
  if (num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      max_blocks_per_seq <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG,
                "sizes must be positive (num_heads=%d num_kv_heads=%d head_dim=%d block_size=%d "
                "max_blocks_per_seq=%d num_blocks=%d)",
                num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks);
  if (num_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "num_heads=%d is not a multiple of num_kv_heads=%d",
                num_heads, num_kv_heads);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale is not finite");
  if (flags & ~(PA_FLAG_VECTOR_ALU | PA_FLAG_PACKED_POOL))
    return fail(PA_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if ((flags & PA_FLAG_PACKED_POOL) &&
      (kv_dtype != PA_DTYPE_BF16 || (flags & PA_FLAG_VECTOR_ALU) || prefix))
    return fail(PA_ERR_UNSUPPORTED,
                "the packed-pool diagnostic runs the bf16 matrix-core kernel without prefixes only");
  const int32_t group = num_heads / num_kv_heads;
  if (!pa::decode_supported((pa::KvType)kv_dtype, head_dim, block_size, group))
    return fail(PA_ERR_UNSUPPORTED,
                "no kernel for head_dim=%d block_size=%d group=%d (compiled: head_dim 64/128, "
                "block_size 16/32, group 1..16)",
                head_dim, block_size, group);
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX ||
      (int64_t)num_seqs * num_heads * head_dim > INT32_MAX * 4LL)
    return fail(PA_ERR_UNSUPPORTED, "shape too large");
  const bool adaptive = partition_tokens == 0;
  if (adaptive) {
    partition_tokens = min_partition_tokens(block_size);
    if (floor_tokens > partition_tokens) partition_tokens = floor_tokens;
  }
  if (partition_tokens < block_size || partition_tokens % block_size != 0)
    return fail(PA_ERR_INVALID_ARG, "partition_tokens=%d is not a positive multiple of %d",
                partition_tokens, block_size);
  if (prefix) {
    if (num_groups < 0) return fail(PA_ERR_INVALID_ARG, "num_groups=%d < 0", num_groups);
    if (kv_dtype != PA_DTYPE_BF16 || (flags & PA_FLAG_VECTOR_ALU))
      return fail(PA_ERR_UNSUPPORTED, "shared-prefix decode runs the bf16 matrix-core kernels only");
    if (num_seqs > kMaxPrefixSeqs)
      return fail(PA_ERR_UNSUPPORTED, "shared-prefix decode handles at most %d sequences",
                  kMaxPrefixSeqs);
  }
  if (num_seqs == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID_ARG, "null device pointer");
  if (prefix && num_groups > 0 && (!group_starts || !prefix_blocks))
    return fail(PA_ERR_INVALID_ARG, "null group array with num_groups=%d", num_groups);
  if (((uintptr_t)out | (uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache) % 16 != 0)
    return fail(PA_ERR_INVALID_ARG, "out, q, k_cache and v_cache must be 16-byte aligned");
  const Layout lay = workspace_layout(num_seqs, num_heads, head_dim, max_blocks_per_seq,
                                      block_size, partition_tokens, prefix);
  if (!workspace || workspace_bytes < lay.total)
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes at %p; %zu bytes needed",
                workspace_bytes, workspace, lay.total);
  if ((uintptr_t)workspace % 256 != 0)
    return fail(PA_ERR_WORKSPACE, "workspace at %p must be 256-byte aligned", workspace);
  if ((int64_t)lay.num_parts_max * num_seqs * num_kv_heads > (INT32_MAX >> 1) ||
      (int64_t)max_blocks_per_seq * num_seqs > (INT32_MAX >> 1))
    return fail(PA_ERR_UNSUPPORTED, "too many work items");

  pa::DecodeParams p;
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.tables = block_tables;
  p.lens = context_lens;
  p.scale_log2 = (float)((double)scale * kLog2e);
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = group;
  p.max_blocks = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.part_blocks_min = lay.part_blocks;
  const int32_t max_tokens = kMaxPartitionTokens < block_size ? block_size : kMaxPartitionTokens;
  p.part_blocks_max = adaptive ? max_tokens / block_size : lay.part_blocks;
  p.num_parts_max = lay.num_parts_max;
  p.balance = adaptive ? 1 : 0;   // the launcher sets the ratio
  p.decode_grid = 0;
  char* ws = (char*)workspace;
  p.ws_ctrl = (int32_t*)(ws + lay.ctrl_off);
  p.ws_items = (int4*)(ws + lay.items_off);
  p.ws_split = (int2*)(ws + lay.split_off);
  p.ws_acc = lay.num_parts_max > 1 ? (float*)(ws + lay.acc_off) : nullptr;
  p.ws_ml = lay.num_parts_max > 1 ? (float*)(ws + lay.ml_off) : nullptr;
  p.group_starts = prefix ? group_starts : nullptr;
  p.prefix_blocks = prefix ? prefix_blocks : nullptr;
  p.num_groups = prefix ? num_groups : 0;
  p.prefix_rows = 0;   // set by the launcher
  p.ws_pitems = prefix ? (int4*)(ws + lay.pitems_off) : nullptr;
  p.packed_pool = (flags & PA_FLAG_PACKED_POOL) ? 1 : 0;
  p.inline_plan = 0;   // set by the launcher
  const auto ev = next_timing_events();
  hipError_t e = pa::launch_decode(p, sizeof(pa::DecodeParams), (pa::KvType)kv_dtype, head_dim,
                                   block_size, (flags & PA_FLAG_VECTOR_ALU) != 0,
                                   (hipStream_t)stream, ev.first, ev.second, write);
  if (e == hipErrorInvalidImage)
    return fail(PA_ERR_LAUNCH,
                "decode launch: the library's objects disagree on the launch-parameter layout "
                "(%zu bytes here); rebuild every object",
                sizeof(pa::DecodeParams));
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

namespace pa {

int decode_with_floor(float* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, float scale,
                      int32_t block_size, int32_t num_seqs, int32_t num_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                      int32_t num_blocks, int32_t kv_dtype, void* workspace,
                      size_t workspace_bytes, int32_t floor_tokens, void* stream) {
  return decode_common(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                       num_seqs, num_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                       num_blocks, kv_dtype, workspace, workspace_bytes, 0, 0, nullptr, nullptr,
                       0, false, stream, nullptr, floor_tokens);
}

int32_t adaptive_partition_limits(int32_t block_size, int32_t* max_tokens) {
  *max_tokens = kMaxPartitionTokens < block_size ? block_size : kMaxPartitionTokens;
  return min_partition_tokens(block_size);
}

}  // namespace pa

extern "C" {

const char* pa_status_string(int32_t status) {
  switch (status) {
    case PA_OK: return "success";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported dtype/shape combination";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_LAUNCH: return "kernel launch failed";
    case PA_ERR_NO_ROOM: return "no room in the block pool";
    default: return "unknown status";
  }
}

const char* pa_status_str(int32_t status) { return pa_status_string(status); }

const char* pa_last_error(void) { return g_last_error; }

// Argument checks of a slot write; PA_OK means it may be launched (a write
// of 0 tokens launches nothing).
static int check_write(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                       const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int32_t kv_dtype) {
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens=%d < 0", num_tokens);
  if (kv_dtype != PA_DTYPE_F32 && kv_dtype != PA_DTYPE_BF16)
    return fail(PA_ERR_UNSUPPORTED, "kv_dtype=%d is neither F32 nor BF16", kv_dtype);
  if (num_blocks <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
    return fail(PA_ERR_INVALID_ARG,
                "sizes must be positive (num_blocks=%d num_kv_heads=%d head_dim=%d block_size=%d)",
                num_blocks, num_kv_heads, head_dim, block_size);
  if (head_dim > 1024) return fail(PA_ERR_UNSUPPORTED, "head_dim=%d > 1024", head_dim);
  if (num_tokens > 0 && (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping))
    return fail(PA_ERR_INVALID_ARG, "null device pointer with num_tokens=%d", num_tokens);
  return PA_OK;
}

int pa_write_kv(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t kv_dtype,
                void* stream) {
  const int st = check_write(k_cache, v_cache, k_new, v_new, slot_mapping, num_tokens,
                             num_blocks, num_kv_heads, head_dim, block_size, kv_dtype);
  if (st != PA_OK) return st;
  if (num_tokens == 0) return ok();
  hipError_t e = pa::launch_write_kv(k_cache, v_cache, k_new, v_new, slot_mapping, num_tokens,
                                     num_blocks, num_kv_heads, head_dim, block_size,
                                     (pa::KvType)kv_dtype, (hipStream_t)stream);
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "write_kv launch: %s", hipGetErrorString(e));
  return ok();
}

int pa_decode_step(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                   const int32_t* slot_mapping, int32_t num_tokens, float* out, const void* q,
                   const int32_t* block_tables, const int32_t* context_lens, float scale,
                   int32_t block_size, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                   int32_t head_dim, int32_t max_blocks_per_seq, int32_t num_blocks,
                   int32_t kv_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_write(k_cache, v_cache, k_new, v_new, slot_mapping, num_tokens,
                             num_blocks, num_kv_heads, head_dim, block_size, kv_dtype);
  if (st != PA_OK) return st;
  if (num_tokens == 0 || num_seqs == 0) {
    // Nothing to share a launch with: the plain calls.  Decode goes first (it
    // launches nothing when num_seqs == 0), so that a failing step launches
    // nothing.
    const int d = pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                            block_size, num_seqs, num_heads, num_kv_heads, head_dim,
                            max_blocks_per_seq, num_blocks, kv_dtype, workspace, workspace_bytes,
                            stream);
    if (d != PA_OK || num_tokens == 0) return d;
    return pa_write_kv(k_cache, v_cache, k_new, v_new, slot_mapping, num_tokens, num_blocks,
                       num_kv_heads, head_dim, block_size, kv_dtype, stream);
  }
  const pa::WriteArgs w =
      pa::make_write_args(k_cache, v_cache, k_new, v_new, slot_mapping, num_tokens, num_blocks,
                          num_kv_heads, head_dim, block_size, (pa::KvType)kv_dtype);
  return decode_common(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                       num_seqs, num_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                       num_blocks, kv_dtype, workspace, workspace_bytes, 0, 0, nullptr, nullptr,
                       0, false, stream, &w);
}

static int copy_blocks_common(const char* what, void* dst_k, void* dst_v, const void* src_k,
                              const void* src_v, const int32_t* src_ids, const int32_t* dst_ids,
                              int32_t num_pairs, int32_t src_blocks, int32_t dst_blocks,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int32_t kv_dtype, void* stream) {
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARG, "%s: num_pairs=%d < 0", what, num_pairs);
  if (kv_dtype != PA_DTYPE_F32 && kv_dtype != PA_DTYPE_BF16)
    return fail(PA_ERR_UNSUPPORTED, "%s: kv_dtype=%d is neither F32 nor BF16", what, kv_dtype);
  if (src_blocks <= 0 || dst_blocks <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
    return fail(PA_ERR_INVALID_ARG,
                "%s: sizes must be positive (blocks %d/%d num_kv_heads=%d head_dim=%d "
                "block_size=%d)",
                what, src_blocks, dst_blocks, num_kv_heads, head_dim, block_size);
  if (num_pairs == 0) return ok();
  if (!dst_k || !dst_v || !src_k || !src_v || !src_ids || !dst_ids)
    return fail(PA_ERR_INVALID_ARG, "%s: null pointer with num_pairs=%d", what, num_pairs);
  const int64_t span = (int64_t)num_kv_heads * head_dim * block_size *
                       (kv_dtype == PA_DTYPE_BF16 ? 2 : 4);
  hipError_t e = pa::launch_copy_blocks(dst_k, dst_v, src_k, src_v, src_ids, dst_ids, num_pairs,
                                        src_blocks, dst_blocks, span, (hipStream_t)stream);
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "%s launch: %s", what, hipGetErrorString(e));
  return ok();
}

int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_blocks,
                   const int32_t* dst_blocks, int32_t num_pairs, int32_t num_blocks,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t kv_dtype,
                   void* stream) {
  return copy_blocks_common("copy_blocks", k_cache, v_cache, k_cache, v_cache, src_blocks,
                            dst_blocks, num_pairs, num_blocks, num_blocks, num_kv_heads, head_dim,
                            block_size, kv_dtype, stream);
}

int pa_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                   const int32_t* src_blocks, const int32_t* dst_blocks, int32_t num_pairs,
                   int32_t src_num_blocks, int32_t dst_num_blocks, int32_t num_kv_heads,
                   int32_t head_dim, int32_t block_size, int32_t kv_dtype, void* stream) {
  return copy_blocks_common("swap_blocks", dst_k, dst_v, src_k, src_v, src_blocks, dst_blocks,
                            num_pairs, src_num_blocks, dst_num_blocks, num_kv_heads, head_dim,
                            block_size, kv_dtype, stream);
}

int32_t pa_decode_partition_tokens(int32_t num_seqs, int32_t num_kv_heads,
                                   int32_t max_blocks_per_seq, int32_t block_size) {
  if (num_seqs < 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 || block_size <= 0) return 0;
  return min_partition_tokens(block_size);
}

size_t pa_decode_workspace_bytes_ex(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t max_blocks_per_seq,
                                    int32_t block_size, int32_t kv_dtype,
                                    int32_t partition_tokens) {
  (void)kv_dtype;
  if (!shapes_valid(num_seqs, num_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size))
    return 0;
  if (partition_tokens == 0) partition_tokens = min_partition_tokens(block_size);
  if (partition_tokens < block_size || partition_tokens % block_size != 0) return 0;
  return workspace_layout(num_seqs, num_heads, head_dim, max_blocks_per_seq, block_size,
                          partition_tokens)
      .total;
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_blocks_per_seq,
                                 int32_t block_size, int32_t kv_dtype) {
  return pa_decode_workspace_bytes_ex(num_seqs, num_heads, num_kv_heads, head_dim,
                                      max_blocks_per_seq, block_size, kv_dtype, 0);
}

int pa_decode_ex(float* out, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, const int32_t* context_lens, float scale,
                 int32_t block_size, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                 int32_t head_dim, int32_t max_blocks_per_seq, int32_t num_blocks,
                 int32_t kv_dtype, void* workspace, size_t workspace_bytes,
                 int32_t partition_tokens, int32_t flags, void* stream) {
  return decode_common(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                       num_seqs, num_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                       num_blocks, kv_dtype, workspace, workspace_bytes, partition_tokens, flags,
                       nullptr, nullptr, 0, false, stream);
}

size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                               int32_t num_kv_heads, int32_t head_dim,
                                               int32_t max_blocks_per_seq, int32_t block_size,
                                               int32_t kv_dtype, int32_t partition_tokens) {
  (void)kv_dtype;
  if (!shapes_valid(num_seqs, num_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size))
    return 0;
  if (partition_tokens == 0) partition_tokens = min_partition_tokens(block_size);
  if (partition_tokens < block_size || partition_tokens % block_size != 0) return 0;
  return workspace_layout(num_seqs, num_heads, head_dim, max_blocks_per_seq, block_size,
                          partition_tokens, true)
      .total;
}

int pa_decode_shared_prefix(float* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            const int32_t* group_starts, const int32_t* prefix_blocks,
                            int32_t num_groups, float scale, int32_t block_size, int32_t num_seqs,
                            int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t max_blocks_per_seq, int32_t num_blocks, int32_t kv_dtype,
                            void* workspace, size_t workspace_bytes, int32_t partition_tokens,
                            void* stream) {
  return decode_common(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                       num_seqs, num_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                       num_blocks, kv_dtype, workspace, workspace_bytes, partition_tokens, 0,
                       group_starts, prefix_blocks, num_groups, true, stream);
}

int pa_decode(float* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, float scale,
              int32_t block_size, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
              int32_t head_dim, int32_t max_blocks_per_seq, int32_t num_blocks, int32_t kv_dtype,
              void* workspace, size_t workspace_bytes, void* stream) {
  return pa_decode_ex(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                      num_seqs, num_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                      num_blocks, kv_dtype, workspace, workspace_bytes, 0, 0, stream);
}

int pa_decode_check(const void* workspace, size_t workspace_bytes, int32_t* flag, void* stream) {
  if (!flag) return fail(PA_ERR_INVALID_ARG, "null flag pointer");
  if (!workspace && workspace_bytes == 0) {
    // The scratch of pa_decode_noalloc on the current device.
    void* ptr = nullptr;
    const int st = pa::noalloc_scratch(&ptr, &workspace_bytes);
    if (st != PA_OK) return st;
    workspace = ptr;
  }
  if (!workspace) return fail(PA_ERR_INVALID_ARG, "null workspace with workspace_bytes=%zu",
                              workspace_bytes);
  if ((uintptr_t)workspace % 256 != 0)
    return fail(PA_ERR_WORKSPACE, "workspace at %p must be 256-byte aligned", workspace);
  if (workspace_bytes < (size_t)pa::kCtrlSize * sizeof(int32_t))
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than any decode workspace",
                workspace_bytes);
  if ((uintptr_t)flag % sizeof(int32_t) != 0)
    return fail(PA_ERR_INVALID_ARG, "flag at %p is not 4-byte aligned", (void*)flag);
  hipError_t e = pa::launch_copy_word((const int32_t*)workspace + pa::kCtrlAbort, flag,
                                      (hipStream_t)stream);
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "decode_check launch: %s", hipGetErrorString(e));
  return ok();
}

int pa_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes == 0) return ok();
  if (!src || !sink) return fail(PA_ERR_INVALID_ARG, "null pointer");
  if (bytes % 16 != 0 || (uintptr_t)src % 16 != 0)
    return fail(PA_ERR_INVALID_ARG, "bytes=%zu and src must be multiples of 16", bytes);
  hipError_t e = pa::launch_probe_read(src, (int64_t)bytes, sink, (hipStream_t)stream);
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "probe_read launch: %s", hipGetErrorString(e));
  return ok();
}

int pa_probe_read_tiles(const void* k_cache, const void* v_cache, const int32_t* tiles,
                        int32_t num_tiles, int32_t tile_bytes, int64_t pool_tiles, uint32_t* sink,
                        void* stream) {
  if (num_tiles < 0 || pool_tiles < 0)
    return fail(PA_ERR_INVALID_ARG, "num_tiles=%d pool_tiles=%lld", num_tiles,
                (long long)pool_tiles);
  if (tile_bytes != 4096 && tile_bytes != 8192)
    return fail(PA_ERR_UNSUPPORTED, "tile_bytes=%d is neither 4096 nor 8192", tile_bytes);
  if (num_tiles == 0) return ok();
  if (!k_cache || !v_cache || !tiles || !sink) return fail(PA_ERR_INVALID_ARG, "null pointer");
  if (((uintptr_t)k_cache | (uintptr_t)v_cache) % 16 != 0)
    return fail(PA_ERR_INVALID_ARG, "caches must be 16-byte aligned");
  hipError_t e = pa::launch_probe_read_tiles(k_cache, v_cache, tiles, num_tiles, tile_bytes,
                                             pool_tiles, sink, (hipStream_t)stream);
  if (e != hipSuccess)
    return fail(PA_ERR_LAUNCH, "probe_read_tiles launch: %s", hipGetErrorString(e));
  return ok();
}

int pa_kernel_timing_begin(int32_t capacity) {
  if (capacity <= 0 || capacity > (1 << 20))
    return fail(PA_ERR_INVALID_ARG, "capacity=%d is not in [1, 2^20]", capacity);
  std::lock_guard<std::mutex> lock(g_timing.mu);
  if (g_timing.on) return fail(PA_ERR_INVALID_ARG, "kernel timing is already on");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
  g_timing.events.reserve((size_t)capacity);
  for (int32_t i = 0; i < capacity; ++i) {
    hipEvent_t a = nullptr, b = nullptr;
    e = hipEventCreate(&a);
    if (e == hipSuccess) {
      e = hipEventCreate(&b);
      if (e != hipSuccess) hipEventDestroy(a);
    }
    if (e != hipSuccess) {
      g_timing.release();
      return fail(PA_ERR_LAUNCH, "hipEventCreate: %s", hipGetErrorString(e));
    }
    g_timing.events.emplace_back(a, b);
  }
  g_timing.device = dev;
  g_timing.used = 0;
  g_timing.on = true;
  return ok();
}

int pa_kernel_timing_end(double* total_ms, int32_t* launches) {
  if (!total_ms || !launches) return fail(PA_ERR_INVALID_ARG, "null output pointer");
  std::lock_guard<std::mutex> lock(g_timing.mu);
  if (!g_timing.on) return fail(PA_ERR_INVALID_ARG, "kernel timing is not on");
  double sum = 0.0;
  hipError_t e = hipSuccess;
  for (size_t i = 0; i < g_timing.used && e == hipSuccess; ++i) {
    float ms = 0.0f;
    e = hipEventSynchronize(g_timing.events[i].second);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, g_timing.events[i].first,
                                                 g_timing.events[i].second);
    sum += ms;
  }
  const size_t used = g_timing.used;
  g_timing.release();
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "kernel timing events: %s", hipGetErrorString(e));
  *total_ms = sum;
  *launches = (int32_t)used;
  return ok();
}

}  // extern "C"
