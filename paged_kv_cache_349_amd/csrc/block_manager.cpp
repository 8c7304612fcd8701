// Host-side KV block manager (C ABI in include/block_manager.h).
//
// Free lists are rings (allocation at the front, release at the back), so
// every operation is O(blocks touched).  Sequences live in a hash map from
// their 64-bit id; each holds its table as a vector of block ids.
#include "block_manager.h"

#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "paged_attention.h"
#include "pa_internal.h"

namespace {

// FIFO of free block ids with room for the whole pool.
class FreeRing {
 public:
  explicit FreeRing(int32_t n) : buf_((size_t)(n > 0 ? n : 1)), head_(0), size_(0) {}
  int32_t size() const { return size_; }
  int32_t capacity() const { return (int32_t)buf_.size(); }
  void push(int32_t b) {
    buf_[(size_t)((head_ + size_) % capacity())] = b;
    ++size_;
  }
  int32_t pop() {
    const int32_t b = buf_[(size_t)head_];
    head_ = (head_ + 1) % capacity();
    --size_;
    return b;
  }
  int32_t at(int32_t i) const { return buf_[(size_t)((head_ + i) % capacity())]; }

 private:
  std::vector<int32_t> buf_;
  int32_t head_, size_;
};

struct Pool {
  explicit Pool(int32_t n) : free(n), ref((size_t)n, 0) {}
  FreeRing free;
  std::vector<int32_t> ref;
  int32_t size() const { return (int32_t)ref.size(); }
  int32_t take() {
    const int32_t b = free.pop();
    ref[(size_t)b] = 1;
    return b;
  }
  void release(int32_t b) {
    if (--ref[(size_t)b] == 0) free.push(b);
  }
};

struct Seq {
  std::vector<int32_t> table;
  int32_t len = 0;
  int32_t pool = PA_POOL_DEVICE;
  uint64_t stamp = 0;   // last batch call that listed it (duplicate check)
};

}  // namespace

struct pa_block_manager {
  pa_block_manager(int32_t nd, int32_t nh, int32_t bs, int32_t mb)
      : pools{Pool(nd), Pool(nh)}, block_size(bs), max_blocks(mb) {}
  Pool pools[2];
  int32_t block_size;
  int32_t max_blocks;
  std::unordered_map<int64_t, Seq> seqs;
  uint64_t stamp = 0;
  std::unordered_map<int32_t, int32_t> scratch;   // per-call block -> count / mapping
  std::vector<Seq*> batch;                          // per-call sequences, in list order

  Seq* find(int64_t id) {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
  const Seq* find(int64_t id) const {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
  int32_t blocks_for(int64_t tokens) const {
    return (int32_t)((tokens + block_size - 1) / block_size);
  }
};

namespace {

using pa::fail;
using pa::succeed;

// Checks shared by the batch calls: every id known, in `pool`, listed once.
// Leaves the sequences in bm->batch (map values do not move on insertion).
int check_batch(pa_block_manager* bm, const int64_t* seqs, int32_t n, int32_t pool) {
  if (n < 0) return fail(PA_ERR_INVALID_ARG, "n=%d < 0", n);
  if (n > 0 && !seqs) return fail(PA_ERR_INVALID_ARG, "null sequence list");
  const uint64_t stamp = ++bm->stamp;
  bm->batch.clear();
  for (int32_t i = 0; i < n; ++i) {
    Seq* s = bm->find(seqs[i]);
    if (!s) return fail(PA_ERR_INVALID_ARG, "unknown sequence %lld", (long long)seqs[i]);
    if (s->pool != pool)
      return fail(PA_ERR_INVALID_ARG, "sequence %lld is in the %s pool", (long long)seqs[i],
                  s->pool == PA_POOL_DEVICE ? "device" : "host");
    if (s->stamp == stamp)
      return fail(PA_ERR_INVALID_ARG, "sequence %lld listed twice", (long long)seqs[i]);
    s->stamp = stamp;
    bm->batch.push_back(s);
  }
  return PA_OK;
}

int swap(pa_block_manager* bm, const int64_t* seqs, int32_t n, int32_t from, int32_t to,
         int32_t* src_blocks, int32_t* dst_blocks, int32_t capacity, int32_t* num_pairs) {
  if (!num_pairs) return fail(PA_ERR_INVALID_ARG, "null num_pairs");
  int st = check_batch(bm, seqs, n, from);
  if (st != PA_OK) return st;
  // Distinct source blocks, in order of first appearance.
  auto& first = bm->scratch;
  first.clear();
  int32_t distinct = 0;
  for (Seq* s : bm->batch)
    for (int32_t b : s->table)
      if (first.emplace(b, distinct).second) ++distinct;
  if (distinct > capacity || (distinct > 0 && (!src_blocks || !dst_blocks)))
    return fail(PA_ERR_INVALID_ARG, "pair arrays hold %d entries, %d needed", capacity, distinct);
  Pool& src = bm->pools[from];
  Pool& dst = bm->pools[to];
  if (distinct > dst.free.size())
    return fail(PA_ERR_NO_ROOM, "no room: %d blocks to move, %d free in the %s pool", distinct,
                dst.free.size(), to == PA_POOL_DEVICE ? "device" : "host");
  // Map each distinct block once; count the references that move.
  std::vector<int32_t> moved((size_t)distinct, 0);
  for (int32_t k = 0; k < distinct; ++k) dst_blocks[k] = -1;
  for (Seq* s : bm->batch) {
    for (int32_t& b : s->table) {
      const int32_t k = first[b];
      if (dst_blocks[k] < 0) {
        src_blocks[k] = b;
        dst_blocks[k] = dst.take();
      } else {
        ++dst.ref[(size_t)dst_blocks[k]];
      }
      ++moved[(size_t)k];
      b = dst_blocks[k];
    }
    s->pool = to;
  }
  for (int32_t k = 0; k < distinct; ++k)
    for (int32_t r = 0; r < moved[(size_t)k]; ++r) src.release(src_blocks[k]);
  *num_pairs = distinct;
  return succeed();
}

int pool_arg(const pa_block_manager* bm, int32_t pool) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "null manager");
  if (pool != PA_POOL_DEVICE && pool != PA_POOL_HOST)
    return fail(PA_ERR_INVALID_ARG, "pool=%d is neither device nor host", pool);
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_bm_create(int32_t num_device_blocks, int32_t num_host_blocks, int32_t block_size,
                 int32_t max_blocks_per_seq, const int32_t* device_free_order,
                 pa_block_manager** out) {
  if (!out) return fail(PA_ERR_INVALID_ARG, "null output pointer");
  *out = nullptr;
  if (num_device_blocks <= 0 || num_host_blocks < 0 || block_size <= 0 || max_blocks_per_seq <= 0)
    return fail(PA_ERR_INVALID_ARG,
                "bad sizes (num_device_blocks=%d num_host_blocks=%d block_size=%d "
                "max_blocks_per_seq=%d)",
                num_device_blocks, num_host_blocks, block_size, max_blocks_per_seq);
  if ((int64_t)num_device_blocks * block_size > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "device slots exceed the int32 slot range");
  pa_block_manager* bm =
      new (std::nothrow) pa_block_manager(num_device_blocks, num_host_blocks, block_size,
                                          max_blocks_per_seq);
  if (!bm) return fail(PA_ERR_INVALID_ARG, "out of host memory");
  Pool& dev = bm->pools[PA_POOL_DEVICE];
  if (device_free_order) {
    std::vector<char> seen((size_t)num_device_blocks, 0);
    for (int32_t i = 0; i < num_device_blocks; ++i) {
      const int32_t b = device_free_order[i];
      if (b < 0 || b >= num_device_blocks || seen[(size_t)b]) {
        delete bm;
        return fail(PA_ERR_INVALID_ARG, "device_free_order is not a permutation (entry %d = %d)",
                    i, b);
      }
      seen[(size_t)b] = 1;
      dev.free.push(b);
    }
  } else {
    for (int32_t b = 0; b < num_device_blocks; ++b) dev.free.push(b);
  }
  for (int32_t b = 0; b < num_host_blocks; ++b) bm->pools[PA_POOL_HOST].free.push(b);
  *out = bm;
  return succeed();
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int pa_bm_add(pa_block_manager* bm, int64_t seq, int32_t num_tokens, int32_t* slots) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "null manager");
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens=%d < 0", num_tokens);
  if (bm->find(seq)) return fail(PA_ERR_INVALID_ARG, "sequence %lld exists", (long long)seq);
  const int32_t nb = bm->blocks_for(num_tokens);
  Pool& dev = bm->pools[PA_POOL_DEVICE];
  if (nb > bm->max_blocks)
    return fail(PA_ERR_NO_ROOM, "no room: %d tokens need %d blocks, max_blocks_per_seq is %d",
                num_tokens, nb, bm->max_blocks);
  if (nb > dev.free.size())
    return fail(PA_ERR_NO_ROOM, "no room: %d blocks needed, %d free", nb, dev.free.size());
  Seq s;
  s.table.reserve((size_t)nb);
  for (int32_t j = 0; j < nb; ++j) s.table.push_back(dev.take());
  s.len = num_tokens;
  if (slots)
    for (int32_t p = 0; p < num_tokens; ++p)
      slots[p] = s.table[(size_t)(p / bm->block_size)] * bm->block_size + p % bm->block_size;
  bm->seqs.emplace(seq, std::move(s));
  return succeed();
}

int pa_bm_append(pa_block_manager* bm, const int64_t* seqs, int32_t n, int32_t* slots,
                 int32_t* cow_src, int32_t* cow_dst, int32_t* num_cow) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "null manager");
  if (!num_cow || (n > 0 && (!slots || !cow_src || !cow_dst)))
    return fail(PA_ERR_INVALID_ARG, "null output array");
  int st = check_batch(bm, seqs, n, PA_POOL_DEVICE);
  if (st != PA_OK) return st;
  Pool& dev = bm->pools[PA_POOL_DEVICE];
  const int32_t bs = bm->block_size;
  // Dry run: blocks needed, counting the references that earlier entries of
  // this batch drop from a shared last block (its last holder writes in place).
  auto& dropped = bm->scratch;
  if (!dropped.empty()) dropped.clear();
  int32_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = bm->batch[(size_t)i];
    const int32_t j = s->len / bs;
    if (s->len % bs == 0) {
      if (j >= bm->max_blocks)
        return fail(PA_ERR_NO_ROOM, "no room: sequence %lld is at max_blocks_per_seq=%d",
                    (long long)seqs[i], bm->max_blocks);
      ++need;
    } else {
      const int32_t last = s->table[(size_t)j];
      auto it = dropped.find(last);
      const int32_t gone = it == dropped.end() ? 0 : it->second;
      if (dev.ref[(size_t)last] - gone > 1) {
        ++need;
        ++dropped[last];
      }
    }
  }
  if (need > dev.free.size())
    return fail(PA_ERR_NO_ROOM, "no room: %d blocks needed, %d free", need, dev.free.size());
  int32_t ncow = 0;
  for (int32_t i = 0; i < n; ++i) {
    Seq* s = bm->batch[(size_t)i];
    const int32_t j = s->len / bs, o = s->len % bs;
    if (o == 0) {
      s->table.push_back(dev.take());
    } else {
      const int32_t last = s->table[(size_t)j];
      if (dev.ref[(size_t)last] > 1) {
        const int32_t fresh = dev.take();
        --dev.ref[(size_t)last];
        s->table[(size_t)j] = fresh;
        cow_src[ncow] = last;
        cow_dst[ncow] = fresh;
        ++ncow;
      }
    }
    slots[i] = s->table[(size_t)j] * bs + o;
    ++s->len;
  }
  *num_cow = ncow;
  return succeed();
}

int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "null manager");
  const Seq* p = bm->find(parent);
  if (!p) return fail(PA_ERR_INVALID_ARG, "unknown sequence %lld", (long long)parent);
  if (bm->find(child)) return fail(PA_ERR_INVALID_ARG, "sequence %lld exists", (long long)child);
  Seq c;
  c.table = p->table;
  c.len = p->len;
  c.pool = p->pool;
  Pool& pool = bm->pools[c.pool];
  for (int32_t b : c.table) ++pool.ref[(size_t)b];
  bm->seqs.emplace(child, std::move(c));
  return succeed();
}

int pa_bm_free(pa_block_manager* bm, int64_t seq) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "null manager");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return fail(PA_ERR_INVALID_ARG, "unknown sequence %lld", (long long)seq);
  Pool& pool = bm->pools[it->second.pool];
  for (int32_t b : it->second.table) pool.release(b);
  bm->seqs.erase(it);
  return succeed();
}

int pa_bm_swap_out(pa_block_manager* bm, const int64_t* seqs, int32_t n, int32_t* src_blocks,
                   int32_t* dst_blocks, int32_t capacity, int32_t* num_pairs) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "null manager");
  return swap(bm, seqs, n, PA_POOL_DEVICE, PA_POOL_HOST, src_blocks, dst_blocks, capacity,
              num_pairs);
}

int pa_bm_swap_in(pa_block_manager* bm, const int64_t* seqs, int32_t n, int32_t* src_blocks,
                  int32_t* dst_blocks, int32_t capacity, int32_t* num_pairs) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "null manager");
  return swap(bm, seqs, n, PA_POOL_HOST, PA_POOL_DEVICE, src_blocks, dst_blocks, capacity,
              num_pairs);
}

int pa_bm_block_tables(const pa_block_manager* bm, const int64_t* seqs, int32_t n,
                       int32_t* tables, int32_t stride, int32_t* context_lens) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "null manager");
  if (n < 0 || stride <= 0) return fail(PA_ERR_INVALID_ARG, "n=%d stride=%d", n, stride);
  if (n > 0 && (!seqs || !tables || !context_lens))
    return fail(PA_ERR_INVALID_ARG, "null array");
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = bm->find(seqs[i]);
    if (!s) return fail(PA_ERR_INVALID_ARG, "unknown sequence %lld", (long long)seqs[i]);
    if (s->pool != PA_POOL_DEVICE)
      return fail(PA_ERR_INVALID_ARG, "sequence %lld is swapped out", (long long)seqs[i]);
    if ((int32_t)s->table.size() > stride)
      return fail(PA_ERR_INVALID_ARG, "sequence %lld holds %zu blocks > stride %d",
                  (long long)seqs[i], s->table.size(), stride);
  }
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = bm->find(seqs[i]);
    int32_t* row = tables + (size_t)i * stride;
    const size_t nb = s->table.size();
    if (nb) std::memcpy(row, s->table.data(), nb * sizeof(int32_t));
    for (size_t j = nb; j < (size_t)stride; ++j) row[j] = -1;
    context_lens[i] = s->len;
  }
  return succeed();
}

int pa_bm_prefix_groups(const pa_block_manager* bm, const int64_t* seqs, int32_t n,
                        int32_t* group_starts, int32_t* prefix_blocks, int32_t* num_groups) {
  if (!bm || !num_groups || n < 0 || !group_starts || (n > 0 && (!seqs || !prefix_blocks)))
    return fail(PA_ERR_INVALID_ARG, "null pointer or n=%d < 0", n);
  std::vector<const Seq*> list((size_t)n);
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = bm->find(seqs[i]);
    if (!s) return fail(PA_ERR_INVALID_ARG, "unknown sequence %lld", (long long)seqs[i]);
    if (s->pool != PA_POOL_DEVICE)
      return fail(PA_ERR_INVALID_ARG, "sequence %lld is swapped out", (long long)seqs[i]);
    list[(size_t)i] = s;
  }
  const int32_t bs = bm->block_size;
  auto whole = [&](const Seq* s) {
    const int32_t w = s->len / bs;
    return w < (int32_t)s->table.size() ? w : (int32_t)s->table.size();
  };
  int32_t g = 0;
  group_starts[0] = 0;
  for (int32_t i = 0; i < n;) {
    const Seq* a = list[(size_t)i];
    int32_t p = whole(a);
    int32_t e = i + 1;
    while (p > 0 && e < n && whole(list[(size_t)e]) > 0 &&
           list[(size_t)e]->table[0] == a->table[0])
      ++e;
    for (int32_t k = i + 1; k < e; ++k) {
      const Seq* b = list[(size_t)k];
      const int32_t lim = p < whole(b) ? p : whole(b);
      int32_t j = 0;
      while (j < lim && b->table[(size_t)j] == a->table[(size_t)j]) ++j;
      p = j;
    }
    prefix_blocks[g] = e - i > 1 ? p : 0;
    group_starts[++g] = e;
    i = e;
  }
  *num_groups = g;
  return succeed();
}

int pa_bm_sequence(const pa_block_manager* bm, int64_t seq, int32_t* table, int32_t* length,
                   int32_t* num_blocks, int32_t* pool) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "null manager");
  const Seq* s = bm->find(seq);
  if (!s) return fail(PA_ERR_INVALID_ARG, "unknown sequence %lld", (long long)seq);
  if (table && !s->table.empty())
    std::memcpy(table, s->table.data(), s->table.size() * sizeof(int32_t));
  if (length) *length = s->len;
  if (num_blocks) *num_blocks = (int32_t)s->table.size();
  if (pool) *pool = s->pool;
  return succeed();
}

int pa_bm_num_free(const pa_block_manager* bm, int32_t pool, int32_t* n) {
  int st = pool_arg(bm, pool);
  if (st != PA_OK) return st;
  if (!n) return fail(PA_ERR_INVALID_ARG, "null output pointer");
  *n = bm->pools[pool].free.size();
  return succeed();
}

int pa_bm_refcounts(const pa_block_manager* bm, int32_t pool, int32_t* counts) {
  int st = pool_arg(bm, pool);
  if (st != PA_OK) return st;
  const Pool& p = bm->pools[pool];
  if (!counts && p.size() > 0) return fail(PA_ERR_INVALID_ARG, "null output pointer");
  if (p.size() > 0) std::memcpy(counts, p.ref.data(), (size_t)p.size() * sizeof(int32_t));
  return succeed();
}

int pa_bm_free_list(const pa_block_manager* bm, int32_t pool, int32_t* blocks, int32_t* n) {
  int st = pool_arg(bm, pool);
  if (st != PA_OK) return st;
  const Pool& p = bm->pools[pool];
  if (!n || (!blocks && p.free.size() > 0)) return fail(PA_ERR_INVALID_ARG, "null output pointer");
  for (int32_t i = 0; i < p.free.size(); ++i) blocks[i] = p.free.at(i);
  *n = p.free.size();
  return succeed();
}

int pa_bm_stats(const pa_block_manager* bm, pa_bm_usage* out) {
  if (!bm || !out) return fail(PA_ERR_INVALID_ARG, "null pointer");
  pa_bm_usage r{};
  r.num_seqs = (int32_t)bm->seqs.size();
  const Pool& dev = bm->pools[PA_POOL_DEVICE];
  const Pool& host = bm->pools[PA_POOL_HOST];
  r.device_blocks_used = dev.size() - dev.free.size();
  r.host_blocks_used = host.size() - host.free.size();
  for (int32_t c : dev.ref) r.device_blocks_shared += c > 1;
  // Positions stored in a block are the same for all its holders (a shared
  // block is never written: copy-on-write), so each block counts once.
  std::vector<char> counted((size_t)dev.size(), 0);
  const int32_t bs = bm->block_size;
  for (const auto& kv : bm->seqs) {
    const Seq& s = kv.second;
    if (s.pool != PA_POOL_DEVICE) continue;
    r.device_tokens_logical += s.len;
    for (size_t j = 0; j < s.table.size(); ++j) {
      const int32_t b = s.table[j];
      if (counted[(size_t)b]) continue;
      counted[(size_t)b] = 1;
      const int64_t fill = (int64_t)s.len - (int64_t)j * bs;
      r.device_tokens_stored += fill < bs ? fill : bs;
    }
  }
  *out = r;
  return succeed();
}

}  // extern "C"
