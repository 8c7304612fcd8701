// Decode attention straight over the paged KV pool (gfx950 / CDNA4).
//
// "PagedAttention and KV memory management", section "The kernel side":
// the kernel reads the sequence's block table, loads each physical block's
// K and V tiles in turn, and computes scores and weighted values without
// first gathering the KV into one buffer.
//
// Work items.  A sequence's context is cut into partitions of part_blocks
// logical blocks; one work item is (sequence s, KV head h, partition p).
// The partition size is chosen per call from the batch's lengths (or given
// by the caller); for a given batch every reduction order depends only on
// logical positions, so results are bitwise reproducible and independent of
// where blocks sit in the pool.
//
// Up to three launches on the caller's stream:
//   plan_items    one workgroup (sharing its launch with the slot write when
//                 a whole step is issued).  Picks the partition size and
//                 lists the non-empty (s, p) pairs in the workspace -- every
//                 full partition first (sequence order), then the partial
//                 last partitions in decreasing size -- plus the sequences
//                 whose partition states must be merged, and, with shared
//                 prefixes, each group's shared blocks and the prefix items.
//                 Not launched for a decode of at most 64 sequences without
//                 shared prefixes: the matrix-core kernel then computes the
//                 same plan itself (lane_plan).
//   decode_*      persistent: as many workgroups as fit on the chip at once,
//                 dealt the first round of the list and claiming the rest
//                 from per-pool counters (the vector-ALU kernel and the
//                 self-planning kernel deal every round in snake order), so
//                 no workgroup is launched for an empty partition and the
//                 workgroups end close together however ragged the context
//                 lengths are.
//   merge_splits  log-sum-exp merge of the partition states of every
//                 sequence listed by the planner: per-head maxima and sums
//                 first, then the weighted sum of the partitions' vectors.
//
// Inside an item, the wave in lane j of the W lanes takes the item's 16-token
// positions j, j + W, ... (whole blocks at block size 16, half blocks at 32;
// the vector-ALU kernel takes whole blocks) and keeps a running softmax state
// (max m, sum l, weighted sum acc) per query head of the group; the W states
// are merged through LDS in lane order.  A sequence with one partition writes
// `out` directly; otherwise the item stores its partition state in the
// workspace for merge_splits.
//
// Matrix-core kernel, bf16 KV.  For each 16-token sub-block:
//   S^T[16 tokens x 16 heads] = K[16 x D] * Q^T[D x 16]      (v_mfma_f32_16x16x32_bf16)
//   O^T[16 d x 16 heads]     += V^T[16 d x 16] * P^T[16 x 16] (v_mfma_f32_16x16x16_bf16)
// The G query heads of a KV group fill the 16-wide head dimension (padded
// with zero queries), so each loaded K/V tile serves all G heads.  Lane l
// holds scores of tokens 4*(l/16)+r (r < 4) for head l%16, which is exactly
// the B operand layout the PV product needs, so P never leaves registers.
// K rows are loaded straight into the A operand (16 bytes per lane per
// instruction); V is stored feature-major in 16-token sub-tiles ([D, 16] per
// 16 tokens of a block), so each lane loads 4 consecutive tokens of one
// feature (8 bytes) for the PV A operand and every 16-token position reads
// one contiguous 4 KB span of K and one of V (D = 128, bf16).
// P enters the PV product as two bf16 operands, hi = bf16(P) and lo =
// bf16(P - hi) (see split_weight), so the weights keep about 16 bits; the
// softmax denominator sums the same hi + lo.
//
// fp32 KV runs the same matrix-core kernel with fp32 products
// (v_mfma_f32_16x16x4_f32; see TileF32).
//
// Vector-ALU kernel (either dtype, on request): the same items and merge;
// scores by lanes over tokens, weighted values by lanes over features.
//
// Shared prefixes (pa_decode_shared_prefix): the matrix-core kernel first
// runs prefix items that read each shared block once for up to 32 query
// rows (see prefix_items), then the sequences' own blocks as above.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdlib>
#include <type_traits>
#include <map>
#include <mutex>
#include <tuple>

#include "pa_internal.h"
#include "pa_write_body.h"

namespace pa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kMaxGroup = 16;   // query heads per KV head the kernels handle
constexpr int kWaves = 4;       // waves per decode workgroup
constexpr int kTailClasses = 256;
constexpr int kMaxLdsSlots = 2;    // LDS state slots of the matrix-core kernel (power of 2)
constexpr int kMaxLdsRecords = 16; // LDS output records of the matrix-core kernel
constexpr int kSpinLimit = 1 << 22; // polls (~0.1 s) before an LDS wait is declared broken
constexpr int kLateStop = 2;        // items of a claim pool left to the first workgroups
constexpr int kPoolShift = 1;       // workgroup b claims from pool (b >> kPoolShift) % kClaimPools
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs; the sign bit rides
// along, so negative values round by magnitude too).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Softmax weights enter the PV matrix product as bf16 operands.  A weight p
// in [0, 1] is split into hi = bf16(p) and lo = bf16(p - hi): p - hi is exact
// in fp32 (hi is within 2^-8 of p, relatively), so hi + lo carries p to about
// 2^-16 relative instead of the 2^-9 of hi alone, at the price of a second
// PV product per sub-block (the kernel is bound by HBM, not by the matrix
// cores).  The softmax denominator sums hi + lo, the weights the two products
// apply together (`sum`).
struct SplitWeight {
  short hi, lo;
  float sum;
};

__device__ __forceinline__ SplitWeight split_weight(float p) {
  const uint32_t h = f32_to_bf16_bits(p);
  const float ph = bf16_bits_to_f32(h);
  const uint32_t l = f32_to_bf16_bits(p - ph);
  return SplitWeight{(short)h, (short)l, ph + bf16_bits_to_f32(l)};
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Max / sum of a value over the four 16-lane rows of a wave (lanes l, l^16,
// l^32, l^48), with the gfx950 row-swap instructions instead of a shuffle
// through LDS (which waits for the LDS path twice).  permlane16_swap(x, x)
// returns the pair {x[l], x[l^16]} in some order in every lane (checked on
// the device: lane l < 16 gets {x[l], x[l+16]}, lane 16 <= l < 32 gets
// {x[l-16], x[l]}, likewise for rows 2 and 3); permlane32_swap the same for
// l^32.  Addition is commutative, so the sums are bitwise those of the
// shuffles.
__device__ __forceinline__ float rows_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t v = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float rows_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t v = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <typename T>
__device__ __forceinline__ float widen(T x);
template <>
__device__ __forceinline__ float widen<float>(float x) { return x; }
template <>
__device__ __forceinline__ float widen<uint16_t>(uint16_t x) { return bf16_bits_to_f32(x); }

__device__ __forceinline__ int clamp_len(const DecodeParams& a, int s, int block_size) {
  const int L = a.lens[s];
  const int Lmax = a.max_blocks * block_size;
  return L < 0 ? 0 : (L > Lmax ? Lmax : L);
}

// ---------------------------------------------------------------------------
// Work list.
// ---------------------------------------------------------------------------

// Cross-lane steps of the planners, through DPP: the operand of an ALU
// instruction is read from another lane of the wave, with no trip through
// LDS.  (ds_bpermute, which the generic shuffles use, goes through the LDS
// pipeline, and the planners' 4 to 16 waves queue on it.)  Controls (GFX9):
// row_shr:n, lane i of a 16-lane row reads lane i - n of the row; row_ror:n,
// lane i reads lane (i - n) mod 16 of the row; wave_shr:1 / wave_shl:1, lane
// i reads lane i - 1 / i + 1; row_bcast:15, every lane of a row reads lane 15
// of the row before; row_bcast:31, every lane reads lane 31.  A lane whose
// source is outside its range, or whose row is left out by ROWS, gets `id`.
constexpr int kDppRowShr = 0x110;     // + n, 1 <= n <= 15
constexpr int kDppRowRor = 0x120;     // + n, 1 <= n <= 15
constexpr int kDppWaveShl1 = 0x130;
constexpr int kDppWaveShr1 = 0x138;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ int dpp_read(int id, int v) {
  return __builtin_amdgcn_update_dpp(id, v, CTRL, ROWS, 0xf, false);
}

// Inclusive scan over the 64 lanes with an associative, commutative `op`
// whose identity is `id`: doubling shifts inside each row, then row 0's total
// into row 1 and row 2's into row 3, then rows 0-1's total into rows 2-3.
template <typename Op>
__device__ __forceinline__ int wave_scan(int v, int id, Op op) {
  v = op(v, dpp_read<kDppRowShr + 1>(id, v));
  v = op(v, dpp_read<kDppRowShr + 2>(id, v));
  v = op(v, dpp_read<kDppRowShr + 4>(id, v));
  v = op(v, dpp_read<kDppRowShr + 8>(id, v));
  v = op(v, dpp_read<kDppRowBcast15, 0xa>(id, v));
  v = op(v, dpp_read<kDppRowBcast31, 0xc>(id, v));
  return v;
}

struct AddOp {
  __device__ int operator()(int a, int b) const { return a + b; }
};
struct MaxOp {
  __device__ int operator()(int a, int b) const { return max(a, b); }
};

__device__ __forceinline__ int wave_scan_sum(int v) { return wave_scan(v, 0, AddOp()); }
__device__ __forceinline__ int wave_scan_max(int v) { return wave_scan(v, INT_MIN, MaxOp()); }

// Float sum and maximum over a wave, every lane gets the result (the order
// of the additions is fixed, so the result is reproducible).
struct AddFOp {
  __device__ int operator()(int a, int b) const {
    return __float_as_int(__int_as_float(a) + __int_as_float(b));
  }
};
struct MaxFOp {
  __device__ int operator()(int a, int b) const {
    return __float_as_int(fmaxf(__int_as_float(a), __int_as_float(b)));
  }
};
__device__ __forceinline__ float wave_sum_f(float v) {
  return __int_as_float(
      __builtin_amdgcn_readlane(wave_scan(__float_as_int(v), 0, AddFOp()), 63));
}
__device__ __forceinline__ float wave_max_f(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(
      wave_scan(__float_as_int(v), __float_as_int(-__builtin_inff()), MaxFOp()), 63));
}

// Sum over a wave (every lane gets it).
__device__ __forceinline__ int wave_sum(int v) {
  return __builtin_amdgcn_readlane(wave_scan_sum(v), 63);
}

// `op` over each run of NW lanes (NW a power of two, at most 16) of a value
// that repeats every NW lanes; every lane gets the result.  Rotations inside
// a row: after the step by n, each lane holds op over 2n consecutive lanes.
template <int NW, typename Op>
__device__ __forceinline__ int lanes_reduce(int v, Op op) {
  static_assert(NW >= 1 && NW <= 16 && (NW & (NW - 1)) == 0, "lanes_reduce width");
  if constexpr (NW >= 2) v = op(v, dpp_read<kDppRowRor + 1>(0, v));
  if constexpr (NW >= 4) v = op(v, dpp_read<kDppRowRor + 2>(0, v));
  if constexpr (NW >= 8) v = op(v, dpp_read<kDppRowRor + 4>(0, v));
  if constexpr (NW >= 16) v = op(v, dpp_read<kDppRowRor + 8>(0, v));
  return v;
}

// Sum over each run of NW lanes of a wave (the value repeats every NW lanes).
template <int NW>
__device__ __forceinline__ int lanes_sum(int v) {
  return lanes_reduce<NW>(v, AddOp());
}

// Inclusive minimum over segments of adjacent lanes with equal `key` (no key
// may recur after another one); the segment's last lane holds its minimum.
// The scan of wave_scan, each step taken only from a lane of the segment:
// with segments contiguous, a source lane with the same key has only lanes
// of the segment between it and this lane.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ int segment_step(int v, int key) {
  const int sv = dpp_read<CTRL, ROWS>(INT_MAX, v);
  const int sk = dpp_read<CTRL, ROWS>(INT_MIN, key);
  return sk == key ? min(v, sv) : v;
}

__device__ __forceinline__ int segment_min(int v, int key) {
  v = segment_step<kDppRowShr + 1>(v, key);
  v = segment_step<kDppRowShr + 2>(v, key);
  v = segment_step<kDppRowShr + 4>(v, key);
  v = segment_step<kDppRowShr + 8>(v, key);
  v = segment_step<kDppRowBcast15, 0xa>(v, key);
  v = segment_step<kDppRowBcast31, 0xc>(v, key);
  return v;
}

constexpr int kPartChoices = 8;
constexpr int kLensCached = 8192;   // context lengths the planner keeps in LDS
constexpr int kDirectItems = 4;     // full partitions a planner thread lists itself

// Partition size: the largest pb = part_blocks_min * 2^k (<= part_blocks_max)
// whose partitions are each at most 1/balance of one workgroup's share of
// `work` blocks over `grid` workgroups (balance 0: always the smallest).
__device__ __forceinline__ int choose_part_blocks(const DecodeParams& a, int64_t work,
                                                  int64_t grid, int balance) {
  int pb = a.part_blocks_min;
  if (balance > 0) {
    const int64_t share = work * a.num_kv_heads / ((grid > 0 ? grid : 1) * balance);
    for (int k = 0; k < kPartChoices && (int64_t)pb * 2 <= share && pb * 2 <= a.part_blocks_max;
         ++k)
      pb *= 2;
  }
  return pb;
}

// The plan of a batch of at most 64 sequences without shared prefixes, in
// one wave's registers: lane s holds sequence s.  The work list is the full
// partitions in sequence order (an empty sequence gets one item that zeroes
// its output), then the partial last partitions by decreasing size, ties by
// sequence.  It is plan_body's list (same partition size, same items, same
// split sequences) except for the order of the partial partitions and of
// the split list, neither of which changes a result.
struct LanePlan {
  int L, nblk;       // this lane's sequence: context (clamped), blocks
  int nfull, incl;   // its full partitions; those of sequences 0 .. s
  int rank;          // position of its partial partition among them
  bool tail;         // it has a partial last partition
  int pb;            // partition size in blocks (uniform)
  int n_full, n_tail;
};

// `len`: context_lens[lane] as read (lanes past the batch: anything).
template <int BS>
__device__ __forceinline__ LanePlan lane_plan(const DecodeParams& a, int len) {
  LanePlan q;
  const int lane = threadIdx.x & 63;
  const bool live = lane < a.num_seqs;
  const int Lmax = a.max_blocks * BS;
  q.L = live ? (len < 0 ? 0 : (len > Lmax ? Lmax : len)) : 0;
  q.nblk = (q.L + BS - 1) / BS;
  q.pb = choose_part_blocks(a, wave_sum(q.nblk), a.decode_grid, a.balance);
  q.nfull = live ? (q.nblk == 0 ? 1 : q.nblk / q.pb) : 0;
  q.incl = wave_scan_sum(q.nfull);
  q.n_full = __builtin_amdgcn_readlane(q.incl, 63);
  // A lane's rank: the lanes with a larger remainder, found bit by bit from
  // the top (`same`: the lanes whose remainder has agreed with this lane's so
  // far; at a bit where this lane has 0, those with 1 are larger), then the
  // earlier lanes with the same remainder.
  const int rem = q.nblk % q.pb;
  q.tail = live && rem != 0;
  uint64_t same = __builtin_amdgcn_ballot_w64(q.tail);
  q.n_tail = __builtin_popcountll(same);
  q.rank = 0;
  for (int b = 31 - __builtin_clz(q.pb); b >= 0; --b) {   // rem < pb
    const uint64_t ones = __builtin_amdgcn_ballot_w64((rem >> b) & 1);
    if ((rem >> b) & 1) {
      same &= ones;
    } else {
      q.rank += __builtin_popcountll(same & ones);
      same &= ~ones;
    }
  }
  q.rank += __builtin_popcountll(same & ((1ull << lane) - 1));
  return q;
}

// The split list of a lane plan and its counts (what merge_splits reads):
// sequences spanning several partitions, up to kMergeShort partitions from
// the front of the list, longer ones from the back.
__device__ __forceinline__ void write_split_list(const DecodeParams& a, const LanePlan& q) {
  const int lane = threadIdx.x & 63;
  const bool live = lane < a.num_seqs;
  const int nparts = (q.nblk + q.pb - 1) / q.pb;
  const uint64_t below = (1ull << lane) - 1;
  const uint64_t short_split = __builtin_amdgcn_ballot_w64(live && nparts > 1 && nparts <= kMergeShort);
  const uint64_t long_split = __builtin_amdgcn_ballot_w64(live && nparts > kMergeShort);
  if (live && nparts > 1) {
    const int at = nparts <= kMergeShort ? __builtin_popcountll(short_split & below)
                                         : a.num_seqs - 1 - __builtin_popcountll(long_split & below);
    a.ws_split[at] = make_int2(lane, nparts);
  }
  if (lane == 0) {
    a.ws_ctrl[kCtrlSplits] = __builtin_popcountll(short_split);
    a.ws_ctrl[kCtrlLongSplits] = __builtin_popcountll(long_split);
  }
}

// The planner of such a batch, in one wave with no barrier: the lane plan
// written out as the work list.
template <int BS>
__device__ __forceinline__ void plan_small(const DecodeParams& a) {
  const int lane = threadIdx.x & 63;
  const LanePlan q = lane_plan<BS>(a, lane < a.num_seqs ? a.lens[lane] : 0);
  const int pbp = choose_part_blocks(a, 0, a.decode_grid / 2, 0);
  // A sequence's first kDirectItems full partitions are listed by its lane,
  // any further ones by all lanes together.
  const int base = q.incl - q.nfull;
  for (int p = 0; p < min(q.nfull, kDirectItems); ++p)
    a.ws_items[base + p] = make_int4(lane, p, q.L, 0);
  for (uint64_t longs = __builtin_amdgcn_ballot_w64(q.nfull > kDirectItems); longs;
       longs &= longs - 1) {
    const int j = __builtin_ctzll(longs);
    const int nj = __builtin_amdgcn_readlane(q.nfull, j);
    const int bj = __builtin_amdgcn_readlane(base, j);
    const int Lj = __builtin_amdgcn_readlane(q.L, j);
    for (int p = kDirectItems + lane; p < nj; p += 64) a.ws_items[bj + p] = make_int4(j, p, Lj, 0);
  }
  if (q.tail) a.ws_items[q.n_full + q.rank] = make_int4(lane, q.nblk / q.pb, q.L, 0);
  write_split_list(a, q);
  if (lane == 0) {
    a.ws_ctrl[kCtrlEntries] = q.n_full + q.n_tail;
    a.ws_ctrl[kCtrlPartBlocks] = q.pb;
    a.ws_ctrl[kCtrlPrefixItems] = 0;
    a.ws_ctrl[kCtrlPrefixPart] = pbp;
    a.ws_ctrl[kCtrlAbort] = 0;
  }
  if (lane < kClaimPools) a.ws_ctrl[kCtrlClaims + lane * kClaimStride] = 0;
}

// Whether plan_small plans this batch.
__host__ __device__ __forceinline__ bool small_plan(const DecodeParams& a) {
  return a.num_seqs <= 64 && a.num_groups == 0;
}


// Maximum over each run of NW lanes of a wave (the value repeats every NW lanes).
template <int NW>
__device__ __forceinline__ int lanes_max(int v) {
  return lanes_reduce<NW>(v, MaxOp());
}

// Block-wide sums of four values at once (one pair of barriers).
template <int NT>
__device__ __forceinline__ int4 block_sum4(int4 v, int4* scratch) {
  constexpr int NW = NT / 64;
  v = make_int4(wave_sum(v.x), wave_sum(v.y), wave_sum(v.z), wave_sum(v.w));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
  __syncthreads();
  const int4 u = scratch[threadIdx.x & (NW - 1)];
  return make_int4(lanes_sum<NW>(u.x), lanes_sum<NW>(u.y), lanes_sum<NW>(u.z), lanes_sum<NW>(u.w));
}

// NT threads (256 or 1024: at least kTailClasses).  GROUPS: the batch may
// come with shared-prefix groups (only then is LDS kept for them).
template <int NT, bool GROUPS>
__device__ __forceinline__ void plan_body(const DecodeParams& a, int block_size) {
  static_assert(NT >= kTailClasses && NT % 64 == 0 && NT <= 1024, "planner width");
  constexpr int NW = NT / 64;
  // Sequences one thread handles in the group stage: all S <= kLensCached of
  // a batch with groups for 1024 threads; 256 threads plan batches of at
  // most 256 sequences.
  constexpr int kPer = NT == 1024 ? kLensCached / NT : 1;
  __shared__ int lens_c[kLensCached];
  __shared__ int cls_off[kTailClasses];
  __shared__ int wave_part[16];
  __shared__ int chunk_incl[NT];
  __shared__ int long_seen;
  __shared__ int run_base;
  __shared__ int nsplit;
  __shared__ int nsplit_long;
  __shared__ int npitems;
  __shared__ int pitems_end;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = a.num_seqs;
  // With groups, S <= kLensCached (checked on the host).
  const bool groups = GROUPS && a.num_groups > 0 && S <= NT * kPer;

  for (int i = tid; i < kTailClasses; i += NT) cls_off[i] = 0;
  if (tid == 0) {
    run_base = 0;
    long_seen = 0;
    nsplit = 0;
    nsplit_long = 0;
    npitems = 0;
    pitems_end = INT_MAX;
  }
  // Group g's bounds and prefix hint, read by thread g (for the first NT
  // groups) together with the lengths, in one memory round trip.
  int reg_lo = 0, reg_hi = 0, reg_pb = 0;
  if (groups && tid < a.num_groups) {
    reg_lo = a.group_starts[tid];
    reg_hi = a.group_starts[tid + 1];
    reg_pb = a.prefix_blocks[tid];
  }
  // One pass over the context lengths (clamped), kept in LDS for the passes
  // below.  S * max_blocks fits in int32 (checked on the host).
  for (int s = tid; s < S; s += NT)
    if (s < kLensCached) lens_c[s] = clamp_len(a, s, block_size);
  auto len_of = [&](int s) { return s < kLensCached ? lens_c[s] : clamp_len(a, s, block_size); };

  // Shared prefixes, one thread per sequence.  A group's prefix is the run of
  // whole blocks that its table entries share and that lies inside every
  // member's context; it is read once per `per_item` sequences.  A group of
  // one shares nothing.  Groups are consecutive runs of sequences, so a
  // sequence's group is the one whose first member is the nearest group
  // start at or before it (a running maximum over the sequences), unless a
  // group-less stretch starts in between.  The groups must be ordered
  // (group_starts non-decreasing), so that no two overlap: a sequence then
  // belongs to one group at most and the prefix work list fits its
  // S * num_parts_max entries.  Otherwise the groups are ignored and the
  // batch is decoded plainly (the same result).
  int* start_c = nullptr;     // per sequence: its shared blocks
  int16_t* bound_c = nullptr; // per sequence: 2 * s + 1 if a group of two or more starts
                              //  at s, 2 * s if a group of one or a group-less run does,
                              //  else -1; later, at a group's start: its end
  int* gmin_c = nullptr;      // at a group's start: min(hint * block_size, member contexts)
  if constexpr (GROUPS) {
    __shared__ int start_s[kLensCached];
    __shared__ int16_t bound_s[kLensCached];
    start_c = start_s;
    bound_c = bound_s;
    gmin_c = start_s;         // start_c is written only after the minima are read
  }
  const int per_item = groups ? (a.prefix_rows / a.group > 0 ? a.prefix_rows / a.group : 1) : 1;
  auto group_at = [&](int g, int& lo_raw, int& hi_raw, int& hint) {
    lo_raw = g < NT ? reg_lo : a.group_starts[g];
    hi_raw = g < NT ? reg_hi : a.group_starts[g + 1];
    hint = g < NT ? reg_pb : a.prefix_blocks[g];
  };
  // Own sequences of the group stage: the contiguous run s0 .. s0 + per - 1.
  const int per = (S + NT - 1) / NT;
  const int s0 = tid * per;
  int head[kPer], pshared[kPer];   // own sequence s0 + j: group start (-1: none), shared blocks
  int bad = 0, pre_mine = 0, mine_pre = 0, mine = 0;
  if (groups) {
    for (int s = tid; s < S; s += NT) bound_c[s] = -1;
    __syncthreads();
    for (int g = tid; g < a.num_groups; g += NT) {
      int lo_raw, hi_raw, hint;
      group_at(g, lo_raw, hi_raw, hint);
      bad |= hi_raw < lo_raw;
      const int lo = max(lo_raw, 0), hi = min(hi_raw, S);
      if (lo < hi) {
        bound_c[lo] = (int16_t)(2 * lo + (hi - lo >= 2));
        if (hi - lo >= 2) gmin_c[lo] = min(max(hint, 0), a.max_blocks) * block_size;
      }
      if (g == a.num_groups - 1 && hi >= 0 && hi < S) bound_c[hi] = (int16_t)(2 * hi);
    }
    __syncthreads();
    // The nearest marker at or before each sequence: a running maximum over
    // the thread's own run, then over the runs of the threads before it.
    int key[kPer];
    int run = -1;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (j < per && s0 + j < S) run = max(run, (int)bound_c[s0 + j]);
      key[j] = run;
    }
    const int incl = wave_scan_max(run);
    __shared__ int wave_max[16];
    if (lane == 63) wave_max[wave] = incl;
    const int up = dpp_read<kDppWaveShr1>(-1, incl);   // lanes before this one
    __syncthreads();
    const int wm = wave_max[lane & (NW - 1)];
    const int before = max(up, lanes_max<NW>((lane & (NW - 1)) < wave ? wm : -1));
    // Shortest context of each group.  The thread folds each run of one
    // group among its sequences and sends all but its last run to LDS; the
    // last runs are folded across the wave first (lanes whose last run is
    // one group's are adjacent: group starts do not decrease along the
    // sequences) and sent by the segment's last lane, so a group of 1024
    // sequences takes 16 LDS atomics on one address, not 1024.
    int cur = -1, cmin = INT_MAX;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int s = s0 + j;
      const int k = max(key[j], before);
      const bool mine_s = j < per && s < S;
      head[j] = mine_s && k >= 0 && (k & 1) ? k >> 1 : -1;
      pshared[j] = 0;
      if (mine_s && head[j] != cur) {
        if (cur >= 0) atomicMin(&gmin_c[cur], cmin);
        cur = head[j];
        cmin = INT_MAX;
      }
      if (head[j] >= 0) cmin = min(cmin, len_of(s));
    }
    cmin = segment_min(cmin, cur);
    const int next = dpp_read<kDppWaveShl1>(-2, cur);
    if (cur >= 0 && next != cur) atomicMin(&gmin_c[cur], cmin);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int s = s0 + j;
      if (j >= per || s >= S) continue;
      const int nblk = (len_of(s) + block_size - 1) / block_size;
      pshared[j] = head[j] >= 0 ? gmin_c[head[j]] / block_size : 0;
      mine_pre += nblk - pshared[j];
      if (pshared[j] > 0 && (s - head[j]) % per_item == 0) pre_mine += pshared[j];
    }
    // Each group's end at its start, for the prefix work list (the markers
    // are no longer read).
    for (int g = tid; g < a.num_groups; g += NT) {
      int lo_raw, hi_raw, hint;
      group_at(g, lo_raw, hi_raw, hint);
      const int lo = max(lo_raw, 0), hi = min(hi_raw, S);
      if (hi - lo >= 2) bound_c[lo] = (int16_t)hi;
    }
  }
  for (int s = tid; s < S; s += NT) mine += (len_of(s) + block_size - 1) / block_size;
  __shared__ int4 sum4[16];
  const int4 sums = block_sum4<NT>(make_int4(bad, pre_mine, mine_pre, mine), sum4);
  const bool prefix = groups && sums.x == 0;
  const int64_t pre_total = prefix ? sums.y : 0;
  const int64_t total = prefix ? sums.z : sums.w;
  if (groups) {
    // After the sums' barriers: every minimum has been read.
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (j < per && s0 + j < S) start_c[s0 + j] = prefix ? pshared[j] : 0;
    __syncthreads();
  }
  // Shared blocks of sequence s.
  auto start_of = [&](int s) { return prefix ? start_c[s] : 0; };

  // Partition size (choose_part_blocks).  Long partitions mean few partition
  // states to merge; short ones spread a long context over many workgroups.
  // Prefix partitions are
  // sized from the prefix work alone, for about one prefix item per CU (half
  // the resident workgroups): the CU's other workgroup streams own blocks
  // meanwhile.  Measured on the parallel-sampling workload (16 prompts of 128
  // blocks, 8 KV heads, 512 workgroups): 64-block prefix partitions 68 us per
  // call, 32 blocks 74 us, 128 blocks 78 us.
  const int pb = choose_part_blocks(a, total, a.decode_grid, a.balance);
  const int pbp = choose_part_blocks(a, pre_total, a.decode_grid / 2, a.balance > 0 ? 1 : 0);
  if (tid == 0) {
    a.ws_ctrl[kCtrlPartBlocks] = pb;
    a.ws_ctrl[kCtrlPrefixPart] = pbp;
    a.ws_ctrl[kCtrlAbort] = 0;
  }
  if (tid < kClaimPools) a.ws_ctrl[kCtrlClaims + tid * kClaimStride] = 0;

  // Partial last partition of a sequence's own blocks: size class, larger
  // partitions in lower classes.  -1 if there is no partial partition.
  auto tail_class = [&](int nblk) {
    const int rem = nblk % pb;
    if (rem == 0) return -1;
    return pb < (1 << 23) ? (pb - rem) * (kTailClasses - 1) / pb
                          : (int)((int64_t)(pb - rem) * (kTailClasses - 1) / pb);
  };

  // Pass 1: full partitions in sequence order (an empty sequence gets one
  // item that zeroes its output); count partial partitions per class; list
  // the sequences whose states are merged: those spanning several partitions
  // and all that have a shared prefix (prefix partitions come first).
  for (int c0 = 0; c0 < S; c0 += NT) {
    const int s = c0 + tid;
    int nfull = 0, L = 0, P = 0;
    if (s < S) {
      L = len_of(s);
      P = start_of(s);
      const int nblk = (L + block_size - 1) / block_size - P;
      nfull = nblk == 0 ? (P == 0 ? 1 : 0) : nblk / pb;
      const int c = tail_class(nblk);
      if (c >= 0) atomicAdd(&cls_off[c], 1);
      const int nown = (nblk + pb - 1) / pb;
      const int npre = (P + pbp - 1) / pbp;
      if (npre + nown > 1 || npre > 0) {
        const int at = npre + nown <= kMergeShort ? atomicAdd(&nsplit, 1)
                                                  : S - 1 - atomicAdd(&nsplit_long, 1);
        a.ws_split[at] = make_int2(s, npre + nown);
      }
    }
    const int incl = wave_scan_sum(nfull);
    if (lane == 63) wave_part[wave] = incl;
    if (nfull > kDirectItems) long_seen = 1;
    __syncthreads();
    const int wsum = wave_part[lane & (NW - 1)];
    const int chunk = lanes_sum<NW>(wsum);
    const int before = lanes_sum<NW>((lane & (NW - 1)) < wave ? wsum : 0);
    // A sequence's first kDirectItems full partitions are listed by its own
    // thread.  Any further ones (long contexts) are listed by all threads,
    // each finding its sequence by binary search over the chunk's inclusive
    // counts: one thread listing a hundred partitions took microseconds.
    const int base = run_base + before + incl - nfull;
    for (int p = 0; p < min(nfull, kDirectItems); ++p) a.ws_items[base + p] = make_int4(s, p, L, P);
    chunk_incl[tid] = before + incl;
    __syncthreads();
    if (long_seen) {
      for (int i = tid; i < chunk; i += NT) {
        int lo = 0, hi = min(S - c0, NT) - 1;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (chunk_incl[mid] > i) hi = mid; else lo = mid + 1;
        }
        const int p = i - (lo > 0 ? chunk_incl[lo - 1] : 0);
        const int sq = c0 + lo;
        if (p >= kDirectItems)
          a.ws_items[run_base + i] = make_int4(sq, p, len_of(sq), start_of(sq));
      }
    }
    __syncthreads();
    if (tid == 0) {
      run_base += chunk;
      long_seen = 0;
    }
    __syncthreads();
  }

  // Class start offsets after the full partitions: exclusive scan of the
  // class counts by the first kTailClasses threads (4 waves).
  {
    const int n = tid < kTailClasses ? cls_off[tid] : 0;
    const int incl = wave_scan_sum(n);
    if (lane == 63 && wave < kTailClasses / 64) wave_part[wave] = incl;
    __syncthreads();
    if (tid < kTailClasses) {
      int before = run_base;
      for (int w = 0; w < wave; ++w) before += wave_part[w];
      cls_off[tid] = before + incl - n;
      if (tid == kTailClasses - 1) {
        a.ws_ctrl[kCtrlEntries] = before + incl;
        a.ws_ctrl[kCtrlSplits] = nsplit;
        a.ws_ctrl[kCtrlLongSplits] = nsplit_long;
      }
    }
    __syncthreads();
  }

  // Pass 2: partial partitions.  The order inside a class is arbitrary; it
  // changes which workgroup computes an item, never the result.
  for (int s = tid; s < S; s += NT) {
    const int L = len_of(s);
    const int P = start_of(s);
    const int nblk = (L + block_size - 1) / block_size - P;
    const int c = tail_class(nblk);
    if (c >= 0) a.ws_items[atomicAdd(&cls_off[c], 1)] = make_int4(s, nblk / pb, L, P);
  }

  // Prefix work list: (first sequence, sequences, partition, prefix blocks)
  // for every run of per_item sequences of a group and every partition of
  // its prefix, listed by the thread of the run's first sequence.  The order
  // is arbitrary (it never changes the result).  With ordered groups the
  // list holds at most sum over groups of members * ceil(P / pbp) <=
  // S * num_parts_max entries; the bound is checked anyway, so that no input
  // can make the planner write past the list.
  if (prefix) {
    const int64_t cap = (int64_t)S * a.num_parts_max;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int s = s0 + j;
      if (j >= per || s >= S || pshared[j] <= 0 || (s - head[j]) % per_item != 0) continue;
      const int P = pshared[j];
      const int n = min(per_item, (int)bound_c[head[j]] - s);
      const int np = (P + pbp - 1) / pbp;
      const int at = atomicAdd(&npitems, np);
      if ((int64_t)at + np > cap) {
        atomicMin(&pitems_end, at);
        continue;
      }
      for (int p = 0; p < np; ++p) a.ws_pitems[at + p] = make_int4(s, n, p, P);
    }
    __syncthreads();
    if (tid == 0) a.ws_ctrl[kCtrlPrefixItems] = min(npitems, pitems_end);
  } else if (tid == 0) {
    a.ws_ctrl[kCtrlPrefixItems] = 0;
  }
}

// The planner alone, or the planner in workgroup 0 and a slot write in the
// others (the step's write and plan are independent, so they share a launch).
// The block size is a template parameter so that the planner's divisions by
// it are shifts.
// NT threads: one wave for batches plan_small plans, 256 for up to 256
// sequences, else 1024 (chosen by launch_decode_shape).
template <int BS, int NT, bool GROUPS>
__global__ __launch_bounds__(NT) void plan_items(DecodeParams a) {
  if constexpr (NT == 64) {
    plan_small<BS>(a);
  } else {
    plan_body<NT, GROUPS>(a, BS);
  }
}

template <typename E, int BS>
__global__ __launch_bounds__(1024) void write_and_plan(DecodeParams a, WriteArgs w) {
  if (blockIdx.x == 0) {
    if (small_plan(a)) {
      if (threadIdx.x < 64) plan_small<BS>(a);
      return;
    }
    plan_body<1024, false>(a, BS);   // a step has no shared-prefix groups
    return;
  }
  write_elements<E>(w, (int64_t)(blockIdx.x - 1) * 1024 + threadIdx.x,
                    (int64_t)(gridDim.x - 1) * 1024);
}

struct Item {
  int s, h, part, L, nblk, b0, b1, nparts;
};

__device__ __forceinline__ Item make_item(int4 e, int h, int block_size, int pb) {
  Item it;
  it.s = e.x;
  it.part = e.y;
  it.h = h;
  it.L = e.z;
  it.nblk = (it.L + block_size - 1) / block_size;
  it.b0 = it.part * pb;
  it.b1 = min(it.b0 + pb, it.nblk);
  it.nparts = (it.nblk + pb - 1) / pb;
  return it;
}

// LDS area of the wave states of one item: m, l [W][kMaxGroup] and acc
// [W][group][D + 4] floats.  The vector-ALU kernel adds its own scratch
// after one such area; the matrix-core kernel keeps two (item parity).
template <int D, int W>
__host__ __device__ constexpr int lds_state_floats(int group) {
  return 2 * W * kMaxGroup + W * group * (D + 4);
}

// LDS output record of one merged item (floats): G*D values, (max, sum)
// per head, and a 4-int header (sequence, KV head, partition, split flag).
template <int D>
__host__ __device__ constexpr int lds_record_floats(int group) {
  return group * D + 2 * kMaxGroup + 4;
}

template <int D, int W>
struct Lds {
  float* m;
  float* l;
  float* acc;
  __device__ Lds(float* smem, int group)
      : m(smem), l(smem + W * kMaxGroup), acc(smem + 2 * W * kMaxGroup) {
    (void)group;
  }
};

// Zero output of a sequence with no tokens.
template <int D, int W>
__device__ __forceinline__ void zero_item(const DecodeParams& a, const Item& it) {
  const int G = a.group;
  for (int idx = threadIdx.x; idx < G * D; idx += 64 * W)
    a.out[((int64_t)it.s * a.num_heads + it.h * G) * D + idx] = 0.f;
}

// Merge the W wave states of this item (wave order), then either finish the
// sequence (one partition) or store the partition state for merge_splits().
template <int D, int W>
__device__ void finish_item(const DecodeParams& a, const Lds<D, W>& sm, const Item& it) {
  const int G = a.group;
  const bool split = it.nparts > 1;
  const int64_t prow = ((int64_t)it.s * a.num_kv_heads + it.h) * a.num_parts_max;
#pragma unroll 1
  for (int idx = threadIdx.x; idx < G * D; idx += 64 * W) {
    const int g = idx / D;
    const int d = idx - g * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, sm.m[w * kMaxGroup + g]);
    float lam = 0.f, val = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mw = sm.m[w * kMaxGroup + g];
      const float c = (mw == kNegInf) ? 0.f : exp2_fast(mw - M);
      lam += sm.l[w * kMaxGroup + g] * c;
      val += sm.acc[(w * G + g) * (D + 4) + d] * c;
    }
    if (!split) {
      a.out[((int64_t)it.s * a.num_heads + it.h * G + g) * D + d] = lam > 0.f ? val / lam : 0.f;
    } else {
      const int64_t row = (prow + it.part) * G + g;
      a.ws_acc[row * D + d] = val;
      if (d == 0) {
        a.ws_ml[row * 2 + 0] = M;
        a.ws_ml[row * 2 + 1] = lam;
      }
    }
  }
}

// Persistent item loop shared by both kernels.  The list (full partitions
// first, then partial ones in decreasing size) is dealt to the G resident
// workgroups in snake order -- round r gives item r*G + b to workgroup b
// when r is even and to workgroup G-1-b when r is odd -- which evens out the
// work per workgroup without any shared counter.  Once a workgroup's item
// is past the end, so are all its later ones.
template <int D, int W, typename Body>
__device__ __forceinline__ void run_items(const DecodeParams& a, int block_size, float* smem,
                                          Body body) {
  const int Hkv = a.num_kv_heads;
  const int total = a.ws_ctrl[kCtrlEntries] * Hkv;
  const int pb = a.ws_ctrl[kCtrlPartBlocks];
  const Lds<D, W> sm(smem, a.group);
  const int G = gridDim.x, b = blockIdx.x;
  for (int r = 0;; ++r) {
    const int item = r * G + ((r & 1) ? G - 1 - b : b);
    if (item >= total) break;
    const int e_idx = item / Hkv;
    const Item it = make_item(a.ws_items[e_idx], item - e_idx * Hkv, block_size, pb);
    if (it.nblk == 0) {
      zero_item<D, W>(a, it);
    } else {
      body(it, sm);              // leaves the wave states in LDS, then syncs
      finish_item<D, W>(a, sm, it);
    }
    __syncthreads();             // LDS is reused by the next item
  }
}

// ---------------------------------------------------------------------------
// Matrix-core kernel, bf16 KV.
// ---------------------------------------------------------------------------

template <int D, int BS>
struct Tile {
  static constexpr int SB = BS / 16;      // 16-token sub-blocks per block
  bf16x8 k[SB][D / 32];                   // QK A operand: token (l%16), 8 features
  i16x4 v[SB][D / 16];                    // PV A operand: feature (l%16), 4 tokens
};

// Buffer resource (gfx9 raw buffer: byte-addressed, stride 0) over `bytes`
// bytes at `base`.  Loads at an offset >= bytes return zero without touching
// memory, so a resource of 0 bytes reads as all zeros.
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
constexpr int kBufferFormatWord = 0x00020000;   // 32-bit data format, no swizzle
// Cache policy of the K/V tile loads: nontemporal.  Every tile is read once
// per call, so it is streamed past the caches instead of displacing lines
// that other waves still use (measured: the whole decode call 4% faster on
// the large-batch workload, bit-identical results).
constexpr int kStreamLoad = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes,
                                           kBufferFormatWord);
}

// Byte offsets of this lane inside a K tile, a V tile and a query group.
// Each load is a buffer load: scalar resource + this fixed vector offset +
// an immediate, so the stream needs no per-load vector address arithmetic.
struct LaneOff {
  uint32_t k, v, q;
};

template <int D, int BS>
__device__ __forceinline__ LaneOff lane_offsets(int lane, int group) {
  const uint32_t row = lane & 15, quad = lane >> 4;
  LaneOff o;
  o.k = (row * D + quad * 8) * 2;      // K row `row`, features 8*quad ..
  o.v = (row * 16 + quad * 4) * 2;     // V feature `row`, tokens 4*quad .. of a 16-token sub-tile
  // Query head `row` of the group; padding heads point past the group so
  // their loads return zeros.
  o.q = (int)row < group ? (row * D + quad * 8) * 2 : (uint32_t)group * D * 2;
  return o;
}

// One 16-token half of a K/V tile of BS tokens (half < BS / 16).  The K
// rows of the half and its feature-major V sub-tile ([D, 16]) are each one
// contiguous 16*D-element span, so a half reads whole cache lines whatever BS
// is (measured on the large-batch workload at block size 32: 208.8 us per
// call with V in 16-token sub-tiles, against 240.3 us with V feature-major
// over the whole 32-token block, where a half covers half of every line).
template <int D, int BS>
__device__ __forceinline__ void load_half(Tile<D, 16>& t, __amdgpu_buffer_rsrc_t kr,
                                          __amdgpu_buffer_rsrc_t vr, const LaneOff& o, int half) {
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
    t.k[0][c] = __builtin_bit_cast(
        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(kr, o.k + (half * 16 * D + c * 32) * 2, 0,
                                                      kStreamLoad));
#pragma unroll
  for (int i = 0; i < D / 16; ++i)
    t.v[0][i] = __builtin_bit_cast(
        i16x4, __builtin_amdgcn_raw_buffer_load_b64(vr, o.v + (half * 16 * D + i * 16 * 16) * 2,
                                                    0, kStreamLoad));
}

// fp32 KV on the matrix cores (v_mfma_f32_16x16x4_f32, fp32 products and
// sums), per 16-token position:
//   S^T[16 tokens x 16 heads] = sum over D/4 products of K[16 x 4] Q^T[4 x 16]
//   O^T[16 d x 16 heads]     += V^T[16 d x 4] P^T[4 x 16], 4 per 16 features
// Token t's K row is held by lanes t, t+16, t+32, t+48, lane quarter q with
// D/4 contiguous features from q*D/4 (four 16-byte loads per 64 features);
// the query the same way per head.  Product j takes feature q*D/4 + j in
// quarter q: a fixed permutation of the sum over features.  V is read as in
// the bf16 kernel, lane (feature d, quarter q) with tokens 4q .. 4q+3 of
// feature d, and PV product c pairs token 4q + c with its weight, which the
// score layout already puts in that lane, so P never leaves registers.
template <int D>
struct TileF32 {
  f32x4 k[D / 16];   // features (D/4)*quad + 4c .. +3 of token (lane % 16)
  f32x4 v[D / 16];   // tokens 4*quad .. +3 of feature 16i + (lane % 16)
};

template <int D>
__device__ __forceinline__ LaneOff lane_offsets_f32(int lane, int group) {
  const uint32_t row = lane & 15, quad = lane >> 4;
  LaneOff o;
  o.k = (row * D + quad * (D / 4)) * 4;
  o.v = (row * 16 + quad * 4) * 4;
  o.q = (int)row < group ? (row * D + quad * (D / 4)) * 4 : (uint32_t)group * D * 4;
  return o;
}

template <int D>
__device__ __forceinline__ void load_half_f32(TileF32<D>& t, __amdgpu_buffer_rsrc_t kr,
                                              __amdgpu_buffer_rsrc_t vr, const LaneOff& o,
                                              int half) {
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    t.k[c] = __builtin_bit_cast(
        f32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, o.k + half * 16 * D * 4 + c * 16, 0,
                                                     kStreamLoad));
#pragma unroll
  for (int i = 0; i < D / 16; ++i)
    t.v[i] = __builtin_bit_cast(
        f32x4, __builtin_amdgcn_raw_buffer_load_b128(vr, o.v + (half * 16 * D + i * 16 * 16) * 4,
                                                     0, kStreamLoad));
}

// Read-only views through the constant address space: uniform reads of
// them become scalar loads, which are counted apart from the vector loads
// that stream the K/V tiles, so waiting for a block id never drains the tile
// pipeline.
#define PA_CONST __attribute__((address_space(4)))

template <typename T>
__device__ __forceinline__ const PA_CONST T* as_const(const T* p) {
  return (const PA_CONST T*)(const void PA_CONST*)(uintptr_t)p;
}

// ---------------------------------------------------------------------------
// Shared-prefix kernel, bf16 KV.
// ---------------------------------------------------------------------------

// Query rows of one prefix item: two 16-column halves of the MFMA tiles.
constexpr int kPrefixRows = 32;

// LDS of the prefix kernel: per wave, (max, sum) and weighted sums of the 32 rows.
template <int D, int W>
__host__ __device__ constexpr int prefix_lds_floats() {
  return 2 * W * kPrefixRows + W * kPrefixRows * (D + 4);
}

// Parallel samples of one prompt ("How does vLLM PagedAttention manage
// Virtual Memory Pages ...", section "Key Technical Innovations", item 3)
// hold the prompt's blocks once; this kernel reads each of those K/V tiles
// once for all the sequences of a prefix item and all their query heads:
// up to 32 query rows (sequence-major, head-minor) in two 16-column halves,
//   S^T[16 tokens x 16 rows] = K[16 x D] * Q^T[D x 16]        per half
//   O^T[16 d x 16 rows]     += V^T[16 d x 16] * P^T[16 x 16]  per half
// so one tile feeds 32 rows' scores and weighted sums.  The streaming
// kernel runs these items first (item bid, bid + NG, ... of workgroup bid),
// then its own work list.  Work item = (prefix item, KV head); the W waves
// take the item's blocks b0 + w,
// b0 + w + W, ... with two tile buffers in flight, and their states are
// merged through LDS in wave order.  The result of each sequence's rows is
// stored as its partition state number `part` (prefix partitions precede
// the sequence's own partitions), for merge_splits.  Prefix blocks are whole
// and inside every member's context, so nothing is masked except blocks
// whose id is outside the pool (which then contribute nothing).
template <int D, int BS, int W>
__device__ __forceinline__ void prefix_items(const DecodeParams& a, float* smem, int bid, int NG) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, quad = lane >> 4;
  const int G = a.group, Hkv = a.num_kv_heads, Hq = a.num_heads;
  const PA_CONST int32_t* ctrl = as_const(a.ws_ctrl);
  const PA_CONST int32_t* pitems = as_const((const int32_t*)a.ws_pitems);
  const PA_CONST int32_t* tables = as_const(a.tables);
  const int total = ctrl[kCtrlPrefixItems] * Hkv;
  const int pbp = ctrl[kCtrlPrefixPart];
  float* sm_m = smem;
  float* sm_l = smem + W * kPrefixRows;
  float* sm_acc = smem + 2 * W * kPrefixRows;
  const uint32_t tile_bytes = (uint32_t)BS * D * 2;
  const LaneOff lo = lane_offsets<D, BS>(lane, G);
  const char* kbase = (const char*)a.k_cache;
  const char* vbase = (const char*)a.v_cache;

  for (int item = bid; item < total; item += NG) {
    const int e = item / Hkv;
    const int kv = item - e * Hkv;
    const int first = pitems[4 * e + 0], nseq = pitems[4 * e + 1];
    const int part = pitems[4 * e + 2], P = pitems[4 * e + 3];
    const int b0 = part * pbp, b1 = min(b0 + pbp, P);
    const int rows = nseq * G;

    // Query operands: row r = 16 * half + col is head r % G of sequence
    // first + r / G; rows past the item's sequences read zeros.
    bf16x8 qop[2][D / 32];
    {
      const uint32_t qbytes = (uint32_t)nseq * Hq * D * 2;
      const __amdgpu_buffer_rsrc_t qr =
          buffer_of((const char*)a.q + (int64_t)first * Hq * D * 2, qbytes);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int r = hh * 16 + col;
        const uint32_t off = r < rows ? ((uint32_t)((r / G) * Hq + kv * G + r % G) * D + quad * 8) * 2
                                      : qbytes;
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
          qop[hh][c] = __builtin_bit_cast(
              bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qr, off + c * 64, 0, 0));
      }
    }

    float m[2] = {kNegInf, kNegInf}, lsum[2] = {0.f, 0.f};
    f32x4 acc[2][D / 16];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < D / 16; ++i) acc[hh][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t trow = (int64_t)first * a.max_blocks;
    // Position k of the wave: 16-token half k % kHalves of its block
    // b0 + w + (k / kHalves) * W (of the first member's table).  Positions
    // past the item's blocks or with an id outside the pool read zeros.
    constexpr int kHalves = BS / 16;
    auto in_item = [&](int k) { return b0 + w + (k / kHalves) * W < b1; };
    auto load_pos = [&](Tile<D, 16>& t, int k, bool& has) {
      const int j = b0 + w + (k / kHalves) * W;
      int id = 0;
      if (j < b1) id = tables[trow + j];
      has = j < b1 && (unsigned)id < (unsigned)a.num_blocks;
      const int64_t off = has ? ((int64_t)id * Hkv + kv) * tile_bytes : 0;
      const uint32_t nb = has ? tile_bytes : 0;
      load_half<D, BS>(t, buffer_of(kbase + off, nb), buffer_of(vbase + off, nb), lo,
                       k % kHalves);
    };

    auto compute = [&](Tile<D, 16>& t, bool has) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        f32x4 sc[Tile<D, 16>::SB];
#pragma unroll
        for (int sb = 0; sb < Tile<D, 16>::SB; ++sb) {
          sc[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < D / 32; ++c)
            sc[sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t.k[sb][c], qop[hh][c], sc[sb], 0, 0, 0);
        }
        float mx = kNegInf;
#pragma unroll
        for (int sb = 0; sb < Tile<D, 16>::SB; ++sb)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const float x = has ? sc[sb][rr] * a.scale_log2 : kNegInf;
            sc[sb][rr] = x;
            mx = fmaxf(mx, x);
          }
        mx = rows_max(mx);
        const float mnew = fmaxf(m[hh], mx);
        const float mref = mnew == kNegInf ? 0.f : mnew;
        const float alpha = exp2_fast(m[hh] - mref);
        m[hh] = mnew;
        i16x4 pw[Tile<D, 16>::SB], pl[Tile<D, 16>::SB];
        float psum = 0.f;
#pragma unroll
        for (int sb = 0; sb < Tile<D, 16>::SB; ++sb)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const SplitWeight sw = split_weight(exp2_fast(sc[sb][rr] - mref));
            pw[sb][rr] = sw.hi;
            pl[sb][rr] = sw.lo;
            psum += sw.sum;
          }
        lsum[hh] = lsum[hh] * alpha + psum;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
          for (int i = 0; i < D / 16; ++i) acc[hh][i] *= alpha;
        }
#pragma unroll
        for (int i = 0; i < D / 16; ++i)
#pragma unroll
          for (int sb = 0; sb < Tile<D, 16>::SB; ++sb) {
            acc[hh][i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(t.v[sb][i], pw[sb], acc[hh][i],
                                                                   0, 0, 0);
            acc[hh][i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(t.v[sb][i], pl[sb], acc[hh][i],
                                                                   0, 0, 0);
          }
      }
    };

    // Two buffers: every step issues the loads of the next position, then
    // computes the current one.  (Three buffers, loading two positions ahead,
    // measured no faster here: 55.0 against 54.8 us per kernel on the
    // parallel-sampling workload.)
    Tile<D, 16> t0, t1;
    bool h0 = false, h1 = false;
    int k = 0;
    load_pos(t0, 0, h0);
    for (;;) {
      load_pos(t1, k + 1, h1);
      if (!in_item(k)) break;
      compute(t0, h0);
      ++k;
      load_pos(t0, k + 1, h0);
      if (!in_item(k)) break;
      compute(t1, h1);
      ++k;
    }

    // Wave state -> LDS (row r of half hh is column col).
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float ls = lsum[hh];
      ls = rows_sum(ls);
      const int r = hh * 16 + col;
      if (quad == 0) {
        sm_m[w * kPrefixRows + r] = m[hh];
        sm_l[w * kPrefixRows + r] = ls;
      }
#pragma unroll
      for (int i = 0; i < D / 16; ++i)
        *reinterpret_cast<f32x4*>(&sm_acc[(w * kPrefixRows + r) * (D + 4) + i * 16 + quad * 4]) =
            acc[hh][i];
    }
    __syncthreads();
    // Merge the W wave states in wave order and store each member's rows as
    // its partition state `part`.
    for (int idx = threadIdx.x; idx < rows * (D / 4); idx += 64 * W) {
      const int r = idx / (D / 4);
      const int d4 = idx - r * (D / 4);
      float M = kNegInf;
#pragma unroll
      for (int v = 0; v < W; ++v) M = fmaxf(M, sm_m[v * kPrefixRows + r]);
      float lam = 0.f;
      f32x4 val = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < W; ++v) {
        const float mv = sm_m[v * kPrefixRows + r];
        const float c = mv == kNegInf ? 0.f : exp2_fast(mv - M);
        lam += sm_l[v * kPrefixRows + r] * c;
        val += *reinterpret_cast<const f32x4*>(&sm_acc[(v * kPrefixRows + r) * (D + 4) + d4 * 4]) * c;
      }
      const int sq = first + r / G, g = r % G;
      const int64_t row = (((int64_t)sq * Hkv + kv) * a.num_parts_max + part) * G + g;
      *reinterpret_cast<f32x4*>(a.ws_acc + row * D + d4 * 4) = val;
      if (d4 == 0) {
        a.ws_ml[row * 2 + 0] = M;
        a.ws_ml[row * 2 + 1] = lam;
      }
    }
    __syncthreads();   // LDS is reused by the next item
  }
}

// One work item as a wave sees it (every field is uniform across the wave).
struct Desc {
  int s, h, L, b0, nparts, part;
  int base;         // packed-pool diagnostic: the sequence's first block id
  int wr;           // the wave's lane in the item: (w + round) mod W
  int nmine;        // the wave's 16-token positions in the item: wr, wr + W, ...
  int npos;         // positions the wave spends on the item: max(nmine, 1)
  bool valid;
};

// Persistent matrix-core kernel.  Each wave walks one stream of positions:
// item after item (dealt, then claimed; see item_for), one position per block it
// owns in the item, and one empty position in an item where it owns none.
// Every step issues the loads of the next position -- which may belong to
// the next item -- into one register buffer and computes the current
// position from the other, so the K/V stream keeps flowing across item
// boundaries.  Each step issues exactly the same loads (a position without a
// block reads block 0, computed fully masked), so the compiler can count
// them and wait only for the buffer it uses.  After the last position of an
// item each wave hands its state to the item's LDS slot; the last wave of
// the workgroup to do so merges them and writes the result (see finish).
// TABLE = false is a diagnostic instantiation for a pool packed sequence by
// sequence (block j of sequence s is block_tables[s, 0] + j): it reads one
// table entry per item instead of one per block, so comparing it with the
// ordinary kernel on the same packed pool isolates the cost of the per-block
// table reads from that of blocks scattered over the pool.
// PLAN = true (batches of at most 64 sequences without shared prefixes): no
// planner launch before this one.  Every wave computes the batch's lane plan
// (lane_plan) itself from the context lengths and finds an item's sequence
// and partition in it; every round is dealt (no claim counters, so nothing in
// the workspace has to be zeroed first); workgroup 0 writes the split list
// for merge_splits.  A wait that gives up is recorded in its own word, which
// merge_splits turns into the call's abort word.
// E: KV element, uint16_t (bf16 bits) or float.
template <typename E, int D, int BS, int W, bool PREFIX, bool TABLE, bool PLAN>
__device__ __forceinline__ void decode_mfma_body(const DecodeParams& a) {
  constexpr bool F32 = sizeof(E) == 4;
  static_assert(!(F32 && PREFIX), "shared prefixes run on bf16 KV only");
  using TileT = typename std::conditional<F32, TileF32<D>, Tile<D, 16>>::type;
  struct QB { bf16x8 v[D / 32]; };
  struct QF { f32x4 v[D / 16]; };
  using QT = typename std::conditional<F32, QF, QB>::type;
  extern __shared__ float smem[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane & 15, quad = lane >> 4;
  const int G = a.group;
  // A block of 32 tokens is streamed as two 16-token positions, so the
  // registers per position (and the occupancy) are those of 16-token blocks.
  constexpr int kHalves = BS / 16;
  const int Hkv = a.num_kv_heads;
  const int NG = gridDim.x, bid = blockIdx.x;

  const PA_CONST int32_t* ctrl = as_const(a.ws_ctrl);
  const PA_CONST int32_t* items = as_const((const int32_t*)a.ws_items);   // int4 entries
  const PA_CONST int32_t* tables = as_const(a.tables);
  LanePlan lp{};
  // Self-planning kernel: the block tables are pulled into the caches while
  // the plan is computed, so that an item's first block id is a cache hit
  // rather than one more HBM round trip after the lengths.  Each lane reads
  // one word of one table line (every wave, so no branch makes the wait for
  // the lengths also wait for this load); the workgroups of one XCD
  // (dispatched round-robin: workgroup b on XCD b % 8) cover every line of
  // the first 2 MB of tables.  The word is used only after the stream (an
  // empty asm statement), so no wait is added for it.
  int warm = 0;
  if constexpr (PLAN) {
    const int len = lane < a.num_seqs ? a.lens[lane] : 0;   // issued first: waited for first
    const int64_t lines = ((int64_t)a.num_seqs * a.max_blocks + 31) / 32;
    const int64_t per_xcd = (NG + 7 - (bid & 7)) >> 3;
    const int64_t line =
        min((int64_t)(bid >> 3) + (int64_t)(lane + 64 * w) * per_xcd, lines - 1);
    warm = a.tables[line * 32];
    lp = lane_plan<BS>(a, len);
  }
  const int total = PLAN ? (lp.n_full + lp.n_tail) * Hkv : ctrl[kCtrlEntries] * Hkv;
  const int pb = PLAN ? lp.pb : ctrl[kCtrlPartBlocks];
  const int pbp = PLAN ? 1 : ctrl[kCtrlPrefixPart];
  if constexpr (PLAN) {
    if (bid == 0 && w == 0) write_split_list(a, lp);
  }
  __shared__ int s_count[kMaxLdsSlots];   // waves that finished the slot's item
  __shared__ int s_epoch[kMaxLdsSlots];   // item the slot is free for

  // A wait that has not ended after kSpinLimit polls (tens of milliseconds;
  // a legitimate one lasts microseconds) means a broken invariant: record it
  // in the workspace and give up, so the kernel still ends.
  auto abort_wait = [&]() {
    if (lane == 0)
      __hip_atomic_store(&a.ws_ctrl[PLAN ? kCtrlAbortPlanned : kCtrlAbort],
                         PLAN ? kAbortMark : 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  // The workgroup's item for round r.  The list (longest items first) is
  // dealt, in snake order, for the first round only -- item b to workgroup
  // b -- and claimed after that: workgroup b takes the next unclaimed item of
  // pool x = (b / 2) % npools (items NG + x, NG + x + npools, ...) until the
  // pool is empty; npools = min(kClaimPools, NG / 2), so every pool has at
  // least two workgroups claiming from it.  The two workgroups sharing a CU stream at different
  // speeds (the first dispatched one gets most of the memory pipeline), and
  // so do CUs on more or less loaded memory paths; claiming lets the faster
  // ones take more of the list, so the workgroups end closer together.
  // Measured on the large-batch workload (512 workgroups, ~4.5 items each):
  // 209.3 us per call with every round dealt in snake order, 204.4 us with 8
  // pools, 199.7 us with 32 (contention on each counter falls), 200.5 us with
  // 64, 202.3 us with 128 (a pool's items are shared by fewer workgroups);
  // claiming the first round too, 201.5 us.  Workgroups are dispatched to
  // the 8 XCDs round-robin (b % 8), so pools x = b % 32 each lived on one XCD
  // and an XCD with slower memory paths still did an eighth of the list
  // (per-workgroup end times: XCD medians 184.5 to 194.0 us); with x =
  // (b / 2) % 32 each pool spans two XCDs: 201.9 vs 203.7 us on one host
  // (x = (b / 8) % 32, all eight XCDs per pool: 203.0 us).  On another host,
  // whose slow XCDs were 2 and 3 (a pair that shared pools under b / 2), all
  // eight XCDs per pool won by a little (188.2 vs 188.7 us, skewed long
  // context 33.6 vs 34.0 us) but plain decode of the parallel-sampling batch
  // lost 13% (158.8 vs 139.7 us): its samples reread their group's shared
  // blocks, and pools confined to two XCDs keep those rereads in one L2 more
  // often.  So two XCDs per pool.  Letting a
  // workgroup whose pool is empty claim from other pools cost more than it
  // saved (a scan of the pools' counters before a workgroup may end: large
  // batch +1 us, small batches +2 to +3 us).  The first wave to need round
  // r's item claims it (one device-scope atomic) and publishes it in LDS for
  // the other waves.  Who computes an item never changes its result.  With
  // fewer than two rounds of items every round is dealt in snake order
  // (round r gives item r*NG + b to workgroup b when r is even and to
  // workgroup NG-1-b when r is odd).
  auto item_of = [&](int r) -> int { return r * NG + ((r & 1) ? NG - 1 - bid : bid); };
  const bool claimed_rounds = !PLAN && total >= 2 * NG;
  // Pools in use: kClaimPools, or fewer on a small grid, so that every pool
  // has a claimer (pool x holds workgroups 2x and 2x + 1 among others).
  const int npools = min(kClaimPools, max(1, NG >> kPoolShift));
  __shared__ int s_claim_busy[4];   // last round whose claim was started
  __shared__ int s_claim_tag[4];    // last round whose claim is published
  __shared__ int s_claim_item[4];
  int32_t* const claims = a.ws_ctrl + kCtrlClaims;
  // One claim from pool y by lane 0, returned to the whole wave.
  auto claim_from = [&](int y) -> int {
    int it = total;
    if (lane == 0) {
      const int j = __hip_atomic_fetch_add(&claims[y * kClaimStride], 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      const int64_t cand = (int64_t)NG + y + (int64_t)j * npools;
      it = cand < total ? (int)cand : total;
    }
    return __builtin_amdgcn_readfirstlane(it);
  };
  auto item_for = [&](int r) -> int {
    if (r == 0 || !claimed_rounds) return item_of(r);
    const int slot = r & 3;
    int claimer = 0;
    if (lane == 0)
      claimer = __hip_atomic_fetch_max(&s_claim_busy[slot], r, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP) < r;
    if (__builtin_amdgcn_readfirstlane(claimer)) {
      const int x = (bid >> kPoolShift) % npools;
      // Pool x holds workgroups 2x and 2x + 1 (mod 2 * npools); its lowest,
      // 2x, is a first workgroup when 2x < num_cus.  Only then may the others
      // stop early: a pool without a first workgroup (fewer than 64 CUs, or an
      // unknown CU count) is emptied by whoever claims from it.
      if (a.num_cus > 0 && bid >= a.num_cus && (x << kPoolShift) < a.num_cus) {
        // A workgroup dispatched after its CU's first one streams slower
        // (timestamps: the last workgroups to end were all of these); it
        // leaves a pool's last kLateStop items to the first workgroups, which
        // claim until the pool is empty.  Kernel with kLateStop 0 / 2 / 4 / 8,
        // alternating builds on one host: skewed long context 33.9 / 33.8 /
        // 35.2 / 36.4 us (uniform items: stopping early idles half the
        // workgroups at the end), gqa 52.2 / 52.1 / 52.1 / 51.7 us, large
        // batch and parallel sampling unchanged.  (On another host kLateStop
        // 8 gave gqa 51.5 against 54.0 us; skewed-long was not measured.)
        int stop = 0;
        if (lane == 0) {
          const int64_t left = (int64_t)total - NG - x;
          const int64_t size = left > 0 ? (left + npools - 1) / npools : 0;
          const int j = __hip_atomic_load(&claims[x * kClaimStride], __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
          stop = size - j < kLateStop;
        }
        if (__builtin_amdgcn_readfirstlane(stop)) {
          if (lane == 0) {
            s_claim_item[slot] = total;
            __hip_atomic_store(&s_claim_tag[slot], r, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
          }
          return total;
        }
      }
      const int item = claim_from(x);
      if (lane == 0) {
        s_claim_item[slot] = item;
        __hip_atomic_store(&s_claim_tag[slot], r, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      return item;
    }
    int item = total;
    if (lane == 0) {
      bool published = true;
      for (int spin = 0; __hip_atomic_load(&s_claim_tag[slot], __ATOMIC_ACQUIRE,
                                           __HIP_MEMORY_SCOPE_WORKGROUP) != r; ++spin) {
        if (spin == kSpinLimit) {
          abort_wait();
          published = false;   // end this wave's stream
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (published) item = s_claim_item[slot];
    }
    return __builtin_amdgcn_readfirstlane(item);
  };

  auto desc = [&](int r) -> Desc {
    Desc d;
    const int item = item_for(r);
    d.valid = item < total;
    // The entry is read before `total` is known (its address does not depend
    // on it), so the first item's list entry and the control words arrive in
    // one memory round trip: round 0's item is the workgroup's index, below
    // the list's capacity.  Fields of an item past the end are not used.
    const int e_idx = min(item / Hkv, a.num_seqs * a.num_parts_max - 1);
    int e_s, e_part, e_L, e_P;
    if constexpr (PLAN) {
      // Entry e of the lane plan: full partition e - (first entry of s) of
      // the sequence s whose full partitions cover e, or the partial
      // partition of rank e - n_full.
      if (e_idx < lp.n_full) {
        e_s = __builtin_popcountll(
            __builtin_amdgcn_ballot_w64(lane < a.num_seqs && lp.incl <= e_idx));
        e_part = e_idx - (__builtin_amdgcn_readlane(lp.incl, e_s) -
                          __builtin_amdgcn_readlane(lp.nfull, e_s));
      } else {
        const uint64_t at = __builtin_amdgcn_ballot_w64(lp.tail && lp.rank == e_idx - lp.n_full);
        e_s = at ? __builtin_ctzll(at) : 0;
        e_part = __builtin_amdgcn_readlane(lp.nblk, e_s) / pb;
      }
      e_L = __builtin_amdgcn_readlane(lp.L, e_s);
      e_P = 0;
    } else {
      e_s = items[4 * e_idx + 0];
      e_part = items[4 * e_idx + 1];
      e_L = items[4 * e_idx + 2];
      e_P = items[4 * e_idx + 3];
    }
    d.s = d.valid ? e_s : 0;
    d.part = d.valid ? e_part : 0;
    d.L = d.valid ? e_L : 0;
    d.h = d.valid ? item - e_idx * Hkv : 0;
    // Blocks before P belong to the sequence's shared prefix, computed by
    // the prefix kernel as the first partition states of the sequence.
    const int P = d.valid ? e_P : 0;
    d.base = !TABLE && d.valid && d.L > 0 ? tables[(int64_t)d.s * a.max_blocks] : 0;
    const int nblk = (d.L + BS - 1) / BS;
    d.b0 = P + d.part * pb;
    const int nb = min(d.b0 + pb, nblk) - d.b0;
    const int npre = (P + pbp - 1) / pbp;
    d.nparts = npre + (nblk - P + pb - 1) / pb;
    d.part += npre;
    // Rotating the waves' lanes from item to item spreads the extra blocks of
    // items whose size is not a multiple of W evenly over the waves.
    d.wr = (w + r) & (W - 1);
    // Waves take the item's live 16-token positions (half blocks at block
    // size 32) in turn: position q = wr + k * W is half q % kHalves of block
    // b0 + q / kHalves.  Dealing whole 32-token blocks to the waves instead
    // made the block-size-32 kernel 1.1% slower (196.2 against 194.0 us on
    // the large-batch workload); at block size 16 the two are the same.
    const int nq = nb > 0 ? (min(d.L, (d.b0 + nb) * BS) - d.b0 * BS + 15) / 16 : 0;
    d.nmine = nq > d.wr ? (nq - d.wr + W - 1) / W : 0;
    d.npos = d.nmine > 0 ? d.nmine : 1;
    return d;
  };

  // Shared prefixes first: every wave of the workgroup takes part (the
  // items end with barriers), and the LDS they use is free again after.
  if constexpr (PREFIX) prefix_items<D, BS, W>(a, smem, bid, NG);
  if (bid >= total) return;          // no work for this workgroup at all
  if (threadIdx.x < kMaxLdsSlots) {
    s_count[threadIdx.x] = 0;
    s_epoch[threadIdx.x] = threadIdx.x;
  }
  if (threadIdx.x < 4) {
    s_claim_busy[threadIdx.x] = -1;
    s_claim_tag[threadIdx.x] = -1;
  }
  __syncthreads();
  Desc cur = desc(0);
  Desc nxt;               // the next round's item, read when first needed
  bool have_nxt = false;
  int r = 0;

  const char* kbase = (const char*)a.k_cache;
  const char* vbase = (const char*)a.v_cache;
  const char* qbase = (const char*)a.q;
  const uint32_t tile_bytes = (uint32_t)BS * D * sizeof(E);
  LaneOff lo;
  if constexpr (F32) lo = lane_offsets_f32<D>(lane, G);
  else lo = lane_offsets<D, BS>(lane, G);

  // Loads of one position into a buffer.  `has` says whether the position
  // holds a block of the wave; a block id outside the pool counts as none,
  // and a position without a block reads zeros (a 0-byte resource).  The
  // item's query is loaded once per item (load_q), not with every position:
  // reloading it (2 KB per wave and position, from the cache) made the whole
  // decode call 4.4% slower (219.5 against 209.8 us on the large-batch
  // workload), the extra cache traffic competing with the tile stream.
  auto load_pos = [&](TileT& t, const Desc& d, int k, bool& has) {
    const int q = d.wr + k * W;
    const int kk = q / kHalves, half = q - kk * kHalves;
    int id = 0;
    if constexpr (TABLE) {
      if (d.valid && k < d.nmine) id = tables[(int64_t)d.s * a.max_blocks + d.b0 + kk];
    } else {
      id = d.base + d.b0 + kk;
    }
    has = d.valid && k < d.nmine && (unsigned)id < (unsigned)a.num_blocks;
    const int64_t off = has ? ((int64_t)id * Hkv + d.h) * tile_bytes : 0;
    const uint32_t nb = has ? tile_bytes : 0;
    if constexpr (F32)
      load_half_f32<D>(t, buffer_of(kbase + off, nb), buffer_of(vbase + off, nb), lo, half);
    else
      load_half<D, BS>(t, buffer_of(kbase + off, nb), buffer_of(vbase + off, nb), lo, half);
  };
  auto load_q = [&](QT& q, const Desc& d) {
    const __amdgpu_buffer_rsrc_t qr = buffer_of(
        qbase + ((int64_t)(d.valid ? d.s : 0) * a.num_heads + d.h * G) * D * sizeof(E),
        d.valid ? (uint32_t)(G * D * sizeof(E)) : 0);
    if constexpr (F32) {
#pragma unroll
      for (int c = 0; c < D / 16; ++c)
        q.v[c] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(qr, lo.q + c * 16, 0, 0));
    } else {
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
        q.v[c] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qr, lo.q + c * 64, 0, 0));
    }
  };

  float m = kNegInf, lsum = 0.f;
  f32x4 acc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One position: scores, online-softmax update, weighted values.  Positions
  // >= live are masked; live <= 0 masks the whole block.
  auto compute = [&](TileT& t, const QT& q, int live) {
    f32x4 sc;
    if constexpr (F32) {
      // Four independent chains of products, added at the end (a single
      // chain of D/4 dependent products would serialise on its latency).
      f32x4 part[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) part[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / 16; ++c)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          part[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(t.k[c][u], q.v[c][u], part[u], 0, 0, 0);
      sc = (part[0] + part[1]) + (part[2] + part[3]);
    } else {
      sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t.k[0][c], q.v[c], sc, 0, 0, 0);
    }
    // Scale into base-2 units, mask dead positions (select, never multiply:
    // the tail of the last block may hold anything), block max per head.
    float mx = kNegInf;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float x = quad * 4 + rr < live ? sc[rr] * a.scale_log2 : kNegInf;
      sc[rr] = x;
      mx = fmaxf(mx, x);
    }
    mx = rows_max(mx);
    const float mnew = fmaxf(m, mx);
    // Exponent reference: the running max, or 0 while every position seen so
    // far is masked (then all weights, the rescale factor included, are 0).
    const float mref = mnew == kNegInf ? 0.f : mnew;
    const float alpha = exp2_fast(m - mref);       // 0 on the first live block
    m = mnew;
    // Rescale every time (alpha is exactly 1 while a head's running max holds,
    // and multiplying by 1 changes nothing): skipping it behind a wave-uniform
    // test made the compiler copy the 32 accumulator registers at every
    // position, which cost as much as the multiplies.  A partly dead block
    // has V of its dead positions zeroed (their weight is 0, but 0 * NaN is
    // NaN).
    float psum = 0.f;
    if constexpr (F32) {
      f32x4 p;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        p[rr] = exp2_fast(sc[rr] - mref);
        psum += p[rr];
      }
      lsum = lsum * alpha + psum;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) acc[i] *= alpha;
      if (live < 16) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const bool dead = quad * 4 + rr >= live;
#pragma unroll
          for (int i = 0; i < D / 16; ++i) t.v[i][rr] = dead ? 0.f : t.v[i][rr];
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int i = 0; i < D / 16; ++i)
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(t.v[i][c], p[c], acc[i], 0, 0, 0);
    } else {
      i16x4 pw, pl;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const SplitWeight sw = split_weight(exp2_fast(sc[rr] - mref));
        pw[rr] = sw.hi;
        pl[rr] = sw.lo;
        psum += sw.sum;
      }
      lsum = lsum * alpha + psum;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) acc[i] *= alpha;
      if (live < 16) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const bool dead = quad * 4 + rr >= live;
#pragma unroll
          for (int i = 0; i < D / 16; ++i) t.v[0][i][rr] = dead ? (short)0 : t.v[0][i][rr];
        }
      }
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(t.v[0][i], pw, acc[i], 0, 0, 0);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(t.v[0][i], pl, acc[i], 0, 0, 0);
      }
    }
  };

  // End of an item, without a barrier: the wave stores its state in the
  // item's LDS state slot and counts itself in; the last of the W waves to
  // arrive merges the W states (in wave order) into the item's LDS output
  // record, while the others go straight on with their next item.  Output
  // records reach global memory only when the record ring is full or the
  // workgroup's last item is merged: a global store makes the wave's next
  // wait for a K/V tile also wait for the store (the vector-memory counter
  // is in order), so stores are kept out of the stream.  Before reusing a
  // state slot a wave waits until the merge of the slot's previous item is
  // done; the slowest wave never waits (every slot it needs was freed by
  // merges of items all waves have passed), so the waits always end.
  const int state_floats = lds_state_floats<D, W>(G);
  const int rec_floats = lds_record_floats<D>(G);
  float* recs = smem + a.lds_slots * state_floats;
  auto finish = [&](const Desc& d, int r_item, bool wg_last) {
    const int slot = r_item & (a.lds_slots - 1);
    const Lds<D, W> sm(smem + slot * state_floats, G);
    for (int spin = 0; __hip_atomic_load(&s_epoch[slot], __ATOMIC_ACQUIRE,
                                         __HIP_MEMORY_SCOPE_WORKGROUP) != r_item; ++spin) {
      if (spin == kSpinLimit) {
        abort_wait();
        return;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    float ls = lsum;
    ls = rows_sum(ls);
    // State index = the wave's lane in the item, so the merge below adds the
    // partial states in an order fixed by logical positions.
    if (quad == 0) {
      sm.m[d.wr * kMaxGroup + g] = m;
      sm.l[d.wr * kMaxGroup + g] = ls;
    }
    if (g < G) {
#pragma unroll
      for (int i = 0; i < D / 16; ++i)
        *reinterpret_cast<f32x4*>(&sm.acc[(d.wr * G + g) * (D + 4) + i * 16 + quad * 4]) =
            acc[i];
    }
    int before = 0;
    if (lane == 0)
      before = __hip_atomic_fetch_add(&s_count[slot], 1, __ATOMIC_ACQ_REL,
                                      __HIP_MEMORY_SCOPE_WORKGROUP);
    before = __builtin_amdgcn_readfirstlane(before);
    if (before != W - 1) return;
    // Last wave: merge into the output record.  Lane (g, quad) handles
    // features i*16 + 4*quad .. +3 of head g.
    const int ri = r_item % a.lds_records;
    float* rec = recs + ri * rec_floats;
    const bool split = d.nparts > 1;
    if (g < G) {
      float M = kNegInf;
#pragma unroll
      for (int v = 0; v < W; ++v) M = fmaxf(M, sm.m[v * kMaxGroup + g]);
      float c[W];
      float lam = 0.f;
#pragma unroll
      for (int v = 0; v < W; ++v) {
        const float mv = sm.m[v * kMaxGroup + g];
        c[v] = (mv == kNegInf) ? 0.f : exp2_fast(mv - M);
        lam += sm.l[v * kMaxGroup + g] * c[v];
      }
      // A whole sequence: scale by 1/lambda (one division per head).
      const float inv = split ? 1.f : (lam > 0.f ? 1.f / lam : 0.f);
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        f32x4 val = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < W; ++v)
          val += *reinterpret_cast<const f32x4*>(&sm.acc[(v * G + g) * (D + 4) + i * 16 +
                                                         quad * 4]) * c[v];
        val *= inv;
        *reinterpret_cast<f32x4*>(&rec[g * D + i * 16 + quad * 4]) = val;
      }
      if (quad == 0) {
        rec[G * D + 2 * g] = M;
        rec[G * D + 2 * g + 1] = lam;
      }
    }
    if (lane == 0) {
      int* hdr = reinterpret_cast<int*>(rec + G * D + 2 * kMaxGroup);
      hdr[0] = d.s;
      hdr[1] = d.h;
      hdr[2] = d.part;
      hdr[3] = split;
      __hip_atomic_store(&s_count[slot], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      __hip_atomic_store(&s_epoch[slot], r_item + a.lds_slots, __ATOMIC_RELEASE,
                         __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    // Flush the records of items r_item - ri .. r_item when the ring is full
    // or this is the workgroup's last item.  Every earlier merge is complete:
    // its wave merged before it finished this item.
    if (ri != a.lds_records - 1 && !wg_last) return;
    for (int j = 0; j <= ri; ++j) {
      const float* rj = recs + j * rec_floats;
      const int* hdr = reinterpret_cast<const int*>(rj + G * D + 2 * kMaxGroup);
      const int s = hdr[0], h = hdr[1], part = hdr[2];
      const bool sp = hdr[3] != 0;
      const int64_t row0 = (((int64_t)s * Hkv + h) * a.num_parts_max + part) * G;
      float* dst = sp ? a.ws_acc + row0 * D : a.out + ((int64_t)s * a.num_heads + h * G) * D;
      for (int e = lane; e < G * D / 4; e += 64)
        *reinterpret_cast<f32x4*>(dst + e * 4) = *reinterpret_cast<const f32x4*>(rj + e * 4);
      if (sp && lane < 2 * G) a.ws_ml[row0 * 2 + lane] = rj[G * D + lane];
    }
  };

  // The stream.  Position (cur, k); its buffer was loaded one step earlier.
  TileT t0, t1;
  // The query of round r's item is in set r & 1: loaded with the item's first
  // position (one position ahead), used until the item ends.
  QT qa, qb;
  bool has0 = false, has1 = false;
  int k = 0;
  load_q(qa, cur);
  load_pos(t0, cur, 0, has0);

  // One step: load the next position into (tn, qn), compute (tc, qc).
  // Returns false when the stream has ended.
  auto step = [&](TileT& tc, bool hc, TileT& tn, bool& hn) -> bool {
    const bool last = k + 1 >= cur.npos;
    if (last && !have_nxt) {
      nxt = desc(r + 1);
      have_nxt = true;
    }
    if (last) {
      if (r & 1) load_q(qa, nxt);
      else load_q(qb, nxt);
    }
    load_pos(tn, last ? nxt : cur, last ? 0 : k + 1, hn);
    const int live =
        hc ? cur.L - cur.b0 * BS - (cur.wr + k * W) * 16 : 0;
    if (r & 1) compute(tc, qb, live);
    else compute(tc, qa, live);
    if (!last) {
      ++k;
      return true;
    }
    finish(cur, r, !nxt.valid);
    m = kNegInf;
    lsum = 0.f;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (!nxt.valid) return false;
    ++r;
    cur = nxt;
    have_nxt = false;
    k = 0;
    return true;
  };

  while (step(t0, has0, t1, has1) && step(t1, has1, t0, has0)) {
  }
  if constexpr (PLAN) asm volatile("" ::"v"(warm));
}

template <int D, int BS, int W, bool PREFIX, bool TABLE = true, bool PLAN = false>
__global__ __launch_bounds__(64 * W) void decode_mfma_bf16(DecodeParams a) {
  decode_mfma_body<uint16_t, D, BS, W, PREFIX, TABLE, PLAN>(a);
}

// fp32 KV: the same work list, stream and merge, with fp32 matrix-core
// products (no shared-prefix phase; no packed-pool diagnostic).
template <int D, int BS, int W, bool PLAN = false>
__global__ __launch_bounds__(64 * W) void decode_mfma_f32(DecodeParams a) {
  decode_mfma_body<float, D, BS, W, false, true, PLAN>(a);
}

// ---------------------------------------------------------------------------
// Vector-ALU kernel (fp32 KV; also bf16 when asked).
// ---------------------------------------------------------------------------

template <typename T, int D, int BS, int W>
__device__ __forceinline__ void valu_item(const DecodeParams& a, const Item& it,
                                          const Lds<D, W>& sm, float* smem) {
  constexpr int NC = 64 / BS;          // lanes per token in the score step
  constexpr int DC = D / NC;           // features per lane in the score step
  constexpr int DL = D / 64;           // features per lane in the weighted sum
  constexpr int VT = BS % 16 == 0 ? 16 : BS;  // tokens per feature-major V sub-tile
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.group;
  const int Hkv = a.num_kv_heads;
  const int tt = lane % BS, ch = lane / BS;

  float* sm_q = smem + 2 * W * kMaxGroup + W * G * (D + 4);   // [G][D]
  float* sm_p = sm_q + G * D;                                 // [W][kMaxGroup][BS]

  const T* qrow = (const T*)a.q + ((int64_t)it.s * a.num_heads + it.h * G) * D;
  for (int idx = threadIdx.x; idx < G * D; idx += 64 * W) sm_q[idx] = widen<T>(qrow[idx]);
  __syncthreads();

  float m[kMaxGroup], lpart[kMaxGroup], acc[kMaxGroup][DL];
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) {
    m[g] = kNegInf;
    lpart[g] = 0.f;
#pragma unroll
    for (int k = 0; k < DL; ++k) acc[g][k] = 0.f;
  }
  const int32_t* trow = a.tables + (int64_t)it.s * a.max_blocks;
  float* p_w = sm_p + w * kMaxGroup * BS;

  for (int j = it.b0 + w; j < it.b1; j += W) {
    const int id = trow[j];
    if ((unsigned)id >= (unsigned)a.num_blocks) continue;
    const int64_t tile = (int64_t)id * Hkv + it.h;
    const T* kt = (const T*)a.k_cache + tile * BS * D;
    const T* vt = (const T*)a.v_cache + tile * BS * D;
    const int valid = min(BS, it.L - j * BS);

    float dot[kMaxGroup];
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g) dot[g] = 0.f;
    const T* krow = kt + tt * D + ch * DC;
    for (int dd = 0; dd < DC; ++dd) {
      const float kv = widen<T>(krow[dd]);
#pragma unroll
      for (int g = 0; g < kMaxGroup; ++g)
        if (g < G) dot[g] += sm_q[g * D + ch * DC + dd] * kv;
    }
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g) {
      if (g >= G) continue;
      float x = dot[g];
#pragma unroll
      for (int off = BS; off < 64; off <<= 1) x += shfl_xor_f(x, off);
      x = tt < valid ? x * a.scale_log2 : kNegInf;
      float mx = x;
#pragma unroll
      for (int off = 1; off < BS; off <<= 1) mx = fmaxf(mx, shfl_xor_f(mx, off));
      const float mnew = fmaxf(m[g], mx);
      const float alpha = exp2_fast(m[g] - mnew);
      const float p = exp2_fast(x - mnew);
      m[g] = mnew;
      lpart[g] = lpart[g] * alpha + (ch == 0 ? p : 0.f);
      if (ch == 0) p_w[g * BS + tt] = p;
#pragma unroll
      for (int k = 0; k < DL; ++k) acc[g][k] *= alpha;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int t = 0; t < valid; ++t) {
#pragma unroll
      for (int k = 0; k < DL; ++k) {
        const float vv = widen<T>(vt[((t / VT) * D + lane + 64 * k) * VT + t % VT]);
#pragma unroll
        for (int g = 0; g < kMaxGroup; ++g)
          if (g < G) acc[g][k] += p_w[g * BS + t] * vv;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) {
    if (g >= G) continue;
    float l = lpart[g];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) l += shfl_xor_f(l, off);
    if (lane == 0) {
      sm.m[w * kMaxGroup + g] = m[g];
      sm.l[w * kMaxGroup + g] = l;
    }
#pragma unroll
    for (int k = 0; k < DL; ++k) sm.acc[(w * G + g) * (D + 4) + lane + 64 * k] = acc[g][k];
  }
  __syncthreads();
}

template <typename T, int D, int BS, int W>
__global__ __launch_bounds__(64 * W) void decode_valu(DecodeParams a) {
  extern __shared__ float smem[];
  run_items<D, W>(a, BS, smem, [&](const Item& it, const Lds<D, W>& sm) {
    valu_item<T, D, BS, W>(a, it, sm, smem);
  });
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the partition states of split sequences, in
// partition order: a running (M, lambda, value) absorbs partition p as
//   M' = max(M, m_p),  lambda' = lambda 2^(M - M') + l_p 2^(m_p - M'),
//   value' = value 2^(M - M') + acc_p 2^(m_p - M'),   out = value / lambda.
// The loads of a partition do not depend on the running state, so a batch of
// partitions is fetched at once.  One workgroup per (split sequence, KV
// head) at a time, four features per thread.
// ---------------------------------------------------------------------------

// Log-sum-exp merge of a split sequence's partition states (m_p, l_p, acc_p),
// per query head g:  M = max_p m_p,  lambda = sum_p l_p 2^(m_p - M),
// out = (sum_p acc_p 2^(m_p - M)) / lambda  (m in base-2 units).
// A unit is one (split sequence, KV head); a column is one (query head,
// 4 features) of it.  The planner lists sequences with at most kMergeShort
// partitions apart from longer ones.
//   Short units: one thread per column loads all of the unit's partitions at
//   once and merges them alone, with no barrier.  Unit u goes to workgroup
//   u % grid, row (u / grid) % R of its R = threads / C rows of C columns:
//   units spread over all workgroups before any takes a second one.
//   Long units: one workgroup per (unit, query head), the last workgroups
//   first, so the G heads of a long sequence's unit are merged by G
//   workgroups at once.  The head's M and lambda come from all threads over
//   thread-strided partitions; rows of threads take contiguous runs of
//   partitions of one column for the weighted sum, whose terms do not depend
//   on one another, and the rows' partial sums are added in row order.  A
//   row's first partitions (8, 16 or kMergeBatch, as many as its run needs)
//   are loaded before the reductions.
//   (One workgroup per unit, all heads together: the skewed long-context
//   workload's merge of a 128-partition sequence took 7.7 us per call.)
// Every order depends only on the partition count, so results are
// reproducible.
constexpr int kMergeWaves = 8;
constexpr int kMergeThreads = 64 * kMergeWaves;
constexpr int kMergeBatch = 32;
constexpr int kMergeGrid = 256;
static_assert(kMergeShort <= kMergeBatch, "a short unit's partitions are loaded in one batch");

typedef float merge_f4 __attribute__((__vector_size__(4 * sizeof(float))));

// One query head of a long unit (sequence s, KV head h, query head gq of the
// group, nparts partition states).  The head's maximum and sum come first
// (thread t takes partitions t, t + threads, ...); then rows of D/4 threads
// take contiguous runs of partitions of one column each, and the rows'
// partial sums are added in row order.  A row's first B partitions are
// loaded before the reductions: clamped addresses, so the compiler issues
// every load of the batch at once (guarded loads measured 1 us slower on a
// cold long unit), with B no larger than a row's run needs, since each
// clamped slot past the run is one more load instruction through the
// texture-address unit.
template <int D, int B>
__device__ __forceinline__ void merge_long_head(const DecodeParams& a, int s, int h, int gq,
                                                int nparts, float* head_max, float* head_sum,
                                                merge_f4* partial) {
  typedef merge_f4 f4;
  constexpr int kCols4 = D / 4;
  constexpr int kRowsH = kMergeThreads / kCols4;
  const int G = a.group, Hkv = a.num_kv_heads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rh = tid / kCols4, ch = tid - rh * kCols4;
  const float2* ml = reinterpret_cast<const float2*>(a.ws_ml);
  const int64_t prow = ((int64_t)s * Hkv + h) * a.num_parts_max;
  const int p_lo = (int)((int64_t)nparts * rh / kRowsH);
  const int p_hi = (int)((int64_t)nparts * (rh + 1) / kRowsH);
  // This row's first batch of weighted sums, in flight during the reductions.
  float mp[B];
  f4 ap[B];
#pragma unroll
  for (int j = 0; j < B; ++j) {
    const int64_t row = (prow + max(min(p_lo + j, p_hi - 1), 0)) * G + gq;
    mp[j] = p_lo + j < p_hi ? a.ws_ml[row * 2] : kNegInf;
    ap[j] = p_lo + j < p_hi ? *reinterpret_cast<const f4*>(a.ws_acc + row * D + ch * 4)
                            : f4{0.f, 0.f, 0.f, 0.f};
  }
  // The thread's first (m, l) pair stays in registers for the sum below
  // (no second read after the barrier); further ones (more partitions than
  // threads) are read again.
  const float2 first = tid < nparts ? ml[(prow + tid) * G + gq] : make_float2(kNegInf, 0.f);
  float m = first.x;
  for (int p = tid + kMergeThreads; p < nparts; p += kMergeThreads)
    m = fmaxf(m, ml[(prow + p) * G + gq].x);
  m = wave_max_f(m);
  if (lane == 0) head_max[wave] = m;
  __syncthreads();
  float M = kNegInf;
#pragma unroll
  for (int v = 0; v < kMergeWaves; ++v) M = fmaxf(M, head_max[v]);
  float l = 0.f;
  if (M != kNegInf) {
    if (first.x != kNegInf) l += first.y * exp2_fast(first.x - M);
    for (int p = tid + kMergeThreads; p < nparts; p += kMergeThreads) {
      const float2 v = ml[(prow + p) * G + gq];
      if (v.x != kNegInf) l += v.y * exp2_fast(v.x - M);
    }
  }
  l = wave_sum_f(l);
  if (lane == 0) head_sum[wave] = l;
  f4 val = {0.f, 0.f, 0.f, 0.f};
  if (M != kNegInf) {
#pragma unroll
    for (int j = 0; j < B; ++j)
      if (mp[j] != kNegInf) val += ap[j] * exp2_fast(mp[j] - M);
    for (int p0 = p_lo + B; p0 < p_hi; p0 += B) {
#pragma unroll
      for (int j = 0; j < B; ++j) {
        const int64_t row = (prow + min(p0 + j, p_hi - 1)) * G + gq;
        mp[j] = a.ws_ml[row * 2];
        ap[j] = *reinterpret_cast<const f4*>(a.ws_acc + row * D + ch * 4);
      }
#pragma unroll
      for (int j = 0; j < B; ++j)
        if (p0 + j < p_hi && mp[j] != kNegInf) val += ap[j] * exp2_fast(mp[j] - M);
    }
  }
  partial[tid] = val;
  __syncthreads();
  if (tid < kCols4) {
    f4 sum = partial[tid];
    for (int rr = 1; rr < kRowsH; ++rr) sum += partial[rr * kCols4 + tid];
    float lam = 0.f;
#pragma unroll
    for (int v = 0; v < kMergeWaves; ++v) lam += head_sum[v];
    *reinterpret_cast<f4*>(a.out + ((int64_t)s * a.num_heads + h * G + gq) * D + tid * 4) =
        lam > 0.f ? sum / lam : f4{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();   // head_max, head_sum and partial are reused by the next unit
}

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_splits(DecodeParams a) {
  typedef merge_f4 f4;
  constexpr int kCols4 = D / 4;
  __shared__ float head_max[kMergeWaves], head_sum[kMergeWaves];
  __shared__ f4 partial[kMergeThreads];
  const int Hkv = a.num_kv_heads, G = a.group, S = a.num_seqs;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int C = G * kCols4;                       // columns per unit, <= 512
  const int R = kMergeThreads / C;                // rows of threads, >= 1
  const int r = tid / C, c = tid - r * C;
  const int g = c / kCols4, d4 = c - g * kCols4;  // this thread's column
  const float2* ml = reinterpret_cast<const float2*>(a.ws_ml);
  // After an attention kernel that planned the batch itself: the call's
  // abort word from the one that kernel writes, which is cleared for the
  // next such call (its waits record only the mark, never clear it).
  if (a.inline_plan && blockIdx.x == 0 && tid == 0) {
    a.ws_ctrl[kCtrlAbort] = a.ws_ctrl[kCtrlAbortPlanned] == kAbortMark;
    a.ws_ctrl[kCtrlAbortPlanned] = 0;
  }
  // Unit counts fit in 31 bits (S * Hq is bounded on the host), so the unit
  // arithmetic is 32-bit: a 64-bit division costs a wave hundreds of
  // instructions before its first load.
  const int n_short = a.ws_ctrl[kCtrlSplits] * Hkv;
  const int n_long = a.ws_ctrl[kCtrlLongSplits] * Hkv;

  // A short unit's list entry is read before the unit counts are known (its
  // index is clamped into the list, and the entry is used only for units
  // below the count), so the first entry and the counts arrive in one memory
  // round trip.  (The same for the long units below measured slower on the
  // skewed long-context workload, 6.56 vs 6.10 us.)
  if (r < R) {
    int u = blockIdx.x + r * gridDim.x;
    int2 e_next = a.ws_split[min(u / Hkv, S - 1)];
    for (; u < n_short; u += (int)gridDim.x * R) {
      const int2 e = e_next;
      e_next = a.ws_split[min((u + (int)gridDim.x * R) / Hkv, S - 1)];
      const int h = u % Hkv;
      const int s = e.x, nparts = e.y;
      const int64_t prow = ((int64_t)s * Hkv + h) * a.num_parts_max;   // partition 0's row
      float2 mlp[kMergeShort];
      f4 ap[kMergeShort];
      float M = kNegInf;
      // Only the unit's partitions are read (a guarded load, not a clamped
      // address the compiler may load from unconditionally): a unit of 2
      // partitions reads 2 states, not kMergeShort.
#pragma unroll
      for (int j = 0; j < kMergeShort; ++j) {
        mlp[j] = make_float2(kNegInf, 0.f);
        ap[j] = f4{0.f, 0.f, 0.f, 0.f};
        if (j < nparts) {
          const int64_t row = (prow + j) * G + g;
          mlp[j] = ml[row];
          ap[j] = *reinterpret_cast<const f4*>(a.ws_acc + row * D + d4 * 4);
        }
      }
#pragma unroll
      for (int j = 0; j < kMergeShort; ++j) M = fmaxf(M, mlp[j].x);
      float lam = 0.f;
      f4 val = {0.f, 0.f, 0.f, 0.f};
      if (M != kNegInf) {
#pragma unroll
        for (int j = 0; j < kMergeShort; ++j)
          if (mlp[j].x != kNegInf) {
            const float w = exp2_fast(mlp[j].x - M);
            lam += mlp[j].y * w;
            val += ap[j] * w;
          }
      }
      *reinterpret_cast<f4*>(a.out + ((int64_t)s * a.num_heads + h * G + g) * D + d4 * 4) =
          lam > 0.f ? val / lam : f4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // Long units, one query head per workgroup (so a long sequence's partition
  // states are read by G workgroups at once, not one): unit u is (split
  // sequence u / (Hkv * G), KV head, query head u % G).  The batch a row of
  // threads loads at once is sized to the row's run of partitions (8, 16 or
  // 32), uniform over the workgroup.
  constexpr int kRowsH = kMergeThreads / kCols4;
  for (int u = gridDim.x - 1 - blockIdx.x; u < n_long * G; u += gridDim.x) {
    const int uh = u / G;                      // (split sequence, KV head)
    const int gq = (int)(u - uh * G);
    const int2 e = a.ws_split[S - 1 - uh / Hkv];
    const int h = uh % Hkv;
    const int span = (e.y + kRowsH - 1) / kRowsH;   // partitions per row, at most
    if (span <= 8)
      merge_long_head<D, 8>(a, e.x, h, gq, e.y, head_max, head_sum, partial);
    else if (span <= 16)
      merge_long_head<D, 16>(a, e.x, h, gq, e.y, head_max, head_sum, partial);
    else
      merge_long_head<D, kMergeBatch>(a, e.x, h, gq, e.y, head_max, head_sum, partial);
  }
}

// ---------------------------------------------------------------------------
// Launch.
// ---------------------------------------------------------------------------

template <int D>
size_t smem_bytes(int group, bool valu, int block_size, int lds_slots, int lds_records) {
  const size_t state = lds_state_floats<D, kWaves>(group);
  if (valu) return (state + (size_t)group * D + (size_t)kWaves * kMaxGroup * block_size) * 4;
  return ((size_t)lds_slots * state + (size_t)lds_records * lds_record_floats<D>(group)) * 4;
}

// LDS of the matrix-core kernel: two state slots and as many output records
// (up to kMaxLdsRecords) as fit in this workgroup's share of the CU's 160 KB
// (8 waves per CU at the kernel's register use: 148 KB * W / 8); a single
// slot when two slots and one record do not fit.
template <int D>
void lds_layout_for(int group, int* slots, int* records) {
  const int budget = 148 * 1024 / 4 * kWaves / 8;
  const int state = lds_state_floats<D, kWaves>(group);
  const int rec = lds_record_floats<D>(group);
  int ns = 2;
  if (ns * state + rec > budget) ns = 1;
  int nr = (budget - ns * state) / rec;
  nr = nr < 1 ? 1 : (nr > kMaxLdsRecords ? kMaxLdsRecords : nr);
  *slots = ns;
  *records = nr;
}

// Compute units of the current device (0 if unknown).  PA_NUM_CUS_OVERRIDE
// (read at every call) replaces it, so tests can check the claim pools of a
// device with fewer CUs, or of one whose count is unknown, on this one.
int cu_count() {
  if (const char* o = getenv("PA_NUM_CUS_OVERRIDE")) return atoi(o);
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  auto found = cache.find(dev);
  if (found != cache.end()) return found->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
  cache.emplace(dev, cus);
  return cus;
}

// Workgroups of `kernel` that fit on the current device at once.
int resident_workgroups(const void* kernel, int threads, size_t smem) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, size_t>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const auto key = std::make_tuple(dev, kernel, smem);
  std::lock_guard<std::mutex> lock(mu);
  auto found = cache.find(key);
  if (found != cache.end()) return found->second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, smem) != hipSuccess)
    return 0;
  const int n = (per_cu < 1 ? 1 : per_cu) * (cus < 1 ? 1 : cus);
  cache.emplace(key, n);
  return n;
}

template <int D, int BS>
hipError_t launch_decode_shape(const DecodeParams& p0, KvType type, bool vector_alu,
                               hipStream_t stream, hipEvent_t ev_before, hipEvent_t ev_after,
                               const WriteArgs* write) {
  const int threads = 64 * kWaves;
  const void* kernel;
  size_t smem;
  DecodeParams p = p0;
  lds_layout_for<D>(p0.group, &p.lds_slots, &p.lds_records);
  // The adaptive partition keeps one partition at most 2/W of a workgroup's
  // share, so each wave's part of it is at most half a wave's share.
  if (p.balance) p.balance = kWaves / 2;
  const bool prefix = p.num_groups > 0;   // bf16 matrix-core kernel only (checked by the API)
  const bool packed = p.packed_pool != 0;  // bf16 matrix-core kernel, no prefixes (checked by the API)
  // A batch the one-wave planner would plan, decoded without a slot write in
  // the same call, is planned inside the attention kernel instead: one
  // launch less (merge_splits, which then always follows, reports its waits).
  const bool plan_inside = !vector_alu && !prefix && !packed && !write && small_plan(p) &&
                           p.num_parts_max > 1;
  p.inline_plan = plan_inside ? 1 : 0;
  const bool f32_mfma = type == KvType::F32 && !vector_alu;
  if (f32_mfma) {
    kernel = plan_inside ? (const void*)decode_mfma_f32<D, BS, kWaves, true>
                         : (const void*)decode_mfma_f32<D, BS, kWaves, false>;
    smem = smem_bytes<D>(p0.group, false, BS, p.lds_slots, p.lds_records);
  } else if (type == KvType::BF16 && !vector_alu) {
    kernel = prefix ? (const void*)decode_mfma_bf16<D, BS, kWaves, true>
             : packed ? (const void*)decode_mfma_bf16<D, BS, kWaves, false, false>
             : plan_inside ? (const void*)decode_mfma_bf16<D, BS, kWaves, false, true, true>
                           : (const void*)decode_mfma_bf16<D, BS, kWaves, false>;
    smem = smem_bytes<D>(p0.group, false, BS, p.lds_slots, p.lds_records);
    if (prefix) {
      const size_t pre = (size_t)prefix_lds_floats<D, kWaves>() * 4;
      smem = smem > pre ? smem : pre;
    }
  } else if (type == KvType::BF16) {
    kernel = (const void*)decode_valu<uint16_t, D, BS, kWaves>;
    smem = smem_bytes<D>(p0.group, true, BS, 0, 0);
  } else {
    kernel = (const void*)decode_valu<float, D, BS, kWaves>;
    smem = smem_bytes<D>(p0.group, true, BS, 0, 0);
  }
  const int resident = resident_workgroups(kernel, threads, smem);
  if (resident <= 0) return hipErrorInvalidDeviceFunction;
  const int64_t max_items = (int64_t)p.num_seqs * p.num_parts_max * p.num_kv_heads;
  p.decode_grid = (int)(max_items < resident ? max_items : resident);
  // Test hook: PA_DECODE_GRID_OVERRIDE (read at every call) lowers the grid,
  // so that tests reach the claim pools of a small grid on this device.
  if (const char* o = getenv("PA_DECODE_GRID_OVERRIDE")) {
    const int g = atoi(o);
    if (g > 0 && g < p.decode_grid) p.decode_grid = g;
  }
  p.num_cus = cu_count();

  p.prefix_rows = kPrefixRows;
  if (write && write->total > 0) {
    int64_t wblocks = (write->total + 1023) / 1024;
    if (wblocks > 4096) wblocks = 4096;   // grid-stride loop covers the rest
    const dim3 grid((unsigned)(1 + wblocks));
    if (write->elem_bytes == 2)
      hipLaunchKernelGGL((write_and_plan<uint16_t, BS>), grid, dim3(1024), 0, stream, p, *write);
    else
      hipLaunchKernelGGL((write_and_plan<uint32_t, BS>), grid, dim3(1024), 0, stream, p, *write);
  } else if (!plan_inside) {
    if (small_plan(p))
      hipLaunchKernelGGL((plan_items<BS, 64, false>), dim3(1), dim3(64), 0, stream, p);
    else if (p.num_seqs <= 256 && prefix)
      hipLaunchKernelGGL((plan_items<BS, 256, true>), dim3(1), dim3(256), 0, stream, p);
    else if (p.num_seqs <= 256)
      hipLaunchKernelGGL((plan_items<BS, 256, false>), dim3(1), dim3(256), 0, stream, p);
    else if (prefix)
      hipLaunchKernelGGL((plan_items<BS, 1024, true>), dim3(1), dim3(1024), 0, stream, p);
    else
      hipLaunchKernelGGL((plan_items<BS, 1024, false>), dim3(1), dim3(1024), 0, stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev_before && (e = hipEventRecord(ev_before, stream)) != hipSuccess) return e;
  if (f32_mfma && plan_inside)
    hipLaunchKernelGGL((decode_mfma_f32<D, BS, kWaves, true>), dim3(p.decode_grid),
                       dim3(threads), smem, stream, p);
  else if (f32_mfma)
    hipLaunchKernelGGL((decode_mfma_f32<D, BS, kWaves, false>), dim3(p.decode_grid),
                       dim3(threads), smem, stream, p);
  else if (type == KvType::BF16 && !vector_alu && prefix)
    hipLaunchKernelGGL((decode_mfma_bf16<D, BS, kWaves, true>), dim3(p.decode_grid),
                       dim3(threads), smem, stream, p);
  else if (type == KvType::BF16 && !vector_alu && packed)
    hipLaunchKernelGGL((decode_mfma_bf16<D, BS, kWaves, false, false>), dim3(p.decode_grid),
                       dim3(threads), smem, stream, p);
  else if (plan_inside)
    hipLaunchKernelGGL((decode_mfma_bf16<D, BS, kWaves, false, true, true>), dim3(p.decode_grid),
                       dim3(threads), smem, stream, p);
  else if (type == KvType::BF16 && !vector_alu)
    hipLaunchKernelGGL((decode_mfma_bf16<D, BS, kWaves, false>), dim3(p.decode_grid),
                       dim3(threads), smem, stream, p);
  else if (type == KvType::BF16)
    hipLaunchKernelGGL((decode_valu<uint16_t, D, BS, kWaves>), dim3(p.decode_grid),
                       dim3(threads), smem, stream, p);
  else
    hipLaunchKernelGGL((decode_valu<float, D, BS, kWaves>), dim3(p.decode_grid), dim3(threads),
                       smem, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev_after && (e = hipEventRecord(ev_after, stream)) != hipSuccess) return e;
  if (p.num_parts_max <= 1) return hipSuccess;
  // One workgroup per (sequence, KV head, query head) of a batch whose every
  // sequence is split, up to kMergeGrid; the kernel loops past that.  Only the planner
  // knows how many sequences are split; a workgroup beyond that count still
  // occupies its wave slots for a memory round trip before it exits, so the
  // grid is kept small.
  const int64_t units = (int64_t)p.num_seqs * p.num_kv_heads * p.group;
  const unsigned mgrid = (unsigned)(units < kMergeGrid ? units : kMergeGrid);
  hipLaunchKernelGGL(merge_splits<D>, dim3(mgrid), dim3(kMergeThreads), 0, stream, p);
  return hipGetLastError();
}

__global__ __launch_bounds__(64) void copy_word(const int32_t* src, int32_t* dst) {
  if (threadIdx.x == 0) *dst = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_copy_word(const int32_t* src, int32_t* flag, hipStream_t stream) {
  hipLaunchKernelGGL(copy_word, dim3(1), dim3(64), 0, stream, src, flag);
  return hipGetLastError();
}

bool decode_supported(KvType type, int32_t head_dim, int32_t block_size, int32_t group) {
  (void)type;
  return (head_dim == 64 || head_dim == 128) && (block_size == 16 || block_size == 32) &&
         group >= 1 && group <= kMaxGroup;
}

hipError_t launch_decode(const DecodeParams& p, size_t params_bytes, KvType type,
                         int32_t head_dim, int32_t block_size, bool vector_alu,
                         hipStream_t stream, hipEvent_t ev_before, hipEvent_t ev_after,
                         const WriteArgs* write) {
  if (params_bytes != sizeof(DecodeParams)) return hipErrorInvalidImage;
  if (head_dim == 64 && block_size == 16)
    return launch_decode_shape<64, 16>(p, type, vector_alu, stream, ev_before, ev_after, write);
  if (head_dim == 64 && block_size == 32)
    return launch_decode_shape<64, 32>(p, type, vector_alu, stream, ev_before, ev_after, write);
  if (head_dim == 128 && block_size == 16)
    return launch_decode_shape<128, 16>(p, type, vector_alu, stream, ev_before, ev_after, write);
  if (head_dim == 128 && block_size == 32)
    return launch_decode_shape<128, 32>(p, type, vector_alu, stream, ev_before, ev_after, write);
  return hipErrorInvalidValue;
}

}  // namespace pa
