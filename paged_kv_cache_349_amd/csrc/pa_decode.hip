// Decode attention straight over the paged KV pool (gfx950 / CDNA4).
//
// "PagedAttention and KV memory management", section "The kernel side":
// the kernel reads the sequence's block table, loads each physical block's
// K and V tiles in turn, and computes scores and weighted values without
// first gathering the KV into one buffer.
//
// Work items.  A sequence's context is cut into partitions of part_blocks
// logical blocks; one work item is (sequence s, KV head h, partition p).
// The cut depends only on the sequence's own length, so every reduction
// order below depends only on logical positions: results are bitwise
// reproducible, independent of where blocks sit in the pool and of the
// other sequences in the batch.
//
// Two launches on the caller's stream:
//   plan_items    one workgroup.  Lists the non-empty (s, p) pairs in the
//                 workspace -- every full partition first (sequence order),
//                 then the partial last partitions in decreasing size -- and
//                 clears the merge counters.
//   decode_*      persistent: as many workgroups as fit on the chip at once,
//                 dealt the list round-robin, so no workgroup is launched for
//                 an empty partition and the work per workgroup stays even
//                 however ragged the context lengths are.
//
// Inside an item, wave w of the W waves takes logical blocks
// b0 + w, b0 + w + W, ... and keeps a running softmax state (max m, sum l,
// weighted sum acc) per query head of the group; the W states are merged
// through LDS in wave order.  A sequence with one partition writes `out`
// directly.  Otherwise the item stores its partition state in the workspace
// and bumps the (s, h) arrival counter; the workgroup that brings it to the
// partition count merges all partitions of (s, h) with a log-sum-exp
// combination, in partition order, and writes `out`.
//
// Matrix-core kernel (bf16).  For each 16-token sub-block:
//   S^T[16 tokens x 16 heads] = K[16 x D] * Q^T[D x 16]      (v_mfma_f32_16x16x32_bf16)
//   O^T[16 d x 16 heads]     += V^T[16 d x 16] * P^T[16 x 16] (v_mfma_f32_16x16x16_bf16)
// The G query heads of a KV group fill the 16-wide head dimension (padded
// with zero queries), so each loaded K/V tile serves all G heads.  Lane l
// holds scores of tokens 4*(l/16)+r (r < 4) for head l%16, which is exactly
// the B operand layout the PV product needs, so P never leaves registers.
// K rows are loaded straight into the A operand (16 bytes per lane per
// instruction); V is stored transposed per block (feature-major), so each lane
// loads 4 consecutive tokens of one feature (8 bytes) for the PV A operand.
// P is rounded to bf16 for the PV product; the softmax denominator sums those
// same rounded weights, so the output is an exact convex combination of them.
//
// Vector-ALU kernel (fp32, and bf16 on request): the same items and merge;
// scores by lanes over tokens, weighted values by lanes over features.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <tuple>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kMaxGroup = 16;   // query heads per KV head the kernels handle
constexpr int kWaves = 4;       // waves per decode workgroup
constexpr int kTailClasses = 256;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even (inputs here are finite, >= 0).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }

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

// Block-wide sum over the planner's 1024 threads (16 waves).
__device__ __forceinline__ int block_sum_1024(int v, int* scratch16) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch16[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) t += scratch16[w];
  return t;
}

constexpr int kPartChoices = 8;

__global__ __launch_bounds__(1024) void plan_items(DecodeParams a, int block_size) {
  __shared__ int cls_off[kTailClasses];
  __shared__ int wave_sum[16];
  __shared__ int run_base;
  __shared__ int nsplit;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = a.num_seqs;

  for (int i = tid; i < kTailClasses; i += 1024) cls_off[i] = 0;
  if (tid == 0) {
    run_base = 0;
    nsplit = 0;
  }

  // Partition size: the largest pb = part_blocks_min * 2^k (<= part_blocks_max)
  // whose partitions are each at most 1/balance of one workgroup's share of
  // all blocks.  Long partitions mean few partition states to merge; short
  // ones spread a long context over many workgroups.
  int pb = a.part_blocks_min;
  if (a.balance > 0 && a.part_blocks_max > pb) {
    int mine = 0;     // S * max_blocks fits in int32 (checked on the host)
    for (int s = tid; s < S; s += 1024)
      mine += (clamp_len(a, s, block_size) + block_size - 1) / block_size;
    const int64_t total = block_sum_1024(mine, wave_sum);
    const int64_t share = total * a.num_kv_heads / ((int64_t)a.decode_grid * a.balance);
    for (int k = 0; k < kPartChoices && (int64_t)pb * 2 <= share &&
                    pb * 2 <= a.part_blocks_max; ++k)
      pb *= 2;
  }
  if (tid == 0) a.ws_ctrl[kCtrlPartBlocks] = pb;
  __syncthreads();

  // Partial last partition of a sequence: size class, larger partitions in
  // lower classes.  -1 if the sequence has no partial partition.
  auto tail_class = [&](int nblk) {
    const int rem = nblk % pb;
    if (rem == 0) return -1;
    return (int)((int64_t)(pb - rem) * (kTailClasses - 1) / pb);
  };

  // Pass 1: full partitions in sequence order (an empty sequence gets one
  // item that zeroes its output); count partial partitions per class; list
  // the sequences that span several partitions.
  for (int c0 = 0; c0 < S; c0 += 1024) {
    const int s = c0 + tid;
    int nfull = 0;
    if (s < S) {
      const int nblk = (clamp_len(a, s, block_size) + block_size - 1) / block_size;
      nfull = nblk == 0 ? 1 : nblk / pb;
      const int c = tail_class(nblk);
      if (c >= 0) atomicAdd(&cls_off[c], 1);
      if (nblk > pb) a.ws_split[atomicAdd(&nsplit, 1)] = s;
    }
    int incl = nfull;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    if (lane == 63) wave_sum[wave] = incl;
    __syncthreads();
    int before = 0, chunk = 0;
    for (int w = 0; w < 16; ++w) {
      before += w < wave ? wave_sum[w] : 0;
      chunk += wave_sum[w];
    }
    const int base = run_base + before + incl - nfull;
    for (int p = 0; p < nfull; ++p) a.ws_items[base + p] = make_int2(s, p);
    __syncthreads();
    if (tid == 0) run_base += chunk;
    __syncthreads();
  }

  // Class start offsets after the full partitions.
  if (tid == 0) {
    int off = run_base;
    for (int c = 0; c < kTailClasses; ++c) {
      const int n = cls_off[c];
      cls_off[c] = off;
      off += n;
    }
    a.ws_ctrl[kCtrlEntries] = off;
    a.ws_ctrl[kCtrlSplits] = nsplit;
  }
  __syncthreads();

  // Pass 2: partial partitions.  The order inside a class is arbitrary; it
  // changes which workgroup computes an item, never the result.
  for (int s = tid; s < S; s += 1024) {
    const int nblk = (clamp_len(a, s, block_size) + block_size - 1) / block_size;
    const int c = tail_class(nblk);
    if (c >= 0) a.ws_items[atomicAdd(&cls_off[c], 1)] = make_int2(s, nblk / pb);
  }
}

struct Item {
  int s, h, part, L, nblk, b0, b1, nparts;
};

__device__ __forceinline__ Item make_item(const DecodeParams& a, int2 e, int h, int block_size,
                                          int pb) {
  Item it;
  it.s = e.x;
  it.part = e.y;
  it.h = h;
  it.L = clamp_len(a, it.s, block_size);
  it.nblk = (it.L + block_size - 1) / block_size;
  it.b0 = it.part * pb;
  it.b1 = min(it.b0 + pb, it.nblk);
  it.nparts = (it.nblk + pb - 1) / pb;
  return it;
}

// LDS areas shared by both kernels (floats): sm_m, sm_l [W][kMaxGroup],
// sm_acc [W][group][D + 4].
template <int D, int W>
struct Lds {
  float* m;
  float* l;
  float* acc;
  __device__ Lds(float* smem, int group) : m(smem), l(smem + W * kMaxGroup),
                                           acc(smem + 2 * W * kMaxGroup) {
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

// Persistent item loop shared by both kernels: workgroup b takes list items
// b, b + G, b + 2G, ... (G = grid size, all resident at once).  The list
// holds full partitions first and partial ones in decreasing size, so the
// round-robin deal evens out the work per workgroup without any shared
// counter: the workgroups left one full partition short are the first to
// receive the largest partial ones.
template <int D, int W, typename Body>
__device__ __forceinline__ void run_items(const DecodeParams& a, int block_size, float* smem,
                                          Body body) {
  const int Hkv = a.num_kv_heads;
  const int total = a.ws_ctrl[kCtrlEntries] * Hkv;
  const int pb = a.ws_ctrl[kCtrlPartBlocks];
  const Lds<D, W> sm(smem, a.group);
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int e_idx = item / Hkv;
    const Item it = make_item(a, a.ws_items[e_idx], item - e_idx * Hkv, block_size, pb);
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

template <int D, int BS>
__device__ __forceinline__ void load_tile(Tile<D, BS>& t, const uint16_t* __restrict__ kt,
                                          const uint16_t* __restrict__ vt, int lane) {
  const int row = lane & 15, quad = lane >> 4;
#pragma unroll
  for (int sb = 0; sb < Tile<D, BS>::SB; ++sb) {
    const uint16_t* kr = kt + (sb * 16 + row) * D + quad * 8;
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
      t.k[sb][c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kr + c * 32));
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      const uint16_t* vr = vt + (i * 16 + row) * BS + sb * 16 + quad * 4;
      t.v[sb][i] = __builtin_bit_cast(i16x4, *reinterpret_cast<const uint2*>(vr));
    }
  }
}

template <int D, int BS, int W>
__device__ __forceinline__ void mfma_item(const DecodeParams& a, const Item& it,
                                          const Lds<D, W>& sm) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane & 15, quad = lane >> 4;
  const int G = a.group;
  const int Hkv = a.num_kv_heads;

  // Query operand: lane holds q[head g][32c + 8*quad .. +7] (zero for padding heads).
  bf16x8 qop[D / 32];
  {
    const uint16_t* qg =
        (const uint16_t*)a.q + ((int64_t)it.s * a.num_heads + it.h * G + g) * D + quad * 8;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (g < G) raw = *reinterpret_cast<const uint4*>(qg + c * 32);
      qop[c] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // Block ids of this wave's blocks, 64 at a time, one per lane: lane k of
  // the current chunk holds the id of the wave's (id_base + k)-th block.
  const int nmine = (it.b1 - (it.b0 + w) + W - 1) / W;   // may be <= 0
  const int32_t* trow = a.tables + (int64_t)it.s * a.max_blocks;
  int id_base = 0;
  int my_id = -1;
  if (lane < nmine) my_id = trow[it.b0 + w + lane * W];

  const uint16_t* kbase = (const uint16_t*)a.k_cache;
  const uint16_t* vbase = (const uint16_t*)a.v_cache;
  const int64_t tile_elems = (int64_t)BS * D;

  float m = kNegInf, lsum = 0.f;
  f32x4 acc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // k increases by one per call, so the next chunk is fetched when k leaves this one.
  auto tile_ptrs = [&](int k, const uint16_t*& kt, const uint16_t*& vt) -> bool {
    if (k - id_base >= 64) {
      id_base += 64;
      my_id = (id_base + lane < nmine) ? trow[it.b0 + w + (id_base + lane) * W] : -1;
    }
    const int id = __builtin_amdgcn_readlane(my_id, k - id_base);
    if ((unsigned)id >= (unsigned)a.num_blocks) return false;
    const int64_t tile = (int64_t)id * Hkv + it.h;
    kt = kbase + tile * tile_elems;
    vt = vbase + tile * tile_elems;
    return true;
  };

  auto compute = [&](Tile<D, BS>& t, int k) {
    const int j = it.b0 + w + k * W;               // logical block number
    const int tok0 = j * BS;
    f32x4 sc[Tile<D, BS>::SB];
#pragma unroll
    for (int sb = 0; sb < Tile<D, BS>::SB; ++sb) {
      sc[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
        sc[sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t.k[sb][c], qop[c], sc[sb], 0, 0, 0);
    }
    // Scale into base-2 units, mask positions >= L (select, never multiply:
    // the tail of the last block may hold anything), block max per head.
    float mx = kNegInf;
#pragma unroll
    for (int sb = 0; sb < Tile<D, BS>::SB; ++sb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pos = tok0 + sb * 16 + quad * 4 + r;
        const float x = pos < it.L ? sc[sb][r] * a.scale_log2 : kNegInf;
        sc[sb][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const float mnew = fmaxf(m, mx);
    const float alpha = exp2_fast(m - mnew);        // 0 on the first block (m = -inf)
    m = mnew;
    i16x4 pb[Tile<D, BS>::SB];
    float psum = 0.f;
#pragma unroll
    for (int sb = 0; sb < Tile<D, BS>::SB; ++sb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t b = f32_to_bf16_bits(exp2_fast(sc[sb][r] - mnew));
        pb[sb][r] = (short)b;
        psum += bf16_bits_to_f32(b);
      }
    lsum = lsum * alpha + psum;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) acc[i] *= alpha;
    // Last block: zero V of masked positions (their weight is 0, but 0 * NaN is NaN).
    if (tok0 + BS > it.L) {
#pragma unroll
      for (int sb = 0; sb < Tile<D, BS>::SB; ++sb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool dead = tok0 + sb * 16 + quad * 4 + r >= it.L;
#pragma unroll
          for (int i = 0; i < D / 16; ++i) t.v[sb][i][r] = dead ? (short)0 : t.v[sb][i][r];
        }
    }
#pragma unroll
    for (int i = 0; i < D / 16; ++i)
#pragma unroll
      for (int sb = 0; sb < Tile<D, BS>::SB; ++sb)
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(t.v[sb][i], pb[sb], acc[i], 0, 0, 0);
  };

  // Two register tiles: the next block's loads are in flight while the
  // current one is computed.
  Tile<D, BS> t0, t1;
  const uint16_t *kt, *vt;
  bool ok0 = false, ok1 = false;
  if (nmine > 0 && (ok0 = tile_ptrs(0, kt, vt))) load_tile<D, BS>(t0, kt, vt, lane);
  for (int k = 0; k < nmine; k += 2) {
    if (k + 1 < nmine && (ok1 = tile_ptrs(k + 1, kt, vt))) load_tile<D, BS>(t1, kt, vt, lane);
    if (ok0) compute(t0, k);
    if (k + 1 >= nmine) break;
    if (k + 2 < nmine && (ok0 = tile_ptrs(k + 2, kt, vt))) load_tile<D, BS>(t0, kt, vt, lane);
    if (ok1) compute(t1, k + 1);
  }

  // Sum l over the four lane quads that hold the same head.
  lsum += shfl_xor_f(lsum, 16);
  lsum += shfl_xor_f(lsum, 32);

  if (quad == 0) {
    sm.m[w * kMaxGroup + g] = m;
    sm.l[w * kMaxGroup + g] = lsum;
  }
  if (g < G) {
#pragma unroll
    for (int i = 0; i < D / 16; ++i)
      *reinterpret_cast<f32x4*>(&sm.acc[(w * G + g) * (D + 4) + i * 16 + quad * 4]) = acc[i];
  }
  __syncthreads();
}

template <int D, int BS, int W>
__global__ __launch_bounds__(64 * W) void decode_mfma_bf16(DecodeParams a) {
  extern __shared__ float smem[];
  run_items<D, W>(a, BS, smem, [&](const Item& it, const Lds<D, W>& sm) {
    mfma_item<D, BS, W>(a, it, sm);
  });
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
        const float vv = widen<T>(vt[(lane + 64 * k) * BS + t]);
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
// partition order: with M = max_p m_p, out = sum_p 2^(m_p - M) acc_p /
// sum_p 2^(m_p - M) l_p.  One workgroup per (split sequence, KV head), four
// features per thread.
// ---------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256) void merge_splits(DecodeParams a, int block_size) {
  typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f4;
  const int Hkv = a.num_kv_heads, G = a.group;
  const int total = a.ws_ctrl[kCtrlSplits] * Hkv;
  const int pb = a.ws_ctrl[kCtrlPartBlocks];
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int s = a.ws_split[item / Hkv];
    const int h = item % Hkv;
    const int nblk = (clamp_len(a, s, block_size) + block_size - 1) / block_size;
    const int nparts = (nblk + pb - 1) / pb;
    const int64_t prow = ((int64_t)s * Hkv + h) * a.num_parts_max;
    for (int idx = threadIdx.x; idx < G * (D / 4); idx += 256) {
      const int g = idx / (D / 4);
      const int d4 = idx - g * (D / 4);
      float M = kNegInf;
      for (int p = 0; p < nparts; ++p) M = fmaxf(M, a.ws_ml[((prow + p) * G + g) * 2]);
      float lam = 0.f;
      f4 val = {0.f, 0.f, 0.f, 0.f};
      for (int p = 0; p < nparts; ++p) {
        const int64_t row = (prow + p) * G + g;
        const float mp = a.ws_ml[row * 2];
        const float c = (mp == kNegInf) ? 0.f : exp2_fast(mp - M);
        lam += a.ws_ml[row * 2 + 1] * c;
        val += *reinterpret_cast<const f4*>(a.ws_acc + row * D + d4 * 4) * c;
      }
      const f4 o = lam > 0.f ? val / lam : f4{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f4*>(a.out + ((int64_t)s * a.num_heads + h * G + g) * D + d4 * 4) = o;
    }
  }
}

// ---------------------------------------------------------------------------
// Launch.
// ---------------------------------------------------------------------------

template <int D>
size_t smem_bytes(int group, bool valu, int block_size) {
  size_t f = 2 * kWaves * kMaxGroup + (size_t)kWaves * group * (D + 4);
  if (valu) f += (size_t)group * D + (size_t)kWaves * kMaxGroup * block_size;
  return f * sizeof(float);
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
                               hipStream_t stream) {
  const int threads = 64 * kWaves;
  const void* kernel;
  size_t smem;
  if (type == KvType::BF16 && !vector_alu) {
    kernel = (const void*)decode_mfma_bf16<D, BS, kWaves>;
    smem = smem_bytes<D>(p0.group, false, BS);
  } else if (type == KvType::BF16) {
    kernel = (const void*)decode_valu<uint16_t, D, BS, kWaves>;
    smem = smem_bytes<D>(p0.group, true, BS);
  } else {
    kernel = (const void*)decode_valu<float, D, BS, kWaves>;
    smem = smem_bytes<D>(p0.group, true, BS);
  }
  const int resident = resident_workgroups(kernel, threads, smem);
  if (resident <= 0) return hipErrorInvalidDeviceFunction;
  DecodeParams p = p0;
  const int64_t max_items = (int64_t)p.num_seqs * p.num_parts_max * p.num_kv_heads;
  p.decode_grid = (int)(max_items < resident ? max_items : resident);

  hipLaunchKernelGGL(plan_items, dim3(1), dim3(1024), 0, stream, p, BS);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (type == KvType::BF16 && !vector_alu)
    hipLaunchKernelGGL((decode_mfma_bf16<D, BS, kWaves>), dim3(p.decode_grid), dim3(threads),
                       smem, stream, p);
  else if (type == KvType::BF16)
    hipLaunchKernelGGL((decode_valu<uint16_t, D, BS, kWaves>), dim3(p.decode_grid),
                       dim3(threads), smem, stream, p);
  else
    hipLaunchKernelGGL((decode_valu<float, D, BS, kWaves>), dim3(p.decode_grid), dim3(threads),
                       smem, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess || p.num_parts_max <= 1) return e;
  const int64_t pairs = (int64_t)p.num_seqs * p.num_kv_heads;
  const unsigned mgrid = (unsigned)(pairs < 2048 ? pairs : 2048);
  hipLaunchKernelGGL(merge_splits<D>, dim3(mgrid), dim3(256), 0, stream, p, BS);
  return hipGetLastError();
}

}  // namespace

bool decode_supported(KvType type, int32_t head_dim, int32_t block_size, int32_t group) {
  (void)type;
  return (head_dim == 64 || head_dim == 128) && (block_size == 16 || block_size == 32) &&
         group >= 1 && group <= kMaxGroup;
}

hipError_t launch_decode(const DecodeParams& p, KvType type, int32_t head_dim,
                         int32_t block_size, bool vector_alu, hipStream_t stream) {
  if (head_dim == 64 && block_size == 16)
    return launch_decode_shape<64, 16>(p, type, vector_alu, stream);
  if (head_dim == 64 && block_size == 32)
    return launch_decode_shape<64, 32>(p, type, vector_alu, stream);
  if (head_dim == 128 && block_size == 16)
    return launch_decode_shape<128, 16>(p, type, vector_alu, stream);
  if (head_dim == 128 && block_size == 32)
    return launch_decode_shape<128, 32>(p, type, vector_alu, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
