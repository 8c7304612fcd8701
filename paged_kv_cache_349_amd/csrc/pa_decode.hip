// Decode attention straight over the paged KV pool (gfx950 / CDNA4).
//
// "PagedAttention and KV memory management", section "The kernel side":
// the kernel reads the sequence's block table, loads each physical block's
// K and V tiles in turn, and computes scores and weighted values without
// first gathering the KV into one buffer.
//
// Work split.  One workgroup of W waves owns (sequence s, KV head h,
// partition p): p covers part_blocks consecutive logical blocks.  Wave w of
// the workgroup takes blocks p*part_blocks + w, + w + W, ... and keeps a
// running softmax state (max m, sum l, weighted sum acc) per query head of
// the group.  At the end the W wave states are merged through LDS in wave
// order.  A sequence with one partition writes `out` directly; otherwise the
// partition's state goes to the workspace and merge_partitions() combines the
// partitions with a log-sum-exp merge, in partition order.  Every reduction
// order depends on logical positions only.
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
// Vector-ALU kernel (fp32, and bf16 on request): the same work split and
// merge; scores by lanes over tokens, weighted values by lanes over features.
#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kMaxGroup = 16;   // query heads per KV head the kernels handle
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

// Shared tail of both kernels: merge the W wave states of this workgroup
// (wave order), then either finish the sequence (one partition) or store the
// partition state for merge_partitions().
//   sm_m, sm_l: [W][kMaxGroup]; sm_acc: [W][group][D + 4]
template <int D, int W>
__device__ __forceinline__ void finish_partition(const DecodeParams& a, const float* sm_m,
                                                 const float* sm_l, const float* sm_acc, int s,
                                                 int h, int part, int nparts) {
  const int G = a.group;
  for (int idx = threadIdx.x; idx < G * D; idx += 64 * W) {
    const int g = idx / D;
    const int d = idx - g * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, sm_m[w * kMaxGroup + g]);
    float lam = 0.f, val = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mw = sm_m[w * kMaxGroup + g];
      const float c = (mw == kNegInf) ? 0.f : exp2_fast(mw - M);
      lam += sm_l[w * kMaxGroup + g] * c;
      val += sm_acc[(w * G + g) * (D + 4) + d] * c;
    }
    if (nparts == 1) {
      a.out[((int64_t)s * a.num_heads + h * G + g) * D + d] = lam > 0.f ? val / lam : 0.f;
    } else {
      const int64_t row = (((int64_t)s * a.num_kv_heads + h) * a.num_parts_max + part) * G + g;
      a.ws_acc[row * D + d] = val;
      if (d == 0) {
        a.ws_ml[row * 2 + 0] = M;
        a.ws_ml[row * 2 + 1] = lam;
      }
    }
  }
}

// Zero output of a sequence with no tokens (written by partition 0).
template <int D, int W>
__device__ __forceinline__ void zero_sequence(const DecodeParams& a, int s, int h) {
  const int G = a.group;
  for (int idx = threadIdx.x; idx < G * D; idx += 64 * W)
    a.out[((int64_t)s * a.num_heads + h * G) * D + idx] = 0.f;
}

// Decode the flat workgroup index into (partition, sequence, KV head) and the
// partition's block range.  Returns false if the workgroup has nothing to do.
struct WorkItem {
  int s, h, part, L, nblk, b0, b1, nparts;
};

__device__ __forceinline__ WorkItem decode_work_item(const DecodeParams& a, int block_size) {
  WorkItem it;
  const int idx = blockIdx.x;
  it.part = idx % a.num_parts_max;
  const int rest = idx / a.num_parts_max;
  it.s = rest % a.num_seqs;
  it.h = rest / a.num_seqs;
  int L = a.lens[it.s];
  const int Lmax = a.max_blocks * block_size;
  L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
  it.L = L;
  it.nblk = (L + block_size - 1) / block_size;
  it.b0 = it.part * a.part_blocks;
  it.b1 = min(it.b0 + a.part_blocks, it.nblk);
  it.nparts = (it.nblk + a.part_blocks - 1) / a.part_blocks;
  return it;
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
__global__ __launch_bounds__(64 * W) void decode_mfma_bf16(DecodeParams a) {
  extern __shared__ float smem[];
  const WorkItem it = decode_work_item(a, BS);
  if (it.nblk == 0) {
    if (it.part == 0) zero_sequence<D, W>(a, it.s, it.h);
    return;
  }
  if (it.b0 >= it.nblk) return;

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

  float* sm_m = smem;
  float* sm_l = smem + W * kMaxGroup;
  float* sm_acc = smem + 2 * W * kMaxGroup;
  if (quad == 0) {
    sm_m[w * kMaxGroup + g] = m;
    sm_l[w * kMaxGroup + g] = lsum;
  }
  if (g < G) {
#pragma unroll
    for (int i = 0; i < D / 16; ++i)
      *reinterpret_cast<f32x4*>(&sm_acc[(w * G + g) * (D + 4) + i * 16 + quad * 4]) = acc[i];
  }
  __syncthreads();
  finish_partition<D, W>(a, sm_m, sm_l, sm_acc, it.s, it.h, it.part, it.nparts);
}

// ---------------------------------------------------------------------------
// Vector-ALU kernel (fp32 KV; also bf16 when asked).
// ---------------------------------------------------------------------------

template <typename T, int D, int BS, int W>
__global__ __launch_bounds__(64 * W) void decode_valu(DecodeParams a) {
  extern __shared__ float smem[];
  const WorkItem it = decode_work_item(a, BS);
  if (it.nblk == 0) {
    if (it.part == 0) zero_sequence<D, W>(a, it.s, it.h);
    return;
  }
  if (it.b0 >= it.nblk) return;

  constexpr int NC = 64 / BS;          // lanes per token in the score step
  constexpr int DC = D / NC;           // features per lane in the score step
  constexpr int DL = D / 64;           // features per lane in the weighted sum
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.group;
  const int Hkv = a.num_kv_heads;
  const int tt = lane % BS, ch = lane / BS;

  float* sm_m = smem;
  float* sm_l = smem + W * kMaxGroup;
  float* sm_acc = smem + 2 * W * kMaxGroup;            // [W][G][D+4]
  float* sm_q = sm_acc + W * G * (D + 4);              // [G][D]
  float* sm_p = sm_q + G * D;                          // [W][kMaxGroup][BS]

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
      sm_m[w * kMaxGroup + g] = m[g];
      sm_l[w * kMaxGroup + g] = l;
    }
#pragma unroll
    for (int k = 0; k < DL; ++k) sm_acc[(w * G + g) * (D + 4) + lane + 64 * k] = acc[g][k];
  }
  __syncthreads();
  finish_partition<D, W>(a, sm_m, sm_l, sm_acc, it.s, it.h, it.part, it.nparts);
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of a sequence's partitions, in partition order.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void merge_partitions(DecodeParams a, int head_dim,
                                                        int block_size) {
  const int s = blockIdx.x % a.num_seqs;
  const int h = blockIdx.x / a.num_seqs;
  int L = a.lens[s];
  const int Lmax = a.max_blocks * block_size;
  L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
  const int nblk = (L + block_size - 1) / block_size;
  const int nparts = (nblk + a.part_blocks - 1) / a.part_blocks;
  if (nparts <= 1) return;
  const int G = a.group, D = head_dim;
  const int64_t row0 = ((int64_t)s * a.num_kv_heads + h) * a.num_parts_max;
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int g = idx / D;
    const int d = idx - g * D;
    float M = kNegInf;
    for (int p = 0; p < nparts; ++p) M = fmaxf(M, a.ws_ml[((row0 + p) * G + g) * 2]);
    float lam = 0.f, val = 0.f;
    for (int p = 0; p < nparts; ++p) {
      const int64_t row = (row0 + p) * G + g;
      const float mp = a.ws_ml[row * 2];
      const float c = (mp == kNegInf) ? 0.f : exp2_fast(mp - M);
      lam += a.ws_ml[row * 2 + 1] * c;
      val += a.ws_acc[row * D + d] * c;
    }
    a.out[((int64_t)s * a.num_heads + h * G + g) * D + d] = lam > 0.f ? val / lam : 0.f;
  }
}

constexpr int kWaves = 4;

template <int D>
size_t smem_bytes(int group, bool valu, int block_size) {
  size_t f = 2 * kWaves * kMaxGroup + (size_t)kWaves * group * (D + 4);
  if (valu) f += (size_t)group * D + (size_t)kWaves * kMaxGroup * block_size;
  return f * sizeof(float);
}

template <int D, int BS>
hipError_t launch_decode_shape(const DecodeParams& p, KvType type, bool vector_alu,
                               hipStream_t stream) {
  const unsigned grid = (unsigned)((int64_t)p.num_parts_max * p.num_seqs * p.num_kv_heads);
  if (type == KvType::BF16 && !vector_alu) {
    hipLaunchKernelGGL((decode_mfma_bf16<D, BS, kWaves>), dim3(grid), dim3(64 * kWaves),
                       smem_bytes<D>(p.group, false, BS), stream, p);
  } else if (type == KvType::BF16) {
    hipLaunchKernelGGL((decode_valu<uint16_t, D, BS, kWaves>), dim3(grid), dim3(64 * kWaves),
                       smem_bytes<D>(p.group, true, BS), stream, p);
  } else {
    hipLaunchKernelGGL((decode_valu<float, D, BS, kWaves>), dim3(grid), dim3(64 * kWaves),
                       smem_bytes<D>(p.group, true, BS), stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.num_parts_max <= 1) return e;
  hipLaunchKernelGGL(merge_partitions, dim3((unsigned)(p.num_seqs * p.num_kv_heads)), dim3(256),
                     0, stream, p, D, BS);
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
