// Shared device-side definitions of the gfx950 attention kernels: vector types,
// bf16 packing, wave-level helpers and the KV / query addressing modes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gqa_attn.h"

namespace gqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -3.0e38f;  // finite floor for running maxima (avoids inf - inf)

constexpr int kHeadDim = 64;
constexpr int kMaxPosition = 1 << 30;  // history lengths of a chunk over a ring are clamped below this

// ---------------------------------------------------------------------------
// device-side metadata checks
//
// Metadata the kernels read from device memory (sequence lengths, query
// offsets, block tables) is clamped so that no access leaves the caller's
// buffers, whatever it holds.  Built with GQA_DEBUG the kernels also record
// every kind of value they had to clamp, as bits of a flag word that
// gqa_attn_debug_flags() reads back; release builds only clamp.
// (the GQA_DBG_* bits of gqa_attn.h)
constexpr unsigned kDbgSeqlensK = GQA_DBG_SEQLENS_K;
constexpr unsigned kDbgBlockTable = GQA_DBG_BLOCK_TABLE;
constexpr unsigned kDbgCuSeqlensQ = GQA_DBG_CU_SEQLENS_Q;
constexpr unsigned kDbgPackedRow = GQA_DBG_PACKED_ROW;
constexpr unsigned kDbgQLen = GQA_DBG_Q_LEN;

#ifdef GQA_DEBUG
static __device__ unsigned int g_debug_flags;  // one per translation unit
#define GQA_FLAG(cond, bit)                                      \
  do {                                                           \
    if (cond) atomicOr(&::gqa::g_debug_flags, (unsigned)(bit));  \
  } while (0)
// Host accessor of this translation unit's flag word (synchronising copy).
#define GQA_DEBUG_FLAGS_ACCESSOR(fn)                                                        \
  hipError_t fn(unsigned int* flags, bool reset) {                                          \
    hipError_t e = hipMemcpyFromSymbol(flags, HIP_SYMBOL(g_debug_flags), sizeof(unsigned)); \
    if (e == hipSuccess && reset) {                                                         \
      const unsigned zero = 0;                                                              \
      e = hipMemcpyToSymbol(HIP_SYMBOL(g_debug_flags), &zero, sizeof(unsigned));            \
    }                                                                                       \
    return e;                                                                               \
  }
#else
#define GQA_FLAG(cond, bit) \
  do {                      \
  } while (0)
#define GQA_DEBUG_FLAGS_ACCESSOR(fn)                       \
  hipError_t fn(unsigned int* flags, bool /*reset*/) {     \
    *flags = 0;                                            \
    return hipSuccess;                                     \
  }
#endif

// ---------------------------------------------------------------------------
// addressing of sequences
//
// A "sequence view" tells a workgroup where its queries and keys live:
//   q_row0     first packed query row of the sequence (row = index over [*, Hq, D])
//   q_len      number of query tokens
//   kv_len     number of KV positions (queries are the newest q_len of them)
// and, per KV position j, the packed KV row (index over [*, Hkv, D]).

enum KvMode : int {
  KV_BATCHED = 0,  // k [B, Lmax, Hkv, D]: row = b * Lmax + j
  KV_PAGED = 1,    // k [Nblk, bs, Hkv, D]: row = table[b][j >> log2bs] * bs + (j & (bs - 1))
  KV_PACKED = 2,   // k [Nrows, Hkv, D]: row = cu_seqlens_k[b] + j
  KV_RING = 3      // a chunk over a ring: positions j >= kv_len - q_len are the chunk's own
                   // rows [Tq, Hkv, D] (row q_row0 + j - (kv_len - q_len)); older ones sit in
                   // the ring [B, W, Hkv, D] of lmax = W slots (row b * W + j % W)
};

// Division of a non-negative int below 2^31 by a divisor d >= 1 fixed for a
// launch, without a division sequence on the device: the host picks a shift
// sh with 2^sh >= d and a multiplier m = floor(2^32 (2^sh - d) / d) + 1, and
// n / d = (umulhi(n, m) + n) >> sh (the round-up method of Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994).
struct FastDiv {
  uint32_t d, m, sh;
};

__host__ __device__ inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t sh = 0;
  while ((1ull << sh) < d) ++sh;
  const uint64_t m = ((1ull << 32) * ((1ull << sh) - d)) / d + 1;
  return FastDiv{d, (uint32_t)m, sh};
}

__host__ __device__ inline int fast_div(int n, const FastDiv& f) {
  const uint32_t t = (uint32_t)(((uint64_t)(uint32_t)n * f.m) >> 32);
  return (int)((t + (uint32_t)n) >> f.sh);
}

struct SeqArgs {
  // query side
  const int32_t* cu_seqlens_q;  // varlen only (NULL for batched)
  const int32_t* seqlens_k;     // varlen/decode (NULL for batched prefill)
  int q_len_fixed;              // batched: S (prefill) or 1 (decode)
  int kv_len_fixed;             // batched prefill: S; decode: Lmax (clamp bound)
  // KV side
  const int32_t* block_table;
  const int32_t* cu_seqlens_k;
  int max_blocks;
  int log2_block;
  int num_blocks;  // paged: number of physical blocks; packed: number of rows
  int lmax;        // batched: Lmax (row stride per sequence); varlen: max_kv_len
  int q_rows;      // varlen: packed query rows (Tq), the bound of cu_seqlens_q
  int ring;        // batched: the cache is a ring of lmax slots and seqlens_k counts the
                   // whole history; the ring holds min(seqlens_k[b], lmax) positions
};

struct SeqView {
  int64_t q_row0;
  int q_len;
  int kv_len;
  int b;
};

// Packed query rows [r0, r1) of sequence b, clamped to [0, q_rows].
__device__ __forceinline__ void q_range(const SeqArgs& a, int b, int& r0, int& r1) {
  const int c0 = a.cu_seqlens_q[b];
  const int c1 = a.cu_seqlens_q[b + 1];
  r0 = min(max(c0, 0), a.q_rows);
  r1 = min(max(c1, r0), a.q_rows);
  GQA_FLAG(r0 != c0 || r1 != c1, kDbgCuSeqlensQ);
}

template <int MODE>
__device__ __forceinline__ SeqView seq_view(const SeqArgs& a, int b, bool varlen_q) {
  SeqView s;
  s.b = b;
  if (varlen_q) {
    int r0, r1;
    q_range(a, b, r0, r1);
    s.q_row0 = r0;
    s.q_len = r1 - r0;
  } else {
    s.q_row0 = (int64_t)b * a.q_len_fixed;
    s.q_len = a.q_len_fixed;
  }
  if (a.seqlens_k) {
    int L0 = a.seqlens_k[b];
    // a ring holds the newest min(L, W) positions of a history of L: in contract
    if (MODE == KV_BATCHED && a.ring) L0 = min(L0, a.lmax);
    int L = L0;
    // bounds of the length: the cache rows of a sequence (batched), the block
    // table's capacity (paged), and max_kv_len (varlen calls: the split plan of
    // their decode rows covers that many keys)
    if (MODE == KV_BATCHED) L = min(L, a.lmax);
    if (MODE == KV_PAGED) L = min(L, min(a.lmax, a.max_blocks << a.log2_block));
    if (MODE == KV_PACKED) L = min(L, a.lmax);
    if (MODE == KV_RING) L = min(L, kMaxPosition);
    L = max(L, 0);
    GQA_FLAG(L != L0, kDbgSeqlensK);
    s.kv_len = L;
  } else {
    s.kv_len = a.kv_len_fixed;
  }
  // queries are the newest positions; never more queries than positions
  GQA_FLAG(s.q_len > s.kv_len, kDbgQLen);
  if (s.q_len > s.kv_len) s.q_len = s.kv_len;
  return s;
}

// KV_RING: the row of key position j, >= 0 in the ring, or -1 - r for row r of the chunk.
__device__ __forceinline__ int64_t ring_chunk_row(const SeqArgs& a, const SeqView& s, int j) {
  const int j0 = s.kv_len - s.q_len;
  if (j >= j0) return -1 - (s.q_row0 + (j - j0));
  return (int64_t)s.b * a.lmax + j % a.lmax;
}

template <int MODE>
__device__ __forceinline__ int64_t kv_row(const SeqArgs& a, const SeqView& s, int j) {
  if (MODE == KV_BATCHED) {
    return (int64_t)s.b * a.lmax + j;
  } else if (MODE == KV_PAGED) {
    const int blk0 = a.block_table[(int64_t)s.b * a.max_blocks + (j >> a.log2_block)];
    const int blk = min(max(blk0, 0), a.num_blocks - 1);
    GQA_FLAG(blk != blk0, kDbgBlockTable);
    return ((int64_t)blk << a.log2_block) + (j & ((1 << a.log2_block) - 1));
  } else {
    const int64_t r0 = (int64_t)a.cu_seqlens_k[s.b] + j;
    int64_t r = r0 < 0 ? 0 : r0;
    r = r < a.num_blocks ? r : (int64_t)a.num_blocks - 1;
    GQA_FLAG(r != r0, kDbgPackedRow);
    return r;
  }
}

// ---------------------------------------------------------------------------
// small helpers

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// two fp32 -> packed bf16x2 (round to nearest even; v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// rotary position encoding («GPT-OSS-20B : Architecture MoE & Résumé du Model
// Card» §3.4): position m turns pair i of a head by the angle m·θ_i

// The default frequency θ_i = 10000^(-2i/d), formed in fp64 and rounded once to
// fp32 (for d = 64 every θ_i lies at least 3e-10 of its size away from an fp32
// rounding boundary, far beyond the fp64 error, so this is the correctly
// rounded fp32 value).  The arguments of every power are constants, so the
// compiler forms the 32 values once, at build time, and a lane selects its own
// (a chain of selects instead of an fp64 power per lane).
__device__ __forceinline__ float rope_default_freq(int i) {
  float f = 0.f;
#pragma unroll
  for (int j = 0; j < kHeadDim / 2; ++j)
    if (i == j) f = (float)__builtin_pow(10000.0, -2.0 * j / kHeadDim);
  return f;
}

// cos and sin (times mscale) of the angle p·f: the angle is formed in fp64 as a
// number of turns (the product of an integer position and an fp32 frequency is
// exact there) and reduced to [-1/2, 1/2] before the hardware sine and cosine,
// which take turns, so positions up to the 131 072-token context keep full
// accuracy.
__device__ __forceinline__ void rope_cos_sin(int p, float f, float mscale, float& cs, float& sn) {
  const double turns = (double)p * (double)f * 0.15915494309189535;  // 1 / (2 pi)
  const float r = (float)(turns - __builtin_rint(turns));
  cs = __builtin_amdgcn_cosf(r) * mscale;
  sn = __builtin_amdgcn_sinf(r) * mscale;
}

// One rotated pair: (a, b) -> (a cos - b sin, a sin + b cos).
__device__ __forceinline__ void rope_rotate(float a, float b, float cs, float sn, float& ra, float& rb) {
  ra = __builtin_fmaf(a, cs, -b * sn);
  rb = __builtin_fmaf(a, sn, b * cs);
}

// Make this wave's LDS writes visible to its other lanes (and order later
// writes after earlier reads): a wavefront-scope release/acquire pair around a
// wave barrier.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace gqa
