// Rotary position encoding of new tokens, fused with their KV-cache append.
//
// «GPT-OSS-20B : Architecture MoE & Résumé du Model Card», §3.4: a token at
// position m is rotated with the frequencies θ_i = 10000^(-2i/d); «GPT-OSS vs
// Qwen3», "Adoption de RoPE": the query and key vectors are turned by an angle
// that depends on the position.  Pair i of a head, (a, b), becomes
// (a cos - b sin, a sin + b cos) at angle m·inv_freq[i]; the pairs are
// (2i, 2i+1) or (i, i + d/2).  The frequency table is an input; without one
// the kernel forms θ_i itself.  `mscale` scales cos and sin alike.
//
// One pass over the new rows: the queries are rotated into q_out (which may
// be q itself), the keys are rotated and written with the values into the
// cache slot of their position (contiguous, paged or ring cache).  The angle
// m·inv_freq[i] is formed in fp64, where the product of an integer position
// and an fp32 frequency is exact, and reduced to a fraction of a turn there,
// so positions up to the 131 072-token context keep full accuracy; sin, cos
// (the hardware instructions) and the rotation itself are fp32.
//
// One wave per new row, 8 lanes per head: lane c = lane % 8 of a head owns the
// pairs 4c .. 4c+3 and moves 16 contiguous bytes of them per load; cos and sin
// of its 4 pairs are computed once per row and reused for every head.
#include "kernels.h"

namespace gqa {
namespace {

constexpr int RP_THREADS = 256;  // 4 waves, one row each

template <typename T>
struct Elt;
template <>
struct Elt<__bf16> {
  static __device__ __forceinline__ float get(const __bf16* p, int i) { return (float)p[i]; }
  static __device__ __forceinline__ void put(__bf16* p, int i, float v) { p[i] = (__bf16)v; }
};
template <>
struct Elt<float> {
  static __device__ __forceinline__ float get(const float* p, int i) { return p[i]; }
  static __device__ __forceinline__ void put(float* p, int i, float v) { p[i] = v; }
};

// Copy of n elements through 16-byte words (n * sizeof(T) is a multiple of 16).
template <typename T, int N>
__device__ __forceinline__ void load_n(T (&dst)[N], const T* src) {
  static_assert((N * sizeof(T)) % 8 == 0, "whole 8-byte words");
  if constexpr ((N * sizeof(T)) % 16 == 0) {
    typedef uint32_t w4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int i = 0; i < (int)(N * sizeof(T) / 16); ++i)
      reinterpret_cast<w4*>(dst)[i] = reinterpret_cast<const w4*>(src)[i];
  } else {
    typedef uint32_t w2 __attribute__((ext_vector_type(2)));
    reinterpret_cast<w2*>(dst)[0] = reinterpret_cast<const w2*>(src)[0];
  }
}
template <typename T, int N>
__device__ __forceinline__ void store_n(T* dst, const T (&src)[N]) {
  if constexpr ((N * sizeof(T)) % 16 == 0) {
    typedef uint32_t w4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int i = 0; i < (int)(N * sizeof(T) / 16); ++i)
      reinterpret_cast<w4*>(dst)[i] = reinterpret_cast<const w4*>(src)[i];
  } else {
    typedef uint32_t w2 __attribute__((ext_vector_type(2)));
    reinterpret_cast<w2*>(dst)[0] = reinterpret_cast<const w2*>(src)[0];
  }
}

// This lane's 4 pairs of up to NH heads (heads h0, h0 + 8, ...), held in
// registers between the loads and the rotation, so that a wave can issue the
// loads of a whole row (queries, keys, values) before any of its math.
template <typename T, int PAIRING, int NH>
struct HeadPairs {
  static constexpr int NX = PAIRING == 0 ? 8 : 4;  // (2i, 2i+1): 8 contiguous elements; (i, i+32): 4 and 4
  T x[NH][NX];
  T y[NH][PAIRING == 0 ? 1 : 4];

  __device__ __forceinline__ void load(const T* src, int h0, int nh, int c) {
#pragma unroll
    for (int u = 0; u < NH; ++u) {
      if (u >= nh) continue;
      if constexpr (PAIRING == 0) {
        load_n<T, 8>(x[u], src + (h0 + 8 * u) * kHeadDim + 8 * c);
      } else {
        load_n<T, 4>(x[u], src + (h0 + 8 * u) * kHeadDim + 4 * c);
        load_n<T, 4>(y[u], src + (h0 + 8 * u) * kHeadDim + 32 + 4 * c);
      }
    }
  }

  // Rotate and store.  dst may be the source (every element was read before).
  __device__ __forceinline__ void rotate_store(T* dst, int h0, int nh, int c, const float (&cs)[4],
                                               const float (&sn)[4]) {
#pragma unroll
    for (int u = 0; u < NH; ++u) {
      if (u >= nh) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float ra, rb;
        if constexpr (PAIRING == 0) {
          rope_rotate(Elt<T>::get(x[u], 2 * j), Elt<T>::get(x[u], 2 * j + 1), cs[j], sn[j], ra, rb);
          Elt<T>::put(x[u], 2 * j, ra);
          Elt<T>::put(x[u], 2 * j + 1, rb);
        } else {
          rope_rotate(Elt<T>::get(x[u], j), Elt<T>::get(y[u], j), cs[j], sn[j], ra, rb);
          Elt<T>::put(x[u], j, ra);
          Elt<T>::put(y[u], j, rb);
        }
      }
      if constexpr (PAIRING == 0) {
        store_n<T, 8>(dst + (h0 + 8 * u) * kHeadDim + 8 * c, x[u]);
      } else {
        store_n<T, 4>(dst + (h0 + 8 * u) * kHeadDim + 4 * c, x[u]);
        store_n<T, 4>(dst + (h0 + 8 * u) * kHeadDim + 32 + 4 * c, y[u]);
      }
    }
  }
};

template <typename T, int PAIRING>
__global__ __launch_bounds__(RP_THREADS) void rope_append_kernel(RopeAppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (RP_THREADS / 64) + (threadIdx.x >> 6);
  if (row >= a.T) return;
  const int c = lane & 7;   // lane within its head group: pairs 4c .. 4c+3
  const int hg = lane >> 3; // head group: heads hg, hg + 8, ...

  // The sources are indexed by the row alone: the loads of its first 64
  // query heads, its first 64 key heads and its first value words go out
  // before the row's position is looked up and its angles formed, so the wave
  // waits for memory once (more heads than 64 follow in later batches).
  const int64_t kv_row = (int64_t)a.Hkv * kHeadDim;
  const T* q = a.q ? reinterpret_cast<const T*>(a.q) + row * a.Hq * kHeadDim : nullptr;
  const T* k = reinterpret_cast<const T*>(a.k) + row * kv_row;
  typedef uint32_t w4 __attribute__((ext_vector_type(4)));
  const w4* vs = reinterpret_cast<const w4*>(reinterpret_cast<const T*>(a.v) + row * kv_row);
  const int words = (int)(kv_row * sizeof(T) / 16);
  HeadPairs<T, PAIRING, 8> qp, kp;
  if (q && hg < a.Hq) qp.load(q, hg, (a.Hq - hg + 7) / 8 < 8 ? (a.Hq - hg + 7) / 8 : 8, c);
  if (hg < a.Hkv) kp.load(k, hg, (a.Hkv - hg + 7) / 8 < 8 ? (a.Hkv - hg + 7) / 8 : 8, c);
  w4 v0 = {0u, 0u, 0u, 0u};
  if (lane < words) v0 = vs[lane];

  // sequence and position of this row (the newest q_len positions of its sequence)
  int b, t, q_len;
  if (a.cu_seqlens_q) {
    if (row >= a.cu_seqlens_q[a.B]) return;
    int lo = 0, hi = a.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.cu_seqlens_q[mid] <= row) lo = mid;
      else hi = mid - 1;
    }
    b = lo;
    q_len = a.cu_seqlens_q[b + 1] - a.cu_seqlens_q[b];
    t = (int)(row - a.cu_seqlens_q[b]);
    if (t < 0 || t >= q_len) return;
  } else {
    b = (int)row;
    t = 0;
    q_len = 1;
  }
  const int L = a.seqlens[b];
  const int p = L - q_len + t;

  float cs[4], sn[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    rope_cos_sin(p, a.inv_freq ? a.inv_freq[4 * c + j] : rope_default_freq(4 * c + j), a.mscale, cs[j], sn[j]);

  // queries (NULL: keys only, the attention rotates its queries itself)
  if (q) {
    T* qo = reinterpret_cast<T*>(a.q_out) + row * a.Hq * kHeadDim;
    if (hg < a.Hq) qp.rotate_store(qo, hg, (a.Hq - hg + 7) / 8 < 8 ? (a.Hq - hg + 7) / 8 : 8, c, cs, sn);
    for (int h0 = hg + 64; h0 < a.Hq; h0 += 64) {
      HeadPairs<T, PAIRING, 8> more;
      more.load(q, h0, (a.Hq - h0 + 7) / 8, c);
      more.rotate_store(qo, h0, (a.Hq - h0 + 7) / 8, c, cs, sn);
    }
  }

  // destination row of this position in the cache (or none)
  int64_t dst = -1;
  if (p >= 0) {
    if (a.cache_kind == 0) {
      if (p < a.cache_len) dst = (int64_t)b * a.cache_len + p;
    } else if (a.cache_kind == 1) {
      const int nb = p >> a.log2_block;
      if (nb < a.max_blocks) {
        int blk = a.block_table[(int64_t)b * a.max_blocks + nb];
        GQA_FLAG(blk < 0 || blk >= a.num_blocks, kDbgBlockTable);
        blk = min(max(blk, 0), a.num_blocks - 1);
        dst = ((int64_t)blk << a.log2_block) + (p & ((1 << a.log2_block) - 1));
      }
    } else {
      if (p >= L - a.cache_len) dst = (int64_t)b * a.cache_len + p % a.cache_len;
    }
  }
  if (dst < 0) return;
  T* kc = reinterpret_cast<T*>(a.k_cache) + dst * kv_row;
  if (hg < a.Hkv) kp.rotate_store(kc, hg, (a.Hkv - hg + 7) / 8 < 8 ? (a.Hkv - hg + 7) / 8 : 8, c, cs, sn);
  for (int h0 = hg + 64; h0 < a.Hkv; h0 += 64) {
    HeadPairs<T, PAIRING, 8> more;
    more.load(k, h0, (a.Hkv - h0 + 7) / 8, c);
    more.rotate_store(kc, h0, (a.Hkv - h0 + 7) / 8, c, cs, sn);
  }
  // values: copied as 16-byte words
  w4* vd = reinterpret_cast<w4*>(reinterpret_cast<T*>(a.v_cache) + dst * kv_row);
  if (lane < words) vd[lane] = v0;
  for (int i = lane + 64; i < words; i += 64) vd[i] = vs[i];
}

}  // namespace

hipError_t launch_rope_append(const RopeAppendArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const int64_t blocks = (a.T + RP_THREADS / 64 - 1) / (RP_THREADS / 64);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
#define GQA_ROPE(TY, PR) hipLaunchKernelGGL((rope_append_kernel<TY, PR>), dim3((unsigned)blocks), dim3(RP_THREADS), 0, s, a)
  if (a.fp32) {
    if (a.pairing == 0) GQA_ROPE(float, 0);
    else GQA_ROPE(float, 1);
  } else {
    if (a.pairing == 0) GQA_ROPE(__bf16, 0);
    else GQA_ROPE(__bf16, 1);
  }
#undef GQA_ROPE
  return hipGetLastError();
}

// Metadata-check flags of this file's kernels (recorded only when built with GQA_DEBUG).
GQA_DEBUG_FLAGS_ACCESSOR(debug_flags_rope)

}  // namespace gqa
