// One decode step of a layer in one launch: the rotary encoding of the new
// token's query and key («GPT-OSS-20B : Architecture MoE & Résumé du Model
// Card» §3.4; «GPT-OSS vs Qwen3», "Adoption de RoPE"), the append of its
// rotated key and its value to the KV cache, and the attention of its query
// over the cached keys -- causal GQA with the per-head sink logit in the
// softmax denominator, on a dense layer or a sliding-window one, optionally
// keeping start-of-sequence sink tokens visible («GPT-OSS vs Qwen3», sections
// "Introduction de Grouped Query Attention", "Utilisation de Sliding Window
// Attention", "Attention Bias et Sinks").
//
// It computes exactly what the rotary append followed by the decode computes:
// the rotation is the shared one of common.h, rounded to bf16 as the append
// stores it, and the attention sees the bf16 rotated query and key.
//
// A workgroup owns one (sequence, KV head): it rotates the query heads of that
// KV head and the new key row, writes the key and value rows to the cache slot
// of the new position (no other workgroup touches that slot), and attends over
// the key range, taking the new position's row from its own LDS copy, so
// nothing in the launch waits for another workgroup's write.  The attention is
// the decode kernels' matrix-core form: the 4 waves take interleaved 32-key
// tiles of the key range (a window of 128 keys: one tile each), stage each
// tile's K and V rows in their own LDS slice, compute S^T = K Q^T on
// v_mfma_f32_16x16x32_bf16 (the query heads as the 16 columns) and
// O^T += V^T P^T with V^T through the transposing LDS read, each with its own
// online softmax; the 4 states are merged in LDS, where the sink enters.
#include "kernels.h"

namespace gqa {
namespace {

constexpr int ST_THREADS = 256;  // 4 waves
constexpr int TK = 32;           // keys per wave tile
constexpr int KSD = 72;          // LDS row stride (elements) of a wave's K tile [key][d]
constexpr int VSD = 80;          // LDS row stride (elements) of a wave's V tile [key][d]
constexpr int WAVE_LDS = TK * KSD + TK * VSD;  // elements per wave

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int KIND>
__device__ __forceinline__ int64_t step_row(const DecodeStepArgs& a, int b, int pos) {
  if (KIND == STEP_CACHE_CONTIGUOUS) return (int64_t)b * a.cache_len + pos;
  if (KIND == STEP_CACHE_RING) return (int64_t)b * a.cache_len + pos % a.cache_len;
  const int blk0 = a.block_table[(int64_t)b * a.max_blocks + (pos >> a.log2_block)];
  const int blk = min(max(blk0, 0), a.num_blocks - 1);
  GQA_FLAG(blk != blk0, kDbgBlockTable);
  return ((int64_t)blk << a.log2_block) + (pos & ((1 << a.log2_block) - 1));
}

template <int KIND>
__global__ __launch_bounds__(ST_THREADS) void decode_step_kernel(DecodeStepArgs a) {
  // per wave: K tile then V tile; after the key loop the same memory holds the merge buffers
  __shared__ __attribute__((aligned(16))) __bf16 lds[4 * WAVE_LDS];
  __shared__ __attribute__((aligned(16))) __bf16 kn_s[kHeadDim];  // the new key row, rotated
  __shared__ __attribute__((aligned(16))) __bf16 vn_s[kHeadDim];  // the new value row

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int lc = lane & 15;  // head column (and key row of the K operand)
  const int lq = lane >> 4;  // lane quarter
  const int b = blockIdx.x / a.Hkv;
  const int g = blockIdx.x % a.Hkv;
  const int G = a.G;

  // The new rows do not depend on the sequence length: they are requested
  // first, beside it.  Every wave loads the Q^T operand (head lc, d = 32 ks +
  // 8 lq .. +7); threads 0..31 take pair t of the new key, threads 64..127 one
  // element of the new value.
  const int64_t qrow = ((int64_t)b * a.Hq + g * G + lc) * kHeadDim;
  u32x4 qw[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
  if (lc < G) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) qw[ks] = *reinterpret_cast<const u32x4*>(a.q + qrow + 32 * ks + 8 * lq);
  }
  const int ri = t & 31;
  const int ia = a.pairing ? ri : 2 * ri, ib = a.pairing ? ri + kHeadDim / 2 : 2 * ri + 1;
  const int64_t ko = ((int64_t)b * a.Hkv + g) * kHeadDim;
  float ka = 0.f, kb = 0.f;
  __bf16 vv = (__bf16)0.f;
  if (t < kHeadDim / 2) {
    ka = (float)a.k_new[ko + ia];
    kb = (float)a.k_new[ko + ib];
  } else if (t >= 64 && t < 64 + kHeadDim) {
    vv = a.v_new[ko + t - 64];
  }

  // the sequence's length counts the new token; the cache bounds it
  const int L0 = a.seqlens[b];
  int L = max(L0, 1);
  if (KIND == STEP_CACHE_CONTIGUOUS) L = min(L, a.cache_len);
  if (KIND == STEP_CACHE_PAGED) L = min(L, a.max_blocks << a.log2_block);
  GQA_FLAG(L != L0, kDbgSeqlensK);
  const int p = L - 1;  // position of the new token

  // ---- keys: the sink tokens below the window, then the window, numbered by a
  // virtual index v in [0, nv): position v for v < ns, lo + v - ns after
  const int W = a.window;
  const int lo = W > 0 ? max(0, L - W) : 0;
  const int ns = W > 0 ? min(a.sink_tokens, lo) : 0;
  const int nv = ns + (L - lo);
  auto pos_of = [&](int v) { return v < ns ? v : lo + (v - ns); };

  // A wave's tile: load i brings key 8 i + lane / 8 of the tile, 16 bytes at
  // d = 8 (lane % 8); rows past the range repeat its last key (masked below,
  // always in bounds), the new position's row is not read (it comes from LDS).
  // The first tile is requested before the rotation work, so its latency
  // overlaps it.
  const int piece = lane & 7;
  u32x4 kreg[4], vreg[4];
  auto request = [&](int v0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pos = pos_of(min(v0 + 8 * i + (lane >> 3), nv - 1));
      kreg[i] = u32x4{0u, 0u, 0u, 0u};
      vreg[i] = u32x4{0u, 0u, 0u, 0u};
      if (pos != p) {
        const int64_t off = (step_row<KIND>(a, b, pos) * a.Hkv + g) * kHeadDim + 8 * piece;
        kreg[i] = *reinterpret_cast<const u32x4*>(a.k_cache + off);
        vreg[i] = *reinterpret_cast<const u32x4*>(a.v_cache + off);
      }
    }
  };
  int v0 = wave * TK;
  if (v0 < nv) request(v0);

  // ---- rotate: the lane's query operand (8 pairs of head lc) and, for threads
  // 0..31, pair t of the new key; every thread forms the cos and sin it needs
  bf16x8 qb[2];
  {
    const float ms = a.mscale;
    if (a.pairing == 0) {
      // pairs (2i, 2i+1): element pairs (2e', 2e'+1) of qw[ks], i = 16 ks + 4 lq + e'
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * ks + 4 * lq + e;
          float cs, sn, ra, rb;
          rope_cos_sin(p, a.inv_freq ? a.inv_freq[i] : rope_default_freq(i), ms, cs, sn);
          rope_rotate(bf16_lo(qw[ks][e]), bf16_hi(qw[ks][e]), cs, sn, ra, rb);
          qw[ks][e] = pack_bf16x2(ra, rb);
        }
      }
    } else {
      // pairs (i, i + 32): element e of qw[0] with element e of qw[1], i = 8 lq + e
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        float r0[2], r1[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int i = 8 * lq + 2 * e2 + h;
          float cs, sn;
          rope_cos_sin(p, a.inv_freq ? a.inv_freq[i] : rope_default_freq(i), ms, cs, sn);
          const float xa = h ? bf16_hi(qw[0][e2]) : bf16_lo(qw[0][e2]);
          const float xb = h ? bf16_hi(qw[1][e2]) : bf16_lo(qw[1][e2]);
          rope_rotate(xa, xb, cs, sn, r0[h], r1[h]);
        }
        qw[0][e2] = pack_bf16x2(r0[0], r0[1]);
        qw[1][e2] = pack_bf16x2(r1[0], r1[1]);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) qb[ks] = __builtin_bit_cast(bf16x8, qw[ks]);
    if (a.q_out && wave == 0 && lc < G) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) *reinterpret_cast<u32x4*>(a.q_out + qrow + 32 * ks + 8 * lq) = qw[ks];
    }
    if (t < kHeadDim / 2) {
      float cs, sn, ra, rb;
      rope_cos_sin(p, a.inv_freq ? a.inv_freq[ri] : rope_default_freq(ri), ms, cs, sn);
      rope_rotate(ka, kb, cs, sn, ra, rb);
      kn_s[ia] = (__bf16)ra;
      kn_s[ib] = (__bf16)rb;
    } else if (t >= 64 && t < 64 + kHeadDim) {
      vn_s[t - 64] = vv;
    }
  }
  __syncthreads();
  // ---- append: the new key and value rows to the cache slot of position p (16-byte words)
  if (t < 16) {
    const int64_t row = step_row<KIND>(a, b, p);
    const u32x4 w = t < 8 ? *reinterpret_cast<const u32x4*>(kn_s + 8 * (t & 7))
                          : *reinterpret_cast<const u32x4*>(vn_s + 8 * (t & 7));
    __bf16* dst = (t < 8 ? a.k_cache : a.v_cache) + (row * a.Hkv + g) * kHeadDim + 8 * (t & 7);
    *reinterpret_cast<u32x4*>(dst) = w;
  }

  // ---- attention over the wave's tiles
  const float c = a.scale_log2;
  __bf16* Kw = lds + wave * WAVE_LDS;
  __bf16* Vw = Kw + TK * KSD;
  const int vofs = (4 * lq + ((lane & 15) >> 2)) * VSD + 4 * (lane & 3);
  float m_run = kNegBig, l_run = 0.f;
  f32x4 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (; v0 < nv; v0 += 4 * TK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = 8 * i + (lane >> 3);
      const int pos = pos_of(min(v0 + key, nv - 1));
      u32x4 kw = kreg[i], vw = vreg[i];
      if (pos == p) {
        kw = *reinterpret_cast<const u32x4*>(kn_s + 8 * piece);
        vw = *reinterpret_cast<const u32x4*>(vn_s + 8 * piece);
      }
      *reinterpret_cast<u32x4*>(Kw + key * KSD + 8 * piece) = kw;
      *reinterpret_cast<u32x4*>(Vw + key * VSD + 8 * piece) = vw;
    }
    wave_lds_sync();  // the tile is visible to every lane of the wave
    if (v0 + 4 * TK < nv) request(v0 + 4 * TK);  // the wave's next tile flies during this one's math

    // S^T: 2 blocks of 16 keys x 16 heads; A operand = K rows 16 kb + lc, d 32 ks + 8 lq
    f32x4 sc[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 kop = *reinterpret_cast<const bf16x8*>(Kw + (16 * kb2 + lc) * KSD + 32 * ks + 8 * lq);
        acc = mfma16(kop, qb[ks], acc);
      }
      sc[kb2] = acc;
    }
    // lane holds keys v0 + 16 kb + 4 lq + r of head lc
    if (v0 + TK > nv) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (v0 + 16 * kb2 + 4 * lq + r >= nv) sc[kb2][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[kb2][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pw = fast_exp2(__builtin_fmaf(sc[kb2][r], c, -m_new));
        sc[kb2][r] = pw;
        rs += pw;
      }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
    // O^T += V^T P^T over the tile's 32 keys: keys {4lq..4lq+3, 16+4lq..16+4lq+3};
    // in lane group lq, lane j reads 4 d of key row 4lq + j/4; the hardware hands
    // lane i the 4 keys at d = 16 dt + i
    bf16x8 pbv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pbv[e] = (__bf16)sc[0][e];
      pbv[4 + e] = (__bf16)sc[1][e];
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const __bf16* base = Vw + vofs + 16 * dt;
      const i16x4 vlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base));
      const i16x4 vhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 16 * VSD));
      const i16x8 vw8 = {vlo[0], vlo[1], vlo[2], vlo[3], vhi[0], vhi[1], vhi[2], vhi[3]};
      o[dt] = mfma16(__builtin_bit_cast(bf16x8, vw8), pbv, o[dt]);
    }
    wave_lds_sync();  // all lanes done reading the tile before the next overwrite
  }

  // ---- merge the 4 waves: per head max, sum and output; then the sink, out = o / l, lse
  __syncthreads();  // every wave is out of its key loop: the tile memory becomes the merge buffers
  float* red_m = reinterpret_cast<float*>(lds);  // [4][16]
  float* red_l = red_m + 64;                    // [4][16]
  float* red_o = red_l + 64;                    // [4][16][68]
  {
    float lt = l_run + __shfl_xor(l_run, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    if (lq == 0) {
      red_m[wave * 16 + lc] = m_run;
      red_l[wave * 16 + lc] = lt;
    }
    // lane holds O^T[d = 16 dt + 4 lq + r][head lc]
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) red_o[(wave * 16 + lc) * 68 + 16 * dt + 4 * lq + r] = o[dt][r];
  }
  __syncthreads();
  const int hh = t >> 4;        // head of this KV head
  const int d0 = (t & 15) * 4;  // 4 output columns
  if (hh < G) {
    float M = red_m[hh];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, red_m[w * 16 + hh]);
    float wsc[4];
    float lsum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wsc[w] = fast_exp2(red_m[w * 16 + hh] - M);
      lsum += red_l[w * 16 + hh] * wsc[w];
    }
    float acc[4];
#pragma unroll
    for (int cq = 0; cq < 4; ++cq) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) sum += red_o[(w * 16 + hh) * 68 + d0 + cq] * wsc[w];
      acc[cq] = sum;
    }
    const int hq = g * G + hh;
    const float s2 = a.sinks ? a.sinks[hq] * kLog2e : -INFINITY;
    const float Mf = fmaxf(M, s2);
    const float scl = fast_exp2(M - Mf);
    const float Z = fast_exp2(s2 - Mf) + lsum * scl;
    const float inv = Z > 0.f ? scl / Z : (Z == 0.f ? 0.f : Z);
    u32x2 w2;
    w2[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    w2[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<u32x2*>(a.out + ((int64_t)b * a.Hq + hq) * kHeadDim + d0) = w2;
    if (a.lse && d0 == 0) a.lse[(int64_t)b * a.Hq + hq] = (Z == 0.f) ? -INFINITY : (Mf + __log2f(Z)) * kLn2;
  }
}

}  // namespace

hipError_t launch_decode_step(const DecodeStepArgs& a, hipStream_t s) {
  const int64_t grid = (int64_t)a.B * a.Hkv;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff || a.G > kStepMaxG) return hipErrorInvalidValue;
  if (a.cache_kind == STEP_CACHE_CONTIGUOUS)
    hipLaunchKernelGGL(decode_step_kernel<STEP_CACHE_CONTIGUOUS>, dim3((unsigned)grid), dim3(ST_THREADS), 0, s, a);
  else if (a.cache_kind == STEP_CACHE_PAGED)
    hipLaunchKernelGGL(decode_step_kernel<STEP_CACHE_PAGED>, dim3((unsigned)grid), dim3(ST_THREADS), 0, s, a);
  else if (a.cache_kind == STEP_CACHE_RING)
    hipLaunchKernelGGL(decode_step_kernel<STEP_CACHE_RING>, dim3((unsigned)grid), dim3(ST_THREADS), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// Metadata-check flags of this file's kernels (recorded only when built with GQA_DEBUG).
GQA_DEBUG_FLAGS_ACCESSOR(debug_flags_step)

}  // namespace gqa
