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
// nothing in the launch waits for another workgroup's write.  The key range
// (the window, or the whole sequence on a dense layer with a short cache) is
// staged through LDS in chunks of 128 keys; each half-wave owns one query
// head (its rotated query in registers, four keys per lane, the online softmax
// within the half-wave, two output columns per lane).  Scores and P V are
// plain fp32 vector arithmetic: the step is bound by its K/V bytes and its
// launch, not by arithmetic.
#include "kernels.h"

namespace gqa {
namespace {

constexpr int ST_THREADS = 256;
constexpr int ST_CHUNK = 128;  // keys staged in LDS at a time
constexpr int ST_RS = 72;      // LDS row stride of a staged K/V row (bf16): 144 bytes spreads the rows' banks

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
  __shared__ float q_s[kStepMaxG][kHeadDim];  // rotated queries (their bf16 values)
  __shared__ __attribute__((aligned(16))) __bf16 kn_s[kHeadDim];  // the new key row, rotated
  __shared__ __attribute__((aligned(16))) __bf16 vn_s[kHeadDim];  // the new value row
  __shared__ __attribute__((aligned(16))) __bf16 k_s[ST_CHUNK * ST_RS];
  __shared__ __attribute__((aligned(16))) __bf16 v_s[ST_CHUNK * ST_RS];
  __shared__ __attribute__((aligned(16))) float p_s[kStepMaxG][ST_CHUNK];  // weights of the chunk

  const int t = threadIdx.x;
  const int b = blockIdx.x / a.Hkv;
  const int g = blockIdx.x % a.Hkv;
  const int G = a.G;

  // The new rows do not depend on the sequence length: they are requested
  // first, beside it.  Thread t takes pair i = t % 32 of query head t / 32 of
  // this KV head; threads 0..31 also pair t of the key, threads 64..127 one
  // element of the value.
  const int rh = t >> 5, ri = t & 31;
  const int ia = a.pairing ? ri : 2 * ri, ib = a.pairing ? ri + kHeadDim / 2 : 2 * ri + 1;
  const int64_t qo = ((int64_t)b * a.Hq + g * G + rh) * kHeadDim;
  const int64_t ko = ((int64_t)b * a.Hkv + g) * kHeadDim;
  float qa = 0.f, qb = 0.f, ka = 0.f, kb = 0.f;
  __bf16 vv = (__bf16)0.f;
  if (rh < G) {
    qa = (float)a.q[qo + ia];
    qb = (float)a.q[qo + ib];
  }
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

  // The chunk's K and V rows go through registers: thread t moves 16-byte
  // piece t % 8 of rows t / 8 + 32 r (r < 4).  The first chunk is requested
  // before the rotation work, so its latency overlaps it; the new position's
  // row is filled in from LDS once it is rotated.
  static_assert(ST_CHUNK * 8 == 4 * ST_THREADS, "four 16-byte pieces of K and of V per thread and chunk");
  u32x4 kreg[4], vreg[4];
  auto request = [&](int c0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = (t >> 3) + 32 * r, piece = t & 7;
      kreg[r] = u32x4{0u, 0u, 0u, 0u};
      vreg[r] = u32x4{0u, 0u, 0u, 0u};
      const int v = c0 + j;
      const int pos = v < ns ? v : lo + (v - ns);
      if (v < nv && pos != p) {
        const int64_t off = (step_row<KIND>(a, b, pos) * a.Hkv + g) * kHeadDim + 8 * piece;
        kreg[r] = *reinterpret_cast<const u32x4*>(a.k_cache + off);
        vreg[r] = *reinterpret_cast<const u32x4*>(a.v_cache + off);
      }
    }
  };
  auto stage = [&](int c0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = (t >> 3) + 32 * r, piece = t & 7;
      const int v = c0 + j;
      const int pos = v < ns ? v : lo + (v - ns);
      u32x4 kw = kreg[r], vw = vreg[r];
      if (v < nv && pos == p) {
        kw = *reinterpret_cast<const u32x4*>(kn_s + 8 * piece);
        vw = *reinterpret_cast<const u32x4*>(vn_s + 8 * piece);
      }
      *reinterpret_cast<u32x4*>(k_s + j * ST_RS + 8 * piece) = kw;
      *reinterpret_cast<u32x4*>(v_s + j * ST_RS + 8 * piece) = vw;
    }
  };
  request(0);

  // ---- rotate (every thread forms the cos and sin of its own pair's angle)
  {
    float cs, sn;
    rope_cos_sin(p, a.inv_freq ? a.inv_freq[ri] : rope_default_freq(ri), a.mscale, cs, sn);
    float ra, rb;
    if (rh < G) {
      rope_rotate(qa, qb, cs, sn, ra, rb);
      const __bf16 ba = (__bf16)ra, bb = (__bf16)rb;
      q_s[rh][ia] = (float)ba;
      q_s[rh][ib] = (float)bb;
      if (a.q_out) {
        a.q_out[qo + ia] = ba;
        a.q_out[qo + ib] = bb;
      }
    }
    if (t < kHeadDim / 2) {
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
    const int piece = t & 7;
    const u32x4 w = t < 8 ? *reinterpret_cast<const u32x4*>(kn_s + 8 * piece)
                          : *reinterpret_cast<const u32x4*>(vn_s + 8 * piece);
    __bf16* dst = (t < 8 ? a.k_cache : a.v_cache) + (row * a.Hkv + g) * kHeadDim + 8 * piece;
    *reinterpret_cast<u32x4*>(dst) = w;
  }

  const float c = a.scale_log2;

  // Half-wave hw = t / 32 owns query head hw of this KV head: its rotated
  // query in registers, its running max and sum (log2 units, the sink as the
  // starting reference: its own term is 1), two output columns per lane.
  const int hh = t >> 5, jj = t & 31;
  const bool live = hh < G;
  float qr[kHeadDim];
#pragma unroll
  for (int e = 0; e < kHeadDim; ++e) qr[e] = live ? q_s[hh][e] : 0.f;
  const float s2 = (a.sinks && live) ? a.sinks[g * G + hh] * kLog2e : -INFINITY;
  float m_run = s2 == -INFINITY ? kNegBig : s2;
  float l_run = s2 == -INFINITY ? 0.f : 1.f;
  float o0 = 0.f, o1 = 0.f;  // output columns 2 jj, 2 jj + 1
  for (int c0 = 0; c0 < nv; c0 += ST_CHUNK) {
    const int nc = min(ST_CHUNK, nv - c0);
    stage(c0);  // the chunk's rows (requested earlier) into LDS, the new position's from its LDS copy
    if (c0 + ST_CHUNK < nv) request(c0 + ST_CHUNK);  // the next chunk flies during this one
    __syncthreads();
    // scores of keys jj + 32 i (i < 4): a half-wave reads 32 consecutive rows at once
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = jj + 32 * i;
      float acc = 0.f;
#pragma unroll
      for (int d8 = 0; d8 < 8; ++d8) {
        const u32x4 kw = *reinterpret_cast<const u32x4*>(k_s + j * ST_RS + 8 * d8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc = __builtin_fmaf(qr[8 * d8 + 2 * e], bf16_lo(kw[e]), acc);
          acc = __builtin_fmaf(qr[8 * d8 + 2 * e + 1], bf16_hi(kw[e]), acc);
        }
      }
      x[i] = (j < nc && live) ? acc * c : -INFINITY;
    }
    // online softmax over the chunk, within the half-wave
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    const float m_new = fmaxf(m_run, mx);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = fast_exp2(x[i] - m_new);
      sum += x[i];
      p_s[hh][jj + 32 * i] = x[i];
    }
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 64);
    const float al = fast_exp2(m_run - m_new);
    l_run = l_run * al + sum;
    m_run = m_new;
    wave_lds_sync();  // the half-wave's weights are visible to its own lanes
    // P V: columns 2 jj, 2 jj + 1 over the chunk's keys, 4 keys per step
    o0 *= al;
    o1 *= al;
    for (int j = 0; j < nc; j += 4) {
      const f32x4 pw = *reinterpret_cast<const f32x4*>(&p_s[hh][j]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t vw = *reinterpret_cast<const uint32_t*>(v_s + (j + i) * ST_RS + 2 * jj);
        o0 = __builtin_fmaf(pw[i], bf16_lo(vw), o0);
        o1 = __builtin_fmaf(pw[i], bf16_hi(vw), o1);
      }
    }
    __syncthreads();  // every wave is done with the chunk before the next is staged
  }

  // ---- out = o / l (the sink's term is in l), lse = m + ln l
  if (live) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const int64_t oo = ((int64_t)b * a.Hq + g * G + hh) * kHeadDim;
    *reinterpret_cast<uint32_t*>(a.out + oo + 2 * jj) = pack_bf16x2(o0 * inv, o1 * inv);
    if (a.lse && jj == 0)
      a.lse[(int64_t)b * a.Hq + g * G + hh] = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
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
