// Decode attention on gfx950: one new query token per sequence, HBM-bound.
//
// The KV cache is streamed once; each K/V row of a KV head serves all the
// query heads of its group («GPT-OSS-20B : Architecture MoE & Résumé du Model
// Card» §3.3, 8 query heads per KV head), and on sliding-window layers only the
// last W positions are read («GPT-OSS vs Qwen3», "Utilisation de Sliding Window
// Attention").  The sink logit («GPT-OSS vs Qwen3», "Attention Bias et Sinks")
// enters once, when the partial results are merged.
//
// Work decomposition: a workgroup owns (sequence, KV head, chunk of up to 16
// query heads, split of the key range).  Its 4 waves take interleaved 64-key
// tiles and keep independent online-softmax states; the 4 states are merged in
// LDS.  With one split the workgroup writes the final output; otherwise it
// writes a partial (max, sum, unnormalised output) and a combine kernel merges
// the splits.
//
// Per tile the scores are S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (K straight
// from global memory in the A layout, Q^T in registers, 16 head columns), and
// the output is O^T += V^T P^T with V^T read from a per-wave transposed LDS copy.
#include "kernels.h"

namespace gqa {
namespace {

constexpr int DT = 64;         // keys per wave tile
constexpr int DTHREADS = 256;  // 4 waves
constexpr int VSD = 68;        // LDS row stride (elements) of the per-wave V^T [d][key]

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int MODE>
__global__ __launch_bounds__(DTHREADS, 2) void decode_split_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 Vt[4][kHeadDim * VSD];
  __shared__ float red_m[4][16];
  __shared__ float red_l[4][16];
  __shared__ __attribute__((aligned(16))) float red_o[4][16][kHeadDim + 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lc = lane & 15;  // head column (and key row of the K operand)
  const int lq = lane >> 4;  // lane quarter

  // blockIdx -> (split, head chunk, KV head, sequence); splits of one
  // (sequence, KV head) are consecutive
  int x = blockIdx.x;
  const int split = x % a.n_splits;
  x /= a.n_splits;
  const int hc = x % a.n_hc;
  x /= a.n_hc;
  const int g = x % a.Hkv;
  const int b = x / a.Hkv;

  const SeqView sv = seq_view<MODE>(a.seq, b, a.varlen_q != 0);
  if (a.varlen_q && sv.q_len != 1) return;  // handled by the prefill-style kernel
  const int L = sv.kv_len;
  const int W = a.window;
  const int lo_all = W > 0 ? max(0, L - W) : 0;
  const int s_lo = lo_all + split * a.split_len;
  const int s_hi = min(L, s_lo + a.split_len);  // exclusive
  const int h_base = g * a.G + hc * 16;
  const int n_heads = min(16, a.G - hc * 16);
  const int64_t q_row = a.varlen_q ? sv.q_row0 : (int64_t)b;

  // Q^T operand: lane holds head lc, d = 32*ks + 8*lq .. +7 (zero for padding heads)
  bf16x8 qb[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (lc < n_heads)
      w = *reinterpret_cast<const u32x4*>(a.q + (q_row * a.Hq + h_base + lc) * (int64_t)kHeadDim + 32 * ks + 8 * lq);
    qb[ks] = __builtin_bit_cast(bf16x8, w);
  }

  float m_run = kNegBig, l_run = 0.f;
  f32x4 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t kv_stride = (int64_t)a.Hkv * kHeadDim;
  const __bf16* kbase = a.k + g * kHeadDim;
  const __bf16* vbase = a.v + g * kHeadDim;
  uint16_t* vt = reinterpret_cast<uint16_t*>(Vt[wave]);

  // K chunk (kb, ks): key 16*kb + lc, d 32*ks + 8*lq (the MFMA A layout)
  // V chunk i: key 8*i + lane/8, d 8*(lane%8) (whole 128-byte rows per 8 lanes)
  u32x4 kreg[8], vreg[8];
  auto load = [&](int j0) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int j = j0 + 16 * kb + lc;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (j < s_hi) w = *reinterpret_cast<const u32x4*>(kbase + kv_row<MODE>(a.seq, sv, j) * kv_stride + 32 * ks + 8 * lq);
        kreg[kb * 2 + ks] = w;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = j0 + 8 * i + (lane >> 3);
      u32x4 w = {0u, 0u, 0u, 0u};
      if (j < s_hi) w = *reinterpret_cast<const u32x4*>(vbase + kv_row<MODE>(a.seq, sv, j) * kv_stride + 8 * (lane & 7));
      vreg[i] = w;
    }
  };

  int j0 = s_lo + wave * DT;
  if (j0 < s_hi) load(j0);
  for (; j0 < s_hi; j0 += 4 * DT) {
    // transposed copy of this tile's V into the wave's LDS slice
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = 8 * i + (lane >> 3);
      const int d0 = 8 * (lane & 7);
      const uint16_t* hv = reinterpret_cast<const uint16_t*>(&vreg[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) vt[(d0 + e) * VSD + key] = hv[e];
    }
    u32x4 kcur[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) kcur[i] = kreg[i];
    const int jn = j0 + 4 * DT;
    if (jn < s_hi) load(jn);  // next tile in flight during this one's math

    // S^T: 4 blocks of 16 keys x 16 heads
    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) acc = mfma16(__builtin_bit_cast(bf16x8, kcur[kb * 2 + ks]), qb[ks], acc);
      s[kb] = acc;
    }
    // lane holds keys j0 + 16*kb + 4*lq + r of head lc
    const bool full = (j0 + DT <= s_hi);
    if (!full) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (j0 + 16 * kb + 4 * lq + r >= s_hi) s[kb][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * a.scale_log2);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(__builtin_fmaf(s[kb][r], a.scale_log2, -m_new));
        s[kb][r] = p;
        rs += p;
      }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;

    wave_lds_sync();  // the V^T stores above are visible to every lane

    // O^T += V^T P^T over 2 k-steps of 32 keys: keys 32u + {4lq..4lq+3, 16+4lq..16+4lq+3}
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      bf16x8 pbv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pbv[e] = (__bf16)s[2 * u][e];
        pbv[4 + e] = (__bf16)s[2 * u + 1][e];
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const uint16_t* vp = &vt[(16 * dt + lc) * VSD + 32 * u + 4 * lq];
        const u32x2 v0 = *reinterpret_cast<const u32x2*>(vp);
        const u32x2 v1 = *reinterpret_cast<const u32x2*>(vp + 16);
        const u32x4 vw = {v0[0], v0[1], v1[0], v1[1]};
        o[dt] = mfma16(__builtin_bit_cast(bf16x8, vw), pbv, o[dt]);
      }
    }
    wave_lds_sync();  // all lanes done reading V^T before the next overwrite
  }

  // ---- merge the 4 waves: per head max m, sum l, output acc[d]
  {
    float lt = l_run + __shfl_xor(l_run, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    if (lq == 0) {
      red_m[wave][lc] = m_run;
      red_l[wave][lc] = lt;
    }
    // lane holds O^T[d = 16*dt + 4*lq + r][head lc]
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) red_o[wave][lc][16 * dt + 4 * lq + r] = o[dt][r];
  }
  __syncthreads();
  {
    const int hh = tid >> 4;         // head within the chunk
    const int d0 = (tid & 15) * 4;   // 4 output columns
    if (hh < n_heads) {
      float M = red_m[0][hh];
#pragma unroll
      for (int w = 1; w < 4; ++w) M = fmaxf(M, red_m[w][hh]);
      float wsc[4];
      float lsum = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        wsc[w] = fast_exp2(red_m[w][hh] - M);
        lsum += red_l[w][hh] * wsc[w];
      }
      float acc[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) t += red_o[w][hh][d0 + c] * wsc[w];
        acc[c] = t;
      }
      const int hq = h_base + hh;
      if (a.n_splits == 1) {
        // fold in the sink and finish
        const float s2 = a.sinks ? a.sinks[hq] * kLog2e : -INFINITY;
        const float Mf = fmaxf(M, s2);
        const float sc = fast_exp2(M - Mf);
        const float Z = fast_exp2(s2 - Mf) + lsum * sc;
        const float inv = Z > 0.f ? sc / Z : (Z == 0.f ? 0.f : Z);
        __bf16* op = a.out + (q_row * a.Hq + hq) * (int64_t)kHeadDim + d0;
        u32x2 w;
        w[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
        w[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
        *reinterpret_cast<u32x2*>(op) = w;
        if (a.lse && d0 == 0) {
          const float v = (Z == 0.f) ? -INFINITY : (Mf + __log2f(Z)) * kLn2;
          a.lse[(int64_t)b * a.lse_sb + (int64_t)hq * a.lse_sh + (a.lse_row0 ? sv.q_row0 : 0)] = v;
        }
      } else {
        const int64_t slot = ((int64_t)b * a.Hq + hq) * a.n_splits + split;
        if (d0 == 0) {
          a.ws_ml[slot * 2 + 0] = M;
          a.ws_ml[slot * 2 + 1] = lsum;
        }
        *reinterpret_cast<f32x4*>(a.ws_acc + slot * kHeadDim + d0) = f32x4{acc[0], acc[1], acc[2], acc[3]};
      }
    }
  }
}

// Merge of the split partials: one wave per (sequence, query head), lane = output column.
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeArgs a) {
  const int lane = threadIdx.x;
  const int hq = blockIdx.x % a.Hq;
  const int b = blockIdx.x / a.Hq;
  int64_t q_row = b;
  int64_t row0 = 0;
  if (a.varlen_q) {
    const int r0 = a.seq.cu_seqlens_q[b];
    if (a.seq.cu_seqlens_q[b + 1] - r0 != 1) return;
    q_row = r0;
    row0 = r0;
  }
  const int64_t base = ((int64_t)b * a.Hq + hq) * a.n_splits;
  const float s2 = a.sinks ? a.sinks[hq] * kLog2e : -INFINITY;
  float M = s2;
  for (int s = lane; s < a.n_splits; s += 64) M = fmaxf(M, a.ws_ml[(base + s) * 2]);
  M = wave_max(M);
  float Z = 0.f;
  for (int s = lane; s < a.n_splits; s += 64) Z += a.ws_ml[(base + s) * 2 + 1] * fast_exp2(a.ws_ml[(base + s) * 2] - M);
  Z = wave_sum(Z) + fast_exp2(s2 - M);
  float acc = 0.f;
  for (int s = 0; s < a.n_splits; ++s) acc += a.ws_acc[(base + s) * kHeadDim + lane] * fast_exp2(a.ws_ml[(base + s) * 2] - M);
  const float inv = Z > 0.f ? 1.f / Z : (Z == 0.f ? 0.f : Z);
  a.out[(q_row * a.Hq + hq) * kHeadDim + lane] = (__bf16)(acc * inv);
  if (a.lse && lane == 0) {
    const float v = (Z == 0.f) ? -INFINITY : (M + __log2f(Z)) * kLn2;
    a.lse[(int64_t)b * a.lse_sb + (int64_t)hq * a.lse_sh + (a.lse_row0 ? row0 : 0)] = v;
  }
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, int kv_mode, hipStream_t s) {
  const int grid = a.B * a.Hkv * a.n_hc * a.n_splits;
  if (grid <= 0) return hipSuccess;
  if (kv_mode == KV_BATCHED)
    hipLaunchKernelGGL((decode_split_kernel<KV_BATCHED>), dim3(grid), dim3(DTHREADS), 0, s, a);
  else if (kv_mode == KV_PAGED)
    hipLaunchKernelGGL((decode_split_kernel<KV_PAGED>), dim3(grid), dim3(DTHREADS), 0, s, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<KV_PACKED>), dim3(grid), dim3(DTHREADS), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_splits == 1) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(a.B * a.Hq), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace gqa
