// Prefill attention on gfx950: bf16 MFMA with fp32 accumulation, online
// softmax with the per-head sink folded into the running max and sum, and
// whole key tiles outside the causal band or the sliding window skipped.
//
// What it computes is the sink + window causal GQA attention of
// «GPT-OSS vs Qwen3» (sections "Introduction de Grouped Query Attention",
// "Utilisation de Sliding Window Attention", "Attention Bias et Sinks") with the
// head layout of «GPT-OSS-20B : Architecture MoE & Résumé du Model Card» §3.3.
//
// Work decomposition.  A workgroup owns one KV head g of one sequence and 8
// "N-tiles"; an N-tile is 32 query positions of one query head of g's group.
// For the 64/8 head layout that is all 8 heads of the group at 32 positions, so
// every K/V tile staged in LDS is used by the whole group.  Each of the 4 waves
// owns two N-tiles (64 query rows).
//
// The scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//   A = K tile rows (keys) read straight from LDS, B = Q^T held in registers.
// In the MFMA result a lane holds 16 keys of ONE query row, so the row max and
// the rescale of the output are per lane (one exchange with lane ^ 32 for the
// max).  The output is also accumulated transposed, O^T += V^T P^T, with P^T
// taken from the score registers as they are (the contraction order over keys
// is free) and V^T read from a transposed LDS copy of the V tile.
#include "kernels.h"

namespace gqa {
namespace {

constexpr int BK = 64;          // keys per tile
constexpr int NTHREADS = 256;   // 4 waves
constexpr int KS = 72;          // LDS row stride (elements) of K [key][d]
constexpr int VS = 68;          // LDS row stride (elements) of V^T [d][key]

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int MODE, bool VARLEN>
__global__ __launch_bounds__(NTHREADS, 2) void prefill_bf16_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 Ks[BK * KS];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[kHeadDim * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 31;  // row of the 32-wide MFMA tile this lane serves
  const int lg = lane >> 5;  // which half of the K dimension / which 4-row group

  // ---- which (sequence, KV head, tile group): heaviest tile groups first, and
  // all workgroups of one (sequence, KV head) on the same XCD (dispatch is
  // round-robin over the 8 XCDs), so its K/V stays in that XCD's L2.
  const int U = a.B * a.Hkv;
  int unit, rank;
  {
    const int x = blockIdx.x;
    if ((U & 7) == 0) {
      const int per = U >> 3;
      const int sidx = x >> 3;
      rank = sidx / per;
      unit = (x & 7) + 8 * (sidx % per);
    } else {
      rank = x / U;
      unit = x % U;
    }
  }
  const int tg = a.wg_per_seq - 1 - rank;
  const int b = unit / a.Hkv;
  const int g = unit - b * a.Hkv;
  const SeqView sv = seq_view<MODE>(a.seq, b, VARLEN);
  const int G = a.G;
  const int n_ntiles = ((sv.q_len + 31) >> 5) * G;
  if (tg < 0 || tg * 8 >= n_ntiles) return;  // uniform over the workgroup
  if (a.skip_single && sv.q_len == 1) return;
  const int pos_off = sv.kv_len - sv.q_len;
  const int W = a.window;

  // ---- this wave's two N-tiles
  int nt_t0[2], nt_hq[2];
  bool nt_valid[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int n = tg * 8 + wave * 2 + i;
    nt_valid[i] = n < n_ntiles;
    const int pb = n / G;
    nt_t0[i] = pb * 32;
    nt_hq[i] = g * G + (n - pb * G);
  }

  // ---- key range of the whole workgroup
  const int n_last = min(tg * 8 + 7, n_ntiles - 1);
  const int t_min = ((tg * 8) / G) * 32;
  const int t_max = min((n_last / G) * 32 + 31, sv.q_len - 1);
  const int p_min = pos_off + t_min;
  const int p_max = pos_off + t_max;
  const int lo = W > 0 ? max(0, p_min - W + 1) : 0;
  const int hi = min(p_max, sv.kv_len - 1);  // inclusive

  // ---- Q^T operands (B of S^T = K Q^T): lane holds row lr, d = 16*ks + 8*lg .. +7
  bf16x8 qb[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = nt_t0[i] + lr;
    const bool ok = nt_valid[i] && t < sv.q_len;
    const __bf16* qp = a.q + ((sv.q_row0 + t) * a.Hq + nt_hq[i]) * (int64_t)kHeadDim + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (ok) w = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
      qb[i][ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // ---- running softmax state per (N-tile, lane): max in log2 units and partial sum
  float m_run[2], l_run[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float s2 = a.sinks ? a.sinks[nt_hq[i]] * kLog2e : -INFINITY;
    const bool none = (s2 == -INFINITY);
    m_run[i] = none ? kNegBig : s2;
    // the sink's own term e^{s-m} = 1 at m = s; only one lane of the pair carries it
    l_run[i] = (none || lg) ? 0.f : 1.f;
  }
  f32x16 o[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][dt][r] = 0.f;

  // ---- tile loader: 512 16-byte chunks of K and of V per tile, 2 of each per thread
  const int64_t kv_stride = (int64_t)a.Hkv * kHeadDim;
  u32x4 kreg[2], vreg[2];
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int chunk = tid + c * NTHREADS;
      const int key = chunk >> 3;
      const int col = (chunk & 7) * 8;
      const int j = j0 + key;
      u32x4 kw = {0u, 0u, 0u, 0u}, vw = {0u, 0u, 0u, 0u};
      if (j <= hi) {
        const int64_t off = kv_row<MODE>(a.seq, sv, j) * kv_stride + g * kHeadDim + col;
        kw = *reinterpret_cast<const u32x4*>(a.k + off);
        vw = *reinterpret_cast<const u32x4*>(a.v + off);
      }
      kreg[c] = kw;
      vreg[c] = vw;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int chunk = tid + c * NTHREADS;
      const int key = chunk >> 3;
      const int col = (chunk & 7) * 8;
      *reinterpret_cast<u32x4*>(&Ks[key * KS + col]) = kreg[c];
      const uint16_t* hv = reinterpret_cast<const uint16_t*>(&vreg[c]);
      uint16_t* vt = reinterpret_cast<uint16_t*>(Vt);
#pragma unroll
      for (int e = 0; e < 8; ++e) vt[(col + e) * VS + key] = hv[e];
    }
  };

  const int j_begin = lo & ~(BK - 1);
  if (j_begin <= hi) load_tile(j_begin);

  for (int j0 = j_begin; j0 <= hi; j0 += BK) {
    __syncthreads();  // everyone is done reading the previous tile
    store_tile();
    __syncthreads();
    if (j0 + BK <= hi) load_tile(j0 + BK);  // in flight during this tile's math

    // classify this key tile for each N-tile: skip / unmasked / masked
    bool active[2], masked[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int plo = pos_off + nt_t0[i];
      const int phi = pos_off + min(nt_t0[i] + 31, sv.q_len - 1);
      const bool none = !nt_valid[i] || j0 > phi || (W > 0 && j0 + BK - 1 <= plo - W);
      const bool full = (j0 + BK - 1 <= plo) && (W <= 0 || j0 > phi - W);
      active[i] = !none;
      masked[i] = !full;
    }
    if (!active[0] && !active[1]) continue;

    // S^T tile: keys 32*mt + (row of the MFMA output) x query rows
    f32x16 s[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[mt][i][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Ks[(32 * mt + lr) * KS + 16 * ks + 8 * lg]);
#pragma unroll
        for (int i = 0; i < 2; ++i) s[mt][i] = mfma32(ka, qb[i][ks], s[mt][i]);
      }
    }

    // online softmax (exp2 domain); lane holds keys 32*mt + 8*(r/4) + 4*lg + r%4 of row lr
    bf16x8 pb[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (masked[i]) {
        const int p = pos_off + nt_t0[i] + lr;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j0 + 32 * mt + 8 * (r >> 2) + 4 * lg + (r & 3);
            const bool vis = key <= p && (W <= 0 || key > p - W);
            if (!vis) s[mt][i][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][i][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run[i], mx * a.scale_log2);
      const float alpha = fast_exp2(m_run[i] - m_new);
      m_run[i] = m_new;
      float rs = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(__builtin_fmaf(s[mt][i][r], a.scale_log2, -m_new));
          s[mt][i][r] = p;
          rs += p;
        }
      l_run[i] = l_run[i] * alpha + rs;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][dt][r] *= alpha;
      // P^T operands: MFMA k-step u takes registers 8*(u%2) .. +7 of score tile u/2
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        bf16x8 t;
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = (__bf16)s[u >> 1][i][8 * (u & 1) + e];
        pb[i][u] = t;
      }
    }

    // O^T += V^T P^T; the key order of k-step u is 16u + {4lg..4lg+3, 8+4lg..8+4lg+3}
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const __bf16* vp = &Vt[(32 * dt + lr) * VS + 16 * u + 4 * lg];
        const u32x2 v0 = *reinterpret_cast<const u32x2*>(vp);
        const u32x2 v1 = *reinterpret_cast<const u32x2*>(vp + 8);
        const u32x4 vw = {v0[0], v0[1], v1[0], v1[1]};
        const bf16x8 va = __builtin_bit_cast(bf16x8, vw);
#pragma unroll
        for (int i = 0; i < 2; ++i) o[i][dt] = mfma32(va, pb[i][u], o[i][dt]);
      }
    }
  }

  // ---- epilogue: normalise, round to bf16, store; log-sum-exp
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (!nt_valid[i]) continue;
    const float lt = l_run[i] + __shfl_xor(l_run[i], 32, 64);
    const int t = nt_t0[i] + lr;
    if (t >= sv.q_len) continue;
    const float inv = lt > 0.f ? 1.f / lt : (lt == 0.f ? 0.f : lt);
    __bf16* op = a.out + ((sv.q_row0 + t) * a.Hq + nt_hq[i]) * (int64_t)kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int d0 = 32 * dt + 8 * c + 4 * lg;
        u32x2 w;
        w[0] = pack_bf16x2(o[i][dt][4 * c + 0] * inv, o[i][dt][4 * c + 1] * inv);
        w[1] = pack_bf16x2(o[i][dt][4 * c + 2] * inv, o[i][dt][4 * c + 3] * inv);
        *reinterpret_cast<u32x2*>(op + d0) = w;
      }
    if (a.lse && lg == 0) {
      const float v = (lt == 0.f) ? -INFINITY : (m_run[i] + __log2f(lt)) * kLn2;
      const int64_t idx = (int64_t)b * a.lse_sb + (int64_t)nt_hq[i] * a.lse_sh + t + (a.lse_row0 ? sv.q_row0 : 0);
      a.lse[idx] = v;
    }
  }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, int kv_mode, bool varlen_q, hipStream_t s) {
  const int grid = a.B * a.Hkv * a.wg_per_seq;
  if (grid <= 0) return hipSuccess;
  if (!varlen_q && kv_mode == KV_BATCHED)
    hipLaunchKernelGGL((prefill_bf16_kernel<KV_BATCHED, false>), dim3(grid), dim3(NTHREADS), 0, s, a);
  else if (varlen_q && kv_mode == KV_PAGED)
    hipLaunchKernelGGL((prefill_bf16_kernel<KV_PAGED, true>), dim3(grid), dim3(NTHREADS), 0, s, a);
  else if (varlen_q && kv_mode == KV_PACKED)
    hipLaunchKernelGGL((prefill_bf16_kernel<KV_PACKED, true>), dim3(grid), dim3(NTHREADS), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace gqa
