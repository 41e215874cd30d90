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
// owns two N-tiles (64 query rows); two workgroups share a CU.
//
// The scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
// A = rows of the K tile (keys) from LDS, B = Q^T held in registers.  In the
// result a lane holds 16 keys of ONE query row, so the row max and the output
// rescale are per lane (one lane^32 exchange for the max).  The output is also
// accumulated transposed, O^T += V^T P^T: P^T comes from the score registers as
// they are (the contraction order over keys is free), and V^T from the V tile,
// stored in LDS in its natural [key][d] layout and read with the transposing
// LDS load ds_read_b64_tr_b16.
//
// Per 64-key tile a wave computes the scores of both its N-tiles (each K
// operand read from LDS feeds two MFMAs), runs the two softmax steps, then
// accumulates P V for both (each V operand feeds two MFMAs).  The two
// workgroups sharing a CU overlap each other's MFMA and VALU phases.  K/V
// tiles are staged one tile ahead in double-buffered LDS, with one workgroup
// barrier per tile.
//
// The softmax keeps a reference max per row but does not track the running
// max tile by tile: the weights are exponentiated against the reference as it
// stands, and the row sum that is accumulated anyway tells whether any weight
// grew too large (past 2^32).  Only then, on a uniform rare branch, is the
// tile recomputed against its true max and the output rescaled.  fp32 sums and
// bf16 weights keep their relative precision at any magnitude, so nothing but
// overflow needs guarding; with a sink the reference starts at the sink logit,
// and without one the first visible tile sets it.
#include "kernels.h"

namespace gqa {
namespace {

constexpr int BK = 64;          // keys per tile
constexpr int NWAVES = 4;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int NT_WG = 2 * NWAVES;  // N-tiles per workgroup
constexpr int KS = 72;          // LDS row stride (elements) of K [key][d]: conflict-free 16-byte row reads
constexpr int VS = 96;          // LDS row stride (elements) of V [key][d]: conflict-free transposing reads
constexpr float kRefit = 0x1p32f;  // a lane's per-tile weight sum past this moves the reference max

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// S^T for both N-tiles: keys 32*mt + (MFMA row) of the tile x 32 query rows
__device__ __forceinline__ void qk_tile(f32x16 (&s0)[2], f32x16 (&s1)[2], const __bf16* ks, const bf16x8 (&qb)[2][4],
                                        int lr, int lg) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(ks + (32 * mt + lr) * KS + 16 * k + 8 * lg);
      s0[mt] = mfma32(ka, qb[0][k], k == 0 ? zero16() : s0[mt]);
      s1[mt] = mfma32(ka, qb[1][k], k == 0 ? zero16() : s1[mt]);
    }
  }
}

// O^T += V^T P^T for one N-tile.  In 16-lane group c of the wave, lane j reads 4
// consecutive d of key row (j/4); the transposing load hands lane i of the
// group the 4 keys at d = dbase + i.  The key order of k-step u matches the
// score registers: 16u + {4lg..4lg+3, 8+4lg..8+4lg+3}.
__device__ __forceinline__ void pv_tile(f32x16 (&o)[2][2], const __bf16* vs, const bf16x8 (&p0)[4],
                                        const bf16x8 (&p1)[4], int vofs) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const __bf16* base = vs + vofs + 16 * u * VS + 32 * dt;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 8 * VS));
      const i16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const bf16x8 va = __builtin_bit_cast(bf16x8, w);
      o[0][dt] = mfma32(va, p0[u], o[0][dt]);
      o[1][dt] = mfma32(va, p1[u], o[1][dt]);
    }
  }
}

// Mask of one N-tile on one 64-key tile.  Lane holds keys
// j0 + 32*mt + 8*(r/4) + 4*lg + r%4 of query row lr; the key is visible iff
// (key - j0 - 4lg) lies in (dl, dh] (dl only counts with a window).  Each
// 32-key half is classified with wave-uniform bounds first: wholly visible
// halves are left alone, wholly hidden ones are cleared, and only a half that
// the causal diagonal or the window edge crosses is compared element by element.
__device__ __forceinline__ void mask_ntile(f32x16 (&s)[2], int j0, int plo, int phi, int W, int dh, int dl) {
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int kb = j0 + 32 * mt;  // first key of this half (uniform)
    const bool hidden = kb > phi || (W > 0 && kb + 31 <= plo - W);
    if (hidden) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[mt][r] = -INFINITY;
      continue;
    }
    if (kb + 31 > plo) {  // causal diagonal crosses this half
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * mt + 8 * (r >> 2) + (r & 3) > dh) s[mt][r] = -INFINITY;
    }
    if (W > 0 && kb <= phi - W) {  // window edge crosses this half
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * mt + 8 * (r >> 2) + (r & 3) <= dl) s[mt][r] = -INFINITY;
    }
  }
}

// Exponentials of one N-tile against the reference max m (log2 units): the
// bf16 P^T operand and this lane's partial row sum of the rounded weights.
__device__ __forceinline__ float exp_ntile(const f32x16 (&s)[2], bf16x8 (&pb)[4], float m, float c) {
  float rs = 0.f;
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f32x2 x = {fast_exp2(__builtin_fmaf(s[u >> 1][8 * (u & 1) + 2 * e], c, -m)),
                       fast_exp2(__builtin_fmaf(s[u >> 1][8 * (u & 1) + 2 * e + 1], c, -m))};
      const bf16x2 pk = __builtin_convertvector(x, bf16x2);
      rs = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, rs, false);
      w[e] = __builtin_bit_cast(uint32_t, pk);
    }
    pb[u] = __builtin_bit_cast(bf16x8, w);
  }
  return rs;
}

// Rare path: some lane's weights on this tile summed past kRefit, i.e. a score
// rose far above the reference max (always so on the first visible tile when
// there is no sink).  Recompute the tile's scores, move the reference to the
// true running max, rescale the output and the sum, and redo the weights.
__device__ __forceinline__ float refit_ntile(f32x16 (&s)[2], bf16x8 (&pb)[4], float& m, float& l, float& alpha,
                                             const __bf16* ks, const bf16x8 (&qb)[4], int lr, int lg, float c, int j0,
                                             int plo, int phi, int W, int dh, int dl) {
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(ks + (32 * mt + lr) * KS + 16 * k + 8 * lg);
      s[mt] = mfma32(ka, qb[k], k == 0 ? zero16() : s[mt]);
      __builtin_amdgcn_sched_barrier(0);
    }
  mask_ntile(s, j0, plo, phi, W, dh, dl);
  float mx = s[0][0];
#pragma unroll
  for (int r = 1; r < 32; ++r) mx = fmaxf(mx, s[r >> 4][r & 15]);
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  const float m_new = fmaxf(m, mx * c);
  alpha = fast_exp2(m - m_new);
  l *= alpha;
  m = m_new;
  return exp_ntile(s, pb, m, c);
}

template <int MODE, bool VARLEN>
__global__ __launch_bounds__(NTHREADS, 2) void prefill_bf16_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 Ks[2][BK * KS];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[2][BK * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (lets per-wave values live in SGPRs)
  const int lr = lane & 31;  // row of the 32-wide MFMA tile this lane serves
  const int lg = lane >> 5;  // which half of the K dimension / which 4-row group

  // ---- which (sequence, KV head, tile group): all workgroups of one
  // (sequence, KV head) go to the same XCD (dispatch is round-robin over the 8
  // XCDs) and are dispatched back to back, heaviest tile group first, so they
  // stream the same K/V tiles at about the same time out of that XCD's L2.
  const int U = a.B * a.Hkv;
  int unit, rank;
  {
    const int x = blockIdx.x;
    if ((U & 7) == 0) {
      const int sidx = x >> 3;
      rank = sidx % a.wg_per_seq;
      unit = (x & 7) + 8 * (sidx / a.wg_per_seq);
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
  if (tg < 0 || tg * NT_WG >= n_ntiles) return;  // uniform over the workgroup
  if (a.skip_single && sv.q_len == 1) return;
  const int pos_off = sv.kv_len - sv.q_len;
  const int W = a.window;
  const float c = a.scale_log2;

  // ---- this wave's two N-tiles
  int nt_t0[2], nt_hq[2], pos0[2], phi[2];
  bool nt_valid[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int n = tg * NT_WG + wave * 2 + i;
    nt_valid[i] = n < n_ntiles;
    const int pb = n / G;
    nt_t0[i] = pb * 32;
    nt_hq[i] = g * G + (n - pb * G);
    pos0[i] = pos_off + nt_t0[i];
    phi[i] = pos_off + min(nt_t0[i] + 31, sv.q_len - 1);
  }

  // ---- key range of the whole workgroup
  const int n_last = min(tg * NT_WG + NT_WG - 1, n_ntiles - 1);
  const int t_min = ((tg * NT_WG) / G) * 32;
  const int t_max = min((n_last / G) * 32 + 31, sv.q_len - 1);
  const int p_min = pos_off + t_min;
  const int p_max = pos_off + t_max;
  const int lo = W > 0 ? max(0, p_min - W + 1) : 0;
  const int hi = min(p_max, sv.kv_len - 1);  // inclusive
  const int j_begin = lo & ~(BK - 1);
  const int n_tiles = hi >= j_begin ? (hi - j_begin) / BK + 1 : 0;

  // ---- Q^T operands (B of S^T = K Q^T): lane holds row lr, d = 16*k + 8*lg .. +7
  bf16x8 qb[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = nt_t0[i] + lr;
    const bool ok = nt_valid[i] && t < sv.q_len;
    const __bf16* qp = a.q + ((sv.q_row0 + t) * a.Hq + nt_hq[i]) * (int64_t)kHeadDim + 8 * lg;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ok) v = *reinterpret_cast<const u32x4*>(qp + 16 * k);
      qb[i][k] = __builtin_bit_cast(bf16x8, v);
    }
  }
  float m_run[2], l_run[2];
  f32x16 o[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float s2 = a.sinks ? a.sinks[nt_hq[i]] * kLog2e : -INFINITY;
    const bool none = (s2 == -INFINITY);
    m_run[i] = none ? kNegBig : s2;
    // the sink's own term e^{s-m} = 1 at m = s; only one lane of the pair carries it
    l_run[i] = (none || lg) ? 0.f : 1.f;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) o[i][dt] = zero16();
  }

  // ---- global -> register -> LDS staging: 512 16-byte chunks per K or V tile, 2 of each per thread
  const int64_t kv_stride = (int64_t)a.Hkv * kHeadDim;
  const __bf16* kbase = a.k + g * kHeadDim;
  const __bf16* vbase = a.v + g * kHeadDim;
  // This thread moves rows r0 and r0 + 32 of every tile (16 bytes at d = 8*(tid%8)).
  // With a paged cache their block ids are fetched one tile ahead, so no K/V
  // load waits on the block table.  Rows past the key range repeat row hi (they
  // are masked, and the loads stay in bounds).
  const int r0 = tid >> 3;
  auto fetch_blk = [&](int t, int (&blk)[2]) {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      blk[cc] = 0;
      if (MODE == KV_PAGED) {
        const int j = min(j_begin + BK * t + r0 + 32 * cc, hi);
        blk[cc] = a.seq.block_table[(int64_t)b * a.seq.max_blocks + (j >> a.seq.log2_block)];
      }
    }
  };
  auto load_kv = [&](int t, const int (&blk)[2], u32x4 (&kreg)[2], u32x4 (&vreg)[2]) {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int j = min(j_begin + BK * t + r0 + 32 * cc, hi);
      int64_t row;
      if (MODE == KV_PAGED) {
        const int bb = min(max(blk[cc], 0), a.seq.num_blocks - 1);
        row = ((int64_t)bb << a.seq.log2_block) + (j & ((1 << a.seq.log2_block) - 1));
      } else {
        row = kv_row<MODE>(a.seq, sv, j);
      }
      const int64_t off = row * kv_stride + (tid & 7) * 8;
      kreg[cc] = *reinterpret_cast<const u32x4*>(kbase + off);
      vreg[cc] = *reinterpret_cast<const u32x4*>(vbase + off);
    }
  };
  auto store_rows = [&](__bf16* dst, int stride, const u32x4 (&reg)[2]) {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int chunk = tid + cc * NTHREADS;
      *reinterpret_cast<u32x4*>(dst + (chunk >> 3) * stride + (chunk & 7) * 8) = reg[cc];
    }
  };

  // lane's address offset for the transposing V reads (see pv_ntile)
  const int vofs = (4 * (lane >> 5) + ((lane & 15) >> 2)) * VS + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // one 64-key tile; K/V of tile t are in buffer t % 2, tile t+1 is staged into the other
  int blk_next[2];  // block ids of tile t+1's rows
  auto body = [&](int t) {
    const int buf = t & 1;
    const int j0 = j_begin + BK * t;
    const bool next = t + 1 < n_tiles;
    u32x4 kreg[2], vreg[2];
    if (next) load_kv(t + 1, blk_next, kreg, vreg);
    int blk_nn[2];
    fetch_blk(t + 2, blk_nn);
    f32x16 s0[2], s1[2];
    bf16x8 p0[4], p1[4];
    qk_tile(s0, s1, Ks[buf], qb, lr, lg);
    const int dh0 = pos0[0] + lr - j0 - 4 * lg, dh1 = pos0[1] + lr - j0 - 4 * lg;
    const int dl0 = W > 0 ? dh0 - W : -0x40000000, dl1 = W > 0 ? dh1 - W : -0x40000000;
    mask_ntile(s0, j0, pos0[0], phi[0], W, dh0, dl0);
    mask_ntile(s1, j0, pos0[1], phi[1], W, dh1, dl1);
    float rs0 = exp_ntile(s0, p0, m_run[0], c);
    float rs1 = exp_ntile(s1, p1, m_run[1], c);
    const bool f0 = __builtin_amdgcn_ballot_w64(rs0 > kRefit) != 0;
    const bool f1 = __builtin_amdgcn_ballot_w64(rs1 > kRefit) != 0;
    float al0 = 1.f, al1 = 1.f;
    if (f0) rs0 = refit_ntile(s0, p0, m_run[0], l_run[0], al0, Ks[buf], qb[0], lr, lg, c, j0, pos0[0], phi[0], W, dh0, dl0);
    if (f1) rs1 = refit_ntile(s1, p1, m_run[1], l_run[1], al1, Ks[buf], qb[1], lr, lg, c, j0, pos0[1], phi[1], W, dh1, dl1);
    if (f0) { o[0][0] *= al0; o[0][1] *= al0; }
    if (f1) { o[1][0] *= al1; o[1][1] *= al1; }
    l_run[0] += rs0;
    l_run[1] += rs1;
    pv_tile(o, Vs[buf], p0, p1, vofs);
    if (next) {
      store_rows(Ks[buf ^ 1], KS, kreg);
      store_rows(Vs[buf ^ 1], VS, vreg);
    }
    blk_next[0] = blk_nn[0];
    blk_next[1] = blk_nn[1];
    __syncthreads();
  };

  if (n_tiles > 0) {
    {
      int blk0[2];
      u32x4 kr[2], vr[2];
      fetch_blk(0, blk0);
      load_kv(0, blk0, kr, vr);
      fetch_blk(1, blk_next);
      store_rows(Ks[0], KS, kr);
      store_rows(Vs[0], VS, vr);
    }
    __syncthreads();
    for (int t = 0; t < n_tiles; ++t) body(t);
  }

  // ---- epilogue: normalise, round to bf16, store; log-sum-exp
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (!nt_valid[i]) continue;
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run[i]), __float_as_uint(l_run[i]), false, false);
    const float lt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const int t = nt_t0[i] + lr;
    if (t >= sv.q_len) continue;
    const float inv = lt > 0.f ? 1.f / lt : (lt == 0.f ? 0.f : lt);
    __bf16* op = a.out + ((sv.q_row0 + t) * a.Hq + nt_hq[i]) * (int64_t)kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int cq = 0; cq < 4; ++cq) {
        const int d0 = 32 * dt + 8 * cq + 4 * lg;
        u32x2 v;
        v[0] = pack_bf16x2(o[i][dt][4 * cq + 0] * inv, o[i][dt][4 * cq + 1] * inv);
        v[1] = pack_bf16x2(o[i][dt][4 * cq + 2] * inv, o[i][dt][4 * cq + 3] * inv);
        *reinterpret_cast<u32x2*>(op + d0) = v;
      }
    if (a.lse && lg == 0) {
      const float v = (lt == 0.f) ? -INFINITY : (m_run[i] + __log2f(lt)) * kLn2;
      const int64_t idx = (int64_t)b * a.lse_sb + (int64_t)nt_hq[i] * a.lse_sh + t + (a.lse_row0 ? sv.q_row0 : 0);
      a.lse[idx] = v;
    }
  }
}

}  // namespace

int prefill_ntiles_per_wg() { return NT_WG; }

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
