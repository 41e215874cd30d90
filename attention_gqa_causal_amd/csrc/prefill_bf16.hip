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
// owns two N-tiles (64 query rows); two workgroups share a CU.  On windowed
// layers, where a tile group is a short job of a few tiles, a workgroup may run
// two adjacent tile groups in turn over the same tiles (see prefill_job).
//
// The scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
// A = rows of the K tile (keys) from LDS, B = Q^T held in registers.  In the
// result a lane holds 16 keys of ONE query row, so all softmax bookkeeping is
// per lane (one lane^32 exchange when a max is needed).  The output is also
// accumulated transposed, O^T += V^T P^T: P^T comes from the score registers as
// they are (the contraction order over keys is free), and V^T from the V tile,
// stored in LDS in its natural [key][d] layout and read with the transposing
// LDS load ds_read_b64_tr_b16.  Each K or V operand read from LDS feeds the
// MFMAs of both of the wave's N-tiles.
//
// Schedule.  A wave issues in order, and a vector instruction cannot issue
// while the wave is held at an MFMA, so a wave that runs all its MFMAs and
// then all its exponentials keeps only one unit busy; the other wave on the
// SIMD does not fill the gap either, since the older wave has issue priority.
// Each 64-key tile is therefore split into its two 32-key halves, which the
// softmax below treats independently, and every phase pairs matrix work with
// independent vector work in a pinned order (one MFMA pair, then about 26
// vector instructions):
//   (a) exponentials of half 0   with   scores of half 1
//   (b) exponentials of half 1   with   P V over half 0
//   (c) P V over half 1          with   scores of half 0 of the next tile
// The row sums use fp32 adds: the bf16 dot instruction would halve their
// count, but it occupies the matrix pipe and stalls the MFMAs beside it.
//
// K/V staging.  Tiles go from global memory straight into LDS with 16-byte
// direct loads (no registers, no LDS store instructions), two tiles ahead,
// into three LDS buffers: the tile being read, the next one, and the one
// landing.  One barrier per tile, between (b) and (c), publishes the next tile.
//
// The softmax keeps a reference max per row but does not track the running
// max tile by tile: the weights are exponentiated against the reference as it
// stands, and the row sum that is accumulated anyway tells whether any weight
// grew too large (past 2^32).  Only then, on a uniform rare branch, is the
// tile recomputed against its true max and the output rescaled.  fp32 sums and
// bf16 weights keep their relative precision at any magnitude, so nothing but
// overflow needs guarding; with a sink the reference starts at the sink logit,
// and without one the first visible tile sets it.
#include <type_traits>

#include "kernels.h"
#include "tile_ops.h"

namespace gqa {
namespace {

constexpr int BK = 64;          // keys per tile
constexpr int NWAVES = 4;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int NT_WG = 2 * NWAVES;  // N-tiles per workgroup
constexpr int NBUF = 3;         // K/V tiles resident in LDS: current, next, and the one being filled
constexpr float kRefit = 0x1p32f;  // a lane's per-tile weight sum past this moves the reference max
constexpr int kSortMax = NTHREADS;  // ragged batches up to this many sequences are dispatched longest first

// S^T of key half h (keys 32h .. 32h+31 of the tile, one per MFMA row) for
// both N-tiles; each K operand read from LDS feeds two MFMAs.
__device__ __forceinline__ void qk_half(f32x16& s0, f32x16& s1, const __bf16* ks, const bf16x8 (&qb)[2][4], int h,
                                        int lr, int lg) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bf16x8 ka = *reinterpret_cast<const bf16x8*>(ks + (32 * h + lr) * RS + kchunk(2 * k + lg, lr));
    s0 = mfma32(ka, qb[0][k], k == 0 ? zero16() : s0);
    s1 = mfma32(ka, qb[1][k], k == 0 ? zero16() : s1);
  }
}

// O^T += V^T P^T over key half h (k-steps u = 2h, 2h+1) for both N-tiles; V^T
// comes from the V tile through the transposing read.
__device__ __forceinline__ void pv_half(f32x16 (&o)[2][2], const __bf16* vs, const bf16x8 (&p0)[2],
                                        const bf16x8 (&p1)[2], int h, const int (&vofs)[2]) {
#pragma unroll
  for (int uu = 0; uu < 2; ++uu) {
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const bf16x8 va = tr_operand(vs, 2 * h + uu, dt, vofs);
      o[0][dt] = mfma32(va, p0[uu], o[0][dt]);
      o[1][dt] = mfma32(va, p1[uu], o[1][dt]);
    }
  }
}

// Exponentials of one N-tile's key half against the reference max m (log2
// units): the two bf16 P^T operands of that half and this lane's partial row
// sum of the weights.  The sum is taken with plain fp32 adds: the bf16 dot
// instruction would do it in half the instructions, but it occupies the matrix
// pipe and so stalls the MFMAs this work is meant to run beside.
__device__ __forceinline__ float exp_half(const f32x16& s, bf16x8 (&pb)[2], float m, float c) {
  float ra = 0.f, rb = 0.f;
#pragma unroll
  for (int uu = 0; uu < 2; ++uu) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f32x2 x = {fast_exp2(__builtin_fmaf(s[8 * uu + 2 * e], c, -m)),
                       fast_exp2(__builtin_fmaf(s[8 * uu + 2 * e + 1], c, -m))};
      ra += x[0];
      rb += x[1];
      w[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
    }
    pb[uu] = __builtin_bit_cast(bf16x8, w);
  }
  return ra + rb;
}

// One eighth of a tile's exponentials for one N-tile: the 8 scores of
// k-step group uu of a key half (one bf16 P^T operand) and their partial sum.
__device__ __forceinline__ float exp_chunk(const f32x16& s, bf16x8& pb, int uu, float m, float c) {
  // the sums start from the first weights, not from 0: 0 + x would cost an add
  // each (the compiler keeps it, as it cannot rule out x = -0)
  float ra, rb;
  u32x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const f32x2 x = {fast_exp2(__builtin_fmaf(s[8 * uu + 2 * e], c, -m)),
                     fast_exp2(__builtin_fmaf(s[8 * uu + 2 * e + 1], c, -m))};
    if (e == 0) {
      ra = x[0];
      rb = x[1];
    } else {
      ra += x[0];
      rb += x[1];
    }
    w[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
  }
  pb = __builtin_bit_cast(bf16x8, w);
  return ra + rb;
}

// Rare path: some lane's weights on this key half summed past kRefit, i.e. a
// score rose far above the reference max (always so on the first visible half
// when there is no sink).  Recompute the half's scores, move the reference to
// the true running max, and redo the weights; the caller rescales the output
// by the returned alpha (the row sum is rescaled here).
template <bool STK>
__device__ __forceinline__ float refit_half(f32x16& s, bf16x8 (&pb)[2], float& m, float& l, float& alpha,
                                            const __bf16* ks, const bf16x8 (&qb)[4], int h, int lr, int lg, float c,
                                            int j0, int plo, int phi, int W, int st, int dh, int dl, int ds) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bf16x8 ka = *reinterpret_cast<const bf16x8*>(ks + (32 * h + lr) * RS + kchunk(2 * k + lg, lr));
    s = mfma32(ka, qb[k], k == 0 ? zero16() : s);
    __builtin_amdgcn_sched_barrier(0);
  }
  mask_half<STK>(s, h, j0, plo, phi, W, st, dh, dl, ds);
  float mx = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  const float m_new = fmaxf(m, mx * c);
  alpha = fast_exp2(m - m_new);
  l *= alpha;
  m = m_new;
  return exp_half(s, pb, m, c);
}

// Rotary encoding of queries that arrive unrotated, applied to the Q operands
// in registers.  Lane (lr, lg) holds row lr of an N-tile, elements
// d = 16k + 8lg + e of qb[k]: with pairs (2j, 2j+1) the four pairs of qb[k] are
// j = 8k + 4lg + e/2; with pairs (j, j + 32) element e of qb[k] (k < 2) pairs
// with element e of qb[k + 2], j = 16k + 8lg + e.  So a lane needs the angles of
// 16 frequencies at its row's position.  Angles and rotation are the helpers the
// rotary append uses, so the operands equal, bit for bit, what it writes.
template <int PAIRING>
__device__ __forceinline__ int rope_pair_index(int u, int lg) {
  return PAIRING == 0 ? 8 * (u >> 2) + 4 * lg + (u & 3) : 16 * (u >> 3) + 8 * lg + (u & 7);
}

// The lane's 16 frequencies: for each u the two candidates (lg = 0, 1) are the
// same for the whole wave, so they come from scalar loads of the table (or are
// the default table's constants) and the lane picks one; nothing here waits on
// the vector loads in flight.
typedef const float __attribute__((address_space(4))) const_f32;  // read through the scalar cache

template <int PAIRING>
__device__ __forceinline__ void rope_freqs(const PrefillArgs& a, int lg, float (&f)[16]) {
  const const_f32* tab = (const const_f32*)a.inv_freq;
  if (tab) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      float f0 = tab[rope_pair_index<PAIRING>(u, 0)], f1 = tab[rope_pair_index<PAIRING>(u, 1)];
      asm("" : "+s"(f0), "+s"(f1));  // two scalar values, then the lane's pick (not one load per lane)
      f[u] = lg ? f1 : f0;
    }
  } else {
#pragma unroll
    for (int u = 0; u < 16; ++u)
      f[u] = lg ? rope_default_freq(rope_pair_index<PAIRING>(u, 1)) : rope_default_freq(rope_pair_index<PAIRING>(u, 0));
  }
}

template <int PAIRING>
__device__ __forceinline__ void rope_angles(const PrefillArgs& a, const float (&f)[16], int p, float (&cs)[16],
                                            float (&sn)[16]) {
#pragma unroll
  for (int u = 0; u < 16; ++u) rope_cos_sin(p, f[u], a.rope_mscale, cs[u], sn[u]);
}

template <int PAIRING>
__device__ __forceinline__ void rope_rotate_q(bf16x8 (&q)[4], const float (&cs)[16], const float (&sn)[16]) {
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int k = PAIRING == 0 ? u >> 2 : u >> 3;
    const int ea = PAIRING == 0 ? 2 * (u & 3) : u & 7;
    const int kb = PAIRING == 0 ? k : k + 2;
    const int eb = PAIRING == 0 ? ea + 1 : ea;
    float ra, rb;
    rope_rotate((float)q[k][ea], (float)q[kb][eb], cs[u], sn[u], ra, rb);
    q[k][ea] = (__bf16)ra;
    q[kb][eb] = (__bf16)rb;
  }
}

// One job: the tile group x of the dispatch order (see below) of one
// (sequence, KV head).  STK: the layer keeps start-of-sequence sink tokens
// visible past its window (a separate instantiation, so that other layers
// carry none of its code).
template <int MODE, bool VARLEN, bool STK, int ROPE = 0, bool TWO = false>
__device__ __forceinline__ void prefill_job(const PrefillArgs& a, const int x, __bf16 (*Ks)[BK * RS],
                                            __bf16 (*Vs)[BK * RS], __bf16* Stg, const int* order = nullptr) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (lets per-wave values live in SGPRs)
  const int lr = lane & 31;  // row of the 32-wide MFMA tile this lane serves
  const int lg = lane >> 5;  // which half of the K dimension / which 4-row group

  // ---- which (sequence, KV head, tile group): all workgroups of one
  // (sequence, KV head) go to the same XCD (dispatch is round-robin over the 8
  // XCDs) and are dispatched back to back, heaviest tile group first, so they
  // stream the same K/V tiles at about the same time out of that XCD's L2.
  // (divisions by the launch's divisors use the launcher's multipliers: a
  // division sequence per job is a good part of a short job's setup)
  //
  // A job is one tile group or (TWO: windowed whole-sequence layers) the two
  // tile groups 2r+1 and 2r in turn.  When the job's key tiles fit the NBUF
  // buffers (the launcher asks for two steps only then, unless forced) the
  // second step reuses them: it loads no tile and repeats none of the job's
  // setup.
  const int U = a.B * a.Hkv;
  int unit, rank;
  {
    if ((U & 7) == 0) {
      const int sidx = x >> 3;
      const int sq = fast_div(sidx, a.div_wg_per_job);
      rank = sidx - sq * a.wg_per_job;
      unit = (x & 7) + 8 * sq;
    } else {
      rank = fast_div(x, a.div_units);
      unit = x - rank * U;
    }
  }
  const int jr = a.wg_per_job - 1 - rank;
  const int tg_hi = TWO ? min(2 * jr + 1, a.wg_per_seq - 1) : jr;  // steps run tg_hi down to tg_lo
  const int tg_lo = TWO ? 2 * jr : jr;
  const int uq = fast_div(unit, a.div_hkv);
  const int g = unit - uq * a.Hkv;
  const int b = order ? order[uq] : uq;  // ragged batches: longest sequences first
  const SeqView sv = seq_view<MODE>(a.seq, b, VARLEN);
  const int G = a.G;
  const int n_ntiles = ((sv.q_len + 31) >> 5) * G;
  if (tg_lo < 0 || tg_lo * NT_WG >= n_ntiles) return;  // uniform over the workgroup
  if (a.skip_single && sv.q_len == 1) return;
  const int pos_off = sv.kv_len - sv.q_len;
  const int W = a.window;
  const float c = a.scale_log2;

  // ---- key range of the whole job
  const int n_last = min(tg_hi * NT_WG + NT_WG - 1, n_ntiles - 1);
  const int t_min = fast_div(tg_lo * NT_WG, a.div_g) * 32;
  const int t_max = min(fast_div(n_last, a.div_g) * 32 + 31, sv.q_len - 1);
  const int p_min = pos_off + t_min;
  const int p_max = pos_off + t_max;
  const int lo = W > 0 ? max(0, p_min - W + 1) : 0;
  const int hi = min(p_max, sv.kv_len - 1);  // inclusive
  const int j_begin = lo & ~(BK - 1);
  // Start-of-sequence sink tokens below the window: their tiles come first
  // (tile t < n_st starts at key BK*t), then the window's tiles.
  const int st = STK && W > 0 ? a.sink_tokens : 0;
  const int n_st = STK ? (min(st, j_begin) + BK - 1) / BK : 0;
  const int n_tiles = n_st + (hi >= j_begin ? (hi - j_begin) / BK + 1 : 0);
  auto tile_j0 = [&](int t) { return t < n_st ? BK * t : j_begin + BK * (t - n_st); };

  // ---- global -> LDS staging with 16-byte direct loads: wave w fills rows
  // 16w .. 16w+15 of a tile, 8 rows per instruction.  With a paged cache the
  // block ids of the rows are fetched one tile ahead of the loads.  Rows past
  // the key range repeat row hi (they are masked, and the loads stay in bounds).
  const int64_t kv_stride = (int64_t)a.Hkv * kHeadDim;
  const __bf16* kbase = a.k + g * kHeadDim;
  const __bf16* vbase = a.v + g * kHeadDim;
  const __bf16* kbase2 = MODE == KV_RING ? a.k2 + g * kHeadDim : nullptr;
  const __bf16* vbase2 = MODE == KV_RING ? a.v2 + g * kHeadDim : nullptr;
  const int dma_chunk = ((lane & 7) ^ kswz(lane >> 3)) * 8;  // logical chunk this lane's LDS slot holds
  // LDS byte addresses of the buffers, formed once (a cast per load would
  // test the address for null each time)
  const uint32_t ks_lds = lds_addr((lds_void*)&Ks[0][0]);
  const uint32_t vs_lds = lds_addr((lds_void*)&Vs[0][0]);
  auto fetch_blk = [&](int t, int (&blk)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      blk[i] = 0;
      if (MODE == KV_PAGED) {
        const int j = min(tile_j0(t) + 16 * wave + 8 * i + (lane >> 3), hi);
        blk[i] = a.seq.block_table[(int64_t)b * a.seq.max_blocks + (j >> a.seq.log2_block)];
      }
    }
  };
  auto dma_tile = [&](int t, const int (&blk)[2], int buf) {
    if constexpr (MODE == KV_BATCHED) {
      // a scalar base per tile and a 32-bit offset per lane (the tile's rows
      // are consecutive cache rows); rows past hi repeat row hi
      const int j0 = tile_j0(t);
      const int64_t tb = ((int64_t)sv.b * a.seq.lmax + j0) * kv_stride;
      const char* kt = reinterpret_cast<const char*>(kbase + tb);
      const char* vt = reinterpret_cast<const char*>(vbase + tb);
      uint32_t off[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = min(16 * wave + 8 * i + (lane >> 3), hi - j0);
        off[i] = (__umul24(r, (uint32_t)kv_stride) + dma_chunk) * 2u;  // r < 64: 24-bit product
      }
      const uint32_t lofs = (uint32_t)(buf * BK * RS + 16 * wave * RS) * 2u;  // wave-uniform slice of 16 rows
      constexpr uint32_t kHalf = 8 * RS * 2;                                  // its second 8 rows
      dma16_kv(kt, vt, off[0], off[1], ks_lds + lofs, ks_lds + lofs + kHalf, vs_lds + lofs, vs_lds + lofs + kHalf);
      return;
    }
    const void* ka[2];
    const void* va[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int j = min(tile_j0(t) + 16 * wave + 8 * i + (lane >> 3), hi);
      int64_t row;
      const __bf16* kb = kbase;
      const __bf16* vb = vbase;
      if (MODE == KV_PAGED) {
        const int bb = min(max(blk[i], 0), a.seq.num_blocks - 1);
        GQA_FLAG(bb != blk[i], kDbgBlockTable);
        row = ((int64_t)bb << a.seq.log2_block) + (j & ((1 << a.seq.log2_block) - 1));
      } else if (MODE == KV_RING) {
        // ring_chunk_row with the slot taken by the launch's multiplier
        // instead of a division sequence per row
        const int jc = sv.kv_len - sv.q_len;
        row = j >= jc ? -1 - (sv.q_row0 + (j - jc))
                      : (int64_t)sv.b * a.seq.lmax + (j - fast_div(j, a.div_ring) * a.seq.lmax);
        if (row < 0) {  // the chunk's own row
          row = -1 - row;
          kb = kbase2;
          vb = vbase2;
        }
      } else {
        row = kv_row<MODE>(a.seq, sv, j);
      }
      const int64_t off = row * kv_stride + dma_chunk;
      ka[i] = kb + off;
      va[i] = vb + off;
    }
    const uint32_t lofs = (uint32_t)(buf * BK * RS + 16 * wave * RS) * 2u;  // wave-uniform slice of 16 rows
    constexpr uint32_t kHalf = 8 * RS * 2;                                  // its second 8 rows
    dma16_kv(ka[0], ka[1], va[0], va[1], ks_lds + lofs, ks_lds + lofs + kHalf, vs_lds + lofs, vs_lds + lofs + kHalf);
  };


  // Per-lane element offsets of the transposing V reads (see pv_half).
  int vofs[2];
  tr_offsets(lane, vofs);

  // ---- Q^T operands (B of S^T = K Q^T) of tile group tg's N-tiles: lane holds
  // row lr, d = 16*k + 8*lg .. +7.  Unconditional loads: a row past the end
  // reads the sequence's last row (its head is valid; its results are never
  // stored).  Without branches around the loads the compiler keeps each
  // operand where its load puts it, so nothing waits for them before their
  // first use (the rotation, or the first scores).  The N-tile's first row is
  // a scalar base, the lane's row a 32-bit offset.
  bf16x8 qb[2][4];
  auto load_q = [&](int tg_q) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int n = tg_q * NT_WG + wave * 2 + i;
      const int pb = fast_div(n, a.div_g);
      const int t0 = min(pb * 32, sv.q_len - 1);
      const int r = min(pb * 32 + lr, sv.q_len - 1) - t0;  // 0 .. 31
      const int hq = g * G + (n - pb * G);
      const char* qt = reinterpret_cast<const char*>(a.q + ((sv.q_row0 + t0) * a.Hq + hq) * (int64_t)kHeadDim);
      const uint32_t qo = (uint32_t)(r * a.Hq * kHeadDim + 8 * lg) * 2u;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        qb[i][k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qt + qo + 32 * k));
    }
  };
  load_q(tg_hi);

  const int n_steps = tg_hi - tg_lo + 1;
  // (unrolled, so that each step's code is specialised for it; the two-step
  // kernel has one tile loop per step to stay within the instruction cache)
#pragma unroll
  for (int step = 0; step < (TWO ? 2 : 1); ++step) {
  if (step >= n_steps) break;  // uniform
  const int tg = tg_hi - step;

  // ---- this wave's two N-tiles
  int nt_t0[2], nt_hq[2], pos0[2], phi[2];
  bool nt_valid[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int n = tg * NT_WG + wave * 2 + i;
    nt_valid[i] = n < n_ntiles;
    const int pb = fast_div(n, a.div_g);
    nt_t0[i] = pb * 32;
    nt_hq[i] = g * G + (n - pb * G);
    pos0[i] = pos_off + nt_t0[i];
    phi[i] = pos_off + min(nt_t0[i] + 31, sv.q_len - 1);
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


  // Tile t runs in three phases, each pairing vector work with independent
  // matrix work so that both units stay busy within the wave:
  //   (a) weights of key half 0          | scores of key half 1
  //   (b) weights of key half 1          | P V over key half 0
  //   -- wait for tile t+1's loads, barrier: tile t+1 is in LDS --
  //   (c) P V over key half 1            | scores of key half 0 of tile t+1
  //       and the loads of tile t+2 are issued
  // Three LDS buffers: tile t is read until (c) of tile t, tile t+1 from (c)
  // of tile t on, and tile t+2 lands in the buffer that tile t-1 left, which
  // every wave finished reading before the barrier of tile t.
  f32x16 sA[2], sB[2];  // scores of key halves 0 and 1, per N-tile
  int blk_next[2];      // block ids of the next tile to load
  // A later step finds every tile in LDS when the job's tiles fit the buffers
  // (the launcher asks for two steps only then); otherwise it streams them
  // again, once every wave is done with the previous step's.
  const bool load = step == 0 || n_tiles > NBUF;
  if (n_tiles > 0) {
    if (load) {
      if (step > 0) __syncthreads();
      int blk0[2];
      fetch_blk(0, blk0);
      dma_tile(0, blk0, 0);
      fetch_blk(1, blk0);
      if (n_tiles > 1) dma_tile(1, blk0, 1);
      fetch_blk(2, blk_next);
    }
    if constexpr (ROPE != 0) {
      // the angles go while the loads fly; the rotation once Q has landed
      float f[16], cs[16], sn[16];
      rope_freqs<ROPE - 1>(a, lg, f);
      rope_angles<ROPE - 1>(a, f, pos0[0] + lr, cs, sn);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      rope_rotate_q<ROPE - 1>(qb[0], cs, sn);
      if (nt_t0[1] != nt_t0[0]) rope_angles<ROPE - 1>(a, f, pos0[1] + lr, cs, sn);
      rope_rotate_q<ROPE - 1>(qb[1], cs, sn);
    }
    if (load) {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
    }
    qk_half(sA[0], sA[1], Ks[0], qb, 0, lr, lg);
    int cur = 0;
    auto body = [&](auto mask_tag, auto h1_tag, int t) {
      constexpr bool MASK = decltype(mask_tag)::value;
      constexpr bool H1 = decltype(h1_tag)::value;  // false: key half 1 is masked for every row (skipped)
      const int nxt = cur == NBUF - 1 ? 0 : cur + 1;
      const int j0 = tile_j0(t);
      const bool has_next = t + 1 < n_tiles;
      const int dh0 = pos0[0] + lr - j0 - 4 * lg, dh1 = pos0[1] + lr - j0 - 4 * lg;
      const int dl0 = W > 0 ? dh0 - W : -0x40000000, dl1 = W > 0 ? dh1 - W : -0x40000000;
      const int ds = STK ? st - j0 - 4 * lg : 0;  // off < ds: a sink token
      bf16x8 pA0[2], pA1[2], pB0[2], pB1[2];
      // Issue priority on dense layers, by phase: (b) 2, (a) 1, (c) 0.  Of the
      // two waves of a SIMD, one in its exponential phases goes before one in
      // its matrix-only phase (c), so the vector unit is not left idle behind
      // the older wave's MFMAs (measured: 10 % on dense layers over equal
      // priorities; windowed layers, whose jobs are mostly masked edge tiles,
      // ran a little slower with it).
      if (W == 0) __builtin_amdgcn_s_setprio(1);
      // (a): the four k-steps of the half-1 scores, each followed by a quarter
      // of the half-0 exponentials (the order is pinned so that every MFMA
      // pair runs while the vector work after it issues)
      if (MASK) {
        mask_half<STK>(sA[0], 0, j0, pos0[0], phi[0], W, st, dh0, dl0, ds);
        mask_half<STK>(sA[1], 0, j0, pos0[1], phi[1], W, st, dh1, dl1, ds);
      }
      float r0, r1;  // set by the first exponential chunk of each N-tile
      {
        bf16x8 ka[4];
        if (H1) {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            ka[k] = *reinterpret_cast<const bf16x8*>(Ks[cur] + (32 + lr) * RS + kchunk(2 * k + lg, lr));
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          fence_schedule();
          if (H1) {
            sB[0] = mfma32(ka[k], qb[0][k], k == 0 ? zero16() : sB[0]);
            sB[1] = mfma32(ka[k], qb[1][k], k == 0 ? zero16() : sB[1]);
          }
          fence_schedule();
          if (k == 0) r0 = exp_chunk(sA[0], pA0[k], k, m_run[0], c);
          else if (k == 1) r0 += exp_chunk(sA[0], pA0[k], k, m_run[0], c);
          else if (k == 2) r1 = exp_chunk(sA[1], pA1[k - 2], k - 2, m_run[1], c);
          else r1 += exp_chunk(sA[1], pA1[k - 2], k - 2, m_run[1], c);
        }
        fence_schedule();
      }
      {
        const bool f0 = __builtin_amdgcn_ballot_w64(r0 > kRefit) != 0;
        const bool f1 = __builtin_amdgcn_ballot_w64(r1 > kRefit) != 0;
        float al0 = 1.f, al1 = 1.f;
        if (f0) r0 = refit_half<STK>(sA[0], pA0, m_run[0], l_run[0], al0, Ks[cur], qb[0], 0, lr, lg, c, j0, pos0[0], phi[0], W, st, dh0, dl0, ds);
        if (f1) r1 = refit_half<STK>(sA[1], pA1, m_run[1], l_run[1], al1, Ks[cur], qb[1], 0, lr, lg, c, j0, pos0[1], phi[1], W, st, dh1, dl1, ds);
        if (f0) { o[0][0] *= al0; o[0][1] *= al0; }
        if (f1) { o[1][0] *= al1; o[1][1] *= al1; }
      }
      l_run[0] += r0;
      l_run[1] += r1;
      if (W == 0) __builtin_amdgcn_s_setprio(2);
      // (b): P V over key half 0 in four steps, each followed by a quarter of
      // the half-1 exponentials
      if (MASK && H1) {
        mask_half<STK>(sB[0], 1, j0, pos0[0], phi[0], W, st, dh0, dl0, ds);
        mask_half<STK>(sB[1], 1, j0, pos0[1], phi[1], W, st, dh1, dl1, ds);
      }
      {
        bf16x8 va[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) va[i] = tr_operand(Vs[cur], i >> 1, i & 1, vofs);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int uu = i >> 1, dt = i & 1;
          fence_schedule();
          o[0][dt] = mfma32(va[i], pA0[uu], o[0][dt]);
          o[1][dt] = mfma32(va[i], pA1[uu], o[1][dt]);
          fence_schedule();
          if (!H1) continue;
          if (i == 0) r0 = exp_chunk(sB[0], pB0[i], i, m_run[0], c);
          else if (i == 1) r0 += exp_chunk(sB[0], pB0[i], i, m_run[0], c);
          else if (i == 2) r1 = exp_chunk(sB[1], pB1[i - 2], i - 2, m_run[1], c);
          else r1 += exp_chunk(sB[1], pB1[i - 2], i - 2, m_run[1], c);
        }
        fence_schedule();
      }
      if (H1) {
        const bool f0 = __builtin_amdgcn_ballot_w64(r0 > kRefit) != 0;
        const bool f1 = __builtin_amdgcn_ballot_w64(r1 > kRefit) != 0;
        float al0 = 1.f, al1 = 1.f;
        if (f0) r0 = refit_half<STK>(sB[0], pB0, m_run[0], l_run[0], al0, Ks[cur], qb[0], 1, lr, lg, c, j0, pos0[0], phi[0], W, st, dh0, dl0, ds);
        if (f1) r1 = refit_half<STK>(sB[1], pB1, m_run[1], l_run[1], al1, Ks[cur], qb[1], 1, lr, lg, c, j0, pos0[1], phi[1], W, st, dh1, dl1, ds);
        if (f0) { o[0][0] *= al0; o[0][1] *= al0; }
        if (f1) { o[1][0] *= al1; o[1][1] *= al1; }
        l_run[0] += r0;
        l_run[1] += r1;
      }
      if (load) {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's loads of tile t+1 have landed
        __syncthreads();
      }
      if (W == 0) __builtin_amdgcn_s_setprio(0);
      // (c)
      if (load && t + 2 < n_tiles) dma_tile(t + 2, blk_next, nxt == NBUF - 1 ? 0 : nxt + 1);
      fetch_blk(t + 3, blk_next);
      if (H1) pv_half(o, Vs[cur], pB0, pB1, 1, vofs);
      if (has_next) qk_half(sA[0], sA[1], Ks[nxt], qb, 0, lr, lg);
      cur = nxt;
    };
    // The window tiles that need no mask for either of this wave's N-tiles
    // form one run [pb, pe): past the window edge of the last row and before
    // the causal diagonal of the first row.  Three loops, one body each (the
    // sink tiles lead the first).
    const int p_first = min(pos0[0], pos0[1]);
    const int p_last = max(phi[0], phi[1]);
    const int t_lo = W > 0 ? max(0, (p_last - W - j_begin + BK) / BK) : 0;  // first t with j0 > p_last - W
    const int t_hi = p_first - j_begin - (BK - 1) >= 0 ? (p_first - j_begin - (BK - 1)) / BK : -1;  // last t with j0 + 63 <= p_first
    const int n_wt = n_tiles - n_st;  // window tiles; the sink tiles all take the masked body
    const int pb = n_st + min(t_lo, n_wt);
    const int pe = max(pb, n_st + min(t_hi + 1, n_wt));
    std::true_type MSK, FULL;
    std::false_type PLN, HALF0;
    if (TWO) {
      // at most NBUF tiles, mostly edges: one (masked) body keeps the code of
      // both steps within the instruction cache
      for (int t = 0; t < n_tiles; ++t) body(MSK, FULL, t);
    } else {
      int t = 0;
      // One sink tile holding at most 32 sink tokens: its key half 1 lies
      // below the window and past the sink tokens, so every row masks it, and
      // the tile runs key half 0 only (the skipped half adds exact zeros).
      if (STK && n_st == 1 && st <= BK / 2) body(MSK, HALF0, t++);
      for (; t < pb; ++t) body(MSK, FULL, t);
      for (int t = pb; t < pe; ++t) body(PLN, FULL, t);
      for (int t = pe; t < n_tiles; ++t) body(MSK, FULL, t);
    }
  }
  // the next step's queries load while this step's output goes out
  if (TWO && step + 1 < n_steps) load_q(tg_hi - step - 1);

  // ---- epilogue: normalise, round to bf16, log-sum-exp.  A lane's registers
  // hold 4-element pieces of 32 different rows, so the output tile goes
  // through LDS and leaves as whole 128-byte rows (8 lanes per row, 16 bytes
  // each) instead of 16 partial writes per row.
  // The row index is re-derived here behind an empty asm, so the compiler does
  // not keep the prologue's 64-bit Q row offset alive across the tile loops
  // (it would spill it).
  int lr_e = lr;
  asm volatile("" : "+v"(lr_e));
  // The wave's rows go through LDS: all 64 ([N-tile][row][64]) in a free K/V
  // buffer once every wave is done with the tiles, or (two steps: the tiles
  // stay) one N-tile at a time through the wave's own 32-row slice.
  constexpr int NP = TWO ? 1 : 2;  // N-tiles per staging pass
  __bf16* stg;
  if (TWO) {
    stg = Stg + wave * 32 * RS;
  } else {
    __syncthreads();
    stg = wave < NBUF ? Ks[wave] : Vs[0];
  }
#pragma unroll
  for (int ps = 0; ps < 2 / NP; ++ps) {
#pragma unroll
    for (int ii = 0; ii < NP; ++ii) {
      const int i = ps * NP + ii;
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run[i]), __float_as_uint(l_run[i]), false, false);
      const float lt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      const float inv = lt > 0.f ? 1.f / lt : (lt == 0.f ? 0.f : lt);
      const int row = 32 * ii + lr_e;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int cq = 0; cq < 4; ++cq) {
          u32x2 v;
          v[0] = pack_bf16x2(o[i][dt][4 * cq + 0] * inv, o[i][dt][4 * cq + 1] * inv);
          v[1] = pack_bf16x2(o[i][dt][4 * cq + 2] * inv, o[i][dt][4 * cq + 3] * inv);
          *reinterpret_cast<u32x2*>(stg + row * RS + kchunk(4 * dt + cq, row) + 4 * lg) = v;  // d = 32dt + 8cq + 4lg
        }
      const int t = nt_t0[i] + lr_e;
      if (nt_valid[i] && t < sv.q_len && a.lse && lg == 0) {
        const float v = (lt == 0.f) ? -INFINITY : (m_run[i] + __log2f(lt)) * kLn2;
        const int64_t idx = (int64_t)b * a.lse_sb + (int64_t)nt_hq[i] * a.lse_sh + t + (a.lse_row0 ? sv.q_row0 : 0);
        a.lse[idx] = v;
      }
    }
    wave_lds_sync();  // the wave reads back only its own rows
    // rows 8j .. 8j+7 of the staged ones: N-tile j / 4 of the pass, row
    // (lane / 8) + 8 (j % 4) of it, 16-byte chunk lane % 8
    u32x4 ov[4 * NP];
#pragma unroll
    for (int j = 0; j < 4 * NP; ++j) {
      const int r = (lane >> 3) + 8 * (j & 3);
      ov[j] = *reinterpret_cast<const u32x4*>(stg + (32 * (j >> 2) + r) * RS + kchunk(lane & 7, r));
    }
    if (TWO) wave_lds_sync();  // read back before the next pass writes the slice
    auto store = [&](int j) {
      const int i = ps * NP + (j >> 2);
      const int r = (lane >> 3) + 8 * (j & 3);
      char* ot = reinterpret_cast<char*>(a.out + ((sv.q_row0 + nt_t0[i]) * a.Hq + nt_hq[i]) * (int64_t)kHeadDim);
      *reinterpret_cast<u32x4*>(ot + (uint32_t)(r * a.Hq * kHeadDim + 8 * (lane & 7)) * 2u) = ov[j];
    };
    // the pass's N-tiles whole (every tile but a sequence's last): no per-row tests
    bool whole = true;
#pragma unroll
    for (int ii = 0; ii < NP; ++ii) whole = whole && nt_valid[ps * NP + ii] && nt_t0[ps * NP + ii] + 31 < sv.q_len;
    if (whole) {
#pragma unroll
      for (int j = 0; j < 4 * NP; ++j) store(j);
    } else {
#pragma unroll
      for (int j = 0; j < 4 * NP; ++j) {
        const int i = ps * NP + (j >> 2);
        if (nt_valid[i] && nt_t0[i] + (lane >> 3) + 8 * (j & 3) < sv.q_len) store(j);
      }
    }
  }
  }  // step
}

template <int MODE, bool VARLEN, bool STK, int ROPE = 0, bool TWO = false>
__global__ __launch_bounds__(NTHREADS, 2) void prefill_bf16_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 Ks[NBUF][BK * RS];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[NBUF][BK * RS];
  // output staging of two-step jobs: 4 waves x 32 rows (so that two
  // workgroups' LDS fits a CU with room to spare)
  __shared__ __attribute__((aligned(16))) __bf16 Stg[TWO ? 4 * 32 * RS : 8];
  const int* order = nullptr;
  if constexpr (VARLEN) {
    // Ragged batches: the sequences' tile groups carry work in proportion to
    // their query and key counts, so the workgroups take the sequences from
    // the most work to the least (as far as the dispatch order goes), instead
    // of in batch order where a long sequence dispatched last runs alone at
    // the end.  Every workgroup ranks the (at most kSortMax) sequences itself.
    __shared__ float seq_w[kSortMax];
    __shared__ int seq_order[kSortMax];
    if (a.sort_seq) {
      const int t = threadIdx.x;
      const int B = a.B;
      if (t < B) {
        const SeqView sv = seq_view<MODE>(a.seq, t, true);
        const int kl = a.window > 0 ? min(sv.kv_len, sv.q_len + a.window) : sv.kv_len;
        seq_w[t] = (a.skip_single && sv.q_len <= 1) ? 0.f : (float)sv.q_len * (float)kl;
      }
      __syncthreads();
      if (t < B) {
        const float w = seq_w[t];
        int r = 0;
        for (int j = 0; j < B; ++j) {
          const float wj = seq_w[j];
          r += (wj > w) || (wj == w && j < t);
        }
        seq_order[r] = t;
      }
      __syncthreads();
      order = seq_order;
    }
  }
  prefill_job<MODE, VARLEN, STK, ROPE, TWO>(a, blockIdx.x, Ks, Vs, Stg, order);  // one call site: inlined once
}

}  // namespace

int prefill_ntiles_per_wg() { return NT_WG; }

hipError_t launch_prefill_bf16(const PrefillArgs& args, int kv_mode, bool varlen_q, hipStream_t s) {
  // (not with the rotation: its extra registers spill in the two-step kernel,
  // which then ran 4-6 % slower than one step)
  const bool two = kv_mode == KV_BATCHED && !varlen_q && args.two_step && !(args.window > 0 && args.sink_tokens > 0) &&
                   !args.rope;
  const int wg_per_job = two ? (args.wg_per_seq + 1) / 2 : args.wg_per_seq;
  const int grid = args.B * args.Hkv * wg_per_job;
  if (grid <= 0) return hipSuccess;
  PrefillArgs a = args;
  a.two_step = two;
  a.wg_per_job = wg_per_job;
  a.div_wg_per_job = make_fastdiv(wg_per_job);
  a.div_hkv = make_fastdiv(a.Hkv);
  a.div_g = make_fastdiv(a.G);
  a.div_units = make_fastdiv(a.B * a.Hkv);
  a.div_ring = make_fastdiv(a.seq.lmax > 0 ? a.seq.lmax : 1);
  const bool stk = a.window > 0 && a.sink_tokens > 0;
  if (a.rope) {  // queries rotated in the kernel: whole-sequence prefill only
    if (kv_mode != KV_BATCHED || varlen_q) return hipErrorInvalidValue;
#define GQA_ROPE_LAUNCH(R)                                                                                          \
  do {                                                                                                              \
    if (stk) hipLaunchKernelGGL((prefill_bf16_kernel<KV_BATCHED, false, true, R>), dim3(grid), dim3(NTHREADS), 0, s, a); \
    else hipLaunchKernelGGL((prefill_bf16_kernel<KV_BATCHED, false, false, R>), dim3(grid), dim3(NTHREADS), 0, s, a);    \
  } while (0)
    if (a.rope == 1) GQA_ROPE_LAUNCH(1);
    else GQA_ROPE_LAUNCH(2);
#undef GQA_ROPE_LAUNCH
    return hipGetLastError();
  }
#define GQA_LAUNCH(M, V)                                                                               \
  do {                                                                                                 \
    if (stk) hipLaunchKernelGGL((prefill_bf16_kernel<M, V, true>), dim3(grid), dim3(NTHREADS), 0, s, a); \
    else hipLaunchKernelGGL((prefill_bf16_kernel<M, V, false>), dim3(grid), dim3(NTHREADS), 0, s, a);    \
  } while (0)
  if (!varlen_q && kv_mode == KV_BATCHED && two)
    hipLaunchKernelGGL((prefill_bf16_kernel<KV_BATCHED, false, false, 0, true>), dim3(grid), dim3(NTHREADS), 0, s, a);
  else if (!varlen_q && kv_mode == KV_BATCHED)
    GQA_LAUNCH(KV_BATCHED, false);
  else if (varlen_q && kv_mode == KV_PAGED)
    GQA_LAUNCH(KV_PAGED, true);
  else if (varlen_q && kv_mode == KV_PACKED)
    GQA_LAUNCH(KV_PACKED, true);
  else if (varlen_q && kv_mode == KV_RING && !stk)
    hipLaunchKernelGGL((prefill_bf16_kernel<KV_RING, true, false>), dim3(grid), dim3(NTHREADS), 0, s, a);
  else
    return hipErrorInvalidValue;
#undef GQA_LAUNCH
  return hipGetLastError();
}

// Metadata-check flags of this file's kernels (recorded only when built with GQA_DEBUG).
GQA_DEBUG_FLAGS_ACCESSOR(debug_flags_prefill)

}  // namespace gqa
