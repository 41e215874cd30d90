// Backward of the prefill on gfx950: gradients of sink + window causal GQA
// attention with respect to q, k, v and the per-head sink logits.
//
// The forward is the attention of «GPT-OSS vs Qwen3» (sections "Introduction
// de Grouped Query Attention", "Utilisation de Sliding Window Attention",
// "Attention Bias et Sinks") with the head layout of «GPT-OSS-20B :
// Architecture MoE & Résumé du Model Card» §3.3; training it (§5 of the same
// page) needs its derivative.  For query head h (KV head g) at position p,
// with the forward's log-sum-exp lse (sink included) and dO = dL/do:
//
//   P_j  = exp(scale <q, k_j> - lse)          weights, recomputed from lse
//   D    = <dO, o>                            = sum_j P_j <dO, v_j>
//   dS_j = P_j (<dO, v_j> - D)                gradient of the logit x_j
//   dq   = scale sum_j dS_j k_j
//   dk_j = scale sum_{p, h in g} dS_j q       dv_j = sum_{p, h in g} P_j dO
//   dsink_h = -sum_p exp(s_h - lse) D         (the sink has no value vector)
//
// The launches, all deterministic (no atomics):
//   1. D per (row, head) from o and dO (bandwidth-bound);
//   2. lse in log2 units and block sums of the sink gradient, then dsinks
//      as the sum of those in a fixed order;
//   3. dK/dV: a workgroup owns 64 keys of one KV head; query tiles of 32
//      positions x 2 heads of the group are staged in LDS (16-byte direct
//      loads, three buffers, two units ahead) and every wave computes, for its
//      32 keys and one of the two heads, S = Q K^T and dP = dO V^T
//      (v_mfma_f32_32x32x16_bf16, K and V rows held in registers as the B
//      operand), the weights P and dS in registers, and accumulates
//      dV += P^T dO and dK += dS^T Q with the score tile itself as the A
//      operand (a lane holds one key and 16 queries, the row order of the
//      contraction) and dO, Q read through the transposing LDS load.  The two
//      waves that share keys but differ in head add their sums through LDS at
//      the end; the result goes out as whole 128-byte rows.  Under the causal
//      mask the first key block sees every query and the last one only its
//      own, so when there are few key blocks per slot of the chip, the query
//      range is cut into up to 4 slabs, each its own workgroup: a key block
//      with several slabs writes fp32 partial sums that a small kernel adds
//      in slab order (deterministic), and one with a single slab writes bf16
//      directly.
//   4. dQ: the forward's decomposition (8 N-tiles of 32 positions x one head
//      per workgroup, K/V tiles staged as in the forward): S^T = K Q^T and
//      dP^T = V dO^T with Q and dO rows in registers, then dQ^T += K^T dS^T.
// Recomputing S and dP in launch 4 costs 6 of its 12 matrix products per key
// block; it buys freedom from atomics on dQ.
#include <algorithm>
#include <type_traits>

#include "kernels.h"
#include "tile_ops.h"

namespace gqa {
namespace {

constexpr int BT = 256;   // threads per workgroup (4 waves)
constexpr int KB = 64;    // keys per dK/dV workgroup
constexpr int QT = 32;    // query positions per staged dK/dV unit
constexpr int BK = 64;    // keys per dQ tile
constexpr int NT_WG = 8;  // dQ: N-tiles (32 positions of one head) per workgroup, two per wave
constexpr int NBUF = 3;   // staged units / tiles resident in LDS

// ---------------------------------------------------------------------------
// 1. D = <dO, o> per (row, head): one wave per (sequence, position) row; the
// lanes walk the row's 16-byte chunks (the heads of a position are
// contiguous) and the lanes of one head add up.
template <typename T>
__global__ __launch_bounds__(BT) void bwd_dot_kernel(BwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (BT / 64) + (threadIdx.x >> 6);
  if (row >= (int64_t)a.B * a.S) return;
  const int b = (int)(row / a.S);
  const int s = (int)(row - (int64_t)b * a.S);
  constexpr int cph = 64 * (int)sizeof(T) / 16;  // 16-byte chunks per head: 8 (bf16) or 16 (fp32)
  const int chunks = a.Hq * cph;
  const u32x4* o = reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(a.o) + row * a.Hq * kHeadDim);
  const u32x4* g = reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(a.dout) + row * a.Hq * kHeadDim);
  for (int c0 = 0; c0 < chunks; c0 += 64) {
    const int c = c0 + lane;  // 64 % cph == 0: the lanes of one head are all in range or all out
    float acc = 0.f;
    if (c < chunks) {
      const u32x4 x = o[c], y = g[c];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (sizeof(T) == 2)
          acc += bf16_lo(x[e]) * bf16_lo(y[e]) + bf16_hi(x[e]) * bf16_hi(y[e]);
        else
          acc += __uint_as_float(x[e]) * __uint_as_float(y[e]);
      }
    }
#pragma unroll
    for (int m = 1; m < cph; m <<= 1) acc += __shfl_xor(acc, m, 64);
    if (c < chunks && (lane & (cph - 1)) == 0) a.dlt[((int64_t)b * a.Hq + c / cph) * a.S + s] = acc;
  }
}

// ---------------------------------------------------------------------------
// 2. Per (sequence, head, block of SB positions): the log-sum-exp copied in
// log2 units (as the exponentials take it), and the block's share of the sink
// gradient, -sum exp(s_h - lse) D, summed in a fixed order (strided per
// thread, then a tree).
constexpr int SB = 1024;
__global__ __launch_bounds__(BT) void bwd_rowstat_kernel(BwdArgs a) {
  __shared__ float red[BT];
  const int nsb = (a.S + SB - 1) / SB;
  const int x = blockIdx.x;
  const int sb = x % nsb;
  const int bh = x / nsb;  // b * Hq + h
  const int h = bh % a.Hq;
  const float s2 = a.sinks ? a.sinks[h] * kLog2e : -INFINITY;
  const int p_end = min(a.S, (sb + 1) * SB);
  float acc = 0.f;
  for (int p = sb * SB + threadIdx.x; p < p_end; p += BT) {
    const int64_t idx = (int64_t)bh * a.S + p;
    const float l2 = a.lse[idx] * kLog2e;
    a.lse2[idx] = l2;
    acc -= fast_exp2(s2 - l2) * a.dlt[idx];
  }
  if (!a.dsinks) return;
  red[threadIdx.x] = acc;
  __syncthreads();
#pragma unroll
  for (int w = BT / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.dsink_part[(int64_t)h * a.B * nsb + (int64_t)(bh / a.Hq) * nsb + sb] = red[0];
}

// dsinks[h]: the partial sums of its (sequence, block) pairs in order.
__global__ __launch_bounds__(64) void bwd_dsink_kernel(BwdArgs a) {
  const int h = blockIdx.x * 64 + threadIdx.x;
  if (h >= a.Hq) return;
  const int n = a.B * ((a.S + SB - 1) / SB);
  float acc = 0.f;
  for (int i = 0; i < n; ++i) acc += a.dsink_part[(int64_t)h * n + i];
  a.dsinks[h] = acc + 0.f;
}

// Last query position that can see a key of the 64-key block starting at j0:
// the sequence end, or the window of the block's last key unless the block
// holds sink tokens (st: the sink tokens of a windowed layer, else 0).
__device__ __forceinline__ int block_p_hi(int j0, int S, int W, int st) {
  const int kmax = min(j0 + KB - 1, S - 1);
  return (W > 0 && j0 >= st) ? min(S - 1, kmax + W - 1) : S - 1;
}

// ---------------------------------------------------------------------------
// 3. dK, dV (bf16).  Workgroup = (sequence b, KV head g, 64-key block); wave w
// owns keys 32*(w%2) .. +31 of the block and, of each staged head pair, head
// w/2.  A staged unit is (query tile of 32 positions, head pair 2i, 2i+1):
// Q and dO rows [2 heads][32][64] in the swizzled row layout, lse and D
// [2 heads][32].
template <bool STK>
__global__ __launch_bounds__(BT, 2) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int TILE = 2 * QT * RS;  // elements of one staged Q (or dO) unit: 8 KB
  __shared__ __attribute__((aligned(16))) __bf16 smem_b[NBUF * 2 * TILE];  // 48 KB
  __shared__ __attribute__((aligned(16))) float smem_f[NBUF * 4 * QT];
  const __bf16* q = reinterpret_cast<const __bf16*>(a.q);
  const __bf16* k = reinterpret_cast<const __bf16*>(a.k);
  const __bf16* v = reinterpret_cast<const __bf16*>(a.v);
  const __bf16* dout = reinterpret_cast<const __bf16*>(a.dout);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lr = lane & 31;
  const int lg = lane >> 5;
  const int kh = wave & 1;   // key half of the block
  const int hh = wave >> 1;  // head of each staged pair

  const int S = a.S, G = a.G, W = a.window;
  const int nkb = (S + KB - 1) / KB;
  // All key blocks of one (sequence, KV head) go to one XCD (dispatch is
  // round-robin over the 8 XCDs), the longest first: they stream the same
  // Q / dO rows out of that XCD's L2.
  const int U = a.B * a.Hkv;
  const int per_unit = nkb * a.n_slabs;  // (slab, key block) jobs of one (sequence, KV head)
  // (divisions by the launch's divisors use the launcher's multipliers)
  int unit, r;
  {
    const int x = blockIdx.x;
    if ((U & 7) == 0) {
      const int sidx = x >> 3;
      const int sq = fast_div(sidx, a.div_per_unit);
      r = sidx - sq * per_unit;
      unit = (x & 7) + 8 * sq;
    } else {
      r = fast_div(x, a.div_units);
      unit = x - r * U;
    }
  }
  const int slab = fast_div(r, a.div_nkb);
  const int kb = r - slab * nkb;
  const int b = fast_div(unit, a.div_hkv);
  const int g = unit - b * a.Hkv;
  const int st = STK && W > 0 ? a.sink_tokens : 0;
  const int j0 = kb * KB;
  const int jw = j0 + 32 * kh;  // this wave's first key
  // queries that can see a key of the block: p >= j0 up to p_hi; this
  // workgroup takes those of its slab
  const int p_hi = block_p_hi(j0, S, W, st);
  const int s_lo = fast_div(j0, a.div_slab_len), s_hi = fast_div(p_hi, a.div_slab_len);
  if (slab < s_lo || slab > s_hi) return;  // uniform: the slab holds no query of the block
  const bool partial = s_hi > s_lo;
  const int t_lo = max(j0, slab * a.slab_len) / QT;
  const int n_qt = min(p_hi, (slab + 1) * a.slab_len - 1) / QT - t_lo + 1;
  const int np = (G + 1) >> 1;  // head pairs
  const int n_units = n_qt * np;

  // K and V rows of this wave's keys as B operands (column = key, k = d)
  const int64_t kv_stride = (int64_t)a.Hkv * kHeadDim;
  bf16x8 kop[4], vop[4];
  {
    const int jr = min(jw + lr, S - 1);
    const int64_t off = ((int64_t)b * S + jr) * kv_stride + g * kHeadDim + 8 * lg;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      kop[kk] = *reinterpret_cast<const bf16x8*>(k + off + 16 * kk);
      vop[kk] = *reinterpret_cast<const bf16x8*>(v + off + 16 * kk);
    }
  }
  // Let these loads land here: a wait for them left to the compiler would sit
  // inside the unit loop, where it would also wait for the staging loads in
  // flight (issued from asm, so not counted by the compiler).
  __builtin_amdgcn_s_waitcnt(kWaitVm0);

  // Staging of a unit (q-tile t, head pair i): wave w fills rows 16w .. 16w+15
  // of the Q and dO tiles (row R = head R / 32 of the pair, query R % 32), 8
  // rows per load; wave 0 also loads lse (log2 units) and D (lane l: head
  // l / 32, query l % 32).  Addresses are a scalar base per unit plus a
  // per-lane 32-bit offset; on the last tile, and for the missing second head
  // of an odd group, rows repeat valid ones (masked, and in bounds).
  const int64_t q_stride = (int64_t)a.Hq * kHeadDim;
  const int dma_chunk = ((lane & 7) ^ kswz(lane >> 3)) * 8;
  uint32_t qoff[2];
#pragma unroll
  for (int ii = 0; ii < 2; ++ii) {
    const int R = 16 * wave + 8 * ii + (lane >> 3);
    qoff[ii] = (uint32_t)((((R & 31) * a.Hq + (R >> 5)) * kHeadDim + dma_chunk) * 2);
  }
  const uint32_t loff = (uint32_t)((lg * S + lr) * 4);
  const uint32_t smem_lds = lds_addr((lds_void*)smem_b);  // formed once: a cast per load tests for null
  auto dma_unit = [&](int t, int i, int buf) {
    const int q0 = (t_lo + t) * QT;
    const bool fast = q0 + QT <= S && 2 * i + 1 < G;  // uniform
    const int64_t ubase = ((int64_t)b * S + q0) * q_stride + (int64_t)(g * G + 2 * i) * kHeadDim;
    const char* qb = reinterpret_cast<const char*>(q + ubase);
    const char* gb = reinterpret_cast<const char*>(dout + ubase);
    uint32_t off[2];
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      off[ii] = qoff[ii];
      if (!fast) {
        const int R = 16 * wave + 8 * ii + (lane >> 3);
        const int pr = min(q0 + (R & 31), S - 1) - q0;
        const int e = min(2 * i + (R >> 5), G - 1) - 2 * i;
        off[ii] = (uint32_t)(((pr * a.Hq + e) * kHeadDim + dma_chunk) * 2);
      }
    }
    // wave-uniform slice of 16 rows of the Q and dO tiles of buffer buf (byte addresses)
    const uint32_t lq = smem_lds + (uint32_t)((2 * buf) * TILE + 16 * wave * RS) * 2u;
    const uint32_t lgo = lq + (uint32_t)TILE * 2u;
    constexpr uint32_t kHalf = 8 * RS * 2;
    dma16_kv(qb, gb, off[0], off[1], lq, lq + kHalf, lgo, lgo + kHalf);
    if (wave == 0) {
      const int64_t lbase = ((int64_t)b * a.Hq + g * G + 2 * i) * S + q0;
      uint32_t off = loff;
      if (!fast) off = (uint32_t)(((min(2 * i + lg, G - 1) - 2 * i) * S + min(q0 + lr, S - 1) - q0) * 4);
      float* ls = smem_f + buf * 4 * QT;
      dma4(reinterpret_cast<const char*>(a.lse2 + lbase), off, (lds_void*)(ls));
      dma4(reinterpret_cast<const char*>(a.dlt + lbase), off, (lds_void*)(ls + 2 * QT));
    }
  };

  f32x16 dk[2], dv[2];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt) {
    dk[dt] = zero16();
    dv[dt] = zero16();
  }
  int vofs[2];
  tr_offsets(lane, vofs);
  const float c = a.scale_log2;

  // unit u = (q-tile t, head pair i), i fastest; (t, i) of the unit being
  // computed and (t2, i2) of the one being staged two ahead
  int t = 0, i = 0, t2 = 0, i2 = 0;
  auto advance = [&](int& tt, int& ip) {
    if (++ip == np) {
      ip = 0;
      ++tt;
    }
  };
  if (n_units > 0) {
    dma_unit(t2, i2, 0);
    advance(t2, i2);
  }
  if (n_units > 1) {
    dma_unit(t2, i2, 1);
    advance(t2, i2);
  }
  // One body per LDS buffer (unit u lives in buffer u % 3), so that the LDS
  // addresses are compile-time offsets.
  auto body = [&](auto bufc, int u) {
    constexpr int BUF = decltype(bufc)::value;
    // Unit u (staged two units ago) has landed for every wave; the buffer of
    // unit u-1 is free again.  Vector memory loads complete in issue order, so
    // waiting until only unit u+1's loads of this wave (4, and 2 more on wave
    // 0) are outstanding leaves them a whole unit more to land.  The LDS reads
    // of unit u-1 are complete too (lgkmcnt 0) before the barrier.
    if (u + 1 < n_units) {
      if (wave == 0) __builtin_amdgcn_s_waitcnt(0x0070 | 6);
      else __builtin_amdgcn_s_waitcnt(0x0070 | 4);
    } else {
      __builtin_amdgcn_s_waitcnt(0x0070);
    }
    asm volatile("s_barrier" ::: "memory");
    if (u + 2 < n_units) {
      dma_unit(t2, i2, (BUF + 2) % NBUF);
      advance(t2, i2);
    }
    const int q0 = (t_lo + t) * QT;
    const int ip = i;
    advance(t, i);
    if (2 * ip + hh >= G) return;
    // (queries q0 .. q0+31) x (keys jw .. jw+31): nothing visible, all
    // visible, or compared element by element
    if (q0 + QT - 1 < jw || q0 >= S || (W > 0 && jw >= st && q0 - W >= jw + 31)) return;
    const bool full = q0 >= jw + 31 && q0 + QT - 1 < S && (W <= 0 || q0 + QT - 1 - W < jw || jw + 31 < st);

    const __bf16* qs = smem_b + (2 * BUF) * TILE + hh * QT * RS;
    const __bf16* gs = smem_b + (2 * BUF + 1) * TILE + hh * QT * RS;
    f32x16 s, dp;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 qa = *reinterpret_cast<const bf16x8*>(qs + lr * RS + kchunk(2 * kk + lg, lr));
      const bf16x8 ga = *reinterpret_cast<const bf16x8*>(gs + lr * RS + kchunk(2 * kk + lg, lr));
      s = mfma32(qa, kop[kk], kk == 0 ? zero16() : s);
      dp = mfma32(ga, vop[kk], kk == 0 ? zero16() : dp);
    }
    // register r: query q0 + 8(r/4) + 4lg + r%4, key jw + lr
    const float* ls = smem_f + BUF * 4 * QT + hh * QT + 4 * lg;
    f32x4 l4[4], d4[4];
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      l4[a4] = *reinterpret_cast<const f32x4*>(ls + 8 * a4);
      d4[a4] = *reinterpret_cast<const f32x4*>(ls + 2 * QT + 8 * a4);
    }
    if (!full) {
      const int dd = jw + lr - q0 - 4 * lg;                             // causal: rr >= dd
      const int hc = S - q0 - 4 * lg;                                   // row exists: rr < hc
      const int hw = (W > 0 && jw + lr >= st) ? dd + W : 0x40000000;  // window: rr < hw
      const int hm = min(hc, hw);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = 8 * (r >> 2) + (r & 3);
        if (rr < dd || rr >= hm) s[r] = -INFINITY;
      }
    }
    bf16x8 pa[2], da[2];
#pragma unroll
    for (int uu = 0; uu < 2; ++uu) {
      u32x4 wp, wd;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r0 = 8 * uu + 2 * e, r1 = r0 + 1;
        const float p0 = fast_exp2(__builtin_fmaf(s[r0], c, -l4[r0 >> 2][r0 & 3]));
        const float p1 = fast_exp2(__builtin_fmaf(s[r1], c, -l4[r1 >> 2][r1 & 3]));
        const f32x2 pp = {p0, p1};
        const f32x2 gg = {p0 * (dp[r0] - d4[r0 >> 2][r0 & 3]), p1 * (dp[r1] - d4[r1 >> 2][r1 & 3])};
        wp[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pp, bf16x2));
        wd[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(gg, bf16x2));
      }
      pa[uu] = __builtin_bit_cast(bf16x8, wp);
      da[uu] = __builtin_bit_cast(bf16x8, wd);
    }
#pragma unroll
    for (int uu = 0; uu < 2; ++uu)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const bf16x8 gt = tr_operand(gs, uu, dt, vofs);
        const bf16x8 qt = tr_operand(qs, uu, dt, vofs);
        dv[dt] = mfma32(pa[uu], gt, dv[dt]);
        dk[dt] = mfma32(da[uu], qt, dk[dt]);
      }
  };
  std::integral_constant<int, 0> B0;
  std::integral_constant<int, 1> B1;
  std::integral_constant<int, 2> B2;
  int u = 0;
  for (; u + NBUF <= n_units; u += NBUF) {
    body(B0, u);
    body(B1, u + 1);
    body(B2, u + 2);
  }
  if (u < n_units) body(B0, u);
  if (u + 1 < n_units) body(B1, u + 1);

  // ---- the two head halves add up through LDS; rows leave as 16-byte chunks
  // (bf16), or as fp32 partial sums of this slab
  __syncthreads();  // every wave is done with the staging buffers (no loads in flight)
  float* red = reinterpret_cast<float*>(smem_b);  // [kh][dK, dV][32 keys][64] fp32: 32 KB
  __bf16* outt = smem_b + 2 * 2 * 32 * 64 * 2;     // [dK, dV][64 keys][64] bf16: 16 KB
  if (hh == 1) {
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int key = 8 * (rr >> 2) + 4 * lg + (rr & 3);
        red[((kh * 2 + 0) * 32 + key) * 64 + 32 * dt + lr] = dk[dt][rr];
        red[((kh * 2 + 1) * 32 + key) * 64 + 32 * dt + lr] = dv[dt][rr];
      }
  }
  __syncthreads();
  if (partial) {
    if (hh == 0) {
      // [dK, dV][64 keys][64] fp32 of (sequence, KV head, key block, slab)
      float* pp = a.part + ((((int64_t)unit * nkb + kb) * a.n_slabs + slab) * 2) * (KB * kHeadDim);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int key = 8 * (rr >> 2) + 4 * lg + (rr & 3);
          const int e = (32 * kh + key) * 64 + 32 * dt + lr;
          pp[e] = (dk[dt][rr] + red[((kh * 2 + 0) * 32 + key) * 64 + 32 * dt + lr]) * a.scale;
          pp[KB * kHeadDim + e] = dv[dt][rr] + red[((kh * 2 + 1) * 32 + key) * 64 + 32 * dt + lr];
        }
    }
    return;
  }
  if (hh == 0) {
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int key = 8 * (rr >> 2) + 4 * lg + (rr & 3);
        const float xk = (dk[dt][rr] + red[((kh * 2 + 0) * 32 + key) * 64 + 32 * dt + lr]) * a.scale;
        const float xv = dv[dt][rr] + red[((kh * 2 + 1) * 32 + key) * 64 + 32 * dt + lr];
        outt[(32 * kh + key) * 64 + 32 * dt + lr] = (__bf16)xk;
        outt[(64 + 32 * kh + key) * 64 + 32 * dt + lr] = (__bf16)xv;
      }
  }
  __syncthreads();
  __bf16* dkp = reinterpret_cast<__bf16*>(a.dk);
  __bf16* dvp = reinterpret_cast<__bf16*>(a.dv);
  for (int cidx = threadIdx.x; cidx < 2 * 64 * 8; cidx += BT) {
    const int tsr = cidx >> 9, row = (cidx >> 3) & 63, ch = cidx & 7;
    const int j = j0 + row;
    if (j < S) {
      __bf16* dst = (tsr ? dvp : dkp) + ((int64_t)b * S + j) * kv_stride + g * kHeadDim + 8 * ch;
      *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(outt + (tsr * 64 + row) * 64 + 8 * ch);
    }
  }
}

// 3b. dK, dV of the key blocks split into several slabs: the fp32 partials
// added in slab order and rounded to bf16.  One workgroup per (sequence, KV
// head, key block); blocks with a single slab were written directly.
template <bool STK>
__global__ __launch_bounds__(BT) void bwd_dkdv_reduce_kernel(BwdArgs a) {
  const int S = a.S, W = a.window;
  const int nkb = (S + KB - 1) / KB;
  const int x = blockIdx.x;
  const int unit = x / nkb;
  const int kb = x - unit * nkb;
  const int st = STK && W > 0 ? a.sink_tokens : 0;
  const int j0 = kb * KB;
  const int s_lo = j0 / a.slab_len, s_hi = block_p_hi(j0, S, W, st) / a.slab_len;
  if (s_hi == s_lo) return;
  const int b = unit / a.Hkv;
  const int g = unit - b * a.Hkv;
  const float* base = a.part + (((int64_t)unit * nkb + kb) * a.n_slabs) * 2 * (KB * kHeadDim);
  const int64_t kv_stride = (int64_t)a.Hkv * kHeadDim;
  // chunk c: tensor c / 512, key (c / 8) % 64, d 8 * (c % 8) .. +7
  for (int c = threadIdx.x; c < 2 * KB * 8; c += BT) {
    const int tsr = c >> 9, row = (c >> 3) & 63, ch = c & 7;
    const int j = j0 + row;
    if (j >= S) continue;
    f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
    for (int sl = s_lo; sl <= s_hi; ++sl) {
      const float* src = base + ((int64_t)sl * 2 + tsr) * (KB * kHeadDim) + row * kHeadDim + 8 * ch;
      lo += *reinterpret_cast<const f32x4*>(src);
      hi += *reinterpret_cast<const f32x4*>(src + 4);
    }
    u32x4 w;
    w[0] = pack_bf16x2(lo[0], lo[1]);
    w[1] = pack_bf16x2(lo[2], lo[3]);
    w[2] = pack_bf16x2(hi[0], hi[1]);
    w[3] = pack_bf16x2(hi[2], hi[3]);
    __bf16* dst = reinterpret_cast<__bf16*>(tsr ? a.dv : a.dk) + ((int64_t)b * S + j) * kv_stride + g * kHeadDim + 8 * ch;
    *reinterpret_cast<u32x4*>(dst) = w;
  }
}

// ---------------------------------------------------------------------------
// 4. dQ (bf16).  Workgroup = (sequence, KV head, 8 N-tiles), two per wave, as
// in the forward; K/V tiles of 64 keys staged in LDS two tiles ahead.
template <bool STK>
__global__ __launch_bounds__(BT, 2) void bwd_dq_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 Ks[NBUF][BK * RS];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[NBUF][BK * RS];
  const __bf16* q = reinterpret_cast<const __bf16*>(a.q);
  const __bf16* dout = reinterpret_cast<const __bf16*>(a.dout);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lr = lane & 31;
  const int lg = lane >> 5;
  const int S = a.S, G = a.G, W = a.window;
  const int n_ntiles = ((S + 31) >> 5) * G;
  const int wg_per_seq = (n_ntiles + NT_WG - 1) / NT_WG;
  const int U = a.B * a.Hkv;
  // (divisions by the launch's divisors use the launcher's multipliers)
  int unit, rank;
  {
    const int x = blockIdx.x;
    if ((U & 7) == 0) {
      const int sidx = x >> 3;
      const int sq = fast_div(sidx, a.div_wg_per_seq);
      rank = sidx - sq * wg_per_seq;
      unit = (x & 7) + 8 * sq;
    } else {
      rank = fast_div(x, a.div_units);
      unit = x - rank * U;
    }
  }
  const int tg = wg_per_seq - 1 - rank;  // the latest positions (most keys) first
  const int b = fast_div(unit, a.div_hkv);
  const int g = unit - b * a.Hkv;

  int nt_t0[2], nt_hq[2], pos0[2], phi[2];
  bool nt_valid[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int n = tg * NT_WG + wave * 2 + i;
    nt_valid[i] = n < n_ntiles;
    const int pb = fast_div(n, a.div_g);
    nt_t0[i] = pb * 32;
    nt_hq[i] = g * G + (n - pb * G);
    pos0[i] = nt_t0[i];
    phi[i] = min(nt_t0[i] + 31, S - 1);
  }
  const int n_last = min(tg * NT_WG + NT_WG - 1, n_ntiles - 1);
  const int t_min = fast_div(tg * NT_WG, a.div_g) * 32;
  const int t_max = min(fast_div(n_last, a.div_g) * 32 + 31, S - 1);
  const int lo = W > 0 ? max(0, t_min - W + 1) : 0;
  const int hi = t_max;  // inclusive
  const int j_begin = lo & ~(BK - 1);
  const int st = STK && W > 0 ? a.sink_tokens : 0;
  const int n_st = STK ? (min(st, j_begin) + BK - 1) / BK : 0;  // sink tiles below the window
  const int n_tiles = n_st + (hi >= j_begin ? (hi - j_begin) / BK + 1 : 0);
  auto tile_j0 = [&](int t) { return t < n_st ? BK * t : j_begin + BK * (t - n_st); };

  // Q and dO rows as B operands (column = query, k = d), lse and D per lane
  bf16x8 qb[2][4], gb[2][4];
  float l2[2], dl[2];
  // (unconditional loads: a row past the end reads the last row, whose head
  // is valid; its results are never stored)
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = min(nt_t0[i] + lr, S - 1);
    const int64_t off = (((int64_t)b * S + t) * a.Hq + nt_hq[i]) * kHeadDim + 8 * lg;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      qb[i][kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q + off + 16 * kk));
      gb[i][kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(dout + off + 16 * kk));
    }
    const int64_t li = ((int64_t)b * a.Hq + nt_hq[i]) * S + t;
    l2[i] = a.lse2[li];
    dl[i] = a.dlt[li];
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);  // as in the dK/dV kernel: no compiler wait on these inside the tile loop
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) acc[i][dt] = zero16();

  const int64_t kv_stride = (int64_t)a.Hkv * kHeadDim;
  const __bf16* kbase = reinterpret_cast<const __bf16*>(a.k) + (int64_t)b * S * kv_stride + g * kHeadDim;
  const __bf16* vbase = reinterpret_cast<const __bf16*>(a.v) + (int64_t)b * S * kv_stride + g * kHeadDim;
  const int dma_chunk = ((lane & 7) ^ kswz(lane >> 3)) * 8;
  // wave w fills rows 16w .. 16w+15 of a tile; rows past the key range repeat
  // row hi (masked, in bounds)
  // (a scalar base per tile and a 32-bit offset per lane)
  const uint32_t ks_lds = lds_addr((lds_void*)&Ks[0][0]);  // formed once: a cast per load tests for null
  const uint32_t vs_lds = lds_addr((lds_void*)&Vs[0][0]);
  auto dma_tile = [&](int t, int buf) {
    const int j0 = tile_j0(t);
    const char* kt = reinterpret_cast<const char*>(kbase + (int64_t)j0 * kv_stride);
    const char* vt = reinterpret_cast<const char*>(vbase + (int64_t)j0 * kv_stride);
    uint32_t off[2];
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int r = min(16 * wave + 8 * ii + (lane >> 3), hi - j0);
      off[ii] = (__umul24(r, (uint32_t)kv_stride) + dma_chunk) * 2u;  // r < 64: 24-bit product
    }
    const uint32_t lofs = (uint32_t)(buf * BK * RS + 16 * wave * RS) * 2u;  // wave-uniform slice of 16 rows
    constexpr uint32_t kHalf = 8 * RS * 2;
    dma16_kv(kt, vt, off[0], off[1], ks_lds + lofs, ks_lds + lofs + kHalf, vs_lds + lofs, vs_lds + lofs + kHalf);
  };
  int vofs[2];
  tr_offsets(lane, vofs);
  const float c = a.scale_log2;

  if (n_tiles > 0) dma_tile(0, 0);
  if (n_tiles > 1) dma_tile(1, 1);
  // One body per LDS buffer (tile t lives in buffer t % 3): compile-time LDS
  // offsets.
  auto body = [&](auto bufc, int t) {
    constexpr int BUF = decltype(bufc)::value;
    // Tile t (staged two tiles ago) has landed for every wave once only tile
    // t+1's loads of this wave (4) are in flight (vector loads complete in
    // issue order); the LDS reads of tile t-1 are done before its buffer takes
    // tile t+2.
    if (t + 1 < n_tiles) __builtin_amdgcn_s_waitcnt(0x0070 | 4);
    else __builtin_amdgcn_s_waitcnt(0x0070);
    asm volatile("s_barrier" ::: "memory");
    if (t + 2 < n_tiles) dma_tile(t + 2, (BUF + 2) % NBUF);
    const int j0 = tile_j0(t);
    const int ds = STK ? st - j0 - 4 * lg : 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 ka[4], va[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        ka[kk] = *reinterpret_cast<const bf16x8*>(Ks[BUF] + (32 * h + lr) * RS + kchunk(2 * kk + lg, lr));
        va[kk] = *reinterpret_cast<const bf16x8*>(Vs[BUF] + (32 * h + lr) * RS + kchunk(2 * kk + lg, lr));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (!nt_valid[i]) continue;
        f32x16 sc, dp;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          sc = mfma32(ka[kk], qb[i][kk], kk == 0 ? zero16() : sc);
          dp = mfma32(va[kk], gb[i][kk], kk == 0 ? zero16() : dp);
        }
        // Dense layers: the vector work of an N-tile runs at a higher issue
        // priority than the matrix work, so of the two waves of a SIMD the one
        // with exponentials to do goes before one that only feeds MFMAs
        // (measured 3-4 % on the dense layer; windowed layers unchanged).
        if (W == 0) __builtin_amdgcn_s_setprio(1);
        const int dh = pos0[i] + lr - j0 - 4 * lg;
        const int dlw = W > 0 ? dh - W : -0x40000000;
        mask_half<STK>(sc, h, j0, pos0[i], phi[i], W, st, dh, dlw, ds);
        bf16x8 db[2];
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r0 = 8 * uu + 2 * e, r1 = r0 + 1;
            const float p0 = fast_exp2(__builtin_fmaf(sc[r0], c, -l2[i]));
            const float p1 = fast_exp2(__builtin_fmaf(sc[r1], c, -l2[i]));
            const f32x2 gg = {p0 * (dp[r0] - dl[i]), p1 * (dp[r1] - dl[i])};
            w[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(gg, bf16x2));
          }
          db[uu] = __builtin_bit_cast(bf16x8, w);
        }
        if (W == 0) __builtin_amdgcn_s_setprio(0);
        // K^T operands are read per N-tile: holding them across both would
        // cost 16 registers the allocator does not have
#pragma unroll
        for (int uu = 0; uu < 2; ++uu)
#pragma unroll
          for (int dt = 0; dt < 2; ++dt)
            acc[i][dt] = mfma32(tr_operand(Ks[BUF], 2 * h + uu, dt, vofs), db[uu], acc[i][dt]);
      }
    }
  };
  {
    std::integral_constant<int, 0> B0;
    std::integral_constant<int, 1> B1;
    std::integral_constant<int, 2> B2;
    int t = 0;
    for (; t + NBUF <= n_tiles; t += NBUF) {
      body(B0, t);
      body(B1, t + 1);
      body(B2, t + 2);
    }
    if (t < n_tiles) body(B0, t);
    if (t + 1 < n_tiles) body(B1, t + 1);
  }

  // ---- epilogue: dq = scale * acc, rounded to bf16; through LDS so that it
  // leaves as whole 128-byte rows (a lane holds pieces of 32 rows)
  int lr_e = lr;
  asm volatile("" : "+v"(lr_e));
  __syncthreads();  // every wave is done with the K/V tiles
  __bf16* stg = wave < NBUF ? Ks[wave] : Vs[0];  // this wave's 64 rows: [N-tile][row][64]
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 32 * i + lr_e;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int cq = 0; cq < 4; ++cq) {
        u32x2 w;
        w[0] = pack_bf16x2(acc[i][dt][4 * cq + 0] * a.scale, acc[i][dt][4 * cq + 1] * a.scale);
        w[1] = pack_bf16x2(acc[i][dt][4 * cq + 2] * a.scale, acc[i][dt][4 * cq + 3] * a.scale);
        *reinterpret_cast<u32x2*>(stg + row * RS + kchunk(4 * dt + cq, row) + 4 * lg) = w;  // d = 32dt + 8cq + 4lg
      }
  }
  wave_lds_sync();  // the wave reads back only its own rows
  __bf16* dq = reinterpret_cast<__bf16*>(a.dq);
  // rows 8j .. 8j+7 of the wave's 64: N-tile j / 4, row (lane / 8) + 8 (j % 4)
  // of it, 16-byte chunk lane % 8; a wave whose two N-tiles are whole stores
  // without per-row tests
  u32x4 ov[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = (lane >> 3) + 8 * (j & 3);
    ov[j] = *reinterpret_cast<const u32x4*>(stg + (32 * (j >> 2) + r) * RS + kchunk(lane & 7, r));
  }
  auto store = [&](int j) {
    const int i = j >> 2;
    const int t = nt_t0[i] + (lane >> 3) + 8 * (j & 3);
    *reinterpret_cast<u32x4*>(dq + (((int64_t)b * S + t) * a.Hq + nt_hq[i]) * kHeadDim + 8 * (lane & 7)) = ov[j];
  };
  const bool whole = nt_valid[0] && nt_valid[1] && max(nt_t0[0], nt_t0[1]) + 31 < S;
  if (whole) {
#pragma unroll
    for (int j = 0; j < 8; ++j) store(j);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (nt_valid[j >> 2] && nt_t0[j >> 2] + (lane >> 3) + 8 * (j & 3) < S) store(j);
  }
}

// ---------------------------------------------------------------------------
// fp32 path (parity, small problems): one wave per output row, lane = d,
// visible pairs enumerated one by one.

// dq of (sequence, position, query head)
__global__ __launch_bounds__(BT) void bwd_dq_fp32_kernel(BwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t id = (int64_t)blockIdx.x * (BT / 64) + (threadIdx.x >> 6);
  if (id >= (int64_t)a.B * a.S * a.Hq) return;
  const int h = (int)(id % a.Hq);
  const int64_t row = id / a.Hq;
  const int p = (int)(row % a.S);
  const int b = (int)(row / a.S);
  const int g = h / a.G;
  const float* q = reinterpret_cast<const float*>(a.q);
  const float* k = reinterpret_cast<const float*>(a.k);
  const float* v = reinterpret_cast<const float*>(a.v);
  const float* dout = reinterpret_cast<const float*>(a.dout);
  const float qd = q[(row * a.Hq + h) * kHeadDim + lane];
  const float gd = dout[(row * a.Hq + h) * kHeadDim + lane];
  const int64_t li = ((int64_t)b * a.Hq + h) * a.S + p;
  const float l2 = a.lse[li] * kLog2e;
  const float D = a.dlt[li];
  const int W = a.window;
  const int jlo = W > 0 ? max(0, p - W + 1) : 0;
  const int ns = W > 0 ? min(a.sink_tokens, jlo) : 0;  // sink tokens below the window
  const int nv = ns + (p - jlo + 1);
  float acc = 0.f;
  for (int vi = 0; vi < nv; ++vi) {
    const int j = vi < ns ? vi : jlo + (vi - ns);
    const int64_t kr = (((int64_t)b * a.S + j) * a.Hkv + g) * kHeadDim + lane;
    const float kd = k[kr];
    const float x = wave_sum(qd * kd) * a.scale_log2;
    const float P = fast_exp2(x - l2);
    const float dp = wave_sum(gd * v[kr]);
    acc += P * (dp - D) * kd;
  }
  reinterpret_cast<float*>(a.dq)[(row * a.Hq + h) * kHeadDim + lane] = acc * a.scale;
}

// dk, dv of (sequence, position, KV head)
__global__ __launch_bounds__(BT) void bwd_dkdv_fp32_kernel(BwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t id = (int64_t)blockIdx.x * (BT / 64) + (threadIdx.x >> 6);
  if (id >= (int64_t)a.B * a.S * a.Hkv) return;
  const int g = (int)(id % a.Hkv);
  const int64_t row = id / a.Hkv;
  const int j = (int)(row % a.S);
  const int b = (int)(row / a.S);
  const float* q = reinterpret_cast<const float*>(a.q);
  const float* k = reinterpret_cast<const float*>(a.k);
  const float* v = reinterpret_cast<const float*>(a.v);
  const float* dout = reinterpret_cast<const float*>(a.dout);
  const float kd = k[(row * a.Hkv + g) * kHeadDim + lane];
  const float vd = v[(row * a.Hkv + g) * kHeadDim + lane];
  const int W = a.window;
  const int st = W > 0 ? a.sink_tokens : 0;
  // queries that see key j: p >= j, inside the window unless j is a sink token
  const int p_end = (W > 0 && j >= st) ? min(a.S, j + W) : a.S;
  float ak = 0.f, av = 0.f;
  for (int hi = 0; hi < a.G; ++hi) {
    const int h = g * a.G + hi;
    for (int p = j; p < p_end; ++p) {
      const int64_t qr = (((int64_t)b * a.S + p) * a.Hq + h) * kHeadDim + lane;
      const float qd = q[qr], gd = dout[qr];
      const int64_t li = ((int64_t)b * a.Hq + h) * a.S + p;
      const float x = wave_sum(qd * kd) * a.scale_log2;
      const float P = fast_exp2(x - a.lse[li] * kLog2e);
      const float dp = wave_sum(gd * vd);
      ak += P * (dp - a.dlt[li]) * qd;
      av += P * gd;
    }
  }
  reinterpret_cast<float*>(a.dk)[(row * a.Hkv + g) * kHeadDim + lane] = ak * a.scale;
  reinterpret_cast<float*>(a.dv)[(row * a.Hkv + g) * kHeadDim + lane] = av;
}

}  // namespace

// Slabs per key block: enough (slab, key block) jobs for about 1024 workgroups
// (2 per slot of a 256-CU chip at 2 workgroups per CU), at most 4 slabs.  On
// the layer-shaped dense call (512 key blocks) that is 2 slabs: 4 slabs (the
// earlier aim of 4096 workgroups) measured 3-5 % slower and 1 slab 20 % slower.
// Windowed layers without sink tokens give every key block the same short
// query range, so they are never cut.
void backward_plan(int B, int S, int Hkv, int window, int sink_tokens, int* n_slabs, int* slab_len) {
  const int64_t jobs = (int64_t)B * Hkv * ((S + KB - 1) / KB);
  int n = 1;
  if (jobs > 0 && jobs < 1024 && !(window > 0 && sink_tokens == 0))
    n = (int)std::min<int64_t>(4, (1024 + jobs - 1) / jobs);
  int len = ((S + n - 1) / n + QT - 1) / QT * QT;
  if (len < QT) len = QT;
  *slab_len = len;
  *n_slabs = (S + len - 1) / len > 1 ? (S + len - 1) / len : 1;
}

hipError_t launch_backward(const BwdArgs& args, hipStream_t s) {
  const BwdArgs& a = args;
  const int64_t rows = (int64_t)a.B * a.S;
  if (rows > 0) {
    const int64_t blocks = (rows + BT / 64 - 1) / (BT / 64);
    if (a.fp32) hipLaunchKernelGGL(bwd_dot_kernel<float>, dim3((unsigned)blocks), dim3(BT), 0, s, a);
    else hipLaunchKernelGGL(bwd_dot_kernel<__bf16>, dim3((unsigned)blocks), dim3(BT), 0, s, a);
    const int64_t nrs = (int64_t)a.B * a.Hq * ((a.S + SB - 1) / SB);
    hipLaunchKernelGGL(bwd_rowstat_kernel, dim3((unsigned)nrs), dim3(BT), 0, s, a);
  }
  if (a.dsinks) hipLaunchKernelGGL(bwd_dsink_kernel, dim3((a.Hq + 63) / 64), dim3(64), 0, s, a);
  if (rows == 0) return hipGetLastError();
  if (a.fp32) {
    const int64_t nq = (rows * a.Hq + 3) / 4, nk = (rows * a.Hkv + 3) / 4;
    hipLaunchKernelGGL(bwd_dkdv_fp32_kernel, dim3((unsigned)nk), dim3(BT), 0, s, a);
    hipLaunchKernelGGL(bwd_dq_fp32_kernel, dim3((unsigned)nq), dim3(BT), 0, s, a);
    return hipGetLastError();
  }
  const bool stk = args.window > 0 && args.sink_tokens > 0;
  const int nkb = (args.S + KB - 1) / KB;
  const unsigned g1 = (unsigned)((int64_t)args.B * args.Hkv * nkb * args.n_slabs);
  const unsigned g1r = (unsigned)((int64_t)args.B * args.Hkv * nkb);
  const int n_ntiles = ((args.S + 31) / 32) * args.G;
  const unsigned g2 = (unsigned)((int64_t)args.B * args.Hkv * ((n_ntiles + NT_WG - 1) / NT_WG));
  BwdArgs ad = args;  // with the divisors of the job mappings
  ad.div_units = make_fastdiv(ad.B * ad.Hkv);
  ad.div_hkv = make_fastdiv(ad.Hkv);
  ad.div_g = make_fastdiv(ad.G);
  ad.div_nkb = make_fastdiv(nkb);
  ad.div_per_unit = make_fastdiv(nkb * ad.n_slabs);
  ad.div_slab_len = make_fastdiv(ad.slab_len);
  ad.div_wg_per_seq = make_fastdiv((n_ntiles + NT_WG - 1) / NT_WG);
  if (stk) {
    hipLaunchKernelGGL(bwd_dkdv_kernel<true>, dim3(g1), dim3(BT), 0, s, ad);
    if (ad.n_slabs > 1) hipLaunchKernelGGL(bwd_dkdv_reduce_kernel<true>, dim3(g1r), dim3(BT), 0, s, ad);
    hipLaunchKernelGGL(bwd_dq_kernel<true>, dim3(g2), dim3(BT), 0, s, ad);
  } else {
    hipLaunchKernelGGL(bwd_dkdv_kernel<false>, dim3(g1), dim3(BT), 0, s, ad);
    if (ad.n_slabs > 1) hipLaunchKernelGGL(bwd_dkdv_reduce_kernel<false>, dim3(g1r), dim3(BT), 0, s, ad);
    hipLaunchKernelGGL(bwd_dq_kernel<false>, dim3(g2), dim3(BT), 0, s, ad);
  }
  return hipGetLastError();
}

// Metadata-check flags of this file's kernels (recorded only when built with GQA_DEBUG).
GQA_DEBUG_FLAGS_ACCESSOR(debug_flags_backward)

}  // namespace gqa
