// Decode attention on gfx950: one new query token per sequence, HBM-bound.
//
// The KV cache is streamed once; each K/V row of a KV head serves all the
// query heads of its group («GPT-OSS-20B : Architecture MoE & Résumé du Model
// Card» §3.3, 8 query heads per KV head), and on sliding-window layers only the
// last W positions are read («GPT-OSS vs Qwen3», "Utilisation de Sliding Window
// Attention"), plus the start-of-sequence sink tokens when asked («GPT-OSS vs
// Qwen3», "Attention Bias et Sinks").  The sink logit («GPT-OSS vs Qwen3», "Attention Bias et Sinks")
// enters once, when the partial results are merged.
//
// Work decomposition: a workgroup owns (sequence, KV head, chunk of up to 16
// query heads, split of the key range).  Its 4 waves take interleaved 64-key
// tiles and keep independent online-softmax states; the 4 states are merged in
// LDS.  With one split the workgroup writes the final output; otherwise it
// writes a partial (max, sum, unnormalised output) and a combine kernel merges
// the splits.
//
// Short key ranges with many (sequence, KV head) units (window or ring layers
// at large batch) take the "solo" form instead: each wave owns a whole unit,
// walks its tiles in order and finishes it itself, with no split and no
// cross-wave merge.
//
// Each wave streams whole 128-byte K and V rows of its key tiles with
// non-temporal loads (the access pattern that reaches the highest HBM rate),
// stages them in its own LDS slice, and computes S^T = K Q^T on
// v_mfma_f32_16x16x32_bf16 (K rows from LDS, Q^T in registers, 16 head
// columns) and O^T += V^T P^T with V^T read by the transposing LDS load.
#include "kernels.h"

namespace gqa {
namespace {

constexpr int DT = 64;         // keys per wave tile
constexpr int DTHREADS = 256;  // 4 waves
constexpr int KSD = 72;        // LDS row stride (elements) of a wave's K tile [key][d]
constexpr int VSD = 80;        // LDS row stride (elements) of a wave's V tile [key][d]
constexpr int WAVE_LDS = DT * KSD + DT * VSD;  // elements per wave

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// streamed once: non-temporal loads keep the KV cache from evicting reusable lines
__device__ __forceinline__ u32x4 load_stream(const __bf16* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// A wave that holds the whole key range of query head hq (one column of O^T:
// lane quarter lq has d = 16*dt + 4*lq + r in o[dt][r]; running max m_run in
// log2 units, sum lt over all four quarters) folds in the sink and writes the
// output row and its log-sum-exp.
__device__ __forceinline__ void finish_column(const DecodeArgs& a, int b, int64_t q_row, int64_t lse_row, int hq,
                                              int lq, float m_run, float lt, const f32x4 (&o)[4]) {
  const float s2 = a.sinks ? a.sinks[hq] * kLog2e : -INFINITY;
  const float Mf = fmaxf(m_run, s2);
  const float sc = fast_exp2(m_run - Mf);
  const float Z = fast_exp2(s2 - Mf) + lt * sc;
  const float inv = Z > 0.f ? sc / Z : (Z == 0.f ? 0.f : Z);
  __bf16* op = a.out + (q_row * a.Hq + hq) * (int64_t)kHeadDim + 4 * lq;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    u32x2 w;
    w[0] = pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv);
    w[1] = pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv);
    *reinterpret_cast<u32x2*>(op + 16 * dt) = w;
  }
  if (a.lse && lq == 0) {
    const float v = (Z == 0.f) ? -INFINITY : (Mf + __log2f(Z)) * kLn2;
    a.lse[(int64_t)b * a.lse_sb + (int64_t)hq * a.lse_sh + lse_row] = v;
  }
}

template <int MODE, bool SOLO>
__global__ __launch_bounds__(DTHREADS, 2) void decode_split_kernel(DecodeArgs a) {
  // per wave: K tile then V tile; after the key loop the same memory holds the
  // 4-wave merge buffers
  __shared__ __attribute__((aligned(16))) __bf16 lds[4 * WAVE_LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lc = lane & 15;  // head column (and key row of the K operand)
  const int lq = lane >> 4;  // lane quarter

  // blockIdx -> (split, head chunk, KV head, sequence); splits of one
  // (sequence, KV head) are consecutive.  Solo: one unit per wave, one split.
  int x = SOLO ? (int)blockIdx.x * 4 + wave : (int)blockIdx.x;
  if (SOLO && x >= a.B * a.Hkv * a.n_hc) return;  // wave-uniform; the solo form has no workgroup barrier
  const int split = SOLO ? 0 : x % a.n_splits;
  if (!SOLO) x /= a.n_splits;
  const int hc = x % a.n_hc;
  x /= a.n_hc;
  const int g = x % a.Hkv;
  const int b = x / a.Hkv;

  const SeqView sv = seq_view<MODE>(a.seq, b, a.varlen_q != 0);
  if (a.varlen_q && sv.q_len != 1) return;  // handled by the prefill-style kernel
  const int L = sv.kv_len;
  const int W = a.window;
  const int lo_all = W > 0 ? max(0, L - W) : 0;
  // Keys read: the sink tokens below the window, then the window, numbered by
  // a "virtual" index v in [0, nv): key v for v < ns, lo_all + v - ns after.
  // Splits and tiles run over v.
  const int ns = W > 0 ? min(a.sink_tokens, lo_all) : 0;
  const int nv = ns + (L - lo_all);
  const int s_lo = split * a.split_len;
  const int s_hi = min(nv, s_lo + a.split_len);  // exclusive
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
  const __bf16* kbase = a.k + g * kHeadDim + 8 * (lane & 7);
  const __bf16* vbase = a.v + g * kHeadDim + 8 * (lane & 7);
  __bf16* Kw = lds + wave * WAVE_LDS;
  __bf16* Vw = Kw + DT * KSD;

  // whole 128-byte rows: load i brings keys 8*i + lane/8, 16 bytes at d = 8*(lane%8);
  // rows past the split repeat its last row (masked below, always in bounds)
  // With a paged cache the block ids of a tile's rows are fetched one tile
  // ahead, so no K/V load waits on the block table.
  u32x4 kreg[8], vreg[8];
  int blk[8];
  auto key_of = [&](int v) { return v < ns ? v : lo_all + (v - ns); };
  auto fetch_blk = [&](int j0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      blk[i] = 0;
      if (MODE == KV_PAGED) {
        const int j = key_of(min(j0 + 8 * i + (lane >> 3), s_hi - 1));
        blk[i] = a.seq.block_table[(int64_t)b * a.seq.max_blocks + (j >> a.seq.log2_block)];
      }
    }
  };
  auto load = [&](int j0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = key_of(min(j0 + 8 * i + (lane >> 3), s_hi - 1));
      int64_t row;
      if (MODE == KV_PAGED) {
        const int bb = min(max(blk[i], 0), a.seq.num_blocks - 1);
        GQA_FLAG(bb != blk[i], kDbgBlockTable);
        row = ((int64_t)bb << a.seq.log2_block) + (j & ((1 << a.seq.log2_block) - 1));
      } else {
        row = kv_row<MODE>(a.seq, sv, j);
      }
      row *= kv_stride;
      kreg[i] = load_stream(kbase + row);
      vreg[i] = load_stream(vbase + row);
    }
  };
  // transposing V reads (see below): lane's row/column offset within the V tile
  const int vofs = (4 * lq + ((lane & 15) >> 2)) * VSD + 4 * (lane & 3);

  constexpr int STEP = SOLO ? DT : 4 * DT;  // a wave's tiles: all of them, or every 4th
  int j0 = s_lo + (SOLO ? 0 : wave * DT);
  if (j0 < s_hi) {
    fetch_blk(j0);
    load(j0);
    fetch_blk(j0 + STEP);
  }
  for (; j0 < s_hi; j0 += STEP) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = 8 * i + (lane >> 3);
      *reinterpret_cast<u32x4*>(Kw + key * KSD + 8 * (lane & 7)) = kreg[i];
      *reinterpret_cast<u32x4*>(Vw + key * VSD + 8 * (lane & 7)) = vreg[i];
    }
    wave_lds_sync();  // the tile is visible to every lane of the wave
    const int jn = j0 + STEP;
    if (jn < s_hi) {
      load(jn);  // next tile in flight during this one's math
      fetch_blk(jn + STEP);
    }

    // S^T: 4 blocks of 16 keys x 16 heads; A operand = K rows 16*kb + lc, d 32*ks + 8*lq
    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Kw + (16 * kb + lc) * KSD + 32 * ks + 8 * lq);
        acc = mfma16(ka, qb[ks], acc);
      }
      s[kb] = acc;
    }
    // lane holds keys j0 + 16*kb + 4*lq + r of head lc
    if (j0 + DT > s_hi) {
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

    // O^T += V^T P^T over 2 k-steps of 32 keys: keys 32u + {4lq..4lq+3, 16+4lq..16+4lq+3}.
    // V^T via the transposing LDS load: in lane group lq, lane j reads 4 d of key
    // row 32u + 4lq + j/4; the hardware hands lane i the 4 keys at d = 16*dt + i.
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
        const __bf16* base = Vw + vofs + 32 * u * VSD + 16 * dt;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 16 * VSD));
        const i16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[dt] = mfma16(__builtin_bit_cast(bf16x8, w), pbv, o[dt]);
      }
    }
    wave_lds_sync();  // all lanes done reading the tile before the next overwrite
  }

  if (SOLO) {
    // the wave holds its unit's whole key range: fold in the sink and finish
    float lt = l_run + __shfl_xor(l_run, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    if (lc < n_heads) finish_column(a, b, q_row, a.lse_row0 ? sv.q_row0 : 0, h_base + lc, lq, m_run, lt, o);
    return;
  }

  // ---- merge the 4 waves: per head max m, sum l, output acc[d]
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
    // lane holds O^T[d = 16*dt + 4*lq + r][head lc]
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) red_o[(wave * 16 + lc) * 68 + 16 * dt + 4 * lq + r] = o[dt][r];
  }
  __syncthreads();
  {
    const int hh = tid >> 4;         // head within the chunk
    const int d0 = (tid & 15) * 4;   // 4 output columns
    if (hh < n_heads) {
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
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) t += red_o[(w * 16 + hh) * 68 + d0 + cq] * wsc[w];
        acc[cq] = t;
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

// ---- whole-row form: 8 KV heads, contiguous cache --------------------------
// With 8 KV heads of 64 columns, one cache position's K (or V) row is 1 KB and
// one wave load brings a whole row (lane i: bytes 16i .. 16i+15).  Whole rows
// stream from HBM faster than the 128-byte per-head pieces the form above
// reads, where the eight pieces of a row are fetched by eight workgroups at
// different times.  A workgroup owns (sequence, split of the key range) and all
// 8 KV heads.  Per 32-position tile each wave loads 8 rows of K and of V into
// registers and stores them in the workgroup's LDS tile; then each wave
// computes 2 KV heads, i.e. 16 query heads as the 16 MFMA columns: columns 0-7
// are the query heads of KV head 2w, columns 8-15 those of KV head 2w+1.  The
// S^T and O^T products take each KV head's operand in turn with the other
// head's columns zeroed in Q^T (resp. P^T), so one accumulator holds both.
// The next two tiles' loads are in flight during a tile's math.
constexpr int RT = 32;           // positions per tile
constexpr int RROW = 1024 + 32;  // LDS row stride in bytes: successive rows start 8 banks apart
constexpr int RKV = RT * RROW;   // bytes of one K (or V) tile

template <int MODE>
__global__ __launch_bounds__(DTHREADS, 2) void decode_rows_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[2 * RKV];  // K tile, V tile

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lc = lane & 15;  // column (query head) of the S^T / O^T tiles; key row of the K operand
  const int lq = lane >> 4;
  const int split = (int)blockIdx.x % a.n_splits;
  const int b = (int)blockIdx.x / a.n_splits;

  const SeqView sv = seq_view<MODE>(a.seq, b, false);
  const int L = sv.kv_len;
  const int W = a.window;
  const int lo_all = W > 0 ? max(0, L - W) : 0;
  const int ns = W > 0 ? min(a.sink_tokens, lo_all) : 0;  // sink tokens below the window
  const int nv = ns + (L - lo_all);                        // keys read, "virtual" index as above
  const int s_lo = split * a.split_len;
  const int s_hi = min(nv, s_lo + a.split_len);
  const int nt = s_hi > s_lo ? (s_hi - s_lo + RT - 1) / RT : 0;

  const int hsel = lc >> 3;  // which of the wave's two KV heads the column belongs to
  const int col = lc & 7;
  const bool live = col < a.G;
  const int hq = (2 * wave + hsel) * a.G + col;
  const int64_t q_row = b;

  // Q^T operands of the two KV heads: the lane's query head, d = 32*ks + 8*lq,
  // in the operand of its own KV head and zero in the other.  The loads go out
  // first and are used only once the first K/V tile is requested, so those
  // requests do not wait for them; idle columns load a valid row and discard it.
  u32x4 qw[2];
  {
    const __bf16* qp = a.q + (q_row * a.Hq + min(hq, a.Hq - 1)) * (int64_t)kHeadDim + 8 * lq;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) qw[ks] = *reinterpret_cast<const u32x4*>(qp + 32 * ks);
  }
  bf16x8 qh[2][2];
  auto take_q = [&]() {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      qh[0][ks] = __builtin_bit_cast(bf16x8, live && hsel == 0 ? qw[ks] : z);
      qh[1][ks] = __builtin_bit_cast(bf16x8, live && hsel == 1 ? qw[ks] : z);
    }
  };

  float m_run = kNegBig, l_run = 0.f;
  f32x4 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto key_of = [&](int v) { return v < ns ? v : lo_all + (v - ns); };
  // tile t: this wave's rows 8*wave + i; rows past the split repeat its last
  // row (masked below, always in bounds)
  auto load = [&](u32x4 (&kr)[8], u32x4 (&vr)[8], int t) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int v = min(s_lo + t * RT + 8 * wave + i, s_hi - 1);
      const int64_t row = kv_row<MODE>(a.seq, sv, key_of(v)) * (8 * kHeadDim);
      kr[i] = load_stream(a.k + row + 8 * lane);
      vr[i] = load_stream(a.v + row + 8 * lane);
    }
  };
  auto store = [&](const u32x4 (&kr)[8], const u32x4 (&vr)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ofs = (8 * wave + i) * RROW + 16 * lane;
      *reinterpret_cast<u32x4*>(lds + ofs) = kr[i];
      *reinterpret_cast<u32x4*>(lds + RKV + ofs) = vr[i];
    }
  };
  // transposing V reads: lane's row / byte offset within a head's 32 x 64 V block
  const int vofs = (4 * lq + (lc >> 2)) * RROW + 8 * (lane & 3);

  auto compute = [&](int t) {
    const int j0 = s_lo + t * RT;
    // S^T: 2 blocks of 16 keys x 16 columns; K operand = key 16*kb + lc, d 32*ks + 8*lq
    f32x4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(
              lds + (16 * kb + lc) * RROW + (2 * wave + e) * 2 * kHeadDim + 2 * (32 * ks + 8 * lq));
          acc = mfma16(ka, qh[e][ks], acc);
        }
      s[kb] = acc;
    }
    // lane holds keys j0 + 16*kb + 4*lq + r of column lc
    if (j0 + RT > s_hi) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (j0 + 16 * kb + 4 * lq + r >= s_hi) s[kb][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * a.scale_log2);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    float rs = 0.f;
    bf16x8 pbv;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(__builtin_fmaf(s[kb][r], a.scale_log2, -m_new));
        rs += p;
        pbv[4 * kb + r] = (__bf16)p;
      }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
    // O^T += V^T P^T over the tile's 32 keys (keys 4lq..4lq+3 and 16+4lq..16+4lq+3
    // in the lane's P^T operand, matching the rows of the transposing V reads)
    const u32x4 z = {0u, 0u, 0u, 0u};
    const u32x4 pw = __builtin_bit_cast(u32x4, pbv);
    const bf16x8 ph[2] = {__builtin_bit_cast(bf16x8, hsel == 0 ? pw : z), __builtin_bit_cast(bf16x8, hsel == 1 ? pw : z)};
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const char* base = lds + RKV + vofs + (2 * wave + e) * 2 * kHeadDim + 2 * 16 * dt;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 16 * RROW));
        const i16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[dt] = mfma16(__builtin_bit_cast(bf16x8, w), ph[e], o[dt]);
      }
  };
  // Two register sets take turns, so two tiles are in flight: per tile, store
  // its set in LDS, request the tile two ahead into that set (its loads fly
  // during this tile's and the next tile's math), compute.  The loop runs the
  // two sets in turn with every request made; the last tiles are peeled off,
  // so inside the loop every path has the same loads in flight.  (Measured
  // against one set: B64 x 8192 -2 %, B8 x 131072 -2 %, ring decode B4096 x
  // W128 -1 %, with one workgroup per CU.)
  auto step = [&](u32x4 (&kr)[8], u32x4 (&vr)[8], int t, bool refill) {
    __syncthreads();  // every wave is done reading the previous tile
    store(kr, vr);
    if (refill) load(kr, vr, t + 2);
    __syncthreads();  // the tile is in LDS
    compute(t);
  };

  if (nt > 0) {
    u32x4 ka[8], va[8], kb[8], vb[8];
    __builtin_amdgcn_sched_barrier(0);  // Q requested first, taken after the first tiles are requested
    load(ka, va, 0);
    if (nt > 1) load(kb, vb, 1);
    __builtin_amdgcn_sched_barrier(0);
    take_q();
    int t = 0;
    for (; t + 3 < nt; t += 2) {
      step(ka, va, t, true);
      step(kb, vb, t + 1, true);
    }
    if (t + 2 < nt) {  // three tiles left: the first one still requests the last
      step(ka, va, t, true);
      step(kb, vb, t + 1, false);
      step(ka, va, t + 2, false);
    } else if (t + 1 < nt) {
      step(ka, va, t, false);
      step(kb, vb, t + 1, false);
    } else {
      step(ka, va, t, false);
    }
  }

  // the wave holds its 16 columns over the split's whole key range
  float lt = l_run + __shfl_xor(l_run, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  if (!live) return;
  if (a.n_splits == 1) {
    finish_column(a, b, q_row, 0, hq, lq, m_run, lt, o);
    return;
  }
  const int64_t slot = ((int64_t)b * a.Hq + hq) * a.n_splits + split;
  if (lq == 0) {
    a.ws_ml[slot * 2 + 0] = m_run;
    a.ws_ml[slot * 2 + 1] = lt;
  }
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) *reinterpret_cast<f32x4*>(a.ws_acc + slot * kHeadDim + 16 * dt + 4 * lq) = o[dt];
}

// Merge of the split partials: one wave per (sequence, query head), lane = output column.
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeArgs a) {
  const int lane = threadIdx.x;
  const int hq = blockIdx.x % a.Hq;
  const int b = blockIdx.x / a.Hq;
  int64_t q_row = b;
  int64_t row0 = 0;
  if (a.varlen_q) {
    int r0, r1;
    q_range(a.seq, b, r0, r1);
    if (r1 - r0 != 1) return;
    q_row = r0;
    row0 = r0;
  }
  const int64_t base = ((int64_t)b * a.Hq + hq) * a.n_splits;
  const int ns = a.n_splits;
  const float s2 = a.sinks ? a.sinks[hq] * kLog2e : -INFINITY;
  float M = s2;
  float Z = 0.f;
  float acc = 0.f;
  if (ns <= 8) {
    // one trip to memory: every split's (m, l) and partial row are loaded
    // before any of them is used; lane s holds split s's (m, l), and the
    // weights reach every lane by readlane
    float m_s = -INFINITY, l_s = 0.f;
    if (lane < ns) {
      m_s = a.ws_ml[(base + lane) * 2];
      l_s = a.ws_ml[(base + lane) * 2 + 1];
    }
    float x[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) x[s] = s < ns ? a.ws_acc[(base + s) * kHeadDim + lane] : 0.f;
    M = wave_max(fmaxf(M, m_s));
    const float w_s = lane < ns ? fast_exp2(m_s - M) : 0.f;
    Z = wave_sum(l_s * w_s) + fast_exp2(s2 - M);
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s < ns) acc += x[s] * __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_s), s));
  } else {
    for (int s = lane; s < ns; s += 64) M = fmaxf(M, a.ws_ml[(base + s) * 2]);
    M = wave_max(M);
    for (int s = lane; s < ns; s += 64) Z += a.ws_ml[(base + s) * 2 + 1] * fast_exp2(a.ws_ml[(base + s) * 2] - M);
    Z = wave_sum(Z) + fast_exp2(s2 - M);
    for (int s = 0; s < ns; ++s) acc += a.ws_acc[(base + s) * kHeadDim + lane] * fast_exp2(a.ws_ml[(base + s) * 2] - M);
  }
  const float inv = Z > 0.f ? 1.f / Z : (Z == 0.f ? 0.f : Z);
  a.out[(q_row * a.Hq + hq) * kHeadDim + lane] = (__bf16)(acc * inv);
  if (a.lse && lane == 0) {
    const float v = (Z == 0.f) ? -INFINITY : (M + __log2f(Z)) * kLn2;
    a.lse[(int64_t)b * a.lse_sb + (int64_t)hq * a.lse_sh + (a.lse_row0 ? row0 : 0)] = v;
  }
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, int kv_mode, hipStream_t s) {
  const int units = a.B * a.Hkv * a.n_hc;
  if (units <= 0) return hipSuccess;
  if (a.solo) {
    if (a.n_splits != 1) return hipErrorInvalidValue;
    const int grid = (units + 3) / 4;
    if (kv_mode == KV_BATCHED)
      hipLaunchKernelGGL((decode_split_kernel<KV_BATCHED, true>), dim3(grid), dim3(DTHREADS), 0, s, a);
    else if (kv_mode == KV_PAGED)
      hipLaunchKernelGGL((decode_split_kernel<KV_PAGED, true>), dim3(grid), dim3(DTHREADS), 0, s, a);
    else
      hipLaunchKernelGGL((decode_split_kernel<KV_PACKED, true>), dim3(grid), dim3(DTHREADS), 0, s, a);
    return hipGetLastError();
  }
  if (a.rows) {
    // whole-row form: 8 KV heads of at most 8 query heads each, contiguous cache, one query per sequence
    if (kv_mode != KV_BATCHED || a.Hkv != 8 || a.G > 8 || a.varlen_q || a.n_hc != 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_rows_kernel<KV_BATCHED>), dim3(a.B * a.n_splits), dim3(DTHREADS), 0, s, a);
  } else {
    const int grid = units * a.n_splits;
    if (kv_mode == KV_BATCHED)
      hipLaunchKernelGGL((decode_split_kernel<KV_BATCHED, false>), dim3(grid), dim3(DTHREADS), 0, s, a);
    else if (kv_mode == KV_PAGED)
      hipLaunchKernelGGL((decode_split_kernel<KV_PAGED, false>), dim3(grid), dim3(DTHREADS), 0, s, a);
    else
      hipLaunchKernelGGL((decode_split_kernel<KV_PACKED, false>), dim3(grid), dim3(DTHREADS), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_splits == 1) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(a.B * a.Hq), dim3(64), 0, s, a);
  return hipGetLastError();
}

// Metadata-check flags of this file's kernels (recorded only when built with GQA_DEBUG).
GQA_DEBUG_FLAGS_ACCESSOR(debug_flags_decode)

}  // namespace gqa
