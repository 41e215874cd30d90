// Argument blocks and launchers of the gfx950 kernels (internal to the library).
#pragma once

#include "common.h"

namespace gqa {

// Prefill-style attention: many query rows per sequence, one workgroup per
// (sequence, KV head, group of 8 tiles of 32 (position, head) query rows).
struct PrefillArgs {
  const __bf16* q;
  const __bf16* k;   // KV_RING: the rings
  const __bf16* v;
  const __bf16* k2;  // KV_RING: the chunk's own rows [Tq, Hkv, D]
  const __bf16* v2;
  const float* sinks;
  __bf16* out;
  float* lse;
  SeqArgs seq;
  int B, Hq, Hkv, G;
  int window;
  int sink_tokens;   // first positions that stay visible past the window (window > 0)
  float scale_log2;  // softmax scale times log2(e)
  int wg_per_seq;    // workgroups per (sequence, KV head)
  int skip_single;   // sequences with q_len == 1 are left to the decode kernel
  int64_t lse_sb;    // lse index = b*lse_sb + h*lse_sh + t (+ q_row0 when lse_row0)
  int64_t lse_sh;
  int lse_row0;
  int sort_seq;      // ragged batches (B <= 256): dispatch the sequences with the most work first
  int rope;          // queries arrive unrotated: 0 no, 1 pairs (2i, 2i+1), 2 pairs (i, i + D/2)
  const float* inv_freq;  // rope: [D/2] or NULL (the default table)
  float rope_mscale;
  // whole-sequence windowed layers whose pairs of tile groups need at most 3
  // key tiles (window <= 128, no sink tokens, G = 8 or a multiple of 16): a
  // workgroup runs two tile groups over the same tiles
  int two_step;
  // filled by the launcher: workgroups per (sequence, KV head), and the
  // divisors of the workgroup-to-job mapping
  int wg_per_job;
  FastDiv div_wg_per_job, div_hkv, div_g, div_units;
  FastDiv div_ring;  // KV_RING: the ring's slot count seq.lmax
};

// Decode-style attention: one query token per sequence, KV split over
// n_splits workgroups per (sequence, KV head, chunk of 16 query heads).
struct DecodeArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const float* sinks;
  __bf16* out;
  float* lse;
  SeqArgs seq;
  int B, Hq, Hkv, G, n_hc;
  int window;
  int sink_tokens;   // first positions that stay visible past the window (window > 0)
  float scale_log2;
  int n_splits;
  int split_len;     // keys per split, a multiple of 64
  float* ws_ml;      // [B*Hq, n_splits, 2]  running max (log2 units) and sum
  float* ws_acc;     // [B*Hq, n_splits, 64] unnormalised output
  int varlen_q;      // queries packed by cu_seqlens_q; sequences with q_len != 1 are skipped
  int64_t lse_sb;    // lse index = b*lse_sb + h*lse_sh (+ q_row0 when lse_row0)
  int64_t lse_sh;
  int lse_row0;
  int solo;          // one (sequence, KV head, head chunk) per wave, whole key range (n_splits == 1)
  int rows;          // whole-row form: a workgroup per (sequence, split) covers all 8 KV heads
};

// fp32 I/O path: one wave per (query row, query head).
struct Fp32Args {
  const float* q;
  const float* k;   // KV_RING: the rings
  const float* v;
  const float* k2;  // KV_RING: the chunk's own rows [Tq, Hkv, D]
  const float* v2;
  const float* sinks;
  float* out;
  float* lse;
  SeqArgs seq;
  int B, Hq, Hkv, G;
  int window;
  int sink_tokens;   // first positions that stay visible past the window (window > 0)
  float scale_log2;
  int max_q_len;
  int varlen_q;
  int64_t lse_sb;
  int64_t lse_sh;
  int lse_row0;
};

// KV append into per-sequence rings of W slots (position p in slot p % W).
struct RingAppendArgs {
  const char* k_new;            // [T, Hkv, D] rows of new tokens
  const char* v_new;
  char* k_ring;                 // [B, W, Hkv, D]
  char* v_ring;
  const int32_t* cu_seqlens_q;  // [B+1] or NULL (then T == B, one new token per sequence)
  const int32_t* seqlens;       // [B] positions including the new tokens
  int64_t T;
  int B, W;
  int row_bytes;                // Hkv * D * element size
};

// Rotary encoding of new rows fused with their KV-cache append.
struct RopeAppendArgs {
  const void* q;                // [T, Hq, D]
  const void* k;                // [T, Hkv, D]
  const void* v;                // [T, Hkv, D]
  void* q_out;                  // [T, Hq, D] (may be q)
  void* k_cache;
  void* v_cache;
  const float* inv_freq;        // [D/2]
  const int32_t* cu_seqlens_q;  // [B+1] or NULL (one row per sequence)
  const int32_t* seqlens;       // [B]
  const int32_t* block_table;   // paged cache only
  int64_t T;
  int B, Hq, Hkv;
  int cache_kind;               // 0 contiguous [B, cache_len, ..], 1 paged, 2 ring of cache_len slots
  int cache_len;
  int max_blocks, log2_block, num_blocks;
  int pairing;                  // 0: (2i, 2i+1); 1: (i, i + D/2)
  float mscale;
  int fp32;
};

// One decode step in one launch: rotary encoding of the new token's query and
// key, append of the rotated key and the value to the cache, attention.
constexpr int kStepMaxG = 16;     // query heads per KV head the fused step supports (the MFMA columns)
constexpr int kStepMaxKeys = 2048;  // keys a query of the fused step may read (one workgroup streams them)
enum StepCacheKind : int { STEP_CACHE_CONTIGUOUS = 0, STEP_CACHE_PAGED = 1, STEP_CACHE_RING = 2 };
struct DecodeStepArgs {
  const __bf16* q;          // [B, Hq, D] new queries, not rotated
  const __bf16* k_new;      // [B, Hkv, D] new keys, not rotated
  const __bf16* v_new;      // [B, Hkv, D]
  __bf16* q_out;            // [B, Hq, D] rotated queries, or NULL
  __bf16* k_cache;          // contiguous [B, cache_len, Hkv, D], paged [Nblk, bs, Hkv, D], ring [B, W, Hkv, D]
  __bf16* v_cache;
  const int32_t* seqlens;   // [B] positions including the new token
  const float* inv_freq;    // [D/2] or NULL (the default table)
  float mscale;
  int pairing;              // 0: (2i, 2i+1); 1: (i, i + D/2)
  int cache_kind;           // StepCacheKind
  int cache_len;            // contiguous: rows per sequence; ring: slots W
  const int32_t* block_table;
  int max_blocks, log2_block, num_blocks;
  const float* sinks;
  __bf16* out;              // [B, Hq, D]
  float* lse;               // [B, Hq] or NULL
  int B, Hq, Hkv, G;
  int window;               // keys of the query: the last `window` positions (0: all), plus sink tokens
  int sink_tokens;
  float scale_log2;
};

// Backward of the prefill over whole sequences [B, S, H, D].
struct BwdArgs {
  const void* q;       // [B, S, Hq, D]
  const void* k;       // [B, S, Hkv, D]
  const void* v;
  const void* o;       // forward output [B, S, Hq, D]
  const void* dout;    // dL/do [B, S, Hq, D]
  const float* lse;    // forward log-sum-exp [B, Hq, S], natural log, sink included
  const float* sinks;  // [Hq] or NULL
  void* dq;            // [B, S, Hq, D]
  void* dk;            // [B, S, Hkv, D]
  void* dv;
  float* dsinks;       // [Hq] or NULL
  float* dlt;          // workspace [B, Hq, S]: <dO, o>
  float* lse2;         // workspace [B, Hq, S]: lse * log2(e)
  float* dsink_part;   // workspace [Hq, B, ceil(S / 1024)]: block sums of the sink gradient
  float* part;         // workspace [B*Hkv, key blocks of 64, n_slabs, 2, 64, 64] fp32 (n_slabs > 1)
  int n_slabs;         // the query range of a key block is cut at multiples of slab_len
  int slab_len;        // a multiple of 32
  int B, S, Hq, Hkv, G;
  int window;
  int sink_tokens;
  float scale;         // softmax scale
  float scale_log2;    // scale * log2(e)
  int fp32;
  // divisors of the workgroup-to-job mappings, filled by the launcher
  FastDiv div_units, div_hkv, div_g, div_nkb, div_per_unit, div_slab_len, div_wg_per_seq;
};

int prefill_ntiles_per_wg();  // N-tiles (32 rows of one head) per prefill workgroup
hipError_t launch_prefill_bf16(const PrefillArgs& a, int kv_mode, bool varlen_q, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs& a, int kv_mode, hipStream_t s);
hipError_t launch_fp32(const Fp32Args& a, int kv_mode, hipStream_t s);
hipError_t launch_ring_append(const RingAppendArgs& a, hipStream_t s);
hipError_t launch_rope_append(const RopeAppendArgs& a, hipStream_t s);
hipError_t launch_backward(const BwdArgs& a, hipStream_t s);
hipError_t launch_decode_step(const DecodeStepArgs& a, hipStream_t s);
void backward_plan(int B, int S, int Hkv, int window, int sink_tokens, int* n_slabs, int* slab_len);  // split of the dK/dV query ranges

// Metadata-check flag words, one per kernel file (common.h); zero unless built
// with GQA_DEBUG.  Each call copies synchronously and optionally clears.
hipError_t debug_flags_backward(unsigned int* flags, bool reset);
hipError_t debug_flags_decode(unsigned int* flags, bool reset);
hipError_t debug_flags_fp32(unsigned int* flags, bool reset);
hipError_t debug_flags_prefill(unsigned int* flags, bool reset);
hipError_t debug_flags_ring(unsigned int* flags, bool reset);
hipError_t debug_flags_rope(unsigned int* flags, bool reset);
hipError_t debug_flags_step(unsigned int* flags, bool reset);

}  // namespace gqa
