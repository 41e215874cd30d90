/*
 * gqa_attn.h -- C ABI of the MI355X (gfx950) attention library.
 *
 * Forward pass of causal grouped-query attention with a learned per-head sink
 * logit and an optional sliding window, over Q/K that already carry their
 * rotary position encoding; the rotary encoding and KV-cache append of new
 * rows; and the backward pass of the prefill.
 *
 * What is computed (for query head h at sequence position p):
 *   G = Hq / Hkv, g = h / G            -- query heads share KV heads in
 *                                         contiguous groups.  «GPT-OSS-20B :
 *                                         Architecture MoE & Résumé du Model
 *                                         Card», §3.3 (64 query heads over 8
 *                                         KV heads, 8 per KV head).
 *   J = { j : j <= p, and (j > p - W or j < n_sink) when W > 0 }
 *                                      -- causal (decoder-only, autoregressive:
 *                                         «OpenAI lance gpt-oss-20b, qui tient
 *                                         sur 16 Go», opening section); a
 *                                         window keeps the W most recent keys
 *                                         counting the query's own position
 *                                         («GPT-OSS vs Qwen3», section
 *                                         "Utilisation de Sliding Window
 *                                         Attention": the last 128 tokens).
 *                                         n_sink ("sink_tokens") keeps the
 *                                         first positions visible past the
 *                                         window edge: the classical
 *                                         start-of-sequence sink tokens of
 *                                         «GPT-OSS vs Qwen3», section
 *                                         "Attention Bias et Sinks" (0 = none;
 *                                         no effect on dense layers).
 *   x_j = scale * <q, k_j[g]>,  s = sinks[h]
 *   o   = sum_{j in J} e^{x_j} v_j[g] / (e^{s} + sum_{j in J} e^{x_j})
 *   lse = ln(e^{s} + sum_{j in J} e^{x_j})
 *                                      -- the sink is a learned logit per head
 *                                         that only adds to the softmax
 *                                         denominator («GPT-OSS vs Qwen3»,
 *                                         section "Attention Bias et Sinks";
 *                                         off-by-one attention when s = 0).
 *   Dense and windowed layers alternate («gpt-oss Deep Dive with Xiaoli Alex
 *   Shen», Key Moments); the caller passes the layer's window on each call.
 *   If J is empty and there is no sink, o = 0 and lse = -inf.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers, row-major, densely packed,
 *     16-byte aligned.  The caller owns every buffer; the library never
 *     allocates device memory, keeps no state between calls and is
 *     thread-safe.  Split-K scratch comes in through `workspace`.
 *   - dtype: GQA_BF16 (inputs/outputs bf16, fp32 accumulation) or GQA_FP32
 *     (everything fp32).  q, k, v and out share the dtype.  sinks and lse are
 *     always fp32.
 *   - sinks: [Hq] fp32, or NULL for no sink (s = -inf: plain softmax).
 *   - lse: optional fp32 output (NULL = not written), natural-log units.
 *   - head_dim D must be 64; Hq must be a positive multiple of Hkv.
 *   - window: 0 = dense causal; W > 0 = the W most recent keys; W < 0 is an
 *     error.  sink_tokens: >= 0 positions at the start of every sequence that
 *     windowed layers keep visible; negative is an error.
 *   - scale: scale > 0 is used as given; scale == 0 selects 1/sqrt(D); a
 *     negative or NaN scale is an error.
 *   - stream: a hipStream_t (NULL = the default stream).  Every launch is
 *     asynchronous on it; the library never synchronises.
 *   - Errors: arguments are validated synchronously, before any launch; on
 *     error a negative status is returned, nothing is launched and `out` is
 *     untouched.  A failed launch returns GQA_ERR_HIP.  No C++ exception
 *     crosses this ABI.  gqa_attn_last_error() gives the detail (per thread).
 *   - Values that live on the device (seqlens, cu_seqlens, block tables) are
 *     not checked on the host.  The kernels clamp lengths to the stated
 *     maxima and block ids to [0, num_blocks) so that no access leaves the
 *     caller's buffers; results for out-of-range metadata are unspecified.
 */
#ifndef GQA_ATTN_H
#define GQA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gqa_dtype { GQA_BF16 = 0, GQA_FP32 = 1 } gqa_dtype;

enum {
  GQA_OK = 0,
  GQA_ERR_INVALID_ARG = -1,   /* NULL pointer, negative size, bad window/scale */
  GQA_ERR_UNSUPPORTED = -2,   /* dtype, head_dim != 64, Hq % Hkv != 0, block size */
  GQA_ERR_WORKSPACE = -3,     /* workspace missing or smaller than required */
  GQA_ERR_HIP = -4            /* a HIP launch failed */
};

/* Library version, as 10000*major + 100*minor + patch. */
int gqa_attn_version(void);

/* Human-readable name of a status code (static string). */
const char* gqa_attn_status_string(int status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* gqa_attn_last_error(void);

/*
 * Device-side metadata checks.
 *
 * Metadata the kernels read from device memory (seqlens_k / seqlens,
 * cu_seqlens_q, cu_seqlens_k, block tables) cannot be validated before the
 * launch without a synchronisation, so the kernels clamp it: a sequence length
 * to the cache capacity, a query range to [0, Tq], a block id to
 * [0, num_blocks), a packed row to [0, num_rows).  No access then leaves the
 * caller's buffers, and results for metadata that needed clamping are
 * unspecified.  A library built with GQA_DEBUG (`python -m
 * attention_gqa_causal_amd.build --debug` writes libgqa_attn_debug.so) also
 * records each kind of value it had to clamp:
 */
enum gqa_debug_flag {
  GQA_DBG_SEQLENS_K = 1,     /* a sequence length < 0, above the cache capacity or above max_kv_len */
  GQA_DBG_BLOCK_TABLE = 2,   /* a block table entry outside [0, num_blocks) */
  GQA_DBG_CU_SEQLENS_Q = 4,  /* cu_seqlens_q outside [0, Tq] or decreasing */
  GQA_DBG_PACKED_ROW = 8,    /* a packed KV row outside [0, num_rows) */
  GQA_DBG_Q_LEN = 16         /* more new query tokens than KV positions */
};

/*
 * ORs the records of every kernel into *flags (GQA_DBG_* bits) and, when
 * reset != 0, clears them.  Synchronises the device (blocking copies), so it
 * is a debugging call, not one for a serving loop.  Release builds set
 * *flags = 0 and return GQA_ERR_UNSUPPORTED without touching the device.
 * Errors: flags == NULL -> GQA_ERR_INVALID_ARG; a failed copy -> GQA_ERR_HIP.
 */
int gqa_attn_debug_flags(unsigned int* flags, int reset);

/*
 * Prefill: causal self-attention over whole sequences of equal length.
 *   q   [B, S, Hq, D]     k, v [B, S, Hkv, D]     out [B, S, Hq, D]
 *   lse [B, Hq, S] fp32 (optional)
 * Position of row t is t.  B == 0 or S == 0 is a no-op returning GQA_OK.
 */
int gqa_attn_prefill(const void* q, const void* k, const void* v, const float* sinks,
                     void* out, float* lse,
                     int B, int S, int Hq, int Hkv, int D,
                     int window, int sink_tokens, float scale, int dtype, void* stream);

/*
 * Prefill whose queries arrive unrotated: the kernel applies the rotary
 * encoding of «GPT-OSS-20B : Architecture MoE & Résumé du Model Card» §3.4
 * («GPT-OSS vs Qwen3», "Adoption de RoPE") to each query row as it loads it,
 * at the row's position t, with the same angles and rotation as
 * gqa_rope_append (inv_freq [D/2] fp32 device or NULL for the default table,
 * mscale, pairing GQA_ROPE_INTERLEAVED or GQA_ROPE_HALVES).  The result
 * equals, bit for bit, gqa_rope_append's q_out passed to gqa_attn_prefill;
 * the rotated queries are not written out.  k must already be rotated
 * (gqa_rope_append with q = q_out = NULL rotates and appends the keys alone).
 * Other arguments, layouts and errors as gqa_attn_prefill; bf16 only
 * (GQA_FP32: GQA_ERR_UNSUPPORTED).
 */
int gqa_attn_prefill_rope(const void* q, const void* k, const void* v, const float* sinks,
                          void* out, float* lse,
                          int B, int S, int Hq, int Hkv, int D,
                          int window, int sink_tokens, float scale,
                          const float* inv_freq, float mscale, int pairing, int dtype, void* stream);

/*
 * Decode: one new query token per sequence against a contiguous KV cache.
 *   q [B, Hq, D]    k_cache, v_cache [B, Lmax, Hkv, D]    out [B, Hq, D]
 *   seqlens [B] int32 (device): cached positions of sequence b INCLUDING the
 *     new token, in [1, Lmax]; the query sits at position seqlens[b] - 1.
 *   lse [B, Hq] fp32 (optional)
 * The sequence is split over up to `gqa_attn_decode_workspace_size`-sized
 * partials; pass a workspace of at least that many bytes (may be NULL when
 * that size is 0).  On windowed layers only the last W positions (and the
 * sink tokens below them) are read.
 */
size_t gqa_attn_decode_workspace_size(int B, int Lmax, int Hq, int Hkv, int D,
                                      int window, int sink_tokens, int dtype);

int gqa_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* seqlens, const float* sinks,
                    void* out, float* lse,
                    int B, int Lmax, int Hq, int Hkv, int D,
                    int window, int sink_tokens, float scale, int dtype,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Allocation-free decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): gqa_attn_decode with the same arguments, minus the workspace.
 * Its split partials live in a fixed array of GQA_NOALLOC_SCRATCH_BYTES
 * (16 MiB) that the library holds on every GPU it runs on until the process
 * ends; the call allocates nothing and makes no allocating library call.
 * A decode that needs more partials than that (gqa_attn_decode_workspace_size
 * of the same arguments above the limit; for 64 query heads roughly
 * B * splits > 990) returns GQA_ERR_WORKSPACE before touching the device.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (on different streams, or from different threads without ordering) race and
 * give unspecified results; calls in order on one stream are safe.  The array
 * needs no clearing (every partial a call reads is written by that call).
 */
#define GQA_NOALLOC_SCRATCH_BYTES (16u << 20)

int gqa_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seqlens, const float* sinks,
                            void* out, float* lse,
                            int B, int Lmax, int Hq, int Hkv, int D,
                            int window, int sink_tokens, float scale, int dtype, void* stream);

/*
 * Variable-length packed queries over a paged (or packed) KV cache; mixes
 * prefill chunks and single-token decode steps in one call.
 *   q [Tq, Hq, D], out [Tq, Hq, D]; sequence b owns query rows
 *     cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (cu_seqlens_q [B+1] int32,
 *     device, non-decreasing, cu_seqlens_q[B] == Tq).
 *   seqlens_k [B] int32 (device): KV positions of sequence b, including its
 *     q_len new tokens; the q_len queries are the newest positions, query t at
 *     position seqlens_k[b] - q_len + t (q_len <= seqlens_k[b]).
 *   Paged (block_table != NULL): k_cache, v_cache [num_blocks, block_size, Hkv, D];
 *     position p of sequence b is slot p % block_size of physical block
 *     block_table[b * max_blocks + p / block_size] (block_table [B, max_blocks]
 *     int32, device).  block_size must be a power of two in [1, 1024].
 *   Packed (block_table == NULL): k_cache, v_cache [num_rows, Hkv, D] and
 *     sequence b's positions start at row cu_seqlens_k[b] (cu_seqlens_k [B+1]
 *     int32, device); num_blocks is then the row count and block_size is ignored.
 *   max_q_len (host): upper bound of any q_len; max_kv_len (host): upper
 *     bound of any seqlens_k[b] (for paged caches at most
 *     max_blocks * block_size).  Both size the grids; a seqlens_k[b] above
 *     max_kv_len is metadata out of range (clamped to it, GQA_DBG_SEQLENS_K).
 *   lse [Hq, Tq] fp32 (optional).
 */
size_t gqa_attn_varlen_workspace_size(int B, int max_q_len, int max_kv_len, int Hq, int Hkv,
                                      int D, int window, int sink_tokens, int dtype);

int gqa_attn_varlen_paged(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                          const int32_t* block_table, int max_blocks, int block_size,
                          const int32_t* cu_seqlens_k, int num_blocks,
                          const float* sinks, void* out, float* lse,
                          int B, int Tq, int max_q_len, int max_kv_len,
                          int Hq, int Hkv, int D,
                          int window, int sink_tokens, float scale, int dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Ring-buffer KV cache of sliding-window layers.
 *
 * A windowed layer attends to the last W positions only («GPT-OSS vs Qwen3»,
 * section "Utilisation de Sliding Window Attention": 128 tokens, to bound the
 * memory use), so its cache needs W slots per sequence instead of the whole
 * history: position p of sequence b lives in slot p % W.
 *   k_ring, v_ring [B, W, Hkv, D] (dtype as below).
 */

/*
 * Writes the K and V rows of new tokens into their ring slots, bit for bit.
 *   k_new, v_new [T, Hkv, D].
 *   cu_seqlens_q == NULL: T == B, row b is the newest token of sequence b, at
 *     position seqlens[b] - 1 (the decode step).
 *   cu_seqlens_q [B+1] int32 (device, non-decreasing): sequence b's new rows
 *     are cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1, the newest q_len positions:
 *     row t at position seqlens[b] - q_len + t (a prefill chunk).
 *   seqlens [B] int32 (device): positions of sequence b including the new rows.
 * Only positions p >= seqlens[b] - W are written; of a chunk longer than the
 * ring the older rows would only be overwritten by newer ones of the same
 * call.  Rows with a negative position are skipped.  dtype sets the element
 * size (GQA_BF16: 2 bytes, GQA_FP32: 4).  Errors as for every entry point;
 * the caller orders this call before the attention that reads the ring.
 */
int gqa_kv_ring_append(const void* k_new, const void* v_new,
                       const int32_t* cu_seqlens_q, const int32_t* seqlens,
                       void* k_ring, void* v_ring,
                       int B, int T, int W, int Hkv, int D, int dtype, void* stream);

/*
 * Decode on a windowed layer against its ring: the new query of sequence b
 * (position seqlens[b] - 1; seqlens counts the new token, whose K/V row is
 * already appended) attends to the min(seqlens[b], W) positions the ring
 * holds, which are exactly the window of W keys ending at the query.
 *   seqlens [B] int32 (device): the whole history of sequence b, any value
 *     >= 1 (it may exceed W; the kernels bound the key count by W themselves).
 * q, out, lse, sinks, scale and dtype as for gqa_attn_decode; the workspace
 * must hold gqa_attn_decode_ring_workspace_size(...) bytes (0 for W <= 1024).
 */
size_t gqa_attn_decode_ring_workspace_size(int B, int W, int Hq, int Hkv, int D, int dtype);

int gqa_attn_decode_ring(const void* q, const void* k_ring, const void* v_ring,
                         const int32_t* seqlens, const float* sinks,
                         void* out, float* lse,
                         int B, int W, int Hq, int Hkv, int D,
                         float scale, int dtype,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Chunked prefill of a sliding-window layer over its ring: a chunk of new
 * tokens attends over the positions its ring still holds plus its own rows,
 * and is appended to the ring afterwards.  «GPT-OSS vs Qwen3», section
 * "Utilisation de Sliding Window Attention": the layer sees the last W tokens
 * only.  A query at position p of a chunk starting at position L0 sees
 * positions p - W + 1 .. p, none older than L0 - W + 1: before the chunk is
 * written the ring holds all of those below L0, and the chunk the rest, so a
 * chunk of any length (shorter than, equal to or longer than W) needs nothing
 * the ring has lost.  Appending first would overwrite slots the chunk's first
 * queries still read.
 *   q [Tq, Hq, D], k_new, v_new [Tq, Hkv, D]: the chunks' rows (rotated, as
 *     every attention input); sequence b owns rows cu_seqlens_q[b] ..
 *     cu_seqlens_q[b+1]-1 (cu_seqlens_q [B+1] int32, device, non-decreasing,
 *     cu_seqlens_q[B] == Tq), its newest q_len positions: row t at position
 *     seqlens[b] - q_len + t.  A chunk of one row is a decode step; q_len 0
 *     leaves the sequence alone.
 *   seqlens [B] int32 (device): positions of sequence b including its chunk
 *     (clamped to [q_len, 2^30]: GQA_DBG_SEQLENS_K / GQA_DBG_Q_LEN).
 *   k_ring, v_ring [B, W, Hkv, D]: before the call, the positions before the
 *     chunk (the last min(L0, W) of 0 .. L0-1, position p in slot p % W, as
 *     gqa_kv_ring_append leaves them); slots never written are not read.
 *   append: nonzero: after the attention the chunk's rows are written to the
 *     rings (gqa_kv_ring_append, on the same stream, so after every read);
 *     0: the rings are left unchanged.
 *   sinks [Hq] fp32 or NULL, out [Tq, Hq, D], lse [Hq, Tq] fp32 (optional),
 *     scale: as gqa_attn_varlen_paged.  The window is W; there are no sink
 *     tokens (a ring does not hold them).
 *   max_q_len (host): upper bound of any q_len (sizes the grid; rows of a
 *     longer chunk past it are not computed).
 * bf16 or fp32.  No workspace.
 */
int gqa_attn_prefill_ring(const void* q, const void* k_new, const void* v_new,
                          const int32_t* cu_seqlens_q, const int32_t* seqlens,
                          void* k_ring, void* v_ring, int append,
                          const float* sinks, void* out, float* lse,
                          int B, int Tq, int max_q_len, int W, int Hq, int Hkv, int D,
                          float scale, int dtype, void* stream);

/*
 * Rotary position encoding of new tokens fused with their KV-cache append.
 *
 * «GPT-OSS-20B : Architecture MoE & Résumé du Model Card», §3.4 "Encodage de
 * Position (RoPE)": a token at position m is turned with the frequencies
 * θ_i = 10000^(-2i/d); «GPT-OSS vs Qwen3», "Adoption de RoPE": queries and keys
 * are rotated by a position-dependent angle.  Pair i of every head, (a, b),
 * becomes (a cos - b sin, a sin + b cos) at angle m * inv_freq[i], with cos and
 * sin both multiplied by mscale (1 for plain RoPE).
 *   pairing: GQA_ROPE_INTERLEAVED pairs coordinates (2i, 2i+1);
 *            GQA_ROPE_HALVES pairs (i, i + D/2).
 *   inv_freq [D/2] fp32 (device), or NULL for the default table
 *     θ_i = 10000^(-2i/D) (formed in fp64 when the library is built and
 *     rounded once to fp32: the correctly rounded values); a context-extension scheme (e.g. YaRN, whose parameters the
 *     pages do not give in full) passes its own table.
 * Rows and positions as for gqa_kv_ring_append: q [T, Hq, D], k, v [T, Hkv, D];
 * without cu_seqlens_q, T == B and row b is at position seqlens[b] - 1; with
 * cu_seqlens_q [B+1], sequence b's rows are its newest q_len positions.
 * Outputs: q_out [T, Hq, D] (may be q itself) holds the rotated queries (q and
 * q_out both NULL: keys only, for an attention call that rotates its queries
 * itself, gqa_attn_prefill_rope); the
 * rotated key row and the value row of position p are written to the cache:
 *   GQA_CACHE_CONTIGUOUS: k_cache, v_cache [B, cache_len, Hkv, D], row p
 *     (positions >= cache_len are not stored);
 *   GQA_CACHE_PAGED: [num_blocks, block_size, Hkv, D], slot p % block_size of
 *     block block_table[b * max_blocks + p / block_size] (power-of-two
 *     block_size <= 1024; ids clamped to [0, num_blocks));
 *   GQA_CACHE_RING: [B, cache_len, Hkv, D] rings, slot p % cache_len, only
 *     the last cache_len positions.
 * Angles are formed in fp64 (exact for integer positions and fp32
 * frequencies); the rotation is fp32 and rounds to the dtype once.
 */
enum { GQA_ROPE_INTERLEAVED = 0, GQA_ROPE_HALVES = 1 };
enum { GQA_CACHE_CONTIGUOUS = 0, GQA_CACHE_PAGED = 1, GQA_CACHE_RING = 2 };

int gqa_rope_append(const void* q, const void* k, const void* v, void* q_out,
                    const int32_t* cu_seqlens_q, const int32_t* seqlens,
                    const float* inv_freq, float mscale, int pairing,
                    void* k_cache, void* v_cache, int cache_kind, int cache_len,
                    const int32_t* block_table, int max_blocks, int block_size, int num_blocks,
                    int B, int T, int Hq, int Hkv, int D, int dtype, void* stream);

/*
 * One decode step of a layer in one launch: the rotary encoding of each
 * sequence's new token (query and key, as gqa_rope_append), the append of the
 * rotated key and the value to the cache, and the attention of the rotated
 * query over the cache (as gqa_attn_decode, or gqa_attn_decode_ring for a ring
 * cache), which sees the new key and value at the new position.  It computes
 * what gqa_rope_append followed by gqa_attn_decode computes, in one launch.
 *   q [B, Hq, D], k_new, v_new [B, Hkv, D] bf16: the new rows, not rotated;
 *   seqlens [B] int32 (device): positions of sequence b including the new
 *     token, which sits at position seqlens[b] - 1;
 *   inv_freq, mscale, pairing: as gqa_rope_append (inv_freq NULL: the default
 *     table θ_i = 10000^(-2i/D));
 *   q_out [B, Hq, D] bf16 or NULL: the rotated queries, if wanted;
 *   cache_kind, cache_len, block_table, max_blocks, block_size, num_blocks:
 *     as gqa_rope_append (contiguous, paged or ring cache);
 *   sinks, out [B, Hq, D], lse [B, Hq] (optional), window, sink_tokens,
 *     scale: as gqa_attn_decode.  With a ring cache the ring is the window
 *     (window 0 or cache_len) and sink_tokens must be 0.
 * bf16 only (fp32: GQA_ERR_UNSUPPORTED), at most 16 query heads per KV head,
 * and at most 2048 keys per query (window + sink_tokens on windowed layers,
 * the cache capacity on dense ones): one workgroup streams a (sequence, KV
 * head)'s keys, which suits windowed layers and short caches; longer key
 * ranges return GQA_ERR_UNSUPPORTED (use gqa_rope_append, then
 * gqa_attn_decode).  Metadata out of range is clamped as for every call.
 */
int gqa_attn_decode_step(const void* q, const void* k_new, const void* v_new, void* q_out,
                         const int32_t* seqlens, const float* inv_freq, float mscale, int pairing,
                         void* k_cache, void* v_cache, int cache_kind, int cache_len,
                         const int32_t* block_table, int max_blocks, int block_size, int num_blocks,
                         const float* sinks, void* out, float* lse,
                         int B, int Hq, int Hkv, int D, int window, int sink_tokens, float scale,
                         int dtype, void* stream);

/*
 * Backward of the prefill: the gradients of a loss L with respect to q, k, v
 * and the sink logits, given dL/dout.  Training the model calls for them
 * («GPT-OSS-20B : Architecture MoE & Résumé du Model Card», §5: pre-training
 * by next-token prediction); the pages print no backward pass, so what is
 * computed is the derivative of the forward definition above, with
 * P_j = e^{x_j - lse} and D = <dL/dout, out> per row and head:
 *   dx_j  = P_j (<dL/dout, v_j> - D)                    (gradient of logit x_j)
 *   dq    = scale sum_j dx_j k_j[g]
 *   dk_j[g] = scale sum over rows and query heads of g of dx_j q
 *   dv_j[g] = sum over rows and query heads of g of P_j dL/dout
 *   dsinks[h] = -sum over rows of e^{s_h - lse} D       (the sink has no value)
 * Same layouts and arguments as gqa_attn_prefill (window, sink_tokens, scale):
 *   q, out, dout, dq [B, S, Hq, D]     k, v, dk, dv [B, S, Hkv, D]
 *   lse [B, Hq, S] fp32: the forward's, as gqa_attn_prefill wrote it (input)
 *   sinks [Hq] fp32 or NULL (no sink)
 *   dsinks [Hq] fp32 output, or NULL (not computed); zeros when sinks is NULL
 * dq, dk, dv are written whole (no accumulation into them) in the dtype of
 * the inputs.  workspace: at least gqa_attn_prefill_backward_workspace_size
 * bytes of device memory, owned by the caller, clobbered by the call (it
 * holds <dL/dout, out> per row and head, and, when there are few key blocks
 * to spread over the chip, fp32 partial sums of dk and dv: 64 MB for
 * B1 S4096 with 8 KV heads).  The
 * result is deterministic (no atomics).  B == 0 or S == 0 writes only dsinks
 * (zeros).  Errors as for every entry point; GQA_ERR_WORKSPACE when the
 * workspace is missing or small.
 */
size_t gqa_attn_prefill_backward_workspace_size(int B, int S, int Hq, int Hkv, int D, int dtype);

int gqa_attn_prefill_backward(const void* q, const void* k, const void* v, const float* sinks,
                              const void* out, const float* lse, const void* dout,
                              void* dq, void* dk, void* dv, float* dsinks,
                              int B, int S, int Hq, int Hkv, int D,
                              int window, int sink_tokens, float scale, int dtype,
                              void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_ATTN_H */
