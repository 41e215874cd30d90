// C ABI of the attention library: argument validation, launch planning (grid
// sizes, split-K count, workspace layout) and dispatch to the gfx950 kernels.
// Every entry point validates first and launches nothing on error; no C++
// exception leaves this file.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <mutex>

#include "gqa_attn.h"
#include "kernels.h"

using namespace gqa;

namespace {

thread_local char g_err[512];

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return GQA_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(GQA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// number of compute units of the current device (cached per device; 256 when
// no device can be queried, e.g. during host-only argument checks)
int num_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    cache[dev] = n;
  }
  return cache[dev];
}

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  if (!s || !*s) return dflt;
  return atoi(s);
}

int check_common(int Hq, int Hkv, int D, int window, int sink_tokens, float scale, int dtype) {
  if (dtype != GQA_BF16 && dtype != GQA_FP32) return fail(GQA_ERR_UNSUPPORTED, "dtype %d is not GQA_BF16 or GQA_FP32", dtype);
  if (Hq <= 0 || Hkv <= 0) return fail(GQA_ERR_INVALID_ARG, "head counts must be positive (Hq=%d, Hkv=%d)", Hq, Hkv);
  if (Hq % Hkv != 0) return fail(GQA_ERR_UNSUPPORTED, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (D != kHeadDim) return fail(GQA_ERR_UNSUPPORTED, "head_dim %d is not supported (only 64)", D);
  if (window < 0) return fail(GQA_ERR_INVALID_ARG, "window %d is negative (0 = dense)", window);
  if (sink_tokens < 0) return fail(GQA_ERR_INVALID_ARG, "sink_tokens %d is negative", sink_tokens);
  if (std::isnan(scale) || scale < 0.f) return fail(GQA_ERR_INVALID_ARG, "scale must be >= 0 (0 = 1/sqrt(D))");
  return GQA_OK;
}

float scale_log2_of(float scale, int D) {
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)D);
  return sc * kLog2e;
}

struct SplitPlan {
  int n_splits;
  int split_len;
  int solo;  // one unit per wave (short key ranges, many units)
  int rows;  // whole-row form: a workgroup per (sequence, split), all 8 KV heads
};

// Split of the decode key range: enough workgroups to keep about 16 per CU in
// the queue (the streaming loads then overlap the merge of finished ones),
// while every split keeps at least 1024 keys (4 tiles of 64 per wave).
//
// A contiguous cache with 8 KV heads of at most 8 query heads each (rows_ok:
// the one-query-per-sequence decode call, ring caches included) takes the
// whole-row form when its (sequence, split) workgroups fill the chip: splits
// of at least 512 keys (one split for shorter ranges), about one workgroup per
// CU in all (two measured 1.5-3 % slower: B64 x 8192 and B8 x 131072).
SplitPlan plan_splits(int B, int Hkv, int G, int Lmax, int window, int sink_tokens, bool rows_ok) {
  // keys read per sequence at most: the window plus the sink tokens below it
  const long wk = window > 0 ? (long)window + sink_tokens : (long)Lmax;
  const int eff = (int)(wk < Lmax ? wk : Lmax);
  const int n_hc = (G + 15) / 16;
  const long units = (long)B * Hkv * n_hc;
  SplitPlan p{1, 64, 0, 0};
  if (eff <= 0 || units <= 0) return p;
  const int rows_env = env_int("GQA_DECODE_ROWS", 1);  // 0: never, 1: when it fills the chip, 2: whenever eligible
  if (rows_ok && Hkv == 8 && G <= 8 && rows_env != 0) {
    const long per_cu = env_int("GQA_DECODE_ROWS_WGS", 1);
    long want = (per_cu * num_cus() + B - 1) / B;
    if (want > eff / 512) want = eff / 512;
    if (want > 64) want = 64;
    if (want < 1) want = 1;
    const int forced = env_int("GQA_DECODE_SPLITS", 0);
    if (forced > 0) want = forced > 256 ? 256 : forced;
    if (rows_env == 2 || (long)B * want >= num_cus()) {
      int len = (int)((eff + want - 1) / want);
      len = (len + 63) & ~63;
      p.rows = 1;
      p.split_len = len;
      p.n_splits = (eff + len - 1) / len;
      return p;
    }
  }
  // Short ranges over many units: one wave per unit fills the chip by itself
  // and skips the cross-wave merge (at most 8 tiles of 64 keys per wave).
  if (eff <= 512 && units >= 8L * num_cus() && env_int("GQA_DECODE_SOLO", 1) != 0) {
    p.solo = 1;
    p.split_len = (eff + 63) & ~63;
    return p;
  }
  const long target = 16L * num_cus();
  long want = (target + units - 1) / units;
  const long max_by_len = eff / 1024;
  if (want > max_by_len) want = max_by_len;
  if (want < 1) want = 1;
  if (want > 64) want = 64;
  const int forced = env_int("GQA_DECODE_SPLITS", 0);
  if (forced > 0) want = forced > 256 ? 256 : forced;
  int len = (int)((eff + want - 1) / want);
  len = (len + 63) & ~63;
  p.split_len = len;
  p.n_splits = (eff + len - 1) / len;
  return p;
}

size_t decode_ws_bytes(const SplitPlan& p, int B, int Hq) {
  if (p.n_splits <= 1) return 0;
  return (size_t)B * Hq * p.n_splits * (2 + kHeadDim) * sizeof(float);
}

}  // namespace

extern "C" {

int gqa_attn_version(void) { return 600; }

int gqa_attn_debug_flags(unsigned int* flags, int reset) {
  if (!flags) return fail(GQA_ERR_INVALID_ARG, "flags is NULL");
  *flags = 0;
#ifndef GQA_DEBUG
  (void)reset;
  return fail(GQA_ERR_UNSUPPORTED, "release build: device-side metadata is clamped but not recorded");
#else
  hipError_t (*const fns[])(unsigned int*, bool) = {gqa::debug_flags_prefill, gqa::debug_flags_decode,
                                                    gqa::debug_flags_fp32,    gqa::debug_flags_ring,
                                                    gqa::debug_flags_rope,    gqa::debug_flags_backward,
                                                    gqa::debug_flags_step};
  for (auto fn : fns) {
    unsigned int v = 0;
    const hipError_t e = fn(&v, reset != 0);
    if (e != hipSuccess) return hip_fail(e, "debug flag copy");
    *flags |= v;
  }
  return ok();
#endif
}

const char* gqa_attn_status_string(int status) {
  switch (status) {
    case GQA_OK: return "GQA_OK";
    case GQA_ERR_INVALID_ARG: return "GQA_ERR_INVALID_ARG";
    case GQA_ERR_UNSUPPORTED: return "GQA_ERR_UNSUPPORTED";
    case GQA_ERR_WORKSPACE: return "GQA_ERR_WORKSPACE";
    case GQA_ERR_HIP: return "GQA_ERR_HIP";
    default: return "GQA_ERR_UNKNOWN";
  }
}

const char* gqa_attn_last_error(void) { return g_err; }

}  // extern "C"

namespace {

// Whole-sequence prefill; rope != 0: the queries arrive unrotated and the
// kernel rotates them (1: pairs (2i, 2i+1), 2: pairs (i, i + D/2)).
int prefill_call(const void* q, const void* k, const void* v, const float* sinks, void* out, float* lse, int B,
                 int S, int Hq, int Hkv, int D, int window, int sink_tokens, float scale, int dtype, int rope,
                 const float* inv_freq, float mscale, void* stream) {
  int rc = check_common(Hq, Hkv, D, window, sink_tokens, scale, dtype);
  if (rc) return rc;
  if (rope && dtype != GQA_BF16) return fail(GQA_ERR_UNSUPPORTED, "the prefill with rotary encoding is bf16 only");
  if (B < 0 || S < 0) return fail(GQA_ERR_INVALID_ARG, "negative size (B=%d, S=%d)", B, S);
  if (B == 0 || S == 0) return ok();
  if (!q || !k || !v || !out) return fail(GQA_ERR_INVALID_ARG, "q, k, v and out must be non-NULL");
  const int G = Hq / Hkv;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);

  SeqArgs seq{};
  seq.q_len_fixed = S;
  seq.kv_len_fixed = S;
  seq.lmax = S;
  const float sl2 = scale_log2_of(scale, D);

  if (dtype == GQA_FP32) {
    if ((long long)B * S * Hq > 0x7fffffffLL) return fail(GQA_ERR_UNSUPPORTED, "problem too large for the fp32 path");
    Fp32Args a{};
    a.q = (const float*)q; a.k = (const float*)k; a.v = (const float*)v; a.sinks = sinks;
    a.out = (float*)out; a.lse = lse; a.seq = seq;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = G; a.window = window; a.sink_tokens = sink_tokens; a.scale_log2 = sl2;
    a.max_q_len = S; a.varlen_q = 0;
    a.lse_sb = (int64_t)Hq * S; a.lse_sh = S; a.lse_row0 = 0;
    hipError_t e = launch_fp32(a, KV_BATCHED, st);
    return e == hipSuccess ? ok() : hip_fail(e, "prefill fp32 launch");
  }

  PrefillArgs a{};
  a.q = (const __bf16*)q; a.k = (const __bf16*)k; a.v = (const __bf16*)v; a.sinks = sinks;
  a.out = (__bf16*)out; a.lse = lse; a.seq = seq;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = G; a.window = window; a.sink_tokens = sink_tokens; a.scale_log2 = sl2;
  const long ntiles = (long)((S + 31) / 32) * G;
  a.wg_per_seq = (int)((ntiles + prefill_ntiles_per_wg() - 1) / prefill_ntiles_per_wg());
  a.skip_single = 0;
  a.lse_sb = (int64_t)Hq * S; a.lse_sh = S; a.lse_row0 = 0;
  if ((long long)B * Hkv * a.wg_per_seq > 0x7fffffffLL) return fail(GQA_ERR_UNSUPPORTED, "grid too large");
  a.rope = rope;
  a.inv_freq = inv_freq;
  a.rope_mscale = mscale;
  // Windowed layers: a workgroup runs two tile groups over the same key tiles
  // when together they need at most 3 tiles of 64 keys (positions 2r*32 ..
  // 2r*32+63 for G = 8, one 32-position block for G a multiple of 16), and
  // when that turns two rounds of workgroups (two resident per CU) into one;
  // with more rounds the finer jobs balance better (measured: S4096 -7 %,
  // S32768 +5 % with two steps).
  // (GQA_PREFILL_TWO_STEP: 0 never, 1 as above, 2 on every windowed layer
  // without sink tokens: where the tiles do not fit, the second step streams
  // them again)
  const int two_env = env_int("GQA_PREFILL_TWO_STEP", 1);
  a.two_step = window > 0 && sink_tokens == 0 &&
               (two_env == 2 || (two_env == 1 && window <= 128 && (G == 8 || G % 16 == 0) &&
                                 (long long)B * Hkv * a.wg_per_seq <= 4LL * num_cus()));
  hipError_t e = launch_prefill_bf16(a, KV_BATCHED, false, st);
  return e == hipSuccess ? ok() : hip_fail(e, "prefill bf16 launch");
}

}  // namespace

extern "C" {

int gqa_attn_prefill(const void* q, const void* k, const void* v, const float* sinks, void* out, float* lse,
                     int B, int S, int Hq, int Hkv, int D, int window, int sink_tokens, float scale, int dtype,
                     void* stream) {
  return prefill_call(q, k, v, sinks, out, lse, B, S, Hq, Hkv, D, window, sink_tokens, scale, dtype, 0, nullptr,
                      1.f, stream);
}

int gqa_attn_prefill_rope(const void* q, const void* k, const void* v, const float* sinks, void* out, float* lse,
                          int B, int S, int Hq, int Hkv, int D, int window, int sink_tokens, float scale,
                          const float* inv_freq, float mscale, int pairing, int dtype, void* stream) {
  if (pairing != 0 && pairing != 1) return fail(GQA_ERR_INVALID_ARG, "pairing %d is not 0 or 1", pairing);
  if (std::isnan(mscale) || std::isinf(mscale)) return fail(GQA_ERR_INVALID_ARG, "mscale must be finite");
  return prefill_call(q, k, v, sinks, out, lse, B, S, Hq, Hkv, D, window, sink_tokens, scale, dtype, pairing + 1,
                      inv_freq, mscale, stream);
}

size_t gqa_attn_decode_workspace_size(int B, int Lmax, int Hq, int Hkv, int D, int window, int sink_tokens,
                                      int dtype) {
  if (dtype != GQA_BF16 || B <= 0 || Lmax <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D != kHeadDim || window < 0 ||
      sink_tokens < 0)
    return 0;
  const SplitPlan p = plan_splits(B, Hkv, Hq / Hkv, Lmax, window, sink_tokens, true);
  return decode_ws_bytes(p, B, Hq);
}

}  // extern "C"

namespace {

// Decode over a batched cache of Lmax rows per sequence.  ring != 0: the cache
// is a ring of Lmax slots and seqlens[b] counts the whole history; the kernels
// take min(seqlens[b], Lmax) positions, every one of them visible.
int decode_call(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens,
                const float* sinks, void* out, float* lse, int B, int Lmax, int Hq, int Hkv, int D,
                int window, int sink_tokens, float scale, int dtype, void* workspace, size_t workspace_bytes,
                void* stream, int ring) {
  int rc = check_common(Hq, Hkv, D, window, sink_tokens, scale, dtype);
  if (rc) return rc;
  if (B < 0 || Lmax < 0) return fail(GQA_ERR_INVALID_ARG, "negative size (B=%d, Lmax=%d)", B, Lmax);
  if (B == 0) return ok();
  if (Lmax == 0) return fail(GQA_ERR_INVALID_ARG, "Lmax must be >= 1 (the cache holds the new token)");
  if (!q || !k_cache || !v_cache || !out || !seqlens)
    return fail(GQA_ERR_INVALID_ARG, "q, k_cache, v_cache, seqlens and out must be non-NULL");
  const int G = Hq / Hkv;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  SeqArgs seq{};
  seq.seqlens_k = seqlens;
  seq.q_len_fixed = 1;
  seq.kv_len_fixed = Lmax;
  seq.lmax = Lmax;
  seq.ring = ring;
  const float sl2 = scale_log2_of(scale, D);

  if (dtype == GQA_FP32) {
    Fp32Args a{};
    a.q = (const float*)q; a.k = (const float*)k_cache; a.v = (const float*)v_cache; a.sinks = sinks;
    a.out = (float*)out; a.lse = lse; a.seq = seq;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = G; a.window = window; a.sink_tokens = sink_tokens; a.scale_log2 = sl2;
    a.max_q_len = 1; a.varlen_q = 0;
    a.lse_sb = Hq; a.lse_sh = 1; a.lse_row0 = 0;
    hipError_t e = launch_fp32(a, KV_BATCHED, st);
    return e == hipSuccess ? ok() : hip_fail(e, "decode fp32 launch");
  }

  const SplitPlan p = plan_splits(B, Hkv, G, Lmax, window, sink_tokens, true);
  const size_t need = decode_ws_bytes(p, B, Hq);
  if (need && (!workspace || workspace_bytes < need))
    return fail(GQA_ERR_WORKSPACE, "decode needs a workspace of %zu bytes (got %zu)", need, workspace ? workspace_bytes : (size_t)0);
  DecodeArgs a{};
  a.q = (const __bf16*)q; a.k = (const __bf16*)k_cache; a.v = (const __bf16*)v_cache; a.sinks = sinks;
  a.out = (__bf16*)out; a.lse = lse; a.seq = seq;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = G; a.n_hc = (G + 15) / 16;
  a.window = window; a.sink_tokens = sink_tokens; a.scale_log2 = sl2;
  a.n_splits = p.n_splits; a.split_len = p.split_len;
  a.ws_ml = (float*)workspace;
  a.ws_acc = need ? (float*)workspace + (size_t)B * Hq * p.n_splits * 2 : nullptr;
  a.varlen_q = 0;
  a.lse_sb = Hq; a.lse_sh = 1; a.lse_row0 = 0;
  a.solo = p.solo;
  a.rows = p.rows;
  if ((long long)B * Hkv * a.n_hc * a.n_splits > 0x7fffffffLL) return fail(GQA_ERR_UNSUPPORTED, "grid too large");
  hipError_t e = launch_decode_bf16(a, KV_BATCHED, st);
  return e == hipSuccess ? ok() : hip_fail(e, "decode bf16 launch");
}

}  // namespace

extern "C" {

int gqa_attn_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens,
                    const float* sinks, void* out, float* lse, int B, int Lmax, int Hq, int Hkv, int D,
                    int window, int sink_tokens, float scale, int dtype, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return decode_call(q, k_cache, v_cache, seqlens, sinks, out, lse, B, Lmax, Hq, Hkv, D, window, sink_tokens,
                     scale, dtype, workspace, workspace_bytes, stream, 0);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free decode: the split partials live in this fixed device array
// (one copy per GPU the library runs on, held until the process ends) instead
// of a caller's workspace.  Host code never uses the array's name as an
// address: the per-device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[GQA_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

// Device address of this GPU's scratch array, looked up once per device (with
// that device current, on the first allocation-free call made on it).
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(GQA_ERR_UNSUPPORTED, "device %d is beyond the 64 the library tracks", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(GQA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GQA_OK;
}

}  // namespace

extern "C" {

int gqa_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens,
                            const float* sinks, void* out, float* lse, int B, int Lmax, int Hq, int Hkv, int D,
                            int window, int sink_tokens, float scale, int dtype, void* stream) {
  int rc = check_common(Hq, Hkv, D, window, sink_tokens, scale, dtype);
  if (rc) return rc;
  if (B < 0 || Lmax < 0) return fail(GQA_ERR_INVALID_ARG, "negative size (B=%d, Lmax=%d)", B, Lmax);
  // the partials this call needs, checked before the device is touched
  size_t need = 0;
  if (dtype == GQA_BF16 && B > 0 && Lmax > 0) {
    const SplitPlan p = plan_splits(B, Hkv, Hq / Hkv, Lmax, window, sink_tokens, true);
    need = decode_ws_bytes(p, B, Hq);
  }
  if (need > (size_t)GQA_NOALLOC_SCRATCH_BYTES)
    return fail(GQA_ERR_WORKSPACE,
                "this decode needs %zu bytes of split partials; the allocation-free decode holds at most %zu "
                "(use gqa_attn_decode with a workspace)",
                need, (size_t)GQA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc) return rc;
  return decode_call(q, k_cache, v_cache, seqlens, sinks, out, lse, B, Lmax, Hq, Hkv, D, window, sink_tokens, scale,
                     dtype, ws, (size_t)GQA_NOALLOC_SCRATCH_BYTES, stream, 0);
}

size_t gqa_attn_varlen_workspace_size(int B, int max_q_len, int max_kv_len, int Hq, int Hkv, int D, int window,
                                      int sink_tokens, int dtype) {
  if (dtype != GQA_BF16 || B <= 0 || max_q_len <= 0 || max_kv_len <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv ||
      D != kHeadDim || window < 0 || sink_tokens < 0)
    return 0;
  const SplitPlan p = plan_splits(B, Hkv, Hq / Hkv, max_kv_len, window, sink_tokens, false);
  return decode_ws_bytes(p, B, Hq);
}

int gqa_attn_varlen_paged(const void* q, const void* k_cache, const void* v_cache, const int32_t* cu_seqlens_q,
                          const int32_t* seqlens_k, const int32_t* block_table, int max_blocks, int block_size,
                          const int32_t* cu_seqlens_k, int num_blocks, const float* sinks, void* out, float* lse,
                          int B, int Tq, int max_q_len, int max_kv_len, int Hq, int Hkv, int D, int window,
                          int sink_tokens, float scale, int dtype, void* workspace, size_t workspace_bytes,
                          void* stream) {
  int rc = check_common(Hq, Hkv, D, window, sink_tokens, scale, dtype);
  if (rc) return rc;
  if (B < 0 || Tq < 0 || max_q_len < 0 || max_kv_len < 0)
    return fail(GQA_ERR_INVALID_ARG, "negative size (B=%d, Tq=%d, max_q_len=%d, max_kv_len=%d)", B, Tq, max_q_len, max_kv_len);
  if (B == 0 || Tq == 0 || max_q_len == 0) return ok();
  if (!q || !k_cache || !v_cache || !out || !cu_seqlens_q || !seqlens_k)
    return fail(GQA_ERR_INVALID_ARG, "q, k_cache, v_cache, cu_seqlens_q, seqlens_k and out must be non-NULL");
  if (num_blocks <= 0) return fail(GQA_ERR_INVALID_ARG, "num_blocks must be >= 1");
  int mode, log2b = 0;
  if (block_table) {
    if (block_size < 1 || block_size > 1024 || (block_size & (block_size - 1)))
      return fail(GQA_ERR_UNSUPPORTED, "block_size %d is not a power of two in [1, 1024]", block_size);
    if (max_blocks <= 0) return fail(GQA_ERR_INVALID_ARG, "max_blocks must be >= 1");
    while ((1 << log2b) < block_size) ++log2b;
    if ((long long)max_blocks * block_size < max_kv_len)
      return fail(GQA_ERR_INVALID_ARG, "max_kv_len %d exceeds the block table capacity %lld", max_kv_len,
                  (long long)max_blocks * block_size);
    mode = KV_PAGED;
  } else {
    if (!cu_seqlens_k) return fail(GQA_ERR_INVALID_ARG, "cu_seqlens_k is required when block_table is NULL");
    mode = KV_PACKED;
  }
  if (max_q_len > max_kv_len) return fail(GQA_ERR_INVALID_ARG, "max_q_len %d exceeds max_kv_len %d", max_q_len, max_kv_len);
  const int G = Hq / Hkv;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  SeqArgs seq{};
  seq.cu_seqlens_q = cu_seqlens_q;
  seq.seqlens_k = seqlens_k;
  seq.block_table = block_table;
  seq.cu_seqlens_k = cu_seqlens_k;
  seq.max_blocks = max_blocks;
  seq.log2_block = log2b;
  seq.num_blocks = num_blocks;
  seq.lmax = max_kv_len;
  seq.q_rows = Tq;
  const float sl2 = scale_log2_of(scale, D);

  if (dtype == GQA_FP32) {
    if ((long long)B * max_q_len * Hq > 0x7fffffffLL) return fail(GQA_ERR_UNSUPPORTED, "problem too large for the fp32 path");
    Fp32Args a{};
    a.q = (const float*)q; a.k = (const float*)k_cache; a.v = (const float*)v_cache; a.sinks = sinks;
    a.out = (float*)out; a.lse = lse; a.seq = seq;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = G; a.window = window; a.sink_tokens = sink_tokens; a.scale_log2 = sl2;
    a.max_q_len = max_q_len; a.varlen_q = 1;
    a.lse_sb = 0; a.lse_sh = Tq; a.lse_row0 = 1;
    hipError_t e = launch_fp32(a, mode, st);
    return e == hipSuccess ? ok() : hip_fail(e, "varlen fp32 launch");
  }

  const SplitPlan p = plan_splits(B, Hkv, G, max_kv_len, window, sink_tokens, false);
  const size_t need = decode_ws_bytes(p, B, Hq);
  if (need && (!workspace || workspace_bytes < need))
    return fail(GQA_ERR_WORKSPACE, "varlen needs a workspace of %zu bytes (got %zu)", need, workspace ? workspace_bytes : (size_t)0);

  if (max_q_len > 1) {
    PrefillArgs a{};
    a.q = (const __bf16*)q; a.k = (const __bf16*)k_cache; a.v = (const __bf16*)v_cache; a.sinks = sinks;
    a.out = (__bf16*)out; a.lse = lse; a.seq = seq;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = G; a.window = window; a.sink_tokens = sink_tokens; a.scale_log2 = sl2;
    const long ntiles = (long)((max_q_len + 31) / 32) * G;
    a.wg_per_seq = (int)((ntiles + prefill_ntiles_per_wg() - 1) / prefill_ntiles_per_wg());
    a.skip_single = 1;
    a.lse_sb = 0; a.lse_sh = Tq; a.lse_row0 = 1;
    a.sort_seq = B <= 256 && env_int("GQA_VARLEN_SORT", 1) != 0;
    if ((long long)B * Hkv * a.wg_per_seq > 0x7fffffffLL) return fail(GQA_ERR_UNSUPPORTED, "grid too large");
    hipError_t e = launch_prefill_bf16(a, mode, true, st);
    if (e != hipSuccess) return hip_fail(e, "varlen prefill launch");
  }
  DecodeArgs a{};
  a.q = (const __bf16*)q; a.k = (const __bf16*)k_cache; a.v = (const __bf16*)v_cache; a.sinks = sinks;
  a.out = (__bf16*)out; a.lse = lse; a.seq = seq;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = G; a.n_hc = (G + 15) / 16;
  a.window = window; a.sink_tokens = sink_tokens; a.scale_log2 = sl2;
  a.n_splits = p.n_splits; a.split_len = p.split_len;
  a.ws_ml = (float*)workspace;
  a.ws_acc = need ? (float*)workspace + (size_t)B * Hq * p.n_splits * 2 : nullptr;
  a.varlen_q = 1;
  a.lse_sb = 0; a.lse_sh = Tq; a.lse_row0 = 1;
  a.solo = p.solo;
  if ((long long)B * Hkv * a.n_hc * a.n_splits > 0x7fffffffLL) return fail(GQA_ERR_UNSUPPORTED, "grid too large");
  hipError_t e = launch_decode_bf16(a, mode, st);
  return e == hipSuccess ? ok() : hip_fail(e, "varlen decode launch");
}

int gqa_kv_ring_append(const void* k_new, const void* v_new, const int32_t* cu_seqlens_q, const int32_t* seqlens,
                       void* k_ring, void* v_ring, int B, int T, int W, int Hkv, int D, int dtype, void* stream) {
  if (dtype != GQA_BF16 && dtype != GQA_FP32) return fail(GQA_ERR_UNSUPPORTED, "dtype %d is not GQA_BF16 or GQA_FP32", dtype);
  if (D != kHeadDim) return fail(GQA_ERR_UNSUPPORTED, "head_dim %d is not supported (only 64)", D);
  if (B < 0 || T < 0 || Hkv <= 0) return fail(GQA_ERR_INVALID_ARG, "bad size (B=%d, T=%d, Hkv=%d)", B, T, Hkv);
  if (W <= 0) return fail(GQA_ERR_INVALID_ARG, "ring size W=%d must be >= 1", W);
  if (!cu_seqlens_q && T != B)
    return fail(GQA_ERR_INVALID_ARG, "without cu_seqlens_q there is one new row per sequence (T=%d, B=%d)", T, B);
  if (B == 0 || T == 0) return ok();
  if (!k_new || !v_new || !k_ring || !v_ring || !seqlens)
    return fail(GQA_ERR_INVALID_ARG, "k_new, v_new, k_ring, v_ring and seqlens must be non-NULL");
  RingAppendArgs a{};
  a.k_new = (const char*)k_new; a.v_new = (const char*)v_new;
  a.k_ring = (char*)k_ring; a.v_ring = (char*)v_ring;
  a.cu_seqlens_q = cu_seqlens_q; a.seqlens = seqlens;
  a.T = T; a.B = B; a.W = W;
  a.row_bytes = Hkv * D * (dtype == GQA_BF16 ? 2 : 4);
  hipError_t e = launch_ring_append(a, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "ring append launch");
}

int gqa_attn_prefill_ring(const void* q, const void* k_new, const void* v_new, const int32_t* cu_seqlens_q,
                          const int32_t* seqlens, void* k_ring, void* v_ring, int append, const float* sinks,
                          void* out, float* lse, int B, int Tq, int max_q_len, int W, int Hq, int Hkv, int D,
                          float scale, int dtype, void* stream) {
  int rc = check_common(Hq, Hkv, D, W, 0, scale, dtype);
  if (rc) return rc;
  if (W <= 0) return fail(GQA_ERR_INVALID_ARG, "ring size W=%d must be >= 1", W);
  if (B < 0 || Tq < 0 || max_q_len < 0)
    return fail(GQA_ERR_INVALID_ARG, "negative size (B=%d, Tq=%d, max_q_len=%d)", B, Tq, max_q_len);
  if (B == 0 || Tq == 0 || max_q_len == 0) return ok();
  if (!q || !k_new || !v_new || !k_ring || !v_ring || !out || !cu_seqlens_q || !seqlens)
    return fail(GQA_ERR_INVALID_ARG, "q, k_new, v_new, k_ring, v_ring, cu_seqlens_q, seqlens and out must be non-NULL");
  const int G = Hq / Hkv;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  SeqArgs seq{};
  seq.cu_seqlens_q = cu_seqlens_q;
  seq.seqlens_k = seqlens;
  seq.lmax = W;
  seq.q_rows = Tq;
  const float sl2 = scale_log2_of(scale, D);
  hipError_t e;
  if (dtype == GQA_FP32) {
    if ((long long)B * max_q_len * Hq > 0x7fffffffLL) return fail(GQA_ERR_UNSUPPORTED, "problem too large for the fp32 path");
    Fp32Args a{};
    a.q = (const float*)q; a.k = (const float*)k_ring; a.v = (const float*)v_ring;
    a.k2 = (const float*)k_new; a.v2 = (const float*)v_new; a.sinks = sinks;
    a.out = (float*)out; a.lse = lse; a.seq = seq;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = G; a.window = W; a.sink_tokens = 0; a.scale_log2 = sl2;
    a.max_q_len = max_q_len; a.varlen_q = 1;
    a.lse_sb = 0; a.lse_sh = Tq; a.lse_row0 = 1;
    e = launch_fp32(a, KV_RING, st);
    if (e != hipSuccess) return hip_fail(e, "ring prefill fp32 launch");
  } else {
    PrefillArgs a{};
    a.q = (const __bf16*)q; a.k = (const __bf16*)k_ring; a.v = (const __bf16*)v_ring;
    a.k2 = (const __bf16*)k_new; a.v2 = (const __bf16*)v_new; a.sinks = sinks;
    a.out = (__bf16*)out; a.lse = lse; a.seq = seq;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = G; a.window = W; a.sink_tokens = 0; a.scale_log2 = sl2;
    const long ntiles = (long)((max_q_len + 31) / 32) * G;
    a.wg_per_seq = (int)((ntiles + prefill_ntiles_per_wg() - 1) / prefill_ntiles_per_wg());
    a.skip_single = 0;
    a.lse_sb = 0; a.lse_sh = Tq; a.lse_row0 = 1;
    a.sort_seq = B <= 256 && env_int("GQA_VARLEN_SORT", 1) != 0;
    if ((long long)B * Hkv * a.wg_per_seq > 0x7fffffffLL) return fail(GQA_ERR_UNSUPPORTED, "grid too large");
    e = launch_prefill_bf16(a, KV_RING, true, st);
    if (e != hipSuccess) return hip_fail(e, "ring prefill launch");
  }
  if (!append) return ok();
  // the chunk joins its rings once every query has read them: same stream, next launch
  RingAppendArgs r{};
  r.k_new = (const char*)k_new; r.v_new = (const char*)v_new;
  r.k_ring = (char*)k_ring; r.v_ring = (char*)v_ring;
  r.cu_seqlens_q = cu_seqlens_q; r.seqlens = seqlens;
  r.T = Tq; r.B = B; r.W = W;
  r.row_bytes = Hkv * D * (dtype == GQA_BF16 ? 2 : 4);
  e = launch_ring_append(r, st);
  return e == hipSuccess ? ok() : hip_fail(e, "ring append launch");
}

int gqa_rope_append(const void* q, const void* k, const void* v, void* q_out, const int32_t* cu_seqlens_q,
                    const int32_t* seqlens, const float* inv_freq, float mscale, int pairing, void* k_cache,
                    void* v_cache, int cache_kind, int cache_len, const int32_t* block_table, int max_blocks,
                    int block_size, int num_blocks, int B, int T, int Hq, int Hkv, int D, int dtype, void* stream) {
  if (dtype != GQA_BF16 && dtype != GQA_FP32) return fail(GQA_ERR_UNSUPPORTED, "dtype %d is not GQA_BF16 or GQA_FP32", dtype);
  if (D != kHeadDim) return fail(GQA_ERR_UNSUPPORTED, "head_dim %d is not supported (only 64)", D);
  if (B < 0 || T < 0 || Hq <= 0 || Hkv <= 0)
    return fail(GQA_ERR_INVALID_ARG, "bad size (B=%d, T=%d, Hq=%d, Hkv=%d)", B, T, Hq, Hkv);
  if (pairing != 0 && pairing != 1) return fail(GQA_ERR_INVALID_ARG, "pairing %d is not 0 or 1", pairing);
  if (std::isnan(mscale) || std::isinf(mscale)) return fail(GQA_ERR_INVALID_ARG, "mscale must be finite");
  if (!cu_seqlens_q && T != B)
    return fail(GQA_ERR_INVALID_ARG, "without cu_seqlens_q there is one new row per sequence (T=%d, B=%d)", T, B);
  int log2b = 0;
  if (cache_kind == 0 || cache_kind == 2) {
    if (cache_len <= 0) return fail(GQA_ERR_INVALID_ARG, "cache_len %d must be >= 1", cache_len);
  } else if (cache_kind == 1) {
    if (block_size < 1 || block_size > 1024 || (block_size & (block_size - 1)))
      return fail(GQA_ERR_UNSUPPORTED, "block_size %d is not a power of two in [1, 1024]", block_size);
    if (max_blocks <= 0 || num_blocks <= 0) return fail(GQA_ERR_INVALID_ARG, "max_blocks and num_blocks must be >= 1");
    if (!block_table && B > 0 && T > 0) return fail(GQA_ERR_INVALID_ARG, "a paged cache needs block_table");
    while ((1 << log2b) < block_size) ++log2b;
  } else {
    return fail(GQA_ERR_INVALID_ARG, "cache_kind %d is not 0 (contiguous), 1 (paged) or 2 (ring)", cache_kind);
  }
  if ((q == nullptr) != (q_out == nullptr))
    return fail(GQA_ERR_INVALID_ARG, "q and q_out are both given or both NULL (keys only)");
  if (B == 0 || T == 0) return ok();
  if (!k || !v || !seqlens || !k_cache || !v_cache)
    return fail(GQA_ERR_INVALID_ARG, "k, v, seqlens, k_cache and v_cache must be non-NULL");
  RopeAppendArgs a{};
  a.q = q; a.k = k; a.v = v; a.q_out = q_out; a.k_cache = k_cache; a.v_cache = v_cache;
  a.inv_freq = inv_freq; a.cu_seqlens_q = cu_seqlens_q; a.seqlens = seqlens; a.block_table = block_table;
  a.T = T; a.B = B; a.Hq = Hq; a.Hkv = Hkv;
  a.cache_kind = cache_kind; a.cache_len = cache_len;
  a.max_blocks = max_blocks; a.log2_block = log2b; a.num_blocks = num_blocks;
  a.pairing = pairing; a.mscale = mscale; a.fp32 = dtype == GQA_FP32;
  hipError_t e = launch_rope_append(a, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "rope append launch");
}

int gqa_attn_decode_step(const void* q, const void* k_new, const void* v_new, void* q_out, const int32_t* seqlens,
                         const float* inv_freq, float mscale, int pairing, void* k_cache, void* v_cache,
                         int cache_kind, int cache_len, const int32_t* block_table, int max_blocks, int block_size,
                         int num_blocks, const float* sinks, void* out, float* lse, int B, int Hq, int Hkv, int D,
                         int window, int sink_tokens, float scale, int dtype, void* stream) {
  int rc = check_common(Hq, Hkv, D, window, sink_tokens, scale, dtype);
  if (rc) return rc;
  if (dtype != GQA_BF16)
    return fail(GQA_ERR_UNSUPPORTED, "the fused decode step is bf16 only (fp32: gqa_rope_append, then gqa_attn_decode)");
  if (Hq / Hkv > kStepMaxG)
    return fail(GQA_ERR_UNSUPPORTED, "the fused decode step takes at most %d query heads per KV head (got %d)",
                kStepMaxG, Hq / Hkv);
  if (B < 0) return fail(GQA_ERR_INVALID_ARG, "negative batch B=%d", B);
  if (pairing != 0 && pairing != 1) return fail(GQA_ERR_INVALID_ARG, "pairing %d is not 0 or 1", pairing);
  if (std::isnan(mscale) || std::isinf(mscale)) return fail(GQA_ERR_INVALID_ARG, "mscale must be finite");
  int log2b = 0;
  long long span = 0;  // the most keys a query reads: one workgroup per (sequence, KV head) streams them all
  if (cache_kind == GQA_CACHE_CONTIGUOUS) {
    if (cache_len <= 0) return fail(GQA_ERR_INVALID_ARG, "cache_len %d must be >= 1", cache_len);
    span = window > 0 ? std::min<long long>((long long)window + sink_tokens, cache_len) : cache_len;
  } else if (cache_kind == GQA_CACHE_PAGED) {
    if (block_size < 1 || block_size > 1024 || (block_size & (block_size - 1)))
      return fail(GQA_ERR_UNSUPPORTED, "block_size %d is not a power of two in [1, 1024]", block_size);
    if (max_blocks <= 0 || num_blocks <= 0) return fail(GQA_ERR_INVALID_ARG, "max_blocks and num_blocks must be >= 1");
    if (!block_table && B > 0) return fail(GQA_ERR_INVALID_ARG, "a paged cache needs block_table");
    while ((1 << log2b) < block_size) ++log2b;
    const long long cap = (long long)max_blocks * block_size;
    span = window > 0 ? std::min<long long>((long long)window + sink_tokens, cap) : cap;
  } else if (cache_kind == GQA_CACHE_RING) {
    if (cache_len <= 0) return fail(GQA_ERR_INVALID_ARG, "ring size %d must be >= 1", cache_len);
    if (window != 0 && window != cache_len)
      return fail(GQA_ERR_INVALID_ARG, "a ring of %d slots is the window; window must be 0 or %d", cache_len, cache_len);
    if (sink_tokens != 0) return fail(GQA_ERR_UNSUPPORTED, "a ring cache holds no start-of-sequence sink tokens");
    window = cache_len;
    span = cache_len;
  } else {
    return fail(GQA_ERR_INVALID_ARG, "cache_kind %d is not 0 (contiguous), 1 (paged) or 2 (ring)", cache_kind);
  }
  if (span > kStepMaxKeys)
    return fail(GQA_ERR_UNSUPPORTED,
                "the fused decode step streams each query's keys in one workgroup and takes at most %d of them "
                "(this call: up to %lld); use gqa_rope_append, then gqa_attn_decode",
                kStepMaxKeys, span);
  if (B == 0) return ok();
  if (!q || !k_new || !v_new || !seqlens || !k_cache || !v_cache || !out)
    return fail(GQA_ERR_INVALID_ARG, "q, k_new, v_new, seqlens, k_cache, v_cache and out must be non-NULL");
  DecodeStepArgs a{};
  a.q = (const __bf16*)q; a.k_new = (const __bf16*)k_new; a.v_new = (const __bf16*)v_new; a.q_out = (__bf16*)q_out;
  a.k_cache = (__bf16*)k_cache; a.v_cache = (__bf16*)v_cache; a.seqlens = seqlens;
  a.inv_freq = inv_freq; a.mscale = mscale; a.pairing = pairing;
  a.cache_kind = cache_kind; a.cache_len = cache_len; a.block_table = block_table;
  a.max_blocks = max_blocks; a.log2_block = log2b; a.num_blocks = num_blocks;
  a.sinks = sinks; a.out = (__bf16*)out; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv;
  a.window = window; a.sink_tokens = sink_tokens; a.scale_log2 = scale_log2_of(scale, D);
  hipError_t e = launch_decode_step(a, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "decode step launch");
}

size_t gqa_attn_decode_ring_workspace_size(int B, int W, int Hq, int Hkv, int D, int dtype) {
  return gqa_attn_decode_workspace_size(B, W, Hq, Hkv, D, 0, 0, dtype);
}

int gqa_attn_decode_ring(const void* q, const void* k_ring, const void* v_ring, const int32_t* seqlens,
                         const float* sinks, void* out, float* lse, int B, int W, int Hq, int Hkv, int D,
                         float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (W <= 0) return fail(GQA_ERR_INVALID_ARG, "ring size W=%d must be >= 1", W);
  // The ring holds exactly the positions of the window ending at the query:
  // min(seqlens[b], W) slots, all visible.  Key order does not enter the
  // result, so this is dense attention over the valid slots of a W-slot cache,
  // whose kernels take min(seqlens[b], W) keys as the ring's length.
  return decode_call(q, k_ring, v_ring, seqlens, sinks, out, lse, B, W, Hq, Hkv, D, 0, 0, scale, dtype, workspace,
                     workspace_bytes, stream, 1);
}

size_t gqa_attn_prefill_backward_workspace_size(int B, int S, int Hq, int Hkv, int D, int dtype) {
  if ((dtype != GQA_BF16 && dtype != GQA_FP32) || B < 0 || S < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv ||
      D != kHeadDim)
    return 0;
  // <dO, o> and lse in log2 units per row and head, then (bf16, key ranges cut into slabs) the fp32
  // dK/dV partial sums of every (sequence, KV head, 64-key block, slab)
  // D and lse in log2 units, block sums of the sink gradient
  size_t bytes = 2 * (((size_t)B * Hq * S * sizeof(float) + 255) & ~(size_t)255) +
                 (((size_t)Hq * B * ((S + 1023) / 1024) * sizeof(float) + 255) & ~(size_t)255);
  int n_slabs = 1, slab_len = 0;
  backward_plan(B, S, Hkv, 0, 0, &n_slabs, &slab_len);  // the largest (dense) plan
  if (dtype == GQA_BF16 && n_slabs > 1)
    bytes += (size_t)B * Hkv * ((S + 63) / 64) * n_slabs * 2 * 64 * kHeadDim * sizeof(float);
  return bytes;
}

int gqa_attn_prefill_backward(const void* q, const void* k, const void* v, const float* sinks, const void* out,
                              const float* lse, const void* dout, void* dq, void* dk, void* dv, float* dsinks,
                              int B, int S, int Hq, int Hkv, int D, int window, int sink_tokens, float scale,
                              int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_common(Hq, Hkv, D, window, sink_tokens, scale, dtype);
  if (rc) return rc;
  if (B < 0 || S < 0) return fail(GQA_ERR_INVALID_ARG, "negative size (B=%d, S=%d)", B, S);
  const size_t need = gqa_attn_prefill_backward_workspace_size(B, S, Hq, Hkv, D, dtype);
  if (B > 0 && S > 0) {
    if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv)
      return fail(GQA_ERR_INVALID_ARG, "q, k, v, out, lse, dout, dq, dk and dv must be non-NULL");
    if (!workspace || workspace_bytes < need)
      return fail(GQA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, need);
    if ((long long)B * S * Hq > 0x7fffffffLL) return fail(GQA_ERR_UNSUPPORTED, "problem too large");
  } else if (!dsinks) {
    return ok();
  }
  BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = out; a.dout = dout; a.lse = lse; a.sinks = sinks;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dsinks = dsinks; a.dlt = (float*)workspace;
  backward_plan(B, S, Hkv, window, sink_tokens, &a.n_slabs, &a.slab_len);
  if (dtype != GQA_BF16) a.n_slabs = 1;
  const size_t row_bytes = ((size_t)B * Hq * S * sizeof(float) + 255) & ~(size_t)255;
  const size_t sink_bytes = ((size_t)Hq * B * ((S + 1023) / 1024) * sizeof(float) + 255) & ~(size_t)255;
  a.lse2 = (float*)((char*)workspace + row_bytes);
  a.dsink_part = (float*)((char*)workspace + 2 * row_bytes);
  a.part = (float*)((char*)workspace + 2 * row_bytes + sink_bytes);
  a.B = B; a.S = S; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv;
  a.window = window; a.sink_tokens = sink_tokens;
  a.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)D);
  a.scale_log2 = scale_log2_of(scale, D);
  a.fp32 = dtype == GQA_FP32;
  hipError_t e = launch_backward(a, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "prefill backward launch");
}

}  // extern "C"
