// fp32 I/O attention: a straightforward, exact-in-fp32 path for callers that
// keep activations in fp32 (prefill, decode and varlen/paged alike).
//
// Same definition as the bf16 kernels (sink + window causal GQA attention of
// «GPT-OSS vs Qwen3», sections "Introduction de Grouped Query Attention",
// "Utilisation de Sliding Window Attention" and "Attention Bias et Sinks", with
// optional start-of-sequence sink tokens kept visible past the window), but
// every product, exponential and sum is fp32 and nothing is rounded to bf16.
// One wave owns one (query row, query head): per 64-key chunk each lane scores
// one key (64-term fp32 dot product), the wave takes the online-softmax step,
// then each lane accumulates one output column over the chunk's keys.
#include "kernels.h"

namespace gqa {
namespace {

template <int MODE>
__global__ __launch_bounds__(64) void attn_fp32_kernel(Fp32Args a) {
  __shared__ float qs[kHeadDim];
  __shared__ float ps[64];
  __shared__ int64_t rows[64];

  const int lane = threadIdx.x;
  const int hq = blockIdx.x % a.Hq;
  int rest = blockIdx.x / a.Hq;
  const int t = rest % a.max_q_len;
  const int b = rest / a.max_q_len;
  const SeqView sv = seq_view<MODE>(a.seq, b, a.varlen_q != 0);
  if (t >= sv.q_len) return;
  const int g = hq / a.G;
  const int p = sv.kv_len - sv.q_len + t;
  const int W = a.window;
  const int lo = W > 0 ? max(0, p - W + 1) : 0;
  // keys visited: the sink tokens below the window, then the window itself,
  // numbered 0 .. nv-1 ("virtual" index v -> key v, or lo + v - ns)
  const int ns = W > 0 ? min(a.sink_tokens, lo) : 0;
  const int nv = ns + (p - lo + 1);
  const int64_t qrow = sv.q_row0 + t;
  const int64_t kv_stride = (int64_t)a.Hkv * kHeadDim;

  qs[lane] = a.q[(qrow * a.Hq + hq) * kHeadDim + lane];
  const float s2 = a.sinks ? a.sinks[hq] * kLog2e : -INFINITY;
  float m_run = (s2 == -INFINITY) ? kNegBig : s2;
  float l_run = (s2 == -INFINITY) ? 0.f : 1.f;
  float acc = 0.f;
  __syncthreads();

  for (int v0 = 0; v0 < nv; v0 += 64) {
    const int vi = v0 + lane;
    const bool live = vi < nv;
    const int j = vi < ns ? vi : lo + (vi - ns);
    float x = -INFINITY;
    int64_t row = 0;
    if (live) {
      row = MODE == KV_RING ? ring_chunk_row(a.seq, sv, j) : kv_row<MODE>(a.seq, sv, j);
      const float* kp = (row < 0 ? a.k2 + (-1 - row) * kv_stride : a.k + row * kv_stride) + g * kHeadDim;
      float dot = 0.f;
      for (int d = 0; d < kHeadDim; ++d) dot = __builtin_fmaf(qs[d], kp[d], dot);
      x = dot * a.scale_log2;
    }
    const float mx = wave_max(x);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    const float pj = live ? exp2f(x - m_new) : 0.f;
    l_run = l_run * alpha + wave_sum(pj);
    acc *= alpha;
    m_run = m_new;
    ps[lane] = pj;
    rows[lane] = row;
    __syncthreads();
    const int n = min(64, nv - v0);
    for (int jj = 0; jj < n; ++jj) {
      const int64_t r = rows[jj];  // KV_RING: -1 - r is a row of the chunk
      const float* vp = r < 0 ? a.v2 + (-1 - r) * kv_stride : a.v + r * kv_stride;
      acc = __builtin_fmaf(ps[jj], vp[g * kHeadDim + lane], acc);
    }
    __syncthreads();
  }
  const float inv = l_run > 0.f ? 1.f / l_run : (l_run == 0.f ? 0.f : l_run);
  a.out[(qrow * a.Hq + hq) * kHeadDim + lane] = acc * inv;
  if (a.lse && lane == 0) {
    const float v = (l_run == 0.f) ? -INFINITY : (m_run + log2f(l_run)) * kLn2;
    a.lse[(int64_t)b * a.lse_sb + (int64_t)hq * a.lse_sh + t + (a.lse_row0 ? sv.q_row0 : 0)] = v;
  }
}

}  // namespace

hipError_t launch_fp32(const Fp32Args& a, int kv_mode, hipStream_t s) {
  const int64_t grid = (int64_t)a.B * a.max_q_len * a.Hq;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (kv_mode == KV_BATCHED)
    hipLaunchKernelGGL((attn_fp32_kernel<KV_BATCHED>), dim3((unsigned)grid), dim3(64), 0, s, a);
  else if (kv_mode == KV_PAGED)
    hipLaunchKernelGGL((attn_fp32_kernel<KV_PAGED>), dim3((unsigned)grid), dim3(64), 0, s, a);
  else if (kv_mode == KV_PACKED)
    hipLaunchKernelGGL((attn_fp32_kernel<KV_PACKED>), dim3((unsigned)grid), dim3(64), 0, s, a);
  else if (kv_mode == KV_RING)
    hipLaunchKernelGGL((attn_fp32_kernel<KV_RING>), dim3((unsigned)grid), dim3(64), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// Metadata-check flags of this file's kernels (recorded only when built with GQA_DEBUG).
GQA_DEBUG_FLAGS_ACCESSOR(debug_flags_fp32)

}  // namespace gqa
