// KV append into the ring buffers of sliding-window layers.
//
// A windowed layer only ever attends to the last W positions of a sequence
// («GPT-OSS vs Qwen3», "Utilisation de Sliding Window Attention": 128 tokens,
// chosen to bound memory), so its cache is a ring of W slots per sequence
// with position p in slot p % W.  This kernel writes the K and V rows of new
// tokens into their slots, bit for bit.  Of a chunk longer than W only the
// last W positions are written: the older ones would land in the same slots
// as newer rows of the same call.
//
// One wave per new row: the Hkv * D elements of a K row and of a V row are
// moved as 16-byte words, 64 lanes side by side.
#include "kernels.h"

namespace gqa {
namespace {

constexpr int RTHREADS = 256;  // 4 waves, one new row each

__global__ __launch_bounds__(RTHREADS) void ring_append_kernel(RingAppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (RTHREADS / 64) + (threadIdx.x >> 6);
  if (row >= a.T) return;

  // sequence of this row and its position
  int b, t, q_len;
  if (a.cu_seqlens_q) {
    // largest b with cu[b] <= row (cu is non-decreasing); rows past cu[B] belong to no sequence
    if (row >= a.cu_seqlens_q[a.B]) return;
    int lo = 0, hi = a.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.cu_seqlens_q[mid] <= row) lo = mid;
      else hi = mid - 1;
    }
    b = lo;
    const int r0 = a.cu_seqlens_q[b];
    q_len = a.cu_seqlens_q[b + 1] - r0;
    t = (int)(row - r0);
    if (t < 0 || t >= q_len) return;
  } else {
    b = (int)row;
    t = 0;
    q_len = 1;
  }
  const int L = a.seqlens[b];
  const int p = L - q_len + t;
  if (p < 0 || p < L - a.W) return;  // not among the last W positions
  const int slot = p % a.W;

  // row_bytes = Hkv * D * element size, a multiple of 16 for D = 64
  const int words = a.row_bytes >> 4;
  const u32x4* ks = reinterpret_cast<const u32x4*>(a.k_new + row * a.row_bytes);
  const u32x4* vs = reinterpret_cast<const u32x4*>(a.v_new + row * a.row_bytes);
  const int64_t dst = ((int64_t)b * a.W + slot) * a.row_bytes;
  u32x4* kd = reinterpret_cast<u32x4*>(a.k_ring + dst);
  u32x4* vd = reinterpret_cast<u32x4*>(a.v_ring + dst);
  for (int i = lane; i < words; i += 64) {
    kd[i] = ks[i];
    vd[i] = vs[i];
  }
}

}  // namespace

hipError_t launch_ring_append(const RingAppendArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const int64_t blocks = (a.T + RTHREADS / 64 - 1) / (RTHREADS / 64);
  hipLaunchKernelGGL(ring_append_kernel, dim3((unsigned)blocks), dim3(RTHREADS), 0, s, a);
  return hipGetLastError();
}

// Metadata-check flags of this file's kernels (recorded only when built with GQA_DEBUG).
GQA_DEBUG_FLAGS_ACCESSOR(debug_flags_ring)

}  // namespace gqa
