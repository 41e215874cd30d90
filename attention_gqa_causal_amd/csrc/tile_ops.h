// MFMA tile operations shared by the gfx950 attention kernels (forward and
// backward): the 32x32x16 bf16 matrix instruction, the swizzled LDS row
// layout, the transposing LDS operand read, and the causal / window / sink
// token mask of a 32-key half tile.
//
// Register layouts of v_mfma_f32_32x32x16_bf16 (D = A B + C):
//   A (32 x 16): lane l holds row l % 32, k = 8 (l / 32) .. +7
//   B (16 x 32): lane l holds column l % 32, k = 8 (l / 32) .. +7
//   C (32 x 32): lane l, register r holds row 8 (r / 4) + 4 (l / 32) + r % 4,
//                column l % 32
// so a C tile can serve directly as the A or B operand of a product that
// contracts over its rows, with the contraction order permuted the same way on
// the other operand (see tr_operand).
#pragma once

#include "common.h"

namespace gqa {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int RS = 64;                 // LDS row (elements): one 128-byte row of 64 bf16, no padding
constexpr unsigned kWaitVm0 = 0x0F70;  // s_waitcnt vmcnt(0), leaving the other counters alone

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// LDS tiles hold rows of 64 bf16 (a key, or a query, with its 64 d) in their
// natural [row][d] layout, one 128-byte row each, with logical 16-byte chunk c
// of row r stored at chunk position c ^ kswz(r), kswz(r) = 2 (r % 4) +
// (r / 4) % 2.  The swizzle spreads the rows that one read instruction touches
// over all banks: the 8 rows of a row read (one chunk each; kswz is a
// permutation of 0..7) and the 4 rows of a transposing read (a pair of
// adjacent chunks each; kswz(r) / 2 differs between any 4 consecutive rows
// that start at a multiple of 4, so the 4 pairs land on different banks).
// It also lets a wave fill 8 whole rows with one 16-byte global-to-LDS load per
// lane: lane i lands at byte 16i of the wave's 8-row slice, so it fetches
// logical chunk (i & 7) ^ kswz(i >> 3) of row i >> 3.
__device__ __forceinline__ int kswz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }
// Element offset of logical 16-byte chunk cc of a row whose index is r (mod 8).
__device__ __forceinline__ int kchunk(int cc, int r) { return ((cc ^ kswz(r)) & 7) * 8; }

// Operand of a product that contracts over the rows of an LDS tile: for
// k-step u (tile rows 16u .. 16u+15) and d-block dt, lane l gets column
// d = 32 dt + l % 32 of the tile, at the 8 rows 16u + {4lg..4lg+3,
// 8+4lg..8+4lg+3} (lg = l / 32) -- the row order of C-tile registers
// 8u .. 8u+7, so the operand pairs with a C tile used as the other operand.
// Serves as A (rows = d) or B (columns = d) alike.  In 16-lane group c of the
// wave, lane j reads 4 consecutive d of tile row (j/4); the transposing load
// hands lane i of the group the 4 rows at d = dbase + i.  vofs: per-lane
// element offsets from tr_offsets.
__device__ __forceinline__ bf16x8 tr_operand(const __bf16* tile, int u, int dt, const int (&vofs)[2]) {
  const __bf16* base = tile + vofs[dt] + 16 * u * RS;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 8 * RS));
  const i16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, w);
}

// Per-lane element offsets of the transposing reads: tile row
// rk = 4*(lane/32) + (lane%16)/4 of each 8-row group, 4 consecutive d from
// d = 32*dt + 16*((lane/16)%2) + 4*(lane%4).
__device__ __forceinline__ void tr_offsets(int lane, int (&vofs)[2]) {
  const int rk = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int c0 = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
  for (int dt = 0; dt < 2; ++dt) vofs[dt] = rk * RS + kchunk(4 * dt + c0, rk) + 4 * (lane & 1);
}

// Mask of one transposed score tile S^T (keys in registers, one query row per
// lane) on key half h.  Lane holds keys j0 + 32h + 8*(r/4) + 4*lg + r%4 of
// query row lr; with off = 32h + 8*(r/4) + r%4 the key is visible iff
// off <= dh (causal) and, on a windowed layer, off > dl (inside the window) or
// off < ds (one of the first st positions, the start-of-sequence sink tokens).
// dh, dl, ds are per-lane bounds, so the per-register offsets stay
// compile-time constants.  The half is classified with wave-uniform bounds
// (plo, phi: the first and last query position of the tile) first: wholly
// visible is left alone, wholly hidden is cleared, and only a half that the
// causal diagonal or the window edge crosses is compared element by element.
template <bool STK>
__device__ __forceinline__ void mask_half(f32x16& s, int h, int j0, int plo, int phi, int W, int st, int dh, int dl,
                                          int ds) {
  const int kb = j0 + 32 * h;  // first key of this half (uniform)
  const bool any_sink = STK && kb < st;
  const bool all_sink = STK && kb + 31 < st;
  if (kb > phi || (W > 0 && !any_sink && kb + 31 <= plo - W)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = -INFINITY;
    return;
  }
  if (kb + 31 > plo) {  // causal diagonal crosses this half
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (32 * h + 8 * (r >> 2) + (r & 3) > dh) s[r] = -INFINITY;
  }
  if (W > 0 && !all_sink && kb <= phi - W) {  // window edge crosses this half
    if (any_sink) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 32 * h + 8 * (r >> 2) + (r & 3);
        if (off <= dl && off >= ds) s[r] = -INFINITY;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * h + 8 * (r >> 2) + (r & 3) <= dl) s[r] = -INFINITY;
    }
  }
}

// Direct global-to-LDS loads (lane i's 16 or 4 bytes land at byte 16 i or 4 i
// past the LDS address, which must be wave-uniform), issued from inline asm.
// The compiler, seeing an LDS write in flight, would make every later LDS read
// wait for it, even reads of another buffer; the tile loops instead wait for
// these loads themselves (s_waitcnt vmcnt, then a barrier) before any wave
// reads the buffer they fill.  M0 takes each LDS address (one wait state
// before the load) and gets its old value back afterwards (one wait state
// after), since the compiler does not track M0 across asm; the leading s_nop
// covers a base address just written to SGPRs by a vector instruction (five
// wait states).  Bases and LDS addresses go through readfirstlane, so they are
// scalar operands whatever the compiler proved.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ uint32_t lds_addr(lds_void* p) {
  return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p)));
}
// 4-byte loads from gbase + voff.
__device__ __forceinline__ void dma4(const char* gbase, uint32_t voff, lds_void* lds_dst) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_nop 4\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
      "global_load_lds_dword %1, %2\n\ts_mov_b32 m0, %0\n\ts_nop 0"
      : "=&s"(saved)
      : "v"(voff), "s"(uniform_ptr(gbase)), "s"(lds_addr(lds_dst))
      : "memory");
}

// The K and V halves of a wave's share of a tile: four 16-byte loads (K rows
// at voff0 and voff1 past kbase, V rows at the same offsets past vbase) under
// one save and restore of M0.  lds_k0 .. lds_v1 are LDS byte addresses.
__device__ __forceinline__ void dma16_kv(const char* kbase, const char* vbase, uint32_t voff0, uint32_t voff1,
                                         uint32_t lds_k0, uint32_t lds_k1, uint32_t lds_v0, uint32_t lds_v1) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_nop 4\n\t"
      "s_mov_b32 m0, %5\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %3\n\t"
      "s_mov_b32 m0, %7\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %4\n\t"
      "s_mov_b32 m0, %6\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %8\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %4\n\t"
      "s_mov_b32 m0, %0\n\ts_nop 0"
      : "=&s"(saved)
      : "v"(voff0), "v"(voff1), "s"(uniform_ptr(kbase)), "s"(uniform_ptr(vbase)),
        "s"(__builtin_amdgcn_readfirstlane(lds_k0)), "s"(__builtin_amdgcn_readfirstlane(lds_k1)),
        "s"(__builtin_amdgcn_readfirstlane(lds_v0)), "s"(__builtin_amdgcn_readfirstlane(lds_v1))
      : "memory");
}

// The same with 64-bit per-lane addresses (K rows at k0, k1, V rows at v0, v1).
__device__ __forceinline__ void dma16_kv(const void* k0, const void* k1, const void* v0, const void* v1,
                                         uint32_t lds_k0, uint32_t lds_k1, uint32_t lds_v0, uint32_t lds_v1) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_nop 4\n\t"
      "s_mov_b32 m0, %5\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %7\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %3, off\n\t"
      "s_mov_b32 m0, %6\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %8\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %4, off\n\t"
      "s_mov_b32 m0, %0\n\ts_nop 0"
      : "=&s"(saved)
      : "v"(k0), "v"(k1), "v"(v0), "v"(v1),
        "s"(__builtin_amdgcn_readfirstlane(lds_k0)), "s"(__builtin_amdgcn_readfirstlane(lds_k1)),
        "s"(__builtin_amdgcn_readfirstlane(lds_v0)), "s"(__builtin_amdgcn_readfirstlane(lds_v1))
      : "memory");
}

// Pin the instruction order: nothing is scheduled across this point.
__device__ __forceinline__ void fence_schedule() { __builtin_amdgcn_sched_barrier(0); }

}  // namespace gqa
