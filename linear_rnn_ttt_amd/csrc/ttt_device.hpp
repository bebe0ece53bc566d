// ttt_device.hpp -- gfx950 (CDNA4) building blocks shared by the TTT scan
// kernels: MFMA wrappers, bf16 hi/lo splitting, cross-lane sums.
//
// MFMA fragment conventions used throughout (64-lane wave, lane l,
// group g = l / 16, column c = l % 16):
//   16x16 accumulator D (f32x4):     lane holds D[4g + i][c],       i = 0..3
//   16x16x16 bf16 A operand (4 bf16): lane holds A[c][4g + i]
//   16x16x16 bf16 B operand (4 bf16): lane holds B[4g + i][c]
//   16x16x32 bf16 A / B operand (8 bf16): lane holds A[c][k(g, j)] /
//       B[k(g, j)][c], j = 0..7, where k(g, j) is the same function for A
//       and B.  The kernels only rely on that: they assign their own meaning
//       ("slot j of group g") to the contraction index, identically in both
//       operands, so the hardware's exact k-order is irrelevant.
// Consequences the kernels use:
//   * an accumulator X is directly the B operand of X and the A operand of
//     X^T for a 16-deep contraction over its row index;
//   * X (16x16, A-operand layout) times the identity gives X in accumulator
//     layout, i.e. a register-level 16x16 transpose on the matrix unit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tttk {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// D = A * B + C, 16x16x32, bf16 operands (8 per lane), fp32 accumulate.
__device__ __forceinline__ f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D = A * B + C, 16x16x16, bf16 operands (4 per lane), fp32 accumulate.
__device__ __forceinline__ f32x4 mfma16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) {
  return __builtin_bit_cast(float, w << 16);
}
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xffff0000u);
}

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): about 16 significant
// bits in two bf16 operands.  Returns {hi(x0,x1), hi(x2,x3)} and the same
// for lo.
struct Split4 {
  u32x2 hi, lo;
};
__device__ __forceinline__ Split4 split4(f32x4 x) {
  Split4 s;
  s.hi.x = pack_bf16(x[0], x[1]);
  s.hi.y = pack_bf16(x[2], x[3]);
  float r0 = x[0] - bf16_lo_to_f32(s.hi.x);
  float r1 = x[1] - bf16_hi_to_f32(s.hi.x);
  float r2 = x[2] - bf16_lo_to_f32(s.hi.y);
  float r3 = x[3] - bf16_hi_to_f32(s.hi.y);
  s.lo.x = pack_bf16(r0, r1);
  s.lo.y = pack_bf16(r2, r3);
  return s;
}

// x = hi + mid + lo, each part the bf16 rounding of what the parts before it
// leave: about 24 significant bits (fp32 precision) in three bf16 operands.
struct Split4x3 {
  u32x2 hi, mid, lo;
};
__device__ __forceinline__ Split4x3 split4x3(f32x4 x) {
  Split4x3 s;
  s.hi.x = pack_bf16(x[0], x[1]);
  s.hi.y = pack_bf16(x[2], x[3]);
  float r0 = x[0] - bf16_lo_to_f32(s.hi.x);
  float r1 = x[1] - bf16_hi_to_f32(s.hi.x);
  float r2 = x[2] - bf16_lo_to_f32(s.hi.y);
  float r3 = x[3] - bf16_hi_to_f32(s.hi.y);
  s.mid.x = pack_bf16(r0, r1);
  s.mid.y = pack_bf16(r2, r3);
  r0 -= bf16_lo_to_f32(s.mid.x);
  r1 -= bf16_hi_to_f32(s.mid.x);
  r2 -= bf16_lo_to_f32(s.mid.y);
  r3 -= bf16_hi_to_f32(s.mid.y);
  s.lo.x = pack_bf16(r0, r1);
  s.lo.y = pack_bf16(r2, r3);
  return s;
}

__device__ __forceinline__ u32x4 cat(u32x2 a, u32x2 b) { return u32x4{a.x, a.y, b.x, b.y}; }

// Workgroup barrier that orders LDS only (release/acquire fences on the
// local address space around s_barrier).  Unlike __syncthreads() it does not
// wait for outstanding global loads and stores, so prefetches and output
// stores stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The same barrier for a wave whose global-to-LDS copies (global_load_lds)
// are still in flight into a buffer that no wave reads before a later
// barrier.  The release fence above counts such copies as LDS writes and
// would wait for them (vmcnt(0)), holding the whole workgroup at the barrier
// for a memory round trip; here only the wave's own LDS accesses are waited
// for.  The "memory" clobber keeps the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void lds_barrier_copies_in_flight() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t fbits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float bitsf(uint32_t x) { return __builtin_bit_cast(float, x); }

// v_permlane32_swap on (a, b) leaves lanes 0-31 of a in place, moves lanes
// 0-31 of b to lanes 32-63 of a, and returns lanes 32-63 of a and b in b's
// place.  Summing the two results: lanes 0-31 get a[l] + a[l+32], lanes
// 32-63 get b[l-32] + b[l].
__device__ __forceinline__ float swap32_sum(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(fbits(a), fbits(b), false, false);
  return bitsf(r[0]) + bitsf(r[1]);
}
// v_permlane16_swap on (a, b) exchanges the odd 16-lane rows of a with the
// even rows of b.  Summing the two results: row 0 gets a0 + a1, row 1
// b0 + b1, row 2 a2 + a3, row 3 b2 + b3 (rows of 16 lanes).
__device__ __forceinline__ float swap16_sum(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(fbits(a), fbits(b), false, false);
  return bitsf(r[0]) + bitsf(r[1]);
}

// Sum over the four 16-lane groups (lanes c, c+16, c+32, c+48), in every lane.
__device__ __forceinline__ float group_sum(float x) {
  const float y = swap16_sum(x, x);
  return swap32_sum(y, y);
}

// Reduce-scatter of four per-lane partial sums over the four lane groups:
// group 0 receives the total of q0, group 1 of q2, group 2 of q1, group 3
// of q3 (three swaps instead of eight for four full group sums).
__device__ __forceinline__ float group_reduce_scatter4(float q0, float q1, float q2, float q3) {
  return swap16_sum(swap32_sum(q0, q1), swap32_sum(q2, q3));
}
// Which quantity group g holds after group_reduce_scatter4.
__device__ __forceinline__ constexpr int rs4_slot(int g) { return g == 1 ? 2 : (g == 2 ? 1 : g); }

}  // namespace tttk
