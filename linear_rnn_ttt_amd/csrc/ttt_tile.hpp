// ttt_tile.hpp -- 16-token tile machinery shared by the gfx950 TTT scan
// kernels: HBM -> LDS staging of q, k, v, eta with global_load_lds, the
// swizzled LDS row layout, bf16 hi/lo operand packing and the small MFMA
// products of the chunked form.
//
// Lane conventions as in ttt_device.hpp: lane l, group g = l / 16,
// column c = l % 16.
#pragma once

#include "ttt_device.hpp"

namespace tttk {

constexpr int D = 64;  // head dimension

template <bool BF16>
struct Io;
template <>
struct Io<true> {
  using E = uint16_t;
};
template <>
struct Io<false> {
  using E = float;
};

// Staged blocks hold rows of 64 elements without padding; the 16-byte chunk
// j of row t sits in slot j ^ (t & 7) of the row, which spreads the
// row-strided operand reads of a 16x16 tile over the LDS banks.
template <bool BF16>
__device__ __forceinline__ int lds_off(int t, int col) {  // element offset
  constexpr int EPC = 16 / sizeof(typename Io<BF16>::E);  // elements per chunk
  return t * D + (((col / EPC) ^ (t & 7)) * EPC) + (col % EPC);
}

// Double-buffered staging area: blocks of TB tiles of NX tensors (q, k, v
// in that order, the first NX of them) and eta.
template <bool BF16, int TB, int NX = 3>
struct Stage {
  using E = typename Io<BF16>::E;
  static constexpr int TOK = TB * 16;
  E qkv[2][NX][TOK * D];
  float eta[2][TOK];
};

#define TTT_LDS __attribute__((address_space(3)))

// Start copying block `blk` (TB tiles) of q, k, v and eta from HBM straight
// into LDS buffer `buf` (global_load_lds: no registers, no VALU).  Four
// waves share the copy; `w` (0..3) is the calling wave's share.  Each wave
// moves 1 KB per instruction; lane l lands at byte 16 l of it, so the lane
// picks the source chunk that belongs in that swizzled slot.  Rows past T
// re-read row T-1 (finite data; their eta is ignored by the scan).
// The share can be issued in `parts` calls (part = 0 .. parts-1), which
// spreads the copy instructions of a block over several tiles.  A null
// tensor (or eta) is not copied.
template <bool BF16, int TB, int NX>
__device__ __forceinline__ void stage_issue(Stage<BF16, TB, NX>& L, const void* q, const void* k,
                                            const void* v, const float* eta, size_t row0,
                                            int blk, int T, int buf, int w, int part = 0,
                                            int parts = 1) {
  using E = typename Io<BF16>::E;
  constexpr int TOK = TB * 16;
  constexpr int RB = D * sizeof(E);            // row bytes
  constexpr int NI = TOK * RB / (4 * 1024);    // instructions per wave per tensor
  const int l = threadIdx.x & 63;
  const int tok0 = blk * TOK;
  const char* src[3] = {static_cast<const char*>(q), static_cast<const char*>(k),
                        static_cast<const char*>(v)};
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    const int off = (NI * w + n) * 1024 + 16 * l;   // byte offset in the block
    const int t = off / RB, slot = (off % RB) / 16;
    const int j = slot ^ (t & 7);
    const int tok = min(tok0 + t, T - 1);
    const size_t goff = (row0 + tok) * (size_t)RB + j * 16;
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      if (!src[x] || (3 * n + x) % parts != part) continue;
      TTT_LDS void* dst = (TTT_LDS void*)(reinterpret_cast<char*>(L.qkv[buf][x]) +
                                          (NI * w + n) * 1024);
      __builtin_amdgcn_global_load_lds(src[x] + goff, dst, 16, 0, 0);
    }
  }
  if (eta && part == 0 && w * 64 + l < TOK) {   // blocks of fewer than 64 tokens: the lanes past TOK idle
    const int tok = min(tok0 + w * 64 + l, T - 1);
    TTT_LDS void* dst = (TTT_LDS void*)(&L.eta[buf][w * 64]);
    __builtin_amdgcn_global_load_lds(eta + row0 + tok, dst, 4, 0, 0);
  }
}

// Wait for this wave's outstanding global->LDS copies (and stores).
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---- LDS operand fetch ---------------------------------------------------
// Four consecutive elements of one row as bf16 hi (and lo for fp32 data).
struct Op4 {
  u32x2 hi, lo;
};
__device__ __forceinline__ Op4 op4(const uint16_t* p) {
  return Op4{*reinterpret_cast<const u32x2*>(p), u32x2{0u, 0u}};
}
__device__ __forceinline__ Op4 op4(const float* p) {
  const Split4 s = split4(*reinterpret_cast<const f32x4*>(p));
  return Op4{s.hi, s.lo};
}
__device__ __forceinline__ Op4 op4_of(f32x4 v) {
  const Split4 s = split4(v);
  return Op4{s.hi, s.lo};
}
__device__ __forceinline__ Op4 op4_of(uint32_t e0, uint32_t e1, uint32_t e2, uint32_t e3) {
  return Op4{u32x2{e0 | (e1 << 16), e2 | (e3 << 16)}, u32x2{0u, 0u}};
}
// Four consecutive elements of one row as fp32.
__device__ __forceinline__ f32x4 val4(const uint16_t* p) {
  const u32x2 w = *reinterpret_cast<const u32x2*>(p);
  return f32x4{bf16_lo_to_f32(w.x), bf16_hi_to_f32(w.x), bf16_lo_to_f32(w.y),
               bf16_hi_to_f32(w.y)};
}
__device__ __forceinline__ f32x4 val4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// The 4 accumulator registers of two 16x16 tiles of X, split into bf16 hi/lo
// and laid out as 16x16x32 operands: slot j < 4 -> tile a element j, slot
// j >= 4 -> tile b element j - 4.
struct Op8 {
  u32x4 hi, lo;
};
__device__ __forceinline__ Op8 split_pair(f32x4 a, f32x4 b) {
  const Split4 sa = split4(a), sb = split4(b);
  return Op8{cat(sa.hi, sb.hi), cat(sa.lo, sb.lo)};
}

// acc + A B over hi/lo parts: hi*hi, plus lo*hi when A has a lo part, plus
// hi*lo when B has one (the lo*lo term is below the split's precision).
template <bool ALO, bool BLO>
__device__ __forceinline__ f32x4 mma8(const Op8& a, const Op8& b, f32x4 acc) {
  acc = mfma32(a.hi, b.hi, acc);
  if (ALO) acc = mfma32(a.lo, b.hi, acc);
  if (BLO) acc = mfma32(a.hi, b.lo, acc);
  return acc;
}

// Rows c of a staged 16-token tile at features 32p + 4g + (0..3) and
// 32p + 16 + 4g + (0..3): the B operand of X^T (16x16x32, slots matching
// split_pair of two state tiles) and the A / B operand of X X'^T.
struct Rows {
  Op8 p[2];
};
template <bool BF16>
__device__ __forceinline__ Rows load_rows(const typename Io<BF16>::E* X, int t0, int c, int g) {
  Rows r;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const Op4 a = op4(X + lds_off<BF16>(t0 + c, 32 * p + 4 * g));
    const Op4 b = op4(X + lds_off<BF16>(t0 + c, 32 * p + 16 + 4 * g));
    r.p[p] = Op8{cat(a.hi, b.hi), cat(a.lo, b.lo)};
  }
  return r;
}
// The state W (four accumulator tiles of one wave) as A operands of W^T.
__device__ __forceinline__ void split_state(Op8 A[2], const f32x4 W[4]) {
#pragma unroll
  for (int p = 0; p < 2; ++p) A[p] = split_pair(W[2 * p], W[2 * p + 1]);
}
// X W for the wave's 16 output columns, transposed: lane (g,c) gets
// (X W)[row c][16w + 4g + i].
template <bool LO>
__device__ __forceinline__ f32x4 times_state(const Op8 A[2], const Rows& X) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < 2; ++p) acc = mma8<true, LO>(A[p], X.p[p], acc);
  return acc;
}
// X Y^T in accumulator layout: lane (g,c) gets x_{4g+i} . y_c.
template <bool LO>
__device__ __forceinline__ f32x4 gram(const Rows& X, const Rows& Y) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < 2; ++p) acc = mma8<LO, LO>(X.p[p], Y.p[p], acc);
  return acc;
}
template <bool ALO, bool BLO>
__device__ __forceinline__ f32x4 mma4(const Op4& a, const Op4& b, f32x4 acc) {
  acc = mfma16(a.hi, b.hi, acc);
  if (ALO) acc = mfma16(a.lo, b.hi, acc);
  if (BLO) acc = mfma16(a.hi, b.lo, acc);
  return acc;
}

// 16x16 transpose of an fp32 tile held as 4 accumulator registers (lane
// (g,c) has X[4g+i][c]) on the matrix unit: X (as the A operand of X^T,
// bf16 hi/lo) times the identity gives X^T in accumulator layout, returned
// re-split as a 16x16x16 operand (lane (g,c) gets X[c][4g+i]).
template <bool LO>
__device__ __forceinline__ Op4 transpose_op(const Split4& x, u32x2 ident) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const f32x4 th = mfma16(x.hi, ident, zero);
  Op4 r;
  r.hi = u32x2{pack_bf16(th[0], th[1]), pack_bf16(th[2], th[3])};
  r.lo = u32x2{0u, 0u};
  if (LO) {
    const f32x4 tl = mfma16(x.lo, ident, zero);
    r.lo = u32x2{pack_bf16(tl[0], tl[1]), pack_bf16(tl[2], tl[3])};
  }
  return r;
}

// Identity (and all-ones) tiles as 16x16x16 B operands: lane (g,c) holds
// I[4g + i][c].
__device__ __forceinline__ u32x2 ident_op(int g, int c) {
  uint32_t e[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) e[i] = (4 * g + i == c) ? 0x3F80u : 0u;
  return u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
}
__device__ __forceinline__ u32x2 ones_op() { return u32x2{0x3F803F80u, 0x3F803F80u}; }

}  // namespace tttk
