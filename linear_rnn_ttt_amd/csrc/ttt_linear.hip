// ttt_linear.hip -- TTT-Linear forward scan for gfx950 (MI355X).
//
// Method: f(x) = x + LN(x W); per token t the state takes the step
// W <- W - eta_t * grad ||f(k_t; W) - v_t||^2 with the gradient taken at the
// state of the start of the current mini-batch, and emits z_t = f(q_t; W_t)
// (dmarx.github.io record LIT-801 on arXiv 2407.04620, "Key takeaways"
// items 1, 2 and 5; the inner model from the codewithpapers.app record's
// "abstract").  For a 16-token tile with gradient factors G (row s = dl/dh
// of token s) this is, exactly,
//     H_k = K W_base                               gradient point
//     G   = LN_backward(2 (K + LN(H_k) - V))
//     H_q = Q W - tril(Q K^T) (eta * G)            W before the tile
//     Z   = Q + LN(H_q)
//     W  <- W - K^T (eta * G)
// (W_base == W for 16-token mini-batches; larger mini-batches keep W_base
// for several tiles).
//
// Mapping onto one CU: one 768-thread workgroup per (batch, head) unit, in
// three kinds of waves; wave w of each kind owns output columns
// 16(w mod 4)..+15, and one wave of each kind shares each SIMD, so the
// others fill the issue slots while one waits on the barrier, the LDS or
// the matrix unit (the update and chain waves run at a higher wave priority).
//   * Waves 0-3 ("chain") run only the serial part of the scan.  With the
//     gradient point K_{t+1} W_{t-2} and the score tiles K_{t-1} K_{t+1}^T,
//     K_t K_{t+1}^T prepared for them, they form
//     K_{t+1} W_t = K_{t+1} W_{t-2} + (K_{t+1} K_{t-1}^T)(-eta G_{t-1})
//     + (K_{t+1} K_t^T)(-eta G_t), of which only the last 16x16 correction
//     waits for tile t's gradient.  The serial path per tile is:
//     correction -> LN sums -> one exchange among the chain waves ->
//     gradient -> transpose.
//   * Waves 4-7 ("update") keep W[:, 16w:16w+16] as four 16x16 fp32 MFMA
//     accumulators.  In period t they apply the update of tile t-1, split
//     W_{t-1} into bf16 hi/lo, form Q_t W_{t-1} and K_{t+2} W_{t-1}, add
//     the tril(K Q^T) correction of tile t-1 to its Q W product, and, one
//     wave per item, prepare the column-independent inputs of tile t+2 for
//     the chain (the two score tiles, k . w_bar and sum_f u_f).  All of
//     these use row operands the wave reads once per period.
//   * Waves 8-11 ("output") take the output pre-activation of tile t-2,
//     exchange its LN sums and store z of tile t-3.  They also issue the
//     input copies, spread over several tiles.
//   * H is produced transposed (H^T = W^T K^T): a lane holds 4 features of
//     ONE token, so LN row sums are in-lane adds plus a reduce-scatter over
//     the 4 lane groups (v_permlane16/32_swap).
//   * LN sums are taken around the shifts k . w_bar and q . w_bar,
//     w_bar = W0 1 / d: the LN gradient of every token sums to zero over the
//     features, so W 1 is a constant of the scan and the shift is the row
//     mean up to rounding (it comes out of the matrix unit).  The means
//     themselves are still reduced from the data: centring on the shift
//     alone would turn the rounding drift of W 1 into gradients whose rows
//     no longer sum to zero, a feedback that grows along the sequence.
//   * Per-feature scalings are products with diagonal tiles on the matrix
//     unit (u = 2 gamma (k - v) + 2 gamma beta, q + beta); dot products of a
//     row with w_bar and 2 gamma are one product with a constant A operand.
//   * fp32 operands enter the bf16 matrix unit as sums of bf16 parts; bf16
//     inputs are exact.  Everything that feeds back into the state carries
//     three parts (hi + mid + lo, about 24 significant bits, fp32 level):
//     W in the gradient point K W, -eta G in the update K^T (-eta G), and
//     both operands of the chain's corrections (score tile and -eta G, six
//     products paired into three 16x16x32 products).  With two parts (about
//     16 bits) the rounding was amplified along the sequence on
//     ill-conditioned units (1.3B-shaped layer at T = 8192: z error 1e-1
//     where a plain fp32 evaluation of the same chunked form stays near the
//     bf16 floor of z).  The output side does not feed back: Q W uses
//     hi + mid, the output correction of bf16 data the hi part of the score
//     tile only.
//   * Row m of the state's accumulator tile r holds input feature
//     32 (r/2) + 8 (m/4) + 4 (r%2) + m%4, so the 8 contraction slots of a
//     lane in a 16x16x32 product with W are 8 consecutive features: every
//     row operand is a single 16-byte LDS read.
//   * Accumulate chains never mix the 16x16x32 and 16x16x16 shapes: on this
//     toolchain a result of one shape fed back to back as the C operand of
//     the other came out wrong in two of its four registers.
//   * q, k, v, eta stream from HBM to LDS in blocks of TB tiles
//     (global_load_lds, double-buffered).
//   * One barrier per tile orders every exchange.  Both loops are free of
//     branches within a tile (past the end: stale rows, gradient forced to
//     zero, z stores dropped by the buffer range check).
//   * SPLIT instances run each unit on two workgroups: the output side (q
//     products, output correction, output LN, z) moves to a second
//     workgroup on another CU, which replays the state from the gradients
//     the first streams to it through device memory (see "Split units"
//     below).
#include <mutex>

#include "ttt_device.hpp"
#include "ttt_kernels.hpp"
#include "ttt_tile.hpp"

namespace tttk {
namespace {

constexpr int NT = 768;  // 4 chain, 4 update and 4 output waves

template <bool BF16>
struct LinCfg {
  static constexpr int TB = BF16 ? 8 : 4;  // tiles per staged block (16 KB per tensor)
};

template <bool BF16>
struct LinLds {
  static constexpr int TB = LinCfg<BF16>::TB;
  Stage<BF16, TB> st;
  // chain LN partial sums around the shift [parity][wave][token]: (sum e,
  // sum e^2, sum gamma^2 e, sum gamma^2 e^2); lane c reads the 16-byte row
  // of token c.  xu[parity][token][wave]: sum u e.
  f32x4 xc[2][4][16];
  f32x4 xu[2][16];
  u32x4 gtb[2][4][64];  // (-eta G_t)^T as [hi, mid], chain wave -> update and output waves
  u32x2 gtl[2][4][64];  // its lo part
  f32x4 bkb[2][4][64];  // (K_{t+2} W_{t-1})^T, update wave -> chain wave
  u32x4 grp[2][2][3][64];  // K_{t+1} K_{t+2}^T, K_t K_{t+2}^T in three bf16 parts,
                           // packed as the three B operands of corr6
  f32x2 tkb[2][16];     // per token of tile t+2: (k . w_bar, sum_f u_f)
  f32x4 hqb[2][4][64];  // output pre-activation of tile t-1 around its shift,
                        // update wave -> output wave
  f32x2 xo[2][16][4];   // output LN: (sum e, sum e^2) per token and wave
  u32x4 mqb[2][64];     // tril(K_t Q_t^T) as [hi, lo] (hi only for bf16 data),
                        // update wave 2 -> every update wave
  float mqm[2][16];     // q . w_bar per token of tile t, update wave 2 -> every update wave
  uint16_t cst[8][D];   // bf16 rows: w_bar hi, 2 gamma hi, w_bar mid, 2 gamma mid,
                        // w_bar lo, 2 gamma lo, zero, zero
};

// LDS of the output workgroup of a split unit: q and k staged in blocks of
// TB = 4 tiles, the unit's gradient stream staged in the same blocks, and
// the exchanges of the output side.
template <bool BF16>
struct OutLds {
  static constexpr int TB = 4;
  Stage<BF16, TB, 2> st;    // q, k
  u32x4 gst[2][TB][4][64];  // (-eta G)^T as [hi, mid]: [buffer][tile][column block][lane]
  u32x4 gsl[2][TB][2][64];  // lo parts, column blocks (2j, 2j+1) as [lo, lo]
  f32x4 hqb[2][4][64];
  f32x2 xo[2][16][4];
  u32x4 mqb[2][64];
  float mqm[2][16];
  uint16_t cst[4][D];
};

template <bool BF16>
union SplitLds {
  LinLds<BF16> c;  // chain workgroup
  OutLds<BF16> o;  // output workgroup
};

struct Ctx {
  int lane, g, c, w, fo;  // w: column block (wave mod 4); fo = 16 w + 4 g
  int unit, head, T, n, tpm;
  size_t row0;            // first row of the unit in [B*H*T, 64]
};

// Staged rows of the tile `tb` tiles after the first tile of block `blk`
// (tb may run past the block, into the other buffer).
template <bool BF16, int TB, int NX>
__device__ __forceinline__ const typename Io<BF16>::E* tile_rows(const Stage<BF16, TB, NX>& st,
                                                                 int x, int blk, int tb) {
  return st.qkv[(blk + tb / TB) & 1][x] + (tb % TB) * 16 * D;
}
template <bool BF16, int TB, int NX>
__device__ __forceinline__ float tile_eta(const Stage<BF16, TB, NX>& st, int blk, int tb, int c) {
  return st.eta[(blk + tb / TB) & 1][(tb % TB) * 16 + c];
}

// Input feature held by row m of the state's accumulator tile r.
__device__ __forceinline__ constexpr int feat(int r, int m) {
  return 32 * (r >> 1) + 8 * (m >> 2) + 4 * (r & 1) + (m & 3);
}

// Row c of a staged tile as the 16x16x32 operand matching the state's
// contraction slots: slot j of product p is feature 32 p + 8 g + j.
template <bool BF16>
__device__ __forceinline__ Rows rows8(const typename Io<BF16>::E* X, int c, int g) {
  Rows r;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    if constexpr (BF16) {
      r.p[p].hi = *reinterpret_cast<const u32x4*>(X + lds_off<true>(c, 32 * p + 8 * g));
      r.p[p].lo = u32x4{0u, 0u, 0u, 0u};
    } else {
      const Split4 a =
          split4(*reinterpret_cast<const f32x4*>(X + lds_off<false>(c, 32 * p + 8 * g)));
      const Split4 b =
          split4(*reinterpret_cast<const f32x4*>(X + lds_off<false>(c, 32 * p + 8 * g + 4)));
      r.p[p] = Op8{cat(a.hi, b.hi), cat(a.lo, b.lo)};
    }
  }
  return r;
}
// K^T of a staged tile as the 16x16x16 A operands of the update of
// accumulator tile r: lane (g,c) holds K[4g + i][feat(r, c)].
template <bool BF16>
__device__ __forceinline__ void cols8(Op4 kt[4], const typename Io<BF16>::E* X, int c, int g) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int f = feat(r, c);
    const auto e0 = X[lds_off<BF16>(4 * g + 0, f)];
    const auto e1 = X[lds_off<BF16>(4 * g + 1, f)];
    const auto e2 = X[lds_off<BF16>(4 * g + 2, f)];
    const auto e3 = X[lds_off<BF16>(4 * g + 3, f)];
    if constexpr (BF16) kt[r] = op4_of(e0, e1, e2, e3);
    else kt[r] = op4_of(f32x4{e0, e1, e2, e3});
  }
}
// Features fo..fo+3 of row c of a bf16 tile: the 16x16x16 B operand of X^T
// restricted to one column block (lane (g,c) holds X[c][16w + 4g + i]).
__device__ __forceinline__ u32x2 quad(const uint16_t* X, int c, int fo) {
  return *reinterpret_cast<const u32x2*>(X + lds_off<true>(c, fo));
}

__device__ __forceinline__ u32x4 zero_unless(bool keep, u32x4 x) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  return keep ? x : z;
}
__device__ __forceinline__ u32x2 zero_unless(bool keep, u32x2 x) {
  const u32x2 z = {0u, 0u};
  return keep ? x : z;
}
// [first, second] part of a 4-register operand tuple: [hi, lo] of a
// two-part split, [hi, mid] of a three-part one
__device__ __forceinline__ u32x2 hi_of(u32x4 g) { return u32x2{g.x, g.y}; }
__device__ __forceinline__ u32x2 lo_of(u32x4 g) { return u32x2{g.z, g.w}; }
__device__ __forceinline__ u32x2 mid_of(u32x4 g) { return u32x2{g.z, g.w}; }
__device__ __forceinline__ u32x4 hilo(const Split4& s) { return cat(s.hi, s.lo); }

// acc + (-eta G)^T S for a score tile S (tokens x tokens) and G, each as
// three bf16 parts: the six products down to a relative size of 2^-16 (hi
// hi, mid hi, lo hi, hi mid, hi lo, mid mid), paired into three 16x16x32
// products whose slots 0-3 and 4-7 hold the two 16-deep operands.  G comes
// as the tuples [hi, mid] and [lo, hi], S as the packed B operands
// [hi, hi], [hi, mid], [lo, mid] (ScoreOps), so that no operand needs a
// register copy (acc may come from LDS).
struct ScoreOps {
  u32x4 b[3];
};
__device__ __forceinline__ f32x4 corr6(u32x4 ghm, u32x4 glh, const ScoreOps& s, f32x4 acc) {
  acc = mfma32(ghm, s.b[0], acc);  // hi hi + mid hi
  acc = mfma32(glh, s.b[1], acc);  // lo hi + hi mid
  acc = mfma32(ghm, s.b[2], acc);  // hi lo + mid mid
  return acc;
}
__device__ __forceinline__ ScoreOps score_ops(const Split4x3& s) {
  return ScoreOps{{cat(s.hi, s.hi), cat(s.hi, s.mid), cat(s.lo, s.mid)}};
}
__device__ __forceinline__ ScoreOps read_score(const u32x4 (&g)[3][64], int lane) {
  return ScoreOps{{g[0][lane], g[1][lane], g[2][lane]}};
}
__device__ __forceinline__ void write_score(u32x4 (&g)[3][64], int lane, const ScoreOps& s) {
#pragma unroll
  for (int i = 0; i < 3; ++i) g[i][lane] = s.b[i];
}

// Dot products of the rows of X with the constant rows (w_bar hi, 2 gamma hi,
// w_bar lo, 2 gamma lo): lane (g,c) gets them for token c in registers 0-3.
template <bool LO>
__device__ __forceinline__ f32x4 stats(const u32x4 ast[2], const Rows& x) {
  f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    d = mfma32(ast[p], x.p[p].hi, d);
    if (LO) d = mfma32(ast[p], x.p[p].lo, d);
  }
  return d;
}

// The state as 16x16x32 A operands of W^T in three bf16 parts: A = [hi,
// mid] (as split_state_mm) and Al = lo.  Each remainder is formed on the
// matrix unit: -I times the packed part, accumulated onto what is left, is
// exact in fp32.
__device__ __forceinline__ void split_state_mm3(Op8 A[2], u32x4 Al[2], const f32x4 W[4],
                                                u32x2 neg_ident) {
  u32x2 hi[4], mid[4], lo[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) hi[r] = u32x2{pack_bf16(W[r][0], W[r][1]), pack_bf16(W[r][2], W[r][3])};
  f32x4 d[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    d[r] = mfma16(neg_ident, hi[r], W[r]);
    mid[r] = u32x2{pack_bf16(d[r][0], d[r][1]), pack_bf16(d[r][2], d[r][3])};
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const f32x4 e = mfma16(neg_ident, mid[r], d[r]);
    lo[r] = u32x2{pack_bf16(e[0], e[1]), pack_bf16(e[2], e[3])};
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    A[p] = Op8{cat(hi[2 * p], hi[2 * p + 1]), cat(mid[2 * p], mid[2 * p + 1])};
    Al[p] = cat(lo[2 * p], lo[2 * p + 1]);
  }
}
// The same split on the VALU (prologue).
__device__ __forceinline__ void split_state3(Op8 A[2], u32x4 Al[2], const f32x4 W[4]) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const Split4x3 a = split4x3(W[2 * p]), b = split4x3(W[2 * p + 1]);
    A[p] = Op8{cat(a.hi, b.hi), cat(a.mid, b.mid)};
    Al[p] = cat(a.lo, b.lo);
  }
}
// X W with W in three parts (the gradient point; see times_state for the
// layout): hi, mid and lo of W against the rows' hi part, plus hi of W
// against the rows' lo part for fp32 data.
template <bool LO>
__device__ __forceinline__ f32x4 times_state3(const Op8 A[2], const u32x4 Al[2], const Rows& X) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    acc = mfma32(A[p].hi, X.p[p].hi, acc);
    acc = mfma32(A[p].lo, X.p[p].hi, acc);
    acc = mfma32(Al[p], X.p[p].hi, acc);
    if (LO) acc = mfma32(A[p].hi, X.p[p].lo, acc);
  }
  return acc;
}

// The state as 16x16x32 A operands of W^T (see split_state), with the lo
// part W - bf16(W) formed on the matrix unit: -I times the packed hi tile,
// accumulated onto W, is exact in fp32 (W - bf16(W) has at most 16
// significant bits), so only the two conversions per pair stay on the VALU.
__device__ __forceinline__ void split_state_mm(Op8 A[2], const f32x4 W[4], u32x2 neg_ident) {
  u32x2 hi[4], lo[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) hi[r] = u32x2{pack_bf16(W[r][0], W[r][1]), pack_bf16(W[r][2], W[r][3])};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const f32x4 d = mfma16(neg_ident, hi[r], W[r]);
    lo[r] = u32x2{pack_bf16(d[0], d[1]), pack_bf16(d[2], d[3])};
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) A[p] = Op8{cat(hi[2 * p], hi[2 * p + 1]), cat(lo[2 * p], lo[2 * p + 1])};
}

// A diagonal 16x16 tile diag(x_{16w + m}) as a 16x16x16 A operand: lane
// (g,c) holds A[c][4g + i], nonzero only at 4g + i == c.
__device__ __forceinline__ u32x2 diag_op(int g, int c, uint32_t bits16) {
  uint32_t e[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) e[i] = (4 * g + i == c) ? bits16 : 0u;
  return u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
}
__device__ __forceinline__ uint32_t bf16_bits(float x) { return pack_bf16(x, 0.f) & 0xffffu; }

// Row stores of z through a buffer resource covering exactly the unit's T
// rows: rows outside [0, T) fail the hardware range check and are dropped.
template <bool BF16>
struct ZOut {
  __amdgpu_buffer_rsrc_t r;
  // z == nullptr (the backward's run for the bases alone): a zero range, so
  // the hardware drops every store
  __device__ __forceinline__ ZOut(void* z, size_t row0, int T) {
    constexpr int RB = D * (BF16 ? 2 : 4);
    r = __builtin_amdgcn_make_buffer_rsrc(static_cast<char*>(z) + row0 * RB, (short)0,
                                          z ? T * RB : 0, 0x00020000);
  }
  __device__ __forceinline__ void store(int tok, int fo, f32x4 v) const {
    if (BF16) {
      const u32x2 o = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
      __builtin_amdgcn_raw_buffer_store_b64(o, r, (tok * D + fo) * 2, 0, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (tok * D + fo) * 4,
                                             0, 0);
    }
  }
};

// ---------------------------------------------------------------------------
template <bool BF16, bool LN, bool RES, bool MB16>
__device__ __forceinline__ void chain_part(LinLds<BF16>& L, const LinearArgs& a, const Ctx& x) {
  constexpr int TB = LinCfg<BF16>::TB;
  const int lane = x.lane, g = x.g, c = x.c, w = x.w, fo = x.fo, n = x.n, T = x.T;
  const int tpm = x.tpm;
  auto mbs = [&](int j) { return MB16 || (j % tpm) == 0; };
  __builtin_amdgcn_s_setprio(2);

  f32x4 gsq = {1.f, 1.f, 1.f, 1.f}, g2x2 = {2.f, 2.f, 2.f, 2.f}, twog = g2x2;
  f32x4 twogb = {0.f, 0.f, 0.f, 0.f};
  float Gam = 64.f;  // sum of gamma^2 over the features
  if (LN) {
    const float* gp = a.gamma + (size_t)x.head * D;
    const float* bp = a.beta + (size_t)x.head * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float gm = gp[fo + i];
      gsq[i] = gm * gm;
      g2x2[i] = 2.f * gsq[i];
      twog[i] = 2.f * gm;
      twogb[i] = 2.f * gm * bp[fo + i];
    }
    Gam = 0.f;
    for (int j = 0; j < D; ++j) Gam += gp[j] * gp[j];
  }
  const u32x2 ident = ident_op(g, c);
  // u^T = diag(2 gamma) (k - v)^T + 2 gamma beta on the matrix unit (bf16
  // data): diag(2 gamma) in three bf16 parts (fp32 precision: u enters the
  // gradient, and with two parts its rounding was amplified along the
  // sequence like that of the state) and their negations.
  u32x2 dph = ident, dpm = {0u, 0u}, dpl = {0u, 0u}, dnh, dnm = {0u, 0u}, dnl = {0u, 0u};
  if (LN) {
    const float t2 = 2.f * a.gamma[(size_t)x.head * D + 16 * w + c];
    const uint32_t h = bf16_bits(t2);
    const float r1 = t2 - __builtin_bit_cast(float, h << 16);
    const uint32_t m = bf16_bits(r1);
    const uint32_t l = bf16_bits(r1 - __builtin_bit_cast(float, m << 16));
    auto neg = [](uint32_t b) { return b ? (b ^ 0x8000u) : 0u; };
    dph = diag_op(g, c, h);
    dpm = diag_op(g, c, m);
    dpl = diag_op(g, c, l);
    dnh = diag_op(g, c, neg(h));
    dnm = diag_op(g, c, neg(m));
    dnl = diag_op(g, c, neg(l));
  } else {
    dnh = diag_op(g, c, 0xBF80u);  // -1
  }
  // k and v of a tile at the wave's features (raw, as staged) and u from them
  struct KV {
    u32x4 k, v;  // bf16: 4 values in .xy; fp32: 4 values
  };
  auto kv_of = [&](int blk, int tb) -> KV {
    KV r;
    if constexpr (BF16) {
      const u32x2 k4 = quad(tile_rows(L.st, 1, blk, tb), c, fo);
      const u32x2 v4 = quad(tile_rows(L.st, 2, blk, tb), c, fo);
      r.k = u32x4{k4.x, k4.y, 0u, 0u};
      r.v = u32x4{v4.x, v4.y, 0u, 0u};
    } else {
      r.k = __builtin_bit_cast(u32x4, val4(tile_rows(L.st, 1, blk, tb) + lds_off<false>(c, fo)));
      r.v = __builtin_bit_cast(u32x4, val4(tile_rows(L.st, 2, blk, tb) + lds_off<false>(c, fo)));
    }
    return r;
  };
  auto u_of = [&](const KV& kv) -> f32x4 {
    if constexpr (BF16) {
      const u32x2 k4 = {kv.k.x, kv.k.y}, v4 = {kv.v.x, kv.v.y};
      f32x4 u = LN ? twogb : f32x4{0.f, 0.f, 0.f, 0.f};
      if (RES) {
        u = mfma16(dph, k4, u);
        if (LN) {
          u = mfma16(dpm, k4, u);
          u = mfma16(dpl, k4, u);
        }
      }
      u = mfma16(dnh, v4, u);
      if (LN) {
        u = mfma16(dnm, v4, u);
        u = mfma16(dnl, v4, u);
      }
      return u;
    } else {
      const f32x4 kk = __builtin_bit_cast(f32x4, kv.k), vv = __builtin_bit_cast(f32x4, kv.v);
      f32x4 u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float kmv = (RES ? kk[i] : 0.f) - vv[i];
        u[i] = LN ? __builtin_fmaf(twog[i], kmv, twogb[i]) : kmv;
      }
      return u;
    }
  };
  // LN partial sums of one tile around its shift, reduced over the 4 lane
  // groups, into this wave's exchange slots.
  auto publish = [&](int par, f32x4 ep, f32x4 u) {
    if (!LN) return;
    f32x4 ge;
#pragma unroll
    for (int i = 0; i < 4; ++i) ge[i] = gsq[i] * ep[i];
    const float q0 = (ep[0] + ep[1]) + (ep[2] + ep[3]);
    const float q2 = (ge[0] + ge[1]) + (ge[2] + ge[3]);
    float q1 = ep[0] * ep[0], q3 = ge[0] * ep[0], q4 = u[0] * ep[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      q1 = __builtin_fmaf(ep[i], ep[i], q1);
      q3 = __builtin_fmaf(ge[i], ep[i], q3);
      q4 = __builtin_fmaf(u[i], ep[i], q4);
    }
    reinterpret_cast<float*>(&L.xc[par][w][c])[rs4_slot(g)] =
        group_reduce_scatter4(q0, q1, q2, q3);
    reinterpret_cast<float*>(&L.xu[par][c])[w] = group_sum(q4);
  };

  lds_barrier();  // A: block 0 staged, constants published
  lds_barrier();  // B: inputs of tiles 0 and 1 published
  f32x4 ep, uc = u_of(kv_of(0, 0));
  float su;       // sum_f u_f of the current tile
  {
    const f32x4 h = L.bkb[0][w][lane];
    const f32x2 tk = L.tkb[0][c];
#pragma unroll
    for (int i = 0; i < 4; ++i) ep[i] = LN ? h[i] - tk.x : h[i];
    su = tk.y;
    publish(0, ep, uc);
  }
  lds_barrier();  // period 0 starts
  u32x4 gtm1 = {};   // (-eta G_{p-1})^T as [hi, mid]
  u32x4 glhm1 = {};  // and as [lo, hi]

  for (int blk = 0; blk * TB <= n + 2; ++blk) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int p = blk * TB + tb;
      if (p > n + 2) break;
      // ---- every LDS read of the period first, so that their latencies
      //      overlap: the exchanged sums of tile p and the inputs of tile
      //      p+1 prepared in the last period.  They are issued in the order
      //      of first use (the groups held in place by scheduling barriers),
      //      so the LN coefficients wait only for the sums: LDS reads return
      //      in order, and the compiler waits for a count, not for all.
      f32x4 xs[4], su4;
      if (LN) {
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) xs[ww] = L.xc[p & 1][ww][c];
        su4 = L.xu[p & 1][c];
      }
      const float eta = tile_eta(L.st, blk, tb, c);
      __builtin_amdgcn_sched_barrier(0);
      const f32x4 bk = L.bkb[(p - 1) & 1][w][lane];  // K_{p+1} W_{p-2}
      const ScoreOps s2 = read_score(L.grp[(p - 1) & 1][1], lane);  // K_{p-1} K_{p+1}^T
      __builtin_amdgcn_sched_barrier(0);
      const KV kvn = kv_of(blk, tb + 1);
      const ScoreOps s1 = read_score(L.grp[(p - 1) & 1][0], lane);  // K_p K_{p+1}^T
      const f32x2 tk = L.tkb[(p - 1) & 1][c];
      __builtin_amdgcn_sched_barrier(0);
      // ---- independent of tile p's gradient: u of tile p+1, the
      //      correction of K_{p+1} W_{p-2} by tile p-1
      const f32x4 un = u_of(kvn);
      const bool keep2 = MB16 || mbs(p + 1) || mbs(p);
      f32x4 h = corr6(zero_unless(keep2, gtm1), zero_unless(keep2, glhm1), s2, bk);
      // ---- gradient of tile p (zero for rows past T, so past the end the
      //      update of W is a no-op)
      u32x4 gt, glh;
      {
        // rows past T: eta taken as zero, so their gradient is zero
        const float etav = p * 16 + c < T ? eta : 0.f;
        f32x4 eg;
        if (LN) {
          const f32x4 S = (xs[0] + xs[1]) + (xs[2] + xs[3]);
          const float S4 = (su4[0] + su4[1]) + (su4[2] + su4[3]);
          const float mr = S[0] * (1.0f / D);
          const float var = __builtin_fmaf(-mr, mr, S[1] * (1.0f / D));
          const float rs = __frsqrt_rn(var + a.eps);
          const float sge = __builtin_fmaf(-mr, Gam, S[2]);
          const float sue = __builtin_fmaf(-mr, su, S4);
          const float sge2 = __builtin_fmaf(mr * mr, Gam, __builtin_fmaf(-2.f * mr, S[2], S[3]));
          const float ma = __builtin_fmaf(2.f * rs, sge, su) * (1.0f / D);
          const float mx = __builtin_fmaf(2.f * rs, sge2, sue) * (rs * (1.0f / D));
          const float c1 = -etav * rs, c2 = c1 * rs;
          const float b0 = -c1 * ma, c2mx = -c2 * mx;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float A = __builtin_fmaf(c2, g2x2[i], c2mx);
            eg[i] = __builtin_fmaf(A, ep[i] - mr, __builtin_fmaf(c1, uc[i], b0));
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) eg[i] = -2.f * etav * (ep[i] + uc[i]);
        }
        // three bf16 parts, each transposed on the matrix unit (exact)
        const Split4x3 s = split4x3(eg);
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        const f32x4 th = mfma16(s.hi, ident, zero);
        const f32x4 tm = mfma16(s.mid, ident, zero);
        const f32x4 tl = mfma16(s.lo, ident, zero);
        gt = u32x4{pack_bf16(th[0], th[1]), pack_bf16(th[2], th[3]), pack_bf16(tm[0], tm[1]),
                   pack_bf16(tm[2], tm[3])};
        glh = u32x4{pack_bf16(tl[0], tl[1]), pack_bf16(tl[2], tl[3]), gt.x, gt.y};
      }
      L.gtb[p & 1][w][lane] = gt;
      L.gtl[p & 1][w][lane] = u32x2{glh.x, glh.y};
      // ---- gradient point of tile p+1 and its LN sums (at p >= n-1 the
      //      tile does not exist: stale rows, unused)
      {
        const bool keep1 = MB16 || mbs(p + 1);
        h = corr6(zero_unless(keep1, gt), zero_unless(keep1, glh), s1, h);
#pragma unroll
        for (int i = 0; i < 4; ++i) ep[i] = LN ? h[i] - tk.x : h[i];
        uc = un;
        su = tk.y;
        publish((p + 1) & 1, ep, uc);
      }
      gtm1 = gt;
      glhm1 = glh;
      lds_barrier();
    }
  }
}

// ---------------------------------------------------------------------------
// Update waves: the state, every product with it, the output correction,
// the column-independent inputs of the chain (one wave each), and the copy
// of the first input block (the output waves issue the later ones).  Every
// row operand of a period is read once, at its start.  SPLIT: the output
// side (q products and output correction) is left to the unit's second
// workgroup, and q is not staged.
template <bool BF16, bool LN, bool RES, bool MB16, bool SPLIT>
__device__ __forceinline__ void update_part(LinLds<BF16>& L, const LinearArgs& a, const Ctx& x) {
  constexpr int TB = LinCfg<BF16>::TB;
  constexpr bool LO = !BF16;
  const int lane = x.lane, g = x.g, c = x.c, w = x.w, n = x.n, T = x.T;
  const int tpm = x.tpm;
  auto mbs = [&](int j) { return MB16 || (j % tpm) == 0; };

  // Wc[r] lane (g,c) = W[feat(r, 4g + i)][16w + c]
  f32x4 Wc[4];
  const float* w0 = a.w0 + (size_t)(a.state0_per_batch ? x.unit : x.head) * D * D;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) Wc[r][i] = w0[feat(r, 4 * g + i) * D + 16 * w + c];
  float s2gb = 0.f;  // sum_f 2 gamma beta
  if (LN) {
    const float* gp = a.gamma + (size_t)x.head * D;
    const float* bp = a.beta + (size_t)x.head * D;
    for (int j = 0; j < D; ++j) s2gb += 2.f * gp[j] * bp[j];
    // constant rows of the dot-product operands, in three bf16 parts: w_bar
    // (wave 0) and 2 gamma (wave 1)
    if (w < 2) {
      float v;
      if (w == 0) {
        v = 0.f;
        for (int j = 0; j < D; ++j) v += w0[lane * D + j];
        v *= 1.0f / D;
      } else {
        v = 2.f * gp[lane];
      }
      const uint32_t h = bf16_bits(v);
      const float r1 = v - __builtin_bit_cast(float, h << 16);
      const uint32_t m = bf16_bits(r1);
      L.cst[w][lane] = (uint16_t)h;
      L.cst[w + 2][lane] = (uint16_t)m;
      L.cst[w + 4][lane] = (uint16_t)bf16_bits(r1 - __builtin_bit_cast(float, m << 16));
      L.cst[w + 6][lane] = 0;
    }
  }
  // "tile -1": no update and no output correction in period 0
  L.gtb[1][w][lane] = u32x4{0u, 0u, 0u, 0u};
  L.gtl[1][w][lane] = u32x2{0u, 0u};
  if (w == 2) {
    L.mqb[1][lane] = u32x4{0u, 0u, 0u, 0u};
    if (lane < 16) L.mqm[1][lane] = 0.f;
  }
  // The tiles past the end are read from stale staging rows (their
  // gradient is zero, but 0 * Inf would not be): buffer 1 starts as zeros
  // in case the sequence never loads it.
  {
    constexpr int N16 = sizeof(L.st.qkv[1]) / 16;
    const int t = threadIdx.x - 256;
    u32x4* b1 = reinterpret_cast<u32x4*>(&L.st.qkv[1][0][0]);
    for (int i = t; i < N16; i += 256) b1[i] = u32x4{0u, 0u, 0u, 0u};
    for (int i = t; i < TB * 16; i += 256) L.st.eta[1][i] = 0.f;
  }
  const u32x2 neg_ident = diag_op(g, c, 0xBF80u);  // -1 on the diagonal
  bool causal[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) causal[i] = (4 * g + i) <= c;

  stage_issue<BF16, TB>(L.st, SPLIT ? nullptr : a.q, a.k, a.v, a.eta, x.row0, 0, T, 0, w);
  wait_vmem();
  lds_barrier();  // A
  // A operands of the dot products with the constant rows: [w_bar, 2 gamma]
  // x [hi, mid] (ast) and [w_bar lo, 2 gamma lo, 0, 0] (ast3)
  u32x4 ast[2] = {}, ast3[2] = {};
  if (LN) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      ast[p] = *reinterpret_cast<const u32x4*>(&L.cst[c & 3][32 * p + 8 * g]);
      ast3[p] = *reinterpret_cast<const u32x4*>(&L.cst[4 + (c & 3)][32 * p + 8 * g]);
    }
  }
  // (k . w_bar, sum_f u_f) of a tile from its rows of k and v (the sum of u
  // with 2 gamma in three parts)
  auto token_inputs = [&](const Rows& kr, const Rows& vr) -> f32x2 {
    const f32x4 sk = stats<LO>(ast, kr);
    const f32x4 sv = stats<LO>(ast, vr);
    const f32x4 sk3 = stats<false>(ast3, kr);
    const f32x4 sv3 = stats<false>(ast3, vr);
    const float su = ((RES ? (sk[1] + sk[3]) + sk3[1] : 0.f) - ((sv[1] + sv[3]) + sv3[1])) + s2gb;
    return f32x2{sk[0] + sk[2], su};
  };
  // the state as [hi, mid] (Ac: also the two parts of the output product)
  // and lo (Al); Ab, Abl: the mini-batch base (b > 16)
  Op8 Ac[2], Ab[2];
  u32x4 Al[2], Abl[2];
  split_state3(Ac, Al, Wc);
  if (!MB16) {
    Ab[0] = Ac[0];
    Ab[1] = Ac[1];
    Abl[0] = Al[0];
    Abl[1] = Al[1];
  }
  // rows of K_p and K_{p+1}, carried from the period that loaded them as
  // the rows of K_{p+2}
  Rows kc0 = rows8<BF16>(tile_rows(L.st, 1, 0, 0), c, g);
  Rows kc1 = rows8<BF16>(tile_rows(L.st, 1, 0, 1), c, g);
  L.bkb[0][w][lane] = times_state3<LO>(Ac, Al, kc0);
  L.bkb[1][w][lane] = times_state3<LO>(Ac, Al, kc1);
  if (w == 0) {
    write_score(L.grp[1][0], lane, score_ops(split4x3(gram<LO>(kc0, kc1))));
  } else if (w == 1) {
    write_score(L.grp[1][1], lane, ScoreOps{});
  } else if (w == 3 && LN) {
    L.tkb[0][c] = token_inputs(kc0, rows8<BF16>(tile_rows(L.st, 2, 0, 0), c, g));
    L.tkb[1][c] = token_inputs(kc1, rows8<BF16>(tile_rows(L.st, 2, 0, 1), c, g));
  }
  lds_barrier();  // B
  lds_barrier();  // period 0 starts

  // the update waves' work of a period is the longest: they go first
  __builtin_amdgcn_s_setprio(3);
  Op4 kt1[4] = {};                   // K_{p-1}^T (16x16x16 A operands)
  f32x4 qw1 = {0.f, 0.f, 0.f, 0.f};  // (Q_{p-1} W_{p-2})^T
  for (int blk = 0; blk * TB <= n + 2; ++blk) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int p = blk * TB + tb;
      if (p > n + 2) break;
      // Start the period's work 192 cycles late (bf16 data): the chain
      // waves' serial work then meets fewer of these matrix products on its
      // SIMD.  (B4 H32 T8192: about 2 % faster than no delay, 0.5 % faster
      // than 256 cycles; 320 cycles or more make this wave's work the longer
      // path.)
      if constexpr (BF16) __builtin_amdgcn_s_sleep(3);
      // every LDS read of the period first
      const auto* Kp = tile_rows(L.st, 1, blk, tb);
      const u32x4 g1 = L.gtb[(p - 1) & 1][w][lane];  // (-eta G_{p-1})^T as [hi, mid]
      const u32x2 gl1 = L.gtl[(p - 1) & 1][w][lane];  // and lo
      // rows of q_p, k_{p+2}, v_{p+2}: read here for bf16 data; for fp32
      // data (hi/lo rows, twice the registers) just before their first use
      Rows qr = {}, kn, vn;
      auto read_q = [&] {
        if constexpr (!SPLIT) qr = rows8<BF16>(tile_rows(L.st, 0, blk, tb), c, g);
      };
      auto read_kn = [&] { kn = rows8<BF16>(tile_rows(L.st, 1, blk, tb + 2), c, g); };
      auto read_vn = [&] {
        if (w == 3 && LN) vn = rows8<BF16>(tile_rows(L.st, 2, blk, tb + 2), c, g);
      };
      if constexpr (BF16) {
        read_q();
        read_kn();
        read_vn();
      }
      u32x4 mq = {};     // tril(K_{p-1} Q_{p-1}^T)
      float muq1 = 0.f;  // q . w_bar, tile p-1
      if constexpr (!SPLIT) {
        mq = L.mqb[(p - 1) & 1][lane];
        if (LN) muq1 = L.mqm[(p - 1) & 1][c];
      }
      const Split4 m1 = {hi_of(mq), lo_of(mq)};
      // rows of K_p and K_{p+1}: carried from the period that read them as
      // K_{p+2} (bf16 data), re-read where used (fp32 data, whose hi/lo rows
      // would not fit in the registers besides the state)
      Rows k0, k1;
      if constexpr (BF16) {
        k0 = kc0;
        k1 = kc1;
      } else {
        if (w == 1 || (!SPLIT && w == 2)) k0 = rows8<BF16>(Kp, c, g);
        if (w == 0) k1 = rows8<BF16>(tile_rows(L.st, 1, blk, tb + 1), c, g);
      }
      __builtin_amdgcn_sched_barrier(0);
      // ---- output pre-activation of tile p-1 around its shift:
      //      (Q W_{p-2})^T + (-eta G_{p-1})^T tril(K Q^T) - q . w_bar
      if constexpr (!SPLIT) {
        f32x4 d = mfma16(hi_of(g1), m1.hi, f32x4{0.f, 0.f, 0.f, 0.f});
        d = mfma16(lo_of(g1), m1.hi, d);
        if (LO) d = mfma16(hi_of(g1), m1.lo, d);
        f32x4 e;
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = (qw1[i] + d[i]) - muq1;
        L.hqb[p & 1][w][lane] = e;
      }
      // ---- W += K_{p-1}^T (-eta G_{p-1}), the gradient in three parts
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        Wc[r] = mfma16(kt1[r].hi, hi_of(g1), Wc[r]);
        Wc[r] = mfma16(kt1[r].hi, mid_of(g1), Wc[r]);
        Wc[r] = mfma16(kt1[r].hi, gl1, Wc[r]);
        if (LO) Wc[r] = mfma16(kt1[r].lo, hi_of(g1), Wc[r]);
      }
      split_state_mm3(Ac, Al, Wc, neg_ident);  // W_{p-1}
      // with b = 16 this is the base of tile p: stored for the backward
      if (a.bases && p < n) {
        float* bp = a.bases + ((size_t)x.unit * n + p) * D * D;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int i = 0; i < 4; ++i) bp[feat(r, 4 * g + i) * D + 16 * w + c] = Wc[r][i];
      }
      if (!MB16 && mbs(p)) {
        Ab[0] = Ac[0];
        Ab[1] = Ac[1];
        Abl[0] = Al[0];
        Abl[1] = Al[1];
      }
      // ---- products of W_{p-1} (past the end: stale rows, unused)
      if constexpr (!BF16) {
        read_q();
        read_kn();
      }
      if constexpr (!SPLIT) qw1 = times_state<LO>(Ac, qr);
      {
        // gradient point two tiles ahead: K_{p+2} W_{p-1}, or the
        // mini-batch's own gradient point when no update reaches it
        f32x4 bk;
        if (MB16 || mbs(p + 2) || mbs(p + 1)) bk = times_state3<LO>(Ac, Al, kn);
        else bk = times_state3<LO>(Ab, Abl, kn);
        L.bkb[p & 1][w][lane] = bk;
      }
      // ---- tile p: its output score tile and shift, for every update
      //      wave in the next period (one wave: they do not depend on the
      //      column block)
      if (!SPLIT && w == 2) {
        f32x4 M = gram<LO>(k0, qr);  // K_p Q_p^T
#pragma unroll
        for (int i = 0; i < 4; ++i) M[i] = causal[i] ? M[i] : 0.f;
        L.mqb[p & 1][lane] = LO ? hilo(split4(M))
                                : u32x4{pack_bf16(M[0], M[1]), pack_bf16(M[2], M[3]), 0u, 0u};
        if (LN) {
          const f32x4 sq = stats<LO>(ast, qr);
          if (g == 0) L.mqm[p & 1][c] = sq[0] + sq[2];
        }
      }
      // ---- column-independent inputs of tile p+2 for the chain, one wave
      //      each: the score tiles K_{p+1} K_{p+2}^T, K_p K_{p+2}^T and
      //      (k . w_bar, sum_f u_f)
      if (w == 0) {
        write_score(L.grp[p & 1][0], lane, score_ops(split4x3(gram<LO>(k1, kn))));
      } else if (w == 1) {
        write_score(L.grp[p & 1][1], lane, score_ops(split4x3(gram<LO>(k0, kn))));
      } else if (w == 3 && LN) {
        if constexpr (!BF16) read_vn();
        L.tkb[p & 1][c] = token_inputs(kn, vn);
      }
      // ---- K_p^T for the next update
      if constexpr (BF16) {
        // half of a row operand times the identity is the transposed 16x16
        // block, whose rows are the state's features feat(r, c)
        const u32x2 ident = ident_op(g, c);
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const u32x4 h = k0.p[r >> 1].hi;
          const f32x4 t = mfma16((r & 1) ? u32x2{h.z, h.w} : u32x2{h.x, h.y}, ident, zero);
          kt1[r] = Op4{u32x2{pack_bf16(t[0], t[1]), pack_bf16(t[2], t[3])}, u32x2{0u, 0u}};
        }
      } else {
        cols8<BF16>(kt1, Kp, c, g);
      }
      if constexpr (BF16) {
        kc0 = kc1;
        kc1 = kn;
      }
      lds_barrier();
    }
  }

  if (a.w_out) {
    float* wo = a.w_out + (size_t)x.unit * D * D;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) wo[feat(r, 4 * g + i) * D + 16 * w + c] = Wc[r][i];
  }
}

// ---------------------------------------------------------------------------
// Output waves: output LN and z.  Period p receives the pre-activation of
// tile p-2 (around its shift), exchanges its LN sums, and stores z of tile
// p-3.  With COPIES they also issue the input copies of the later blocks.
template <bool BF16, bool LN, bool RES, bool COPIES, class Lds>
__device__ __forceinline__ void output_part(Lds& L, const LinearArgs& a, const Ctx& x) {
  constexpr int TB = Lds::TB;
  const int lane = x.lane, g = x.g, c = x.c, w = x.w, fo = x.fo, n = x.n, T = x.T;

  f32x4 gam = {1.f, 1.f, 1.f, 1.f}, bet = {0.f, 0.f, 0.f, 0.f};
  if (LN) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gam[i] = a.gamma[(size_t)x.head * D + fo + i];
      bet[i] = a.beta[(size_t)x.head * D + fo + i];
    }
  }
  L.hqb[1][w][lane] = f32x4{0.f, 0.f, 0.f, 0.f};  // "tile -2"
  const u32x2 ident = ident_op(g, c);
  const ZOut<BF16> zo(a.z, x.row0, T);

  lds_barrier();  // A
  lds_barrier();  // B
  lds_barrier();  // period 0 starts

  // q + beta (the residual part of z) of tiles p-1, p-2 and p-3; the
  // pre-activation of tile p-3 around its shift
  f32x4 qb1 = {0.f, 0.f, 0.f, 0.f}, qb2 = qb1, qb3 = qb1, eq3 = qb1;
  constexpr int PARTS = TB >= 7 ? 4 : 1;  // periods over which a refill is issued
  for (int blk = 0; blk * TB <= n + 2; ++blk) {
    const bool next_block = (blk + 1) * TB < n;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int p = blk * TB + tb;
      if (p > n + 2) break;
      // refill the other buffer (nobody reads tiles before p any more), a
      // part per period so that no period carries all the copy instructions
      if (COPIES && tb < PARTS && next_block)
        stage_issue<BF16, TB>(L.st, a.q, a.k, a.v, a.eta, x.row0, blk + 1, T, (blk + 1) & 1, w,
                              tb, PARTS);
      // every LDS read of the period first
      const f32x4 e = L.hqb[(p - 1) & 1][w][lane];  // tile p-2
      f32x4 s01 = {}, s23 = {};
      if (LN) {
        s01 = *reinterpret_cast<const f32x4*>(&L.xo[(p - 1) & 1][c][0]);
        s23 = *reinterpret_cast<const f32x4*>(&L.xo[(p - 1) & 1][c][2]);
      }
      const auto* Qp = tile_rows(L.st, 0, blk, tb);
      u32x2 q4 = {0u, 0u};
      f32x4 qv = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BF16) q4 = quad(Qp, c, fo);
      else qv = val4(Qp + lds_off<false>(c, fo));
      __builtin_amdgcn_sched_barrier(0);
      if (LN) {
        // ---- z of tile p-3 (its LN sums came with the last barrier)
        const f32x4 s = s01 + s23;
        const float mr = (s[0] + s[2]) * (1.0f / D);
        const float var = __builtin_fmaf(-mr, mr, (s[1] + s[3]) * (1.0f / D));
        const float rs = __frsqrt_rn(var + a.eps);
        f32x4 zf;
#pragma unroll
        for (int i = 0; i < 4; ++i) zf[i] = __builtin_fmaf(gam[i] * rs, eq3[i] - mr, qb3[i]);
        zo.store((p - 3) * 16 + c, fo, zf);
        // ---- LN sums of tile p-2
        const float q6 = (e[0] + e[1]) + (e[2] + e[3]);
        float q7 = e[0] * e[0];
#pragma unroll
        for (int i = 1; i < 4; ++i) q7 = __builtin_fmaf(e[i], e[i], q7);
        const float t = swap32_sum(q6, q7);
        // groups 0, 1 hold the sum of q6, groups 2, 3 that of q7
        reinterpret_cast<float*>(&L.xo[p & 1][c][w])[g >> 1] = swap16_sum(t, t);
      } else {
        zo.store((p - 2) * 16 + c, fo, qb2 + e);
      }
      eq3 = e;
      qb3 = qb2;
      qb2 = qb1;
      // ---- q + beta of tile p (past the end: stale rows, unused)
      if constexpr (BF16) {
        qb1 = RES ? mfma16(ident, q4, bet) : bet;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) qb1[i] = (RES ? qv[i] : 0.f) + bet[i];
      }
      // the next block must be visible by the barrier that opens the period
      // reading its first tile two ahead; until then the copies stay in
      // flight across the barriers
      if constexpr (COPIES) {
        if (tb == TB - 3 && next_block) wait_vmem();
        lds_barrier_copies_in_flight();
      } else {
        lds_barrier();
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Split units: two workgroups per (batch, head) unit.  The first (the chain
// workgroup) runs the chain and update waves as above without the output
// side; it publishes every tile's (-eta G)^T to a gradient stream in device
// memory.  The second (the output workgroup, on another CU) replays the
// state updates from that stream and forms the outputs.  Only the output
// workgroup ever waits for the other, so the pair cannot deadlock.
//
// Gradient stream of a unit (6 KB per tile, n tiles): tile t, column block
// b, lane l at byte ((4 t + b) * 64 + l) * 16, the [hi, mid] bf16 pairs of
// the chain's gtb; then, from byte 4096 n, tile t, column-block pair j,
// lane l at byte 4096 n + ((2 t + j) * 64 + l) * 16, the lo parts (gtl) of
// column blocks 2j and 2j+1.
// Publication: wave h (0, 1) of the chain workgroup's hand-off pair owns
// column blocks 2h, 2h+1 and a counter of complete tiles.

constexpr int KLAG = 3;              // periods between a tile's stores and its publication
constexpr uint32_t SC1 = 16;         // cache policy: agent-coherent access
constexpr int SPIN_LIMIT = 1 << 21;  // polls (about 1 us each) before giving up

// Chain workgroup, waves 8-9: the copies of k, v and eta for the blocks
// after the first (two of the four shares each).
template <bool BF16>
__device__ __forceinline__ void feed_copy_part(LinLds<BF16>& L, const LinearArgs& a,
                                               const Ctx& x, int cw) {
  constexpr int TB = LinCfg<BF16>::TB;
  constexpr int PARTS = TB >= 7 ? 4 : 1;
  const int n = x.n, T = x.T;
  lds_barrier();  // A
  lds_barrier();  // B
  lds_barrier();  // period 0 starts
  for (int blk = 0; blk * TB <= n + 2; ++blk) {
    const bool next_block = (blk + 1) * TB < n;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int p = blk * TB + tb;
      if (p > n + 2) break;
      if (tb < PARTS && next_block) {
#pragma unroll
        for (int sh = 0; sh < 2; ++sh)
          stage_issue<BF16, TB>(L.st, nullptr, a.k, a.v, a.eta, x.row0, blk + 1, T,
                                (blk + 1) & 1, 2 * cw + sh, tb, PARTS);
      }
      if (tb == TB - 3 && next_block) wait_vmem();
      lds_barrier_copies_in_flight();
    }
  }
}

// Chain workgroup, waves 10-11: the hand-off.  In period p the gradient of
// tile p-1 (published by the chain waves at the barrier that opened the
// period) goes from LDS to the stream with agent-coherent stores.  This
// wave issues no other memory instruction, and its vector memory counter
// retires stores in order, so after the three stores of tile p-1 the stores
// of tile p-1-KLAG are complete once at most 4 KLAG instructions remain
// outstanding (three stores and one counter store per later period); the
// counter then publishes tiles 0 .. p-1-KLAG.  The lag keeps the wait from
// ever holding the barrier.
template <bool BF16>
__device__ __forceinline__ void handoff_part(LinLds<BF16>& L, const LinearArgs& a, const Ctx& x,
                                             int h) {
  static_assert(KLAG == 3, "the vmcnt below is 4 KLAG");
  const int lane = x.lane, n = x.n;
  const __amdgpu_buffer_rsrc_t gs = __builtin_amdgcn_make_buffer_rsrc(
      a.ws_g + (size_t)x.unit * n * 1536, (short)0, n * 6144, 0x00020000);
  uint32_t* cnt = a.ws_flags + ((size_t)x.unit * 2 + h) * 32;
  lds_barrier();  // A
  lds_barrier();  // B
  lds_barrier();  // period 0 starts
  for (int p = 0; p <= n + 2; ++p) {
    if (p >= 1 && p - 1 < n) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int b = 2 * h + j;
        const u32x4 v = L.gtb[(p - 1) & 1][b][lane];
        __builtin_amdgcn_raw_buffer_store_b128(v, gs, (((p - 1) * 4 + b) * 64 + lane) * 16, 0, SC1);
      }
      const u32x4 lo = cat(L.gtl[(p - 1) & 1][2 * h][lane], L.gtl[(p - 1) & 1][2 * h + 1][lane]);
      __builtin_amdgcn_raw_buffer_store_b128(lo, gs, n * 4096 + (((p - 1) * 2 + h) * 64 + lane) * 16,
                                             0, SC1);
      asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
      if (lane == 0)
        __hip_atomic_store(cnt, (uint32_t)max(p - KLAG, 0), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    lds_barrier();
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (lane == 0) __hip_atomic_store(cnt, (uint32_t)n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Output workgroup, waves 0-3: the state, replayed from the gradient stream,
// and the output pre-activation of every tile, as the update waves of the
// one-workgroup kernel form them (same periods, same products).
template <bool BF16, bool LN, bool RES>
__device__ __forceinline__ void out_state_part(OutLds<BF16>& L, const LinearArgs& a,
                                               const Ctx& x) {
  constexpr int TB = OutLds<BF16>::TB;
  constexpr bool LO = !BF16;
  const int lane = x.lane, g = x.g, c = x.c, w = x.w, n = x.n;

  f32x4 Wc[4];  // lane (g,c) of tile r: W[feat(r, 4g + i)][16w + c]
  const float* w0 = a.w0 + (size_t)(a.state0_per_batch ? x.unit : x.head) * D * D;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) Wc[r][i] = w0[feat(r, 4 * g + i) * D + 16 * w + c];
  if (LN && w < 2) {
    // constant rows of the dot-product operand: w_bar (wave 0), 2 gamma (wave 1)
    float v;
    if (w == 0) {
      v = 0.f;
      for (int j = 0; j < D; ++j) v += w0[lane * D + j];
      v *= 1.0f / D;
    } else {
      v = 2.f * a.gamma[(size_t)x.head * D + lane];
    }
    const uint32_t h = bf16_bits(v);
    L.cst[w][lane] = (uint16_t)h;
    L.cst[w + 2][lane] = (uint16_t)bf16_bits(v - __builtin_bit_cast(float, h << 16));
  }
  if (w == 2) {  // "tile -1": no output correction in period 0
    L.mqb[1][lane] = u32x4{0u, 0u, 0u, 0u};
    if (lane < 16) L.mqm[1][lane] = 0.f;
  }
  {
    // the tiles past the end are read from stale staging rows: buffer 1
    // starts as zeros in case the sequence never loads it
    constexpr int N16 = sizeof(L.st.qkv[1]) / 16;
    u32x4* b1 = reinterpret_cast<u32x4*>(&L.st.qkv[1][0][0]);
    for (int i = threadIdx.x; i < N16; i += 256) b1[i] = u32x4{0u, 0u, 0u, 0u};
  }
  const u32x2 neg_ident = diag_op(g, c, 0xBF80u);
  bool causal[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) causal[i] = (4 * g + i) <= c;

  lds_barrier();  // A: block 0 of q, k and of the gradient stream staged
  u32x4 ast[2] = {};
  if (LN) {
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
      ast[pp] = *reinterpret_cast<const u32x4*>(&L.cst[c & 3][32 * pp + 8 * g]);
  }
  lds_barrier();  // B
  lds_barrier();  // period 0 starts

  Op4 kt1[4] = {};                   // K_{p-1}^T (16x16x16 A operands)
  f32x4 qw1 = {0.f, 0.f, 0.f, 0.f};  // (Q_{p-1} W_{p-2})^T
  Op8 Ac[2];
  for (int blk = 0; blk * TB <= n + 2; ++blk) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int p = blk * TB + tb;
      if (p > n + 2) break;
      // every LDS read of the period first: (-eta G_{p-1})^T (zero before
      // the first tile and past the last), the rows of tile p, the output
      // score tile and shift of tile p-1
      const int tp = max(p - 1, 0);
      const bool live = p >= 1 && p - 1 < n;
      const u32x4 g1 = zero_unless(live, L.gst[(tp / TB) & 1][tp % TB][w][lane]);
      const u32x4 gl2 = L.gsl[(tp / TB) & 1][tp % TB][w >> 1][lane];
      const u32x2 gl1 = zero_unless(live, (w & 1) ? u32x2{gl2.z, gl2.w} : u32x2{gl2.x, gl2.y});
      const auto* Kp = tile_rows(L.st, 1, blk, tb);
      const Rows qr = rows8<BF16>(tile_rows(L.st, 0, blk, tb), c, g);
      const Rows kr = rows8<BF16>(Kp, c, g);
      const u32x4 mq = L.mqb[(p - 1) & 1][lane];
      const float muq1 = LN ? L.mqm[(p - 1) & 1][c] : 0.f;
      const Split4 m1 = {hi_of(mq), lo_of(mq)};
      __builtin_amdgcn_sched_barrier(0);
      // ---- output pre-activation of tile p-1 around its shift
      {
        f32x4 d = mfma16(hi_of(g1), m1.hi, f32x4{0.f, 0.f, 0.f, 0.f});
        d = mfma16(lo_of(g1), m1.hi, d);
        if (LO) d = mfma16(hi_of(g1), m1.lo, d);
        f32x4 e;
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = (qw1[i] + d[i]) - muq1;
        L.hqb[p & 1][w][lane] = e;
      }
      // ---- W += K_{p-1}^T (-eta G_{p-1}), the gradient in three parts
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        Wc[r] = mfma16(kt1[r].hi, hi_of(g1), Wc[r]);
        Wc[r] = mfma16(kt1[r].hi, mid_of(g1), Wc[r]);
        Wc[r] = mfma16(kt1[r].hi, gl1, Wc[r]);
        if (LO) Wc[r] = mfma16(kt1[r].lo, hi_of(g1), Wc[r]);
      }
      split_state_mm(Ac, Wc, neg_ident);  // W_{p-1} as [hi, mid], as the update waves form it
      qw1 = times_state<LO>(Ac, qr);      // past the end: stale rows, unused
      // ---- tile p: output score tile and shift for the next period
      if (w == 2) {
        f32x4 M = gram<LO>(kr, qr);  // K_p Q_p^T
#pragma unroll
        for (int i = 0; i < 4; ++i) M[i] = causal[i] ? M[i] : 0.f;
        L.mqb[p & 1][lane] = LO ? hilo(split4(M))
                                : u32x4{pack_bf16(M[0], M[1]), pack_bf16(M[2], M[3]), 0u, 0u};
        if (LN) {
          const f32x4 sq = stats<LO>(ast, qr);
          if (g == 0) L.mqm[p & 1][c] = sq[0] + sq[2];
        }
      }
      // ---- K_p^T for the next update
      if constexpr (BF16) {
        const u32x2 ident = ident_op(g, c);
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const u32x4 hh = kr.p[r >> 1].hi;
          const f32x4 t = mfma16((r & 1) ? u32x2{hh.z, hh.w} : u32x2{hh.x, hh.y}, ident, zero);
          kt1[r] = Op4{u32x2{pack_bf16(t[0], t[1]), pack_bf16(t[2], t[3])}, u32x2{0u, 0u}};
        }
      } else {
        cols8<BF16>(kt1, Kp, c, g);
      }
      lds_barrier();
    }
  }
}

// Output workgroup, waves 8-11: copies of q and k, and of the gradient
// stream once the chain workgroup has published it.  Block b of the stream
// is copied in period 1 of block b-1 (nobody reads its buffer after period
// 0 of that block) and waited for, with q and k, by the end of block b-1.
// If the chain workgroup does not publish within the spin limit (about two
// seconds; a block takes microseconds), this and every later block is
// filled with NaN instead and an error word is set, so that the failure
// shows in z.
template <bool BF16>
__device__ __forceinline__ void out_copy_part(OutLds<BF16>& L, const LinearArgs& a,
                                              const Ctx& x, int cw) {
  constexpr int TB = OutLds<BF16>::TB;
  constexpr int PARTS = TB >= 7 ? 4 : 1;
  const int lane = x.lane, n = x.n, T = x.T;
  const uint32_t* gsrc = a.ws_g + (size_t)x.unit * n * 1536;
  const uint32_t* lsrc = gsrc + (size_t)n * 1024;  // lo parts
  bool ok = true;  // cleared for good by a spin that reaches the limit
  auto stage_grad = [&](int b, int buf) {
    const uint32_t need = (uint32_t)min(n, (b + 1) * TB);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t* f = a.ws_flags + ((size_t)x.unit * 2 + h) * 32;
      int spins = 0;
      while (ok && __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
        if (++spins > SPIN_LIMIT) ok = false;
        __builtin_amdgcn_s_sleep(2);
      }
    }
    const u32x4 nan4 = {0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
    for (int i = cw; i < TB; i += 4) {
      const int t = min(b * TB + i, n - 1);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        if (ok) {
          TTT_LDS void* dst = (TTT_LDS void*)&L.gst[buf][i][cb][0];
          __builtin_amdgcn_global_load_lds(gsrc + ((size_t)(4 * t + cb) * 64 + lane) * 4, dst, 16,
                                           0, SC1);
        } else {
          L.gst[buf][i][cb][lane] = nan4;
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (ok) {
          TTT_LDS void* dst = (TTT_LDS void*)&L.gsl[buf][i][j][0];
          __builtin_amdgcn_global_load_lds(lsrc + ((size_t)(2 * t + j) * 64 + lane) * 4, dst, 16,
                                           0, SC1);
        } else {
          L.gsl[buf][i][j][lane] = nan4;
        }
      }
    }
    if (!ok && lane == 0) a.ws_flags[(size_t)a.B * a.H * 64] = 1u;
  };
  stage_issue<BF16, TB>(L.st, a.q, a.k, nullptr, nullptr, x.row0, 0, T, 0, cw);
  stage_grad(0, 0);
  wait_vmem();
  lds_barrier();  // A
  lds_barrier();  // B
  lds_barrier();  // period 0 starts
  for (int blk = 0; blk * TB <= n + 2; ++blk) {
    const bool next_block = (blk + 1) * TB < n;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int p = blk * TB + tb;
      if (p > n + 2) break;
      if (tb < PARTS && next_block)
        stage_issue<BF16, TB>(L.st, a.q, a.k, nullptr, nullptr, x.row0, blk + 1, T,
                              (blk + 1) & 1, cw, tb, PARTS);
      if (tb == 1 && next_block) stage_grad(blk + 1, (blk + 1) & 1);
      if (tb == TB - 1 && next_block) wait_vmem();
      lds_barrier_copies_in_flight();
    }
  }
}

template <bool BF16, bool LN, bool RES, bool MB16, bool SPLIT>
__global__ __launch_bounds__(NT, 1) void ttt_linear_fwd(LinearArgs a) {
  Ctx x;
  const int tid = threadIdx.x;
  // the wave index is uniform across a wave: keep it (and the branches on
  // the wave's role) scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int units = a.B * a.H;
  const bool out_wg = SPLIT && (int)blockIdx.x >= units;
  x.lane = tid & 63;
  x.g = x.lane >> 4;
  x.c = x.lane & 15;
  x.w = wave & 3;
  x.fo = 16 * x.w + 4 * x.g;
  x.unit = out_wg ? (int)blockIdx.x - units : (int)blockIdx.x;
  x.head = x.unit % a.H;
  x.T = a.T;
  x.n = (a.T + 15) / 16;
  x.tpm = MB16 ? 1 : a.tiles_per_mb;
  x.row0 = (size_t)x.unit * a.T;
  if constexpr (!SPLIT) {
    __shared__ LinLds<BF16> L;
    if (wave < 4) chain_part<BF16, LN, RES, MB16>(L, a, x);
    else if (wave < 8) update_part<BF16, LN, RES, MB16, false>(L, a, x);
    else output_part<BF16, LN, RES, true>(L, a, x);
  } else {
    __shared__ SplitLds<BF16> S;
    if (!out_wg) {
      if (wave < 4) chain_part<BF16, LN, RES, MB16>(S.c, a, x);
      else if (wave < 8) update_part<BF16, LN, RES, MB16, true>(S.c, a, x);
      else if (wave < 10) feed_copy_part<BF16>(S.c, a, x, wave - 8);
      else handoff_part<BF16>(S.c, a, x, wave - 10);
    } else {
      if (wave < 4) out_state_part<BF16, LN, RES>(S.o, a, x);
      else if (wave < 8) output_part<BF16, LN, RES, false>(S.o, a, x);
      else out_copy_part<BF16>(S.o, a, x, wave - 8);
    }
  }
}

__global__ void zero_words(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

template <bool BF16, bool LN, bool RES, bool SPLIT>
hipError_t launch4(const LinearArgs& a, hipStream_t s) {
  const int units = a.B * a.H;
  const dim3 grid(SPLIT ? 2 * units : units), block(NT);
  if (SPLIT) {
    // publication counters and error words start at zero (a fill kernel
    // rather than a memset, so that the launch can be captured in a graph)
    const int words = units * 64 + 32;
    hipLaunchKernelGGL(zero_words, dim3((words + 255) / 256), dim3(256), 0, s, a.ws_flags, words);
  }
  if (a.tiles_per_mb == 1)
    hipLaunchKernelGGL((ttt_linear_fwd<BF16, LN, RES, true, SPLIT>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((ttt_linear_fwd<BF16, LN, RES, false, SPLIT>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <bool BF16, bool LN, bool RES>
hipError_t launch3(const LinearArgs& a, hipStream_t s) {
  return a.split ? launch4<BF16, LN, RES, true>(a, s) : launch4<BF16, LN, RES, false>(a, s);
}

template <bool BF16>
hipError_t launch1(const LinearArgs& a, bool ln, bool res, hipStream_t s) {
  if (ln) return res ? launch3<BF16, true, true>(a, s) : launch3<BF16, true, false>(a, s);
  return res ? launch3<BF16, false, true>(a, s) : launch3<BF16, false, false>(a, s);
}

// Scratch of the no-allocation split launch: gradient stream and counters
// in one fixed array per device, for callers that cannot allocate.
constexpr uint64_t SCRATCH_BYTES = 128ull << 20;
static __device__ __align__(256) uint8_t scratch[SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[MAX_DEVICES] = {};

}  // namespace

const uint64_t kLinearScratchBytes = SCRATCH_BYTES;

hipError_t linear_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    // the array's name is a host-side stand-in: its device address on the
    // current device comes from the runtime, once per device
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    scratch_ptr[dev] = p;
  }
  *ptr = scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_linear(const LinearArgs& a, bool bf16, bool ln, bool residual,
                         hipStream_t stream) {
  return bf16 ? launch1<true>(a, ln, residual, stream) : launch1<false>(a, ln, residual, stream);
}

}  // namespace tttk
