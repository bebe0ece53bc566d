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
// Mapping onto one CU: one 512-thread workgroup per (batch, head) unit.
//   * Waves 4-7 ("state" waves) keep W[:, 16w:16w+16] as four 16x16 fp32
//     MFMA accumulators.  In period t they apply the update of tile t-1,
//     split W_{t-1} into bf16 hi/lo, and form Q_t W_{t-1} (output of tile
//     t) and K_{t+2} W_{t-1} (gradient point two tiles ahead).
//   * Waves 0-3 ("chain" waves) own the same column blocks and run the
//     serial part: they bring K_{t+1} W_{t-2} up to date with the two
//     updates it misses, K_{t+1} W_t = K_{t+1} W_{t-2}
//     + (K_{t+1} K_{t-1}^T)(-eta G_{t-1}) + (K_{t+1} K_t^T)(-eta G_t), of
//     which only the last 16x16 correction waits for tile t's gradient.  The
//     serial path per tile is: correction -> LN sums -> one exchange among
//     the chain waves -> gradient -> transpose.  Off that path the chain
//     waves also finish the outputs (tril(K Q^T) correction, output LN, z).
//   * A chain wave and a state wave share each SIMD, so one fills the issue
//     slots while the other waits on the barrier, the LDS or the matrix
//     unit; the chain waves run at a higher wave priority.
//   * H is produced transposed (H^T = W^T K^T): a lane holds 4 features of
//     ONE token, so LN row sums are in-lane adds plus a reduce-scatter over
//     the 4 lane groups (v_permlane16/32_swap).
//   * LN sums are taken around the shift k . w_bar with w_bar = W0 1 / d: the
//     LN gradient of every token sums to zero over the features, so W 1 is a
//     constant of the scan and k . w_bar is the exact row mean up to
//     rounding.  The shift comes out of the matrix unit.
//   * fp32 operands enter the bf16 matrix unit as hi + lo bf16 pairs (about
//     16 significant bits); bf16 inputs are exact.  hi and lo terms share
//     16x16x32 products where the 8 operand slots allow it.  The output
//     correction of bf16 data uses the hi part of the score tile only: its
//     error does not feed back into the state.
//   * Row m of the state's accumulator tile r holds input feature
//     32 (r/2) + 8 (m/4) + 4 (r%2) + m%4, so the 8 contraction slots of a
//     lane in a 16x16x32 product with W are 8 consecutive features: every
//     row operand (K, Q, w_bar) is a single 16-byte LDS read.
//   * Accumulate chains never mix the 16x16x32 and 16x16x16 shapes: on this
//     toolchain a result of one shape fed back to back as the C operand of
//     the other came out wrong in two of its four registers.
//   * q, k, v, eta stream from HBM to LDS in blocks of TB tiles
//     (global_load_lds, double-buffered), issued by the state waves.
//   * One barrier per tile orders every exchange: the chain's LN sums,
//     -eta G (chain -> state), Q_t W_{t-1} and K_{t+2} W_{t-1}
//     (state -> chain).  Both loops are free of branches within a tile;
//     tiles past the end compute on stale rows with their gradient forced
//     to zero, and z stores past the end are dropped by the buffer range
//     check.
#include "ttt_device.hpp"
#include "ttt_kernels.hpp"
#include "ttt_tile.hpp"

namespace tttk {
namespace {

constexpr int NT = 512;  // 4 chain waves + 4 state waves

template <bool BF16>
struct LinCfg {
  static constexpr int TB = BF16 ? 8 : 4;  // tiles per staged block (16 KB per tensor)
};

template <bool BF16>
struct LinLds {
  Stage<BF16, LinCfg<BF16>::TB> st;
  // chain LN partial sums [parity][wave][round][token][quantity]: the 16
  // tokens of one (wave, round) are 16 consecutive 16-byte rows, so the
  // readers (lane c reads token c) hit distinct banks.
  f32x4 xc[2][4][2][16];
  u32x4 gtb[2][4][64];  // (-eta G_t)^T operand, chain wave -> state wave
  f32x4 qwb[2][4][64];  // (Q_t W_{t-1})^T, state wave -> chain wave
  f32x4 bkb[2][4][64];  // (K_{t+2} W_{t-1})^T, state wave -> chain wave
  float wbar[D];        // W0 1 / d
};

struct Ctx {
  int lane, g, c, w, fo;  // w: column block (wave mod 4); fo = 16 w + 4 g
  int unit, head, T, n, tpm;
  size_t row0;            // first row of the unit in [B*H*T, 64]
};

// Staged rows of the tile `tb` tiles after the first tile of block `blk`
// (tb may run past the block, into the other buffer).
template <bool BF16, int TB>
__device__ __forceinline__ const typename Io<BF16>::E* tile_rows(const Stage<BF16, TB>& st,
                                                                 int x, int blk, int tb) {
  return st.qkv[(blk + tb / TB) & 1][x] + (tb % TB) * 16 * D;
}
template <bool BF16, int TB>
__device__ __forceinline__ float tile_eta(const Stage<BF16, TB>& st, int blk, int tb, int c) {
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
      const Split4 a = split4(*reinterpret_cast<const f32x4*>(X + lds_off<false>(c, 32 * p + 8 * g)));
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

__device__ __forceinline__ u32x4 zero_unless(bool keep, u32x4 x) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  return keep ? x : z;
}
__device__ __forceinline__ u32x2 hi_of(u32x4 g) { return u32x2{g.x, g.y}; }
__device__ __forceinline__ u32x2 lo_of(u32x4 g) { return u32x2{g.z, g.w}; }

// acc + (-eta G)^T S for a score tile S (tokens x tokens, accumulator
// layout, split into bf16 hi/lo) and G given as [hi, lo]: the hi*hi, lo*hi
// and hi*lo terms as a chain of 16x16x16 products on sub-operands of the
// two tuples (no register moves; acc may be a value loaded from LDS).
__device__ __forceinline__ f32x4 corr(u32x4 gt, const Split4& s, f32x4 acc) {
  acc = mfma16(hi_of(gt), s.hi, acc);
  acc = mfma16(lo_of(gt), s.hi, acc);
  acc = mfma16(hi_of(gt), s.lo, acc);
  return acc;
}

// w_bar as 16x16x32 A operands (every row the same, slots as in rows8):
// mfma(wbar, rows of X) gives x . w_bar for each token of X in every
// register of its lane.
__device__ __forceinline__ void wbar_ops(const float* wb, int g, u32x4 op[2]) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const f32x4 m0 = *reinterpret_cast<const f32x4*>(&wb[32 * p + 8 * g]);
    const f32x4 m1 = *reinterpret_cast<const f32x4*>(&wb[32 * p + 8 * g + 4]);
    op[p] = split_pair(m0, m1).hi;  // a shift need not be exact
  }
}
__device__ __forceinline__ float shift_of(const u32x4 wb[2], const Rows& x) {
  f32x4 m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < 2; ++p) m = mfma32(wb[p], x.p[p].hi, m);
  return m[0];
}

// Row stores of z through a buffer resource covering exactly the unit's T
// rows: rows outside [0, T) fail the hardware range check and are dropped.
template <bool BF16>
struct ZOut {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ ZOut(void* z, size_t row0, int T) {
    constexpr int RB = D * (BF16 ? 2 : 4);
    r = __builtin_amdgcn_make_buffer_rsrc(static_cast<char*>(z) + row0 * RB, (short)0, T * RB,
                                          0x00020000);
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
// Chain waves.  The inputs of tile j's gradient that do not depend on the
// scan are prepared two periods ahead.
struct Prep {
  f32x4 u;     // LN: 2 gamma (k - v) + 2 gamma beta, else k - v (no k without residual)
  float su;    // in-lane sum of u
  float mu;    // k . w_bar
  Split4 p1;   // K_{j-1} K_j^T, bf16 hi/lo
  Split4 p2;   // K_{j-2} K_j^T
};

template <bool BF16, bool LN, bool RES>
__device__ __forceinline__ Prep prepare(const typename Io<BF16>::E* Kj,
                                        const typename Io<BF16>::E* Vj, const Rows& km1,
                                        const Rows& km2, const u32x4 wb[2], f32x4 twog,
                                        f32x4 twogb, int c, int g, int fo) {
  constexpr bool LO = !BF16;
  Prep r;
  const f32x4 kv = val4(Kj + lds_off<BF16>(c, fo));
  const f32x4 vv = val4(Vj + lds_off<BF16>(c, fo));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float kmv = (RES ? kv[i] : 0.f) - vv[i];
    r.u[i] = LN ? __builtin_fmaf(twog[i], kmv, twogb[i]) : kmv;
  }
  r.su = (r.u[0] + r.u[1]) + (r.u[2] + r.u[3]);
  const Rows kj = rows8<BF16>(Kj, c, g);
  r.mu = LN ? shift_of(wb, kj) : 0.f;
  r.p1 = split4(gram<LO>(km1, kj));
  r.p2 = split4(gram<LO>(km2, kj));
  return r;
}

template <bool BF16, bool LN, bool RES, bool MB16>
__device__ __forceinline__ void chain_part(LinLds<BF16>& L, const LinearArgs& a, const Ctx& x) {
  constexpr int TB = LinCfg<BF16>::TB;
  constexpr bool LO = !BF16;
  using E = typename Io<BF16>::E;
  const int lane = x.lane, g = x.g, c = x.c, w = x.w, fo = x.fo, n = x.n, T = x.T;
  const int tpm = x.tpm;
  auto mbs = [&](int j) { return MB16 || (j % tpm) == 0; };
  __builtin_amdgcn_s_setprio(2);

  f32x4 gam = {1.f, 1.f, 1.f, 1.f}, bet = {0.f, 0.f, 0.f, 0.f};
  f32x4 gsq = gam, g2x2 = {2.f, 2.f, 2.f, 2.f}, twog = g2x2, twogb = bet;
  float Gam = 64.f;  // sum of gamma^2 over the features
  if (LN) {
    const float* gp = a.gamma + (size_t)x.head * D;
    const float* bp = a.beta + (size_t)x.head * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gam[i] = gp[fo + i];
      bet[i] = bp[fo + i];
      gsq[i] = gam[i] * gam[i];
      g2x2[i] = 2.f * gsq[i];
      twog[i] = 2.f * gam[i];
      twogb[i] = 2.f * gam[i] * bet[i];
    }
    Gam = 0.f;
    for (int j = 0; j < D; ++j) Gam += gp[j] * gp[j];
  }
  const u32x2 ident = ident_op(g, c);
  bool causal[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) causal[i] = (4 * g + i) <= c;
  const ZOut<BF16> zo(a.z, x.row0, T);

  lds_barrier();  // A: block 0 staged, w_bar published
  u32x4 wb[2] = {};
  if (LN) wbar_ops(L.wbar, g, wb);
  const Rows k0 = rows8<BF16>(tile_rows(L.st, 1, 0, 0), c, g);
  const Prep p0 = prepare<BF16, LN, RES>(tile_rows(L.st, 1, 0, 0), tile_rows(L.st, 2, 0, 0), k0,
                                         k0, wb, twog, twogb, c, g, fo);
  Prep nx = prepare<BF16, LN, RES>(tile_rows(L.st, 1, 0, 1), tile_rows(L.st, 2, 0, 1), k0, k0,
                                   wb, twog, twogb, c, g, fo);
  lds_barrier();  // B: K_0 W0 and K_1 W0 published by the state waves
  f32x4 ep, uc = p0.u;
  {
    const f32x4 h = L.bkb[0][w][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) ep[i] = h[i] - p0.mu;
    if (LN) {
      f32x4 ge;
#pragma unroll
      for (int i = 0; i < 4; ++i) ge[i] = gsq[i] * ep[i];
      const float q0 = (ep[0] + ep[1]) + (ep[2] + ep[3]);
      const float q2 = (ge[0] + ge[1]) + (ge[2] + ge[3]);
      float q1 = ep[0] * ep[0], q3 = ge[0] * ep[0], q4 = uc[0] * ep[0];
#pragma unroll
      for (int i = 1; i < 4; ++i) {
        q1 = __builtin_fmaf(ep[i], ep[i], q1);
        q3 = __builtin_fmaf(ge[i], ep[i], q3);
        q4 = __builtin_fmaf(uc[i], ep[i], q4);
      }
      reinterpret_cast<float*>(&L.xc[0][w][0][c])[rs4_slot(g)] =
          group_reduce_scatter4(q0, q1, q2, q3);
      reinterpret_cast<float*>(&L.xc[0][w][1][c])[rs4_slot(g)] =
          group_reduce_scatter4(q4, p0.su, 0.f, 0.f);
    }
  }
  lds_barrier();  // period 0 starts

  // carried from period to period (p is the current period)
  u32x4 gtm1 = {};                        // (-eta G_{p-1})^T as [hi, lo]
  Split4 m1 = {};                         // tril(K_{p-1} Q_{p-1}^T) (hi only for bf16 data)
  float muq1 = 0.f;                       // q . w_bar, tile p-1
  f32x4 qb1 = {0.f, 0.f, 0.f, 0.f};       // q + beta (residual part of z), tile p-1
  f32x4 qb2 = qb1, eq2 = qb1;             // tile p-2: q + beta, centred H_q

  for (int blk = 0; blk * TB <= n + 1; ++blk) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int p = blk * TB + tb;
      if (p > n + 1) break;
      f32x4 s1 = {0.f, 0.f, 0.f, 0.f}, s2 = s1;
      if (LN) {
        s1 = L.xc[p & 1][0][0][c];
        s2 = L.xc[p & 1][0][1][c];
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) {
          s1 += L.xc[p & 1][ww][0][c];
          s2 += L.xc[p & 1][ww][1][c];
        }
      }
      // ---- gradient of tile p (zero for rows past T, so past the end the
      //      state waves' update is a no-op)
      u32x4 gt;
      {
        const float eta = tile_eta(L.st, blk, tb, c);
        const bool valid = p * 16 + c < T;
        f32x4 eg;
        if (LN) {
          const float mr = s1[0] * (1.0f / D);
          const float var = __builtin_fmaf(-mr, mr, s1[1] * (1.0f / D));
          const float rs = __frsqrt_rn(var + a.eps);
          const float sge = __builtin_fmaf(-mr, Gam, s1[2]);
          const float sue = __builtin_fmaf(-mr, s2[1], s2[0]);
          const float sge2 = __builtin_fmaf(mr * mr, Gam, __builtin_fmaf(-2.f * mr, s1[2], s1[3]));
          const float ma = (s2[1] + 2.f * rs * sge) * (1.0f / D);
          const float mx = (rs * sue + 2.f * rs * rs * sge2) * (1.0f / D);
          const float c1 = -eta * rs, c2 = -eta * rs * rs;
          const float b0 = -c1 * ma, c2mx = -c2 * mx;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float A = __builtin_fmaf(c2, g2x2[i], c2mx);
            eg[i] = __builtin_fmaf(A, ep[i] - mr, __builtin_fmaf(c1, uc[i], b0));
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) eg[i] = -2.f * eta * (ep[i] + uc[i]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) eg[i] = valid ? eg[i] : 0.f;
        const Split4 s = split4(eg);
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        const f32x4 th = mfma16(s.hi, ident, zero);
        const f32x4 tl = mfma16(s.lo, ident, zero);
        gt = u32x4{pack_bf16(th[0], th[1]), pack_bf16(th[2], th[3]), pack_bf16(tl[0], tl[1]),
                   pack_bf16(tl[2], tl[3])};
      }
      L.gtb[p & 1][w][lane] = gt;

      // ---- z of tile p-2 (its output LN sums came with this exchange)
      if (LN) {
        const float mr = s2[2] * (1.0f / D);
        const float var = __builtin_fmaf(-mr, mr, s2[3] * (1.0f / D));
        const float rs = __frsqrt_rn(var + a.eps);
        f32x4 zf;
#pragma unroll
        for (int i = 0; i < 4; ++i) zf[i] = __builtin_fmaf(gam[i] * rs, eq2[i] - mr, qb2[i]);
        zo.store((p - 2) * 16 + c, fo, zf);
      }
      // ---- output pre-activation of tile p-1:
      //      H_q^T = (Q W_{p-2})^T + (-eta G_{p-1})^T tril(K Q^T)
      f32x4 eq = {0.f, 0.f, 0.f, 0.f};
      {
        f32x4 hq = L.qwb[(p - 1) & 1][w][lane];
        hq = mfma16(hi_of(gtm1), m1.hi, hq);
        hq = mfma16(lo_of(gtm1), m1.hi, hq);
        if (LO) hq = mfma16(hi_of(gtm1), m1.lo, hq);
        if (LN) {
#pragma unroll
          for (int i = 0; i < 4; ++i) eq[i] = hq[i] - muq1;
        } else {
          zo.store((p - 1) * 16 + c, fo, qb1 + hq);
        }
      }
      // ---- gradient point of tile p+1 and the exchange of its LN sums
      //      (with the output sums of tile p-1)
      {
        f32x4 h = L.bkb[(p - 1) & 1][w][lane];  // K_{p+1} W_{p-2}
        h = corr(zero_unless(MB16 || mbs(p + 1) || mbs(p), gtm1), nx.p2, h);
        h = corr(zero_unless(MB16 || mbs(p + 1), gt), nx.p1, h);
#pragma unroll
        for (int i = 0; i < 4; ++i) ep[i] = h[i] - nx.mu;
        uc = nx.u;
        if (LN) {
          f32x4 ge;
#pragma unroll
          for (int i = 0; i < 4; ++i) ge[i] = gsq[i] * ep[i];
          const float q0 = (ep[0] + ep[1]) + (ep[2] + ep[3]);
          const float q2 = (ge[0] + ge[1]) + (ge[2] + ge[3]);
          const float q6 = (eq[0] + eq[1]) + (eq[2] + eq[3]);
          float q1 = ep[0] * ep[0], q3 = ge[0] * ep[0], q4 = uc[0] * ep[0], q7 = eq[0] * eq[0];
#pragma unroll
          for (int i = 1; i < 4; ++i) {
            q1 = __builtin_fmaf(ep[i], ep[i], q1);
            q3 = __builtin_fmaf(ge[i], ep[i], q3);
            q4 = __builtin_fmaf(uc[i], ep[i], q4);
            q7 = __builtin_fmaf(eq[i], eq[i], q7);
          }
          reinterpret_cast<float*>(&L.xc[(p + 1) & 1][w][0][c])[rs4_slot(g)] =
              group_reduce_scatter4(q0, q1, q2, q3);
          reinterpret_cast<float*>(&L.xc[(p + 1) & 1][w][1][c])[rs4_slot(g)] =
              group_reduce_scatter4(q4, nx.su, q6, q7);
        }
      }
      // ---- tile p: output-side inputs; tile p+2: gradient inputs (past
      //      the end: stale rows, unused)
      {
        const E* Qp = tile_rows(L.st, 0, blk, tb);
        const Rows qr = rows8<BF16>(Qp, c, g);
        const Rows kp = rows8<BF16>(tile_rows(L.st, 1, blk, tb), c, g);
        const Rows kp1 = rows8<BF16>(tile_rows(L.st, 1, blk, tb + 1), c, g);
        f32x4 M = gram<LO>(kp, qr);  // K_p Q_p^T
#pragma unroll
        for (int i = 0; i < 4; ++i) M[i] = causal[i] ? M[i] : 0.f;
        qb2 = qb1;
        eq2 = eq;
        if (LO) m1 = split4(M);
        else m1.hi = u32x2{pack_bf16(M[0], M[1]), pack_bf16(M[2], M[3])};
        muq1 = LN ? shift_of(wb, qr) : 0.f;
        const f32x4 qv = val4(Qp + lds_off<BF16>(c, fo));
#pragma unroll
        for (int i = 0; i < 4; ++i) qb1[i] = (RES ? qv[i] : 0.f) + (LN ? bet[i] : 0.f);
        nx = prepare<BF16, LN, RES>(tile_rows(L.st, 1, blk, tb + 2),
                                    tile_rows(L.st, 2, blk, tb + 2), kp1, kp, wb, twog, twogb,
                                    c, g, fo);
      }
      gtm1 = gt;
      lds_barrier();
    }
  }
}

// ---------------------------------------------------------------------------
template <bool BF16, bool LN, bool RES, bool MB16>
__device__ __forceinline__ void state_part(LinLds<BF16>& L, const LinearArgs& a, const Ctx& x) {
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
  if (LN && w == 0) {
    float s = 0.f;
    for (int j = 0; j < D; ++j) s += w0[lane * D + j];
    L.wbar[lane] = s * (1.0f / D);
  }
  // "tile -1": no update and a zero output in period 0
  L.gtb[1][w][lane] = u32x4{0u, 0u, 0u, 0u};
  L.qwb[1][w][lane] = f32x4{0.f, 0.f, 0.f, 0.f};
  // The tiles past the end are read from stale staging rows (their
  // gradient is zero, but 0 * Inf would not be): buffer 1 starts as zeros
  // in case the sequence never loads it.
  {
    constexpr int N16 = sizeof(L.st.qkv[1]) / 16;
    u32x4* b1 = reinterpret_cast<u32x4*>(&L.st.qkv[1][0][0]);
    for (int i = threadIdx.x - 256; i < N16; i += 256) b1[i] = u32x4{0u, 0u, 0u, 0u};
    for (int i = threadIdx.x - 256; i < LinCfg<BF16>::TB * 16; i += 256) L.st.eta[1][i] = 0.f;
  }

  stage_issue<BF16, TB>(L.st, a.q, a.k, a.v, a.eta, x.row0, 0, T, 0, w);
  wait_vmem();
  lds_barrier();  // A
  Op8 Ac[2], Ab[2];
  split_state(Ac, Wc);
  if (!MB16) {
    Ab[0] = Ac[0];
    Ab[1] = Ac[1];
  }
  L.bkb[0][w][lane] = times_state<LO>(Ac, rows8<BF16>(tile_rows(L.st, 1, 0, 0), c, g));
  L.bkb[1][w][lane] = times_state<LO>(Ac, rows8<BF16>(tile_rows(L.st, 1, 0, 1), c, g));
  lds_barrier();  // B
  lds_barrier();  // period 0 starts

  Op4 kt1[4] = {};  // K_{p-1}^T (16x16x16 A operands)
  for (int blk = 0; blk * TB <= n + 1; ++blk) {
    const bool next_block = (blk + 1) * TB < n;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int p = blk * TB + tb;
      if (p > n + 1) break;
      // refill the other buffer: nobody reads tiles before p any more
      if (tb == 0 && next_block)
        stage_issue<BF16, TB>(L.st, a.q, a.k, a.v, a.eta, x.row0, blk + 1, T, (blk + 1) & 1, w);
      const u32x4 g1 = L.gtb[(p - 1) & 1][w][lane];  // (-eta G_{p-1})^T as [hi, lo]
      // ---- state update with tile p-1: W += K^T (-eta G)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        Wc[r] = mfma16(kt1[r].hi, hi_of(g1), Wc[r]);
        Wc[r] = mfma16(kt1[r].hi, lo_of(g1), Wc[r]);
        if (LO) Wc[r] = mfma16(kt1[r].lo, hi_of(g1), Wc[r]);
      }
      split_state(Ac, Wc);  // W_{p-1}
      if (!MB16 && mbs(p)) {
        Ab[0] = Ac[0];
        Ab[1] = Ac[1];
      }
      // ---- products of W_{p-1} (past the end: stale rows, unused)
      const auto* Kp = tile_rows(L.st, 1, blk, tb);
      L.qwb[p & 1][w][lane] = times_state<LO>(Ac, rows8<BF16>(tile_rows(L.st, 0, blk, tb), c, g));
      cols8<BF16>(kt1, Kp, c, g);
      {
        // gradient point two tiles ahead: K_{p+2} W_{p-1}, or the
        // mini-batch's own gradient point when no update reaches it
        const Rows kn = rows8<BF16>(tile_rows(L.st, 1, blk, tb + 2), c, g);
        f32x4 bk;
        if (MB16 || mbs(p + 2) || mbs(p + 1)) bk = times_state<LO>(Ac, kn);
        else bk = times_state<LO>(Ab, kn);
        L.bkb[p & 1][w][lane] = bk;
      }
      // the next block must be visible by the barrier that opens the period
      // reading its first tile two ahead
      if (tb == TB - 3 && next_block) wait_vmem();
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

template <bool BF16, bool LN, bool RES, bool MB16>
__global__ __launch_bounds__(NT, 1) void ttt_linear_fwd(LinearArgs a) {
  __shared__ LinLds<BF16> L;
  Ctx x;
  const int tid = threadIdx.x;
  x.lane = tid & 63;
  x.g = x.lane >> 4;
  x.c = x.lane & 15;
  x.w = (tid >> 6) & 3;
  x.fo = 16 * x.w + 4 * x.g;
  x.unit = blockIdx.x;
  x.head = x.unit % a.H;
  x.T = a.T;
  x.n = (a.T + 15) / 16;
  x.tpm = MB16 ? 1 : a.tiles_per_mb;
  x.row0 = (size_t)x.unit * a.T;
  if (tid < 256) chain_part<BF16, LN, RES, MB16>(L, a, x);
  else state_part<BF16, LN, RES, MB16>(L, a, x);
}

template <bool BF16, bool LN, bool RES>
hipError_t launch3(const LinearArgs& a, hipStream_t s) {
  const dim3 grid(a.B * a.H), block(NT);
  if (a.tiles_per_mb == 1)
    hipLaunchKernelGGL((ttt_linear_fwd<BF16, LN, RES, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((ttt_linear_fwd<BF16, LN, RES, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch1(const LinearArgs& a, bool ln, bool res, hipStream_t s) {
  if (ln) return res ? launch3<BF16, true, true>(a, s) : launch3<BF16, true, false>(a, s);
  return res ? launch3<BF16, false, true>(a, s) : launch3<BF16, false, false>(a, s);
}

}  // namespace

hipError_t launch_linear(const LinearArgs& a, bool bf16, bool ln, bool residual,
                         hipStream_t stream) {
  return bf16 ? launch1<true>(a, ln, residual, stream) : launch1<false>(a, ln, residual, stream);
}

}  // namespace tttk
