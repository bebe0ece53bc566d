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
// Mapping onto one CU:
//   * one 256-thread workgroup (4 waves, one per SIMD) per (batch, head)
//     unit; wave w owns output columns 16w..16w+15 of W, H, G and Z;
//   * the state never leaves the registers: W[:, 16w:16w+16] is four 16x16
//     fp32 MFMA accumulators per wave, updated in place by the update product;
//   * H is produced transposed (H^T = W^T K^T): a lane holds 4 features of
//     ONE token, so LN row sums are 3 in-lane adds plus a reduce-scatter over
//     the 4 lane groups (v_permlane16/32_swap);
//   * LN sums are taken around the shift k . w_bar with w_bar = W 1 / d: the
//     LN gradient of every token sums to zero over the features, so W 1 is a
//     constant of the scan and k . w_bar is the exact row mean up to rounding.
//     The shift comes out of the matrix unit (w_bar as an A operand), so no
//     serial mean pass precedes the variance;
//   * the 4 waves exchange 8 partial sums per token per tile through LDS,
//     behind ONE barrier: 6 for the gradient of tile t and 2 for the output
//     LN of tile t-1 (the output path runs one tile behind the state chain);
//   * fp32 operands enter the bf16 matrix unit as hi + lo bf16 pairs (about
//     16 significant bits); bf16 inputs are exact;
//   * q, k, v, eta stream from HBM in blocks of 8 tiles: the next block is
//     loaded into registers while the current one is processed from LDS.
#include "ttt_device.hpp"
#include "ttt_kernels.hpp"
#include "ttt_tile.hpp"

namespace tttk {
namespace {

constexpr int NT = 256;  // threads per workgroup

template <bool BF16>
struct LinCfg {
  static constexpr int TB = BF16 ? 8 : 4;  // tiles per staged block (16 KB per tensor)
};

template <bool BF16>
struct LinLds {
  Stage<BF16, LinCfg<BF16>::TB> st;
  // LN partial sums [parity][wave][round][token][quantity slot]: the 16
  // tokens of one (wave, round) are 16 consecutive 16-byte rows, so the
  // readers (lane c reads token c) hit distinct banks.
  f32x4 xch[2][4][2][16];
  float wbar[D];  // W0 1 / d
};

template <bool BF16, bool LN, bool RES, bool MB16>
__global__ __launch_bounds__(NT, 1) void ttt_linear_fwd(LinearArgs a) {
  using E = typename Io<BF16>::E;
  constexpr int TB = LinCfg<BF16>::TB;
  constexpr bool LO = !BF16;  // inputs carry a lo part (fp32 data)
  __shared__ LinLds<BF16> L;

  const int tid = threadIdx.x;
  const int w = tid >> 6;          // wave: output columns 16w..16w+15
  const int lane = tid & 63;
  const int g = lane >> 4;         // lane group
  const int c = lane & 15;         // lane column
  const int unit = blockIdx.x;     // (batch, head)
  const int head = unit % a.H;
  const int T = a.T;
  const int tpm = MB16 ? 1 : a.tiles_per_mb;
  const size_t row0 = (size_t)unit * T;
  const int fo = 16 * w + 4 * g;   // transposed tiles: lane holds token c, features fo..fo+3

  // ---- prologue ---------------------------------------------------------
  // Wc[r] lane (g,c) = W[16r + 4g + i][16w + c]
  f32x4 Wc[4];
  const float* w0 = a.w0 + (size_t)(a.state0_per_batch ? unit : head) * D * D;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) Wc[r][i] = w0[(16 * r + 4 * g + i) * D + 16 * w + c];

  f32x4 gam = {1.f, 1.f, 1.f, 1.f}, bet = {0.f, 0.f, 0.f, 0.f};
  f32x4 g2x2 = {2.f, 2.f, 2.f, 2.f}, twog = g2x2, twogb = bet;
  float Gam = 64.f;  // sum of gamma^2 over the features
  u32x4 wbar[2] = {};  // w_bar (bf16) as a 16x16x32 A operand (every row the same)
  if (LN) {
    const float* gp = a.gamma + (size_t)head * D;
    const float* bp = a.beta + (size_t)head * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gam[i] = gp[fo + i];
      bet[i] = bp[fo + i];
      g2x2[i] = 2.f * gam[i] * gam[i];
      twog[i] = 2.f * gam[i];
      twogb[i] = 2.f * gam[i] * bet[i];
    }
    Gam = 0.f;
    for (int j = 0; j < D; ++j) Gam += gp[j] * gp[j];
    if (tid < D) {
      float s = 0.f;
      for (int j = 0; j < D; ++j) s += w0[tid * D + j];
      L.wbar[tid] = s * (1.0f / D);
    }
  }
  // causal mask of the 16x16 score tile: lane holds M[s = 4g+i][t = c]
  bool causal[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) causal[i] = (4 * g + i) <= c;
  // identity as a 16x16x16 B operand: lane (g,c) holds I[4g + i][c]
  u32x2 ident;
  {
    uint32_t e[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) e[i] = (4 * g + i == c) ? 0x3F80u : 0u;
    ident = u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
  }

  const int n_tiles = (T + 15) / 16;
  stage_issue<BF16, TB>(L.st, a.q, a.k, a.v, a.eta, row0, 0, T, 0);
  wait_vmem();
  lds_barrier();
  if (LN) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const f32x4 m0 = *reinterpret_cast<const f32x4*>(&L.wbar[32 * p + 4 * g]);
      const f32x4 m1 = *reinterpret_cast<const f32x4*>(&L.wbar[32 * p + 16 + 4 * g]);
      wbar[p] = split_pair(m0, m1).hi;  // a shift need not be exact
    }
  }

  // Carried from tile to tile (t is the tile of the current iteration):
  //   Wc       state before the pending update of tile t-1 (zero at t = 0)
  //   gt, kt   the pending update of tile t-1: W -= K^T (eta G)
  //   bk       K_t times the state before that update
  //   pm       K_{t-1} K_t^T, to correct bk by the pending update
  //   mu4      K_t w_bar, the LN shift of tile t
  //   Ab       gradient point of the current mini-batch (mini-batches of
  //            several tiles; otherwise the state itself)
  // Everything for tile t+1 is formed before tile t's barrier from data
  // that does not depend on tile t's gradient, so the serial chain per tile
  // is: correction -> LN sums -> exchange -> gradient -> transpose.
  Op8 Ab[2];
  Op4 gt = {}, kt[4] = {};
  Rows kb = load_rows<BF16>(L.st.qkv[0][1], 0, c, g);
  f32x4 bk, pm = {0.f, 0.f, 0.f, 0.f}, mu4 = pm;
  split_state(Ab, Wc);
  bk = times_state<LO>(Ab, kb);
  if (LN) {
#pragma unroll
    for (int p = 0; p < 2; ++p) mu4 = mfma32(wbar[p], kb.p[p].hi, mu4);
  }
  // output path of the previous tile
  f32x4 hq_prev = {0.f, 0.f, 0.f, 0.f}, qb_prev = hq_prev;
  float muq_prev = 0.f;
  int tok_prev = -1;

  for (int blk = 0; blk * TB < n_tiles; ++blk) {
    const int buf = blk & 1;
    const bool next_block = (blk + 1) * TB < n_tiles;
    const E* Lq = L.st.qkv[buf][0];
    const E* Lk = L.st.qkv[buf][1];
    const E* Lv = L.st.qkv[buf][2];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int tile = blk * TB + tb;
      if (tile >= n_tiles) break;
      const int par = tile & 1;
      const int t0 = tb * 16;               // first row of the tile in the block
      const int tok = tile * 16 + c;
      const bool mb_start = MB16 || (tile % tpm) == 0;
      const bool mb_start_next = MB16 || ((tile + 1) % tpm) == 0;
      // the next block must be visible by the barrier of this tile, for the
      // lookahead of the block's last tile
      if (tb == TB - 2 && next_block) wait_vmem();

      // ===== [A] gradient point of tile t: K_t W_t = K_t W_{t-1} - (K_t K_{t-1}^T)(eta G)_{t-1}
      f32x4 hk = mb_start ? correct<true>(gt, pm, bk) : bk;
      const float eta = L.st.eta[buf][t0 + c];
      const f32x4 kres = val4(Lk + lds_off<BF16>(t0 + c, fo));
      const f32x4 vres = val4(Lv + lds_off<BF16>(t0 + c, fo));

      // ===== [B] independent of tile t's gradient: pending update, output
      //       products of tile t, products for tile t+1
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        Wc[r] = mfma16(kt[r].hi, gt.hi, Wc[r]);
        Wc[r] = mfma16(kt[r].hi, gt.lo, Wc[r]);
        if (LO) Wc[r] = mfma16(kt[r].lo, gt.hi, Wc[r]);
      }
      Op8 Ac[2];
      split_state(Ac, Wc);                   // W_t
      if (!MB16 && mb_start) {
        Ab[0] = Ac[0];
        Ab[1] = Ac[1];
      }
      const Rows qr = load_rows<BF16>(Lq, t0, c, g);
      const f32x4 qres = val4(Lq + lds_off<BF16>(t0 + c, fo));
      const f32x4 hqb = times_state<LO>(Ac, qr);       // (Q_t W_t)^T
      f32x4 M = gram<LO>(kb, qr);                      // K_t Q_t^T
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!causal[i]) M[i] = 0.f;
      float muq = 0.f;
      if (LN) {
        f32x4 m4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < 2; ++p) m4 = mfma32(wbar[p], qr.p[p].hi, m4);
        muq = m4[0];
      }
      load_cols<BF16>(kt, Lk, t0, c, g);              // K_t^T, for the next update
      // tile t+1 (first tile of the next buffer after the last of this block;
      // past the end the products are formed from stale data and unused)
      const bool wrap = tb == TB - 1;
      const Rows kn = load_rows<BF16>(wrap ? L.st.qkv[buf ^ 1][1] : Lk, wrap ? 0 : t0 + 16, c, g);
      const f32x4 bk_next = times_state<LO>(mb_start_next ? Ac : Ab, kn);
      const f32x4 pm_next = mb_start_next ? gram<LO>(kb, kn) : pm;
      f32x4 mu_next = {0.f, 0.f, 0.f, 0.f};
      if (LN) {
#pragma unroll
        for (int p = 0; p < 2; ++p) mu_next = mfma32(wbar[p], kn.p[p].hi, mu_next);
      }

      // ===== [C] local LN sums: gradient of tile t, output of tile t-1
      f32x4 ep = {0.f, 0.f, 0.f, 0.f}, u = ep, eq = ep;
      float S[8];
      if (LN) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ep[i] = hk[i] - mu4[0];
          u[i] = __builtin_fmaf(twog[i], (RES ? kres[i] : 0.f) - vres[i], twogb[i]);
          eq[i] = hq_prev[i] - muq_prev;
        }
        f32x4 ge;
#pragma unroll
        for (int i = 0; i < 4; ++i) ge[i] = gam[i] * gam[i] * ep[i];
        const float q0 = (ep[0] + ep[1]) + (ep[2] + ep[3]);
        const float q2 = (ge[0] + ge[1]) + (ge[2] + ge[3]);
        const float q5 = (u[0] + u[1]) + (u[2] + u[3]);
        const float q6 = (eq[0] + eq[1]) + (eq[2] + eq[3]);
        float q1 = ep[0] * ep[0], q3 = ge[0] * ep[0], q4 = u[0] * ep[0], q7 = eq[0] * eq[0];
#pragma unroll
        for (int i = 1; i < 4; ++i) {
          q1 = __builtin_fmaf(ep[i], ep[i], q1);
          q3 = __builtin_fmaf(ge[i], ep[i], q3);
          q4 = __builtin_fmaf(u[i], ep[i], q4);
          q7 = __builtin_fmaf(eq[i], eq[i], q7);
        }
        // ===== [D] exchange across the 4 waves
        const float r1 = group_reduce_scatter4(q0, q1, q2, q3);
        const float r2 = group_reduce_scatter4(q4, q5, q6, q7);
        reinterpret_cast<float*>(&L.xch[par][w][0][c])[rs4_slot(g)] = r1;
        reinterpret_cast<float*>(&L.xch[par][w][1][c])[rs4_slot(g)] = r2;
        lds_barrier();
        f32x4 s1 = {0.f, 0.f, 0.f, 0.f}, s2 = s1;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
          s1 += L.xch[par][ww][0][c];
          s2 += L.xch[par][ww][1][c];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          S[j] = s1[j];
          S[4 + j] = s2[j];
        }
      } else if (tb == TB - 2 && next_block) {
        lds_barrier();                       // publish the next block
      }

      // ===== [E] finish the previous tile's output
      {
        f32x4 zf;
        if (LN) {
          const float mr = S[6] * (1.0f / D);
          const float var = __builtin_fmaf(-mr, mr, S[7] * (1.0f / D));
          const float rs = __frsqrt_rn(var + a.eps);
#pragma unroll
          for (int i = 0; i < 4; ++i) zf[i] = __builtin_fmaf(gam[i] * rs, eq[i] - mr, qb_prev[i]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) zf[i] = qb_prev[i] + hq_prev[i];
        }
        if (tok_prev >= 0 && tok_prev < T) {
          if (BF16) {
            const u32x2 o = {pack_bf16(zf[0], zf[1]), pack_bf16(zf[2], zf[3])};
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.z) + (row0 + tok_prev) * D + fo) = o;
          } else {
            *reinterpret_cast<f32x4*>(static_cast<float*>(a.z) + (row0 + tok_prev) * D + fo) = zf;
          }
        }
      }

      // ===== [F] gradient of tile t, transposed on the matrix unit
      const bool valid = tok < T;
      f32x4 eg;
      if (LN) {
        const float mr = S[0] * (1.0f / D);
        const float var = __builtin_fmaf(-mr, mr, S[1] * (1.0f / D));
        const float rs = __frsqrt_rn(var + a.eps);
        const float sge = __builtin_fmaf(-mr, Gam, S[2]);
        const float sue = __builtin_fmaf(-mr, S[5], S[4]);
        const float sge2 = __builtin_fmaf(mr * mr, Gam, __builtin_fmaf(-2.f * mr, S[2], S[3]));
        float ma = (S[5] + 2.f * rs * sge) * (1.0f / D);
        float mx = (rs * sue + 2.f * rs * rs * sge2) * (1.0f / D);
        float c1 = -eta * rs, c2 = -eta * rs * rs;
        if (!valid) ma = mx = c1 = c2 = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = ep[i] - mr;
          eg[i] = __builtin_fmaf(c1, u[i] - ma, c2 * (e * (g2x2[i] - mx)));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          eg[i] = valid ? -2.f * eta * (hk[i] + (RES ? kres[i] : 0.f) - vres[i]) : 0.f;
      }
      {
        const Split4 s = split4(eg);
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        const f32x4 th = mfma16(s.hi, ident, zero);
        const f32x4 tl = mfma16(s.lo, ident, zero);
        gt.hi = u32x2{pack_bf16(th[0], th[1]), pack_bf16(th[2], th[3])};
        gt.lo = u32x2{pack_bf16(tl[0], tl[1]), pack_bf16(tl[2], tl[3])};
      }

      // ===== [G] output pre-activation of tile t; carry to tile t+1
      hq_prev = correct<true>(gt, M, hqb);         // H_q^T = (Q W_t)^T + (-eta G)^T tril(K Q^T)
      muq_prev = muq;
#pragma unroll
      for (int i = 0; i < 4; ++i) qb_prev[i] = (RES ? qres[i] : 0.f) + (LN ? bet[i] : 0.f);
      tok_prev = tok;
      bk = bk_next;
      pm = pm_next;
      mu4 = mu_next;
      kb = kn;

      // refill the other buffer once every wave is past the previous block
      if (tb == 0 && next_block) {
        if (!LN) lds_barrier();
        stage_issue<BF16, TB>(L.st, a.q, a.k, a.v, a.eta, row0, blk + 1, T, buf ^ 1);
      }
    }  // tiles of the block
  }

  // ---- drain: last update and the last tile's output --------------------
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    Wc[r] = mfma16(kt[r].hi, gt.hi, Wc[r]);
    Wc[r] = mfma16(kt[r].hi, gt.lo, Wc[r]);
    if (LO) Wc[r] = mfma16(kt[r].lo, gt.hi, Wc[r]);
  }
  {
    f32x4 zf;
    if (LN) {
      f32x4 eq;
#pragma unroll
      for (int i = 0; i < 4; ++i) eq[i] = hq_prev[i] - muq_prev;
      const float q6 = (eq[0] + eq[1]) + (eq[2] + eq[3]);
      float q7 = eq[0] * eq[0];
#pragma unroll
      for (int i = 1; i < 4; ++i) q7 = __builtin_fmaf(eq[i], eq[i], q7);
      const int par = n_tiles & 1;
      const float r2 = group_reduce_scatter4(0.f, 0.f, q6, q7);
      reinterpret_cast<float*>(&L.xch[par][w][1][c])[rs4_slot(g)] = r2;
      lds_barrier();
      f32x4 s2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) s2 += L.xch[par][ww][1][c];
      const float mr = s2[2] * (1.0f / D);
      const float var = __builtin_fmaf(-mr, mr, s2[3] * (1.0f / D));
      const float rs = __frsqrt_rn(var + a.eps);
#pragma unroll
      for (int i = 0; i < 4; ++i) zf[i] = __builtin_fmaf(gam[i] * rs, eq[i] - mr, qb_prev[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) zf[i] = qb_prev[i] + hq_prev[i];
    }
    if (tok_prev < T) {
      if (BF16) {
        const u32x2 o = {pack_bf16(zf[0], zf[1]), pack_bf16(zf[2], zf[3])};
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.z) + (row0 + tok_prev) * D + fo) = o;
      } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.z) + (row0 + tok_prev) * D + fo) = zf;
      }
    }
  }

  // ---- epilogue: final state ------------------------------------------
  if (a.w_out) {
    float* wo = a.w_out + (size_t)unit * D * D;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) wo[(16 * r + 4 * g + i) * D + 16 * w + c] = Wc[r][i];
  }
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
