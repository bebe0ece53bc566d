// ttt_mlp.hip -- TTT-MLP forward scan for gfx950 (MI355X).
//
// Method: the inner model is a two-layer MLP with LayerNorm and residual,
// f(x) = x + LN(GELU(x W1 + b1) W2 + b2) (codewithpapers.app record of
// arXiv 2407.04620, "abstract"; dmarx.github.io record LIT-801, "Key
// takeaways" item 5); its weights and biases are the state, updated by one
// gradient step on ||f(k; S) - v||^2 per 16-token mini-batch with the
// gradients taken at the state of the mini-batch start, and the layer emits
// z_t = f(q_t; S_t) (items 1 and 2).  GELU is the exact erf form; the
// hidden width is 4d = 256.  Per 16-token tile (rows of K, Q, V), exactly:
//     P_k = K W1 + b1,  A_k = GELU(P_k),  O_k = A_k W2 + b2
//     G_o = LN_backward(2 (K + LN(O_k) - V))              dl/dO_k
//     G_p = (G_o W2^T) * GELU'(P_k)                        dl/dP_k
//     P_q = Q W1 + b1 - tril(Q K^T + 1) (eta G_p)
//     O_q = GELU(P_q) W2 + b2 - tril(A_q A_k^T + 1) (eta G_o)
//     Z   = Q + LN(O_q)
//     W1 -= K^T (eta G_p),  b1 -= 1^T (eta G_p),
//     W2 -= A_k^T (eta G_o), b2 -= 1^T (eta G_o)
// (the "+ 1" terms are the bias updates seen by later tokens of the tile).
//
// Mapping onto one CU:
//   * one 256-thread workgroup (4 waves) per (batch, head) unit; wave w owns
//     hidden units 64w..64w+63: W1[:, 64w:64w+64], b1[64w:64w+64] and
//     W2[64w:64w+64, :] stay in fp32 MFMA accumulator registers for the
//     whole sequence (the biases as 16x16 tiles with equal columns, updated
//     by a product with an all-ones operand);
//   * the hidden pre-activations are produced transposed (lane: 4 hidden
//     units of one token), the output pre-activations as per-wave partial
//     sums over the wave's hidden units, added across waves in LDS; wave w
//     then owns output features 16w..16w+15 for the LayerNorm, whose row
//     sums are exchanged once per LN;
//   * W2 is needed with either index contracted (A_k W2 and G_o W2^T): the
//     W2^T operand is made each tile by a transpose on the matrix unit;
//   * with bf16 inputs the products take plain bf16 operands (state kept in
//     fp32); with fp32 inputs every operand is a bf16 hi + lo pair.
#include <math.h>

#include "ttt_device.hpp"
#include "ttt_kernels.hpp"
#include "ttt_tile.hpp"

namespace tttk {
namespace {

constexpr int NT = 256;   // threads per workgroup
constexpr int MH = 256;   // hidden width
constexpr int TBM = 4;    // tiles per staged block

template <bool BF16>
struct MlpLds {
  Stage<BF16, TBM> st;
  f32x4 part[4][4][64];   // per-wave partial O^T tiles [wave][feature tile][lane]
  f32x4 xch[4][2][16];    // LN partial sums [wave][round][token]
  u32x4 gath[4][2][64];   // -eta G_o of each wave's feature tile: [wave][layout][lane]
};

// erf-form GELU and its derivative: GELU(x) = x Phi(x),
// GELU'(x) = Phi(x) + x phi(x), Phi(x) = (1 + erf(x / sqrt 2)) / 2.
__device__ __forceinline__ void gelu2(float x, float& y, float& dy) {
  const float ph = 0.5f * (1.0f + erff(x * 0.70710678118654752f));
  y = x * ph;
  dy = ph + x * 0.39894228040143268f * expf(-0.5f * x * x);
}
__device__ __forceinline__ float gelu(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}

// Sums over 16 features of each token in the LN layout (lane (g,c): token
// c, features 4g+i of the wave's tile), combined across the 4 waves through
// LDS with local centring.  Returns, per token, the mean, 1/sigma and the
// two means the LN backward needs (when `bwd`):
//   ma = mean(gamma gy), mx = mean(gamma gy xhat) with gy = u + 2 gamma^2 xhat.
struct LnStat {
  float mean, rs, ma, mx;
};
template <bool BWD>
__device__ __forceinline__ LnStat ln_stats(f32x4 (&xch)[4][2][16], f32x4 h, f32x4 u,
                                           f32x4 gam2, const float (&Gam)[4], float eps, int w,
                                           int g, int c) {
  const float s1 = group_sum(h[0] + h[1] + h[2] + h[3]);
  const float mw = s1 * (1.0f / 16.0f);
  f32x4 e;
  float P = 0.f, A = 0.f, Bq = 0.f, C = 0.f, U = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    e[i] = h[i] - mw;
    P += e[i] * e[i];
    if (BWD) {
      A += gam2[i] * e[i];
      Bq += u[i] * e[i];
      C += gam2[i] * e[i] * e[i];
      U += u[i];
    }
  }
  P = group_sum(P);
  if (BWD) {
    A = group_sum(A);
    Bq = group_sum(Bq);
    C = group_sum(C);
    U = group_sum(U);
  }
  if (g == 0) {
    xch[w][0][c] = f32x4{s1, P, A, Bq};
    xch[w][1][c] = f32x4{C, U, 0.f, 0.f};
  }
  lds_barrier();
  f32x4 s0[4], s1v[4];
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) {
    s0[ww] = xch[ww][0][c];
    s1v[ww] = xch[ww][1][c];
  }
  const float mu = (s0[0][0] + s0[1][0] + s0[2][0] + s0[3][0]) * (1.0f / 64.0f);
  float M2 = 0.f, SgE = 0.f, SuE = 0.f, SgE2 = 0.f, Su = 0.f;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) {
    const float dl = s0[ww][0] * (1.0f / 16.0f) - mu;   // local mean - mean
    M2 += s0[ww][1] + 16.0f * dl * dl;
    if (BWD) {
      SgE += s0[ww][2] + dl * Gam[ww];
      SuE += s0[ww][3] + dl * s1v[ww][1];
      SgE2 += s1v[ww][0] + 2.0f * dl * s0[ww][2] + dl * dl * Gam[ww];
      Su += s1v[ww][1];
    }
  }
  LnStat r;
  r.mean = mu;
  r.rs = __frsqrt_rn(M2 * (1.0f / 64.0f) + eps);
  r.ma = (Su + 2.0f * r.rs * SgE) * (1.0f / 64.0f);
  r.mx = (r.rs * SuE + 2.0f * r.rs * r.rs * SgE2) * (1.0f / 64.0f);
  return r;
}

template <bool BF16, bool LN, bool RES>
__global__ __launch_bounds__(NT, 1) void ttt_mlp_fwd(MlpArgs a) {
  using E = typename Io<BF16>::E;
  constexpr bool SP = !BF16;  // hi + lo operands
  __shared__ MlpLds<BF16> L;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int c = lane & 15;
  const int unit = blockIdx.x;
  const int head = unit % a.H;
  const int T = a.T;
  const size_t row0 = (size_t)unit * T;
  const int HB = 64 * w;          // the wave's hidden units
  const int fo = 16 * w + 4 * g;  // LN layout: lane holds token c, features fo..fo+3
  const size_t s0 = a.state0_per_batch ? (size_t)unit : (size_t)head;

  // ---- state --------------------------------------------------------------
  // W1c[r][n] lane (g,c) = W1[16r + 4g + i][HB + 16n + c]
  // W2c[n][f] lane (g,c) = W2[HB + 16n + 4g + i][16f + c]
  // b1v[n]    lane (g,c) = b1[HB + 16n + 4g + i]      (any c)
  // b2w       lane (g,c) = b2[16w + 4g + i]           (any c)
  f32x4 W1c[4][4], W2c[4][4], b1v[4], b2w;
  {
    const float* w1 = a.w1 + s0 * D * MH;
    const float* w2 = a.w2 + s0 * MH * D;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          W1c[r][n][i] = w1[(16 * r + 4 * g + i) * MH + HB + 16 * n + c];
          W2c[r][n][i] = w2[(HB + 16 * r + 4 * g + i) * D + 16 * n + c];
        }
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) b1v[n][i] = a.b1[s0 * MH + HB + 16 * n + 4 * g + i];
#pragma unroll
    for (int i = 0; i < 4; ++i) b2w[i] = a.b2[s0 * D + fo + i];
  }

  f32x4 gam = {1.f, 1.f, 1.f, 1.f}, bet = {0.f, 0.f, 0.f, 0.f}, gam2 = gam;
  float Gam[4] = {16.f, 16.f, 16.f, 16.f};
  if (LN) {
    const float* gp = a.gamma + (size_t)head * D;
    const float* bp = a.beta + (size_t)head * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gam[i] = gp[fo + i];
      bet[i] = bp[fo + i];
      gam2[i] = gam[i] * gam[i];
    }
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      float s = 0.f;
      for (int j = 0; j < 16; ++j) s += gp[16 * ww + j] * gp[16 * ww + j];
      Gam[ww] = s;
    }
  }
  bool causal[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) causal[i] = (4 * g + i) <= c;
  const u32x2 ident = ident_op(g, c);
  const Op4 ones = {ones_op(), u32x2{0u, 0u}};

  const int n_tiles = (T + 15) / 16;
  stage_issue<BF16, TBM>(L.st, a.q, a.k, a.v, a.eta, row0, 0, T, 0, tid >> 6);
  wait_vmem();
  lds_barrier();

  for (int tile = 0; tile < n_tiles; ++tile) {
    const int blk = tile / TBM, tb = tile % TBM, buf = blk & 1;
    const bool next_block = (blk + 1) * TBM < n_tiles;
    if (tb == 0 && next_block) {
      // every wave has passed the previous tile's barriers: the other buffer
      // (previous block) is free
      stage_issue<BF16, TBM>(L.st, a.q, a.k, a.v, a.eta, row0, blk + 1, T, buf ^ 1,
                             tid >> 6);
    }
    const E* Lq = L.st.qkv[buf][0];
    const E* Lk = L.st.qkv[buf][1];
    const E* Lv = L.st.qkv[buf][2];
    const int t0 = tb * 16;
    const int tok = tile * 16 + c;
    const bool valid = tok < T;
    const float eta = L.st.eta[buf][t0 + c];

    const Rows kb = load_rows<BF16>(Lk, t0, c, g);
    const Rows qb = load_rows<BF16>(Lq, t0, c, g);
    Op4 kt[4];
    load_cols<BF16>(kt, Lk, t0, c, g);
    const f32x4 kres = val4(Lk + lds_off<BF16>(t0 + c, fo));
    const f32x4 vres = val4(Lv + lds_off<BF16>(t0 + c, fo));
    const f32x4 qres = val4(Lq + lds_off<BF16>(t0 + c, fo));

    // ---- hidden pre-activations (transposed: lane = token c, hidden
    //      HB + 16n + 4g + i) ------------------------------------------------
    f32x4 Pk[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      Pk[n] = b1v[n];
#pragma unroll
      for (int p = 0; p < 2; ++p)
        Pk[n] = mma8<SP, SP>(split_pair(W1c[2 * p][n], W1c[2 * p + 1][n]), kb.p[p], Pk[n]);
    }
    f32x4 Ak[4], Dk[4];
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float y, dy;
        gelu2(Pk[n][i], y, dy);
        Ak[n][i] = y;
        Dk[n][i] = dy;
      }

    // W2 as the A operand of W2^T for feature tile f, hidden tiles 2q, 2q+1:
    // slots -> hidden HB + 32q + 4g + j (j<4), HB + 32q + 16 + 4g + j - 4 (j>=4)
    auto w2op = [&](int q, int f) { return split_pair(W2c[2 * q][f], W2c[2 * q + 1][f]); };

    // ---- O_k: partial over the wave's hidden units, summed across waves --
    {
      Op8 Akop[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) Akop[q] = split_pair(Ak[2 * q], Ak[2 * q + 1]);
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 2; ++q) o = mma8<SP, SP>(w2op(q, f), Akop[q], o);
        L.part[w][f][lane] = o;
      }
    }
    lds_barrier();
    f32x4 ok = b2w;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) ok += L.part[ww][w][lane];

    // ---- dl/dO_k for the wave's 16 output features, times -eta ------------
    f32x4 ego;
    if (LN) {
      f32x4 u;
#pragma unroll
      for (int i = 0; i < 4; ++i) u[i] = 2.f * gam[i] * ((RES ? kres[i] : 0.f) + bet[i] - vres[i]);
      const LnStat st = ln_stats<true>(L.xch, ok, u, gam2, Gam, a.eps, w, g, c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float xh = (ok[i] - st.mean) * st.rs;
        const float av = u[i] + 2.f * gam2[i] * xh;
        ego[i] = valid ? -eta * st.rs * (av - st.ma - xh * st.mx) : 0.f;  // padding: exactly 0
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ego[i] = valid ? -2.f * eta * (ok[i] + (RES ? kres[i] : 0.f) - vres[i]) : 0.f;
    }

    // ---- share -eta G_o of every feature tile with every wave ---------------
    const Split4 es = split4(ego);
    const Op4 got_own = transpose_op<SP>(es, ident);   // lane: token 4g+i, feature 16w+c
    L.gath[w][0][lane] = cat(es.hi, es.lo);
    L.gath[w][1][lane] = cat(got_own.hi, got_own.lo);
    lds_barrier();
    Op4 egoL[4], got[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const u32x4 x = L.gath[f][0][lane];
      const u32x4 y = L.gath[f][1][lane];
      egoL[f] = Op4{u32x2{x[0], x[1]}, u32x2{x[2], x[3]}};  // lane: token c, feats 16f+4g+i
      got[f] = Op4{u32x2{y[0], y[1]}, u32x2{y[2], y[3]}};   // lane: token 4g+i, feat 16f+c
    }

    // ---- -eta dl/dP_k = ((-eta G_o) W2^T) * GELU'(P_k) ----------------------
    f32x4 egp[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const Op4 w2t = transpose_op<SP>(split4(W2c[n][f]), ident);  // lane: W2[HB+16n+c][16f+4g+i]
        acc = mma4<SP, SP>(w2t, egoL[f], acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) egp[n][i] = acc[i] * Dk[n][i];
    }
    Op4 gpt[4];   // lane: token 4g+i, hidden HB+16n+c
#pragma unroll
    for (int n = 0; n < 4; ++n) gpt[n] = transpose_op<SP>(split4(egp[n]), ident);

    // ---- output: P_q, A_q, O_q (state before this tile's update) ------------
    f32x4 Pq[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      Pq[n] = b1v[n];
#pragma unroll
      for (int p = 0; p < 2; ++p)
        Pq[n] = mma8<SP, SP>(split_pair(W1c[2 * p][n], W1c[2 * p + 1][n]), qb.p[p], Pq[n]);
    }
    {
      f32x4 M = gram<SP>(kb, qb);   // lane: k_{4g+i} . q_c
#pragma unroll
      for (int i = 0; i < 4; ++i) M[i] = causal[i] ? M[i] + 1.f : 0.f;
#pragma unroll
      for (int n = 0; n < 4; ++n) Pq[n] = correct<SP>(gpt[n], M, Pq[n]);
    }
    f32x4 Aq[4];
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) Aq[n][i] = gelu(Pq[n][i]);
    {
      // this wave's share of tril(A_q A_k^T + 1): lane M[s = 4g+i][t = c]
      f32x4 Ma = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const Split4 sk = split4(Ak[n]), sq = split4(Aq[n]);
        Ma = mma4<SP, SP>(Op4{sk.hi, sk.lo}, Op4{sq.hi, sq.lo}, Ma);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) Ma[i] = causal[i] ? Ma[i] + (w == 0 ? 1.f : 0.f) : 0.f;
      Op8 Aqop[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) Aqop[q] = split_pair(Aq[2 * q], Aq[2 * q + 1]);
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 2; ++q) o = mma8<SP, SP>(w2op(q, f), Aqop[q], o);
        o = correct<SP>(got[f], Ma, o);
        L.part[w][f][lane] = o;
      }
    }
    lds_barrier();
    f32x4 oq = b2w;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) oq += L.part[ww][w][lane];
    f32x4 zf;
    if (LN) {
      const f32x4 none = {0.f, 0.f, 0.f, 0.f};
      const LnStat st = ln_stats<false>(L.xch, oq, none, gam2, Gam, a.eps, w, g, c);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        zf[i] = (RES ? qres[i] : 0.f) + gam[i] * ((oq[i] - st.mean) * st.rs) + bet[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) zf[i] = (RES ? qres[i] : 0.f) + oq[i];
      lds_barrier();  // every wave has read the partials before they are rewritten
    }
    if (valid) {
      if (BF16) {
        const u32x2 o = {pack_bf16(zf[0], zf[1]), pack_bf16(zf[2], zf[3])};
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.z) + (row0 + tok) * D + fo) = o;
      } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.z) + (row0 + tok) * D + fo) = zf;
      }
    }

    // ---- state update ---------------------------------------------------------
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      Op4 akt;   // lane: token 4g+i, hidden HB+16n+c
      akt = transpose_op<SP>(split4(Ak[n]), ident);
#pragma unroll
      for (int r = 0; r < 4; ++r) W1c[r][n] = mma4<SP, SP>(kt[r], gpt[n], W1c[r][n]);
      b1v[n] = mma4<SP, false>(gpt[n], ones, b1v[n]);
#pragma unroll
      for (int f = 0; f < 4; ++f) W2c[n][f] = mma4<SP, SP>(akt, got[f], W2c[n][f]);
    }
    b2w = mma4<SP, false>(got_own, ones, b2w);

    // the next block must be visible to every wave before its first tile
    if (tb == TBM - 1 && next_block) {
      wait_vmem();
      lds_barrier();
    }
  }

  // ---- final state ------------------------------------------------------------
  if (a.w1_out) {
    float* w1 = a.w1_out + (size_t)unit * D * MH;
    float* w2 = a.w2_out + (size_t)unit * MH * D;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          w1[(16 * r + 4 * g + i) * MH + HB + 16 * n + c] = W1c[r][n][i];
          w2[(HB + 16 * r + 4 * g + i) * D + 16 * n + c] = W2c[r][n][i];
        }
    if (c == 0) {
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) a.b1_out[(size_t)unit * MH + HB + 16 * n + 4 * g + i] = b1v[n][i];
#pragma unroll
      for (int i = 0; i < 4; ++i) a.b2_out[(size_t)unit * D + fo + i] = b2w[i];
    }
  }
}

template <bool BF16, bool LN, bool RES>
hipError_t launch3(const MlpArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((ttt_mlp_fwd<BF16, LN, RES>), dim3(a.B * a.H), dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch1(const MlpArgs& a, bool ln, bool res, hipStream_t s) {
  if (ln) return res ? launch3<BF16, true, true>(a, s) : launch3<BF16, true, false>(a, s);
  return res ? launch3<BF16, false, true>(a, s) : launch3<BF16, false, false>(a, s);
}

}  // namespace

hipError_t launch_mlp(const MlpArgs& a, bool bf16, bool ln, bool residual, hipStream_t stream) {
  return bf16 ? launch1<true>(a, ln, residual, stream) : launch1<false>(a, ln, residual, stream);
}

}  // namespace tttk
