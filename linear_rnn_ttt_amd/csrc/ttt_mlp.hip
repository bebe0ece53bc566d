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
// Two kernels.  ttt_mlp_fwd_b16 (further down) serves bf16 data; the
// kernel described here, ttt_mlp_fwd, serves fp32 data (the BF16 template
// argument is kept so that both operand forms stay in one place, but only
// its fp32 instances are launched).
//
// Mapping onto one CU: one 512-thread workgroup (8 waves, two per SIMD) per
// (batch, head) unit.
//   * Wave w owns hidden units 32w..32w+31: W1[:, 32w:32w+32], b1[32w:32w+32]
//     and W2[32w:32w+32, :] stay in fp32 MFMA accumulator registers for the
//     whole sequence.  W2 is kept twice, as W2 and as W2^T: the forward
//     product A W2 contracts the hidden index and the backward product
//     G_o W2^T the feature index, and an accumulator tile only serves a
//     contraction over its row index.  Both copies take the same rank-16
//     update with the two operands swapped, which is cheaper than a
//     transpose of W2 every tile.  b1 is held as 16x16 tiles with equal
//     columns, updated by a product with an all-ones operand; b2 likewise,
//     feature tile w % 4 in wave w.  Waves 0-3 add their b2 tile to their
//     O_k partial sums, waves 4-7 to their O_q partial sums, so each sum
//     holds b2 once.
//   * Hidden pre-activations come out transposed (lane: 4 hidden units of
//     one token), the output pre-activations as per-wave partial sums over
//     the wave's hidden units, added up in LDS.
//   * Waves 0-3 run the LayerNorm backward of O_k (wave w: output features
//     16w..16w+15) and publish -eta G_o; waves 4-7 run the LayerNorm of the
//     previous tile's O_q and store Z.  Deferring the output by one tile lets
//     both LayerNorms share the three workgroup barriers of a tile.
//   * With bf16 inputs the products take plain bf16 operands (state kept in
//     fp32); with fp32 inputs every operand is a bf16 hi + lo pair.
//   * Every product is a 16x16x16 chain (the score tile K Q^T aside, a
//     16x16x32 product from zero): mixed-shape accumulator chains gave wrong
//     values on this toolchain.  P_k, P_q and the O partials accumulate onto
//     the bias tiles, so the biases cost no VALU adds.
#include <math.h>

#include "ttt_device.hpp"
#include "ttt_kernels.hpp"
#include "ttt_tile.hpp"

namespace tttk {
namespace {

constexpr int NW = 8;         // waves per workgroup
constexpr int NT = 64 * NW;   // threads per workgroup
constexpr int MH = 256;       // hidden width
constexpr int HW = MH / NW;   // hidden units per wave

// Tiles per staged block: 4 (bf16) or 2 (fp32) keep the workgroup's LDS
// near 125 KB.
template <bool BF16>
constexpr int tiles_per_block() {
  return BF16 ? 4 : 2;
}

// Phi(-y) for y in [0, 5] is read from a table in LDS (filled at start from
// phi_exp) and interpolated linearly between steps of 1/384: within 2.1e-7
// of the table's function, so within 5e-7 of Phi; beyond y = 5 the table's
// last step is used (Phi(-5) = 2.9e-7).  This takes the reciprocal and the
// exponential of GELU off the VALU.
constexpr int PHI_STEPS = 384;
constexpr int PHI_N = 5 * PHI_STEPS;

template <bool BF16>
struct MlpLds {
  Stage<BF16, tiles_per_block<BF16>()> st;
  f32x4 pk[NW][4][64];    // partial O_k^T tiles [wave][feature tile][lane]
  f32x4 pq[NW][4][64];    // partial O_q^T tiles, summed one tile later
  f32x4 xk[4][2][16];     // LN partial sums of O_k [feature tile][round][token]
  f32x4 xq[4][2][16];     // the same for O_q (round 0 only)
  u32x4 gath[4][2][64];   // -eta G_o per feature tile, in two layouts
  f32x4 gam[16], bet[16]; // LN gamma, beta of the head (4 features per entry)
  f32x4 gsq;              // sum of gamma^2 over each 16-feature tile
  // tiles every wave needs, formed by one wave [tile parity]:
  u32x4 mq[2][64];        // tril(K Q^T + 1) as [hi, lo]
  u32x4 ktb[2][4][64];    // K^T tiles (lane: token 4g+i, feature 16r+c) as [hi, lo]
  f32x2 phit[PHI_N];      // Phi(-y) at y = i / PHI_STEPS: (value, next - value)
};

// Phi(x) and e^{-x^2/2} with one exponential and one reciprocal.  For
// y >= 0, erfc(y) is approximated by t (a1 + t (a2 + t (a3 + t (a4 + t a5))))
// e^{-y^2} with t = 1 / (1 + p y) (Abramowitz and Stegun, Handbook of
// Mathematical Functions, formula 7.1.26: absolute error at most 1.5e-7),
// here at y = |x| / sqrt 2, so that e^{-y^2} is also the Gaussian factor of
// GELU'.  In fp32 the result is within 3e-7 of Phi.  (The three-term
// formula 7.1.25, error 2.5e-5, measurably raised the bf16 scan's error
// against the oracle, although GELU values only enter the matrix unit as
// bf16 operands: its error is systematic, not rounding noise.)
struct PhiExp {
  float h, ex;   // Phi(-|x|), e^{-x^2/2}
};
__device__ __forceinline__ PhiExp phi_exp(float x) {
  constexpr float P = 0.3275911f * 0.70710678118654752f;   // p / sqrt 2
  constexpr float A1 = 0.5f * 0.254829592f;                 // a_i / 2: Phi(-y) = erfc / 2
  constexpr float A2 = 0.5f * -0.284496736f;
  constexpr float A3 = 0.5f * 1.421413741f;
  constexpr float A4 = 0.5f * -1.453152027f;
  constexpr float A5 = 0.5f * 1.061405429f;
  const float t = __builtin_amdgcn_rcpf(fmaf(fabsf(x), P, 1.0f));
  const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, A5, A4), A3), A2), A1);
  const float ex = __builtin_amdgcn_exp2f(x * x * -0.72134752044448170f);   // e^{-x^2/2}
  return PhiExp{poly * ex, ex};
}
// Phi(-|x|) from the table.
__device__ __forceinline__ float phi_neg_tab(const f32x2* tab, float x) {
  const float u = fminf(fabsf(x) * (float)PHI_STEPS, (float)PHI_N - 0.001f);
  const f32x2 e = tab[(int)u];
  return fmaf(__builtin_amdgcn_fractf(u), e.y, e.x);
}
// GELU and GELU' (GELU'(x) = Phi(x) + x phi(x); phi from one exponential).
__device__ __forceinline__ void gelu2(const f32x2* tab, float x, float& y, float& dy) {
  const float h = phi_neg_tab(tab, x);
  const float phi = x >= 0.f ? 1.0f - h : h;
  y = x * phi;
  const float ex = __builtin_amdgcn_exp2f(x * x * -0.72134752044448170f);   // e^{-x^2/2}
  dy = fmaf(x * ex, 0.39894228040143268f, phi);
}
// GELU alone: x Phi(x) = max(x, 0) - |x| Phi(-|x|) for either sign of x.
__device__ __forceinline__ float gelu(const f32x2* tab, float x) {
  return fmaf(-fabsf(x), phi_neg_tab(tab, x), fmaxf(x, 0.f));
}

// LayerNorm statistics of a 16-token x 64-feature tile spread over four
// waves (lane (g,c) of the wave for feature tile ft: token c, features
// 16 ft + 4g + i).  ln_publish writes the wave's sums over its 16 features,
// centred on their local mean; after a barrier ln_combine merges the four
// (parallel-variance update) into, per token, the mean, 1/sigma and, for the
// backward (gy = u + 2 gamma^2 xhat), ma = mean(gamma gy) and
// mx = mean(gamma gy xhat).
template <bool BWD>
__device__ __forceinline__ void ln_publish(f32x4 (&x)[4][2][16], int ft, f32x4 h, f32x4 u,
                                           f32x4 gam, int g, int c) {
  const f32x4 gam2 = gam * gam;
  const float s1 = group_sum(h[0] + h[1] + h[2] + h[3]);
  const float mw = s1 * (1.0f / 16.0f);
  float P = 0.f, A = 0.f, Bq = 0.f, C = 0.f, U = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float e = h[i] - mw;
    P += e * e;
    if (BWD) {
      A += gam2[i] * e;
      Bq += u[i] * e;
      C += gam2[i] * e * e;
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
    x[ft][0][c] = f32x4{s1, P, A, Bq};
    if (BWD) x[ft][1][c] = f32x4{C, U, 0.f, 0.f};
  }
}

struct LnStat {
  float mean, rs, ma, mx;
};
template <bool BWD>
__device__ __forceinline__ LnStat ln_combine(const f32x4 (&x)[4][2][16], f32x4 Gam, float eps,
                                             int c) {
  f32x4 s0[4], s1v[4];
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) {
    s0[ww] = x[ww][0][c];
    if (BWD) s1v[ww] = x[ww][1][c];
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
  r.ma = 0.f;
  r.mx = 0.f;
  if (BWD) {
    r.ma = (Su + 2.0f * r.rs * SgE) * (1.0f / 64.0f);
    r.mx = (r.rs * SuE + 2.0f * r.rs * r.rs * SgE2) * (1.0f / 64.0f);
  }
  return r;
}

// Feature tile r (features 16r + 4g + 0..3 of row c) of a staged row
// operand: the 16x16x16 B operand of X^T restricted to that tile.
__device__ __forceinline__ Op4 row_tile(const Rows& x, int r) {
  const Op8& p = x.p[r >> 1];
  const int h = 2 * (r & 1);
  return Op4{u32x2{p.hi[h], p.hi[h + 1]}, u32x2{p.lo[h], p.lo[h + 1]}};
}
__device__ __forceinline__ u32x4 hilo_of(const Split4& s) { return cat(s.hi, s.lo); }
__device__ __forceinline__ Op4 op4_from(u32x4 x) {
  return Op4{u32x2{x[0], x[1]}, u32x2{x[2], x[3]}};
}

template <bool BF16, bool LN, bool RES>
__global__ __launch_bounds__(NT, 1) void ttt_mlp_fwd(MlpArgs a) {
  using E = typename Io<BF16>::E;
  constexpr bool SP = !BF16;   // hi + lo operands
  constexpr int TBM = tiles_per_block<BF16>();
  __shared__ MlpLds<BF16> L;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int c = lane & 15;
  const int unit = blockIdx.x;
  const int head = unit % a.H;
  const int T = a.T;
  const size_t row0 = (size_t)unit * T;
  const int HB = HW * w;          // the wave's hidden units
  const bool kside = w < 4;       // LN backward of O_k (else: LN of O_q and Z)
  const int ft = w & 3;           // feature tile of the wave's LN role
  const int fo = 16 * ft + 4 * g; // LN layout: lane holds token c, features fo..fo+3
  const size_t s0 = a.state0_per_batch ? (size_t)unit : (size_t)head;

  // ---- state --------------------------------------------------------------
  // W1c[r][n] lane (g,c) = W1[16r + 4g + i][HB + 16n + c]
  // W2c[n][f] lane (g,c) = W2[HB + 16n + 4g + i][16f + c]
  // W2t[f][n] lane (g,c) = W2[HB + 16n + c][16f + 4g + i]
  // b1v[n]    lane (g,c) = b1[HB + 16n + 4g + i]      (any c)
  // b2q       lane (g,c) = b2[16ft + 4g + i]          (any c)
  f32x4 W1c[4][2], W2c[2][4], W2t[4][2], b1v[2], b2q;
  {
    const float* w1 = a.w1 + s0 * D * MH;
    const float* w2 = a.w2 + s0 * MH * D;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          W1c[r][n][i] = w1[(16 * r + 4 * g + i) * MH + HB + 16 * n + c];
          W2c[n][r][i] = w2[(HB + 16 * n + 4 * g + i) * D + 16 * r + c];
          W2t[r][n][i] = w2[(HB + 16 * n + c) * D + 16 * r + 4 * g + i];
        }
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) b1v[n][i] = a.b1[s0 * MH + HB + 16 * n + 4 * g + i];
#pragma unroll
    for (int i = 0; i < 4; ++i) b2q[i] = a.b2[s0 * D + 16 * ft + 4 * g + i];
  }

  // LN parameters in LDS (read where used: fewer live registers)
  if (LN && w == 0) {
    const float* gp = a.gamma + (size_t)head * D;
    const float* bp = a.beta + (size_t)head * D;
    reinterpret_cast<float*>(L.gam)[lane] = gp[lane];
    reinterpret_cast<float*>(L.bet)[lane] = bp[lane];
    if (lane < 4) {
      float s = 0.f;
      for (int j = 0; j < 16; ++j) s += gp[16 * lane + j] * gp[16 * lane + j];
      reinterpret_cast<float*>(&L.gsq)[lane] = s;
    }
  }
  auto ln_gam = [&]() { return L.gam[fo >> 2]; };
  auto ln_bet = [&]() { return L.bet[fo >> 2]; };
  bool causal[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) causal[i] = (4 * g + i) <= c;
  const u32x2 ident = ident_op(g, c);
  const Op4 ones = {ones_op(), u32x2{0u, 0u}};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  // Q side: O_q of a finished tile -> LN -> Z (waves 4-7).  Partial sums
  // are summed and published before one barrier, normalised and stored
  // after the next.
  auto q_publish = [&](f32x4& oq) {
    f32x4 s = zero;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) s += L.pq[ww][ft][lane];
    oq = s;
    if (LN) ln_publish<false>(L.xq, ft, oq, zero, ln_gam(), g, c);
  };
  auto q_store = [&](f32x4 oq, f32x4 qres, int t_tile) {
    f32x4 zf;
    if (LN) {
      const LnStat st = ln_combine<false>(L.xq, L.gsq, a.eps, c);
      const f32x4 gam = ln_gam(), bet = ln_bet();
#pragma unroll
      for (int i = 0; i < 4; ++i)
        zf[i] = (RES ? qres[i] : 0.f) + gam[i] * ((oq[i] - st.mean) * st.rs) + bet[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) zf[i] = (RES ? qres[i] : 0.f) + oq[i];
    }
    const int tok = 16 * t_tile + c;
    if (tok < T) {
      if (BF16) {
        const u32x2 o = {pack_bf16(zf[0], zf[1]), pack_bf16(zf[2], zf[3])};
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.z) + (row0 + tok) * D + fo) = o;
      } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.z) + (row0 + tok) * D + fo) = zf;
      }
    }
  };

  for (int i = tid; i < PHI_N; i += NT) {
    const float t0 = phi_exp((float)i / (float)PHI_STEPS).h;
    const float t1 = phi_exp((float)(i + 1) / (float)PHI_STEPS).h;
    L.phit[i] = f32x2{t0, t1 - t0};
  }

  const int n_tiles = (T + 15) / 16;
  stage_issue<BF16, TBM>(L.st, a.q, a.k, a.v, a.eta, row0, 0, T, 0, w & 3, w >> 2, 2);
  wait_vmem();
  lds_barrier();

  f32x4 qprev = zero;   // Q side: residual rows of the previous tile
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int blk = tile / TBM, tb = tile % TBM, buf = blk & 1;
    const bool next_block = (blk + 1) * TBM < n_tiles;
    if (tb == 0 && next_block) {
      // every wave has passed the previous tile's last barrier, after which
      // nothing reads the other buffer (previous block)
      stage_issue<BF16, TBM>(L.st, a.q, a.k, a.v, a.eta, row0, blk + 1, T, buf ^ 1, w & 3,
                             w >> 2, 2);
    }
    const E* Lq = L.st.qkv[buf][0];
    const E* Lk = L.st.qkv[buf][1];
    const E* Lv = L.st.qkv[buf][2];
    const int t0 = tb * 16;

    // ================= phase A: K-side forward, O_k partials ==============
    const Rows kb = load_rows<BF16>(Lk, t0, c, g);
    const Rows qb = load_rows<BF16>(Lq, t0, c, g);

    // The 16-deep products below accumulate onto the bias tiles (themselves
    // 16x16x16 results), so the biases cost no VALU adds.
    // W1 as the A operand of W1^T, per 16-feature tile r
    Op4 w1t[4][2];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int n = 0; n < 2; ++n) w1t[r][n] = op4_of(W1c[r][n]);

    // hidden pre-activations, transposed: lane = token c, hidden HB + 16n + 4g + i
    f32x4 Ak[2], Dk[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      f32x4 acc = b1v[n];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc = mma4<SP, SP>(w1t[r][n], row_tile(kb, r), acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float y, dy;
        gelu2(L.phit, acc[i], y, dy);
        Ak[n][i] = y;
        Dk[n][i] = dy;
      }
    }
    const Op4 ak[2] = {op4_of(Ak[0]), op4_of(Ak[1])};   // A_k^T as B operands

    // W2 as the A operand of W2^T: w2t[n][f] for hidden tile n, feature tile f
    Op4 w2t[2][4];
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int f = 0; f < 4; ++f) w2t[n][f] = op4_of(W2c[n][f]);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      f32x4 o = (kside && f == ft) ? b2q : zero;
#pragma unroll
      for (int n = 0; n < 2; ++n) o = mma4<SP, SP>(w2t[n][f], ak[n], o);
      L.pk[w][f][lane] = o;
    }

    // the output side's products that need no gradient: Q W1 + b1
    f32x4 Pq[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      f32x4 acc = b1v[n];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc = mma4<SP, SP>(w1t[r][n], row_tile(qb, r), acc);
      Pq[n] = acc;
    }
    // tiles every wave needs, one wave each: tril(Q K^T + 1) (lane:
    // k_{4g+i} . q_c + 1) and K^T (lane: token 4g+i, feature 16r+c; from the
    // rows by a product with the identity, exact for bf16 parts)
    if (w == 0) {
      f32x4 M = gram<SP>(kb, qb);
#pragma unroll
      for (int i = 0; i < 4; ++i) M[i] = causal[i] ? M[i] + 1.f : 0.f;
      L.mq[tile & 1][lane] = hilo_of(split4(M));
    } else if (w == 1) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const Op4 kr = row_tile(kb, r);
        const Op4 t = transpose_op<SP>(Split4{kr.hi, kr.lo}, ident);
        L.ktb[tile & 1][r][lane] = cat(t.hi, t.lo);
      }
    }
    // A_k^T tiles for the W2 update: lane = token 4g+i, hidden HB + 16n + c
    const Op4 akt[2] = {transpose_op<SP>(Split4{ak[0].hi, ak[0].lo}, ident),
                        transpose_op<SP>(Split4{ak[1].hi, ak[1].lo}, ident)};

    lds_barrier();   // (1) O_k partials of this tile, O_q partials of the last

    // ================= phase B: LN sums ===================================
    f32x4 ok = zero, oq = zero, u = zero;   // u: the part of gamma dl/dy that is not in xhat
    if (kside) {
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) ok += L.pk[ww][ft][lane];
      const f32x4 kres = val4(Lk + lds_off<BF16>(t0 + c, fo));
      const f32x4 vres = val4(Lv + lds_off<BF16>(t0 + c, fo));
      if (LN) {
        const f32x4 gam = ln_gam(), bet = ln_bet();
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = 2.f * gam[i] * ((RES ? kres[i] : 0.f) + bet[i] - vres[i]);
        ln_publish<true>(L.xk, ft, ok, u, gam, g, c);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = (RES ? kres[i] : 0.f) - vres[i];
      }
    } else if (tile > 0) {
      q_publish(oq);
    }
    if (LN) lds_barrier();   // (2) LN partial sums

    // ================= phase C: -eta G_o (K side), Z of the last tile (Q side)
    if (kside) {
      const bool valid = 16 * tile + c < T;
      const float eta = L.st.eta[buf][t0 + c];
      f32x4 ego;
      if (LN) {
        const LnStat st = ln_combine<true>(L.xk, L.gsq, a.eps, c);
        const f32x4 gam = ln_gam();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float xh = (ok[i] - st.mean) * st.rs;
          const float gy = u[i] + 2.f * gam[i] * gam[i] * xh;   // gamma dl/dy
          ego[i] = valid ? -eta * st.rs * (gy - st.ma - xh * st.mx) : 0.f;   // padding: exactly 0
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) ego[i] = valid ? -2.f * eta * (ok[i] + u[i]) : 0.f;
      }
      const Split4 es = split4(ego);
      const Op4 got_own = transpose_op<SP>(es, ident);   // lane: token 4g+i, feature 16ft+c
      L.gath[ft][0][lane] = cat(es.hi, es.lo);
      L.gath[ft][1][lane] = cat(got_own.hi, got_own.lo);
    } else {
      if (tile > 0) q_store(oq, qprev, tile - 1);
      qprev = val4(Lq + lds_off<BF16>(t0 + c, fo));
    }
    lds_barrier();   // (3) -eta G_o of every feature tile

    // ================= phase D: backprop, output partials, update =========
    Op4 egoL[4], got[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const u32x4 x = L.gath[f][0][lane];
      const u32x4 y = L.gath[f][1][lane];
      egoL[f] = Op4{u32x2{x[0], x[1]}, u32x2{x[2], x[3]}};   // lane: token c, feats 16f+4g+i
      got[f] = Op4{u32x2{y[0], y[1]}, u32x2{y[2], y[3]}};    // lane: token 4g+i, feat 16f+c
    }

    // -eta dl/dP_k = ((-eta G_o) W2^T) * GELU'(P_k), transposed like P_k
    Op4 gpt[2];   // lane: token 4g+i, hidden HB + 16n + c
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      f32x4 acc = zero;
#pragma unroll
      for (int f = 0; f < 4; ++f) acc = mma4<SP, SP>(op4_of(W2t[f][n]), egoL[f], acc);
      gpt[n] = transpose_op<SP>(split4(acc * Dk[n]), ident);
    }

    // K^T tiles and tril(Q K^T + 1), as formed by waves 1 and 0
    Op4 kt[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) kt[r] = op4_from(L.ktb[tile & 1][r][lane]);
    const Op4 Mq = op4_from(L.mq[tile & 1][lane]);
    // W1 and b1 first: the next tile's first products wait on them
#pragma unroll
    for (int n = 0; n < 2; ++n) {
#pragma unroll
      for (int r = 0; r < 4; ++r) W1c[r][n] = mma4<SP, SP>(kt[r], gpt[n], W1c[r][n]);
      b1v[n] = mma4<SP, false>(gpt[n], ones, b1v[n]);
    }

    // output: P_q, A_q, this wave's share of O_q (state before this tile's update)
    f32x4 Aq[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const f32x4 p = mma4<SP, SP>(gpt[n], Mq, Pq[n]);   // - tril(Q K^T + 1) (eta G_p)
#pragma unroll
      for (int i = 0; i < 4; ++i) Aq[n][i] = gelu(L.phit, p[i]);
    }
    const Op4 aq[2] = {op4_of(Aq[0]), op4_of(Aq[1])};
    // W2 operands again (cheaper than holding them since the first use)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int f = 0; f < 4; ++f) asm volatile("" : "+v"(W2c[n][f]));
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int f = 0; f < 4; ++f) w2t[n][f] = op4_of(W2c[n][f]);
    {
      // this wave's share of tril(A_q A_k^T + 1): lane M[s = 4g+i][t = c]
      f32x4 Ma = zero;
#pragma unroll
      for (int n = 0; n < 2; ++n) Ma = mma4<SP, SP>(ak[n], aq[n], Ma);
#pragma unroll
      for (int i = 0; i < 4; ++i) Ma[i] = causal[i] ? Ma[i] + (w == 0 ? 1.f : 0.f) : 0.f;
      const Op4 Mas = op4_of(Ma);
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        f32x4 o = (!kside && f == ft) ? b2q : zero;
#pragma unroll
        for (int n = 0; n < 2; ++n) o = mma4<SP, SP>(w2t[n][f], aq[n], o);
        o = mma4<SP, SP>(got[f], Mas, o);   // - tril(A_q A_k^T + 1) (eta G_o)
        L.pq[w][f][lane] = o;
      }
    }

    // W2 (both layouts) and b2
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        W2c[n][f] = mma4<SP, SP>(akt[n], got[f], W2c[n][f]);
        W2t[f][n] = mma4<SP, SP>(got[f], akt[n], W2t[f][n]);
      }
    b2q = mma4<SP, false>(got[ft], ones, b2q);

    // the next block must be visible to every wave before its first tile
    if (tb == TBM - 1 && next_block) {
      wait_vmem();
      lds_barrier();
    }
  }

  // ---- Z of the last tile -----------------------------------------------------
  lds_barrier();
  f32x4 oq = zero;
  if (!kside) q_publish(oq);
  if (LN) lds_barrier();
  if (!kside) q_store(oq, qprev, n_tiles - 1);

  // ---- final state ------------------------------------------------------------
  if (a.w1_out) {
    // fresh lane indices: keeps the compiler from holding the prologue's
    // per-lane state offsets live through the loop for these stores
    int g = lane >> 4, c = lane & 15;
    asm volatile("" : "+v"(g), "+v"(c));
    float* w1 = a.w1_out + (size_t)unit * D * MH;
    float* w2 = a.w2_out + (size_t)unit * MH * D;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          w1[(16 * r + 4 * g + i) * MH + HB + 16 * n + c] = W1c[r][n][i];
          w2[(HB + 16 * n + 4 * g + i) * D + 16 * r + c] = W2c[n][r][i];
        }
    if (c == 0) {
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) a.b1_out[(size_t)unit * MH + HB + 16 * n + 4 * g + i] = b1v[n][i];
      if (kside) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a.b2_out[(size_t)unit * D + 16 * ft + 4 * g + i] = b2q[i];
      }
    }
  }
}

// ===========================================================================
// bf16 data: ttt_mlp_fwd_b16<LN, RES>.  Wave w again owns hidden units
// 32w..32w+31 (W1 and W2 in accumulator registers, no transposed copy of
// W2), with the work reorganised around the matrix unit's 32-deep product
// (on gfx950 a 16x16x32 bf16 product issues at the rate of a 16x16x16 one,
// so it halves the matrix time of every product whose contraction is 32
// deep or more) and around two barriers per tile:
//   phase A  P_k = K W1 + b1 with tokens as rows, GELU and GELU' (one
//            exponential and one reciprocal), A_k transposed once on the
//            matrix unit, the O_k partial over the wave's hidden units;
//            Q W1 + b1 for the output;
//   barrier 1
//   phase B  waves 0-3: LayerNorm backward of O_k, each wave on 4 whole
//            tokens (16 lanes per token, 4 features per lane: the
//            feature sums are DPP row sums, no exchange), -eta G_o
//            published as rows and as columns; waves 4-7: LayerNorm of the
//            previous tile's O_q and its z;
//   barrier 2
//   phase D  U_p = (U_o W2^T) * GELU'(P_k) with tokens as rows (the layout
//            every consumer of U_p takes; W2 with features as rows comes from
//            a transpose of its bf16 tiles on the matrix unit, which costs what
//            updating a second, transposed copy of W2 would, and frees 32
//            registers); the output pre-activation from the state at the
//            tile's start, P_q = Q W1 + b1 + tril(Q K^T + 1) U_p; the
//            updates of W1, b1, W2; then the rest of the output,
//            O_q = A_q W2 + b2 + tril(A_q A_k^T + 1) U_o (the bf16 W2 tiles
//            of the tile's start), and the update of b2.  (Taking the output
//            from the updated state minus the strictly upper terms instead
//            would share W2's conversion with the next tile, but early in a
//            sequence, where a tile's update is large next to the state, the
//            subtraction cancels: z errors of 3.8e-2 on the first tokens of
//            a tile.)
// Every accumulate chain keeps one product shape: the bias tiles are
// updated by 32-deep products with zero upper slots, because they seed the
// 32-deep chains of P and O.
constexpr int GSTEPS = 192;           // table entries per unit of x
constexpr float GR = 6.0f;            // table range [-GR, GR)
constexpr int GN = 2 * 6 * GSTEPS;    // entries

struct MlpLdsB {
  Stage<true, 4> st;
  f32x4 pk[NW][16][16];   // O_k^T partials: [wave][token][chunk ^ token], chunk m = features 4m..4m+3
  f32x4 pq[NW][16][16];   // O_q^T partials of the previous tile, same layout
  // -eta G_o rows: [token][4p + g] = features 32p+4g+(0..3), 32p+16+4g+(0..3);
  // rows padded to 9 chunks, so that the 16 tokens a read spans start in
  // different banks
  u32x4 uor[16][9];
  // -eta G_o columns: [feature tile f][lane (g,c)] = tokens 4g+(0..3) of
  // feature 16f+c; tiles padded by 2 entries (the 2-byte writes of one lane
  // to the four tiles fall in different banks)
  u32x2 uoc[4][66];
  u32x2 mq[2][64];        // tril(K Q^T + 1) [tile parity][lane (g,c)]: k_{4g+i} . q_c + 1, 4g+i <= c
  u32x2 ktb[2][4][64];    // K^T [tile parity][feature tile r][lane (g,c)]: K[4g+i][16r+c]
  f32x4 b2[2][16];        // b2 at the start of tile t in [t & 1] (features 4m..4m+3)
  f32x2 gphi[GN];         // (Phi, next Phi - Phi) at x_i = -GR + i / GSTEPS
};

// The four fp32 values of a lane as one 4-element bf16 operand.
__device__ __forceinline__ u32x2 pk4(f32x4 v) {
  return u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
}

// GELU and GELU' of the hidden pre-activations of the gradient point, which
// sit on the scan's serial path: evaluated per value (phi_exp: one
// reciprocal and one exponential), not read from LDS, whose latency and
// data-dependent bank conflicts cost more there (5 % of the scan).
__device__ __forceinline__ void gelu_both(float x, float& y, float& dy) {
  const PhiExp pe = phi_exp(x);
  const float phi = x >= 0.f ? 1.0f - pe.h : pe.h;
  y = x * phi;
  dy = fmaf(x * pe.ex, 0.39894228040143268f, phi);
}
// GELU alone (the output side, off the serial path): x Phi(x) with Phi
// interpolated linearly in the table (step 1/192: within 8.2e-7).  Outside
// [-GR, GR) the end entries are used: Phi is 0 or 1 there to within 1e-9,
// so x Phi stays exact to that level for any x.
__device__ __forceinline__ float gelu_only(const f32x2* tphi, float x) {
  const float u = __builtin_amdgcn_fmed3f(fmaf(x, (float)GSTEPS, GR * GSTEPS), 0.f,
                                          (float)GN - 0.002f);
  const f32x2 e = tphi[(int)u];
  return x * fmaf(__builtin_amdgcn_fractf(u), e[1], e[0]);
}

// x from another lane of the same 16-lane row (DPP control CTRL).
template <int CTRL>
__device__ __forceinline__ float rdpp(float x) {
  return bitsf(static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(fbits(x)), CTRL, 0xf, 0xf, false)));
}
// Sums over each 16-lane row, in every lane of the row (lanes l^1, l^2,
// then the mirrored lane of the half row and of the row).
template <int N>
__device__ __forceinline__ void row_sums(float (&x)[N]) {
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += rdpp<0xB1>(x[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += rdpp<0x4E>(x[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += rdpp<0x141>(x[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += rdpp<0x140>(x[j]);
}

template <bool LN, bool RES>
__global__ __launch_bounds__(NT, 1) void ttt_mlp_fwd_b16(MlpArgs a) {
  __shared__ MlpLdsB L;
  constexpr int TBM = 4;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int c = lane & 15;
  const int unit = blockIdx.x;
  const int head = unit % a.H;
  const int T = a.T;
  const size_t row0 = (size_t)unit * T;
  const int HB = HW * w;          // the wave's hidden units
  const bool kside = w < 4;       // phase B: LN backward of O_k (else LN of O_q and z)
  const int ft = w & 3;           // feature tile of the wave's b2 copy
  // phase B layout: token 4 ft + jb of the tile, features 4 mb .. 4 mb + 3
  const int jb = lane >> 4, mb = lane & 15;
  const int tokb = 4 * ft + jb;
  const size_t s0 = a.state0_per_batch ? (size_t)unit : (size_t)head;

  // ---- state --------------------------------------------------------------
  // W1c[r][n] lane (g,c) = W1[16r + 4g + i][HB + 16n + c]
  // W2c[n][f] lane (g,c) = W2[HB + 16n + 4g + i][16f + c]
  // b1r[n]    lane (g,c) = b1[HB + 16n + c]        (any i: token rows)
  // b1h[n]    lane (g,c) = b1[HB + 16n + 4g + i]   (any c: hidden rows)
  // b2q       lane (g,c) = b2[16ft + 4g + i]       (any c; waves 0-3, which
  //                                                publish it to LDS for the
  //                                                LayerNorm inputs)
  // (W2 with features as rows, for U_o W2^T, is formed from W2c each tile
  // by a transpose on the matrix unit.)
  f32x4 W1c[4][2], W2c[2][4], b1r[2], b1h[2], b2q;
  {
    const float* w1 = a.w1 + s0 * D * MH;
    const float* w2 = a.w2 + s0 * MH * D;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          W1c[r][n][i] = w1[(16 * r + 4 * g + i) * MH + HB + 16 * n + c];
          W2c[n][r][i] = w2[(HB + 16 * n + 4 * g + i) * D + 16 * r + c];
        }
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        b1r[n][i] = a.b1[s0 * MH + HB + 16 * n + c];
        b1h[n][i] = a.b1[s0 * MH + HB + 16 * n + 4 * g + i];
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) b2q[i] = a.b2[s0 * D + 16 * ft + 4 * g + i];
    if (kside && c == 0) L.b2[0][4 * ft + g] = b2q;
  }
  // LN parameters of the lane's phase-B features
  f32x4 gam = {1.f, 1.f, 1.f, 1.f}, bet = {0.f, 0.f, 0.f, 0.f};
  if (LN) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gam[i] = a.gamma[(size_t)head * D + 4 * mb + i];
      bet[i] = a.beta[(size_t)head * D + 4 * mb + i];
    }
  }
  const u32x2 ident = ident_op(g, c);
  const u32x2 ones = ones_op();
  const u32x2 z2 = {0u, 0u};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  // Phi table
  for (int i = tid; i < GN; i += NT) {
    const float p0 = 0.5f * erfcf((GR - (float)i / (float)GSTEPS) * 0.70710678118654752f);
    const float p1 = 0.5f * erfcf((GR - (float)(i + 1) / (float)GSTEPS) * 0.70710678118654752f);
    L.gphi[i] = f32x2{p0, p1 - p0};
  }

  const int n_tiles = (T + 15) / 16;
  stage_issue<true, TBM>(L.st, a.q, a.k, a.v, a.eta, row0, 0, T, 0, w & 3, w >> 2, 2);
  wait_vmem();
  lds_barrier();

  f32x4 qres = zero;   // q rows of the tile whose z phase B stores

  // LN of the previous tile's O_q and its z (waves 4-7)
  auto output_store = [&](int tp) {
    f32x4 o = L.b2[tp & 1][mb];
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) o += L.pq[ww][tokb][mb ^ tokb];
    f32x4 zf;
    if (LN) {
      float s[1] = {(o[0] + o[1]) + (o[2] + o[3])};
      row_sums(s);
      const float mu = s[0] * (1.0f / D);
      f32x4 e;
#pragma unroll
      for (int i = 0; i < 4; ++i) e[i] = o[i] - mu;
      float v[1] = {(e[0] * e[0] + e[1] * e[1]) + (e[2] * e[2] + e[3] * e[3])};
      row_sums(v);
      const float rs = __frsqrt_rn(v[0] * (1.0f / D) + a.eps);
#pragma unroll
      for (int i = 0; i < 4; ++i) zf[i] = (RES ? qres[i] : 0.f) + fmaf(gam[i] * rs, e[i], bet[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) zf[i] = (RES ? qres[i] : 0.f) + o[i];
    }
    const int tok = 16 * tp + tokb;
    if (tok < T)
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.z) + (row0 + tok) * D + 4 * mb) = pk4(zf);
  };

  for (int tile = 0; tile < n_tiles; ++tile) {
    const int blk = tile / TBM, tb = tile % TBM, buf = blk & 1;
    const bool next_block = (blk + 1) * TBM < n_tiles;
    const uint16_t* Lq = L.st.qkv[buf][0];
    const uint16_t* Lk = L.st.qkv[buf][1];
    const uint16_t* Lv = L.st.qkv[buf][2];
    const int t0 = tb * 16;

    // ================= phase A ==============================================
    const Rows kb = load_rows<true>(Lk, t0, c, g);
    // W1 as 16x16x32 operands: B of K W1 ([feature slot][hidden c]) and A of
    // (Q W1)^T ([hidden c][feature slot]) are the same registers
    u32x4 w1b[2][2];
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int p = 0; p < 2; ++p) w1b[n][p] = cat(pk4(W1c[2 * p][n]), pk4(W1c[2 * p + 1][n]));
    // P_k with tokens as rows: lane (g,c) = P_k[4g+i][HB + 16n + c]
    f32x4 Ak[2], Dk[2];
    u32x2 akr[2], akh[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      f32x4 acc = mfma32(kb.p[0].hi, w1b[n][0], b1r[n]);
      acc = mfma32(kb.p[1].hi, w1b[n][1], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float y, dy;
        gelu_both(acc[i], y, dy);
        Ak[n][i] = y;
        Dk[n][i] = dy;
      }
      akr[n] = pk4(Ak[n]);
      // hidden rows: lane (g,c) = A_k[c][HB + 16n + 4g + i]
      akh[n] = pk4(mfma16(akr[n], ident, zero));
    }
    // W2 at the tile's start as bf16 tiles (until its update in phase D):
    // pairs of them are the A operands of W2^T ([feature c][hidden slot])
    u32x2 w2h[2][4];
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int f = 0; f < 4; ++f) w2h[n][f] = pk4(W2c[n][f]);
    {
      const u32x4 akb = cat(akh[0], akh[1]);
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        L.pk[w][c][(4 * f + g) ^ c] = mfma32(cat(w2h[0][f], w2h[1][f]), akb, zero);
      }
    }
    // Q W1 + b1 (hidden rows) for this tile's output
    const Rows qb = load_rows<true>(Lq, t0, c, g);
    f32x4 Pq[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      f32x4 acc = mfma32(w1b[n][0], qb.p[0].hi, b1h[n]);
      Pq[n] = mfma32(w1b[n][1], qb.p[1].hi, acc);
    }
    // tiles every wave needs, one wave each
    if (w == 0) {
      f32x4 M = gram<false>(kb, qb);   // lane (g,c): k_{4g+i} . q_c
#pragma unroll
      for (int i = 0; i < 4; ++i) M[i] = (4 * g + i <= c) ? M[i] + 1.f : 0.f;
      L.mq[tile & 1][lane] = pk4(M);
    } else if (w == 1) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const Op4 kr = row_tile(kb, r);
        L.ktb[tile & 1][r][lane] = transpose_op<false>(Split4{kr.hi, kr.lo}, ident).hi;
      }
    }
    lds_barrier_copies_in_flight();   // (1)
    if (tb == 0 && next_block) {
      // every wave has passed barrier 1, after which nothing reads the other
      // buffer (the previous block)
      stage_issue<true, TBM>(L.st, a.q, a.k, a.v, a.eta, row0, blk + 1, T, buf ^ 1, w & 3,
                             w >> 2, 2);
    }

    // ================= phase B ==============================================
    if (kside) {
      f32x4 o = L.b2[tile & 1][mb];
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) o += L.pk[ww][tokb][mb ^ tokb];
      const f32x4 kr = val4(Lk + lds_off<true>(t0 + tokb, 4 * mb));
      const f32x4 vr = val4(Lv + lds_off<true>(t0 + tokb, 4 * mb));
      const float eta = 16 * tile + tokb < T ? L.st.eta[buf][t0 + tokb] : 0.f;
      f32x4 uo;
      if (LN) {
        float s[1] = {(o[0] + o[1]) + (o[2] + o[3])};
        row_sums(s);
        const float mu = s[0] * (1.0f / D);
        f32x4 e;
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = o[i] - mu;
        float v[1] = {(e[0] * e[0] + e[1] * e[1]) + (e[2] * e[2] + e[3] * e[3])};
        row_sums(v);
        const float rs = __frsqrt_rn(v[0] * (1.0f / D) + a.eps);
        f32x4 xh, gy;
        float m[2] = {0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xh[i] = e[i] * rs;
          const float tg = 2.f * gam[i];
          // gamma dl/dy = 2 gamma (k + gamma xhat + beta - v)
          gy[i] = tg * (((RES ? kr[i] : 0.f) + bet[i] - vr[i]) + gam[i] * xh[i]);
          m[0] += gy[i];
          m[1] = fmaf(gy[i], xh[i], m[1]);
        }
        row_sums(m);
        const float ma = m[0] * (1.0f / D), mx = m[1] * (1.0f / D);
        const float c1 = -eta * rs;
#pragma unroll
        for (int i = 0; i < 4; ++i) uo[i] = c1 * fmaf(-xh[i], mx, gy[i] - ma);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) uo[i] = -2.f * eta * (o[i] + (RES ? kr[i] : 0.f) - vr[i]);
      }
      // rows: features 4 mb .. 4 mb + 3 = 16 f + 4 gg + (0..3)
      const u32x2 ub = pk4(uo);
      const int f = mb >> 2, gg = mb & 3;
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint32_t*>(&L.uor[tokb][4 * (f >> 1) + gg]) +
                                2 * (f & 1)) = ub;
      // columns: lane 16 (tokb / 4) + 4 gg + i of tile f, slot tokb % 4
      uint16_t* col = reinterpret_cast<uint16_t*>(&L.uoc[f][16 * (tokb >> 2) + 4 * gg]) + (tokb & 3);
      col[0] = (uint16_t)(ub.x & 0xffffu);
      col[4] = (uint16_t)(ub.x >> 16);
      col[8] = (uint16_t)(ub.y & 0xffffu);
      col[12] = (uint16_t)(ub.y >> 16);
    } else {
      if (tile > 0) output_store(tile - 1);
      qres = val4(Lq + lds_off<true>(t0 + tokb, 4 * mb));
    }
    lds_barrier_copies_in_flight();   // (2)

    // ================= phase D ==============================================
    const u32x4 uo0 = L.uor[c][g], uo1 = L.uor[c][4 + g];
    u32x2 uoc[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) uoc[f] = L.uoc[f][lane];
    // W2's bf16 tiles: the A operands of the output's A_q W2 and,
    // transposed on the matrix unit, the B operands [feature slot][hidden c]
    // of U_o W2^T
    u32x2 upr[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      u32x2 wt[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) wt[f] = pk4(mfma16(w2h[n][f], ident, zero));
      f32x4 u = mfma32(uo0, cat(wt[0], wt[1]), zero);
      u = mfma32(uo1, cat(wt[2], wt[3]), u);
      upr[n] = pk4(u * Dk[n]);   // U_p = (U_o W2^T) * GELU'(P_k), token rows
    }
    // output pre-activation P_q = Q W1 + b1 + tril(Q K^T + 1) U_p (state at
    // the tile's start)
    const u32x2 mqv = L.mq[tile & 1][lane];
    f32x4 pq[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) pq[n] = mfma32(cat(upr[n], z2), cat(mqv, z2), Pq[n]);
    // updates: from here on the output reads only the bf16 tiles of phase A,
    // so the update products do not depend on it; issued ahead of the
    // output's GELU and dependent products, they give the scheduler matrix
    // work to overlap with that chain (3.5 % faster than after the output)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const u32x2 kt = L.ktb[tile & 1][r][lane];
#pragma unroll
      for (int n = 0; n < 2; ++n) W1c[r][n] = mfma16(kt, upr[n], W1c[r][n]);
    }
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      b1r[n] = mfma32(cat(ones, z2), cat(upr[n], z2), b1r[n]);
      b1h[n] = mfma32(cat(upr[n], z2), cat(ones, z2), b1h[n]);
    }
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int f = 0; f < 4; ++f) W2c[n][f] = mfma16(akr[n], uoc[f], W2c[n][f]);
    // output: A_q and this wave's share of O_q
    {
      f32x4 aq[2];
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) aq[n][i] = gelu_only(L.gphi, pq[n][i]);
      const u32x4 aqb = cat(pk4(aq[0]), pk4(aq[1]));
      // this wave's share of tril(A_q A_k^T + 1): lane (g,c) at s' = 4g+i, s = c
      f32x4 ma = mfma32(cat(akh[0], akh[1]), aqb, zero);
#pragma unroll
      for (int i = 0; i < 4; ++i) ma[i] = (4 * g + i <= c) ? ma[i] + (w == 0 ? 1.f : 0.f) : 0.f;
      const u32x2 mas = pk4(ma);
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        f32x4 o = mfma32(cat(w2h[0][f], w2h[1][f]), aqb, zero);
        o = mfma32(cat(uoc[f], z2), cat(mas, z2), o);   // + tril(A_q A_k^T + 1) U_o
        L.pq[w][c][(4 * f + g) ^ c] = o;   // summed after barrier 1 of the next tile
      }
    }
    if (kside) {
      // (uoc[ft] re-read: a register array indexed by the wave's ft would
      // be a chain of selects)
      b2q = mfma32(cat(L.uoc[ft][lane], z2), cat(ones, z2), b2q);
      if (c == 0) L.b2[(tile + 1) & 1][4 * ft + g] = b2q;   // read after barrier 1 of the next tile
    }

    // the next block must be visible to every wave before its first tile
    if (tb == TBM - 1 && next_block) {
      wait_vmem();
      lds_barrier();
    }
  }

  // ---- z of the last tile ----------------------------------------------------
  lds_barrier();
  if (!kside) output_store(n_tiles - 1);

  // ---- final state ------------------------------------------------------------
  if (a.w1_out) {
    int g = lane >> 4, c = lane & 15;
    asm volatile("" : "+v"(g), "+v"(c));
    float* w1 = a.w1_out + (size_t)unit * D * MH;
    float* w2 = a.w2_out + (size_t)unit * MH * D;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          w1[(16 * r + 4 * g + i) * MH + HB + 16 * n + c] = W1c[r][n][i];
          w2[(HB + 16 * n + 4 * g + i) * D + 16 * r + c] = W2c[n][r][i];
        }
    if (c == 0) {
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) a.b1_out[(size_t)unit * MH + HB + 16 * n + 4 * g + i] = b1h[n][i];
      if (kside) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a.b2_out[(size_t)unit * D + 16 * ft + 4 * g + i] = b2q[i];
      }
    }
  }
}

template <bool BF16, bool LN, bool RES>
hipError_t launch3(const MlpArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((ttt_mlp_fwd<BF16, LN, RES>), dim3(a.B * a.H), dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <bool LN, bool RES>
hipError_t launch_b16(const MlpArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((ttt_mlp_fwd_b16<LN, RES>), dim3(a.B * a.H), dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch1(const MlpArgs& a, bool ln, bool res, hipStream_t s) {
  if constexpr (BF16) {
    if (ln) return res ? launch_b16<true, true>(a, s) : launch_b16<true, false>(a, s);
    return res ? launch_b16<false, true>(a, s) : launch_b16<false, false>(a, s);
  } else {
    if (ln) return res ? launch3<false, true, true>(a, s) : launch3<false, true, false>(a, s);
    return res ? launch3<false, false, true>(a, s) : launch3<false, false, false>(a, s);
  }
}

}  // namespace

hipError_t launch_mlp(const MlpArgs& a, bool bf16, bool ln, bool residual, hipStream_t stream) {
  return bf16 ? launch1<true>(a, ln, residual, stream) : launch1<false>(a, ln, residual, stream);
}

}  // namespace tttk
