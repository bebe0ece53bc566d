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
//   * one 256-thread workgroup (4 waves) per (batch, head) unit; wave w
//     owns output columns 16w..16w+15 of W and of every H, G, Z tile;
//   * the state never leaves the registers: W[:, 16w:16w+16] is four 16x16
//     MFMA accumulators per wave, updated in place by the update product;
//   * H is produced transposed (H^T = W^T K^T), so a lane holds 4 features
//     of ONE token and the LN row sums are 3 in-lane adds plus 2 cross-group
//     steps; the 4 waves exchange 6 (chain) or 2 (output) partial sums per
//     token through LDS, one barrier each;
//   * fp32 operands are fed to the bf16 matrix unit as hi + lo bf16 pairs
//     (about 16 significant bits); bf16 inputs are exact;
//   * q, k, v, eta stream from HBM in 16 KB-per-tensor blocks: the next
//     block is loaded into registers while the current one is processed
//     from LDS, then written to the other LDS buffer.
#include "ttt_device.hpp"
#include "ttt_kernels.hpp"

namespace tttk {
namespace {

constexpr int D = 64;
constexpr int NT = 256;  // threads per workgroup

template <bool BF16>
struct Io;
template <>
struct Io<true> {
  using E = uint16_t;
  static constexpr int TB = 8;     // tiles per staged block (128 tokens)
  static constexpr int ROW = 72;   // LDS row stride in elements (144 B)
  static constexpr int CPR = 8;    // 16-byte chunks per 64-element row
};
template <>
struct Io<false> {
  using E = float;
  static constexpr int TB = 4;     // 64 tokens
  static constexpr int ROW = 68;   // 272 B
  static constexpr int CPR = 16;
};

template <bool BF16>
struct Lds {
  using E = typename Io<BF16>::E;
  static constexpr int TOK = Io<BF16>::TB * 16;
  static constexpr int ROW = Io<BF16>::ROW;
  E qkv[2][3][TOK * ROW];       // staged q, k, v blocks (double buffered)
  float eta[2][TOK];
  float stats_k[2][16][4][8];   // chain LN partial sums [parity][token][wave]
  float stats_q[2][16][4][4];   // output LN partial sums
};

// Per-thread registers holding the next staged block.
template <bool BF16>
struct Staged {
  u32x4 r[3][4];
  float eta;
};

template <bool BF16>
__device__ __forceinline__ void stage_load(Staged<BF16>& s, const LinearArgs& a,
                                           size_t row0, int tok0, int T) {
  using E = typename Io<BF16>::E;
  constexpr int CPR = Io<BF16>::CPR;
  const int tid = threadIdx.x;
  const char* src[3] = {static_cast<const char*>(a.q), static_cast<const char*>(a.k),
                        static_cast<const char*>(a.v)};
#pragma unroll
  for (int t = 0; t < 3; ++t) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int id = j * NT + tid;
      const int row = id / CPR, cc = id % CPR;
      const int tok = tok0 + row;
      if (tok < T) {
        const char* p = src[t] + (row0 + tok) * (size_t)D * sizeof(E) + cc * 16;
        s.r[t][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
      } else {
        s.r[t][j] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  constexpr int TOK = Io<BF16>::TB * 16;
  if (tid < TOK) {
    const int tok = tok0 + tid;
    s.eta = tok < T ? a.eta[row0 + tok] : 0.0f;
  }
}

template <bool BF16>
__device__ __forceinline__ void stage_store(const Staged<BF16>& s, Lds<BF16>& L, int buf) {
  using E = typename Io<BF16>::E;
  constexpr int CPR = Io<BF16>::CPR;
  constexpr int ROW = Io<BF16>::ROW;
  const int tid = threadIdx.x;
#pragma unroll
  for (int t = 0; t < 3; ++t) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int id = j * NT + tid;
      const int row = id / CPR, cc = id % CPR;
      char* p = reinterpret_cast<char*>(L.qkv[buf][t]) + (row * ROW) * sizeof(E) + cc * 16;
      *reinterpret_cast<u32x4*>(p) = s.r[t][j];
    }
  }
  constexpr int TOK = Io<BF16>::TB * 16;
  if (tid < TOK) L.eta[buf][tid] = s.eta;
}

// Four consecutive elements of one LDS row as float, plus their bf16 hi/lo.
struct Frag4 {
  f32x4 f;
  u32x2 hi, lo;
};

__device__ __forceinline__ Frag4 frag4(const uint16_t* p) {
  Frag4 r;
  r.hi = *reinterpret_cast<const u32x2*>(p);
  r.lo = u32x2{0u, 0u};
  r.f = f32x4{bf16_lo_to_f32(r.hi.x), bf16_hi_to_f32(r.hi.x), bf16_lo_to_f32(r.hi.y),
              bf16_hi_to_f32(r.hi.y)};
  return r;
}
__device__ __forceinline__ Frag4 frag4(const float* p) {
  Frag4 r;
  r.f = *reinterpret_cast<const f32x4*>(p);
  Split4 s = split4(r.f);
  r.hi = s.hi;
  r.lo = s.lo;
  return r;
}

// Four elements of one LDS column (stride `row` elements).
__device__ __forceinline__ Frag4 frag4_col(const uint16_t* p, int row) {
  Frag4 r;
  uint32_t e0 = p[0], e1 = p[row], e2 = p[2 * row], e3 = p[3 * row];
  r.hi = u32x2{e0 | (e1 << 16), e2 | (e3 << 16)};
  r.lo = u32x2{0u, 0u};
  r.f = f32x4{bf16_lo_to_f32(r.hi.x), bf16_hi_to_f32(r.hi.x), bf16_lo_to_f32(r.hi.y),
              bf16_hi_to_f32(r.hi.y)};
  return r;
}
__device__ __forceinline__ Frag4 frag4_col(const float* p, int row) {
  Frag4 r;
  r.f = f32x4{p[0], p[row], p[2 * row], p[3 * row]};
  Split4 s = split4(r.f);
  r.hi = s.hi;
  r.lo = s.lo;
  return r;
}

template <bool BF16, bool LN, bool RES, bool MB16>
__global__ __launch_bounds__(NT) void ttt_linear_fwd(LinearArgs a) {
  using E = typename Io<BF16>::E;
  constexpr int TB = Io<BF16>::TB;
  constexpr int ROW = Io<BF16>::ROW;
  constexpr int TOK = TB * 16;
  __shared__ Lds<BF16> L;

  const int tid = threadIdx.x;
  const int w = tid >> 6;          // wave: output columns 16w..16w+15
  const int lane = tid & 63;
  const int g = lane >> 4;         // lane group
  const int c = lane & 15;         // lane column
  const int unit = blockIdx.x;     // (batch, head)
  const int head = unit % a.H;
  const int T = a.T;
  const size_t row0 = (size_t)unit * T;

  // ---- prologue: state, LN parameters --------------------------------
  // Wc[r] lane (g,c) = W[16r + 4g + i][16w + c]
  f32x4 Wc[4], Wb[4];
  {
    const float* w0 = a.w0 + (size_t)(a.state0_per_batch ? unit : head) * D * D;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) Wc[r][i] = w0[(16 * r + 4 * g + i) * D + 16 * w + c];
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) Wb[r] = Wc[r];

  // lane (g,c) works on features fo..fo+3 of token c in the transposed tiles
  const int fo = 16 * w + 4 * g;
  f32x4 gam = {1.f, 1.f, 1.f, 1.f}, bet = {0.f, 0.f, 0.f, 0.f}, gam2 = gam;
  float Gam[4] = {16.f, 16.f, 16.f, 16.f};  // sum of gamma^2 over each wave's columns
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

  // identity as a 16x16x16 B operand: lane (g,c) holds I[4g + i][c]
  u32x2 ident;
  {
    uint32_t e[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) e[i] = (4 * g + i == c) ? 0x3F80u : 0u;
    ident = u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
  }

  const int n_tiles = (T + 15) / 16;
  const int n_blocks = (n_tiles + TB - 1) / TB;

  Staged<BF16> st;
  stage_load<BF16>(st, a, row0, 0, T);
  stage_store<BF16>(st, L, 0);
  __syncthreads();
  if (n_blocks > 1) stage_load<BF16>(st, a, row0, TOK, T);

  for (int blk = 0; blk < n_blocks; ++blk) {
    const int buf = blk & 1;
    const E* Lq = L.qkv[buf][0];
    const E* Lk = L.qkv[buf][1];
    const E* Lv = L.qkv[buf][2];
    for (int tb = 0; tb < TB; ++tb) {
      const int tile = blk * TB + tb;
      if (tile >= n_tiles) break;
      const int par = tile & 1;
      if (!MB16 && (tile % a.tiles_per_mb) == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) Wb[r] = Wc[r];
      }
      const E* Kt = Lk + tb * 16 * ROW;
      const E* Qt = Lq + tb * 16 * ROW;
      const E* Vt = Lv + tb * 16 * ROW;
      const int tok = tile * 16 + c;     // this lane's token (transposed layout)
      const bool valid = tok < T;
      const float eta = L.eta[buf][tb * 16 + c];

      // ---- operands from LDS ------------------------------------------
      Frag4 kc[4], qc[4], kt[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        kc[r] = frag4(Kt + c * ROW + 16 * r + 4 * g);          // K[c][16r+4g+i]
        qc[r] = frag4(Qt + c * ROW + 16 * r + 4 * g);          // Q[c][16r+4g+i]
        kt[r] = frag4_col(Kt + (4 * g) * ROW + 16 * r + c, ROW);  // K[4g+i][16r+c]
      }
      const f32x4 kres = frag4(Kt + c * ROW + fo).f;
      const f32x4 qres = frag4(Qt + c * ROW + fo).f;
      const f32x4 vres = frag4(Vt + c * ROW + fo).f;
      // K and Q rows c, features 32p + 8g + j, as 16x16x32 operands
      u32x4 krow_hi[2], krow_lo[2], qrow_hi[2], qrow_lo[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        Frag4 k0 = frag4(Kt + c * ROW + 32 * p + 8 * g);
        Frag4 k1 = frag4(Kt + c * ROW + 32 * p + 8 * g + 4);
        Frag4 q0 = frag4(Qt + c * ROW + 32 * p + 8 * g);
        Frag4 q1 = frag4(Qt + c * ROW + 32 * p + 8 * g + 4);
        krow_hi[p] = cat(k0.hi, k1.hi);
        krow_lo[p] = cat(k0.lo, k1.lo);
        qrow_hi[p] = cat(q0.hi, q1.hi);
        qrow_lo[p] = cat(q0.lo, q1.lo);
      }

      // ---- split the state into bf16 hi/lo operands ----------------------
      // A[r] as the A operand of W^T: slot j<4 -> hi of W[16r+4g+j][16w+c],
      // slot j>=4 -> lo of the same element.
      u32x4 Ab[4], Ac[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        Split4 s = split4(MB16 ? Wc[r] : Wb[r]);
        Ab[r] = cat(s.hi, s.lo);
      }
      if (MB16) {
#pragma unroll
        for (int r = 0; r < 4; ++r) Ac[r] = Ab[r];
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          Split4 s = split4(Wc[r]);
          Ac[r] = cat(s.hi, s.lo);
        }
      }

      // ---- H_k^T = W_base^T K^T  (lane: token c, features fo..fo+3) -----
      f32x4 hk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        hk = mfma32(Ab[r], cat(kc[r].hi, kc[r].hi), hk);
        if (!BF16) hk = mfma32(Ab[r], cat(kc[r].lo, kc[r].lo), hk);
      }

      // ---- gradient factor G (dl/dh of token c) ------------------------
      f32x4 G;
      if (LN) {
        const float s1 = group_sum(hk[0] + hk[1] + hk[2] + hk[3]);
        const float mw = s1 * (1.0f / 16.0f);
        f32x4 e, u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          e[i] = hk[i] - mw;
          u[i] = 2.0f * gam[i] * ((RES ? kres[i] : 0.0f) + bet[i] - vres[i]);
        }
        float P = 0.f, A = 0.f, Bq = 0.f, C = 0.f, U = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          P += e[i] * e[i];
          A += gam2[i] * e[i];
          Bq += u[i] * e[i];
          C += gam2[i] * e[i] * e[i];
          U += u[i];
        }
        P = group_sum(P);
        A = group_sum(A);
        Bq = group_sum(Bq);
        C = group_sum(C);
        U = group_sum(U);
        if (g == 0) {
          f32x4* dst = reinterpret_cast<f32x4*>(L.stats_k[par][c][w]);
          dst[0] = f32x4{s1, P, A, Bq};
          dst[1] = f32x4{C, U, 0.f, 0.f};
        }
        __syncthreads();
        f32x4 s0[4], s1v[4];
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
          const f32x4* src = reinterpret_cast<const f32x4*>(L.stats_k[par][c][ww]);
          s0[ww] = src[0];
          s1v[ww] = src[1];
        }
        const float mu = (s0[0][0] + s0[1][0] + s0[2][0] + s0[3][0]) * (1.0f / 64.0f);
        float M2 = 0.f, SgE = 0.f, SuE = 0.f, SgE2 = 0.f, Su = 0.f, dme = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
          const float dl = s0[ww][0] * (1.0f / 16.0f) - mu;   // local mean - mean
          M2 += s0[ww][1] + 16.0f * dl * dl;
          SgE += s0[ww][2] + dl * Gam[ww];
          SuE += s0[ww][3] + dl * s1v[ww][1];
          SgE2 += s1v[ww][0] + 2.0f * dl * s0[ww][2] + dl * dl * Gam[ww];
          Su += s1v[ww][1];
          if (ww == w) dme = dl;
        }
        const float rs = __frsqrt_rn(M2 * (1.0f / 64.0f) + a.eps);
        const float ma = (Su + 2.0f * rs * SgE) * (1.0f / 64.0f);
        const float max = (rs * SuE + 2.0f * rs * rs * SgE2) * (1.0f / 64.0f);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float xh = (e[i] + dme) * rs;
          const float av = u[i] + 2.0f * gam2[i] * xh;
          G[i] = rs * (av - ma - xh * max);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) G[i] = 2.0f * (hk[i] + (RES ? kres[i] : 0.0f) - vres[i]);
      }

      // -eta * G, zero for padding tokens past T
      f32x4 eg;
#pragma unroll
      for (int i = 0; i < 4; ++i) eg[i] = valid ? -eta * G[i] : 0.0f;

      // ---- transpose -eta*G on the matrix unit: lane gets token 4g+i,
      //      column 16w+c; slots j<4 hi, j>=4 lo -----------------------------
      u32x4 gop;
      {
        const Split4 s = split4(eg);
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        const f32x4 th = mfma16(s.hi, ident, zero);
        const f32x4 tl = mfma16(s.lo, ident, zero);
        gop = u32x4{pack_bf16(th[0], th[1]), pack_bf16(th[2], th[3]), pack_bf16(tl[0], tl[1]),
                    pack_bf16(tl[2], tl[3])};
      }

      // ---- output pre-activation H_q^T = W^T Q^T - (eta G)^T tril(Q K^T)^T
      f32x4 hq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        hq = mfma32(Ac[r], cat(qc[r].hi, qc[r].hi), hq);
        if (!BF16) hq = mfma32(Ac[r], cat(qc[r].lo, qc[r].lo), hq);
      }
      {
        // M = K Q^T: lane (g,c) holds M[s = 4g+i][t = c] = k_s . q_t
        f32x4 m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          m = mfma32(krow_hi[p], qrow_hi[p], m);
          if (!BF16) {
            m = mfma32(krow_hi[p], qrow_lo[p], m);
            m = mfma32(krow_lo[p], qrow_hi[p], m);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * g + i > c) m[i] = 0.0f;                 // causal: s <= t
        const Split4 ms = split4(m);
        hq = mfma32(gop, cat(ms.hi, ms.hi), hq);
        hq = mfma32(gop, cat(ms.lo, ms.lo), hq);
      }

      // ---- state update W <- W - K^T (eta G) ---------------------------
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        Wc[r] = mfma32(cat(kt[r].hi, kt[r].hi), gop, Wc[r]);
        if (!BF16) Wc[r] = mfma32(cat(kt[r].lo, kt[r].lo), gop, Wc[r]);
      }

      // ---- output: Z = Q + LN(H_q) ------------------------------------
      f32x4 zf;
      if (LN) {
        const float s1 = group_sum(hq[0] + hq[1] + hq[2] + hq[3]);
        const float mw = s1 * (1.0f / 16.0f);
        f32x4 e;
        float P = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          e[i] = hq[i] - mw;
          P += e[i] * e[i];
        }
        P = group_sum(P);
        if (g == 0) *reinterpret_cast<f32x4*>(L.stats_q[par][c][w]) = f32x4{s1, P, 0.f, 0.f};
        __syncthreads();
        f32x4 sq[4];
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) sq[ww] = *reinterpret_cast<const f32x4*>(L.stats_q[par][c][ww]);
        const float mu = (sq[0][0] + sq[1][0] + sq[2][0] + sq[3][0]) * (1.0f / 64.0f);
        float M2 = 0.f, dme = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
          const float dl = sq[ww][0] * (1.0f / 16.0f) - mu;
          M2 += sq[ww][1] + 16.0f * dl * dl;
          if (ww == w) dme = dl;
        }
        const float rs = __frsqrt_rn(M2 * (1.0f / 64.0f) + a.eps);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          zf[i] = (RES ? qres[i] : 0.0f) + gam[i] * ((e[i] + dme) * rs) + bet[i];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) zf[i] = (RES ? qres[i] : 0.0f) + hq[i];
      }
      if (valid) {
        if (BF16) {
          u32x2 o = {pack_bf16(zf[0], zf[1]), pack_bf16(zf[2], zf[3])};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.z) + (row0 + tok) * D + fo) = o;
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.z) + (row0 + tok) * D + fo) = zf;
        }
      }
    }  // tiles of the block

    if (blk + 1 < n_blocks) {
      stage_store<BF16>(st, L, buf ^ 1);
      __syncthreads();
      if (blk + 2 < n_blocks) stage_load<BF16>(st, a, row0, (blk + 2) * TOK, T);
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
