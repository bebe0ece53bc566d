// ttt_backward.hip -- the backward pass (vector-Jacobian product) of the
// TTT-Linear forward scan, for gfx950.
//
// The outer loop trains the projections behind q, k and v, the initial state
// W0 and the per-token learning rate (dmarx.github.io record LIT-801, "Key
// takeaways" item 2); with the LN parameters of the inner model that is every
// input of the scan.  Given dz [B,H,T,64] (and optionally dW_T on the final
// state) this computes the gradients of sum_t <dz_t, z_t> + <dW_T, W_T> with
// respect to q, k, v, eta, W0, gamma and beta.
//
// Forward, per mini-batch of 16 tokens with base W (items 1, 2 and 5): rows
// h_s = k_s W, x_s = LN-normalised h_s with rho_s = 1/sigma_s,
// t_s = v_s - beta - [k_s], a_s = 2 gamma (gamma x_s - t_s), the loss
// gradient at the base g_s = rho_s (a_s - mean a_s - x_s mean(a_s x_s)),
// o_i = q_i W - sum_{s<=i} eta_s (q_i . k_s) g_s,  z_i = [q_i] + LN(o_i),
// next base W - sum_s eta_s k_s^T g_s.
//
// Backward, mini-batches in reverse, A = adjoint of the next base:
//   DO  = LN backward of dZ                      (dgamma, dbeta partials)
//   dQ  = [dZ] + DO W^T - (tril(DO G^T) * eta) K
//   KA  = K A + triu(K Q^T) DO,   GA = G A^T + triu(G DO^T) Q
//   deta_s = -KA_s . g_s,  dg_s = -eta_s KA_s  -> backward of g_s -> dh_s, dt_s
//   dV  = dT,  dK = DH W^T - eta GA - [dT],  A <- A + Q^T DO + K^T DH
// and dW0 = A after the first mini-batch.  ([.] = only with the residual.)
//
// Kernel: one 256-thread workgroup per (batch, head) unit.  Phase 1 replays
// the forward recurrence of the bases and stores each mini-batch's base in
// the workspace (16 KB per mini-batch: the device has room for every base,
// so nothing is recomputed); phase 2 walks the mini-batches in reverse.
// Lane f of wave w holds column f of rows 16w..16w+15 of W, of W^T, of A and
// of A^T; a product X M of a 16-token tile X (LDS) with such a matrix is
// formed as four 16-row shares reduced through LDS, after which wave w owns
// token rows 4w..4w+3 (lane f = feature f) for the per-token LN algebra,
// whose sums are butterflies over the wave.  fp32 arithmetic throughout.
// Tokens past T (a last partial mini-batch) are zero rows with zero
// gradient factors; they add nothing and nothing is stored for them.
#include "ttt_backward.hpp"
#include "ttt_device.hpp"

namespace tttk {
namespace {

constexpr int DD = 64;         // head dimension
constexpr int NW = 4;          // waves per unit
constexpr int RW = DD / NW;    // rows of the state per wave
constexpr int TB = 16;         // tokens per mini-batch tile
constexpr int RO = TB / NW;    // token rows owned per wave
constexpr int LS = 68;         // LDS row stride of token tiles (16-byte rows, 2-way Gram reads)
constexpr int WS = 65;         // LDS row stride of the state tile (conflict-free transpose)
constexpr float INV_D = 1.0f / DD;

struct __attribute__((aligned(16))) BwdLds {
  float k[TB][LS];
  float q[TB][LS];
  float g[TB][LS];
  float dO[TB][LS];
  float dh[TB][LS];
  float w[DD][WS];
  float red[3][NW][TB][DD];   // per-wave shares of up to three products
  // masked, scaled Gram tiles (see gram_masks)
  float m1[TB][TB + 1], u1[TB][TB + 1];   // from Q K^T
  float m2[TB][TB + 1], u2[TB][TB + 1];   // from DO G^T
  float eta[TB];
  float dln[2][NW][DD];
};

template <bool BF16>
__device__ __forceinline__ float ld_io(const void* p, size_t i) {
  if constexpr (BF16) {
    const uint32_t b = static_cast<const uint16_t*>(p)[i];
    return __builtin_bit_cast(float, b << 16);
  } else {
    return static_cast<const float*>(p)[i];
  }
}

template <bool BF16>
__device__ __forceinline__ void st_io(void* p, size_t i, float x) {
  if constexpr (BF16) {
    static_cast<uint16_t*>(p)[i] = static_cast<uint16_t>(pack_bf16(x, 0.f) & 0xffffu);
  } else {
    static_cast<float*>(p)[i] = x;
  }
}

// Rows row0..row0+15 of a [.., 64] io tensor into an LDS tile; rows at or
// past `valid` are zero.  Thread tid moves 4 consecutive features.
template <bool BF16>
__device__ __forceinline__ void load_tile(float (*dst)[LS], const void* src, size_t row0,
                                          int valid, int tid) {
  const int i = tid >> 4, c = (tid & 15) * 4;
  float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
  if (i < valid) {
    const size_t e = (row0 + i) * DD + c;
    if constexpr (BF16) {
      const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(src) + e);
      x = make_float4(bf16_lo_to_f32(u.x), bf16_hi_to_f32(u.x), bf16_lo_to_f32(u.y),
                      bf16_hi_to_f32(u.y));
    } else {
      x = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + e);
    }
  }
  *reinterpret_cast<float4*>(&dst[i][c]) = x;
}

// This wave's share of the product X M for the 16 token rows of X, into
// red[slot][w]: sum_r X[i][16w + r] M[r], M[r] = column f of row 16w + r.
// (The row loop is only partly unrolled so that the LDS reads of X are not
// all hoisted into registers at once.)
__device__ __forceinline__ void share_rows(BwdLds& L, int slot, const float (*X)[LS],
                                           const float (&M)[RW], int w, int f) {
#pragma unroll 2
  for (int i = 0; i < TB; ++i) {
    const float4* x = reinterpret_cast<const float4*>(&X[i][RW * w]);
    float acc = 0.f;
#pragma unroll
    for (int m = 0; m < RW / 4; ++m) {
      const float4 y = x[m];
      acc = __builtin_fmaf(y.x, M[4 * m + 0], acc);
      acc = __builtin_fmaf(y.y, M[4 * m + 1], acc);
      acc = __builtin_fmaf(y.z, M[4 * m + 2], acc);
      acc = __builtin_fmaf(y.w, M[4 * m + 3], acc);
    }
    L.red[slot][w][i][f] = acc;
  }
}

__device__ __forceinline__ float red_sum(const BwdLds& L, int slot, int i, int f) {
  return (L.red[slot][0][i][f] + L.red[slot][1][i][f]) +
         (L.red[slot][2][i][f] + L.red[slot][3][i][f]);
}

// Row Gram matrix S[i][s] = X_i . Y_s of two 16-token tiles, stored as the
// two masked forms the token-row sums use:
//   M[i][s] = eta_s S[i][s] for s <= i (else 0)   -- sums over s <= i
//   U[s][i] = S[i][s]       for i >= s (else 0)   -- sums over i >= s
// Thread tid forms entry (tid / 16, tid % 16).
__device__ __forceinline__ void gram_masks(const float (*X)[LS], const float (*Y)[LS],
                                           const float* eta, float (*M)[TB + 1],
                                           float (*U)[TB + 1], int tid) {
  const int i = tid >> 4, s = tid & 15;
  float acc = 0.f;
#pragma unroll 4
  for (int m = 0; m < DD / 4; ++m) {
    const float4 x = *reinterpret_cast<const float4*>(&X[i][4 * m]);
    const float4 y = *reinterpret_cast<const float4*>(&Y[s][4 * m]);
    acc = __builtin_fmaf(x.x, y.x, acc);
    acc = __builtin_fmaf(x.y, y.y, acc);
    acc = __builtin_fmaf(x.z, y.z, acc);
    acc = __builtin_fmaf(x.w, y.w, acc);
  }
  M[i][s] = s <= i ? eta[s] * acc : 0.f;
  U[s][i] = i >= s ? acc : 0.f;
}

// x from another lane of the same 16-lane row (DPP control CTRL).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return bitsf(static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(fbits(x)), CTRL, 0xf, 0xf, false)));
}

// N sums over the 64 lanes of the wave at once, in every lane: butterflies
// within each 16-lane row on DPP (lanes l^1, l^2, then the mirrored lane of
// the half row and of the row), then across the four rows with permlane
// swaps -- all VALU, no LDS round trip.  Every lane ends with the same bits.
template <int N>
__device__ __forceinline__ void wave_sums(float (&x)[N]) {
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += dpp<0xB1>(x[j]);    // quad_perm 1,0,3,2
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += dpp<0x4E>(x[j]);    // quad_perm 2,3,0,1
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += dpp<0x141>(x[j]);   // row_half_mirror
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += dpp<0x140>(x[j]);   // row_mirror
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] = group_sum(x[j]);
}

// The inner loss gradient at the base for this wave's token rows, and what
// its backward needs.
struct Inner {
  float x[RO], rho[RO], t[RO], a[RO], ma[RO], mx[RO], g[RO];
};

template <bool LN, bool RES>
__device__ __forceinline__ void inner_grad(const float (&h)[RO], const float (&vr)[RO],
                                           const float (&kr)[RO], float gam, float bet,
                                           float eps, Inner& R) {
  if constexpr (LN) {
    float s[RO], xc[RO];
#pragma unroll
    for (int j = 0; j < RO; ++j) s[j] = h[j];
    wave_sums(s);
#pragma unroll
    for (int j = 0; j < RO; ++j) {
      xc[j] = h[j] - s[j] * INV_D;
      s[j] = xc[j] * xc[j];
    }
    wave_sums(s);
    float s2[2 * RO];
#pragma unroll
    for (int j = 0; j < RO; ++j) {
      R.rho[j] = 1.0f / __builtin_sqrtf(s[j] * INV_D + eps);
      R.x[j] = xc[j] * R.rho[j];
      R.t[j] = vr[j] - bet - (RES ? kr[j] : 0.f);
      R.a[j] = 2.f * gam * (gam * R.x[j] - R.t[j]);
      s2[j] = R.a[j];
      s2[RO + j] = R.a[j] * R.x[j];
    }
    wave_sums(s2);
#pragma unroll
    for (int j = 0; j < RO; ++j) {
      R.ma[j] = s2[j] * INV_D;
      R.mx[j] = s2[RO + j] * INV_D;
      R.g[j] = R.rho[j] * (R.a[j] - R.ma[j] - R.x[j] * R.mx[j]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < RO; ++j) {
      R.t[j] = vr[j] - (RES ? kr[j] : 0.f);
      R.g[j] = 2.f * (h[j] - R.t[j]);
    }
  }
}

template <bool BF16, bool LN, bool RES>
__global__ __launch_bounds__(NW * 64) void ttt_linear_bwd_k(BackwardArgs a) {
  __shared__ BwdLds L;
  const int unit = blockIdx.x;
  const int head = unit % a.H;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int f = tid & 63;
  const int T = a.T;
  const int tiles = (T + TB - 1) / TB;
  const size_t row_unit = static_cast<size_t>(unit) * T;   // first token row of the unit
  float* bases = a.ws_base + static_cast<size_t>(unit) * tiles * DD * DD;
  const float* w0 = a.w0 + (a.state0_per_batch ? static_cast<size_t>(unit)
                                                : static_cast<size_t>(head)) * DD * DD;
  float gam = 1.f, bet = 0.f;
  if (LN) {
    gam = a.gamma[head * DD + f];
    bet = a.beta[head * DD + f];
  }

  // ---- phase 1: the bases of every mini-batch ------------------------------
  float Wr[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) Wr[r] = w0[(RW * w + r) * DD + f];
  for (int c = 0; c < tiles; ++c) {
    const int t0 = c * TB;
    const int nv = min(TB, T - t0);
    load_tile<BF16>(L.k, a.k, row_unit + t0, nv, tid);
    if (tid < TB) L.eta[tid] = tid < nv ? a.eta[row_unit + t0 + tid] : 0.f;
    float vr[RO];
#pragma unroll
    for (int j = 0; j < RO; ++j) {
      const int i = RO * w + j;
      vr[j] = i < nv ? ld_io<BF16>(a.v, (row_unit + t0 + i) * DD + f) : 0.f;
    }
    float* base = bases + static_cast<size_t>(c) * DD * DD;
#pragma unroll
    for (int r = 0; r < RW; ++r) base[(RW * w + r) * DD + f] = Wr[r];
    lds_barrier();
    share_rows(L, 0, L.k, Wr, w, f);
    lds_barrier();
    float h[RO], kr[RO];
#pragma unroll
    for (int j = 0; j < RO; ++j) {
      h[j] = red_sum(L, 0, RO * w + j, f);
      kr[j] = L.k[RO * w + j][f];
    }
    Inner R;
    inner_grad<LN, RES>(h, vr, kr, gam, bet, a.eps, R);
#pragma unroll
    for (int j = 0; j < RO; ++j) {
      const int i = RO * w + j;
      L.g[i][f] = i < nv ? L.eta[i] * R.g[j] : 0.f;
    }
    lds_barrier();
    // W <- W - sum_s k_s^T (eta_s g_s) on this wave's rows
#pragma unroll 2
    for (int s = 0; s < TB; ++s) {
      const float gs = L.g[s][f];
      const float4* kk = reinterpret_cast<const float4*>(&L.k[s][RW * w]);
#pragma unroll
      for (int m = 0; m < RW / 4; ++m) {
        const float4 y = kk[m];
        Wr[4 * m + 0] = __builtin_fmaf(-y.x, gs, Wr[4 * m + 0]);
        Wr[4 * m + 1] = __builtin_fmaf(-y.y, gs, Wr[4 * m + 1]);
        Wr[4 * m + 2] = __builtin_fmaf(-y.z, gs, Wr[4 * m + 2]);
        Wr[4 * m + 3] = __builtin_fmaf(-y.w, gs, Wr[4 * m + 3]);
      }
    }
    lds_barrier();
  }

  // ---- phase 2: the mini-batches in reverse ---------------------------------
  float Ar[RW], At[RW];
  if (a.dw_final) {
    const float* A0 = a.dw_final + static_cast<size_t>(unit) * DD * DD;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      Ar[r] = A0[(RW * w + r) * DD + f];
      At[r] = A0[f * DD + RW * w + r];
    }
  } else {
#pragma unroll
    for (int r = 0; r < RW; ++r) Ar[r] = At[r] = 0.f;
  }
  float dgam = 0.f, dbet = 0.f;
  for (int c = tiles - 1; c >= 0; --c) {
    const int t0 = c * TB;
    const int nv = min(TB, T - t0);
    const float* base = bases + static_cast<size_t>(c) * DD * DD;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      Wr[r] = base[(RW * w + r) * DD + f];   // written by this thread in phase 1
      L.w[RW * w + r][f] = Wr[r];
    }
    load_tile<BF16>(L.k, a.k, row_unit + t0, nv, tid);
    load_tile<BF16>(L.q, a.q, row_unit + t0, nv, tid);
    if (tid < TB) L.eta[tid] = tid < nv ? a.eta[row_unit + t0 + tid] : 0.f;
    float vr[RO], dzr[RO];
    bool ok[RO];
#pragma unroll
    for (int j = 0; j < RO; ++j) {
      const int i = RO * w + j;
      ok[j] = i < nv;
      vr[j] = ok[j] ? ld_io<BF16>(a.v, (row_unit + t0 + i) * DD + f) : 0.f;
      dzr[j] = ok[j] ? ld_io<BF16>(a.dz, (row_unit + t0 + i) * DD + f) : 0.f;
    }
    lds_barrier();  // B1: W, K, Q, eta tiles

    float Wt[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) Wt[r] = L.w[f][RW * w + r];
    float kr[RO], er[RO];
#pragma unroll
    for (int j = 0; j < RO; ++j) {
      kr[j] = L.k[RO * w + j][f];
      er[j] = L.eta[RO * w + j];
    }
    share_rows(L, 0, L.k, Wr, w, f);   // K W
    share_rows(L, 1, L.q, Wr, w, f);   // Q W
    gram_masks(L.q, L.k, L.eta, L.m1, L.u1, tid);
    lds_barrier();  // B2: shares of K W and Q W, S1

    float qw[RO];
    Inner R;
    {
      float h[RO];
#pragma unroll
      for (int j = 0; j < RO; ++j) {
        h[j] = red_sum(L, 0, RO * w + j, f);
        qw[j] = red_sum(L, 1, RO * w + j, f);
      }
      inner_grad<LN, RES>(h, vr, kr, gam, bet, a.eps, R);
    }
#pragma unroll
    for (int j = 0; j < RO; ++j) {
      R.g[j] = ok[j] ? R.g[j] : 0.f;
      L.g[RO * w + j][f] = R.g[j];
    }
    lds_barrier();  // B3: G

    // o_i = (Q W)_i - sum_{s<=i} eta_s S1[i][s] g_s, then the output LN backward
    float dO[RO];
    {
      float o[RO];
#pragma unroll
      for (int j = 0; j < RO; ++j) {
        const int i = RO * w + j;
        float acc = qw[j];
#pragma unroll
        for (int s = 0; s < TB; ++s) acc = __builtin_fmaf(-L.m1[i][s], L.g[s][f], acc);
        o[j] = acc;
      }
      if constexpr (LN) {
        float s[RO], xc[RO];
#pragma unroll
        for (int j = 0; j < RO; ++j) s[j] = o[j];
        wave_sums(s);
#pragma unroll
        for (int j = 0; j < RO; ++j) {
          xc[j] = o[j] - s[j] * INV_D;
          s[j] = xc[j] * xc[j];
        }
        wave_sums(s);
        float xo[RO], dx[RO], s2[2 * RO];
        float rho_o[RO];
#pragma unroll
        for (int j = 0; j < RO; ++j) {
          rho_o[j] = 1.0f / __builtin_sqrtf(s[j] * INV_D + a.eps);
          xo[j] = xc[j] * rho_o[j];
          dx[j] = gam * dzr[j];
          s2[j] = dx[j];
          s2[RO + j] = dx[j] * xo[j];
          dgam += ok[j] ? dzr[j] * xo[j] : 0.f;
          dbet += dzr[j];
        }
        wave_sums(s2);
#pragma unroll
        for (int j = 0; j < RO; ++j) {
          const float d = rho_o[j] * (dx[j] - s2[j] * INV_D - xo[j] * (s2[RO + j] * INV_D));
          dO[j] = ok[j] ? d : 0.f;
        }
      } else {
#pragma unroll
        for (int j = 0; j < RO; ++j) dO[j] = dzr[j];
      }
    }
#pragma unroll
    for (int j = 0; j < RO; ++j) L.dO[RO * w + j][f] = dO[j];
    lds_barrier();  // B4: DO

    share_rows(L, 0, L.dO, Wt, w, f);   // DO W^T
    share_rows(L, 1, L.k, Ar, w, f);    // K A
    share_rows(L, 2, L.g, At, w, f);    // G A^T
    gram_masks(L.dO, L.g, L.eta, L.m2, L.u2, tid);
    lds_barrier();  // B5: shares, S2

    float ga[RO], dt[RO], dh[RO];
    {
      float ka[RO];
#pragma unroll
      for (int j = 0; j < RO; ++j) {
        const int i = RO * w + j;
        float dq = red_sum(L, 0, i, f) + (RES ? dzr[j] : 0.f);
        float kacc = red_sum(L, 1, i, f);
        float gacc = red_sum(L, 2, i, f);
#pragma unroll 4
        for (int s = 0; s < TB; ++s) {
          dq = __builtin_fmaf(-L.m2[i][s], L.k[s][f], dq);      // tokens s <= i
          kacc = __builtin_fmaf(L.u1[i][s], L.dO[s][f], kacc);  // tokens s >= i
          gacc = __builtin_fmaf(L.u2[i][s], L.q[s][f], gacc);
        }
        ka[j] = kacc;
        ga[j] = gacc;
        if (ok[j]) st_io<BF16>(a.dq, (row_unit + t0 + i) * DD + f, dq);
      }
      // deta_i = -KA_i . g_i and the backward of g_i for u = -eta_i KA_i
      float u[RO];
#pragma unroll
      for (int j = 0; j < RO; ++j) u[j] = -er[j] * ka[j];
      if constexpr (LN) {
        float s[4 * RO];
#pragma unroll
        for (int j = 0; j < RO; ++j) {
          s[j] = ka[j] * R.g[j];
          s[RO + j] = u[j] * (R.a[j] - R.ma[j] - R.x[j] * R.mx[j]);
          s[2 * RO + j] = u[j];
          s[3 * RO + j] = u[j] * R.x[j];
        }
        wave_sums(s);
        float dx[RO], da[RO], s2[2 * RO];
#pragma unroll
        for (int j = 0; j < RO; ++j) {
          const float mu_u = s[2 * RO + j] * INV_D, mux = s[3 * RO + j] * INV_D;
          da[j] = R.rho[j] * (u[j] - mu_u - R.x[j] * mux);
          dx[j] = -R.rho[j] * (R.mx[j] * u[j] + R.a[j] * mux) + 2.f * gam * gam * da[j];
          dt[j] = -2.f * gam * da[j];
          s2[j] = dx[j];
          s2[RO + j] = dx[j] * R.x[j];
        }
        wave_sums(s2);
#pragma unroll
        for (int j = 0; j < RO; ++j) {
          const float drho = s[RO + j];
          const float d = R.rho[j] * (dx[j] - s2[j] * INV_D - R.x[j] * (s2[RO + j] * INV_D)) -
                          drho * R.rho[j] * R.rho[j] * R.x[j] * INV_D;
          dh[j] = ok[j] ? d : 0.f;
          dt[j] = ok[j] ? dt[j] : 0.f;
          dgam += ok[j] ? 2.f * (2.f * gam * R.x[j] - R.t[j]) * da[j] : 0.f;
          dbet -= dt[j];
        }
        if (f == 0) {
#pragma unroll
          for (int j = 0; j < RO; ++j)
            if (ok[j]) a.deta[row_unit + t0 + RO * w + j] = -s[j];
        }
      } else {
        float s[RO];
#pragma unroll
        for (int j = 0; j < RO; ++j) s[j] = ka[j] * R.g[j];
        wave_sums(s);
#pragma unroll
        for (int j = 0; j < RO; ++j) {
          dh[j] = ok[j] ? 2.f * u[j] : 0.f;
          dt[j] = ok[j] ? -2.f * u[j] : 0.f;
        }
        if (f == 0) {
#pragma unroll
          for (int j = 0; j < RO; ++j)
            if (ok[j]) a.deta[row_unit + t0 + RO * w + j] = -s[j];
        }
      }
#pragma unroll
      for (int j = 0; j < RO; ++j) {
        const int i = RO * w + j;
        if (ok[j]) st_io<BF16>(a.dv, (row_unit + t0 + i) * DD + f, dt[j]);
        L.dh[i][f] = dh[j];
      }
    }
    lds_barrier();  // B6: DH

    share_rows(L, 0, L.dh, Wt, w, f);   // DH W^T
    // A <- A + Q^T DO + K^T DH (rows 16w + r, column f), and the same for A^T
#pragma unroll 2
    for (int i = 0; i < TB; ++i) {
      const float dOf = L.dO[i][f], dhf = L.dh[i][f], qf = L.q[i][f], kf = L.k[i][f];
      const float4* qq = reinterpret_cast<const float4*>(&L.q[i][RW * w]);
      const float4* kk = reinterpret_cast<const float4*>(&L.k[i][RW * w]);
      const float4* oo = reinterpret_cast<const float4*>(&L.dO[i][RW * w]);
      const float4* hh = reinterpret_cast<const float4*>(&L.dh[i][RW * w]);
#pragma unroll
      for (int m = 0; m < RW / 4; ++m) {
        const float4 q4 = qq[m], k4 = kk[m], o4 = oo[m], h4 = hh[m];
        Ar[4 * m + 0] = __builtin_fmaf(k4.x, dhf, __builtin_fmaf(q4.x, dOf, Ar[4 * m + 0]));
        Ar[4 * m + 1] = __builtin_fmaf(k4.y, dhf, __builtin_fmaf(q4.y, dOf, Ar[4 * m + 1]));
        Ar[4 * m + 2] = __builtin_fmaf(k4.z, dhf, __builtin_fmaf(q4.z, dOf, Ar[4 * m + 2]));
        Ar[4 * m + 3] = __builtin_fmaf(k4.w, dhf, __builtin_fmaf(q4.w, dOf, Ar[4 * m + 3]));
        At[4 * m + 0] = __builtin_fmaf(h4.x, kf, __builtin_fmaf(o4.x, qf, At[4 * m + 0]));
        At[4 * m + 1] = __builtin_fmaf(h4.y, kf, __builtin_fmaf(o4.y, qf, At[4 * m + 1]));
        At[4 * m + 2] = __builtin_fmaf(h4.z, kf, __builtin_fmaf(o4.z, qf, At[4 * m + 2]));
        At[4 * m + 3] = __builtin_fmaf(h4.w, kf, __builtin_fmaf(o4.w, qf, At[4 * m + 3]));
      }
    }
    lds_barrier();  // B7: shares of DH W^T; every tile read done
#pragma unroll
    for (int j = 0; j < RO; ++j) {
      const int i = RO * w + j;
      const float dk = red_sum(L, 0, i, f) - er[j] * ga[j] - (RES ? dt[j] : 0.f);
      if (ok[j]) st_io<BF16>(a.dk, (row_unit + t0 + i) * DD + f, dk);
    }
  }

  // ---- dW0 of this unit and its LN-parameter partial sums --------------------
  float* dst = (a.state0_per_batch ? a.dw0 : a.ws_dw0) + static_cast<size_t>(unit) * DD * DD;
#pragma unroll
  for (int r = 0; r < RW; ++r) dst[(RW * w + r) * DD + f] = Ar[r];
  L.dln[0][w][f] = dgam;
  L.dln[1][w][f] = dbet;
  lds_barrier();
  if (w == 0) {
    float* p = a.ws_dln + static_cast<size_t>(unit) * 2 * DD;
    p[f] = (L.dln[0][0][f] + L.dln[0][1][f]) + (L.dln[0][2][f] + L.dln[0][3][f]);
    p[DD + f] = (L.dln[1][0][f] + L.dln[1][1][f]) + (L.dln[1][2][f] + L.dln[1][3][f]);
  }
}

// Sums over the batch, one workgroup per head: dW0 of a shared initial state
// and the LN parameter gradients (in batch order, deterministic).
__global__ __launch_bounds__(256) void ttt_linear_bwd_sum_k(BackwardArgs a) {
  const int h = blockIdx.x;
  if (!a.state0_per_batch) {
    for (int e = threadIdx.x; e < DD * DD; e += 256) {
      float s = 0.f;
      for (int b = 0; b < a.B; ++b)
        s += a.ws_dw0[(static_cast<size_t>(b) * a.H + h) * DD * DD + e];
      a.dw0[static_cast<size_t>(h) * DD * DD + e] = s;
    }
  }
  if (a.dgamma) {
    for (int e = threadIdx.x; e < 2 * DD; e += 256) {
      float s = 0.f;
      for (int b = 0; b < a.B; ++b)
        s += a.ws_dln[(static_cast<size_t>(b) * a.H + h) * 2 * DD + e];
      if (e < DD)
        a.dgamma[h * DD + e] = s;
      else
        a.dbeta[h * DD + e - DD] = s;
    }
  }
}

template <bool BF16, bool LN>
hipError_t launch_b2(const BackwardArgs& a, bool res, hipStream_t s) {
  const dim3 grid(a.B * a.H), block(NW * 64);
  if (res)
    hipLaunchKernelGGL((ttt_linear_bwd_k<BF16, LN, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((ttt_linear_bwd_k<BF16, LN, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_backward(const BackwardArgs& a, bool bf16, bool ln, bool residual,
                                  hipStream_t stream) {
  hipError_t e;
  if (bf16)
    e = ln ? launch_b2<true, true>(a, residual, stream) : launch_b2<true, false>(a, residual, stream);
  else
    e = ln ? launch_b2<false, true>(a, residual, stream)
           : launch_b2<false, false>(a, residual, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ttt_linear_bwd_sum_k, dim3(a.H), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tttk
