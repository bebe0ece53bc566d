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
//   dQ  = [dZ] + DO W^T - M2 K,        M2 = tril(DO G^T) * eta
//   KA  = K A + U1 DO,                 U1 = triu(K Q^T)
//   GA  = G A^T + U2 Q,                U2 = triu(G DO^T)
//   deta_s = -KA_s . g_s,  dg_s = -eta_s KA_s  -> backward of g_s -> dh_s, dt_s
//   dV  = dT,  dK = DH W^T - eta GA - [dT],  A <- A + Q^T DO + K^T DH
// and dW0 = A after the first mini-batch.  ([.] = only with the residual;
// o uses M1 = tril(Q K^T) * eta the same way.)
//
// Mini-batches of 16 n tokens (n > 1; b >= T is batch GD over the whole
// sequence, item 3) are walked one 16-token tile at a time: every tile's
// gradients are taken at the mini-batch's base W_b, while its outputs see
// the state W_c at the tile's start (W_b plus the earlier tiles' updates).
// So K W, DH W^T use W_b and Q W, DO W^T use W_c, and the adjoint splits in
// two: A, of the running state (A <- A + Q^T DO per tile), and B, of the
// base (B <- B + K^T DH), folded into A at the mini-batch's first tile.
// The workspace holds W_c of every tile; W_b is the first tile's.
//
// Kernel: one 512-thread workgroup (8 waves) per (batch, head) unit.  Phase 1
// replays the forward recurrence and stores the state at every 16-token
// tile's start in the workspace (16 KB per tile: the device has room for
// all of them, so nothing is recomputed); phase 2 walks the tiles in reverse.
// With 16-token mini-batches the two phases are three launches: the replay,
// then the part of every tile that needs no adjoint (everything up to the
// output LN's backward, and dq), one workgroup per unit and tile over the
// whole device, which leaves a record per tile in the workspace, then the
// reverse walk, which only does what depends on the adjoint.
// Every product runs on the fp32 matrix unit (16x16x4 products: exact fp32
// products, fp32 accumulation): the recurrences of the states and of the
// adjoint amplify rounding on ill-conditioned units, where products of bf16
// hi/lo parts (about 16 significant bits) were not enough.  The four primal
// waves (0-3) hold column block w of W and of A (fp32 accumulators, updated
// in place) and form K W, Q W, the Q/K Grams, the output correction, K A and
// the A update; the four dual waves (4-7) hold column block w - 4 of W^T and
// A^T and form the DO/G Grams, DO W^T, G A^T, DH W^T and the A^T update.
// Each Gram tile is formed in both orientations, so every masked coefficient
// tile is already in the A-operand layout.  Product tiles go through LDS to
// the token-row algebra (LN forward and backward), where wave w owns token
// rows 2w, 2w+1 with lane f holding feature f and sums are DPP/permlane
// butterflies over the wave.  Tokens past T (a last partial tile) are zero
// rows with zero gradient factors; nothing is stored for them.
#include "ttt_backward.hpp"
#include "ttt_device.hpp"

namespace tttk {
namespace {

constexpr int DD = 64;         // head dimension
constexpr int NW = 8;          // waves per unit (two per SIMD)
constexpr int TB = 16;         // tokens per mini-batch tile
constexpr int RO = TB / NW;    // token rows owned per wave
constexpr int LS = 68;         // LDS row stride (floats): 16-byte rows, spread banks
constexpr float INV_D = 1.0f / DD;

// One mini-batch's tiles in LDS (two in flight in phase 2).
struct __attribute__((aligned(16))) TileBuf {
  float k[TB][LS];
  float q[TB][LS];
  float g[TB][LS];
  float dO[TB][LS];
  float dh[TB][LS];
  float w[DD][LS];            // the state at the tile's start
  float wb[DD][LS];           // the mini-batch's base (mini-batches of several tiles)
  float t[3][TB][LS];         // product tiles on their way to the token-row algebra
  float eta[TB];
};

struct __attribute__((aligned(16))) BwdLds {
  TileBuf b[2];
  float dln[2][NW][DD];
};

// Roles of the kernel.  kWhole: the whole pass (replay, then the reverse
// walk with every tile's front half computed on the way).  For 16-token
// mini-batches the pass runs as three launches instead: kReplay (phase 1
// alone), kFront (the front half of one tile per workgroup: the loads, K W,
// Q W, the Grams, both LNs, dq = [dZ] + DO W^T - M2 K, none of which needs
// the adjoint; every tile of every unit at once) and kBack (the reverse walk
// over the records kFront leaves: K A, G A^T, the LN-gradient backward, the
// A update and dk).
constexpr int kWhole = 0, kReplay = 1, kFront = 2, kBack = 3;

// One tile of the front half in LDS (no base of several tiles, no DH, two
// product tiles): three front workgroups fit on a CU.
struct __attribute__((aligned(16))) FrontBuf {
  float k[TB][LS];
  float q[TB][LS];
  float g[TB][LS];
  float dO[TB][LS];
  float w[DD][LS];
  float t[2][TB][LS];
  float eta[TB];
};
struct __attribute__((aligned(16))) FrontLds {
  FrontBuf b[1];
  float dln[2][NW][DD];
};
// The reverse walk's tiles (no base of several tiles): with bf16 data the
// adjoint update takes DO and DH as three bf16 parts each, stored
// transposed -- [part][feature][token pair], rows of 40 bytes -- so that a
// matrix-unit fragment (4 tokens of one feature) is one 8-byte read.
struct __attribute__((aligned(16))) BackBuf {
  float k[TB][LS];
  float q[TB][LS];
  float g[TB][LS];
  float dO[TB][LS];
  float dh[TB][LS];
  float w[DD][LS];
  float t[3][TB][LS];
  float eta[TB];
  uint32_t dot[3][DD][10];
  uint32_t dht[3][DD][10];
};
struct __attribute__((aligned(16))) BackLds {
  BackBuf b[2];
  float dln[2][NW][DD];
};
template <int ROLE>
struct LdsOf {
  using type = BwdLds;
};
template <>
struct LdsOf<kFront> {
  using type = FrontLds;
};
template <>
struct LdsOf<kBack> {
  using type = BackLds;
};

// Two values as three bf16 parts each (hi, mid, lo: about 24 significant
// bits), packed in pairs: part p of (x0, x1) in u[p].
__device__ __forceinline__ void split2x3(float x0, float x1, uint32_t (&u)[3]) {
  u[0] = pack_bf16(x0, x1);
  float r0 = x0 - bf16_lo_to_f32(u[0]), r1 = x1 - bf16_hi_to_f32(u[0]);
  u[1] = pack_bf16(r0, r1);
  r0 -= bf16_lo_to_f32(u[1]);
  r1 -= bf16_hi_to_f32(u[1]);
  u[2] = pack_bf16(r0, r1);
}
// A fragment of exact bf16 values held as fp32: the four values packed.
__device__ __forceinline__ u32x2 pack_frag(f32x4 x) {
  return u32x2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
}

// Offsets (floats) in a front record (kBwdRecFloats per unit and tile).
constexpr int REC_X = 0, REC_G = 1024, REC_DO = 2048, REC_RHO = 3072, REC_MA = 3088,
              REC_MX = 3104, REC_U1 = 3120, REC_U2 = 3376, REC_DLN = 3632;
static_assert(REC_DLN + 2 * DD <= kBwdRecFloats && kBwdRecFloats % 64 == 0,
              "front record layout");

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

// Per-token outputs of one unit go through a buffer resource whose range
// ends at the unit's last token: rows past T are dropped by the hardware, so
// the stores need no branch (a store under a branch makes the compiler wait
// for every outstanding memory operation at the loop head, the prefetch
// loads' wait included).
struct UnitOut {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ UnitOut(void* base, size_t first, uint32_t bytes) {
    r = __builtin_amdgcn_make_buffer_rsrc(static_cast<char*>(base) + first, (short)0,
                                          static_cast<int>(bytes), 0x00020000);
  }
};

// Element (token row `row` of the unit, feature f) of a [.., 64] io output.
template <bool BF16>
__device__ __forceinline__ void store_row(const UnitOut& o, int row, int f, float x) {
  if constexpr (BF16)
    __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(pack_bf16(x, 0.f) & 0xffffu),
                                          o.r, (row * DD + f) * 2, 0, 0);
  else
    __builtin_amdgcn_raw_buffer_store_b32(fbits(x), o.r, (row * DD + f) * 4, 0, 0);
}

// Tiles are fetched a mini-batch ahead into registers and stored to LDS
// when they are due.  The loads are unconditional -- rows at or past the
// last valid token re-read that token -- and the zero rows are made when
// the data is used: a load under a branch would be waited for at the end
// of the branch, which is what the prefetch is there to avoid.

// Thread tid's share of rows row0..row0+15 of a [.., 64] io tensor: 4
// consecutive features of row tid / 16 (raw; see put_fetched).
template <bool BF16>
__device__ __forceinline__ uint4 fetch_tile(const void* src, size_t row0, int valid, int tid) {
  const int i = min(tid >> 4, valid - 1), c = (tid & 15) * 4;
  const size_t e = (row0 + i) * DD + c;
  if constexpr (BF16) {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(src) + e);
    return make_uint4(u.x, u.y, 0u, 0u);
  } else {
    return *reinterpret_cast<const uint4*>(static_cast<const float*>(src) + e);
  }
}

// Store a fetched share, zero for rows at or past `valid`.
template <bool BF16>
__device__ __forceinline__ void put_fetched(float (*dst)[LS], int tid, uint4 u, int valid) {
  float4 x;
  if constexpr (BF16)
    x = make_float4(bf16_lo_to_f32(u.x), bf16_hi_to_f32(u.x), bf16_lo_to_f32(u.y),
                    bf16_hi_to_f32(u.y));
  else
    x = make_float4(bitsf(u.x), bitsf(u.y), bitsf(u.z), bitsf(u.w));
  if ((tid >> 4) >= valid) x = make_float4(0.f, 0.f, 0.f, 0.f);
  *reinterpret_cast<float4*>(&dst[tid >> 4][(tid & 15) * 4]) = x;
}

// What one mini-batch tile needs from global memory, per thread (raw).
struct Fetch {
  uint4 k;           // token-tile share (k, or q for threads 256-511 in phase 2)
  float4 w[2];       // share of the stored state at the tile's start (phase 2)
  float4 wb[2];      // share of the mini-batch's base (phase 2, several tiles)
  float eta;         // eta of token tid % 16
  float v[4], dz[4];  // this wave's token rows, feature f
  // kBack: the tile's front record -- G and DO shares (elements 2 tid,
  // 2 tid + 1), x and the LN row terms of this wave's rows, the masked Gram
  // fragment (U1 for the primal waves, U2 for the dual ones) and the front
  // half's dgamma, dbeta partial at feature f
  float2 gr, dor;
  float x[4], rho[4], ma[4], mx[4];
  f32x4 u;
  float dln0, dln1;
};

// ---- matrix-unit fragments (lane l: g = l / 16, c = l % 16) ---------------
// A 16-deep product D += A B takes, per lane, the fragment A[c][4g + i] of
// A and B[4g + i][c] of B (i = 0..3); the accumulator holds D[4g + i][c].

__device__ __forceinline__ f32x4 f4(float a, float b, float c, float d) {
  return f32x4{a, b, c, d};
}

// The four fp32 values of a fragment, as they are: every product runs on
// the fp32 matrix unit (exact fp32 products, fp32 accumulation).
using Frag = f32x4;

// D += A B over 16 k as four 16x16x4 fp32 products.  The j-th takes each
// lane's own element j (k = 4g + j), so the fragment layout above serves
// unchanged: the k order differs from the natural one, the sum does not.
__device__ __forceinline__ f32x4 mma(const Frag& a, const Frag& b, f32x4 d) {
#pragma unroll
  for (int j = 0; j < 4; ++j) d = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], d, 0, 0, 0);
  return d;
}
__device__ __forceinline__ Frag frag(f32x4 x) { return x; }

// Row fragment: X[c][col0 .. col0+3] (A operand of X, or B operand of X^T).
__device__ __forceinline__ Frag row_frag(const float (*X)[LS], int c, int col0) {
  const float4 x = *reinterpret_cast<const float4*>(&X[c][col0]);
  return f4(x.x, x.y, x.z, x.w);
}

// Column fragment: X[r0 + i][col] for i = 0..3 (B operand of X, or A
// operand of X^T).
__device__ __forceinline__ Frag col_frag(const float (*X)[LS], int r0, int col) {
  return f4(X[r0][col], X[r0 + 1][col], X[r0 + 2][col], X[r0 + 3][col]);
}

// Store an accumulator tile D[4g + i][c] at rows 0..15, columns col0 + c.
__device__ __forceinline__ void put_tile(float (*T)[LS], int g, int c, int col0, f32x4 d) {
#pragma unroll
  for (int i = 0; i < 4; ++i) T[4 * g + i][col0 + c] = d[i];
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

// One mini-batch's per-wave registers between its phase-2 steps.
struct TileRegs {
  int t0, nv;
  bool ok[RO];
  float vr[RO], dzr[RO], kr[RO], er[RO];
  f32x4 qw, s1, s1t;   // primal waves
  Frag Wt[4];        // dual waves
  Inner R;
  float ga[RO], dt[RO];
  f32x4 u;           // kBack: U1 (primal) or U2 (dual) from the front record
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

template <bool BF16, bool LN, bool RES, bool MB16, int ROLE>
__global__ __launch_bounds__(NW * 64) void ttt_linear_bwd_k(BackwardArgs a) {
  static_assert(ROLE == kWhole || MB16, "the split roles are for 16-token mini-batches");
  __shared__ typename LdsOf<ROLE>::type L;
  const int T = a.T;
  const int tiles = (T + TB - 1) / TB;
  // kFront: one workgroup per (unit, tile), tile fastest
  const int unit = ROLE == kFront ? static_cast<int>(blockIdx.x) / tiles
                                  : static_cast<int>(blockIdx.x);
  const int head = unit % a.H;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // waves 0-3 hold W and A (column block w), waves 4-7 W^T and A^T (column
  // block w - 4); wave w shares its SIMD with wave w +- 4
  const bool primal = w < 4;
  const int cb = w & 3;
  const int f = tid & 63;                                   // feature of the token-row algebra
  const int g = f >> 4, c = f & 15;                         // matrix-unit lane coordinates
  const int col = 16 * cb + c;                              // this lane's product column
  const int nmb = MB16 ? 1 : a.tiles_per_mb;   // 16-token tiles per mini-batch
  const size_t row_unit = static_cast<size_t>(unit) * T;   // first token row of the unit
  float* bases = a.ws_base + static_cast<size_t>(unit) * tiles * DD * DD;
  const float* w0 = a.w0 + (a.state0_per_batch ? static_cast<size_t>(unit)
                                                : static_cast<size_t>(head)) * DD * DD;
  float gam = 1.f, bet = 0.f;
  if (LN) {
    gam = a.gamma[head * DD + f];
    bet = a.beta[head * DD + f];
  }
  const int tq = tid & 255;              // share of a token tile (threads 0-255: k, 256-511: q)

  // ---- phase 1: the bases of every mini-batch ------------------------------
  // Wacc[rt][i] = W[16 rt + 4g + i][col] (updated by the primal waves only;
  // the base stores of the dual waves go to a zero-range resource)
  Fetch F;
  if constexpr (ROLE == kWhole || ROLE == kReplay) {
  f32x4 Wacc[4], Wb[4];   // the state and (several tiles per mini-batch) its base
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) Wacc[rt][i] = w0[(16 * rt + 4 * g + i) * DD + col];
  const __amdgpu_buffer_rsrc_t rbase = __builtin_amdgcn_make_buffer_rsrc(
      bases, (short)0, primal ? static_cast<int>(static_cast<uint32_t>(tiles) * DD * DD * 4) : 0,
      0x00020000);
  // tile ct's k, eta and v rows, fetched while tile ct - 1 computes
  auto fetch1 = [&](int ct, Fetch& F) {
    const int t0 = ct * TB;
    const int nv = min(TB, T - t0);
    F.k = fetch_tile<BF16>(a.k, row_unit + t0, nv, tq);
    F.eta = a.eta[row_unit + t0 + min(tid & 15, nv - 1)];
#pragma unroll
    for (int j = 0; j < RO; ++j)
      F.v[j] = ld_io<BF16>(a.v, (row_unit + t0 + min(RO * w + j, nv - 1)) * DD + f);
  };
  if (!a.bases_saved) fetch1(0, F);
  for (int ct = 0; ct < tiles && !a.bases_saved; ++ct) {
    const int t0 = ct * TB;
    const int nv = min(TB, T - t0);
    if (!MB16 && ct % nmb == 0) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) Wb[rt] = Wacc[rt];
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_buffer_store_b32(
            fbits(Wacc[rt][i]), rbase, ((ct * DD + 16 * rt + 4 * g + i) * DD + col) * 4, 0, 0);
    if (tid < 256) put_fetched<BF16>(L.b[0].k, tq, F.k, nv);
    if (tid < TB) L.b[0].eta[tid] = tid < nv ? F.eta : 0.f;
    float vr[RO];
#pragma unroll
    for (int j = 0; j < RO; ++j) vr[j] = RO * w + j < nv ? F.v[j] : 0.f;
    fetch1(min(ct + 1, tiles - 1), F);   // unconditional: the last one re-reads a tile
    lds_barrier();
    if (primal) {
      f32x4 h = f4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        h = mma(row_frag(L.b[0].k, c, 16 * kt + 4 * g),
                             frag(MB16 ? Wacc[kt] : Wb[kt]), h);
      put_tile(L.b[0].t[0], g, c, 16 * cb, h);
    }
    lds_barrier();
    {
      float h[RO], kr[RO];
#pragma unroll
      for (int j = 0; j < RO; ++j) {
        h[j] = L.b[0].t[0][RO * w + j][f];
        kr[j] = L.b[0].k[RO * w + j][f];
      }
      Inner R;
      inner_grad<LN, RES>(h, vr, kr, gam, bet, a.eps, R);
#pragma unroll
      for (int j = 0; j < RO; ++j) {
        const int i = RO * w + j;
        L.b[0].g[i][f] = i < nv ? -L.b[0].eta[i] * R.g[j] : 0.f;   // -eta g: the update's right factor
      }
    }
    lds_barrier();
    if (primal) {
      // W[:, cols] += K^T (-eta G)[:, cols]; row tile rt of W takes the
      // A operand K^T[16 rt + c][4g + i] = K[4g + i][16 rt + c]
      const Frag ug = col_frag(L.b[0].g, 4 * g, col);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
        Wacc[rt] = mma(col_frag(L.b[0].k, 4 * g, 16 * rt + c), ug, Wacc[rt]);
    }
    lds_barrier();
  }
  __syncthreads();   // every base stored before any wave reads one back
  }
  if constexpr (ROLE == kReplay) return;

  // ---- phase 2: the mini-batches in reverse, two in flight ------------------
  // Only part of a mini-batch's work needs A, the adjoint carried between
  // mini-batches (K A, G A^T, the LN-gradient backward, the A update, dK);
  // the front part of the next (earlier) mini-batch -- its loads, K W, Q W,
  // the Grams and both LNs -- does not.  Each barrier interval pairs a
  // token-row step of one mini-batch with a matrix-unit step of the other,
  // in separate LDS buffers:
  //   I1: back S5(c)  + front S0(c-1)      I2: back S6(c) + front S1(c-1)
  //   I3: back S7(c)  + front S2(c-1)      I4: back S8(c) + front S3(c-1)
  //   I5: front S4(c-1)
  constexpr uint32_t ES = BF16 ? 2 : 4;
  const UnitOut o_dq(a.dq, row_unit * DD * ES, static_cast<uint32_t>(T) * DD * ES);
  const UnitOut o_dk(a.dk, row_unit * DD * ES, static_cast<uint32_t>(T) * DD * ES);
  const UnitOut o_dv(a.dv, row_unit * DD * ES, static_cast<uint32_t>(T) * DD * ES);
  const UnitOut o_de(a.deta, row_unit * 4, static_cast<uint32_t>(T) * 4);
  // Am: the primal waves' A[16 rt + 4g + i][col], the dual waves'
  // A^T[16 rt + 4g + i][col] = A[col][16 rt + 4g + i]; from dw_final through
  // a buffer resource of zero range when it is NULL (reads return zero)
  // Bm: the adjoint of the mini-batch's base from its tiles' gradients so
  // far (several tiles per mini-batch), folded into Am at its first tile
  f32x4 Am[4], Bm[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) Bm[rt] = f4(0.f, 0.f, 0.f, 0.f);
  if constexpr (ROLE != kFront) {
    const float* A0 = a.dw_final ? a.dw_final + static_cast<size_t>(unit) * DD * DD : a.w0;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(A0), (short)0, a.dw_final ? DD * DD * 4 : 0, 0x00020000);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * g + i;
        Am[rt][i] = bitsf(__builtin_amdgcn_raw_buffer_load_b32(
            ra, (primal ? r * DD + col : col * DD + r) * 4, 0, 0));
      }
  }
  // tile ct's base, k (threads 0-255) or q (256-511), eta, v and dz rows,
  // fetched two stages ahead (float4 e of the base: row e / 16, columns
  // 4 (e % 16) ..)
  const void* kq = tid < 256 ? a.k : a.q;
  auto fetch2 = [&](int ct, Fetch& F) {
    const int t0 = ct * TB;
    const int nv = min(TB, T - t0);
    const float4* base =
        reinterpret_cast<const float4*>(bases + static_cast<size_t>(ct) * DD * DD);
#pragma unroll
    for (int m = 0; m < 2; ++m) F.w[m] = base[tid + NW * 64 * m];
    if (!MB16) {
      const float4* mb = reinterpret_cast<const float4*>(
          bases + static_cast<size_t>(ct - ct % nmb) * DD * DD);
#pragma unroll
      for (int m = 0; m < 2; ++m) F.wb[m] = mb[tid + NW * 64 * m];
    }
    F.k = fetch_tile<BF16>(kq, row_unit + t0, nv, tq);
    F.eta = a.eta[row_unit + t0 + min(tid & 15, nv - 1)];
#pragma unroll
    for (int j = 0; j < RO; ++j) {
      const size_t row = row_unit + t0 + min(RO * w + j, nv - 1);
      F.v[j] = ld_io<BF16>(a.v, row * DD + f);
      if constexpr (ROLE != kBack) F.dz[j] = ld_io<BF16>(a.dz, row * DD + f);
    }
    if constexpr (ROLE == kBack) {
      const float* rec = a.ws_front + (static_cast<size_t>(unit) * tiles + ct) * kBwdRecFloats;
      F.gr = reinterpret_cast<const float2*>(rec + REC_G)[tid];
      F.dor = reinterpret_cast<const float2*>(rec + REC_DO)[tid];
#pragma unroll
      for (int j = 0; j < RO; ++j) {
        const int i = RO * w + j;
        if constexpr (LN) {
          F.x[j] = rec[REC_X + i * DD + f];
          F.rho[j] = rec[REC_RHO + i];
          F.ma[j] = rec[REC_MA + i];
          F.mx[j] = rec[REC_MX + i];
        }
      }
      F.u = reinterpret_cast<const f32x4*>(rec + (primal ? REC_U1 : REC_U2))[f];
      F.dln0 = rec[REC_DLN + f];
      F.dln1 = rec[REC_DLN + DD + f];
    }
  };
  float dgam = 0.f, dbet = 0.f;

  // S0: the prefetched tile ct into buffer X, its rows into S; fetch ct - 1
  auto S0 = [&](int ct, auto& X, TileRegs& S) {
    S.t0 = ct * TB;
    S.nv = min(TB, T - S.t0);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int e = tid + NW * 64 * m;
      *reinterpret_cast<float4*>(&X.w[e >> 4][4 * (e & 15)]) = F.w[m];
      if constexpr (!MB16) *reinterpret_cast<float4*>(&X.wb[e >> 4][4 * (e & 15)]) = F.wb[m];
    }
    put_fetched<BF16>(tid < 256 ? X.k : X.q, tq, F.k, S.nv);
    if (tid < TB) X.eta[tid] = tid < S.nv ? F.eta : 0.f;
#pragma unroll
    for (int j = 0; j < RO; ++j) {
      S.ok[j] = RO * w + j < S.nv;
      S.vr[j] = S.ok[j] ? F.v[j] : 0.f;
      S.dzr[j] = S.ok[j] ? F.dz[j] : 0.f;
    }
    if constexpr (ROLE == kBack) {
      // the front record: G and DO to LDS (zero rows past T as written),
      // the LN row terms and the Gram fragment to registers, and the front
      // half's LN-parameter partial into wave 0's sums
      *reinterpret_cast<float2*>(&X.g[(2 * tid) >> 6][(2 * tid) & 63]) = F.gr;
      *reinterpret_cast<float2*>(&X.dO[(2 * tid) >> 6][(2 * tid) & 63]) = F.dor;
#pragma unroll
      for (int j = 0; j < RO; ++j) {
        S.R.x[j] = F.x[j];
        S.R.rho[j] = F.rho[j];
        S.R.ma[j] = F.ma[j];
        S.R.mx[j] = F.mx[j];
      }
      S.u = F.u;
      if (w == 0) {
        dgam += F.dln0;
        dbet += F.dln1;
      }
    }
    // unconditional (the last one re-reads a tile); kFront has one tile
    if constexpr (ROLE != kFront) fetch2(max(ct - 1, 0), F);
  };
  // S1: primal: K W (to the row algebra), Q W, the two Q/K Grams; dual: its
  // W^T column block (B operand) for DO W^T and DH W^T
  auto S1 = [&](auto& X, TileRegs& S) {
    if (primal) {
      f32x4 h = f4(0.f, 0.f, 0.f, 0.f);
      S.qw = h;
      S.s1 = h;
      S.s1t = h;
      u32x2 qb[4], kb[4];   // bf16 data: the rows as bf16 (exact) for the Grams
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const Frag wb = col_frag(X.w, 16 * kt + 4 * g, col);   // W[16kt + 4g + i][col]
        const Frag kf = row_frag(X.k, c, 16 * kt + 4 * g);
        const Frag qf = row_frag(X.q, c, 16 * kt + 4 * g);
        if constexpr (MB16)
          h = mma(kf, wb, h);
        else
          h = mma(kf, col_frag(X.wb, 16 * kt + 4 * g, col), h);
        S.qw = mma(qf, wb, S.qw);
        if constexpr (BF16) {
          qb[kt] = u32x2{pack_bf16(qf[0], qf[1]), pack_bf16(qf[2], qf[3])};
          kb[kt] = u32x2{pack_bf16(kf[0], kf[1]), pack_bf16(kf[2], kf[3])};
        } else {
          S.s1 = mma(qf, kf, S.s1);     // s1[i]  = q_{4g+i} . k_c
          S.s1t = mma(kf, qf, S.s1t);   // s1t[i] = k_{4g+i} . q_c
        }
      }
      if constexpr (BF16) {
        // the same Grams from the exact bf16 rows: two 16x16x32 products each
        // (bf16 x bf16 products are exact in fp32) instead of 32 fp32 ones
#pragma unroll
        for (int kp = 0; kp < 4; kp += 2) {
          S.s1 = mfma32(cat(qb[kp], qb[kp + 1]), cat(kb[kp], kb[kp + 1]), S.s1);
          S.s1t = mfma32(cat(kb[kp], kb[kp + 1]), cat(qb[kp], qb[kp + 1]), S.s1t);
        }
      }
      put_tile(X.t[0], g, c, 16 * cb, h);
    } else {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) S.Wt[kt] = row_frag(X.w, col, 16 * kt + 4 * g);
    }
#pragma unroll
    for (int j = 0; j < RO; ++j) {
      S.kr[j] = X.k[RO * w + j][f];
      S.er[j] = X.eta[RO * w + j];
    }
  };
  // S2: the inner LN gradient G on this wave's rows
  auto S2 = [&](auto& X, TileRegs& S) {
    float h[RO];
#pragma unroll
    for (int j = 0; j < RO; ++j) h[j] = X.t[0][RO * w + j][f];
    inner_grad<LN, RES>(h, S.vr, S.kr, gam, bet, a.eps, S.R);
#pragma unroll
    for (int j = 0; j < RO; ++j) {
      S.R.g[j] = S.ok[j] ? S.R.g[j] : 0.f;
      X.g[RO * w + j][f] = S.R.g[j];
    }
  };
  // S3: o = Q W - M1 G with M1[c][s] = eta_s (q_c . k_s) for s <= c, whose
  // A-layout entries (row c, column s = 4g + i) are s1t
  auto S3 = [&](auto& X, TileRegs& S) {
    if (primal) {
      float m[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = 4 * g + i;
        m[i] = s <= c ? -X.eta[s] * S.s1t[i] : 0.f;
      }
      const f32x4 o =
          mma(frag(f4(m[0], m[1], m[2], m[3])), col_frag(X.g, 4 * g, col), S.qw);
      put_tile(X.t[1], g, c, 16 * cb, o);
    }
  };
  // S4: the output LN backward on this wave's rows
  auto S4 = [&](auto& X, TileRegs& S) {
    float dO[RO];
    if constexpr (LN) {
      float o[RO], s[RO], xc[RO];
#pragma unroll
      for (int j = 0; j < RO; ++j) s[j] = o[j] = X.t[1][RO * w + j][f];
      wave_sums(s);
#pragma unroll
      for (int j = 0; j < RO; ++j) {
        xc[j] = o[j] - s[j] * INV_D;
        s[j] = xc[j] * xc[j];
      }
      wave_sums(s);
      float xo[RO], dx[RO], s2[2 * RO], rho_o[RO];
#pragma unroll
      for (int j = 0; j < RO; ++j) {
        rho_o[j] = 1.0f / __builtin_sqrtf(s[j] * INV_D + a.eps);
        xo[j] = xc[j] * rho_o[j];
        dx[j] = gam * S.dzr[j];
        s2[j] = dx[j];
        s2[RO + j] = dx[j] * xo[j];
        dgam += S.ok[j] ? S.dzr[j] * xo[j] : 0.f;
        dbet += S.dzr[j];
      }
      wave_sums(s2);
#pragma unroll
      for (int j = 0; j < RO; ++j) {
        const float d = rho_o[j] * (dx[j] - s2[j] * INV_D - xo[j] * (s2[RO + j] * INV_D));
        dO[j] = S.ok[j] ? d : 0.f;
      }
    } else {
#pragma unroll
      for (int j = 0; j < RO; ++j) dO[j] = S.dzr[j];
    }
#pragma unroll
    for (int j = 0; j < RO; ++j) X.dO[RO * w + j][f] = dO[j];
  };
  // S5: primal: KA = K A + U1 DO; dual: dQ' = DO W^T - M2 K and
  // GA = G A^T + U2 Q with the DO/G Grams.  M2, U1, U2 in A layout (row c,
  // column s = 4g + i).
  // U1 in A layout from the primal waves' Q/K Gram
  auto u1_of = [&](const TileRegs& S) {
    f32x4 u1;
#pragma unroll
    for (int i = 0; i < 4; ++i) u1[i] = 4 * g + i >= c ? S.s1[i] : 0.f;   // q_s . k_c, s >= c
    return u1;
  };
  auto S5 = [&](auto& X, TileRegs& S) {
    if (primal) {
      f32x4 pka = f4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        pka = mma(row_frag(X.k, c, 16 * kt + 4 * g), frag(Am[kt]), pka);
      const f32x4 u1 = ROLE == kBack ? S.u : u1_of(S);
      pka = mma(frag(u1), col_frag(X.dO, 4 * g, col), pka);
      put_tile(X.t[1], g, c, 16 * cb, pka);
    } else if constexpr (ROLE == kBack) {
      // G A^T + U2 Q, U2 from the record (dq was the front half's)
      f32x4 pga = f4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        pga = mma(row_frag(X.g, c, 16 * kt + 4 * g), frag(Am[kt]), pga);
      pga = mma(frag(S.u), col_frag(X.q, 4 * g, col), pga);
      put_tile(X.t[2], g, c, 16 * cb, pga);
    } else {
      f32x4 pdq = f4(0.f, 0.f, 0.f, 0.f), pga = pdq, s2 = pdq, s2t = pdq;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const Frag df = row_frag(X.dO, c, 16 * kt + 4 * g);
        const Frag gf = row_frag(X.g, c, 16 * kt + 4 * g);
        pdq = mma(df, S.Wt[kt], pdq);
        pga = mma(gf, frag(Am[kt]), pga);
        s2 = mma(df, gf, s2);     // s2[i]  = do_{4g+i} . g_c
        s2t = mma(gf, df, s2t);   // s2t[i] = g_{4g+i} . do_c
      }
      float m2[4], u2[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = 4 * g + i;
        m2[i] = s <= c ? -X.eta[s] * s2t[i] : 0.f;   // -eta_s (do_c . g_s), s <= c
        u2[i] = s >= c ? s2[i] : 0.f;                // do_s . g_c, s >= c
      }
      pdq = mma(frag(f4(m2[0], m2[1], m2[2], m2[3])),
                             col_frag(X.k, 4 * g, col), pdq);
      pga = mma(frag(f4(u2[0], u2[1], u2[2], u2[3])),
                             col_frag(X.q, 4 * g, col), pga);
      put_tile(X.t[0], g, c, 16 * cb, pdq);
      put_tile(X.t[2], g, c, 16 * cb, pga);
    }
  };
  // kFront: the adjoint-free part of S5 -- dual: dQ' = DO W^T - M2 K into
  // t[0] and U2 (from the DO/G Grams) into the record; primal wave 0: U1
  auto S5f = [&](auto& X, TileRegs& S, float* rec) {
    if (primal) {
      if (w == 0) reinterpret_cast<f32x4*>(rec + REC_U1)[f] = u1_of(S);
    } else {
      f32x4 pdq = f4(0.f, 0.f, 0.f, 0.f), s2 = pdq, s2t = pdq;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const Frag df = row_frag(X.dO, c, 16 * kt + 4 * g);
        const Frag gf = row_frag(X.g, c, 16 * kt + 4 * g);
        pdq = mma(df, S.Wt[kt], pdq);
        s2 = mma(df, gf, s2);     // s2[i]  = do_{4g+i} . g_c
        s2t = mma(gf, df, s2t);   // s2t[i] = g_{4g+i} . do_c
      }
      f32x4 m2, u2;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = 4 * g + i;
        m2[i] = s <= c ? -X.eta[s] * s2t[i] : 0.f;   // -eta_s (do_c . g_s), s <= c
        u2[i] = s >= c ? s2[i] : 0.f;                // do_s . g_c, s >= c
      }
      pdq = mma(frag(m2), col_frag(X.k, 4 * g, col), pdq);
      put_tile(X.t[0], g, c, 16 * cb, pdq);
      if (w == 4) reinterpret_cast<f32x4*>(rec + REC_U2)[f] = u2;
    }
  };
  // S6: dq, deta and the LN-gradient backward on this wave's rows: DH, dv
  auto S6 = [&](auto& X, TileRegs& S) {
    const int t0 = S.t0;
    float ka[RO], dh[RO];
    if constexpr (ROLE == kBack) {
      // what S1 and S2 would have left: eta and k rows, g, and t, a from the
      // record's x (the same operations, so the same values)
#pragma unroll
      for (int j = 0; j < RO; ++j) {
        const int i = RO * w + j;
        S.er[j] = X.eta[i];
        S.kr[j] = X.k[i][f];
        S.R.g[j] = X.g[i][f];
        if constexpr (LN) {
          S.R.t[j] = S.vr[j] - bet - (RES ? S.kr[j] : 0.f);
          S.R.a[j] = 2.f * gam * (gam * S.R.x[j] - S.R.t[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < RO; ++j) {
      const int i = RO * w + j;
      ka[j] = X.t[1][i][f];
      S.ga[j] = X.t[2][i][f];
      if constexpr (ROLE != kBack) {
        const float dq = X.t[0][i][f] + (RES ? S.dzr[j] : 0.f);
        store_row<BF16>(o_dq, t0 + i, f, dq);
      }
    }
    // deta_i = -KA_i . g_i and the backward of g_i for u = -eta_i KA_i
    float u[RO], de[RO];
#pragma unroll
    for (int j = 0; j < RO; ++j) u[j] = -S.er[j] * ka[j];
    const Inner& R = S.R;
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
        de[j] = -s[j];
        const float mu_u = s[2 * RO + j] * INV_D, mux = s[3 * RO + j] * INV_D;
        da[j] = R.rho[j] * (u[j] - mu_u - R.x[j] * mux);
        dx[j] = -R.rho[j] * (R.mx[j] * u[j] + R.a[j] * mux) + 2.f * gam * gam * da[j];
        S.dt[j] = -2.f * gam * da[j];
        s2[j] = dx[j];
        s2[RO + j] = dx[j] * R.x[j];
      }
      wave_sums(s2);
#pragma unroll
      for (int j = 0; j < RO; ++j) {
        const float drho = s[RO + j];
        const float d = R.rho[j] * (dx[j] - s2[j] * INV_D - R.x[j] * (s2[RO + j] * INV_D)) -
                        drho * R.rho[j] * R.rho[j] * R.x[j] * INV_D;
        dh[j] = S.ok[j] ? d : 0.f;
        S.dt[j] = S.ok[j] ? S.dt[j] : 0.f;
        dgam += S.ok[j] ? 2.f * (2.f * gam * R.x[j] - R.t[j]) * da[j] : 0.f;
        dbet -= S.dt[j];
      }
    } else {
      float s[RO];
#pragma unroll
      for (int j = 0; j < RO; ++j) s[j] = ka[j] * R.g[j];
      wave_sums(s);
#pragma unroll
      for (int j = 0; j < RO; ++j) {
        de[j] = -s[j];
        dh[j] = S.ok[j] ? 2.f * u[j] : 0.f;
        S.dt[j] = S.ok[j] ? -2.f * u[j] : 0.f;
      }
    }
    {
      // lanes 0 .. RO-1 store this wave's rows (the others are dropped)
      const int off = f < RO ? (t0 + RO * w + f) * 4 : 0x7ffffff0;
      __builtin_amdgcn_raw_buffer_store_b32(fbits(f == 0 ? de[0] : de[RO - 1]), o_de.r, off, 0,
                                            0);
    }
#pragma unroll
    for (int j = 0; j < RO; ++j) {
      const int i = RO * w + j;
      store_row<BF16>(o_dv, t0 + i, f, S.dt[j]);
      X.dh[i][f] = dh[j];
    }
    if constexpr (ROLE == kBack && BF16) {
      // DO and DH of this wave's two token rows in three bf16 parts,
      // transposed, for the adjoint update
      static_assert(RO == 2, "one token pair per wave");
      uint32_t po[3], ph[3];
      split2x3(X.dO[RO * w][f], X.dO[RO * w + 1][f], po);
      split2x3(dh[0], dh[1], ph);
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        X.dot[p][f][w] = po[p];
        X.dht[p][f][w] = ph[p];
      }
    }
  };
  // S7: primal: A += Q^T DO + K^T DH; dual: DH W^T, and A^T += DO^T Q +
  // DH^T K.  The A operand of row tile rt of X^T is X[4g + i][16 rt + c].
  // With several tiles per mini-batch the output term Q^T DO goes to the
  // adjoint of the state at the tile's start and the gradient term K^T DH
  // to that of the mini-batch's base (Bm); the two meet at its first tile.
  auto S7 = [&](auto& X, TileRegs& S) {
    if constexpr (ROLE == kBack && BF16) {
      // q and k are exact in bf16: Q^T DO and K^T DH as bf16 products with DO
      // and DH in three parts -- hi and mid paired in one 32-deep product,
      // the two lo parts in another; exact products, fp32 accumulation.
      // The chain keeps one product shape: a 16-deep product accumulating
      // right behind a 32-deep one gave wrong values here.
      auto parts = [&](const uint32_t (&t)[3][DD][10], int feat, u32x2 (&o)[3]) {
#pragma unroll
        for (int p = 0; p < 3; ++p) o[p] = *reinterpret_cast<const u32x2*>(&t[p][feat][2 * g]);
      };
      if (primal) {
        u32x2 dop[3], dhp[3];   // B operands: DO, DH [4g + i][col]
        parts(X.dot, col, dop);
        parts(X.dht, col, dhp);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const u32x2 qa = pack_frag(col_frag(X.q, 4 * g, 16 * rt + c));   // Q^T[16 rt + c][4g + i]
          const u32x2 ka = pack_frag(col_frag(X.k, 4 * g, 16 * rt + c));
          Am[rt] = mfma32(cat(qa, qa), cat(dop[0], dop[1]), Am[rt]);
          Am[rt] = mfma32(cat(qa, ka), cat(dop[2], dhp[2]), Am[rt]);
          Am[rt] = mfma32(cat(ka, ka), cat(dhp[0], dhp[1]), Am[rt]);
        }
      } else {
        f32x4 pdk = f4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          pdk = mma(row_frag(X.dh, c, 16 * kt + 4 * g), row_frag(X.w, col, 16 * kt + 4 * g), pdk);
        put_tile(X.t[0], g, c, 16 * cb, pdk);
        const u32x2 qb = pack_frag(col_frag(X.q, 4 * g, col));   // B operands: Q, K [4g + i][col]
        const u32x2 kb = pack_frag(col_frag(X.k, 4 * g, col));
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          u32x2 dop[3], dhp[3];   // A operands: DO^T, DH^T [16 rt + c][4g + i]
          parts(X.dot, 16 * rt + c, dop);
          parts(X.dht, 16 * rt + c, dhp);
          Am[rt] = mfma32(cat(dop[0], dop[1]), cat(qb, qb), Am[rt]);
          Am[rt] = mfma32(cat(dop[2], dhp[2]), cat(qb, kb), Am[rt]);
          Am[rt] = mfma32(cat(dhp[0], dhp[1]), cat(kb, kb), Am[rt]);
        }
      }
    } else {
    if (primal) {
      const Frag dob = col_frag(X.dO, 4 * g, col), dhb = col_frag(X.dh, 4 * g, col);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        Am[rt] = mma(col_frag(X.q, 4 * g, 16 * rt + c), dob, Am[rt]);
        if (MB16)
          Am[rt] = mma(col_frag(X.k, 4 * g, 16 * rt + c), dhb, Am[rt]);
        else
          Bm[rt] = mma(col_frag(X.k, 4 * g, 16 * rt + c), dhb, Bm[rt]);
      }
    } else {
      f32x4 pdk = f4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        if constexpr (ROLE == kBack)
          pdk = mma(row_frag(X.dh, c, 16 * kt + 4 * g), row_frag(X.w, col, 16 * kt + 4 * g), pdk);
        else if constexpr (MB16)
          pdk = mma(row_frag(X.dh, c, 16 * kt + 4 * g), S.Wt[kt], pdk);
        else
          pdk = mma(row_frag(X.dh, c, 16 * kt + 4 * g), row_frag(X.wb, col, 16 * kt + 4 * g), pdk);
      }
      put_tile(X.t[0], g, c, 16 * cb, pdk);
      const Frag qb = col_frag(X.q, 4 * g, col), kb = col_frag(X.k, 4 * g, col);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        Am[rt] = mma(col_frag(X.dO, 4 * g, 16 * rt + c), qb, Am[rt]);
        if (MB16)
          Am[rt] = mma(col_frag(X.dh, 4 * g, 16 * rt + c), kb, Am[rt]);
        else
          Bm[rt] = mma(col_frag(X.dh, 4 * g, 16 * rt + c), kb, Bm[rt]);
      }
    }
    }
    if (!MB16 && (S.t0 / TB) % nmb == 0) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        Am[rt] += Bm[rt];
        Bm[rt] = f4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };
  // S8: dk on this wave's rows
  auto S8 = [&](auto& X, TileRegs& S) {
#pragma unroll
    for (int j = 0; j < RO; ++j) {
      const int i = RO * w + j;
      const float dk = X.t[0][i][f] - S.er[j] * S.ga[j] - (RES ? S.dt[j] : 0.f);
      store_row<BF16>(o_dk, S.t0 + i, f, dk);
    }
  };

  if constexpr (ROLE == kFront) {
    // one tile: its front half and its record
    const int ct = static_cast<int>(blockIdx.x) % tiles;
    float* rec = a.ws_front + (static_cast<size_t>(unit) * tiles + ct) * kBwdRecFloats;
    auto& X = L.b[0];
    TileRegs S;
    fetch2(ct, F);
    S0(ct, X, S);
    lds_barrier();
    S1(X, S);
    lds_barrier();
    S2(X, S);
    lds_barrier();
    S3(X, S);
    lds_barrier();
    S4(X, S);
    lds_barrier();
    S5f(X, S, rec);
    lds_barrier();
#pragma unroll
    for (int j = 0; j < RO; ++j) {
      const int i = RO * w + j;
      store_row<BF16>(o_dq, S.t0 + i, f, X.t[0][i][f] + (RES ? S.dzr[j] : 0.f));
      rec[REC_G + i * DD + f] = S.R.g[j];
      rec[REC_DO + i * DD + f] = X.dO[i][f];
      if constexpr (LN) {
        rec[REC_X + i * DD + f] = S.R.x[j];
        if (f == 0) {
          rec[REC_RHO + i] = S.R.rho[j];
          rec[REC_MA + i] = S.R.ma[j];
          rec[REC_MX + i] = S.R.mx[j];
        }
      }
    }
    // the tile's dgamma, dbeta (output LN), summed over the waves in order
    L.dln[0][w][f] = dgam;
    L.dln[1][w][f] = dbet;
    lds_barrier();
    if (w == 0) {
      float sg = 0.f, sb = 0.f;
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        sg += L.dln[0][v][f];
        sb += L.dln[1][v][f];
      }
      rec[REC_DLN + f] = sg;
      rec[REC_DLN + DD + f] = sb;
    }
    return;
  } else if constexpr (ROLE == kBack) {
    // the reverse walk over the records: per tile three barrier intervals,
    // [dk of the tile after it, S5, the loads of the tile before it], [S6],
    // [S7] -- dk reads only the tile's t[0], which neither S5 (t[1], t[2]
    // of the current tile) nor the loads (inputs and record of the tile
    // before, in the same buffer) touch
    struct Tail {
      int t0;
      float er[RO], ga[RO], dt[RO];
    };
    auto tail_of = [&](const TileRegs& S) {
      Tail t;
      t.t0 = S.t0;
#pragma unroll
      for (int j = 0; j < RO; ++j) {
        t.er[j] = S.er[j];
        t.ga[j] = S.ga[j];
        t.dt[j] = S.dt[j];
      }
      return t;
    };
    auto S8t = [&](auto& X, const Tail& t) {
#pragma unroll
      for (int j = 0; j < RO; ++j) {
        const int i = RO * w + j;
        const float dk = X.t[0][i][f] - t.er[j] * t.ga[j] - (RES ? t.dt[j] : 0.f);
        store_row<BF16>(o_dk, t.t0 + i, f, dk);
      }
    };
    TileRegs Sb, Sf;
    Tail tl;
    fetch2(tiles - 1, F);
    S0(tiles - 1, L.b[(tiles - 1) & 1], Sb);
    lds_barrier();
    if (tiles > 1) {
      {
        auto& Xb = L.b[(tiles - 1) & 1];
        S5(Xb, Sb);
        S0(tiles - 2, L.b[tiles & 1], Sf);
        lds_barrier();
        S6(Xb, Sb);
        lds_barrier();
        S7(Xb, Sb);
        lds_barrier();
        tl = tail_of(Sb);
        Sb = Sf;
      }
      for (int ct = tiles - 2; ct >= 1; --ct) {
        auto& Xb = L.b[ct & 1];
        S8t(L.b[(ct + 1) & 1], tl);
        S5(Xb, Sb);
        S0(ct - 1, L.b[(ct - 1) & 1], Sf);
        lds_barrier();
        S6(Xb, Sb);
        lds_barrier();
        S7(Xb, Sb);
        lds_barrier();
        tl = tail_of(Sb);
        Sb = Sf;
      }
      S8t(L.b[1], tl);   // tile 1
    }
    auto& X = L.b[0];
    S5(X, Sb);
    lds_barrier();
    S6(X, Sb);
    lds_barrier();
    S7(X, Sb);
    lds_barrier();
    S8(X, Sb);
  } else {
    TileRegs Sb, Sf;
    fetch2(tiles - 1, F);
    {
      // prologue: the front half of the last mini-batch
      TileBuf& X = L.b[(tiles - 1) & 1];
      S0(tiles - 1, X, Sb);
      lds_barrier();
      S1(X, Sb);
      lds_barrier();
      S2(X, Sb);
      lds_barrier();
      S3(X, Sb);
      lds_barrier();
      S4(X, Sb);
      lds_barrier();
    }
    for (int ct = tiles - 1; ct >= 1; --ct) {
      TileBuf& Xb = L.b[ct & 1];         // the back half of mini-batch ct
      TileBuf& Xf = L.b[(ct - 1) & 1];   // the front half of mini-batch ct - 1
      S5(Xb, Sb);
      S0(ct - 1, Xf, Sf);
      lds_barrier();  // I1
      S6(Xb, Sb);
      S1(Xf, Sf);
      lds_barrier();  // I2
      S7(Xb, Sb);
      S2(Xf, Sf);
      lds_barrier();  // I3
      S8(Xb, Sb);
      S3(Xf, Sf);
      lds_barrier();  // I4
      S4(Xf, Sf);
      lds_barrier();  // I5
      Sb = Sf;
    }
    {
      // epilogue: the back half of the first mini-batch
      TileBuf& X = L.b[0];
      S5(X, Sb);
      lds_barrier();
      S6(X, Sb);
      lds_barrier();
      S7(X, Sb);
      lds_barrier();
      S8(X, Sb);
    }
  }

  // ---- dW0 of this unit and its LN-parameter partial sums --------------------
  if (primal) {
    float* dst = (a.state0_per_batch ? a.dw0 : a.ws_dw0) + static_cast<size_t>(unit) * DD * DD;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(16 * rt + 4 * g + i) * DD + col] = Am[rt][i];
  }
  L.dln[0][w][f] = dgam;
  L.dln[1][w][f] = dbet;
  lds_barrier();
  if (w == 0) {
    float sg = 0.f, sb = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      sg += L.dln[0][v][f];
      sb += L.dln[1][v][f];
    }
    float* p = a.ws_dln + static_cast<size_t>(unit) * 2 * DD;
    p[f] = sg;
    p[DD + f] = sb;
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

template <bool BF16, bool LN, bool MB16, int ROLE>
hipError_t launch_role(const BackwardArgs& a, bool res, dim3 grid, hipStream_t s) {
  const dim3 block(NW * 64);
  if (res)
    hipLaunchKernelGGL((ttt_linear_bwd_k<BF16, LN, true, MB16, ROLE>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((ttt_linear_bwd_k<BF16, LN, false, MB16, ROLE>), grid, block, 0, s, a);
  return hipGetLastError();
}

// 16-token mini-batches: the front half of every tile and the reverse walk
// (the host API has the forward kernel store the bases first; kReplay runs
// only for a caller of this launcher that did neither); longer mini-batches:
// the whole pass.
template <bool BF16, bool LN>
hipError_t launch_b2(const BackwardArgs& a, bool res, hipStream_t s) {
  const int units = a.B * a.H;
  if (a.tiles_per_mb != 1) return launch_role<BF16, LN, false, kWhole>(a, res, dim3(units), s);
  const int tiles = (a.T + TB - 1) / TB;
  hipError_t e = hipSuccess;
  if (!a.bases_saved) e = launch_role<BF16, LN, true, kReplay>(a, res, dim3(units), s);
  if (e == hipSuccess) e = launch_role<BF16, LN, true, kFront>(a, res, dim3(units * tiles), s);
  if (e == hipSuccess) e = launch_role<BF16, LN, true, kBack>(a, res, dim3(units), s);
  return e;
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
