// ttt_mlp_decode.hip -- one token of the TTT-MLP scan per (batch, head)
// unit: the streaming (decode) step, for gfx950.
//
// The inner model is f(x) = x + LN(GELU(x W1 + b1) W2 + b2) with d = 64
// features and m = 256 hidden units (codewithpapers.app record of arXiv
// 2407.04620, TTT-MLP; GELU in its exact erf form).  As for TTT-Linear
// (dmarx.github.io record LIT-801, "Key takeaways" items 1, 2 and 5) every
// gradient of a mini-batch is taken at the state the mini-batch started
// from, the base, and a stream carries the state S = (W1, b1, W2, b2), the
// base and the token's position j in its mini-batch.  One step:
//     base = (j == 0) ? S : S_base
//     p = k W1b + b1b,  a = GELU(p),  o = a W2b + b2b       (at the base)
//     g_o = LN_backward(2 (k + LN(o) - v)),  g_p = (g_o W2b^T) * GELU'(p)
//     u_o = -eta g_o,  u_p = -eta g_p
//     W1 += k^T u_p,  b1 += u_p,  W2 += a^T u_o,  b2 += u_o
//     z  = q + LN(GELU(q W1 + b1) W2 + b2)                  (new state)
//     S_base <- base                                         (j == 0 only)
// The output's first product is taken from the old W1, corrected with the
// rank-1 change: q W1_new + b1_new = q W1 + b1 + (q . k + 1) u_p, so both
// products with W1 leave in one reduction.
//
// The step moves the state: 132 KB read, 132 KB written and 132 KB of base
// read (j > 0) or written (j == 0) per unit -- it is bound by memory.  One
// 1024-thread workgroup per unit, the state in registers:
//   W1 (64 x 256): wave w, lane l holds column n = 64 (w % 4) + l, rows
//                  16 (w / 4) .. +16 (the thread's feature quarter);
//   W2 (256 x 64): wave w holds rows 16 w .. +16, lane l column l.
// Every load and store of a wave covers one contiguous 256-byte row; the
// state goes through buffer resources, the row offset (wave-uniform) in the
// scalar offset, so no per-access address arithmetic is needed.  Products
// over features reduce the four quarters through LDS; products over hidden
// units reduce the sixteen waves through LDS; g_o W2^T (over the features
// of a W2 row) is a reduce-scatter across a wave's lanes.  fp32 arithmetic
// throughout.
#include "ttt_device.hpp"
#include "ttt_stream.hpp"

namespace tttk {
namespace {

constexpr int DD = 64;         // features d
constexpr int HM = 256;        // hidden units m
constexpr int NWV = 16;        // waves per unit
constexpr int FR = DD / 4;     // W1 rows per thread (one feature quarter)
constexpr int HR = HM / NWV;   // W2 rows per wave

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

// x from another lane of the same 16-lane row (DPP control CTRL).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return bitsf(static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(fbits(x)), CTRL, 0xf, 0xf, false)));
}

// N sums over the 64 lanes of the wave at once, in every lane: butterflies
// within each 16-lane row on DPP, then across the four rows.
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

__device__ __forceinline__ float wave_sum(float x) {
  float s[1] = {x};
  wave_sums(s);
  return s[0];
}

// LN over the 64 features held one per lane: x_hat and 1 / sigma.
__device__ __forceinline__ void ln_stats(float h, float eps, float& xh, float& rs) {
  const float mu = wave_sum(h) * (1.0f / DD);
  const float xc = h - mu;
  const float var = wave_sum(xc * xc) * (1.0f / DD);
  rs = 1.0f / __builtin_sqrtf(var + eps);
  xh = xc * rs;
}

// Buffer resource over `bytes` bytes from `base`; accesses past the end read
// zero and write nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(float* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ float ld(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return bitsf(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ void st(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                   float x) {
  __builtin_amdgcn_raw_buffer_store_b32(fbits(x), r, voff, soff, 0);
}

// Reduce-scatter of 16 per-lane values over the 64 lanes of the wave: the
// returned value of lane l is the wave's total of x[l / 4].  Halves of the
// wave (permlane32 swaps), then its 16-lane rows (permlane16 swaps) take
// 8 + 4 sums; within a row lanes l and l ^ 8 (rotation by 8), then the
// mirrored lanes of each half row (they differ in bit 2), then the lanes of
// a quad finish the sum.
__device__ __forceinline__ float wave_reduce_scatter16(const float (&x)[16], int l) {
  float y[8], z[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = swap32_sum(x[i], x[i + 8]);   // lanes < 32: i, else i + 8
#pragma unroll
  for (int i = 0; i < 4; ++i) z[i] = swap16_sum(y[i], y[i + 4]);   // row rho: i + 4 rho
  const bool b3 = (l >> 3) & 1, b2 = (l >> 2) & 1;
  const float k0 = b3 ? z[2] : z[0], s0 = b3 ? z[0] : z[2];
  const float k1 = b3 ? z[3] : z[1], s1 = b3 ? z[1] : z[3];
  const float u0 = k0 + dpp<0x128>(s0);                            // row_ror:8
  const float u1 = k1 + dpp<0x128>(s1);
  const float kk = b2 ? u1 : u0, ss = b2 ? u0 : u1;
  float v = kk + dpp<0x141>(ss);                                   // row_half_mirror
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  return v;
}

// x of lane `src` (wave-uniform) in every lane.
__device__ __forceinline__ float lane_of(float x, int src) {
  return bitsf(static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(fbits(x)), src)));
}

// Phi(x), the standard normal distribution function, from erf.
__device__ __forceinline__ float norm_cdf(float x) {
  return 0.5f * (1.0f + erff(x * 0.70710678118654752f));
}

// GELU(x) = x Phi(x) and GELU'(x) = Phi(x) + x phi(x).
__device__ __forceinline__ void gelu2(float x, float& y, float& dy) {
  const float c = norm_cdf(x);
  y = x * c;
  dy = __builtin_fmaf(x * 0.39894228040143268f, __expf(-0.5f * x * x), c);
}

template <bool BF16, bool LN, bool RES>
__global__ __launch_bounds__(NWV * 64) __attribute__((amdgpu_waves_per_eu(8)))
void ttt_mlp_decode_k(MlpDecodeArgs a) {
  __shared__ float sp[2][4][HM];   // per-quarter partials of k W1b and q W1
  __shared__ float sak[HM];        // a = GELU(p) at the base
  __shared__ float saq[HM];        // GELU of the output's hidden layer
  __shared__ float sgw[HM];        // g_o W2b^T
  __shared__ float so[NWV][DD];    // per-wave partials of a W2
  const int unit = blockIdx.x;
  const int head = unit % a.H;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  const int fq = w >> 2;             // W1 rows FR fq .. +FR
  const int n = 64 * (w & 3) + l;    // W1 column, the thread's hidden unit
  const int nr = HR * w;             // W2 rows nr .. +HR
  const size_t row = (size_t)unit * DD;
  const size_t o1 = (size_t)unit * DD * HM;
  // this thread's rows: W1 rows FR fq .. +FR, W2 rows nr .. +HR; element
  // (row r of them, column n of W1 or l of W2) at a constant offset
  const size_t q1 = o1 + (size_t)FR * fq * HM, q2 = o1 + (size_t)nr * DD;
  constexpr uint32_t MB1 = FR * HM * 4, MB2 = HR * DD * 4;
  const auto W1 = rsrc(a.w1 + q1, MB1), W2 = rsrc(a.w2 + q2, MB2);
  const auto W1b = rsrc(a.w1_base + q1, MB1), W2b = rsrc(a.w2_base + q2, MB2);
  const uint32_t v1 = n * 4, v2 = l * 4;
  auto s1 = [](int r) { return static_cast<uint32_t>(r * HM * 4); };
  auto s2 = [](int r) { return static_cast<uint32_t>(r * DD * 4); };
  float* b1 = a.b1 + (size_t)unit * HM;
  float* b1b = a.b1_base + (size_t)unit * HM;
  float* b2 = a.b2 + row;
  float* b2b = a.b2_base + row;
  const bool fresh = a.pos == 0;
  // the gradient's base: the state itself when a mini-batch starts
  const auto R1 = fresh ? W1 : W1b, R2 = fresh ? W2 : W2b;
  const float* b1s = fresh ? b1 : b1b;
  const float* b2s = fresh ? b2 : b2b;

  // the base and the token first; the state's rows are loaded as the base's
  // registers free up, so that two units fit a compute unit's registers
  float w1b[FR], w2b[HR];
#pragma unroll
  for (int r = 0; r < FR; ++r) w1b[r] = ld(R1, v1, s1(r));
#pragma unroll
  for (int r = 0; r < HR; ++r) w2b[r] = ld(R2, v2, s2(r));
  const float b1bn = b1s[n];
  const float b2bf = b2s[l];
  const float kf = ld_io<BF16>(a.k, row + l);
  const float vf = ld_io<BF16>(a.v, row + l);
  const float qf = ld_io<BF16>(a.q, row + l);
  const float eta = a.eta[unit];
  float gam = 1.f, bet = 0.f;
  if (LN) {
    gam = a.gamma[(size_t)head * DD + l];
    bet = a.beta[(size_t)head * DD + l];
  }
  if (fresh) {   // the state becomes the new mini-batch's base
#pragma unroll
    for (int r = 0; r < FR; ++r) st(W1b, v1, s1(r), w1b[r]);
#pragma unroll
    for (int r = 0; r < HR; ++r) st(W2b, v2, s2(r), w2b[r]);
    if (fq == 0) b1b[n] = b1bn;
    if (w == 0) b2b[l] = b2bf;
  }

  // k W1b over this thread's feature quarter (k of those features from the
  // lanes that hold them)
  float pk = 0.f;
#pragma unroll
  for (int r = 0; r < FR; ++r) pk = __builtin_fmaf(lane_of(kf, FR * fq + r), w1b[r], pk);
  sp[0][fq][n] = pk;
  // the state's W1 rows (at a mini-batch's start the rows just read, again:
  // a second read from the cache costs less than holding both copies)
  float w1r[FR];
#pragma unroll
  for (int r = 0; r < FR; ++r) w1r[r] = ld(W1, v1, s1(r));
  __syncthreads();
  const float p = ((sp[0][0][n] + sp[0][1][n]) + (sp[0][2][n] + sp[0][3][n])) + b1bn;
  float an, dn;
  gelu2(p, an, dn);
  if (fq == 0) sak[n] = an;
  __syncthreads();

  // o = a W2b + b2b: this wave's rows, then the sixteen waves
  float ok = 0.f;
#pragma unroll
  for (int r = 0; r < HR; ++r) ok = __builtin_fmaf(sak[nr + r], w2b[r], ok);
  so[w][l] = ok;
  __syncthreads();
  float o = b2bf;
#pragma unroll
  for (int v = 0; v < NWV; ++v) o += so[v][l];

  // gradient with respect to o (every wave, the same), and q . k
  float go, qk;
  if (LN) {
    float xh, rs;
    ln_stats(o, a.eps, xh, rs);
    const float gy = 2.f * ((RES ? kf : 0.f) + __builtin_fmaf(gam, xh, bet) - vf);
    const float gg = gam * gy;
    float m[3] = {gg, gg * xh, qf * kf};
    wave_sums(m);
    go = (gg - m[0] * (1.0f / DD) - xh * (m[1] * (1.0f / DD))) * rs;
    qk = m[2];
  } else {
    go = 2.f * ((RES ? kf : 0.f) + o - vf);
    qk = wave_sum(qf * kf);
  }
  const float uo = -eta * go;

  // g_o W2b^T on this wave's rows (sums over the lanes)
  static_assert(HR == 16, "one reduce-scatter per wave's W2 rows");
  float gw[HR];
#pragma unroll
  for (int r = 0; r < HR; ++r) gw[r] = go * w2b[r];
  const float gws = wave_reduce_scatter16(gw, l);
  if ((l & 3) == 0) sgw[nr + (l >> 2)] = gws;
  float w2r[HR];   // the state's W2 rows
#pragma unroll
  for (int r = 0; r < HR; ++r) w2r[r] = ld(W2, v2, s2(r));
  // q W1 over the quarter, from the state before the update
  float pq = 0.f;
#pragma unroll
  for (int r = 0; r < FR; ++r) pq = __builtin_fmaf(lane_of(qf, FR * fq + r), w1r[r], pq);
  sp[1][fq][n] = pq;
  const float b1n = b1[n];   // the state's biases
  const float b2f = b2[l];
  __syncthreads();

  // u_p = -eta (g_o W2b^T) * GELU'(p); W1 += k^T u_p, b1 += u_p
  const float up = -eta * (sgw[n] * dn);
#pragma unroll
  for (int r = 0; r < FR; ++r)
    st(W1, v1, s1(r), __builtin_fmaf(lane_of(kf, FR * fq + r), up, w1r[r]));
  const float b1new = b1n + up;
  if (fq == 0) b1[n] = b1new;
  // the output's hidden layer from the old W1 and the rank-1 change
  const float pqn = ((sp[1][0][n] + sp[1][1][n]) + (sp[1][2][n] + sp[1][3][n])) +
                    __builtin_fmaf(qk, up, b1new);
  float aq, daq;
  gelu2(pqn, aq, daq);
  (void)daq;
  if (fq == 0) saq[n] = aq;
  // W2 += a^T u_o and b2 += u_o
#pragma unroll
  for (int r = 0; r < HR; ++r) {
    w2r[r] = __builtin_fmaf(sak[nr + r], uo, w2r[r]);
    st(W2, v2, s2(r), w2r[r]);
  }
  const float b2n = b2f + uo;
  if (w == 0) b2[l] = b2n;
  __syncthreads();

  float oq = 0.f;
#pragma unroll
  for (int r = 0; r < HR; ++r) oq = __builtin_fmaf(saq[nr + r], w2r[r], oq);
  so[w][l] = oq;
  __syncthreads();
  if (w == 0) {
    float y = b2n;
#pragma unroll
    for (int v = 0; v < NWV; ++v) y += so[v][l];
    if (LN) {
      float xh, rs;
      ln_stats(y, a.eps, xh, rs);
      y = __builtin_fmaf(gam, xh, bet);
    }
    st_io<BF16>(a.z, row + l, (RES ? qf : 0.f) + y);
  }
}

template <bool BF16, bool LN>
hipError_t launch_m2(const MlpDecodeArgs& a, bool res, hipStream_t s) {
  const dim3 grid(a.B * a.H), block(NWV * 64);
  if (res)
    hipLaunchKernelGGL((ttt_mlp_decode_k<BF16, LN, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((ttt_mlp_decode_k<BF16, LN, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_m1(const MlpDecodeArgs& a, bool ln, bool res, hipStream_t s) {
  return ln ? launch_m2<BF16, true>(a, res, s) : launch_m2<BF16, false>(a, res, s);
}

}  // namespace

hipError_t launch_mlp_decode(const MlpDecodeArgs& a, bool bf16, bool ln, bool residual,
                             hipStream_t stream) {
  return bf16 ? launch_m1<true>(a, ln, residual, stream) : launch_m1<false>(a, ln, residual, stream);
}

}  // namespace tttk
