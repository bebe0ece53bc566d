// ttt_decode.hip -- one token of the TTT-Linear scan per (batch, head) unit:
// the streaming (decode) step, for gfx950.
//
// Method as in ttt_linear.hip (dmarx.github.io record LIT-801 on arXiv
// 2407.04620, "Key takeaways" items 1, 2 and 5): within a mini-batch of b
// tokens every gradient is taken at the state the mini-batch started from
// (the base), and the state absorbs the tokens one by one; z_t uses the
// state after token t.  A stream therefore carries three things between
// tokens: the state W, the base W_base and the position j of the next token
// in its mini-batch.  One step, for token t at position j:
//     base = (j == 0) ? W : W_base            (a new mini-batch starts at W)
//     g    = LN_backward(2 (k + LN(k base) - v))       (row gradient at base)
//     W   <- W - eta k^T g
//     z    = q + LN(q W)
//     W_base <- base                           (written only when j == 0)
// Running the step over a sequence with j = t mod b from W0 reproduces the
// forward scan.
//
// The step moves the state (16 KB of W read and written, 16 KB of W_base
// read or written per unit) and does 3 d^2 multiply-adds per unit: it is
// bound by memory.  One 256-thread workgroup per unit: lane f owns feature
// column f, wave w rows 16w..16w+15 of W and of the base, all loaded at once
// (coalesced 256-byte rows); the two row-sums of products (k base, q W)
// are reduced across the four waves through LDS, the LN sums across the
// 64 lanes of a wave.  Arithmetic is fp32 throughout (no matrix unit: the
// products are matrix-vector).
#include "ttt_device.hpp"
#include "ttt_kernels.hpp"

namespace tttk {
namespace {

constexpr int DD = 64;        // head dimension
constexpr int DW = 4;         // waves per unit
constexpr int RW = DD / DW;   // rows of W per wave

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
// within each 16-lane row on DPP (lanes l^1, l^2, then the mirrored lane of
// the half row and of the row), then across the four rows with permlane
// swaps -- all VALU, no LDS round trip.
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

template <bool BF16, bool LN, bool RES>
__global__ __launch_bounds__(DW * 64) void ttt_linear_decode_k(DecodeArgs a) {
  __shared__ float red[2][DW][DD];  // per-wave partial sums of k.base and q.W
  const int unit = blockIdx.x;
  const int head = unit % a.H;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int f = threadIdx.x & 63;
  const size_t row = (size_t)unit * DD;  // this unit's token row in [B,H,d]
  const size_t st = (size_t)unit * DD * DD;
  float* W = a.w + st;
  float* Wb = a.w_base + st;
  const bool fresh = a.pos == 0;

  // every load first: this wave's rows of W (and of the base), the token
  float wr[RW], br[RW], kr[RW], qr[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) wr[r] = W[(w * RW + r) * DD + f];
  if (!fresh) {
#pragma unroll
    for (int r = 0; r < RW; ++r) br[r] = Wb[(w * RW + r) * DD + f];
  }
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    kr[r] = ld_io<BF16>(a.k, row + w * RW + r);
    qr[r] = ld_io<BF16>(a.q, row + w * RW + r);
  }
  const float kf = ld_io<BF16>(a.k, row + f);
  const float vf = ld_io<BF16>(a.v, row + f);
  const float qf = ld_io<BF16>(a.q, row + f);
  const float eta = a.eta[unit];
  float gam = 1.f, bet = 0.f;
  if (LN) {
    gam = a.gamma[(size_t)head * DD + f];
    bet = a.beta[(size_t)head * DD + f];
  }
  if (fresh) {
#pragma unroll
    for (int r = 0; r < RW; ++r) br[r] = wr[r];
  }

  // h = k base (column f), reduced over the four waves' rows
  float hk = 0.f;
#pragma unroll
  for (int r = 0; r < RW; ++r) hk = __builtin_fmaf(kr[r], br[r], hk);
  red[0][w][f] = hk;
  __syncthreads();
  hk = (red[0][0][f] + red[0][1][f]) + (red[0][2][f] + red[0][3][f]);

  // gradient of the token's loss with respect to h (every wave, the same)
  float g;
  if (LN) {
    float xh, rs;
    ln_stats(hk, a.eps, xh, rs);
    const float gy = 2.f * ((RES ? kf : 0.f) + __builtin_fmaf(gam, xh, bet) - vf);
    const float gg = gam * gy;
    float m[2] = {gg, gg * xh};
    wave_sums(m);
    g = (gg - m[0] * (1.0f / DD) - xh * (m[1] * (1.0f / DD))) * rs;
  } else {
    g = 2.f * ((RES ? kf : 0.f) + hk - vf);
  }

  // W <- W - eta k^T g on this wave's rows, and q W from the new rows
  const float eg = -eta * g;
  float hq = 0.f;
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const float wn = __builtin_fmaf(kr[r], eg, wr[r]);
    W[(w * RW + r) * DD + f] = wn;
    if (fresh) Wb[(w * RW + r) * DD + f] = wr[r];
    hq = __builtin_fmaf(qr[r], wn, hq);
  }
  red[1][w][f] = hq;
  __syncthreads();
  if (w == 0) {
    hq = (red[1][0][f] + red[1][1][f]) + (red[1][2][f] + red[1][3][f]);
    float y = hq;
    if (LN) {
      float xh, rs;
      ln_stats(hq, a.eps, xh, rs);
      y = __builtin_fmaf(gam, xh, bet);
    }
    st_io<BF16>(a.z, row + f, (RES ? qf : 0.f) + y);
  }
}

template <bool BF16, bool LN>
hipError_t launch_d2(const DecodeArgs& a, bool res, hipStream_t s) {
  const dim3 grid(a.B * a.H), block(DW * 64);
  if (res)
    hipLaunchKernelGGL((ttt_linear_decode_k<BF16, LN, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((ttt_linear_decode_k<BF16, LN, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_d1(const DecodeArgs& a, bool ln, bool res, hipStream_t s) {
  return ln ? launch_d2<BF16, true>(a, res, s) : launch_d2<BF16, false>(a, res, s);
}

}  // namespace

hipError_t launch_linear_decode(const DecodeArgs& a, bool bf16, bool ln, bool residual,
                                hipStream_t stream) {
  return bf16 ? launch_d1<true>(a, ln, residual, stream)
              : launch_d1<false>(a, ln, residual, stream);
}

}  // namespace tttk
