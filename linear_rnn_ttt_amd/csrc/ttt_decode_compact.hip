// ttt_decode_compact.hip -- one token of the TTT-Linear scan per (batch,
// head) unit with a compact pending state, for gfx950.
//
// Within a mini-batch every gradient is taken at the base (dmarx.github.io
// record LIT-801, "Key takeaways" items 1, 2 and 5), so after the tokens
// s < j of the current mini-batch the state is
//     W = W_base + sum_{s<j} k_s^T u_s,     u_s = -eta_s g_s,
// a rank-j change of the base.  A stream can therefore carry the base and
// the mini-batch's rows (k_s, u_s) -- 16 x 512 B for b = 16 -- instead of W
// and W_base (2 x 16 KB).  One step at position j:
//     j == 0: W_base <- W_base + sum_{s<b} k_s^T u_s   (the previous
//             mini-batch's rows; zero at the start of a stream)
//     g   = LN_backward(2 (k + LN(k W_base) - v)),   u = -eta g
//     o   = q W_base + sum_{s<j} (q . k_s) u_s + (q . k) u   (= q W_j)
//     z   = q + LN(o);   slot j <- (k, u)
// Moved per unit and token: W_base read (16 KB), j history slots read and
// one written (512 B each), and at j == 0 the base written and the b slots
// read once -- about 22 KB per token for b = 16 against 48 KB for the
// (W, W_base) form.  Arithmetic fp32 (matrix-vector products).
//
// Layout as in ttt_decode.hip: one 256-thread workgroup per unit, lane f
// holds column f, wave w rows 16w..16w+15 of the base; row-sums reduced
// across the waves through LDS, LN sums across a wave's 64 lanes.
#include "ttt_device.hpp"
#include "ttt_stream.hpp"

namespace tttk {
namespace {

constexpr int DD = 64;
constexpr int DW = 4;
constexpr int RW = DD / DW;
constexpr int MB_MAX = 64;   // history slots of the largest instance
using LdsPtr = __attribute__((address_space(3))) void*;

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

// MBM: history slots the instance holds in LDS (16 or 64): the 16-slot
// instance needs 10 KB, so more workgroups fit on a CU to hide memory latency.
template <bool BF16, bool LN, bool RES, int MBM>
__global__ __launch_bounds__(DW * 64) void ttt_linear_decode_compact_k(CompactArgs a) {
  __shared__ float hk[MBM][DD];      // history rows k_s
  __shared__ float hu[MBM][DD];      // history rows u_s
  __shared__ float red[2][DW][DD];   // per-wave partial sums of k.W_base and q.W_base
  __shared__ float coef[MBM];        // q . k_s
  const int unit = blockIdx.x;
  const int head = unit % a.H;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int f = tid & 63;
  const size_t row = (size_t)unit * DD;
  float* Wb = a.w_base + (size_t)unit * DD * DD;
  float* hist = a.hist + (size_t)unit * a.mb * 2 * DD;
  const int j = a.pos;
  // history rows needed: all b at a mini-batch start (the fold), else s < j
  const int nh = j == 0 ? a.mb : j;

  float wr[RW], kr[RW], qr[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    wr[r] = Wb[(w * RW + r) * DD + f];
    kr[r] = ld_io<BF16>(a.k, row + w * RW + r);
    qr[r] = ld_io<BF16>(a.q, row + w * RW + r);
  }
  // the history rows straight from memory into LDS (global_load_lds: lane f
  // of the wave lands at word f of the row; all rows in flight at once)
  for (int s = w; s < nh; s += DW) {
    __builtin_amdgcn_global_load_lds(hist + s * 2 * DD + f, (LdsPtr)&hk[s][0], 4, 0, 0);
    __builtin_amdgcn_global_load_lds(hist + s * 2 * DD + DD + f, (LdsPtr)&hu[s][0], 4, 0, 0);
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
  __syncthreads();

  if (j == 0) {
    // the previous mini-batch folds into the base: W_base += sum_s k_s^T u_s
    for (int s = 0; s < a.mb; ++s) {
      const float us = hu[s][f];
#pragma unroll
      for (int r = 0; r < RW; ++r) wr[r] = __builtin_fmaf(hk[s][w * RW + r], us, wr[r]);
    }
#pragma unroll
    for (int r = 0; r < RW; ++r) Wb[(w * RW + r) * DD + f] = wr[r];
  }

  // k.W_base and q.W_base (column f), this wave's rows
  float hk_ = 0.f, hq = 0.f;
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    hk_ = __builtin_fmaf(kr[r], wr[r], hk_);
    hq = __builtin_fmaf(qr[r], wr[r], hq);
  }
  red[0][w][f] = hk_;
  red[1][w][f] = hq;
  // q . k_s for the history rows the output needs (s < j): wave w takes
  // s = w + 4i, all of them in one batch of butterflies
  if (j > w) {
    constexpr int NS = MBM / DW;
    float d[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int s = w + DW * i;
      d[i] = s < j ? qf * hk[s][f] : 0.f;
    }
    wave_sums(d);
    if (f == 0) {
#pragma unroll
      for (int i = 0; i < NS; ++i)
        if (w + DW * i < j) coef[w + DW * i] = d[i];
    }
  }
  __syncthreads();
  const float h = (red[0][0][f] + red[0][1][f]) + (red[0][2][f] + red[0][3][f]);

  // gradient of the token's loss at the base, u = -eta g (every wave, the same)
  float g, qk;
  if (LN) {
    float xh, rs;
    ln_stats(h, a.eps, xh, rs);
    const float gy = 2.f * ((RES ? kf : 0.f) + __builtin_fmaf(gam, xh, bet) - vf);
    const float gg = gam * gy;
    float m[3] = {gg, gg * xh, qf * kf};
    wave_sums(m);
    g = (gg - m[0] * (1.0f / DD) - xh * (m[1] * (1.0f / DD))) * rs;
    qk = m[2];
  } else {
    g = 2.f * ((RES ? kf : 0.f) + h - vf);
    qk = wave_sum(qf * kf);
  }
  const float u = -eta * g;

  if (w == 0) {
    // o = q W_base + sum_{s<j} (q . k_s) u_s + (q . k) u
    float o = (red[1][0][f] + red[1][1][f]) + (red[1][2][f] + red[1][3][f]);
    for (int s = 0; s < j; ++s) o = __builtin_fmaf(coef[s], hu[s][f], o);
    o = __builtin_fmaf(qk, u, o);
    float y = o;
    if (LN) {
      float xh, rs;
      ln_stats(o, a.eps, xh, rs);
      y = __builtin_fmaf(gam, xh, bet);
    }
    st_io<BF16>(a.z, row + f, (RES ? qf : 0.f) + y);
    // this token's history slot
    hist[j * 2 * DD + f] = kf;
    hist[j * 2 * DD + DD + f] = u;
  }
}

template <bool BF16, bool LN, int MBM>
hipError_t launch_c3(const CompactArgs& a, bool res, hipStream_t s) {
  const dim3 grid(a.B * a.H), block(DW * 64);
  if (res)
    hipLaunchKernelGGL((ttt_linear_decode_compact_k<BF16, LN, true, MBM>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((ttt_linear_decode_compact_k<BF16, LN, false, MBM>), grid, block, 0, s,
                       a);
  return hipGetLastError();
}

template <bool BF16, bool LN>
hipError_t launch_c2(const CompactArgs& a, bool res, hipStream_t s) {
  return a.mb <= 16 ? launch_c3<BF16, LN, 16>(a, res, s) : launch_c3<BF16, LN, MB_MAX>(a, res, s);
}

template <bool BF16>
hipError_t launch_c1(const CompactArgs& a, bool ln, bool res, hipStream_t s) {
  return ln ? launch_c2<BF16, true>(a, res, s) : launch_c2<BF16, false>(a, res, s);
}

}  // namespace

hipError_t launch_linear_decode_compact(const CompactArgs& a, bool bf16, bool ln, bool residual,
                                        hipStream_t stream) {
  return bf16 ? launch_c1<true>(a, ln, residual, stream)
              : launch_c1<false>(a, ln, residual, stream);
}

}  // namespace tttk
