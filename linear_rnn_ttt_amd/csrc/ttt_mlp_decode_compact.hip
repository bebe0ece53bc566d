// ttt_mlp_decode_compact.hip -- one token of the TTT-MLP scan per (batch,
// head) unit with a compact pending state, for gfx950.
//
// Within a mini-batch every gradient is taken at the base (dmarx.github.io
// record LIT-801, "Key takeaways" items 1, 2 and 5; the inner model
// f(x) = x + LN(GELU(x W1 + b1) W2 + b2) of the codewithpapers.app record of
// arXiv 2407.04620, TTT-MLP), so after the tokens s < j of the current
// mini-batch the state is the base plus rank-1 terms:
//     W1 = W1b + sum_s k_s^T u1_s,   b1 = b1b + sum_s u1_s,
//     W2 = W2b + sum_s a_s^T u2_s,   b2 = b2b + sum_s u2_s,
// with u1 = -eta g_p, u2 = -eta g_o and a = GELU(k W1b + b1b), all taken at
// the base.  A stream can carry the base and the mini-batch's rows
// (k, u1, a, u2) -- 2.5 KB per token -- instead of the state and the base
// (2 x 132 KB).  One step at position j:
//     j == 0: the previous mini-batch's rows fold into the base (zero rows
//             at the start of a stream), which is written back
//     the gradient at the base, as in ttt_mlp_decode.hip -> u1, u2, a
//     p_q = q W1b + b1b + sum_{s<=j} (q . k_s + 1) u1_s
//     o_q = GELU(p_q) W2b + b2b + sum_{s<=j} (GELU(p_q) . a_s + 1) u2_s
//     z   = q + LN(o_q);   slot j <- (k, u1, a, u2)
// Moved per unit and token: the base read (132 KB), the j earlier slots
// read and slot j written (2.5 KB each), and at j == 0 the b slots read and
// the base written once -- about 165 KB per token for b = 16 against 397 KB
// for the (S, S_base) form.
//
// Layout as in ttt_mlp_decode.hip (1024 threads per unit, the base in
// registers, 64 VGPRs so that two units share a compute unit); the slots
// live in LDS (40 KB for b <= 16).  fp32 arithmetic.
#include "ttt_device.hpp"
#include "ttt_mlp_compact.hpp"

namespace tttk {
namespace {

constexpr int DD = 64;         // features d
constexpr int HM = 256;        // hidden units m
constexpr int NWV = 16;        // waves per unit
constexpr int FR = DD / 4;     // W1 rows per thread (one feature quarter)
constexpr int HR = HM / NWV;   // W2 rows per wave
constexpr int MBM = 16;        // history slots held in LDS (mini-batch <= 16)
constexpr int SLOT = 2 * DD + 2 * HM;                              // floats per slot
constexpr int OK = 0, OU1 = DD, OA = DD + HM, OU2 = DD + 2 * HM;   // k, u1, a, u2
static_assert(MBM == NWV, "wave w takes the dot product with slot w");
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

// N sums over the 64 lanes of the wave at once, in every lane.
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

// Reduce-scatter of 16 per-lane values over the wave: lane l returns the
// wave's total of x[l / 4] (as in ttt_mlp_decode.hip).
__device__ __forceinline__ float wave_reduce_scatter16(const float (&x)[16], int l) {
  float y[8], z[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = swap32_sum(x[i], x[i + 8]);
#pragma unroll
  for (int i = 0; i < 4; ++i) z[i] = swap16_sum(y[i], y[i + 4]);
  const bool b3 = (l >> 3) & 1, b2 = (l >> 2) & 1;
  const float k0 = b3 ? z[2] : z[0], s0 = b3 ? z[0] : z[2];
  const float k1 = b3 ? z[3] : z[1], s1 = b3 ? z[1] : z[3];
  const float u0 = k0 + dpp<0x128>(s0);   // row_ror:8
  const float u1 = k1 + dpp<0x128>(s1);
  const float kk = b2 ? u1 : u0, ss = b2 ? u0 : u1;
  float v = kk + dpp<0x141>(ss);          // row_half_mirror
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  return v;
}

// LN over the 64 features held one per lane: x_hat and 1 / sigma.
__device__ __forceinline__ void ln_stats(float h, float eps, float& xh, float& rs) {
  const float mu = wave_sum(h) * (1.0f / DD);
  const float xc = h - mu;
  const float var = wave_sum(xc * xc) * (1.0f / DD);
  rs = 1.0f / __builtin_sqrtf(var + eps);
  xh = xc * rs;
}

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

// x of lane `src` (wave-uniform) in every lane.
__device__ __forceinline__ float lane_of(float x, int src) {
  return bitsf(static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(fbits(x)), src)));
}

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
void ttt_mlp_decode_compact_k(MlpCompactArgs a) {
  __shared__ float hs[MBM][SLOT];        // the mini-batch's slots (k, u1, a, u2)
  __shared__ float sp[2][4][HM];         // per-quarter partials of k W1b and q W1b
  __shared__ float sak[HM];              // a = GELU(p) at the base
  __shared__ float saq[HM];              // GELU of the output's hidden layer
  __shared__ float sgw[HM];              // g_o W2b^T
  __shared__ float so[NWV][DD];          // per-wave partials of a_q W2b
  __shared__ float coef[MBM];            // q . k_s
  __shared__ float dpart[4][MBM + 1];    // per-wave partials of a_q . a_s, then a_q . a
  const int unit = blockIdx.x;
  const int head = unit % a.H;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int fq = w >> 2;             // W1 rows FR fq .. +FR
  const int n = 64 * (w & 3) + l;    // W1 column, the thread's hidden unit
  const int nr = HR * w;             // W2 rows nr .. +HR
  const size_t row = (size_t)unit * DD;
  const size_t o1 = (size_t)unit * DD * HM;
  const size_t q1 = o1 + (size_t)FR * fq * HM, q2 = o1 + (size_t)nr * DD;
  constexpr uint32_t MB1 = FR * HM * 4, MB2 = HR * DD * 4;
  const auto W1b = rsrc(a.w1_base + q1, MB1), W2b = rsrc(a.w2_base + q2, MB2);
  const uint32_t v1 = n * 4, v2 = l * 4;
  auto s1 = [](int r) { return static_cast<uint32_t>(r * HM * 4); };
  auto s2 = [](int r) { return static_cast<uint32_t>(r * DD * 4); };
  float* b1b = a.b1_base + (size_t)unit * HM;
  float* b2b = a.b2_base + row;
  float* hist = a.hist + (size_t)unit * a.mb * SLOT;
  const int j = a.pos;
  // slots needed: all b at a mini-batch start (the fold), else s < j
  const int nh = j == 0 ? a.mb : j;

  float w1b[FR], w2b[HR];
#pragma unroll
  for (int r = 0; r < FR; ++r) w1b[r] = ld(W1b, v1, s1(r));
#pragma unroll
  for (int r = 0; r < HR; ++r) w2b[r] = ld(W2b, v2, s2(r));
  float b1bn = b1b[n];
  float b2bf = b2b[l];
  {  // the slots, contiguous in LDS as in memory, copied straight from memory
     // into LDS (global_load_lds: lane l of a wave lands at word l of the
     // wave's 64-word chunk; no registers, and every chunk in flight at once)
    const int ne = nh * SLOT;
    for (int i = 0; i * NWV * 64 < ne; ++i) {
      const int e = i * NWV * 64 + tid;
      LdsPtr dst = (LdsPtr)(&hs[0][0] + i * NWV * 64 + w * 64);
      if (e < ne) __builtin_amdgcn_global_load_lds(hist + e, dst, 4, 0, 0);
    }
  }
  const float kf = ld_io<BF16>(a.k, row + l);
  const float vf = ld_io<BF16>(a.v, row + l);
  const float qf = ld_io<BF16>(a.q, row + l);
  const float eta = a.eta[unit];
  float gam = 1.f, bet = 0.f;
  if (LN) {
    gam = a.gamma[(size_t)head * DD + l];
    bet = a.beta[(size_t)head * DD + l];
  }
  __syncthreads();

  if (j == 0) {
    // the previous mini-batch folds into the base
    for (int s = 0; s < a.mb; ++s) {
      const float u1 = hs[s][OU1 + n];
      const float u2 = hs[s][OU2 + l];
#pragma unroll
      for (int r = 0; r < FR; ++r) w1b[r] = __builtin_fmaf(hs[s][OK + FR * fq + r], u1, w1b[r]);
#pragma unroll
      for (int r = 0; r < HR; ++r) w2b[r] = __builtin_fmaf(hs[s][OA + nr + r], u2, w2b[r]);
      b1bn += u1;
      b2bf += u2;
    }
#pragma unroll
    for (int r = 0; r < FR; ++r) st(W1b, v1, s1(r), w1b[r]);
#pragma unroll
    for (int r = 0; r < HR; ++r) st(W2b, v2, s2(r), w2b[r]);
    if (fq == 0) b1b[n] = b1bn;
    if (w == 0) b2b[l] = b2bf;
  }

  // k W1b and q W1b over this thread's feature quarter; q . k_s for the
  // slots the output needs (s < j), wave w taking slot w
  float pk = 0.f, pq = 0.f;
#pragma unroll
  for (int r = 0; r < FR; ++r) {
    pk = __builtin_fmaf(lane_of(kf, FR * fq + r), w1b[r], pk);
    pq = __builtin_fmaf(lane_of(qf, FR * fq + r), w1b[r], pq);
  }
  sp[0][fq][n] = pk;
  sp[1][fq][n] = pq;
  if (w < j) {
    const float c = wave_sum(qf * hs[w][OK + l]);
    if (l == 0) coef[w] = c;
  }
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
  __syncthreads();

  // u1 = -eta (g_o W2b^T) * GELU'(p); the output's hidden layer
  const float up = -eta * (sgw[n] * dn);
  float pqn = ((sp[1][0][n] + sp[1][1][n]) + (sp[1][2][n] + sp[1][3][n])) + b1bn;
  for (int s = 0; s < j; ++s) pqn = __builtin_fmaf(coef[s] + 1.f, hs[s][OU1 + n], pqn);
  pqn = __builtin_fmaf(qk + 1.f, up, pqn);
  float aq, daq;
  gelu2(pqn, aq, daq);
  (void)daq;
  float* slot = hist + (size_t)j * SLOT;
  if (fq == 0) {
    saq[n] = aq;
    slot[OU1 + n] = up;
    slot[OA + n] = an;
  }
  __syncthreads();

  // a_q W2b over this wave's rows; a_q . a_s (s < j) and a_q . a over the
  // hidden units, which waves 0-3 hold one per lane
  float oq = 0.f;
#pragma unroll
  for (int r = 0; r < HR; ++r) oq = __builtin_fmaf(saq[nr + r], w2b[r], oq);
  so[w][l] = oq;
  if (w < 4) {
    float d[MBM];
#pragma unroll
    for (int s = 0; s < MBM; ++s) d[s] = s < j ? aq * hs[s][OA + n] : 0.f;
    const float ds = wave_reduce_scatter16(d, l);
    if ((l & 3) == 0) dpart[w][l >> 2] = ds;
    const float dk = wave_sum(aq * an);
    if (l == 0) dpart[w][MBM] = dk;
  }
  __syncthreads();
  if (w == 0) {
    float y = b2bf;
#pragma unroll
    for (int v = 0; v < NWV; ++v) y += so[v][l];
    for (int s = 0; s < j; ++s) {
      const float ds = (dpart[0][s] + dpart[1][s]) + (dpart[2][s] + dpart[3][s]);
      y = __builtin_fmaf(ds + 1.f, hs[s][OU2 + l], y);
    }
    const float dk = (dpart[0][MBM] + dpart[1][MBM]) + (dpart[2][MBM] + dpart[3][MBM]);
    y = __builtin_fmaf(dk + 1.f, uo, y);
    if (LN) {
      float xh, rs;
      ln_stats(y, a.eps, xh, rs);
      y = __builtin_fmaf(gam, xh, bet);
    }
    st_io<BF16>(a.z, row + l, (RES ? qf : 0.f) + y);
    slot[OK + l] = kf;
    slot[OU2 + l] = uo;
  }
}

template <bool BF16, bool LN>
hipError_t launch_mc2(const MlpCompactArgs& a, bool res, hipStream_t s) {
  const dim3 grid(a.B * a.H), block(NWV * 64);
  if (res)
    hipLaunchKernelGGL((ttt_mlp_decode_compact_k<BF16, LN, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((ttt_mlp_decode_compact_k<BF16, LN, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_mc1(const MlpCompactArgs& a, bool ln, bool res, hipStream_t s) {
  return ln ? launch_mc2<BF16, true>(a, res, s) : launch_mc2<BF16, false>(a, res, s);
}

}  // namespace

hipError_t launch_mlp_decode_compact(const MlpCompactArgs& a, bool bf16, bool ln, bool residual,
                                     hipStream_t stream) {
  return bf16 ? launch_mc1<true>(a, ln, residual, stream)
              : launch_mc1<false>(a, ln, residual, stream);
}

}  // namespace tttk
