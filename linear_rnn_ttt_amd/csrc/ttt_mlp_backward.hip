// ttt_mlp_backward.hip -- backward pass of the TTT-MLP forward scan for gfx950.
//
// The outer loop trains the projections behind q, k and v, the initial
// state and the per-token learning rate (dmarx.github.io record LIT-801,
// "Key takeaways" item 2), so training needs the vector-Jacobian product of
// the scan: for cotangents dz (and optionally dS_T on the final state) the
// gradients of  L = sum_t <dz_t, z_t> + <dS_T, S_T>  with respect to q, k,
// v, eta, the initial state S = (W1, b1, W2, b2) and the LN gamma, beta, for
// the inner model f(x) = x + LN(GELU(x W1 + b1) W2 + b2) (the
// codewithpapers.app record's "abstract"; exact erf GELU) with 16-token
// mini-batches.
//
// Per mini-batch (base S, rows k, v, q, eta; n <= 16 tokens), the forward
// is, exactly,
//     P = K W1 + b1, A = GELU(P), O = A W2 + b2, x = LN-normalised O,
//     t = V - beta - res K, a = 2 gamma (gamma x - t),
//     G_o = rho (a - mean a - x mean(a x)),  U = G_o W2^T,  G_p = U GELU'(P),
//     PQ = Q W1 + b1 - (tril(Q K^T + 1) eta) G_p,  AQ = GELU(PQ),
//     OQ = AQ W2 + b2 - (tril(AQ A^T + 1) eta) G_o,  z = res Q + LN(OQ),
//     next base = S - (K^T (eta G_p), sum eta G_p, A^T (eta G_o), sum eta G_o),
// and its adjoint, walked over the mini-batches in reverse with the adjoint
// (A1, a1, A2, a2) of the next base, is
//     DOq = LN backward of dz,  dPQ = (DOq W2^T - (tril(DOq G_o^T) eta) A) GELU'(PQ),
//     dQ = res dz + dPQ W1^T - (tril(dPQ G_p^T) eta) K,
//     KA = K A1 + a1 + triu(K Q^T + 1) dPQ,   AA = A A2 + a2 + triu(A AQ^T + 1) DOq,
//     GA1 = G_p A1^T + triu(G_p dPQ^T) Q,   GA2 = G_o A2^T + triu(G_o DOq^T) AQ,
//     deta = -rowsum(KA G_p) - rowsum(AA G_o),
//     dU = -eta KA GELU'(P),  dG_o = -eta AA + dU W2,  LN-gradient backward -> dO, dt,
//     dV = dt,  dP = (-eta GA2 + dO W2^T) GELU'(P) - eta KA U GELU''(P),
//     dK = dP W1^T - eta GA1 - res dt,
//     A1 += Q^T dPQ + K^T dP,  a1 += sum(dPQ + dP),
//     A2 += AQ^T DOq + A^T dO + dU^T G_o,  a2 += sum(DOq + dO)
// (the same equations in fp64 numpy are checked against the autograd oracle
// on the CPU).  After the first mini-batch (A1, a1, A2, a2) is the gradient
// of the initial state.
//
// Mapping: one 512-thread workgroup (8 waves) per (batch, head) unit, two
// phases.  Phase 1 replays the forward recurrence and stores the base of
// every mini-batch in the unit's workspace; phase 2 walks the mini-batches
// in reverse.  Every product is a set of 16x16 output tiles on the matrix
// unit in fp32 (v_mfma_f32_16x16x4_f32: exact fp32 products, fp32
// accumulation), dealt round-robin to the waves, with operands read from the
// unit's workspace (bases, adjoint, per-tile intermediates: about 17 MB per
// unit at T = 2048, resident in L2 while the unit runs) and the small masked
// coefficient tiles from LDS.  Row-wise work (GELU, both LNs and the
// LN-gradient backward) runs on the VALU between the products, one
// workgroup barrier per dependent step.  Rows past T have eta = 0 and
// dz = 0 and zero inputs, so they add nothing; their outputs are not stored.
#include <hip/hip_runtime.h>

#include "ttt_device.hpp"
#include "ttt_mlp_backward.hpp"

namespace tttk {
namespace {

constexpr int D = 64;    // head dimension
constexpr int M = 256;   // hidden width
constexpr int NB = 16;   // tokens per mini-batch
constexpr int NT = 512;  // threads per workgroup
constexpr int NWV = NT / 64;
constexpr int SZ = D * M + M + M * D + D;  // floats of one state (W1, b1, W2, b2)
constexpr int OB1 = D * M, OW2 = D * M + M, OB2 = D * M + M + M * D;
constexpr int NY = 12;     // per-tile 16x64 intermediates (LDS)
constexpr int YD = D + 4;  // their row stride (rows 4 banks apart)
constexpr int XM = M + 4;  // row stride of the 16x256 intermediates
// the eight 16x256 intermediates X0..X7: five that the products read often
// in LDS, the three only used elementwise (P, U, KA / dU) in the workspace
constexpr int NXL = 5, NXG = 3;
constexpr int XSLOT[8] = {0, 0, 1, 1, 2, 3, 2, 4};   // slot in LDS or in the workspace
constexpr bool XLDS[8] = {false, true, false, true, true, true, false, true};
static_assert(SZ == MLP_BWD_STATE_FLOATS && NXG * NB * XM + 2 * D == MLP_BWD_TILE_FLOATS,
              "workspace layout and host size disagree");


__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Products C[m][n] = sum_k a(m, k) b(k, n) on 16x16 output tiles.  The
// contraction is given as one or more stretches (Seg<K>: K values of k, a
// multiple of 16, with their own a and b; k counts from 0 in each), so that
// operands stacked from different arrays need no select per element.  In a
// 16-k chunk lane (g, c) feeds a(m0 + c, k0 + 4g + j) and b(k0 + 4g + j,
// n0 + c) to product j (j < 4): its four k are consecutive, so a row-major
// operand is one 16-byte read.  The next chunk's operands are fetched before
// the current chunk's four products.
template <int K_, class FA, class FB>
struct Seg {
  static constexpr int K = K_;
  FA a;
  FB b;
};
template <int K, class FA, class FB>
__device__ __forceinline__ Seg<K, FA, FB> seg(FA a, FB b) {
  static_assert(K % 16 == 0 && K > 0, "stretches of whole 16-k chunks");
  return Seg<K, FA, FB>{a, b};
}

template <class SG>
__device__ __forceinline__ void fetch(const SG& sg, int m0, int n0, int g, int c, int k0, float* av,
                                      float* bv) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    av[j] = sg.a(m0 + c, k0 + 4 * g + j);
    bv[j] = sg.b(k0 + 4 * g + j, n0 + c);
  }
}

template <int G, class SG>
__device__ __forceinline__ void fetch_g(const SG& sg, int m0, int n0, int g, int c, int k0, int kd,
                                        float (&av)[G][4], float (&bv)[G][4]) {
#pragma unroll
  for (int q = 0; q < G; ++q) fetch(sg, m0, n0, g, c, k0 + q * kd, av[q], bv[q]);
  // keep the group's loads ahead of the products that follow: left alone,
  // the scheduler sinks each load next to its product, one round trip each
  __builtin_amdgcn_sched_barrier(0);
}
template <int G>
__device__ __forceinline__ void mma_g(const float (&av)[G][4], const float (&bv)[G][4], f32x4& acc) {
#pragma unroll
  for (int q = 0; q < G; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = mfma4(av[q][j], bv[q][j], acc);
}

// chunks first, first + step, ... of one stretch accumulated onto acc, in
// groups of G chunks whose operands are fetched together (one memory round
// trip per group).  Two register sets take turns, every fetch in the loop
// is unconditional and the loop head sees the same fetches in flight on
// every entry, so each group's products wait only for that group's operands
// (a conditional fetch, or copying one set into the other, makes the
// compiler wait for all).
template <class SG>
__device__ __forceinline__ void run_seg(const SG& sg, int m0, int n0, int g, int c, int first,
                                        int step, f32x4& acc) {
  constexpr int CH = SG::K / 16;
  constexpr int G = CH < 4 ? CH : 4;
  if (first >= CH) return;
  const int nch = (CH - first + step - 1) / step;   // chunks of this wave
  const int ngr = nch / G, rem = nch - ngr * G;
  const int kd = 16 * step;                         // k between a wave's chunks
  int k0 = 16 * first;
  if (ngr > 0) {
    float a0[G][4], b0[G][4], a1[G][4], b1[G][4];
    fetch_g<G>(sg, m0, n0, g, c, k0, kd, a0, b0);
    int i = 0;
#pragma unroll 1
    for (; i + 2 < ngr; i += 2) {
      fetch_g<G>(sg, m0, n0, g, c, k0 + (i + 1) * G * kd, kd, a1, b1);
      mma_g<G>(a0, b0, acc);
      fetch_g<G>(sg, m0, n0, g, c, k0 + (i + 2) * G * kd, kd, a0, b0);
      mma_g<G>(a1, b1, acc);
    }
    if (ngr - i == 2) {
      fetch_g<G>(sg, m0, n0, g, c, k0 + (i + 1) * G * kd, kd, a1, b1);
      mma_g<G>(a0, b0, acc);
      mma_g<G>(a1, b1, acc);
    } else {
      mma_g<G>(a0, b0, acc);
    }
    k0 += ngr * G * kd;
  }
#pragma unroll 1
  for (int r = 0; r < rem; ++r) {
    float av[1][4], bv[1][4];
    fetch_g<1>(sg, m0, n0, g, c, k0 + r * kd, kd, av, bv);
    mma_g<1>(av, bv, acc);
  }
}

// lane indices behind an empty asm: the operand addresses derived from them
// are formed at each product instead of being hoisted out of the mini-batch
// loop and held live in registers for every product site
__device__ __forceinline__ void lane_gc(int& g, int& c) {
  g = (threadIdx.x & 63) >> 4;
  c = threadIdx.x & 15;
  asm volatile("" : "+v"(g), "+v"(c));
}

// The same for the row-wise passes: an index derived from the thread id is
// taken through an empty asm where a pass starts, so the LDS addresses of
// that pass are formed there (the per-row offsets folding into the
// instructions) instead of being hoisted, one register each, out of the
// mini-batch loop.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Operand registers of one tile's whole contraction (every stretch at most
// 64 deep, i.e. one group): fetched together, one round trip per tile.
template <class... SG>
struct Bufs;
template <>
struct Bufs<> {};
template <class S0, class... R>
struct Bufs<S0, R...> {
  static constexpr int CH = S0::K / 16;
  float a[CH][4], b[CH][4];
  Bufs<R...> rest;
};
__device__ __forceinline__ void fetch_all(Bufs<>&, int, int, int, int) {}
template <class S0, class... R>
__device__ __forceinline__ void fetch_all(Bufs<S0, R...>& bf, int m0, int n0, int g, int c,
                                          const S0& s0, const R&... r) {
#pragma unroll
  for (int q = 0; q < Bufs<S0, R...>::CH; ++q) fetch(s0, m0, n0, g, c, 16 * q, bf.a[q], bf.b[q]);
  fetch_all(bf.rest, m0, n0, g, c, r...);
}
__device__ __forceinline__ void mma_all(const Bufs<>&, f32x4&) {}
template <class S0, class... R>
__device__ __forceinline__ void mma_all(const Bufs<S0, R...>& bf, f32x4& acc) {
#pragma unroll
  for (int q = 0; q < Bufs<S0, R...>::CH; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = mfma4(bf.a[q][j], bf.b[q][j], acc);
  mma_all(bf.rest, acc);
}

// R x C output (multiples of 16): tiles dealt to waves w0, w0 + nw, ... of
// the workgroup, tile (m0, n0) ending in epi(m0, n0, acc, pre), acc[i] at
// lane (g, c) being C[m0 + 4g + i][n0 + c] and pre = pre(m0, n0) a value the
// epilogue needs from memory (the old state or adjoint tile, or workspace
// intermediates), fetched one tile ahead.  When every stretch is at most 64
// deep, a tile's operands are fetched in one go, and with few operand
// registers (at most 24) the next tile's operands and pre are fetched while
// the current tile's products run (two register sets, tiles in pairs; the
// last fetch repeats the last tile).
template <int R, int C, class PRE, class EPI, class... SG>
__device__ __forceinline__ void gemm_p(int wave, int w0, int nw, PRE pre, EPI epi,
                                       const SG&... sg) {
  static_assert(R % 16 == 0 && C % 16 == 0, "tile multiples");
  int g, c;
  lane_gc(g, c);
  constexpr int TN = C / 16, TILES = (R / 16) * TN;
  constexpr bool SMALL = ((SG::K <= 64) && ...);
  constexpr int REGS = ((SG::K / 2) + ...);   // operand floats per lane and tile
  if (wave < w0 || wave >= w0 + nw) return;
  const int t0 = wave - w0;
  if constexpr (SMALL && REGS <= 24) {
    const int nt = (TILES - t0 + nw - 1) / nw;   // tiles of this wave
    auto tm = [&](int i) { return ((t0 + min(i, nt - 1) * nw) / TN) * 16; };
    auto tn = [&](int i) { return ((t0 + min(i, nt - 1) * nw) % TN) * 16; };
    Bufs<SG...> A, B;
    auto pa = pre(tm(0), tn(0));
    fetch_all(A, tm(0), tn(0), g, c, sg...);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll 1
    for (int i = 0; i < nt; i += 2) {
      auto pb = pre(tm(i + 1), tn(i + 1));
      fetch_all(B, tm(i + 1), tn(i + 1), g, c, sg...);
      __builtin_amdgcn_sched_barrier(0);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      mma_all(A, acc);
      epi(tm(i), tn(i), acc, pa);
      if (i + 1 >= nt) break;
      pa = pre(tm(i + 2), tn(i + 2));
      fetch_all(A, tm(i + 2), tn(i + 2), g, c, sg...);
      __builtin_amdgcn_sched_barrier(0);
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
      mma_all(B, acc);
      epi(tm(i + 1), tn(i + 1), acc, pb);
    }
  } else if constexpr (SMALL) {
#pragma unroll 1
    for (int t = t0; t < TILES; t += nw) {
      const int m0 = (t / TN) * 16, n0 = (t % TN) * 16;
      const auto pv = pre(m0, n0);
      Bufs<SG...> A;
      fetch_all(A, m0, n0, g, c, sg...);
      __builtin_amdgcn_sched_barrier(0);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      mma_all(A, acc);
      epi(m0, n0, acc, pv);
    }
  } else {
    int t = t0;
    auto nxt = pre((t / TN) * 16, (t % TN) * 16);
#pragma unroll 1
    for (; t < TILES; t += nw) {
      const int m0 = (t / TN) * 16, n0 = (t % TN) * 16;
      const auto cur = nxt;
      const int tq = t + nw < TILES ? t + nw : t;
      nxt = pre((tq / TN) * 16, (tq % TN) * 16);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      (run_seg(sg, m0, n0, g, c, 0, 1, acc), ...);
      epi(m0, n0, acc, cur);
    }
  }
}

struct Zero {
  __device__ f32x4 operator()(int, int) const { return f32x4{0.f, 0.f, 0.f, 0.f}; }
};

template <int R, int C, class EPI, class... SG>
__device__ __forceinline__ void gemm_s(int wave, int w0, int nw, EPI epi, const SG&... sg) {
  gemm_p<R, C>(
      wave, w0, nw, Zero{}, [&](int m0, int n0, f32x4 acc, const f32x4&) { epi(m0, n0, acc); },
      sg...);
}

template <int R, int C, int K, class FA, class FB, class EPI>
__device__ __forceinline__ void gemm(int wave, int w0, int nw, FA a, FB b, EPI epi) {
  gemm_s<R, C>(wave, w0, nw, epi, seg<K>(a, b));
}

// The same product with the contraction split over S waves per output tile,
// for products of few tiles (TILES * S <= 8 waves): wave w takes tile
// w % TILES and the 16-k chunks (counted over all stretches) w / TILES,
// w / TILES + S, ...; the partial tiles meet in `part` (LDS, (S - 1) * TILES
// tiles) and the first wave of each tile adds them up and runs epi.  Every
// wave of the workgroup must call it (it holds a barrier).  Consecutive
// calls alternate between two `part` buffers, so a buffer is written again
// only after a later barrier that follows its reads.
template <int CB, int S, class SG>
__device__ __forceinline__ void run_seg_ks(const SG& sg, int m0, int n0, int g, int c, int p,
                                           f32x4& acc) {
  // first local chunk whose global index CB + l is p mod S
  const int first = ((p - CB) % S + S) % S;
  run_seg(sg, m0, n0, g, c, first, S, acc);
}
template <int R, int C, int S, class EPI, class SG0>
__device__ __forceinline__ void ks_body(int p, int m0, int n0, int g, int c, f32x4& acc,
                                        const SG0& s0) {
  run_seg_ks<0, S>(s0, m0, n0, g, c, p, acc);
}
template <int R, int C, int S, class EPI, class SG0, class SG1>
__device__ __forceinline__ void ks_body(int p, int m0, int n0, int g, int c, f32x4& acc,
                                        const SG0& s0, const SG1& s1) {
  run_seg_ks<0, S>(s0, m0, n0, g, c, p, acc);
  run_seg_ks<SG0::K / 16, S>(s1, m0, n0, g, c, p, acc);
}
template <int R, int C, int S, class EPI, class... SG>
__device__ __forceinline__ void gemm_kss(int wave, f32x4* part, EPI epi, const SG&... sg) {
  static_assert(R % 16 == 0 && C % 16 == 0, "tile multiples");
  constexpr int TN = C / 16, TILES = (R / 16) * TN;
  static_assert(TILES * S <= NWV && S >= 1, "one wave per tile and part");
  int g, c;
  lane_gc(g, c);
  const int lane = threadIdx.x & 63;
  const int t = wave % TILES, p = wave / TILES;
  const int m0 = (t / TN) * 16, n0 = (t % TN) * 16;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (p < S) {
    ks_body<R, C, S, EPI>(p, m0, n0, g, c, acc, sg...);
    if (p > 0) part[((p - 1) * TILES + t) * 64 + lane] = acc;
  }
  __syncthreads();
  if (p == 0) {
#pragma unroll
    for (int q = 1; q < S; ++q) acc += part[((q - 1) * TILES + t) * 64 + lane];
    epi(m0, n0, acc);
  }
}
template <int R, int C, int K, int S, class FA, class FB, class EPI>
__device__ __forceinline__ void gemm_ks(int wave, f32x4* part, FA a, FB b, EPI epi) {
  gemm_kss<R, C, S>(wave, part, epi, seg<K>(a, b));
}

// two stretches: a1, a2, b1, b2, epi
template <int R, int C, int K1, int K2, class FA1, class FA2, class FB1, class FB2, class EPI>
__device__ __forceinline__ void gemm2(int wave, int w0, int nw, FA1 a1, FA2 a2, FB1 b1, FB2 b2,
                                      EPI epi) {
  gemm_s<R, C>(wave, w0, nw, epi, seg<K1>(a1, b1), seg<K2>(a2, b2));
}
template <int R, int C, int K1, int K2, int S, class FA1, class FA2, class FB1, class FB2,
          class EPI>
__device__ __forceinline__ void gemm_ks2(int wave, f32x4* part, FA1 a1, FA2 a2, FB1 b1, FB2 b2,
                                         EPI epi) {
  gemm_kss<R, C, S>(wave, part, epi, seg<K1>(a1, b1), seg<K2>(a2, b2));
}

// Sum over the 32 lanes of a half-wave.
__device__ __forceinline__ float sum32(float x) {
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// GELU(x) = x Phi(x), GELU'(x) = Phi(x) + x phi(x), GELU''(x) = phi(x) (2 - x^2).
__device__ __forceinline__ float phi_cdf(float x) { return 0.5f * (1.f + erff(x * 0.70710678118654752f)); }
__device__ __forceinline__ float phi_pdf(float x) { return 0.39894228040143268f * expf(-0.5f * x * x); }
__device__ __forceinline__ float gelu(float x) { return x * phi_cdf(x); }
__device__ __forceinline__ float gelu1(float x) { return phi_cdf(x) + x * phi_pdf(x); }
__device__ __forceinline__ float gelu2(float x) { return phi_pdf(x) * (2.f - x * x); }

template <bool BF16>
__device__ __forceinline__ float ld_io(const void* p, size_t i) {
  if constexpr (BF16) {
    const uint16_t u = static_cast<const uint16_t*>(p)[i];
    return __builtin_bit_cast(float, static_cast<uint32_t>(u) << 16);
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

struct Lds {
  float m[8][16][17];   // masked 16x16 coefficient tiles
  float eta[16];
  float rho[16], ma[16], mx[16];   // K-side LN: 1/sigma, mean(a), mean(a x)
  f32x4 part[2][7][64];            // partial tiles of the split-contraction products
  union {
    float y[NY][NB][YD];           // per-tile 16 x 64 intermediates, rows padded
    float dln[16][2][D];           // after the walk: dgamma, dbeta partials per token slot
  };
  float x[NXL][NB][XM];            // the LDS-resident 16 x 256 intermediates
};

template <bool BF16, bool LN, bool RES>
__global__ __launch_bounds__(NT) void ttt_mlp_bwd_k(MlpBackwardArgs a) {
  __shared__ Lds L;
  const int unit = blockIdx.x, head = unit % a.H;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = a.T, n = (T + 15) / 16;
  // 16-byte aligned: the workspace starts on 256 bytes and unit_floats is a
  // multiple of 4, so row-major state reads can be 16-byte loads
  float* ws = static_cast<float*>(
      __builtin_assume_aligned(a.ws + static_cast<size_t>(unit) * a.unit_floats, 16));
  float* bases = ws;
  float* adj = ws + static_cast<size_t>(n) * SZ;
  float* Xb = adj + SZ;
  float* dln_out = ws + a.unit_floats - 2 * D;   // the unit's dgamma, dbeta
  auto X = [&](int i) { return XLDS[i] ? &L.x[XSLOT[i]][0][0] : Xb + XSLOT[i] * NB * XM; };
  auto Y = [&](int i) { return &L.y[i][0][0]; };
  const float* gam = a.gamma + static_cast<size_t>(head) * D;
  const float* bet = a.beta + static_cast<size_t>(head) * D;
  const size_t row0 = static_cast<size_t>(unit) * T;   // first token row of the unit

  // ---- base 0 = the initial state; adjoint = dS_T (or zero); dln = 0
  {
    const size_t s0 = a.state0_per_batch ? unit : head;
    const float* src[4] = {a.w1 + s0 * D * M, a.b1 + s0 * M, a.w2 + s0 * M * D, a.b2 + s0 * D};
    const int off[4] = {0, OB1, OW2, OB2}, len[4] = {D * M, M, M * D, D};
    for (int p = 0; p < 4; ++p)
      for (int i = tid; i < len[p]; i += NT) bases[off[p] + i] = src[p][i];
    const float* fin[4] = {a.dw1_final, a.db1_final, a.dw2_final, a.db2_final};
    for (int p = 0; p < 4; ++p)
      for (int i = tid; i < len[p]; i += NT)
        adj[off[p] + i] = fin[p] ? fin[p][static_cast<size_t>(unit) * len[p] + i] : 0.f;
  }
  // dgamma, dbeta partials of this thread's token slot (2 wave + lane / 32)
  // and features 2 (lane % 32), +1, summed over the tiles
  float dg_acc[2] = {0.f, 0.f}, db_acc[2] = {0.f, 0.f};

  // inputs of tile c as fp32 rows (zero past T): K -> Y0, Q -> Y1, V -> Y2,
  // dz -> Y3 (with_dz), eta -> LDS (zero past T)
  auto load_tile = [&](int c, bool with_dz) {
    for (int i = opaque(tid); i < NB * D; i += NT) {
      const int s = i / D, f = i % D, tok = c * NB + s;
      const bool ok = tok < T;
      const size_t e = (row0 + tok) * D + f;
      Y(0)[s * YD + f] = ok ? ld_io<BF16>(a.k, e) : 0.f;
      Y(1)[s * YD + f] = ok ? ld_io<BF16>(a.q, e) : 0.f;
      Y(2)[s * YD + f] = ok ? ld_io<BF16>(a.v, e) : 0.f;
      if (with_dz) Y(3)[s * YD + f] = ok ? ld_io<BF16>(a.dz, e) : 0.f;
    }
    if (tid < NB) L.eta[tid] = c * NB + tid < T ? a.eta[row0 + c * NB + tid] : 0.f;
  };

  // K side at base S (steps shared by both phases):
  //   X0 = P, X1 = A, Y4 = O, Y5 = x, Y2 = t (overwrites v), Y6 = G_o,
  //   X2 = U, X3 = G_p; LDS: rho, ma, mx.
  auto kside = [&](const float* S) {
    const float* W1 = S;
    const float* b1 = S + OB1;
    const float* W2 = S + OW2;
    const float* b2 = S + OB2;
    gemm<NB, M, D>(wave, 0, NWV, [&](int m, int k) { return Y(0)[m * YD + k]; },
                   [&](int k, int nn) { return W1[k * M + nn]; },
                   [&](int m0, int n0, f32x4 acc) {
                     const int nn = n0 + (lane & 15);
#pragma unroll
                     for (int i = 0; i < 4; ++i) {
                       const float p = acc[i] + b1[nn];
                       X(0)[(m0 + 4 * g + i) * XM + nn] = p;
                       X(1)[(m0 + 4 * g + i) * XM + nn] = gelu(p);
                     }
                   });
    __syncthreads();
    gemm_ks<NB, D, M, 2>(wave, L.part[0][0], [&](int m, int k) { return X(1)[m * XM + k]; },
                   [&](int k, int j) { return W2[k * D + j]; },
                   [&](int m0, int n0, f32x4 acc) {
                     const int j = n0 + (lane & 15);
#pragma unroll
                     for (int i = 0; i < 4; ++i) Y(4)[(m0 + 4 * g + i) * YD + j] = acc[i] + b2[j];
                   });
    __syncthreads();
    // LN of O and the loss gradient G_o: wave w has tokens 2w, 2w+1; lane
    // half h, feature pair 2(l % 32), +1
    {
      const int ol = opaque(lane), s = 2 * wave + (ol >> 5), f = 2 * (ol & 31);
      float o[2], t[2], x[2], av[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        o[u] = Y(4)[s * YD + f + u];
        const float kk = RES ? Y(0)[s * YD + f + u] : 0.f;
        t[u] = Y(2)[s * YD + f + u] - (LN ? bet[f + u] : 0.f) - kk;
      }
      if (LN) {
        const float mu = sum32(o[0] + o[1]) * (1.f / D);
        const float var = sum32((o[0] - mu) * (o[0] - mu) + (o[1] - mu) * (o[1] - mu)) * (1.f / D);
        const float rho = 1.f / sqrtf(var + a.eps);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          x[u] = (o[u] - mu) * rho;
          av[u] = 2.f * gam[f + u] * (gam[f + u] * x[u] - t[u]);
        }
        const float ma = sum32(av[0] + av[1]) * (1.f / D);
        const float mx = sum32(av[0] * x[0] + av[1] * x[1]) * (1.f / D);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          Y(5)[s * YD + f + u] = x[u];
          Y(6)[s * YD + f + u] = rho * (av[u] - ma - x[u] * mx);
        }
        if ((lane & 31) == 0) {
          L.rho[s] = rho;
          L.ma[s] = ma;
          L.mx[s] = mx;
        }
      } else {
#pragma unroll
        for (int u = 0; u < 2; ++u) Y(6)[s * YD + f + u] = 2.f * (o[u] - t[u]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) Y(2)[s * YD + f + u] = t[u];
    }
    __syncthreads();
    // U = G_o W2^T, G_p = U GELU'(P)
    gemm_p<NB, M>(
        wave, 0, NWV,
        [&](int m0, int n0) {   // P of the tile, from the workspace
          f32x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = X(0)[(m0 + 4 * g + i) * XM + n0 + (lane & 15)];
          return v;
        },
        [&](int m0, int n0, f32x4 acc, const f32x4& pv) {
          const int nn = n0 + (lane & 15);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = (m0 + 4 * g + i) * XM + nn;
            X(2)[e] = acc[i];
            X(3)[e] = acc[i] * gelu1(pv[i]);
          }
        },
        seg<D>([&](int m, int k) { return Y(6)[m * YD + k]; },
               [&](int k, int nn) { return W2[nn * D + k]; }));
    __syncthreads();
  };

  // ---- phase 1: replay the forward recurrence, storing every base
  for (int c = 0; c + 1 < n; ++c) {
    load_tile(c, false);
    __syncthreads();
    const float* S = bases + static_cast<size_t>(c) * SZ;
    float* Sn = bases + static_cast<size_t>(c + 1) * SZ;
    kside(S);
    // W1' = W1 - K^T (eta G_p), W2' = W2 - A^T (eta G_o)
    // (the old tile of S is fetched one tile ahead)
    gemm_p<D, M>(
        wave, 0, NWV,
        [&](int m0, int n0) {
          f32x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = S[(m0 + 4 * g + i) * M + n0 + (lane & 15)];
          return v;
        },
        [&](int m0, int n0, f32x4 acc, f32x4 old) {
#pragma unroll
          for (int i = 0; i < 4; ++i) Sn[(m0 + 4 * g + i) * M + n0 + (lane & 15)] = old[i] - acc[i];
        },
        seg<NB>([&](int f, int s) { return Y(0)[s * YD + f]; },
                [&](int s, int nn) { return L.eta[s] * X(3)[s * XM + nn]; }));
    gemm_p<M, D>(
        wave, 0, NWV,
        [&](int m0, int n0) {
          f32x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = S[OW2 + (m0 + 4 * g + i) * D + n0 + (lane & 15)];
          return v;
        },
        [&](int m0, int n0, f32x4 acc, f32x4 old) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            Sn[OW2 + (m0 + 4 * g + i) * D + n0 + (lane & 15)] = old[i] - acc[i];
        },
        seg<NB>([&](int nn, int s) { return X(1)[s * XM + nn]; },
                [&](int s, int j) { return L.eta[s] * Y(6)[s * YD + j]; }));
    for (int nn = opaque(tid); nn < M + D; nn += NT) {
      float sum = 0.f;
      if (nn < M) {
        for (int s = 0; s < NB; ++s) sum += L.eta[s] * X(3)[s * XM + nn];
        Sn[OB1 + nn] = S[OB1 + nn] - sum;
      } else {
        const int j = nn - M;
        for (int s = 0; s < NB; ++s) sum += L.eta[s] * Y(6)[s * YD + j];
        Sn[OB2 + j] = S[OB2 + j] - sum;
      }
    }
    __syncthreads();
  }

  // ---- phase 2: the mini-batches in reverse
  for (int c = n - 1; c >= 0; --c) {
    load_tile(c, true);
    __syncthreads();
    const float* S = bases + static_cast<size_t>(c) * SZ;
    const float* W1 = S;
    const float* b1 = S + OB1;
    const float* W2 = S + OW2;
    const float* b2 = S + OB2;
    kside(S);
    const float* K = Y(0);
    const float* Q = Y(1);
    const float* P = X(0);
    const float* A = X(1);
    const float* Gp = X(3);
    const float* Go = Y(6);
    auto tril_eta = [&](int idx, int i, int s, float v) {  // [i][s] for s <= i, scaled by eta_s
      L.m[idx][i][s] = s <= i ? v * L.eta[s] : 0.f;
    };
    // M1 = tril(Q K^T + 1) eta
    gemm_ks<NB, NB, D, 4>(wave, L.part[1][0], [&](int i, int f) { return Q[i * YD + f]; },
                    [&](int f, int s) { return K[s * YD + f]; },
                    [&](int m0, int n0, f32x4 acc) {
#pragma unroll
                      for (int i = 0; i < 4; ++i)
                        tril_eta(0, 4 * g + i, lane & 15, acc[i] + 1.f);
                    });
    __syncthreads();
    // PQ = Q W1 + b1 - M1 G_p -> X4, AQ = GELU(PQ) -> X5
    gemm2<NB, M, D, NB>(
        wave, 0, NWV,
        [&](int i, int k) { return Q[i * YD + k]; },
        [&](int i, int k) { return -L.m[0][i][k]; },
        [&](int k, int nn) { return W1[k * M + nn]; },
        [&](int k, int nn) { return Gp[k * XM + nn]; },
        [&](int m0, int n0, f32x4 acc) {
          const int nn = n0 + (lane & 15);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = acc[i] + b1[nn];
            X(4)[(m0 + 4 * g + i) * XM + nn] = p;
            X(5)[(m0 + 4 * g + i) * XM + nn] = gelu(p);
          }
        });
    __syncthreads();
    const float* AQ = X(5);
    // M2 = tril(AQ A^T + 1) eta
    gemm_ks<NB, NB, M, 8>(wave, L.part[0][0], [&](int i, int k) { return AQ[i * XM + k]; },
                    [&](int k, int s) { return A[s * XM + k]; },
                    [&](int m0, int n0, f32x4 acc) {
#pragma unroll
                      for (int i = 0; i < 4; ++i)
                        tril_eta(1, 4 * g + i, lane & 15, acc[i] + 1.f);
                    });
    __syncthreads();
    // OQ = AQ W2 + b2 - M2 G_o -> Y7
    gemm_ks2<NB, D, M, NB, 2>(
        wave, L.part[1][0],
        [&](int i, int k) { return AQ[i * XM + k]; },
        [&](int i, int k) { return -L.m[1][i][k]; },
        [&](int k, int j) { return W2[k * D + j]; },
        [&](int k, int j) { return Go[k * YD + j]; },
        [&](int m0, int n0, f32x4 acc) {
          const int j = n0 + (lane & 15);
#pragma unroll
          for (int i = 0; i < 4; ++i) Y(7)[(m0 + 4 * g + i) * YD + j] = acc[i] + b2[j];
        });
    __syncthreads();
    // output LN backward: DOq -> Y7; dgamma, dbeta
    {
      const int ol = opaque(lane), s = 2 * wave + (ol >> 5), f = 2 * (ol & 31);
      float o[2], dz[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        o[u] = Y(7)[s * YD + f + u];
        dz[u] = Y(3)[s * YD + f + u];
      }
      if (LN) {
        const float mu = sum32(o[0] + o[1]) * (1.f / D);
        const float var = sum32((o[0] - mu) * (o[0] - mu) + (o[1] - mu) * (o[1] - mu)) * (1.f / D);
        const float rho = 1.f / sqrtf(var + a.eps);
        float x[2], gd[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          x[u] = (o[u] - mu) * rho;
          gd[u] = gam[f + u] * dz[u];
        }
        const float m1 = sum32(gd[0] + gd[1]) * (1.f / D);
        const float m2 = sum32(gd[0] * x[0] + gd[1] * x[1]) * (1.f / D);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          Y(7)[s * YD + f + u] = rho * (gd[u] - m1 - x[u] * m2);
          dg_acc[u] += dz[u] * x[u];
          db_acc[u] += dz[u];
        }
      } else {
#pragma unroll
        for (int u = 0; u < 2; ++u) Y(7)[s * YD + f + u] = dz[u];
      }
    }
    __syncthreads();
    const float* DOq = Y(7);
    // Mdo = tril(DOq G_o^T) eta
    gemm_ks<NB, NB, D, 4>(wave, L.part[0][0], [&](int i, int j) { return DOq[i * YD + j]; },
                    [&](int j, int s) { return Go[s * YD + j]; },
                    [&](int m0, int n0, f32x4 acc) {
#pragma unroll
                      for (int i = 0; i < 4; ++i) tril_eta(2, 4 * g + i, lane & 15, acc[i]);
                    });
    __syncthreads();
    // dPQ = (DOq W2^T - Mdo A) GELU'(PQ) -> X4
    gemm2<NB, M, D, NB>(
        wave, 0, NWV,
        [&](int i, int k) { return DOq[i * YD + k]; },
        [&](int i, int k) { return -L.m[2][i][k]; },
        [&](int k, int nn) { return W2[nn * D + k]; },
        [&](int k, int nn) { return A[k * XM + nn]; },
        [&](int m0, int n0, f32x4 acc) {
          const int nn = n0 + (lane & 15);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = (m0 + 4 * g + i) * XM + nn;
            X(4)[e] = acc[i] * gelu1(X(4)[e]);
          }
        });
    __syncthreads();
    const float* dPQ = X(4);
    // the masked coefficient tiles that need dPQ / DOq, one wave each:
    //   Mdp = tril(dPQ G_p^T) eta, Tk = triu(K Q^T + 1), Ta = triu(A AQ^T + 1),
    //   Tgp = triu(G_p dPQ^T), Tgo = triu(G_o DOq^T)   ([s][i] for i >= s)
    auto triu_put = [&](int idx, int s, int i, float v) { L.m[idx][s][i] = i >= s ? v : 0.f; };
    gemm_ks<NB, NB, M, 8>(wave, L.part[1][0], [&](int i, int k) { return dPQ[i * XM + k]; },
                    [&](int k, int s) { return Gp[s * XM + k]; },
                    [&](int m0, int n0, f32x4 acc) {
#pragma unroll
                      for (int i = 0; i < 4; ++i) tril_eta(3, 4 * g + i, lane & 15, acc[i]);
                    });
    gemm_ks<NB, NB, D, 4>(wave, L.part[0][0], [&](int s, int f) { return K[s * YD + f]; },
                    [&](int f, int i) { return Q[i * YD + f]; },
                    [&](int m0, int n0, f32x4 acc) {
#pragma unroll
                      for (int i = 0; i < 4; ++i) triu_put(4, 4 * g + i, lane & 15, acc[i] + 1.f);
                    });
    gemm_ks<NB, NB, M, 8>(wave, L.part[1][0], [&](int s, int k) { return A[s * XM + k]; },
                    [&](int k, int i) { return AQ[i * XM + k]; },
                    [&](int m0, int n0, f32x4 acc) {
#pragma unroll
                      for (int i = 0; i < 4; ++i) triu_put(5, 4 * g + i, lane & 15, acc[i] + 1.f);
                    });
    gemm_ks<NB, NB, M, 8>(wave, L.part[0][0], [&](int s, int k) { return Gp[s * XM + k]; },
                    [&](int k, int i) { return dPQ[i * XM + k]; },
                    [&](int m0, int n0, f32x4 acc) {
#pragma unroll
                      for (int i = 0; i < 4; ++i) triu_put(6, 4 * g + i, lane & 15, acc[i]);
                    });
    gemm_ks<NB, NB, D, 4>(wave, L.part[1][0], [&](int s, int j) { return Go[s * YD + j]; },
                    [&](int j, int i) { return DOq[i * YD + j]; },
                    [&](int m0, int n0, f32x4 acc) {
#pragma unroll
                      for (int i = 0; i < 4; ++i) triu_put(7, 4 * g + i, lane & 15, acc[i]);
                    });
    __syncthreads();
    const float* A1 = adj;
    const float* a1 = adj + OB1;
    const float* A2 = adj + OW2;
    const float* a2 = adj + OB2;
    // dQ = res dz + dPQ W1^T - Mdp K (stored); KA = K A1 + a1 + Tk dPQ -> X6;
    // AA = A A2 + a2 + Ta DOq -> Y8; GA1 = G_p A1^T + Tgp Q -> Y9;
    // GA2 = G_o A2^T + Tgo AQ -> X7
    gemm_ks2<NB, D, M, NB, 2>(
        wave, L.part[0][0],
        [&](int i, int k) { return dPQ[i * XM + k]; },
        [&](int i, int k) { return -L.m[3][i][k]; },
        [&](int k, int f) { return W1[f * M + k]; },
        [&](int k, int f) { return K[k * YD + f]; },
        [&](int m0, int n0, f32x4 acc) {
          const int f = n0 + (lane & 15);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int s = m0 + 4 * g + i, tok = c * NB + s;
            const float v = acc[i] + (RES ? Y(3)[s * YD + f] : 0.f);
            if (tok < T) st_io<BF16>(a.dq, (row0 + tok) * D + f, v);
          }
        });
    gemm2<NB, M, D, NB>(
        wave, 0, NWV,
        [&](int s, int k) { return K[s * YD + k]; },
        [&](int s, int k) { return L.m[4][s][k]; },
        [&](int k, int nn) { return A1[k * M + nn]; },
        [&](int k, int nn) { return dPQ[k * XM + nn]; },
        [&](int m0, int n0, f32x4 acc) {
          const int nn = n0 + (lane & 15);
#pragma unroll
          for (int i = 0; i < 4; ++i) X(6)[(m0 + 4 * g + i) * XM + nn] = acc[i] + a1[nn];
        });
    gemm_ks2<NB, D, M, NB, 2>(
        wave, L.part[1][0],
        [&](int s, int k) { return A[s * XM + k]; },
        [&](int s, int k) { return L.m[5][s][k]; },
        [&](int k, int j) { return A2[k * D + j]; },
        [&](int k, int j) { return DOq[k * YD + j]; },
        [&](int m0, int n0, f32x4 acc) {
          const int j = n0 + (lane & 15);
#pragma unroll
          for (int i = 0; i < 4; ++i) Y(8)[(m0 + 4 * g + i) * YD + j] = acc[i] + a2[j];
        });
    gemm_ks2<NB, D, M, NB, 2>(
        wave, L.part[0][0],
        [&](int s, int k) { return Gp[s * XM + k]; },
        [&](int s, int k) { return L.m[6][s][k]; },
        [&](int k, int f) { return A1[f * M + k]; },
        [&](int k, int f) { return Q[k * YD + f]; },
        [&](int m0, int n0, f32x4 acc) {
          const int f = n0 + (lane & 15);
#pragma unroll
          for (int i = 0; i < 4; ++i) Y(9)[(m0 + 4 * g + i) * YD + f] = acc[i];
        });
    gemm2<NB, M, D, NB>(
        wave, 0, NWV,
        [&](int s, int k) { return Go[s * YD + k]; },
        [&](int s, int k) { return L.m[7][s][k]; },
        [&](int k, int nn) { return A2[nn * D + k]; },
        [&](int k, int nn) { return AQ[k * XM + nn]; },
        [&](int m0, int n0, f32x4 acc) {
          const int nn = n0 + (lane & 15);
#pragma unroll
          for (int i = 0; i < 4; ++i) X(7)[(m0 + 4 * g + i) * XM + nn] = acc[i];
        });
    __syncthreads();
    // deta = -rowsum(KA G_p) - rowsum(AA G_o); dU = -eta KA GELU'(P) -> X6;
    // -eta KA U GELU''(P) -> X2
    {
      const int ol = opaque(lane), s = 2 * wave + (ol >> 5), l32 = ol & 31;
      float acc = 0.f;
      for (int nn = l32; nn < M; nn += 32) acc += X(6)[s * XM + nn] * Gp[s * XM + nn];
      for (int j = l32; j < D; j += 32) acc += Y(8)[s * YD + j] * Go[s * YD + j];
      acc = sum32(acc);
      const int tok = c * NB + s;
      if (l32 == 0 && tok < T) a.deta[row0 + tok] = -acc;
    }
    __syncthreads();
    {
      // all 24 workspace loads in flight before the arithmetic
      static_assert(NB * M == 8 * NT, "eight elements per thread");
      const int i0 = opaque(tid);
      float pv[8], kv[8], uv[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int i = i0 + r * NT, e = (i / M) * XM + i % M;
        pv[r] = P[e];
        kv[r] = X(6)[e];
        uv[r] = X(2)[e];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int i = i0 + r * NT, s = i / M, e = s * XM + i % M;
        const float dgp = -L.eta[s] * kv[r];
        X(2)[e] = dgp * uv[r] * gelu2(pv[r]);
        X(6)[e] = dgp * gelu1(pv[r]);
      }
    }
    __syncthreads();
    const float* dU = X(6);
    // dG_o = -eta AA + dU W2 -> Y8
    gemm_ks<NB, D, M, 2>(wave, L.part[1][0], [&](int s, int k) { return dU[s * XM + k]; },
                   [&](int k, int j) { return W2[k * D + j]; },
                   [&](int m0, int n0, f32x4 acc) {
                     const int j = n0 + (lane & 15);
#pragma unroll
                     for (int i = 0; i < 4; ++i) {
                       const int s = m0 + 4 * g + i;
                       Y(8)[s * YD + j] = acc[i] - L.eta[s] * Y(8)[s * YD + j];
                     }
                   });
    __syncthreads();
    // LN-gradient backward: dO -> Y10, dt -> Y11 (dv stored), dgamma, dbeta
    {
      const int ol = opaque(lane), s = 2 * wave + (ol >> 5), f = 2 * (ol & 31);
      const int tok = c * NB + s;
      float u[2], dO[2], dt[2];
#pragma unroll
      for (int v = 0; v < 2; ++v) u[v] = Y(8)[s * YD + f + v];
      if (LN) {
        const float rho = L.rho[s], ma = L.ma[s], mx = L.mx[s];
        float x[2], t[2], av[2];
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          x[v] = Y(5)[s * YD + f + v];
          t[v] = Y(2)[s * YD + f + v];
          av[v] = 2.f * gam[f + v] * (gam[f + v] * x[v] - t[v]);
        }
        const float drho = sum32(u[0] * (av[0] - ma - x[0] * mx) + u[1] * (av[1] - ma - x[1] * mx));
        const float mu_ = sum32(u[0] + u[1]) * (1.f / D);
        const float mux = sum32(u[0] * x[0] + u[1] * x[1]) * (1.f / D);
        float da[2], dx[2];
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          da[v] = rho * (u[v] - mu_ - x[v] * mux);
          dx[v] = -rho * (mx * u[v] + av[v] * mux) + 2.f * gam[f + v] * gam[f + v] * da[v];
          dt[v] = -2.f * gam[f + v] * da[v];
        }
        const float mdx = sum32(dx[0] + dx[1]) * (1.f / D);
        const float mdxx = sum32(dx[0] * x[0] + dx[1] * x[1]) * (1.f / D);
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          dO[v] = rho * (dx[v] - mdx - x[v] * mdxx) - drho * rho * rho * x[v] * (1.f / D);
          dg_acc[v] += 2.f * (2.f * gam[f + v] * x[v] - t[v]) * da[v];
          db_acc[v] -= dt[v];
        }
      } else {
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          dO[v] = 2.f * u[v];
          dt[v] = -2.f * u[v];
        }
      }
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        Y(10)[s * YD + f + v] = dO[v];
        Y(11)[s * YD + f + v] = dt[v];
        if (tok < T) st_io<BF16>(a.dv, (row0 + tok) * D + f + v, dt[v]);
      }
    }
    __syncthreads();
    const float* dOk = Y(10);
    // dP = (-eta GA2 + dO W2^T) GELU'(P) + X2 -> X7
    struct PX2 { f32x4 p, x2; };
    gemm_p<NB, M>(
        wave, 0, NWV,
        [&](int m0, int n0) {   // P and X2 of the tile, from the workspace
          PX2 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = (m0 + 4 * g + i) * XM + n0 + (lane & 15);
            v.p[i] = P[e];
            v.x2[i] = X(2)[e];
          }
          return v;
        },
        [&](int m0, int n0, f32x4 acc, const PX2& v) {
          const int nn = n0 + (lane & 15);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int s = m0 + 4 * g + i, e = s * XM + nn;
            X(7)[e] = (acc[i] - L.eta[s] * X(7)[e]) * gelu1(v.p[i]) + v.x2[i];
          }
        },
        seg<D>([&](int s, int k) { return dOk[s * YD + k]; },
               [&](int k, int nn) { return W2[nn * D + k]; }));
    __syncthreads();
    const float* dP = X(7);
    // dK = dP W1^T - eta GA1 - res dt (stored)
    gemm_ks<NB, D, M, 2>(wave, L.part[0][0], [&](int s, int k) { return dP[s * XM + k]; },
                   [&](int k, int f) { return W1[f * M + k]; },
                   [&](int m0, int n0, f32x4 acc) {
                     const int f = n0 + (lane & 15);
#pragma unroll
                     for (int i = 0; i < 4; ++i) {
                       const int s = m0 + 4 * g + i, tok = c * NB + s;
                       const float v = acc[i] - L.eta[s] * Y(9)[s * YD + f] -
                                       (RES ? Y(11)[s * YD + f] : 0.f);
                       if (tok < T) st_io<BF16>(a.dk, (row0 + tok) * D + f, v);
                     }
                   });
    // A1 += Q^T dPQ + K^T dP;  A2 += AQ^T DOq + A^T dO + dU^T G_o
    float* A1w = adj;
    float* A2w = adj + OW2;
    gemm_p<D, M>(
        wave, 0, NWV,
        [&](int m0, int n0) {
          f32x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = A1w[(m0 + 4 * g + i) * M + n0 + (lane & 15)];
          return v;
        },
        [&](int m0, int n0, f32x4 acc, f32x4 old) {
#pragma unroll
          for (int i = 0; i < 4; ++i) A1w[(m0 + 4 * g + i) * M + n0 + (lane & 15)] = old[i] + acc[i];
        },
        seg<NB>([&](int f, int k) { return Q[k * YD + f]; },
                [&](int k, int nn) { return dPQ[k * XM + nn]; }),
        seg<NB>([&](int f, int k) { return K[k * YD + f]; },
                [&](int k, int nn) { return dP[k * XM + nn]; }));
    gemm_p<M, D>(
        wave, 0, NWV,
        [&](int m0, int n0) {
          f32x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = A2w[(m0 + 4 * g + i) * D + n0 + (lane & 15)];
          return v;
        },
        [&](int m0, int n0, f32x4 acc, f32x4 old) {
#pragma unroll
          for (int i = 0; i < 4; ++i) A2w[(m0 + 4 * g + i) * D + n0 + (lane & 15)] = old[i] + acc[i];
        },
        seg<NB>([&](int nn, int k) { return AQ[k * XM + nn]; },
                [&](int k, int j) { return DOq[k * YD + j]; }),
        seg<NB>([&](int nn, int k) { return A[k * XM + nn]; },
                [&](int k, int j) { return dOk[k * YD + j]; }),
        seg<NB>([&](int nn, int k) { return dU[k * XM + nn]; },
                [&](int k, int j) { return Go[k * YD + j]; }));
    for (int nn = opaque(tid); nn < M + D; nn += NT) {
      float sum = 0.f;
      if (nn < M) {
        // all 32 loads in flight before the sum (one round trip)
        float u[NB], w[NB];
#pragma unroll
        for (int s = 0; s < NB; ++s) {
          u[s] = dPQ[s * XM + nn];
          w[s] = dP[s * XM + nn];
        }
        const float prev = adj[OB1 + nn];
#pragma unroll
        for (int s = 0; s < NB; ++s) sum += u[s] + w[s];
        adj[OB1 + nn] = prev + sum;
      } else {
        const int j = nn - M;
        for (int s = 0; s < NB; ++s) sum += DOq[s * YD + j] + dOk[s * YD + j];
        adj[OB2 + j] += sum;
      }
    }
    __syncthreads();
  }

  // ---- the initial state's gradient (per batch: directly; shared: summed
  // over the batch by the second kernel from the workspace) and dgamma, dbeta
  if (a.state0_per_batch) {
    float* dst[4] = {a.dw1 + static_cast<size_t>(unit) * D * M, a.db1 + static_cast<size_t>(unit) * M,
                     a.dw2 + static_cast<size_t>(unit) * M * D, a.db2 + static_cast<size_t>(unit) * D};
    const int off[4] = {0, OB1, OW2, OB2}, len[4] = {D * M, M, M * D, D};
    for (int p = 0; p < 4; ++p)
      for (int i = tid; i < len[p]; i += NT) dst[p][i] = adj[off[p] + i];
  }
  {
    const int slot = 2 * wave + (lane >> 5), f = 2 * (lane & 31);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      L.dln[slot][0][f + u] = dg_acc[u];
      L.dln[slot][1][f + u] = db_acc[u];
    }
  }
  __syncthreads();
  for (int i = tid; i < 2 * D; i += NT) {   // slots summed in a fixed order
    float sum = 0.f;
    for (int sl = 0; sl < 16; ++sl) sum += L.dln[sl][i / D][i % D];
    dln_out[i] = sum;
  }
}

// Sums over the batch, one workgroup per head, in batch order
// (deterministic): the gradient of a shared initial state, dgamma, dbeta.
__global__ __launch_bounds__(256) void ttt_mlp_bwd_sum_k(MlpBackwardArgs a) {
  const int h = blockIdx.x;
  const int n = (a.T + 15) / 16;
  auto unit_ws = [&](int b) {
    return a.ws + static_cast<size_t>(b * a.H + h) * a.unit_floats;
  };
  if (!a.state0_per_batch) {
    float* dst[4] = {a.dw1 + static_cast<size_t>(h) * D * M, a.db1 + static_cast<size_t>(h) * M,
                     a.dw2 + static_cast<size_t>(h) * M * D, a.db2 + static_cast<size_t>(h) * D};
    const int off[4] = {0, OB1, OW2, OB2}, len[4] = {D * M, M, M * D, D};
    for (int p = 0; p < 4; ++p)
      for (int i = threadIdx.x; i < len[p]; i += 256) {
        float s = 0.f;
        for (int b = 0; b < a.B; ++b) s += unit_ws(b)[static_cast<size_t>(n) * SZ + off[p] + i];
        dst[p][i] = s;
      }
  }
  if (a.dgamma) {
    const size_t dln_off = a.unit_floats - 2 * D;
    for (int e = threadIdx.x; e < 2 * D; e += 256) {
      float s = 0.f;
      for (int b = 0; b < a.B; ++b) s += unit_ws(b)[dln_off + e];
      if (e < D)
        a.dgamma[h * D + e] = s;
      else
        a.dbeta[h * D + e - D] = s;
    }
  }
}

template <bool BF16, bool LN>
hipError_t launch_m2(const MlpBackwardArgs& a, bool res, hipStream_t s) {
  const dim3 grid(a.B * a.H), block(NT);
  if (res)
    hipLaunchKernelGGL((ttt_mlp_bwd_k<BF16, LN, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((ttt_mlp_bwd_k<BF16, LN, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mlp_backward(const MlpBackwardArgs& a, bool bf16, bool ln, bool residual,
                               hipStream_t stream) {
  hipError_t e;
  if (bf16)
    e = ln ? launch_m2<true, true>(a, residual, stream) : launch_m2<true, false>(a, residual, stream);
  else
    e = ln ? launch_m2<false, true>(a, residual, stream)
           : launch_m2<false, false>(a, residual, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ttt_mlp_bwd_sum_k, dim3(a.H), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tttk
