// ttt_input.hip -- the input side of a TTT layer for gfx950: q, k and v of
// every head and the token-dependent learning rate, made from the layer
// input in one bf16 matrix-unit product with a per-column epilogue.
//
// The outer loop trains the projections theta_Q, theta_K, theta_V that turn
// the layer input into the inner loop's queries, keys and values, and a
// learning rate that depends on the token (dmarx.github.io record LIT-801,
// "Key takeaways" item 2; the QKV projection matrices of the nowfound.app
// launch page, "In the maker's words").  With x [M = B T, D] and the stacked
// weights W_in [N = 3 H 64 + H, D] (both bf16, D contiguous):
//     Y = x W_in^T                      (fp32 accumulation)
//     column n < 3 H 64: feature n % 64 of head (n / 64) % H of q, k or v
//         (n / (64 H)), stored bf16 (round to nearest even) into [B, H, T, 64];
//     column 3 H 64 + h: the gate of head h,
//         eta = eta_base / (1 + exp(-(y + b_eta[h]))), stored fp32 into [B, H, T].
//
// Tiling: a 256 x 128 output tile per workgroup, 512 threads as 8 waves in
// a 4 x 2 grid, each wave 64 x 64 (4 x 4 accumulators of 16 x 16, fp32).
// D is walked in steps of 64 through two LDS buffers; while the matrix unit
// works on one step, the next step's tiles wait in registers to be written
// to the other buffer and the one after is on its way from memory
// (16-byte loads, 8 lanes per 128-byte row segment): one barrier per step.  In
// LDS the 16-byte chunk q of row r sits at chunk q ^ (r % 8), so the rows a
// fragment read touches spread over the banks (measured 6-12 % faster than
// padding the rows to 72 or 80 bf16, and no padding bytes).  Operands are 16x16x32 bf16 fragments: lane
// (g, c) reads 8 consecutive k of row c -- the same k slots for A (x) and B
// (W_in), which is all the product needs.  Rows past M and weight rows
// past N are clamped on load (valid memory, results unused) and dropped
// on store.
//
// Tile order: consecutive workgroup ids land on the 8 XCDs in turn, so the
// id is remapped to give each XCD a contiguous run of tiles; within a run
// the N tiles of one x row block come one after another, so that block
// (256 rows, 1 MB at D = 2048) is read from HBM once per XCD and then from
// its L2.
#include "ttt_device.hpp"
#include "ttt_input.hpp"

namespace tttk {
namespace {

constexpr int BM = 256, BN = 128, BK = 64, NT = 512, LDK = BK, HD = 64, XCDS = 8;

struct InLds {
  uint16_t a[2][BM][LDK];
  uint16_t b[2][BN][LDK];
};

__device__ __forceinline__ float sigmoid(float y) { return 1.0f / (1.0f + expf(-y)); }

__global__ __launch_bounds__(NT) void ttt_input_k(InputArgs a) {
  __shared__ InLds L;
  const int M = a.B * a.T, N = 3 * a.H * HD + a.H, D = a.D;
  const int ntm = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN, nt = ntm * ntn;
  const int per = (nt + XCDS - 1) / XCDS;
  const int tile = (blockIdx.x % XCDS) * per + blockIdx.x / XCDS;
  if (tile >= nt) return;
  const int m0 = (tile / ntn) * BM, n0 = (tile % ntn) * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;

  // this thread's 16-byte pieces of a step: x rows lr + 64 j (j < 4) and
  // W_in rows lr + 64 j (j < 2), k offset lk within the step
  const int lr = tid >> 3, lk = (tid & 7) * 8;
  const uint16_t* xg = static_cast<const uint16_t*>(a.x);
  const uint16_t* wg = static_cast<const uint16_t*>(a.w);
  const uint16_t* pa[4];
  const uint16_t* pb[2];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    pa[j] = xg + static_cast<size_t>(min(m0 + lr + 64 * j, M - 1)) * D + lk;
#pragma unroll
  for (int j = 0; j < 2; ++j)
    pb[j] = wg + static_cast<size_t>(min(n0 + lr + 64 * j, N - 1)) * D + lk;
  const int steps = D / BK;
  // two register sets of staged pieces: a step's tiles are loaded two steps
  // before they are written to LDS, so a load has two steps of products to
  // arrive in (one step is shorter than a memory round trip)
  struct Stage {
    u32x4 a[4], b[2];
  };
  auto gload = [&](Stage& r, int step) {
    const int k0 = min(step, steps - 1) * BK;   // past the end: the last step again
#pragma unroll
    for (int j = 0; j < 4; ++j) r.a[j] = *reinterpret_cast<const u32x4*>(pa[j] + k0);
#pragma unroll
    for (int j = 0; j < 2; ++j) r.b[j] = *reinterpret_cast<const u32x4*>(pb[j] + k0);
  };
  auto lstore = [&](int buf, const Stage& r) {
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4*>(&L.a[buf][lr + 64 * j][lk ^ ((lr & 7) << 3)]) = r.a[j];
#pragma unroll
    for (int j = 0; j < 2; ++j) *reinterpret_cast<u32x4*>(&L.b[buf][lr + 64 * j][lk ^ ((lr & 7) << 3)]) = r.b[j];
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      u32x4 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(&L.a[buf][64 * wm + 16 * i + c][(32 * kk + 8 * g) ^ ((c & 7) << 3)]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const u32x4*>(&L.b[buf][64 * wn + 16 * j + c][(32 * kk + 8 * g) ^ ((c & 7) << 3)]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
    }
  };

  // step s: multiply LDS buffer s % 2; write step s + 1 (loaded at step
  // s - 1) to the other buffer; load step s + 3 into the freed set.  Two
  // steps per iteration so the register sets are named statically.
  Stage r0, r1;
  gload(r0, 0);
  gload(r1, 1);
  lstore(0, r0);
  gload(r0, 2);
  lds_barrier();
  for (int s = 0; s < steps; s += 2) {
    compute(0);
    lstore(1, r1);
    gload(r1, s + 3);
    lds_barrier();
    if (s + 1 < steps) compute(1);
    lstore(0, r0);
    gload(r0, s + 4);
    lds_barrier();
  }

  // epilogue: accumulator (i, j) holds Y[m0 + 64 wm + 16 i + 4 g + r][n0 + 64 wn + 16 j + c].
  // A wave's 64 columns are one head of q, k or v (3 H 64 is a multiple of
  // 64), i.e. 64 whole 128-byte output rows: they are staged through the
  // wave's own LDS region (free after the last barrier; chunks swizzled as in
  // the loop) and stored 16 bytes per lane, 8 lanes per row.  The gate columns go out one value per lane.
  const int T = a.T, H = a.H, QKV = 3 * H * HD;
  const int nb0 = n0 + 64 * wn;
  if (nb0 < QKV) {
    uint16_t (*W)[LDK] = reinterpret_cast<uint16_t (*)[LDK]>(&L.a[0][0][0]) + 64 * wave;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          W[16 * i + 4 * g + r][(16 * j + c) ^ (((4 * g + r) & 7) << 3)] =
              static_cast<uint16_t>(pack_bf16(acc[i][j][r], 0.f) & 0xffffu);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's own rows, in order
    const int which = nb0 / (H * HD), h = (nb0 / HD) % H;
    uint16_t* out = which == 0 ? static_cast<uint16_t*>(a.q)
                               : which == 1 ? static_cast<uint16_t*>(a.k)
                                            : static_cast<uint16_t*>(a.v);
    const int col = 8 * (lane & 7);
#pragma unroll
    for (int pass = 0; pass < 8; ++pass) {
      const int row = (lane >> 3) + 8 * pass;
      const int m = m0 + 64 * wm + row;
      const u32x4 val = *reinterpret_cast<const u32x4*>(&W[row][col ^ ((row & 7) << 3)]);
      if (m < M) {
        const int b = m / T, t = m - b * T;
        *reinterpret_cast<u32x4*>(out + ((static_cast<size_t>(b) * H + h) * T + t) * HD + col) =
            val;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 64 * wm + 16 * i + 4 * g + r;
        if (m >= M) continue;
        const int b = m / T, t = m - b * T;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int h = nb0 + 16 * j + c - QKV;
          if (h < H)
            a.eta[(static_cast<size_t>(b) * H + h) * T + t] =
                a.eta_base * sigmoid(acc[i][j][r] + a.b_eta[h]);
        }
      }
  }
}

}  // namespace

uint32_t input_grid(const InputArgs& a) {
  const int64_t M = static_cast<int64_t>(a.B) * a.T, N = 3 * a.H * HD + a.H;
  const int64_t nt = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  return static_cast<uint32_t>((nt + XCDS - 1) / XCDS * XCDS);
}

hipError_t launch_input(const InputArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(ttt_input_k, dim3(input_grid(a)), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tttk
