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
// id is remapped to give each XCD a contiguous run of tiles.  Within a run
// the tiles go by groups of 4 x row blocks (256 rows, 1 MB each at
// D = 2048), column by column inside a group: the 32 tiles an XCD works on
// at once then share 4 x blocks and 8 W_in tiles (8 MB) rather than one x
// block and 32 W_in tiles (17 MB), so W_in is streamed 4x less often
// (measured at B4 T8192, D = 2048: 0.90 -> 0.87 ms; groups of 2 or 8
// rows: 0.88 ms).
#include "ttt_device.hpp"
#include "ttt_input.hpp"

#define TTT_LDS __attribute__((address_space(3)))

namespace tttk {
namespace {

constexpr int BM = 256, BN = 128, BK = 64, NT = 512, LDK = BK, HD = 64, XCDS = 8, GM = 4;

struct InLds {
  uint16_t a[3][BM][LDK];
  uint16_t b[3][BN][LDK];
};

__device__ __forceinline__ float sigmoid(float y) { return 1.0f / (1.0f + expf(-y)); }

__global__ __launch_bounds__(NT) void ttt_input_k(InputArgs a) {
  __shared__ InLds L;
  const int M = a.B * a.T, N = 3 * a.H * HD + a.H, D = a.D;
  const int ntm = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN, nt = ntm * ntn;
  const int per = (nt + XCDS - 1) / XCDS;
  const int tile = (blockIdx.x % XCDS) * per + blockIdx.x / XCDS;
  if (tile >= nt) return;
  // groups of GM row blocks, their tiles column by column
  const int grp = tile / (GM * ntn), within = tile % (GM * ntn);
  const int gsize = min(GM, ntm - grp * GM);
  const int m0 = (grp * GM + within % gsize) * BM, n0 = (within / gsize) * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;

  // Copies go straight from memory into LDS (global_load_lds: no registers).
  // One wave instruction moves 1 KB: 8 rows of 128 bytes, lane l landing at
  // byte 16 l -- row l / 8, chunk l % 8 of the block -- so each lane fetches
  // the source chunk that belongs in that (swizzled) slot.  Per step the x
  // tile is 32 such blocks and the W_in tile 16; wave w copies x blocks
  // w + 8 j (j < 4) and W_in blocks w + 8 j (j < 2).
  const int cr = lane >> 3, cq = lane & 7;
  const uint16_t* xg = static_cast<const uint16_t*>(a.x);
  const uint16_t* wg = static_cast<const uint16_t*>(a.w);
  const uint16_t* pa[4];
  const uint16_t* pb[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 8 * (wave + 8 * j) + cr;   // row of the x tile
    pa[j] = xg + static_cast<size_t>(min(m0 + r, M - 1)) * D + 8 * (cq ^ (r & 7));
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 8 * (wave + 8 * j) + cr;   // row of the W_in tile
    pb[j] = wg + static_cast<size_t>(min(n0 + r, N - 1)) * D + 8 * (cq ^ (r & 7));
  }
  const int steps = D / BK;
  auto issue = [&](int buf, int step) {
    const int k0 = min(step, steps - 1) * BK;   // past the end: the last step again
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_global_load_lds(pa[j] + k0, (TTT_LDS void*)&L.a[buf][8 * (wave + 8 * j)][0],
                                       16, 0, 0);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_global_load_lds(pb[j] + k0, (TTT_LDS void*)&L.b[buf][8 * (wave + 8 * j)][0],
                                       16, 0, 0);
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
        af[i] = *reinterpret_cast<const u32x4*>(
            &L.a[buf][64 * wm + 16 * i + c][(32 * kk + 8 * g) ^ ((c & 7) << 3)]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const u32x4*>(
            &L.b[buf][64 * wn + 16 * j + c][(32 * kk + 8 * g) ^ ((c & 7) << 3)]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
    }
  };

  // Three LDS buffers: at step s the products read buffer s % 3 while the
  // copies of step s + 1 (issued a step ago) land and those of step s + 2 are
  // issued into the third.  Before the step's barrier each wave waits for its
  // own copies of step s + 1 only (six instructions issued after them may
  // still be in flight): the barrier's usual LDS fence would wait for all.
  issue(0, 0);
  issue(1, 1);
  asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  lds_barrier_copies_in_flight();
  int cur = 0;
  for (int s = 0; s < steps; ++s) {
    compute(cur);
    issue(cur == 0 ? 2 : cur - 1, s + 2);   // buffer (s + 2) % 3
    asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    lds_barrier_copies_in_flight();
    cur = cur == 2 ? 0 : cur + 1;
  }
  // the last copies (repeats of the last step) must land before the LDS is
  // reused below
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lds_barrier_copies_in_flight();

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
