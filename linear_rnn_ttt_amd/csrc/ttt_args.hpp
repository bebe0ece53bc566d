// ttt_args.hpp -- the launch arguments of every gfx950 kernel: plain structs
// of device pointers and sizes.  No HIP dependency: the host-side validation
// (ttt_validate.cpp) fills them and builds with a plain C++ compiler.
#pragma once

#include <stdint.h>

namespace tttk {

struct LinearArgs {
  const void* q;          // [B,H,T,64] bf16 or fp32
  const void* k;
  const void* v;
  const float* eta;       // [B,H,T]
  const float* w0;        // [H,64,64] or [B,H,64,64]
  const float* gamma;     // [H,64] (unused without LN)
  const float* beta;
  void* z;                // [B,H,T,64]
  float* w_out;           // [B,H,64,64] or nullptr
  int32_t B, H, T;
  int32_t tiles_per_mb;   // mini-batch size / 16
  float eps;
  int32_t state0_per_batch;
  // Two workgroups per unit (see ttt_linear.hip) when split != 0: the
  // gradient stream (6 KB per unit and 16-token tile) and the publication
  // counters [units][2][32] u32 (zeroed before the launch), followed by 32
  // u32 of error words.
  uint32_t* ws_g;
  uint32_t* ws_flags;
  int32_t split;
  // When set (mini-batch 16): the base of every tile, [units][tiles][64][64],
  // stored for the backward pass.
  float* bases;
};

struct MlpArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* eta;
  const float* w1;        // [H,64,256] or [B,H,64,256]
  const float* b1;        // [H,256]
  const float* w2;        // [H,256,64]
  const float* b2;        // [H,64]
  const float* gamma;
  const float* beta;
  void* z;
  float* w1_out;          // all four nullptr or all set
  float* b1_out;
  float* w2_out;
  float* b2_out;
  int32_t B, H, T;
  float eps;
  int32_t state0_per_batch;
};

// One token of the TTT-Linear scan per unit (ttt_decode.hip).
struct DecodeArgs {
  const void* q;          // [B,H,64] bf16 or fp32
  const void* k;
  const void* v;
  const float* eta;       // [B,H]
  float* w;               // [B,H,64,64] state, read and written
  float* w_base;          // [B,H,64,64] mini-batch base: read (pos > 0) or written (pos == 0)
  const float* gamma;     // [H,64] (unused without LN)
  const float* beta;
  void* z;                // [B,H,64]
  int32_t B, H;
  int32_t pos;            // position of the token in its mini-batch
  float eps;
};

struct CompactArgs {
  const void* q;          // [B,H,64] bf16 or fp32
  const void* k;
  const void* v;
  const float* eta;       // [B,H]
  float* w_base;          // [B,H,64,64] the mini-batch's base, read (and written at pos 0)
  float* hist;            // [B,H,mb,2,64]: slot s holds k_s and u_s = -eta_s g_s
  const float* gamma;     // [H,64] (unused without LN)
  const float* beta;
  void* z;                // [B,H,64]
  int32_t B, H;
  int32_t pos;            // position of the token in its mini-batch
  int32_t mb;             // mini-batch size (history slots), at most 64
  float eps;
};

struct MlpDecodeArgs {
  const void* q;          // [B,H,64] bf16 or fp32
  const void* k;
  const void* v;
  const float* eta;       // [B,H]
  float* w1;              // [B,H,64,256] state, read and written
  float* b1;              // [B,H,256]
  float* w2;              // [B,H,256,64]
  float* b2;              // [B,H,64]
  float* w1_base;         // the mini-batch base, same shapes: read (pos > 0)
  float* b1_base;         // or written (pos == 0)
  float* w2_base;
  float* b2_base;
  const float* gamma;     // [H,64] (unused without LN)
  const float* beta;
  void* z;                // [B,H,64]
  int32_t B, H;
  int32_t pos;            // position of the token in its mini-batch
  float eps;
};

// Floats per (unit, 16-token tile) record of the backward's front half:
// x, G, DO [16][64] each, rho, mean(a), mean(a x) [16] each, the two masked
// Gram fragments [64 lanes][4] each, and the tile's dgamma, dbeta partials
// [2][64]; padded to a multiple of 256 bytes.
constexpr int kBwdRecFloats = 3776;

struct BackwardArgs {
  const void* q;            // [B,H,T,64] bf16 or fp32
  const void* k;
  const void* v;
  const float* eta;         // [B,H,T]
  const float* w0;          // [H,64,64] or [B,H,64,64]
  const float* gamma;       // [H,64] (unused without LN)
  const float* beta;
  const void* dz;           // [B,H,T,64], like q
  const float* dw_final;    // [B,H,64,64] or nullptr (zero)
  void* dq;                 // [B,H,T,64], like q
  void* dk;
  void* dv;
  float* deta;              // [B,H,T]
  float* dw0;               // like w0
  float* dgamma;            // [H,64] or nullptr (no LN)
  float* dbeta;
  // workspace: the base of every 16-token mini-batch of every unit
  // [units][tiles][64][64], the per-unit dW0 [units][64][64] (not used with a
  // per-batch initial state, whose dW0 is written in place), and the per-unit
  // LN parameter gradients [units][2][64]
  float* ws_base;
  float* ws_dw0;
  float* ws_dln;
  // 16-token mini-batches: the per-tile records of the adjoint-free front
  // half [units][tiles][kBwdRecFloats] (nullptr otherwise)
  float* ws_front;
  int32_t B, H, T;
  int32_t tiles_per_mb;     // mini-batch / 16
  float eps;
  int32_t state0_per_batch;
  int32_t bases_saved;      // the forward stored the bases already: no replay
};

struct MlpCompactArgs {
  const void* q;          // [B,H,64] bf16 or fp32
  const void* k;
  const void* v;
  const float* eta;       // [B,H]
  float* w1_base;         // [B,H,64,256] the mini-batch's base: read, and
  float* b1_base;         // [B,H,256]    written at pos 0 (after the fold)
  float* w2_base;         // [B,H,256,64]
  float* b2_base;         // [B,H,64]
  float* hist;            // [B,H,mb,640]: slot s holds k_s[64], u1_s[256], a_s[256], u2_s[64]
  const float* gamma;     // [H,64] (unused without LN)
  const float* beta;
  void* z;                // [B,H,64]
  int32_t B, H;
  int32_t pos;            // position of the token in its mini-batch
  int32_t mb;             // mini-batch size (history slots), at most 16
  float eps;
};

// Backward of the TTT-MLP scan (ttt_mlp_backward.hip).
struct MlpBackwardArgs {
  const void* q;            // [B,H,T,64] bf16 or fp32
  const void* k;
  const void* v;
  const float* eta;         // [B,H,T]
  const float* w1;          // initial state [H,64,256] / [H,256] / [H,256,64] / [H,64]
  const float* b1;          //   (leading [B,H] with state0_per_batch)
  const float* w2;
  const float* b2;
  const float* gamma;       // [H,64] (unused without LN)
  const float* beta;
  const void* dz;           // [B,H,T,64], like q
  const float* dw1_final;   // cotangent of the final state [B,H,...], all four or none
  const float* db1_final;
  const float* dw2_final;
  const float* db2_final;
  void* dq;                 // [B,H,T,64], like q
  void* dk;
  void* dv;
  float* deta;              // [B,H,T]
  float* dw1;               // like the initial state (summed over the batch when shared)
  float* db1;
  float* dw2;
  float* db2;
  float* dgamma;            // [H,64] or nullptr (no LN)
  float* dbeta;
  // workspace: per unit, unit_floats floats: the base of every 16-token
  // mini-batch (MLP_BWD_STATE_FLOATS each), the adjoint state, per-tile
  // intermediates (MLP_BWD_TILE_FLOATS) ending in the unit's dgamma, dbeta
  float* ws;
  uint64_t unit_floats;
  int32_t B, H, T;
  float eps;
  int32_t state0_per_batch;
};

// Floats of one TTT-MLP state (W1 64x256, b1 256, W2 256x64, b2 64) and of
// the backward's per-tile intermediates of one unit kept in the workspace
// (three 16x256 ones, rows padded to 260 floats; the rest live in LDS).
constexpr uint64_t MLP_BWD_STATE_FLOATS = 64 * 256 + 256 + 256 * 64 + 64;
constexpr uint64_t MLP_BWD_TILE_FLOATS = 3 * 16 * 260 + 2 * 64;

// The input side (ttt_input_projection): Y = x W_in^T, then per column the
// q/k/v store or the learning-rate gate.
struct InputArgs {
  const void* x;          // [M = B T, D] bf16
  const void* w;          // [N = 3 H 64 + H, D] bf16
  const float* b_eta;     // [H]
  void* q;                // [B, H, T, 64] bf16
  void* k;
  void* v;
  float* eta;             // [B, H, T]
  int32_t B, T, D, H;
  float eta_base;
};

}  // namespace tttk

