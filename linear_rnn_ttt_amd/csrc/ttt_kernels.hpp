// ttt_kernels.hpp -- launch interface between the host API (ttt_api.cpp) and
// the gfx950 kernels.  Plain structs of device pointers and sizes; the host
// API has validated every field before a launcher is called.
#pragma once

#include <hip/hip_runtime.h>
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
  // gradient stream [units][T/16 tiles][4][64] x 16 B and the publication
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

// Device address of the fixed scratch array of the no-allocation split
// launch on the current device (looked up once per device), and its size.
hipError_t linear_scratch(void** ptr);
extern const uint64_t kLinearScratchBytes;

// Each returns the hipError_t of the launch.
hipError_t launch_linear(const LinearArgs& a, bool bf16, bool ln, bool residual,
                         hipStream_t stream);
hipError_t launch_mlp(const MlpArgs& a, bool bf16, bool ln, bool residual,
                      hipStream_t stream);
hipError_t launch_linear_decode(const DecodeArgs& a, bool bf16, bool ln, bool residual,
                                hipStream_t stream);

}  // namespace tttk
