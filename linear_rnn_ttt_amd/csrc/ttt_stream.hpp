// ttt_stream.hpp -- launch interfaces of the streaming steps: TTT-Linear
// with a compact pending state (ttt_decode_compact.hip) and TTT-MLP
// (ttt_mlp_decode.hip).  Plain structs of device pointers and sizes; the
// host API has validated every field.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tttk {

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

hipError_t launch_linear_decode_compact(const CompactArgs& a, bool bf16, bool ln, bool residual,
                                        hipStream_t stream);

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

hipError_t launch_mlp_decode(const MlpDecodeArgs& a, bool bf16, bool ln, bool residual,
                             hipStream_t stream);

}  // namespace tttk
