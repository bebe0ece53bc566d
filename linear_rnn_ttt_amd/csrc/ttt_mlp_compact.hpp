// ttt_mlp_compact.hpp -- launch interface of the TTT-MLP streaming step with
// a compact pending state (ttt_mlp_decode_compact.hip).  Plain struct of
// device pointers and sizes; the host API has validated every field.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tttk {

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

hipError_t launch_mlp_decode_compact(const MlpCompactArgs& a, bool bf16, bool ln, bool residual,
                                     hipStream_t stream);

}  // namespace tttk
