// ttt_backward.hpp -- launch interface of the TTT-Linear backward scan
// (ttt_backward.hip).  Plain struct of device pointers and sizes; the host
// API has validated every field before the launcher is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tttk {

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
  int32_t B, H, T;
  float eps;
  int32_t state0_per_batch;
  int32_t bases_saved;      // the forward stored the bases already: no replay
};

// Two kernels on `stream`: the scan (one workgroup per unit) and the sums
// over the batch.  Returns the hipError_t of the launches.
hipError_t launch_linear_backward(const BackwardArgs& a, bool bf16, bool ln, bool residual,
                                  hipStream_t stream);

}  // namespace tttk
