// ttt_api.cpp -- C ABI entry points (include/ttt.h): each validates its
// arguments on the host (ttt_validate.cpp: no HIP call, so argument errors
// are reported the same way with or without a GPU) and then launches the
// gfx950 kernels on the caller's stream.
#include "ttt.h"

#include <hip/hip_runtime.h>

#include <cstdint>

#include "ttt_backward.hpp"
#include "ttt_input.hpp"
#include "ttt_kernels.hpp"
#include "ttt_mlp_backward.hpp"
#include "ttt_mlp_compact.hpp"
#include "ttt_stream.hpp"
#include "ttt_validate.hpp"

namespace {

ttt_status status_of(hipError_t e) { return e == hipSuccess ? TTT_OK : TTT_ERR_DEVICE; }

bool ln_of(const ttt_params* p) { return !(p->flags & TTT_NO_LN); }
bool res_of(const ttt_params* p) { return !(p->flags & TTT_NO_RESIDUAL); }
bool bf16_of(const ttt_params* p) { return p->io_dtype == TTT_BF16; }

ttt_status linear_launch(const ttt_params* p, const tttk::LinearArgs& a, void* hip_stream) {
  return status_of(tttk::launch_linear(a, bf16_of(p), ln_of(p), res_of(p),
                                       static_cast<hipStream_t>(hip_stream)));
}

// The split launch needs both workgroups of every unit resident at once:
// at most half the device's compute units' worth of units.
ttt_status check_split_units(const ttt_params* p) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return TTT_ERR_DEVICE;
  if (2ull * static_cast<uint64_t>(p->B) * p->H > static_cast<uint64_t>(cus))
    return TTT_ERR_UNSUPPORTED;
  return TTT_OK;
}

}  // namespace

extern "C" {

const char* ttt_status_string(ttt_status s) {
  switch (s) {
    case TTT_OK: return "ok";
    case TTT_ERR_NULL: return "a required pointer is NULL";
    case TTT_ERR_SHAPE:
      return "B, H, T, d, mini_batch or hidden out of range, or the workspace is too small";
    case TTT_ERR_UNSUPPORTED:
      return "configuration not built for gfx950 (needs d = 64; Linear: mini_batch a multiple "
             "of 16; MLP: hidden = 256, mini_batch = 16; split Linear: 2*B*H at most the "
             "compute units)";
    case TTT_ERR_ALIAS: return "an output buffer or workspace overlaps another argument";
    case TTT_ERR_DEVICE: return "HIP reported an error at kernel launch";
    case TTT_ERR_ARG:
      return "bad io_dtype, flags, ln_eps or state0_per_batch, or a misaligned workspace";
    case TTT_ERR_TOO_LARGE:
      return "the problem needs more scratch than the no-allocation entry point's fixed array "
             "(TTT_NOALLOC_SCRATCH_BYTES per device) holds";
  }
  return "unknown ttt_status";
}

int32_t ttt_abi_version(void) { return TTT_ABI_VERSION; }

ttt_status ttt_linear_forward(const ttt_params* p, const void* q, const void* k, const void* v,
                              const float* eta, const float* w0, const float* ln_gamma,
                              const float* ln_beta, void* z, float* w_out, void* hip_stream) {
  tttk::LinearArgs a;
  const ttt_status st = tttv::linear_forward(p, q, k, v, eta, w0, ln_gamma, ln_beta, z, w_out,
                                             nullptr, 0, &a);
  if (st != TTT_OK) return st;
  return linear_launch(p, a, hip_stream);
}

uint64_t ttt_linear_split_workspace_bytes(const ttt_params* p) {
  uint64_t elems = 0;
  if (tttv::check_common(p, &elems) != TTT_OK) return 0;
  return tttv::split_layout(p).total;
}

ttt_status ttt_linear_forward_split(const ttt_params* p, const void* q, const void* k,
                                    const void* v, const float* eta, const float* w0,
                                    const float* ln_gamma, const float* ln_beta, void* z,
                                    float* w_out, void* workspace, uint64_t workspace_bytes,
                                    void* hip_stream) {
  tttk::LinearArgs a;
  ttt_status st = tttv::linear_split(p, q, k, v, eta, w0, ln_gamma, ln_beta, z, w_out,
                                     workspace, workspace_bytes, &a);
  if (st != TTT_OK) return st;
  if ((st = check_split_units(p)) != TTT_OK) return st;
  return linear_launch(p, a, hip_stream);
}

ttt_status ttt_linear_forward_split_noalloc(const ttt_params* p, const void* q, const void* k,
                                            const void* v, const float* eta, const float* w0,
                                            const float* ln_gamma, const float* ln_beta,
                                            void* z, float* w_out, void* hip_stream) {
  static_assert(TTT_NOALLOC_SCRATCH_BYTES == 128ull << 20, "header and library disagree");
  tttk::LinearArgs a;
  ttt_status st = tttv::linear_split_noalloc(p, q, k, v, eta, w0, ln_gamma, ln_beta, z, w_out,
                                             tttk::kLinearScratchBytes, &a);
  if (st != TTT_OK) return st;
  if ((st = check_split_units(p)) != TTT_OK) return st;
  void* scratch = nullptr;
  if (tttk::linear_scratch(&scratch) != hipSuccess) return TTT_ERR_DEVICE;
  tttv::set_split_workspace(p, scratch, &a);
  return linear_launch(p, a, hip_stream);
}

ttt_status ttt_linear_decode_step(const ttt_params* p, int32_t pos, const void* q,
                                  const void* k, const void* v, const float* eta, float* w,
                                  float* w_base, const float* ln_gamma, const float* ln_beta,
                                  void* z, void* hip_stream) {
  tttk::DecodeArgs a;
  const ttt_status st = tttv::linear_decode(p, pos, q, k, v, eta, w, w_base, ln_gamma, ln_beta,
                                            z, &a);
  if (st != TTT_OK) return st;
  return status_of(tttk::launch_linear_decode(a, bf16_of(p), ln_of(p), res_of(p),
                                              static_cast<hipStream_t>(hip_stream)));
}

ttt_status ttt_linear_decode_step_compact(const ttt_params* p, int32_t pos, const void* q,
                                          const void* k, const void* v, const float* eta,
                                          float* w_base, float* hist, const float* ln_gamma,
                                          const float* ln_beta, void* z, void* hip_stream) {
  tttk::CompactArgs a;
  const ttt_status st = tttv::linear_decode_compact(p, pos, q, k, v, eta, w_base, hist,
                                                    ln_gamma, ln_beta, z, &a);
  if (st != TTT_OK) return st;
  return status_of(tttk::launch_linear_decode_compact(a, bf16_of(p), ln_of(p), res_of(p),
                                                      static_cast<hipStream_t>(hip_stream)));
}

ttt_status ttt_mlp_decode_step(const ttt_params* p, int32_t hidden, int32_t pos, const void* q,
                               const void* k, const void* v, const float* eta, float* w1,
                               float* b1, float* w2, float* b2, float* w1_base, float* b1_base,
                               float* w2_base, float* b2_base, const float* ln_gamma,
                               const float* ln_beta, void* z, void* hip_stream) {
  tttk::MlpDecodeArgs a;
  const ttt_status st = tttv::mlp_decode(p, hidden, pos, q, k, v, eta, w1, b1, w2, b2, w1_base,
                                         b1_base, w2_base, b2_base, ln_gamma, ln_beta, z, &a);
  if (st != TTT_OK) return st;
  return status_of(tttk::launch_mlp_decode(a, bf16_of(p), ln_of(p), res_of(p),
                                           static_cast<hipStream_t>(hip_stream)));
}

ttt_status ttt_mlp_decode_step_compact(const ttt_params* p, int32_t hidden, int32_t pos,
                                       const void* q, const void* k, const void* v,
                                       const float* eta, float* w1_base, float* b1_base,
                                       float* w2_base, float* b2_base, float* hist,
                                       const float* ln_gamma, const float* ln_beta, void* z,
                                       void* hip_stream) {
  tttk::MlpCompactArgs a;
  const ttt_status st = tttv::mlp_decode_compact(p, hidden, pos, q, k, v, eta, w1_base,
                                                 b1_base, w2_base, b2_base, hist, ln_gamma,
                                                 ln_beta, z, &a);
  if (st != TTT_OK) return st;
  return status_of(tttk::launch_mlp_decode_compact(a, bf16_of(p), ln_of(p), res_of(p),
                                                   static_cast<hipStream_t>(hip_stream)));
}

ttt_status ttt_linear_forward_save(const ttt_params* p, const void* q, const void* k,
                                   const void* v, const float* eta, const float* w0,
                                   const float* ln_gamma, const float* ln_beta, void* z,
                                   float* w_out, void* workspace, uint64_t workspace_bytes,
                                   void* hip_stream) {
  tttk::LinearArgs a;
  const ttt_status st = tttv::linear_forward_save(p, q, k, v, eta, w0, ln_gamma, ln_beta, z,
                                                  w_out, workspace, workspace_bytes, &a);
  if (st != TTT_OK) return st;
  return linear_launch(p, a, hip_stream);
}

uint64_t ttt_linear_backward_workspace_bytes(const ttt_params* p) {
  uint64_t elems = 0;
  if (tttv::check_common(p, &elems) != TTT_OK) return 0;
  return tttv::backward_layout(p).total;
}

ttt_status ttt_linear_backward(const ttt_params* p, const void* q, const void* k, const void* v,
                               const float* eta, const float* w0, const float* ln_gamma,
                               const float* ln_beta, const void* dz, const float* dw_final,
                               void* dq, void* dk, void* dv, float* deta, float* dw0,
                               float* dln_gamma, float* dln_beta, void* workspace,
                               uint64_t workspace_bytes, void* hip_stream) {
  tttk::BackwardArgs a;
  const ttt_status st = tttv::linear_backward(p, q, k, v, eta, w0, ln_gamma, ln_beta, dz,
                                              dw_final, dq, dk, dv, deta, dw0, dln_gamma,
                                              dln_beta, workspace, workspace_bytes, &a);
  if (st != TTT_OK) return st;
  if (p->mini_batch == 16 && !(p->flags & TTT_BASES_SAVED)) {
    // the bases from the forward kernel, which holds each one anyway (faster
    // than the backward's own replay); the walk then reads them as saved
    tttk::LinearArgs la;
    const ttt_status sf = tttv::linear_forward_bases(p, q, k, v, eta, w0, ln_gamma, ln_beta,
                                                     workspace, &la);
    if (sf != TTT_OK) return sf;
    const ttt_status sl = linear_launch(p, la, hip_stream);
    if (sl != TTT_OK) return sl;
    a.bases_saved = 1;
  }
  return status_of(tttk::launch_linear_backward(a, bf16_of(p), ln_of(p), res_of(p),
                                                static_cast<hipStream_t>(hip_stream)));
}

ttt_status ttt_mlp_forward(const ttt_params* p, int32_t hidden, const void* q, const void* k,
                           const void* v, const float* eta, const float* w1_0, const float* b1_0,
                           const float* w2_0, const float* b2_0, const float* ln_gamma,
                           const float* ln_beta, void* z, float* w1_out, float* b1_out,
                           float* w2_out, float* b2_out, void* hip_stream) {
  tttk::MlpArgs a;
  const ttt_status st = tttv::mlp_forward(p, hidden, q, k, v, eta, w1_0, b1_0, w2_0, b2_0,
                                          ln_gamma, ln_beta, z, w1_out, b1_out, w2_out, b2_out,
                                          &a);
  if (st != TTT_OK) return st;
  return status_of(tttk::launch_mlp(a, bf16_of(p), ln_of(p), res_of(p),
                                    static_cast<hipStream_t>(hip_stream)));
}

uint64_t ttt_mlp_backward_workspace_bytes(const ttt_params* p, int32_t hidden) {
  uint64_t elems = 0;
  if (tttv::check_common(p, &elems) != TTT_OK || hidden != 256) return 0;
  return tttv::mlp_backward_workspace_bytes(p);
}

ttt_status ttt_mlp_backward(const ttt_params* p, int32_t hidden, const void* q, const void* k,
                            const void* v, const float* eta, const float* w1_0,
                            const float* b1_0, const float* w2_0, const float* b2_0,
                            const float* ln_gamma, const float* ln_beta, const void* dz,
                            const float* dw1_final, const float* db1_final,
                            const float* dw2_final, const float* db2_final, void* dq, void* dk,
                            void* dv, float* deta, float* dw1, float* db1, float* dw2,
                            float* db2, float* dln_gamma, float* dln_beta, void* workspace,
                            uint64_t workspace_bytes, void* hip_stream) {
  tttk::MlpBackwardArgs a;
  const ttt_status st = tttv::mlp_backward(
      p, hidden, q, k, v, eta, w1_0, b1_0, w2_0, b2_0, ln_gamma, ln_beta, dz, dw1_final,
      db1_final, dw2_final, db2_final, dq, dk, dv, deta, dw1, db1, dw2, db2, dln_gamma, dln_beta,
      workspace, workspace_bytes, &a);
  if (st != TTT_OK) return st;
  return status_of(tttk::launch_mlp_backward(a, bf16_of(p), ln_of(p), res_of(p),
                                             static_cast<hipStream_t>(hip_stream)));
}

ttt_status ttt_input_projection(const ttt_params* p, int32_t d_model, const void* x,
                                const void* w_in, const float* b_eta, float eta_base, void* q,
                                void* k, void* v, float* eta, void* hip_stream) {
  tttk::InputArgs a;
  const ttt_status st =
      tttv::input_projection(p, d_model, x, w_in, b_eta, eta_base, q, k, v, eta, &a);
  if (st != TTT_OK) return st;
  return status_of(tttk::launch_input(a, static_cast<hipStream_t>(hip_stream)));
}

}  // extern "C"
