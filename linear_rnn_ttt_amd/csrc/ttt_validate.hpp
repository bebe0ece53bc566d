// ttt_validate.hpp -- host-side argument checks of the C ABI (include/ttt.h):
// every check an entry point makes before it launches anything, and the fill
// of the kernels' launch arguments.  No HIP dependency: ttt_validate.cpp
// builds with a plain C++ compiler (and so with the host sanitizers).  Each
// function returns TTT_OK and fills *a, or the status of the first failed
// check with *a unspecified.
#pragma once

#include <stdint.h>

#include "ttt.h"
#include "ttt_args.hpp"

namespace tttv {

// Shared shape / flag checks.  *elems receives B*H*T*d.
ttt_status check_common(const ttt_params* p, uint64_t* elems);

// Workspace of a split Linear launch: publication counters (two 128-byte
// lines per unit), 32 error words, then the gradient stream (6 KB per
// 16-token tile and unit).
struct SplitLayout {
  uint64_t stream_offset, total;
};
SplitLayout split_layout(const ttt_params* p);

// Workspace of the backward scan: every mini-batch base of every unit
// (16 KB per 16-token tile and unit), the per-unit dW0 (16 KB per unit) and
// the per-unit LN parameter gradients (512 B per unit).
struct BackwardLayout {
  uint64_t dw0_offset, dln_offset, front_offset, total;
};
BackwardLayout backward_layout(const ttt_params* p);

// ttt_linear_forward.  A non-null workspace (split launch) is checked for
// size, alignment and overlap; the workspace fields of *a stay unset.
ttt_status linear_forward(const ttt_params* p, const void* q, const void* k, const void* v,
                          const float* eta, const float* w0, const float* ln_gamma,
                          const float* ln_beta, void* z, float* w_out, void* workspace,
                          uint64_t workspace_bytes, tttk::LinearArgs* a);

// ttt_linear_forward_split: as linear_forward with a required workspace,
// no in-place resume, and the workspace fields of *a set (split = 1).  The
// unit-count limit (half the device's compute units) is the caller's check.
ttt_status linear_split(const ttt_params* p, const void* q, const void* k, const void* v,
                        const float* eta, const float* w0, const float* ln_gamma,
                        const float* ln_beta, void* z, float* w_out, void* workspace,
                        uint64_t workspace_bytes, tttk::LinearArgs* a);

// ttt_linear_forward_split_noalloc up to the scratch lookup: the arguments
// of the split launch without a workspace, then the problem's scratch need
// against scratch_bytes (TTT_ERR_TOO_LARGE).  The workspace fields of *a
// stay unset.
ttt_status linear_split_noalloc(const ttt_params* p, const void* q, const void* k,
                                const void* v, const float* eta, const float* w0,
                                const float* ln_gamma, const float* ln_beta, void* z,
                                float* w_out, uint64_t scratch_bytes, tttk::LinearArgs* a);

// The workspace fields of a split launch at `workspace` (split_layout).
void set_split_workspace(const ttt_params* p, void* workspace, tttk::LinearArgs* a);

// ttt_linear_backward with 16-token mini-batches and no saved bases: the
// forward in its base-saving form with no z and no final state, storing the
// bases into the backward's (already validated) workspace.
ttt_status linear_forward_bases(const ttt_params* p, const void* q, const void* k,
                                const void* v, const float* eta, const float* w0,
                                const float* ln_gamma, const float* ln_beta, void* workspace,
                                tttk::LinearArgs* a);

// ttt_linear_forward_save.
ttt_status linear_forward_save(const ttt_params* p, const void* q, const void* k,
                               const void* v, const float* eta, const float* w0,
                               const float* ln_gamma, const float* ln_beta, void* z,
                               float* w_out, void* workspace, uint64_t workspace_bytes,
                               tttk::LinearArgs* a);

// ttt_linear_decode_step.
ttt_status linear_decode(const ttt_params* p, int32_t pos, const void* q, const void* k,
                         const void* v, const float* eta, float* w, float* w_base,
                         const float* ln_gamma, const float* ln_beta, void* z,
                         tttk::DecodeArgs* a);

// ttt_linear_decode_step_compact.
ttt_status linear_decode_compact(const ttt_params* p, int32_t pos, const void* q,
                                 const void* k, const void* v, const float* eta, float* w_base,
                                 float* hist, const float* ln_gamma, const float* ln_beta,
                                 void* z, tttk::CompactArgs* a);

// ttt_mlp_decode_step.
ttt_status mlp_decode(const ttt_params* p, int32_t hidden, int32_t pos, const void* q,
                      const void* k, const void* v, const float* eta, float* w1, float* b1,
                      float* w2, float* b2, float* w1_base, float* b1_base, float* w2_base,
                      float* b2_base, const float* ln_gamma, const float* ln_beta, void* z,
                      tttk::MlpDecodeArgs* a);

// ttt_mlp_decode_step_compact.
ttt_status mlp_decode_compact(const ttt_params* p, int32_t hidden, int32_t pos, const void* q,
                              const void* k, const void* v, const float* eta, float* w1_base,
                              float* b1_base, float* w2_base, float* b2_base, float* hist,
                              const float* ln_gamma, const float* ln_beta, void* z,
                              tttk::MlpCompactArgs* a);

// ttt_linear_backward (p->flags may carry TTT_BASES_SAVED).
ttt_status linear_backward(const ttt_params* p, const void* q, const void* k, const void* v,
                           const float* eta, const float* w0, const float* ln_gamma,
                           const float* ln_beta, const void* dz, const float* dw_final,
                           void* dq, void* dk, void* dv, float* deta, float* dw0,
                           float* dln_gamma, float* dln_beta, void* workspace,
                           uint64_t workspace_bytes, tttk::BackwardArgs* a);

// ttt_mlp_forward.
ttt_status mlp_forward(const ttt_params* p, int32_t hidden, const void* q, const void* k,
                       const void* v, const float* eta, const float* w1_0, const float* b1_0,
                       const float* w2_0, const float* b2_0, const float* ln_gamma,
                       const float* ln_beta, void* z, float* w1_out, float* b1_out,
                       float* w2_out, float* b2_out, tttk::MlpArgs* a);

// Workspace of the TTT-MLP backward: per unit, the base of every 16-token
// mini-batch, the adjoint state and the per-tile intermediates.
uint64_t mlp_backward_unit_floats(const ttt_params* p);
uint64_t mlp_backward_workspace_bytes(const ttt_params* p);

// ttt_mlp_backward.
ttt_status mlp_backward(const ttt_params* p, int32_t hidden, const void* q, const void* k,
                        const void* v, const float* eta, const float* w1_0, const float* b1_0,
                        const float* w2_0, const float* b2_0, const float* ln_gamma,
                        const float* ln_beta, const void* dz, const float* dw1_final,
                        const float* db1_final, const float* dw2_final, const float* db2_final,
                        void* dq, void* dk, void* dv, float* deta, float* dw1, float* db1,
                        float* dw2, float* db2, float* dln_gamma, float* dln_beta,
                        void* workspace, uint64_t workspace_bytes, tttk::MlpBackwardArgs* a);

// ttt_input_projection.
ttt_status input_projection(const ttt_params* p, int32_t d_model, const void* x,
                            const void* w_in, const float* b_eta, float eta_base, void* q,
                            void* k, void* v, float* eta, tttk::InputArgs* a);

}  // namespace tttv
