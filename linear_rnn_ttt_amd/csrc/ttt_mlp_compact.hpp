// ttt_mlp_compact.hpp -- launch interface of the TTT-MLP streaming step with
// a compact pending state (ttt_mlp_decode_compact.hip).  Argument struct in
// ttt_args.hpp; the host API has validated every field.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ttt_args.hpp"

namespace tttk {

hipError_t launch_mlp_decode_compact(const MlpCompactArgs& a, bool bf16, bool ln, bool residual,
                                     hipStream_t stream);

}  // namespace tttk
