// ttt_mlp_backward.hpp -- launch interface of the TTT-MLP backward scan
// (ttt_mlp_backward.hip).  Argument struct in ttt_args.hpp; the host API has
// validated every field before the launcher is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ttt_args.hpp"

namespace tttk {

// Two kernels on `stream`: the scan (one workgroup per unit) and the sums
// over the batch.  Returns the hipError_t of the launches.
hipError_t launch_mlp_backward(const MlpBackwardArgs& a, bool bf16, bool ln, bool residual,
                               hipStream_t stream);

}  // namespace tttk
