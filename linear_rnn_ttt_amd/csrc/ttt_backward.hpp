// ttt_backward.hpp -- launch interface of the TTT-Linear backward scan
// (ttt_backward.hip).  Argument struct in ttt_args.hpp; the host API
// has validated every field before the launcher is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ttt_args.hpp"

namespace tttk {

// Kernels on `stream`: the scan -- one launch (one workgroup per unit) for
// mini-batches of several tiles; for 16-token ones the replay of the bases
// (unless the forward saved them), the front half of every tile (one
// workgroup per unit and tile) and the reverse walk (one per unit) -- then
// the sums over the batch.  Returns the hipError_t of the launches.
hipError_t launch_linear_backward(const BackwardArgs& a, bool bf16, bool ln, bool residual,
                                  hipStream_t stream);

}  // namespace tttk
