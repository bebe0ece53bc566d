// ttt_kernels.hpp -- launch interface between the host API (ttt_api.cpp) and
// the gfx950 scan and streaming-step kernels (argument structs in
// ttt_args.hpp; the host API has validated every field before a launcher is
// called).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ttt_args.hpp"

namespace tttk {

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
