// ttt_input.hpp -- launch interface of the input side (ttt_input.hip):
// q, k, v and the learning-rate gate from the layer input.  Argument struct
// in ttt_args.hpp; the host API has validated every field before the
// launcher is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ttt_args.hpp"

namespace tttk {

// Workgroups of the launch (a multiple of the 8 XCDs).
uint32_t input_grid(const InputArgs& a);

// One kernel on `stream`.  Returns the hipError_t of the launch.
hipError_t launch_input(const InputArgs& a, hipStream_t stream);

}  // namespace tttk
