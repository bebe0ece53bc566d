// ttt_stream.hpp -- launch interfaces of the streaming steps: TTT-Linear
// with a compact pending state (ttt_decode_compact.hip) and TTT-MLP
// (ttt_mlp_decode.hip).  Argument structs in
// ttt_args.hpp; the host API has validated every field.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ttt_args.hpp"

namespace tttk {

hipError_t launch_linear_decode_compact(const CompactArgs& a, bool bf16, bool ln, bool residual,
                                        hipStream_t stream);

hipError_t launch_mlp_decode(const MlpDecodeArgs& a, bool bf16, bool ln, bool residual,
                             hipStream_t stream);

}  // namespace tttk
