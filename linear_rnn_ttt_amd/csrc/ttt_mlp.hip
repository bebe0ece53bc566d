// ttt_mlp.hip -- TTT-MLP forward scan for gfx950 (placeholder launcher until
// the kernel lands).
#include "ttt_kernels.hpp"

namespace tttk {

hipError_t launch_mlp(const MlpArgs&, bool, bool, bool, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace tttk
