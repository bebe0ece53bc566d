"""MI355X (gfx950) TTT layer: the TTT-Linear and TTT-MLP scans (forward,
backward, streaming step) and the input side that feeds them.

The scan runs in hand-written HIP kernels behind the C ABI of
``include/ttt.h`` (library ``libttt_amd.so``, built in-tree by
``linear_rnn_ttt_amd.build``).  This package is the thin Python side:
argument marshalling, with PyTorch supplying device memory and streams.
"""
from ._lib import TTTArgumentError, TTTError, abi_version, status_string  # noqa: F401
from .ops import (ttt_input_projection, ttt_linear_backward,  # noqa: F401
                  ttt_linear_decode_step, ttt_linear_decode_step_compact, ttt_linear_forward,
                  ttt_linear_forward_split_noalloc, ttt_mlp_decode_step,
                  ttt_mlp_backward, ttt_mlp_decode_step_compact, ttt_mlp_forward)

__all__ = ["ttt_linear_forward", "ttt_linear_forward_split_noalloc", "ttt_linear_decode_step",
           "ttt_linear_decode_step_compact", "ttt_linear_backward", "ttt_mlp_backward", "ttt_mlp_forward", "ttt_mlp_decode_step",
           "ttt_mlp_decode_step_compact", "ttt_input_projection",
           "abi_version",
           "status_string",
           "TTTError", "TTTArgumentError"]
