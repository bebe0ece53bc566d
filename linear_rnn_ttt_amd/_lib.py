"""ctypes binding of libttt_amd.so (include/ttt.h).  Argument marshalling
only: every step of the scan runs in the library's gfx950 kernels.  The
library is loaded on first use and its absence is an error, never a
fallback."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libttt_amd.so")

TTT_OK, TTT_ERR_NULL, TTT_ERR_SHAPE, TTT_ERR_UNSUPPORTED = 0, 1, 2, 3
TTT_ERR_ALIAS, TTT_ERR_DEVICE, TTT_ERR_ARG, TTT_ERR_TOO_LARGE = 4, 5, 6, 7
TTT_NOALLOC_SCRATCH_BYTES = 128 << 20
TTT_F32, TTT_BF16 = 0, 1
TTT_NO_LN, TTT_NO_RESIDUAL, TTT_BASES_SAVED = 1, 2, 4

EXPORTS = ("ttt_linear_forward", "ttt_linear_split_workspace_bytes", "ttt_linear_forward_split",
           "ttt_linear_forward_split_noalloc",
           "ttt_linear_decode_step", "ttt_linear_decode_step_compact", "ttt_linear_forward_save",
           "ttt_linear_backward_workspace_bytes", "ttt_linear_backward",
           "ttt_mlp_backward_workspace_bytes", "ttt_mlp_backward",
           "ttt_mlp_forward", "ttt_mlp_decode_step",
           "ttt_mlp_decode_step_compact", "ttt_input_projection", "ttt_status_string",
           "ttt_abi_version")


class TTTParams(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
        ("d", ctypes.c_int32), ("mini_batch", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
        ("flags", ctypes.c_uint32), ("ln_eps", ctypes.c_float),
        ("state0_per_batch", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libttt_amd.so is not built (expected at %s); run "
            "`python -m linear_rnn_ttt_amd.build` (hipcc, gfx950)" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    L.ttt_linear_forward.argtypes = [ctypes.POINTER(TTTParams)] + [P] * 10
    L.ttt_linear_forward.restype = ctypes.c_int
    L.ttt_linear_split_workspace_bytes.argtypes = [ctypes.POINTER(TTTParams)]
    L.ttt_linear_split_workspace_bytes.restype = ctypes.c_uint64
    L.ttt_linear_forward_split.argtypes = ([ctypes.POINTER(TTTParams)] + [P] * 10 +
                                           [ctypes.c_uint64, P])
    L.ttt_linear_forward_split.restype = ctypes.c_int
    L.ttt_linear_forward_split_noalloc.argtypes = [ctypes.POINTER(TTTParams)] + [P] * 10
    L.ttt_linear_forward_split_noalloc.restype = ctypes.c_int
    L.ttt_linear_decode_step.argtypes = [ctypes.POINTER(TTTParams), ctypes.c_int32] + [P] * 10
    L.ttt_linear_decode_step.restype = ctypes.c_int
    L.ttt_linear_decode_step_compact.argtypes = ([ctypes.POINTER(TTTParams), ctypes.c_int32] +
                                                 [P] * 10)
    L.ttt_linear_decode_step_compact.restype = ctypes.c_int
    L.ttt_mlp_decode_step.argtypes = ([ctypes.POINTER(TTTParams), ctypes.c_int32, ctypes.c_int32]
                                      + [P] * 16)
    L.ttt_mlp_decode_step.restype = ctypes.c_int
    L.ttt_mlp_decode_step_compact.argtypes = ([ctypes.POINTER(TTTParams), ctypes.c_int32,
                                               ctypes.c_int32] + [P] * 13)
    L.ttt_mlp_decode_step_compact.restype = ctypes.c_int
    L.ttt_linear_forward_save.argtypes = ([ctypes.POINTER(TTTParams)] + [P] * 10 +
                                          [ctypes.c_uint64, P])
    L.ttt_linear_forward_save.restype = ctypes.c_int
    L.ttt_linear_backward_workspace_bytes.argtypes = [ctypes.POINTER(TTTParams)]
    L.ttt_linear_backward_workspace_bytes.restype = ctypes.c_uint64
    L.ttt_linear_backward.argtypes = ([ctypes.POINTER(TTTParams)] + [P] * 17 +
                                      [ctypes.c_uint64, P])
    L.ttt_linear_backward.restype = ctypes.c_int
    L.ttt_mlp_backward_workspace_bytes.argtypes = [ctypes.POINTER(TTTParams), ctypes.c_int32]
    L.ttt_mlp_backward_workspace_bytes.restype = ctypes.c_uint64
    L.ttt_mlp_backward.argtypes = ([ctypes.POINTER(TTTParams), ctypes.c_int32] + [P] * 26 +
                                   [ctypes.c_uint64, P])
    L.ttt_mlp_backward.restype = ctypes.c_int
    L.ttt_mlp_forward.argtypes = [ctypes.POINTER(TTTParams), ctypes.c_int32] + [P] * 16
    L.ttt_mlp_forward.restype = ctypes.c_int
    L.ttt_input_projection.argtypes = ([ctypes.POINTER(TTTParams), ctypes.c_int32, P, P, P,
                                        ctypes.c_float] + [P] * 5)
    L.ttt_input_projection.restype = ctypes.c_int
    L.ttt_status_string.argtypes = [ctypes.c_int]
    L.ttt_status_string.restype = ctypes.c_char_p
    L.ttt_abi_version.argtypes = []
    L.ttt_abi_version.restype = ctypes.c_int32
    _lib = L
    return L


def status_string(code: int) -> str:
    return lib().ttt_status_string(int(code)).decode()


def abi_version() -> int:
    return int(lib().ttt_abi_version())


class TTTError(RuntimeError):
    def __init__(self, func: str, code: int):
        self.code = int(code)
        super().__init__("%s: %s (status %d)" % (func, status_string(code), code))


class TTTArgumentError(TTTError, ValueError):
    pass


def check(func: str, code: int) -> None:
    if code == TTT_OK:
        return
    if code == TTT_ERR_DEVICE:
        raise TTTError(func, code)
    raise TTTArgumentError(func, code)
