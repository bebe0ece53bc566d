"""A plain fp32 evaluation of the scan, for grounding the GPU tolerance on
ill-conditioned units.

TEST INFRASTRUCTURE ONLY.  It compiles a copy of the oracle's C source
(``oracle/ttt_oracle.c``) with every ``double`` turned into ``float``
(``#define double float``): the same token-by-token algorithm, the same summation
order, with each operation rounded to fp32 instead of fp64.  Nothing of the
GPU path is involved.  The copy has its own ABI (fp32 outputs and an fp32
epsilon in the configuration struct), declared here.  The system headers
are included before the macro, so libm keeps its fp64 signatures (an fp32
argument is widened, the result rounded back to fp32).

Use: on a unit where this fp32 evaluation itself misses the workload's
tolerance against the fp64 oracle, the scan is too ill-conditioned for any
evaluation carrying fp32-level operands to be held to that tolerance; only
there may the GPU be held to a multiple of the fp32 evaluation's error
instead (tests/_parity.py)."""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ttt_oracle.c")
_lib = None


class _Cfg(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int), ("H", ctypes.c_int), ("T", ctypes.c_int),
        ("d", ctypes.c_int), ("mini_batch", ctypes.c_int),
        ("use_ln", ctypes.c_int), ("use_residual", ctypes.c_int),
        ("ln_eps", ctypes.c_float), ("state0_per_batch", ctypes.c_int),
    ]


def build(out_dir: str | None = None) -> str:
    """Compile the fp32 copy; returns the library path."""
    out_dir = out_dir or tempfile.mkdtemp(prefix="ttt_oracle_f32_")
    lib = os.path.join(out_dir, "libttt_oracle_f32.so")
    unit = os.path.join(out_dir, "ttt_oracle_f32.c")
    with open(unit, "w") as f:
        f.write("#include <math.h>\n#include <pthread.h>\n#include <stdlib.h>\n"
                "#include <string.h>\n#define double float\n#include \"%s\"\n" % SRC)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared",
                           "-I", os.path.join(ROOT, "oracle"), "-o", lib, unit, "-lm",
                           "-lpthread"])
    return lib


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        lib.ttt_oracle_linear.argtypes = [ctypes.POINTER(_Cfg)] + [P] * 9 + [ctypes.c_int]
        lib.ttt_oracle_linear.restype = ctypes.c_int
        lib.ttt_oracle_mlp.argtypes = ([ctypes.POINTER(_Cfg), ctypes.c_int] + [P] * 15
                                       + [ctypes.c_int])
        lib.ttt_oracle_mlp.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _cfg(q, mini_batch, eps):
    B, H, T, d = q.shape
    return _Cfg(B, H, T, d, int(mini_batch), 1, 1, float(eps), 0)


def linear(q, k, v, eta, w0, gamma, beta, *, mini_batch=16, eps=1e-6, n_threads=None):
    """TTT-Linear scan in fp32 (LN and residual on, W0 [H,d,d] shared over
    the batch).  Returns z [B,H,T,d] and the final state [B,H,d,d] (fp32)."""
    lib = _load()
    q, k, v, eta, w0, gamma, beta = (_f32(x) for x in (q, k, v, eta, w0, gamma, beta))
    B, H, T, d = q.shape
    z = np.empty((B, H, T, d), np.float32)
    w = np.empty((B, H, d, d), np.float32)
    rc = lib.ttt_oracle_linear(ctypes.byref(_cfg(q, mini_batch, eps)), _p(q), _p(k), _p(v),
                               _p(eta), _p(w0), _p(gamma), _p(beta), _p(z), _p(w),
                               int(n_threads or os.cpu_count() or 1))
    if rc != 0:
        raise ValueError("fp32 oracle failed (%d)" % rc)
    return z, w


def mlp(q, k, v, eta, w1, b1, w2, b2, gamma, beta, *, mini_batch=16, eps=1e-6,
        n_threads=None):
    """TTT-MLP scan in fp32.  Returns z and (w1, b1, w2, b2) final (fp32)."""
    lib = _load()
    q, k, v, eta, w1, b1, w2, b2, gamma, beta = (
        _f32(x) for x in (q, k, v, eta, w1, b1, w2, b2, gamma, beta))
    B, H, T, d = q.shape
    m = w1.shape[-1]
    z = np.empty((B, H, T, d), np.float32)
    out = [np.empty((B, H, d, m), np.float32), np.empty((B, H, m), np.float32),
           np.empty((B, H, m, d), np.float32), np.empty((B, H, d), np.float32)]
    rc = lib.ttt_oracle_mlp(ctypes.byref(_cfg(q, mini_batch, eps)), m, _p(q), _p(k), _p(v),
                            _p(eta), _p(w1), _p(b1), _p(w2), _p(b2), _p(gamma), _p(beta),
                            _p(z), *[_p(x) for x in out], int(n_threads or os.cpu_count() or 1))
    if rc != 0:
        raise ValueError("fp32 oracle failed (%d)" % rc)
    return z, tuple(out)
