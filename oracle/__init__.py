"""fp64 CPU oracle of the TTT-layer forward scan (ctypes binding).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the GPU path (``linear_rnn_ttt_amd``) and never imports it.

The arithmetic lives in ``ttt_oracle.c`` (plain C, fp64, one token at a
time, explicit gradients); its header states the sources on the pages, the
readings taken where they are silent, and the layouts.  This module only
marshals numpy arrays.

Functions
---------
linear(q, k, v, eta, w0, gamma, beta, ...) -> (z, w)
mlp(q, k, v, eta, w1, b1, w2, b2, gamma, beta, ...) -> (z, (w1, b1, w2, b2))
linear_loss_grad(W, k, v, gamma, beta, ...) -> (loss, dW)
mlp_loss_grad(W1, b1, W2, b2, k, v, gamma, beta, ...) -> (loss, grads)
linear_apply / mlp_apply: the inner model f for one token.
linear_decode_step(W, W_base, q, k, v, eta, gamma, beta, pos=...) -> (z, W, W_base):
    one token of the TTT-Linear scan for one unit, the streaming form.
mlp_decode_step(S, S_base, q, k, v, eta, gamma, beta, pos=...) -> (z, S, S_base):
    the same for TTT-MLP, S = (W1, b1, W2, b2).
build(): compile ``libttt_oracle.so`` with gcc.

The backward pass of the TTT-Linear scan (its vector-Jacobian product) is in
``oracle/backward.py`` (fp64 torch autograd through the scan written out
token by token).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ttt_oracle.c")
_LIB = os.path.join(_HERE, "libttt_oracle.so")
# A prebuilt oracle library to load instead (used by the mutation test,
# which compiles deliberately broken copies and checks the pins catch them).
_OVERRIDE = os.environ.get("TTT_ORACLE_LIB_OVERRIDE")
_lib = None


class _Cfg(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int), ("H", ctypes.c_int), ("T", ctypes.c_int),
        ("d", ctypes.c_int), ("mini_batch", ctypes.c_int),
        ("use_ln", ctypes.c_int), ("use_residual", ctypes.c_int),
        ("ln_eps", ctypes.c_double), ("state0_per_batch", ctypes.c_int),
    ]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math).  Returns the path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
            "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _OVERRIDE:
        _lib = _declare(ctypes.CDLL(_OVERRIDE))
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    _lib = _declare(ctypes.CDLL(_LIB))
    return _lib


def _declare(lib):
    P = ctypes.c_void_p
    lib.ttt_oracle_linear.argtypes = [ctypes.POINTER(_Cfg)] + [P] * 9 + [ctypes.c_int]
    lib.ttt_oracle_linear.restype = ctypes.c_int
    lib.ttt_oracle_mlp.argtypes = ([ctypes.POINTER(_Cfg), ctypes.c_int] + [P] * 15
                                   + [ctypes.c_int])
    lib.ttt_oracle_mlp.restype = ctypes.c_int
    lib.ttt_oracle_linear_loss_grad.argtypes = ([ctypes.c_int] * 3 + [ctypes.c_double]
                                                + [P] * 6)
    lib.ttt_oracle_linear_loss_grad.restype = ctypes.c_double
    lib.ttt_oracle_mlp_loss_grad.argtypes = ([ctypes.c_int] * 4 + [ctypes.c_double]
                                             + [P] * 12)
    lib.ttt_oracle_mlp_loss_grad.restype = ctypes.c_double
    lib.ttt_oracle_linear_apply.argtypes = ([ctypes.c_int] * 3 + [ctypes.c_double]
                                            + [P] * 5)
    lib.ttt_oracle_linear_apply.restype = None
    lib.ttt_oracle_mlp_apply.argtypes = ([ctypes.c_int] * 4 + [ctypes.c_double]
                                         + [P] * 8)
    lib.ttt_oracle_mlp_apply.restype = None
    return lib


def _f32(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    return a


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _threads(n):
    if n is None:
        n = os.cpu_count() or 1
    return int(n)


def linear(q, k, v, eta, w0, gamma=None, beta=None, *, mini_batch=16,
           layer_norm=True, residual=True, eps=1e-6, state0_per_batch=False,
           n_threads=None):
    """TTT-Linear forward scan.  q, k, v [B,H,T,d]; eta [B,H,T];
    w0 [H,d,d] (or [B,H,d,d] with state0_per_batch); gamma, beta [H,d].
    Returns z [B,H,T,d] and the final state [B,H,d,d], both fp64."""
    lib = _load()
    q, k, v, eta, w0 = (_f32(x) for x in (q, k, v, eta, w0))
    B, H, T, d = q.shape
    assert k.shape == v.shape == q.shape and eta.shape == (B, H, T)
    assert w0.shape == ((B, H, d, d) if state0_per_batch else (H, d, d))
    if layer_norm:
        gamma, beta = _f32(gamma), _f32(beta)
        assert gamma.shape == beta.shape == (H, d)
    else:
        gamma = beta = None
    cfg = _Cfg(B, H, T, d, int(mini_batch), int(bool(layer_norm)),
               int(bool(residual)), float(eps), int(bool(state0_per_batch)))
    z = np.empty((B, H, T, d), np.float64)
    w = np.empty((B, H, d, d), np.float64)
    rc = lib.ttt_oracle_linear(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(eta),
                               _ptr(w0), _ptr(gamma), _ptr(beta), _ptr(z), _ptr(w),
                               _threads(n_threads))
    if rc != 0:
        raise ValueError("ttt_oracle_linear failed (%d)" % rc)
    return z, w


def mlp(q, k, v, eta, w1, b1, w2, b2, gamma=None, beta=None, *, mini_batch=16,
        layer_norm=True, residual=True, eps=1e-6, state0_per_batch=False,
        n_threads=None):
    """TTT-MLP forward scan.  w1 [H,d,m], b1 [H,m], w2 [H,m,d], b2 [H,d]
    (leading B with state0_per_batch).  Returns z and (w1, b1, w2, b2) final,
    each with a leading [B,H]."""
    lib = _load()
    q, k, v, eta, w1, b1, w2, b2 = (_f32(x) for x in (q, k, v, eta, w1, b1, w2, b2))
    B, H, T, d = q.shape
    m = w1.shape[-1]
    lead = (B, H) if state0_per_batch else (H,)
    assert w1.shape == lead + (d, m) and b1.shape == lead + (m,)
    assert w2.shape == lead + (m, d) and b2.shape == lead + (d,)
    if layer_norm:
        gamma, beta = _f32(gamma), _f32(beta)
    else:
        gamma = beta = None
    cfg = _Cfg(B, H, T, d, int(mini_batch), int(bool(layer_norm)),
               int(bool(residual)), float(eps), int(bool(state0_per_batch)))
    z = np.empty((B, H, T, d), np.float64)
    ow1 = np.empty((B, H, d, m)); ob1 = np.empty((B, H, m))
    ow2 = np.empty((B, H, m, d)); ob2 = np.empty((B, H, d))
    rc = lib.ttt_oracle_mlp(ctypes.byref(cfg), m, _ptr(q), _ptr(k), _ptr(v), _ptr(eta),
                            _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(gamma),
                            _ptr(beta), _ptr(z), _ptr(ow1), _ptr(ob1), _ptr(ow2),
                            _ptr(ob2), _threads(n_threads))
    if rc != 0:
        raise ValueError("ttt_oracle_mlp failed (%d)" % rc)
    return z, (ow1, ob1, ow2, ob2)


def linear_loss_grad(W, k, v, gamma=None, beta=None, *, layer_norm=True,
                     residual=True, eps=1e-6, grad=True):
    lib = _load()
    W, k, v = _f64(W), _f64(k), _f64(v)
    d = k.shape[0]
    g = np.empty((d, d)) if grad else None
    gam = _f64(gamma) if layer_norm else None
    bet = _f64(beta) if layer_norm else None
    loss = lib.ttt_oracle_linear_loss_grad(d, int(layer_norm), int(residual), float(eps),
                                           _ptr(W), _ptr(k), _ptr(v), _ptr(gam),
                                           _ptr(bet), _ptr(g))
    return loss, g


def mlp_loss_grad(W1, b1, W2, b2, k, v, gamma=None, beta=None, *, layer_norm=True,
                  residual=True, eps=1e-6, grad=True):
    lib = _load()
    W1, b1, W2, b2, k, v = (_f64(x) for x in (W1, b1, W2, b2, k, v))
    d, m = W1.shape
    gam = _f64(gamma) if layer_norm else None
    bet = _f64(beta) if layer_norm else None
    gs = [np.empty((d, m)), np.empty(m), np.empty((m, d)), np.empty(d)] if grad else [None] * 4
    loss = lib.ttt_oracle_mlp_loss_grad(d, m, int(layer_norm), int(residual), float(eps),
                                        _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2), _ptr(k),
                                        _ptr(v), _ptr(gam), _ptr(bet),
                                        *[_ptr(x) for x in gs])
    return loss, (tuple(gs) if grad else None)


def linear_apply(W, x, gamma=None, beta=None, *, layer_norm=True, residual=True, eps=1e-6):
    lib = _load()
    W, x = _f64(W), _f64(x)
    d = x.shape[0]
    out = np.empty(d)
    lib.ttt_oracle_linear_apply(d, int(layer_norm), int(residual), float(eps), _ptr(W),
                                _ptr(x), _ptr(_f64(gamma) if layer_norm else None),
                                _ptr(_f64(beta) if layer_norm else None), _ptr(out))
    return out


def mlp_apply(W1, b1, W2, b2, x, gamma=None, beta=None, *, layer_norm=True,
              residual=True, eps=1e-6):
    lib = _load()
    W1, b1, W2, b2, x = (_f64(a) for a in (W1, b1, W2, b2, x))
    d, m = W1.shape
    out = np.empty(d)
    lib.ttt_oracle_mlp_apply(d, m, int(layer_norm), int(residual), float(eps), _ptr(W1),
                             _ptr(b1), _ptr(W2), _ptr(b2), _ptr(x),
                             _ptr(_f64(gamma) if layer_norm else None),
                             _ptr(_f64(beta) if layer_norm else None), _ptr(out))
    return out


def linear_decode_step(W, W_base, q, k, v, eta, gamma=None, beta=None, *, pos,
                       layer_norm=True, residual=True, eps=1e-6):
    """One token of the TTT-Linear scan for one unit, carrying the stream's
    state W, its mini-batch base W_base and the token's position pos in its
    mini-batch (the LIT-801 record, "Key takeaways" items 1, 2 and 5: every
    gradient of a mini-batch is taken at the state the mini-batch started
    from, the state takes the tokens one by one, z uses the state after its
    own token).  A new mini-batch (pos == 0) starts from the current W.
    Returns (z, W_new, base) in fp64; base is the W_base to carry."""
    W = _f64(W)
    base = W if pos == 0 else _f64(W_base)
    _, g = linear_loss_grad(base, k, v, gamma, beta, layer_norm=layer_norm,
                            residual=residual, eps=eps)
    W_new = W - float(eta) * g
    z = linear_apply(W_new, q, gamma, beta, layer_norm=layer_norm, residual=residual, eps=eps)
    return z, W_new, base.copy()


def mlp_decode_step(S, S_base, q, k, v, eta, gamma=None, beta=None, *, pos,
                    layer_norm=True, residual=True, eps=1e-6):
    """One token of the TTT-MLP scan for one unit, carrying the stream's state
    S = (W1, b1, W2, b2), its mini-batch base S_base and the token's position
    pos in its mini-batch (the LIT-801 record, "Key takeaways" items 1, 2 and
    5, as linear_decode_step).  Returns (z, S_new, base) in fp64."""
    S = tuple(_f64(x) for x in S)
    base = S if pos == 0 else tuple(_f64(x) for x in S_base)
    _, grads = mlp_loss_grad(*base, k, v, gamma, beta, layer_norm=layer_norm,
                             residual=residual, eps=eps)
    S_new = tuple(x - float(eta) * gx for x, gx in zip(S, grads))
    z = mlp_apply(*S_new, q, gamma, beta, layer_norm=layer_norm, residual=residual, eps=eps)
    return z, S_new, tuple(x.copy() for x in base)
