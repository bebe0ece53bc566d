"""Python entry points with the names of the C ABI (include/ttt.h).

PyTorch provides device memory and the stream; these functions check and
marshal arguments, allocate the outputs with torch, and call the library,
which launches the gfx950 kernels asynchronously on the current stream.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib

__all__ = ["ttt_linear_forward", "ttt_linear_forward_split_noalloc", "ttt_linear_decode_step",
           "ttt_linear_decode_step_compact", "ttt_linear_backward", "ttt_mlp_forward",
           "ttt_mlp_backward", "ttt_mlp_decode_step", "ttt_mlp_decode_step_compact",
           "ttt_input_projection"]

HEAD_DIM = 64


def _dev_tensor(name, t, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor (got %s)" % (name, t.device))
    if device is not None and t.device != device:
        raise ValueError("%s must be on %s, like q (got %s)" % (name, device, t.device))
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _ptr(t) -> Optional[int]:
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _params(q, mini_batch, eps, layer_norm, residual, state0_per_batch):
    if q.dtype == torch.bfloat16:
        io = _lib.TTT_BF16
    elif q.dtype == torch.float32:
        io = _lib.TTT_F32
    else:
        raise ValueError("q, k, v must be bfloat16 or float32 (got %s)" % q.dtype)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d]")
    B, H, T, d = q.shape
    flags = (0 if layer_norm else _lib.TTT_NO_LN) | (0 if residual else _lib.TTT_NO_RESIDUAL)
    return _lib.TTTParams(B, H, T, d, int(mini_batch), io, flags, float(eps),
                          int(bool(state0_per_batch)))


def _stream(q, stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream(q.device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# When the two-workgroup launch is chosen by default (measured on MI355X,
# 256 CUs, steady state).  bf16 data at T = 8192: 32 units 8 % faster, 64
# units 6 %, 96 units 5 %, 128 units (every CU busy) no gain, since the
# shader clock drops with the load; at T = 2048 it loses about 2 % to the
# second workgroup's lag.  fp32 data, whose update waves carry 1.5x the
# matrix products of bf16 data and so delay the chain more: 24 % faster at
# 128 units, 31 % at 64, 26 % at 96 units with T = 2048.
SPLIT_POLICY = {"bf16": (3 / 8, 4096), "f32": (1 / 2, 1024)}  # (max B*H / CUs, min T)


def linear_uses_split(B: int, H: int, T: int, device=None, dtype=torch.bfloat16) -> bool:
    """The launch ttt_linear_forward picks when split=None."""
    cus = _compute_units(torch.device("cuda") if device is None else device)
    share, min_t = SPLIT_POLICY["bf16" if dtype == torch.bfloat16 else "f32"]
    return B * H <= share * cus and T >= min_t


def _compute_units(dev) -> int:
    return torch.cuda.get_device_properties(dev).multi_processor_count


def ttt_linear_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, eta: torch.Tensor,
                       w0: torch.Tensor, ln_gamma: Optional[torch.Tensor] = None,
                       ln_beta: Optional[torch.Tensor] = None, *, mini_batch: int = 16,
                       eps: float = 1e-6, layer_norm: bool = True, residual: bool = True,
                       state0_per_batch: bool = False, z: Optional[torch.Tensor] = None,
                       w_out: Optional[torch.Tensor] = None, return_state: bool = True,
                       split: Optional[bool] = None, workspace: Optional[torch.Tensor] = None,
                       save_for_backward: Optional[torch.Tensor] = None,
                       stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """TTT-Linear forward scan on the GPU; returns (z [B,H,T,d], W_final
    [B,H,d,d] fp32 or None).  See include/ttt.h for the semantics.

    split: True runs ttt_linear_forward_split (two workgroups per unit, a
    device workspace; B*H at most half the compute units), False
    ttt_linear_forward; None decides by linear_uses_split.  The results are
    the same either way.  workspace: a uint8 GPU tensor of at
    least ttt_linear_split_workspace_bytes bytes to use instead of a fresh
    one.

    save_for_backward: a uint8 GPU tensor of at least
    ttt_linear_backward_workspace_bytes bytes; the scan then runs as
    ttt_linear_forward_save (one workgroup per unit, mini-batch 16) and
    stores every mini-batch base there, for ttt_linear_backward(...,
    workspace=that tensor, bases_saved=True)."""
    _dev_tensor("q", q)
    B, H, T, d = q.shape
    _dev_tensor("k", k, q.dtype, q.shape, device=q.device)
    _dev_tensor("v", v, q.dtype, q.shape, device=q.device)
    _dev_tensor("eta", eta, torch.float32, (B, H, T), device=q.device)
    _dev_tensor("w0", w0, torch.float32, (B, H, d, d) if state0_per_batch else (H, d, d),
                device=q.device)
    if layer_norm:
        _dev_tensor("ln_gamma", ln_gamma, torch.float32, (H, d), device=q.device)
        _dev_tensor("ln_beta", ln_beta, torch.float32, (H, d), device=q.device)
    else:
        ln_gamma = ln_beta = None
    if z is None:
        z = torch.empty_like(q)
    _dev_tensor("z", z, q.dtype, q.shape, device=q.device)
    if w_out is None and return_state:
        w_out = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device)
    if w_out is not None:
        _dev_tensor("w_out", w_out, torch.float32, (B, H, d, d), device=q.device)
    p = _params(q, mini_batch, eps, layer_norm, residual, state0_per_batch)
    if split is None:   # the split launch has no in-place form
        split = (linear_uses_split(B, H, T, q.device, q.dtype) and
                 (w_out is None or w_out.data_ptr() != w0.data_ptr()))
    args = (ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w0), _ptr(ln_gamma),
            _ptr(ln_beta), _ptr(z), _ptr(w_out))
    with torch.cuda.device(q.device):   # the library launches on the current device
        if save_for_backward is not None:
            _dev_tensor("save_for_backward", save_for_backward, torch.uint8, device=q.device)
            rc = _lib.lib().ttt_linear_forward_save(*args, _ptr(save_for_backward),
                                                    save_for_backward.numel(),
                                                    _stream(q, stream))
            _lib.check("ttt_linear_forward_save", rc)
        elif split:
            need = int(_lib.lib().ttt_linear_split_workspace_bytes(ctypes.byref(p)))
            if workspace is None:
                workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
            _dev_tensor("workspace", workspace, torch.uint8, device=q.device)
            rc = _lib.lib().ttt_linear_forward_split(*args, _ptr(workspace),
                                                     workspace.numel(), _stream(q, stream))
            _lib.check("ttt_linear_forward_split", rc)
        else:
            rc = _lib.lib().ttt_linear_forward(*args, _stream(q, stream))
            _lib.check("ttt_linear_forward", rc)
    return z, w_out


def ttt_linear_forward_split_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                     eta: torch.Tensor, w0: torch.Tensor,
                                     ln_gamma: Optional[torch.Tensor] = None,
                                     ln_beta: Optional[torch.Tensor] = None, *,
                                     z: torch.Tensor, w_out: Optional[torch.Tensor] = None,
                                     mini_batch: int = 16, eps: float = 1e-6,
                                     layer_norm: bool = True, residual: bool = True,
                                     state0_per_batch: bool = False, stream=None) -> None:
    """ttt_linear_forward_split_noalloc of include/ttt.h: the two-workgroup
    TTT-Linear scan with its scratch in the library's fixed per-device array
    instead of a workspace.  Nothing is allocated here either: the caller
    passes z [B,H,T,d] and, optionally, w_out [B,H,d,d] fp32."""
    _dev_tensor("q", q)
    B, H, T, d = q.shape
    _dev_tensor("k", k, q.dtype, q.shape, device=q.device)
    _dev_tensor("v", v, q.dtype, q.shape, device=q.device)
    _dev_tensor("eta", eta, torch.float32, (B, H, T), device=q.device)
    _dev_tensor("w0", w0, torch.float32, (B, H, d, d) if state0_per_batch else (H, d, d),
                device=q.device)
    if layer_norm:
        _dev_tensor("ln_gamma", ln_gamma, torch.float32, (H, d), device=q.device)
        _dev_tensor("ln_beta", ln_beta, torch.float32, (H, d), device=q.device)
    else:
        ln_gamma = ln_beta = None
    _dev_tensor("z", z, q.dtype, q.shape, device=q.device)
    if w_out is not None:
        _dev_tensor("w_out", w_out, torch.float32, (B, H, d, d), device=q.device)
    p = _params(q, mini_batch, eps, layer_norm, residual, state0_per_batch)
    with torch.cuda.device(q.device):   # the library launches on the current device
        rc = _lib.lib().ttt_linear_forward_split_noalloc(
            ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w0), _ptr(ln_gamma),
            _ptr(ln_beta), _ptr(z), _ptr(w_out), _stream(q, stream))
    _lib.check("ttt_linear_forward_split_noalloc", rc)


def ttt_linear_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                           eta: torch.Tensor, w: torch.Tensor, w_base: torch.Tensor,
                           ln_gamma: Optional[torch.Tensor] = None,
                           ln_beta: Optional[torch.Tensor] = None, *, pos: int,
                           mini_batch: int = 16, eps: float = 1e-6, layer_norm: bool = True,
                           residual: bool = True, z: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """One token per (batch, head) unit of the TTT-Linear scan (streaming
    step); returns z [B,H,d].  w and w_base [B,H,d,d] fp32 are the stream's
    state and mini-batch base, updated in place; pos is the token's position
    in its mini-batch (t mod mini_batch).  See include/ttt.h."""
    _dev_tensor("q", q)
    if q.dim() != 3:
        raise ValueError("q must be [B, H, d] (one token per unit)")
    B, H, d = q.shape
    _dev_tensor("k", k, q.dtype, q.shape, device=q.device)
    _dev_tensor("v", v, q.dtype, q.shape, device=q.device)
    _dev_tensor("eta", eta, torch.float32, (B, H), device=q.device)
    _dev_tensor("w", w, torch.float32, (B, H, d, d), device=q.device)
    _dev_tensor("w_base", w_base, torch.float32, (B, H, d, d), device=q.device)
    if layer_norm:
        _dev_tensor("ln_gamma", ln_gamma, torch.float32, (H, d), device=q.device)
        _dev_tensor("ln_beta", ln_beta, torch.float32, (H, d), device=q.device)
    else:
        ln_gamma = ln_beta = None
    if z is None:
        z = torch.empty_like(q)
    _dev_tensor("z", z, q.dtype, q.shape, device=q.device)
    p = _params(q.unsqueeze(2), mini_batch, eps, layer_norm, residual, True)
    with torch.cuda.device(q.device):   # the library launches on the current device
        rc = _lib.lib().ttt_linear_decode_step(ctypes.byref(p), int(pos), _ptr(q), _ptr(k),
                                               _ptr(v), _ptr(eta), _ptr(w), _ptr(w_base),
                                               _ptr(ln_gamma), _ptr(ln_beta), _ptr(z),
                                               _stream(q, stream))
    _lib.check("ttt_linear_decode_step", rc)
    return z


def ttt_mlp_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, eta: torch.Tensor,
                        state, base, ln_gamma: Optional[torch.Tensor] = None,
                        ln_beta: Optional[torch.Tensor] = None, *, pos: int,
                        mini_batch: int = 16, eps: float = 1e-6, layer_norm: bool = True,
                        residual: bool = True, z: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """One token per (batch, head) unit of the TTT-MLP scan (streaming step);
    returns z [B,H,d].  state and base are (w1 [B,H,d,m], b1 [B,H,m],
    w2 [B,H,m,d], b2 [B,H,d]) fp32, the stream's state and mini-batch base,
    updated in place; pos is the token's position in its mini-batch.  See
    include/ttt.h."""
    _dev_tensor("q", q)
    if q.dim() != 3:
        raise ValueError("q must be [B, H, d] (one token per unit)")
    B, H, d = q.shape
    _dev_tensor("k", k, q.dtype, q.shape, device=q.device)
    _dev_tensor("v", v, q.dtype, q.shape, device=q.device)
    _dev_tensor("eta", eta, torch.float32, (B, H), device=q.device)
    if len(state) != 4 or len(base) != 4:
        raise ValueError("state and base are (w1, b1, w2, b2)")
    m = state[0].shape[-1] if state[0].dim() == 4 else -1
    shapes = ((B, H, d, m), (B, H, m), (B, H, m, d), (B, H, d))
    for tag, group in (("", state), ("_base", base)):
        for name, t, shp in zip(("w1", "b1", "w2", "b2"), group, shapes):
            _dev_tensor(name + tag, t, torch.float32, shp, device=q.device)
    if layer_norm:
        _dev_tensor("ln_gamma", ln_gamma, torch.float32, (H, d), device=q.device)
        _dev_tensor("ln_beta", ln_beta, torch.float32, (H, d), device=q.device)
    else:
        ln_gamma = ln_beta = None
    if z is None:
        z = torch.empty_like(q)
    _dev_tensor("z", z, q.dtype, q.shape, device=q.device)
    p = _params(q.unsqueeze(2), mini_batch, eps, layer_norm, residual, True)
    with torch.cuda.device(q.device):   # the library launches on the current device
        rc = _lib.lib().ttt_mlp_decode_step(ctypes.byref(p), int(m), int(pos), _ptr(q), _ptr(k),
                                            _ptr(v), _ptr(eta), *[_ptr(t) for t in state],
                                            *[_ptr(t) for t in base], _ptr(ln_gamma),
                                            _ptr(ln_beta), _ptr(z), _stream(q, stream))
    _lib.check("ttt_mlp_decode_step", rc)
    return z


def ttt_mlp_decode_step_compact(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                eta: torch.Tensor, base, hist: torch.Tensor,
                                ln_gamma: Optional[torch.Tensor] = None,
                                ln_beta: Optional[torch.Tensor] = None, *, pos: int,
                                mini_batch: int = 16, eps: float = 1e-6,
                                layer_norm: bool = True, residual: bool = True,
                                z: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The TTT-MLP streaming step with a compact pending state; returns z
    [B,H,d].  base = (w1, b1, w2, b2) fp32 (the mini-batch's base) and hist
    [B,H,mini_batch,2d+2m] fp32 (its rows k, u1, a, u2; zero at a stream's
    start) are updated in place.  See include/ttt.h."""
    _dev_tensor("q", q)
    if q.dim() != 3:
        raise ValueError("q must be [B, H, d] (one token per unit)")
    B, H, d = q.shape
    _dev_tensor("k", k, q.dtype, q.shape, device=q.device)
    _dev_tensor("v", v, q.dtype, q.shape, device=q.device)
    _dev_tensor("eta", eta, torch.float32, (B, H), device=q.device)
    if len(base) != 4:
        raise ValueError("base is (w1, b1, w2, b2)")
    m = base[0].shape[-1] if base[0].dim() == 4 else -1
    shapes = ((B, H, d, m), (B, H, m), (B, H, m, d), (B, H, d))
    for name, t, shp in zip(("w1", "b1", "w2", "b2"), base, shapes):
        _dev_tensor(name + "_base", t, torch.float32, shp, device=q.device)
    _dev_tensor("hist", hist, torch.float32, (B, H, mini_batch, 2 * d + 2 * m), device=q.device)
    if layer_norm:
        _dev_tensor("ln_gamma", ln_gamma, torch.float32, (H, d), device=q.device)
        _dev_tensor("ln_beta", ln_beta, torch.float32, (H, d), device=q.device)
    else:
        ln_gamma = ln_beta = None
    if z is None:
        z = torch.empty_like(q)
    _dev_tensor("z", z, q.dtype, q.shape, device=q.device)
    p = _params(q.unsqueeze(2), mini_batch, eps, layer_norm, residual, True)
    with torch.cuda.device(q.device):   # the library launches on the current device
        rc = _lib.lib().ttt_mlp_decode_step_compact(
            ctypes.byref(p), int(m), int(pos), _ptr(q), _ptr(k), _ptr(v), _ptr(eta),
            *[_ptr(t) for t in base], _ptr(hist), _ptr(ln_gamma), _ptr(ln_beta), _ptr(z),
            _stream(q, stream))
    _lib.check("ttt_mlp_decode_step_compact", rc)
    return z


def ttt_linear_decode_step_compact(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                   eta: torch.Tensor, w_base: torch.Tensor, hist: torch.Tensor,
                                   ln_gamma: Optional[torch.Tensor] = None,
                                   ln_beta: Optional[torch.Tensor] = None, *, pos: int,
                                   mini_batch: int = 16, eps: float = 1e-6,
                                   layer_norm: bool = True, residual: bool = True,
                                   z: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The streaming step with a compact pending state; returns z [B,H,d].
    w_base [B,H,d,d] fp32 (the mini-batch's base) and hist
    [B,H,mini_batch,2,d] fp32 (its rows k_s, u_s; zero at a stream's start)
    are updated in place.  See include/ttt.h."""
    _dev_tensor("q", q)
    if q.dim() != 3:
        raise ValueError("q must be [B, H, d] (one token per unit)")
    B, H, d = q.shape
    _dev_tensor("k", k, q.dtype, q.shape, device=q.device)
    _dev_tensor("v", v, q.dtype, q.shape, device=q.device)
    _dev_tensor("eta", eta, torch.float32, (B, H), device=q.device)
    _dev_tensor("w_base", w_base, torch.float32, (B, H, d, d), device=q.device)
    _dev_tensor("hist", hist, torch.float32, (B, H, mini_batch, 2, d), device=q.device)
    if layer_norm:
        _dev_tensor("ln_gamma", ln_gamma, torch.float32, (H, d), device=q.device)
        _dev_tensor("ln_beta", ln_beta, torch.float32, (H, d), device=q.device)
    else:
        ln_gamma = ln_beta = None
    if z is None:
        z = torch.empty_like(q)
    _dev_tensor("z", z, q.dtype, q.shape, device=q.device)
    p = _params(q.unsqueeze(2), mini_batch, eps, layer_norm, residual, True)
    with torch.cuda.device(q.device):
        rc = _lib.lib().ttt_linear_decode_step_compact(
            ctypes.byref(p), int(pos), _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w_base),
            _ptr(hist), _ptr(ln_gamma), _ptr(ln_beta), _ptr(z), _stream(q, stream))
    _lib.check("ttt_linear_decode_step_compact", rc)
    return z


def ttt_linear_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, eta: torch.Tensor,
                        w0: torch.Tensor, ln_gamma: Optional[torch.Tensor],
                        ln_beta: Optional[torch.Tensor], dz: torch.Tensor,
                        dw_final: Optional[torch.Tensor] = None, *, mini_batch: int = 16,
                        eps: float = 1e-6, layer_norm: bool = True, residual: bool = True,
                        state0_per_batch: bool = False, workspace: Optional[torch.Tensor] = None,
                        bases_saved: bool = False, stream=None) -> Tuple[torch.Tensor, ...]:
    """Backward pass of the TTT-Linear scan for cotangents dz [B,H,T,d] (and
    dw_final [B,H,d,d] on the final state, or None); same inputs and options
    as ttt_linear_forward.  Returns (dq, dk, dv, deta, dw0, dln_gamma,
    dln_beta); dw0 has w0's shape (summed over the batch when w0 is shared),
    the LN gradients are [H,d] (zeros without LN).  workspace: a uint8 GPU
    tensor of at least ttt_linear_backward_workspace_bytes bytes to use
    instead of a fresh one.  bases_saved: the workspace holds the bases a
    ttt_linear_forward(..., save_for_backward=workspace) call stored for
    these inputs (TTT_BASES_SAVED): the backward skips replaying them.  See
    include/ttt.h."""
    _dev_tensor("q", q)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d]")
    B, H, T, d = q.shape
    dev = q.device
    for name, t in (("k", k), ("v", v), ("dz", dz)):
        _dev_tensor(name, t, q.dtype, q.shape, device=dev)
    _dev_tensor("eta", eta, torch.float32, (B, H, T), device=dev)
    w0_shape = (B, H, d, d) if state0_per_batch else (H, d, d)
    _dev_tensor("w0", w0, torch.float32, w0_shape, device=dev)
    if layer_norm:
        _dev_tensor("ln_gamma", ln_gamma, torch.float32, (H, d), device=dev)
        _dev_tensor("ln_beta", ln_beta, torch.float32, (H, d), device=dev)
    else:
        ln_gamma = ln_beta = None
    if dw_final is not None:
        _dev_tensor("dw_final", dw_final, torch.float32, (B, H, d, d), device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    deta = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    dw0 = torch.empty(w0_shape, dtype=torch.float32, device=dev)
    dgamma = torch.empty((H, d), dtype=torch.float32, device=dev)
    dbeta = torch.empty((H, d), dtype=torch.float32, device=dev)
    p = _params(q, mini_batch, eps, layer_norm, residual, state0_per_batch)
    need = int(_lib.lib().ttt_linear_backward_workspace_bytes(ctypes.byref(p)))
    if bases_saved:
        if workspace is None:
            raise ValueError("bases_saved needs the workspace the forward saved them in")
        p.flags |= _lib.TTT_BASES_SAVED
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev_tensor("workspace", workspace, torch.uint8, device=dev)
    with torch.cuda.device(dev):   # the library launches on the current device
        rc = _lib.lib().ttt_linear_backward(
            ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w0), _ptr(ln_gamma),
            _ptr(ln_beta), _ptr(dz), _ptr(dw_final), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(deta),
            _ptr(dw0), _ptr(dgamma), _ptr(dbeta), _ptr(workspace), workspace.numel(),
            _stream(q, stream))
    _lib.check("ttt_linear_backward", rc)
    return dq, dk, dv, deta, dw0, dgamma, dbeta


def ttt_mlp_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, eta: torch.Tensor,
                     w1: torch.Tensor, b1: torch.Tensor, w2: torch.Tensor, b2: torch.Tensor,
                     ln_gamma: Optional[torch.Tensor], ln_beta: Optional[torch.Tensor],
                     dz: torch.Tensor, dstate_final=None, *, mini_batch: int = 16,
                     eps: float = 1e-6, layer_norm: bool = True, residual: bool = True,
                     state0_per_batch: bool = False, workspace: Optional[torch.Tensor] = None,
                     stream=None) -> Tuple[torch.Tensor, ...]:
    """Backward pass of the TTT-MLP scan for cotangents dz [B,H,T,d] (and
    dstate_final, a tuple of four [B,H,...] fp32 cotangents of the final
    state, or None); same inputs and options as ttt_mlp_forward.  Returns
    (dq, dk, dv, deta, dw1, db1, dw2, db2, dln_gamma, dln_beta); the state
    gradients have the initial state's shapes (summed over the batch when it
    is shared), the LN gradients are [H,d] (zeros without LN).  workspace: a
    uint8 GPU tensor of at least ttt_mlp_backward_workspace_bytes bytes to
    use instead of a fresh one.  See include/ttt.h."""
    _dev_tensor("q", q)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d]")
    B, H, T, d = q.shape
    m = w1.shape[-1]
    dev = q.device
    for name, t in (("k", k), ("v", v), ("dz", dz)):
        _dev_tensor(name, t, q.dtype, q.shape, device=dev)
    _dev_tensor("eta", eta, torch.float32, (B, H, T), device=dev)
    lead = (B, H) if state0_per_batch else (H,)
    shapes = [(d, m), (m,), (m, d), (d,)]
    state = [w1, b1, w2, b2]
    for name, t, sh in zip(("w1", "b1", "w2", "b2"), state, shapes):
        _dev_tensor(name, t, torch.float32, lead + sh, device=dev)
    if layer_norm:
        _dev_tensor("ln_gamma", ln_gamma, torch.float32, (H, d), device=dev)
        _dev_tensor("ln_beta", ln_beta, torch.float32, (H, d), device=dev)
    else:
        ln_gamma = ln_beta = None
    fin = [None] * 4
    if dstate_final is not None:
        fin = list(dstate_final)
        for name, t, sh in zip(("dw1_final", "db1_final", "dw2_final", "db2_final"), fin, shapes):
            _dev_tensor(name, t, torch.float32, (B, H) + sh, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    deta = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    dstate = [torch.empty(lead + sh, dtype=torch.float32, device=dev) for sh in shapes]
    dgamma = torch.zeros((H, d), dtype=torch.float32, device=dev)
    dbeta = torch.zeros((H, d), dtype=torch.float32, device=dev)
    p = _params(q, mini_batch, eps, layer_norm, residual, state0_per_batch)
    need = int(_lib.lib().ttt_mlp_backward_workspace_bytes(ctypes.byref(p), m))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev_tensor("workspace", workspace, torch.uint8, device=dev)
    with torch.cuda.device(dev):   # the library launches on the current device
        rc = _lib.lib().ttt_mlp_backward(
            ctypes.byref(p), m, _ptr(q), _ptr(k), _ptr(v), _ptr(eta),
            *[_ptr(t) for t in state], _ptr(ln_gamma), _ptr(ln_beta), _ptr(dz),
            *[_ptr(t) for t in fin], _ptr(dq), _ptr(dk), _ptr(dv), _ptr(deta),
            *[_ptr(t) for t in dstate], _ptr(dgamma if layer_norm else None),
            _ptr(dbeta if layer_norm else None), _ptr(workspace), workspace.numel(),
            _stream(q, stream))
    _lib.check("ttt_mlp_backward", rc)
    return (dq, dk, dv, deta, *dstate, dgamma, dbeta)


def ttt_mlp_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, eta: torch.Tensor,
                    w1: torch.Tensor, b1: torch.Tensor, w2: torch.Tensor, b2: torch.Tensor,
                    ln_gamma: Optional[torch.Tensor] = None,
                    ln_beta: Optional[torch.Tensor] = None, *, mini_batch: int = 16,
                    eps: float = 1e-6, layer_norm: bool = True, residual: bool = True,
                    state0_per_batch: bool = False, z: Optional[torch.Tensor] = None,
                    state_out=None, return_state: bool = True, stream=None):
    """TTT-MLP forward scan on the GPU; returns (z, (W1, b1, W2, b2) final
    or None).  See include/ttt.h for the semantics."""
    _dev_tensor("q", q)
    B, H, T, d = q.shape
    m = w1.shape[-1]
    _dev_tensor("k", k, q.dtype, q.shape, device=q.device)
    _dev_tensor("v", v, q.dtype, q.shape, device=q.device)
    _dev_tensor("eta", eta, torch.float32, (B, H, T), device=q.device)
    lead = (B, H) if state0_per_batch else (H,)
    _dev_tensor("w1", w1, torch.float32, lead + (d, m), device=q.device)
    _dev_tensor("b1", b1, torch.float32, lead + (m,), device=q.device)
    _dev_tensor("w2", w2, torch.float32, lead + (m, d), device=q.device)
    _dev_tensor("b2", b2, torch.float32, lead + (d,), device=q.device)
    if layer_norm:
        _dev_tensor("ln_gamma", ln_gamma, torch.float32, (H, d), device=q.device)
        _dev_tensor("ln_beta", ln_beta, torch.float32, (H, d), device=q.device)
    else:
        ln_gamma = ln_beta = None
    if z is None:
        z = torch.empty_like(q)
    _dev_tensor("z", z, q.dtype, q.shape, device=q.device)
    if state_out is None and return_state:
        f = dict(dtype=torch.float32, device=q.device)
        state_out = (torch.empty((B, H, d, m), **f), torch.empty((B, H, m), **f),
                     torch.empty((B, H, m, d), **f), torch.empty((B, H, d), **f))
    if state_out is not None:
        for name, t, shp in zip(("w1_out", "b1_out", "w2_out", "b2_out"), state_out,
                                ((B, H, d, m), (B, H, m), (B, H, m, d), (B, H, d))):
            _dev_tensor(name, t, torch.float32, shp, device=q.device)
    outs = state_out if state_out is not None else (None,) * 4
    p = _params(q, mini_batch, eps, layer_norm, residual, state0_per_batch)
    with torch.cuda.device(q.device):   # the library launches on the current device
        rc = _lib.lib().ttt_mlp_forward(ctypes.byref(p), int(m), _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(eta), _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2),
                                        _ptr(ln_gamma), _ptr(ln_beta), _ptr(z),
                                        *[_ptr(t) for t in outs], _stream(q, stream))
    _lib.check("ttt_mlp_forward", rc)
    return z, state_out


def ttt_input_projection(x: torch.Tensor, w_in: torch.Tensor, b_eta: torch.Tensor, *,
                         heads: int, eta_base: float, head_dim: int = 64,
                         out=None, stream=None) -> Tuple[torch.Tensor, ...]:
    """The input side of a TTT layer on the GPU: from x [B,T,D] (bf16) and
    the stacked weights w_in [3*H*d + H, D] (bf16; theta_Q, theta_K, theta_V
    rows of every head, then one gate row per head) and b_eta [H] (fp32),
    returns (q, k, v, eta): q, k, v [B,H,T,d] bf16 in the scan's layout and
    eta = eta_base * sigmoid(x . w_gate + b_eta) [B,H,T] fp32.  out: an
    optional tuple of four tensors to write instead.  See include/ttt.h."""
    _dev_tensor("x", x, torch.bfloat16)
    if x.dim() != 3:
        raise ValueError("x must be [B, T, D]")
    B, T, D = x.shape
    H, d = int(heads), int(head_dim)
    dev = x.device
    _dev_tensor("w_in", w_in, torch.bfloat16, (3 * H * d + H, D), device=dev)
    _dev_tensor("b_eta", b_eta, torch.float32, (H,), device=dev)
    if out is None:
        q, k, v = (torch.empty((B, H, T, d), dtype=torch.bfloat16, device=dev) for _ in range(3))
        eta = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    else:
        q, k, v, eta = out
        for name, t in (("q", q), ("k", k), ("v", v)):
            _dev_tensor(name, t, torch.bfloat16, (B, H, T, d), device=dev)
        _dev_tensor("eta", eta, torch.float32, (B, H, T), device=dev)
    p = _lib.TTTParams(B, H, T, d, 16, _lib.TTT_BF16, 0, 1e-6, 0)
    with torch.cuda.device(dev):
        rc = _lib.lib().ttt_input_projection(
            ctypes.byref(p), D, _ptr(x), _ptr(w_in), _ptr(b_eta), float(eta_base), _ptr(q),
            _ptr(k), _ptr(v), _ptr(eta), _stream(x, stream))
    _lib.check("ttt_input_projection", rc)
    return q, k, v, eta
