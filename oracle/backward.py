"""fp64 CPU oracle of the TTT-Linear and TTT-MLP scans' backward passes.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this module.  It shares no
code with the GPU path (``linear_rnn_ttt_amd``) and never imports it.

What it computes.  The outer loop trains the projections that make q, k and
v, the initial state W0 and the per-token learning rate eta (dmarx.github.io
record LIT-801, "Key takeaways" item 2), and the LN parameters of the inner
model f are parameters of it as well.  Training therefore needs the
vector-Jacobian product of the forward scan: for cotangents dz [B,H,T,d]
(and, optionally, dW_T [B,H,d,d] on the final state) the gradients of

    L = sum_t <dz_t, z_t> + <dW_T, W_T>

with respect to q, k, v, eta, W0, gamma and beta.  This is the plain
definition of the backward, so the oracle is that definition written out:
the forward scan of ``oracle.linear`` (items 1, 2 and 5: W_t = W_{t-1} -
eta_t grad l(W_base; k_t, v_t), every gradient of a mini-batch of b tokens
at the state the mini-batch started from, z_t = f(q_t; W_t), with
f(x; W) = x + LN(x W)) is rebuilt token by token in torch fp64 ops, each
inner gradient grad l is taken by autograd with its graph kept
(create_graph), and torch.autograd.grad differentiates L through the whole
scan.  No blocking, reordering or hand-written adjoint: the tests pin it by
central differences of the C oracle's forward and by closed forms.

``mlp_backward`` does the same for the TTT-MLP scan (inner model
f(x) = x + LN(GELU(x W1 + b1) W2 + b2), the codewithpapers.app record's
"abstract"; state S = (W1, b1, W2, b2), exact erf GELU): the gradients of
sum_t <dz_t, z_t> + <dS_T, S_T> with respect to q, k, v, eta, the initial
state and gamma, beta.
"""
from __future__ import annotations

import numpy as np
import torch


def _t(a, requires_grad=False):
    t = torch.from_numpy(np.array(a, dtype=np.float64))
    return t.requires_grad_(requires_grad)


def _layer_norm(h, gamma, beta, eps):
    """LN over the d features: biased variance, eps inside the root."""
    mu = h.mean(-1, keepdim=True)
    var = ((h - mu) ** 2).mean(-1, keepdim=True)
    return (h - mu) / torch.sqrt(var + eps) * gamma + beta


def _f(x, W, gamma, beta, layer_norm, residual, eps):
    """The inner model on a row x [..., d] with state W [..., d, d]."""
    y = (x.unsqueeze(-2) @ W).squeeze(-2)
    if layer_norm:
        y = _layer_norm(y, gamma, beta, eps)
    return x + y if residual else y


def linear_backward(q, k, v, eta, w0, gamma, beta, dz, dw_final=None, *, mini_batch=16,
                    layer_norm=True, residual=True, eps=1e-6, state0_per_batch=False):
    """Gradients of L = sum <dz, z> + <dW_T, W_T> for the TTT-Linear scan.

    q, k, v, dz [B,H,T,d]; eta [B,H,T]; w0 [H,d,d] (or [B,H,d,d] with
    state0_per_batch); gamma, beta [H,d] (ignored without LN); dw_final
    [B,H,d,d] or None (zero).  Returns a dict of fp64 arrays: dq, dk, dv
    [B,H,T,d], deta [B,H,T], dw0 in w0's shape (summed over the batch when
    w0 is shared), dgamma and dbeta [H,d] (summed over batch and tokens;
    zero without LN)."""
    B, H, T, d = np.shape(q)
    Q, K, V = _t(q, True), _t(k, True), _t(v, True)
    E = _t(eta, True)
    W0 = _t(w0, True)
    G = _t(gamma if layer_norm else np.ones((H, d)), True)
    Bt = _t(beta if layer_norm else np.zeros((H, d)), True)
    W = W0 if state0_per_batch else W0.unsqueeze(0).expand(B, H, d, d)
    f = lambda x, S: _f(x, S, G, Bt, layer_norm, residual, eps)

    z = []
    for t0 in range(0, T, mini_batch):
        W_base = W
        for t in range(t0, min(t0 + mini_batch, T)):
            loss = ((f(K[:, :, t], W_base) - V[:, :, t]) ** 2).sum()
            (grad_w,) = torch.autograd.grad(loss, W_base, create_graph=True)
            W = W - E[:, :, t, None, None] * grad_w
            z.append(f(Q[:, :, t], W))
    Z = torch.stack(z, 2)
    L = (Z * _t(dz)).sum()
    if dw_final is not None:
        L = L + (W * _t(dw_final)).sum()
    grads = torch.autograd.grad(L, [Q, K, V, E, W0, G, Bt], allow_unused=True)
    out = {}
    for name, g, like in zip(("dq", "dk", "dv", "deta", "dw0", "dgamma", "dbeta"), grads,
                             (Q, K, V, E, W0, G, Bt)):
        out[name] = (torch.zeros_like(like) if g is None else g).detach().numpy()
    if not layer_norm:
        out["dgamma"] = np.zeros((H, d))
        out["dbeta"] = np.zeros((H, d))
    return out


def _gelu(x):
    """GELU, exact erf form: x Phi(x)."""
    return 0.5 * x * (1.0 + torch.erf(x / np.sqrt(2.0)))


def _f_mlp(x, W1, b1, W2, b2, gamma, beta, layer_norm, residual, eps):
    """The TTT-MLP inner model on a row x [..., d]: x + LN(GELU(x W1 + b1) W2 + b2)."""
    a = _gelu((x.unsqueeze(-2) @ W1).squeeze(-2) + b1)
    y = (a.unsqueeze(-2) @ W2).squeeze(-2) + b2
    if layer_norm:
        y = _layer_norm(y, gamma, beta, eps)
    return x + y if residual else y


def mlp_backward(q, k, v, eta, w1, b1, w2, b2, gamma, beta, dz, dstate_final=None, *,
                 mini_batch=16, layer_norm=True, residual=True, eps=1e-6,
                 state0_per_batch=False):
    """Gradients of L = sum <dz, z> + <dS_T, S_T> for the TTT-MLP scan.

    q, k, v, dz [B,H,T,d]; eta [B,H,T]; w1 [H,d,m], b1 [H,m], w2 [H,m,d],
    b2 [H,d] (leading [B,H] with state0_per_batch); gamma, beta [H,d]
    (ignored without LN); dstate_final None or a tuple of four cotangents
    with the final state's shapes [B,H,...].  Returns a dict of fp64
    arrays: dq, dk, dv, deta, dw1, db1, dw2, db2 (the initial state's
    shapes, summed over the batch when shared), dgamma, dbeta [H,d]."""
    B, H, T, d = np.shape(q)
    Q, K, V = _t(q, True), _t(k, True), _t(v, True)
    E = _t(eta, True)
    S0 = [_t(x, True) for x in (w1, b1, w2, b2)]
    G = _t(gamma if layer_norm else np.ones((H, d)), True)
    Bt = _t(beta if layer_norm else np.zeros((H, d)), True)
    S = S0 if state0_per_batch else [x.unsqueeze(0).expand((B,) + tuple(x.shape)) for x in S0]
    f = lambda x, St: _f_mlp(x, *St, G, Bt, layer_norm, residual, eps)

    z = []
    for t0 in range(0, T, mini_batch):
        base = S
        for t in range(t0, min(t0 + mini_batch, T)):
            loss = ((f(K[:, :, t], base) - V[:, :, t]) ** 2).sum()
            grads = torch.autograd.grad(loss, base, create_graph=True)
            e = E[:, :, t]
            S = [x - e.reshape(e.shape + (1,) * (x.dim() - 2)) * gx for x, gx in zip(S, grads)]
            z.append(f(Q[:, :, t], S))
    Z = torch.stack(z, 2)
    L = (Z * _t(dz)).sum()
    if dstate_final is not None:
        for x, dx in zip(S, dstate_final):
            L = L + (x * _t(dx)).sum()
    grads = torch.autograd.grad(L, [Q, K, V, E] + S0 + [G, Bt], allow_unused=True)
    out = {}
    names = ("dq", "dk", "dv", "deta", "dw1", "db1", "dw2", "db2", "dgamma", "dbeta")
    for name, g, like in zip(names, grads, [Q, K, V, E] + S0 + [G, Bt]):
        out[name] = (torch.zeros_like(like) if g is None else g).detach().numpy()
    if not layer_norm:
        out["dgamma"] = np.zeros((H, d))
        out["dbeta"] = np.zeros((H, d))
    return out
