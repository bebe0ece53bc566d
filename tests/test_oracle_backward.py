"""Pins of the backward oracle (oracle/backward.py) to things other than itself.

* Central differences (Richardson-extrapolated, fp64) of the C oracle's
  forward, taken token by token through oracle.linear_decode_step (whose
  loop equals the scan, tests/test_oracle_linear.py), along random
  directions for every input class, every flag combination, ragged lengths,
  a shared and a per-batch initial state, with and without a cotangent on
  the final state.
* Theorem-1 mode (no LN, no residual, eta = 1/2, W0 = 0, b = T: the scan is
  causal linear attention, dmarx.github.io record LIT-801, "Key takeaways"
  item 3): every gradient has a closed form in q, k, v, dz and dW_T.
* eta = 0: the state never moves, so k and v get no gradient and the rest
  is the gradient of z_t = q_t + LN(q_t W0) in closed form.
"""
import numpy as np
import pytest

import oracle
from oracle.backward import linear_backward

NAMES = ("q", "k", "v", "eta", "w0", "gamma", "beta")


def _problem(rng, B, H, T, d, per_batch=False):
    q, k, v = (rng.standard_normal((B, H, T, d)) / np.sqrt(d) for _ in range(3))
    eta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, T)))) / d * 4
    w0 = rng.standard_normal(((B, H) if per_batch else (H,)) + (d, d)) * 0.3
    gamma = 1.0 + 0.3 * rng.standard_normal((H, d))
    beta = 0.3 * rng.standard_normal((H, d))
    return dict(q=q, k=k, v=v, eta=eta, w0=w0, gamma=gamma, beta=beta)


def _objective(x, dz, dwT, b, ln, res, eps, per_batch):
    """L = sum <dz, z> + <dW_T, W_T> from the fp64 C oracle, token by token."""
    B, H, T, d = x["q"].shape
    L = 0.0
    for bi in range(B):
        for h in range(H):
            W = x["w0"][bi, h] if per_batch else x["w0"][h]
            Wb = None
            for t in range(T):
                z, W, Wb = oracle.linear_decode_step(
                    W, Wb, x["q"][bi, h, t], x["k"][bi, h, t], x["v"][bi, h, t],
                    x["eta"][bi, h, t], x["gamma"][h], x["beta"][h], pos=t % b,
                    layer_norm=ln, residual=res, eps=eps)
                L += float(dz[bi, h, t] @ z)
            if dwT is not None:
                L += float((dwT[bi, h] * W).sum())
    return L


def _directional(x, name, D, step, **kw):
    def at(s):
        y = dict(x)
        y[name] = x[name] + s * D
        return _objective(y, **kw)
    d1 = (at(step) - at(-step)) / (2 * step)
    d2 = (at(step / 2) - at(-step / 2)) / step
    return (4 * d2 - d1) / 3


@pytest.mark.parametrize("ln,res", [(True, True), (True, False), (False, True),
                                    (False, False)])
@pytest.mark.parametrize("b,T,per_batch,final", [(4, 21, False, True), (16, 21, True, False),
                                                 (3, 10, False, False)])
def test_backward_matches_central_differences(ln, res, b, T, per_batch, final):
    rng = np.random.default_rng(1000 + 7 * b + T + 2 * ln + res)
    B, H, d = 2, 2, 8
    x = _problem(rng, B, H, T, d, per_batch)
    dz = rng.standard_normal((B, H, T, d))
    dwT = rng.standard_normal((B, H, d, d)) if final else None
    eps = 1e-5
    g = linear_backward(x["q"], x["k"], x["v"], x["eta"], x["w0"], x["gamma"], x["beta"], dz,
                        dwT, mini_batch=b, layer_norm=ln, residual=res, eps=eps,
                        state0_per_batch=per_batch)
    kw = dict(dz=dz, dwT=dwT, b=b, ln=ln, res=res, eps=eps, per_batch=per_batch)
    for name in NAMES:
        grad = g["d" + name]
        assert grad.shape == x[name].shape, name
        if name in ("gamma", "beta") and not ln:
            assert not grad.any()
            continue
        for trial in range(2):
            D = rng.standard_normal(x[name].shape)
            fd = _directional(x, name, D, 1e-3, **kw)
            an = float((grad * D).sum())
            scale = np.linalg.norm(grad) * np.linalg.norm(D)
            assert abs(fd - an) <= 1e-7 * max(scale, 1e-3), (name, trial, fd, an)


def test_backward_theorem1_closed_forms():
    rng = np.random.default_rng(5)
    T, d = 12, 6
    q, k, v, dz = (rng.standard_normal((1, 1, T, d)) for _ in range(4))
    dwT = rng.standard_normal((1, 1, d, d))
    eta = np.full((1, 1, T), 0.5)
    w0 = np.zeros((1, d, d))
    g = linear_backward(q, k, v, eta, w0, None, None, dz, dwT, mini_batch=T,
                        layer_norm=False, residual=False)
    Q, K, V, DZ, A = q[0, 0], k[0, 0], v[0, 0], dz[0, 0], dwT[0, 0]
    causal = np.tril(np.ones((T, T)))            # [t, s]: s <= t
    QK = Q @ K.T                                 # [t, s] = q_t . k_s
    DV = DZ @ V.T                                # [t, s] = dz_t . v_s
    dq = (causal * DV) @ K
    dk = (causal * DV).T @ Q + V @ A.T
    dv = (causal * QK).T @ DZ + K @ A
    deta = 2 * (causal * QK * DV).sum(0) + 2 * np.einsum("sf,fg,sg->s", K, A, V)
    P = np.cumsum(K[:, :, None] * K[:, None, :], axis=0)    # P_t = sum_{s<=t} k_s^T k_s
    I = np.eye(d)
    dw0 = sum((I - P[t]) @ np.outer(Q[t], DZ[t]) for t in range(T)) + (I - P[-1]) @ A
    for name, want in (("dq", dq), ("dk", dk), ("dv", dv), ("deta", deta), ("dw0", dw0)):
        got = g[name].reshape(want.shape)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12, err_msg=name)


def _ln_fwd(h, gamma, beta, eps):
    mu = h.mean(-1, keepdims=True)
    sig = np.sqrt(((h - mu) ** 2).mean(-1, keepdims=True) + eps)
    xh = (h - mu) / sig
    return xh * gamma + beta, xh, sig


def test_backward_eta_zero_closed_form():
    rng = np.random.default_rng(6)
    B, H, T, d = 1, 2, 9, 8
    x = _problem(rng, B, H, T, d)
    x["eta"] = np.zeros((B, H, T))
    dz = rng.standard_normal((B, H, T, d))
    g = linear_backward(*(x[n] for n in NAMES), dz, mini_batch=4)
    assert not g["dk"].any() and not g["dv"].any()
    for h in range(H):
        Q, DZ, W0, gam = x["q"][0, h], dz[0, h], x["w0"][h], x["gamma"][h]
        _, xh, sig = _ln_fwd(Q @ W0, gam, x["beta"][h], 1e-6)
        a = DZ * gam
        do = (a - a.mean(-1, keepdims=True) - xh * (a * xh).mean(-1, keepdims=True)) / sig
        np.testing.assert_allclose(g["dq"][0, h], DZ + do @ W0.T, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(g["dw0"][h], Q.T @ do, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(g["dgamma"][h], (DZ * xh).sum(0), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(g["dbeta"][h], DZ.sum(0), rtol=1e-12, atol=1e-12)
