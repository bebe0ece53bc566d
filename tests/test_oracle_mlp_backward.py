"""Pins of the TTT-MLP backward oracle (oracle.backward.mlp_backward) to
things other than itself.

* Central differences (Richardson-extrapolated, fp64) of the C oracle's
  forward, taken token by token through oracle.mlp_decode_step (whose loop
  equals the scan, tests/test_oracle_mlp.py), along random directions for
  every input class (q, k, v, eta, the four state tensors, gamma, beta),
  every flag combination, ragged lengths, a shared and a per-batch initial
  state, with and without a cotangent on the final state.
* eta = 0: the state never moves, so k and v get no gradient, and the rest
  is the gradient of z_t = q_t + LN(GELU(q_t W1 + b1) W2 + b2) at the
  initial state, written out here with numpy and math.erf.
"""
import math

import numpy as np
import pytest

import oracle
from oracle.backward import mlp_backward

NAMES = ("q", "k", "v", "eta", "w1", "b1", "w2", "b2", "gamma", "beta")
STATE = ("w1", "b1", "w2", "b2")


def _problem(rng, B, H, T, d, m, per_batch=False):
    q, k, v = (rng.standard_normal((B, H, T, d)) / np.sqrt(d) for _ in range(3))
    eta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, T)))) / d * 4
    lead = (B, H) if per_batch else (H,)
    x = dict(q=q, k=k, v=v, eta=eta,
             w1=rng.standard_normal(lead + (d, m)) * 0.4,
             b1=rng.standard_normal(lead + (m,)) * 0.2,
             w2=rng.standard_normal(lead + (m, d)) * 0.4,
             b2=rng.standard_normal(lead + (d,)) * 0.2,
             gamma=1.0 + 0.3 * rng.standard_normal((H, d)),
             beta=0.3 * rng.standard_normal((H, d)))
    return x


def _objective(x, dz, dST, b, ln, res, eps, per_batch):
    """L = sum <dz, z> + <dS_T, S_T> from the fp64 C oracle, token by token."""
    B, H, T, d = x["q"].shape
    L = 0.0
    for bi in range(B):
        for h in range(H):
            S = tuple(x[n][bi, h] if per_batch else x[n][h] for n in STATE)
            Sb = None
            for t in range(T):
                z, S, Sb = oracle.mlp_decode_step(
                    S, Sb, x["q"][bi, h, t], x["k"][bi, h, t], x["v"][bi, h, t],
                    x["eta"][bi, h, t], x["gamma"][h], x["beta"][h], pos=t % b,
                    layer_norm=ln, residual=res, eps=eps)
                L += float(dz[bi, h, t] @ z)
            if dST is not None:
                L += sum(float((c[bi, h] * s).sum()) for c, s in zip(dST, S))
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
@pytest.mark.parametrize("b,T,per_batch,final", [(4, 11, False, True), (16, 19, True, False),
                                                 (3, 7, False, False)])
def test_mlp_backward_matches_central_differences(ln, res, b, T, per_batch, final):
    rng = np.random.default_rng(2000 + 7 * b + T + 2 * ln + res)
    B, H, d, m = 2, 2, 6, 12
    x = _problem(rng, B, H, T, d, m, per_batch)
    dz = rng.standard_normal((B, H, T, d))
    dST = tuple(rng.standard_normal((B, H) + x[n].shape[-(2 if n[0] == "w" else 1):])
                for n in STATE) if final else None
    eps = 1e-5
    g = mlp_backward(*(x[n] for n in NAMES), dz, dST, mini_batch=b, layer_norm=ln,
                     residual=res, eps=eps, state0_per_batch=per_batch)
    kw = dict(dz=dz, dST=dST, b=b, ln=ln, res=res, eps=eps, per_batch=per_batch)
    for name in NAMES:
        grad = g["d" + name]
        assert grad.shape == x[name].shape, name
        if name in ("gamma", "beta") and not ln:
            assert not grad.any()
            continue
        for trial in range(2):
            D = rng.standard_normal(x[name].shape)
            fd = _directional(x, name, D, 1e-4, **kw)
            an = float((grad * D).sum())
            scale = np.linalg.norm(grad) * np.linalg.norm(D)
            assert abs(fd - an) <= 1e-7 * max(scale, 1e-3), (name, trial, fd, an)


def _ln_fwd(h, gamma, beta, eps):
    mu = h.mean(-1, keepdims=True)
    sig = np.sqrt(((h - mu) ** 2).mean(-1, keepdims=True) + eps)
    xh = (h - mu) / sig
    return xh * gamma + beta, xh, sig


def test_mlp_backward_eta_zero_closed_form():
    rng = np.random.default_rng(7)
    B, H, T, d, m = 1, 2, 9, 6, 12
    x = _problem(rng, B, H, T, d, m)
    x["eta"] = np.zeros((B, H, T))
    dz = rng.standard_normal((B, H, T, d))
    g = mlp_backward(*(x[n] for n in NAMES), dz, mini_batch=4)
    assert not g["dk"].any() and not g["dv"].any()
    erf = np.vectorize(math.erf)
    for h in range(H):
        Q, DZ, gam = x["q"][0, h], dz[0, h], x["gamma"][h]
        W1, b1, W2, b2 = (x[n][h] for n in STATE)
        P = Q @ W1 + b1
        Phi = 0.5 * (1 + erf(P / math.sqrt(2)))
        A = P * Phi                                      # GELU
        dgelu = Phi + P * np.exp(-0.5 * P * P) / math.sqrt(2 * math.pi)
        _, xh, sig = _ln_fwd(A @ W2 + b2, gam, x["beta"][h], 1e-6)
        a = DZ * gam
        DO = (a - a.mean(-1, keepdims=True) - xh * (a * xh).mean(-1, keepdims=True)) / sig
        DP = (DO @ W2.T) * dgelu
        want = {"dq": DZ + DP @ W1.T, "dw1": Q.T @ DP, "db1": DP.sum(0), "dw2": A.T @ DO,
                "db2": DO.sum(0), "dgamma": (DZ * xh).sum(0), "dbeta": DZ.sum(0)}
        for name, w in want.items():
            got = g[name][0, h] if name == "dq" else g[name][h]
            np.testing.assert_allclose(got, w, rtol=1e-10, atol=1e-12, err_msg=name)
