"""Pins of the fp64 oracle (TTT-MLP) against what the pages and the
mathematics fix, independently of the oracle's own code.

Sources: codewithpapers.app record of arXiv 2407.04620, "abstract" (the
hidden state of TTT-MLP is a two-layer MLP); dmarx.github.io record
LIT-801, "Key takeaways" items 1, 2 and 5 (update/output rules, loss,
mini-batch b = 16, LayerNorm and residual in f).  Hidden width 4d and GELU
are the workload's choice, not the pages'.

Independent references: torch autograd with F.gelu (exact erf) and
F.layer_norm in fp64, Richardson-extrapolated central differences, closed
forms (eta = 0) and structural invariants.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def _f_torch(x, S, gamma, beta, ln=True, res=True, eps=1e-6):
    W1, b1, W2, b2 = S
    o = F.gelu(x @ W1 + b1, approximate="none") @ W2 + b2
    y = F.layer_norm(o, (o.shape[-1],), gamma, beta, eps) if ln else o
    return (x if res else 0) + y


def _grad_torch(S, k, v, gamma, beta, ln=True, res=True, eps=1e-6):
    S = [s.detach().clone().requires_grad_(True) for s in S]
    loss = ((_f_torch(k, S, gamma, beta, ln, res, eps) - v) ** 2).sum()
    return torch.autograd.grad(loss, S)


def _scan_torch(q, k, v, eta, S0, gamma, beta, b, ln=True, res=True):
    T = q.shape[0]
    S = [s.clone() for s in S0]
    z = torch.empty_like(q)
    for t0 in range(0, T, b):
        Sb = [s.clone() for s in S]
        for t in range(t0, min(t0 + b, T)):
            g = _grad_torch(Sb, k[t], v[t], gamma, beta, ln, res)
            S = [s - eta[t] * gi for s, gi in zip(S, g)]
            z[t] = _f_torch(q[t], S, gamma, beta, ln, res)
    return z, S


def _problem(rng, B=1, H=1, T=20, d=8, m=32, ws=0.3):
    q, k, v = (rng.standard_normal((B, H, T, d)).astype(np.float32) for _ in range(3))
    eta = (0.02 + 0.05 * rng.random((B, H, T))).astype(np.float32)
    w1 = (ws * rng.standard_normal((H, d, m))).astype(np.float32)
    b1 = (0.1 * rng.standard_normal((H, m))).astype(np.float32)
    w2 = (ws * rng.standard_normal((H, m, d))).astype(np.float32)
    b2 = (0.1 * rng.standard_normal((H, d))).astype(np.float32)
    gamma = (1 + 0.2 * rng.standard_normal((H, d))).astype(np.float32)
    beta = (0.2 * rng.standard_normal((H, d))).astype(np.float32)
    return q, k, v, eta, w1, b1, w2, b2, gamma, beta


def _close(a, b, rel):
    b = np.asarray(b)
    return np.abs(np.asarray(a) - b).max() <= rel * max(1e-300, np.abs(b).max())


def test_gelu_is_exact_erf_gelu():
    """With W1 = W2 = I, zero biases, no LN and no residual, f(x) = GELU(x)."""
    d = 16
    x = np.linspace(-6, 6, d)
    out = oracle.mlp_apply(np.eye(d), np.zeros(d), np.eye(d), np.zeros(d), x,
                           layer_norm=False, residual=False)
    ref = F.gelu(_t(x), approximate="none").numpy()
    assert _close(out, ref, 1e-15)
    assert out[np.argmin(np.abs(x))] == pytest.approx(ref[np.argmin(np.abs(x))], abs=1e-16)


@pytest.mark.parametrize("ln,res", [(True, True), (False, False)])
def test_mlp_grad_richardson_finite_differences(ln, res):
    rng = np.random.default_rng(61)
    d, m = 6, 12
    S = [0.4 * rng.standard_normal((d, m)), 0.1 * rng.standard_normal(m),
         0.4 * rng.standard_normal((m, d)), 0.1 * rng.standard_normal(d)]
    k, v = rng.standard_normal(d), rng.standard_normal(d)
    gamma, beta = 1 + 0.2 * rng.standard_normal(d), 0.2 * rng.standard_normal(d)
    kw = dict(layer_norm=ln, residual=res)
    _, g = oracle.mlp_loss_grad(*S, k, v, gamma, beta, **kw)

    def loss_at(S2):
        return oracle.mlp_loss_grad(*S2, k, v, gamma, beta, grad=False, **kw)[0]

    def central(p, idx, h):
        Sp = [s.copy() for s in S]
        Sm = [s.copy() for s in S]
        Sp[p][idx] += h
        Sm[p][idx] -= h
        return (loss_at(Sp) - loss_at(Sm)) / (2 * h)

    h = 1e-4
    for p in range(4):
        fd = np.zeros_like(S[p])
        for idx in np.ndindex(S[p].shape):
            fd[idx] = (4 * central(p, idx, h / 2) - central(p, idx, h)) / 3
        assert _close(g[p], fd, 1e-8), p


def test_mlp_loss_and_grad_match_autograd():
    rng = np.random.default_rng(62)
    d, m = 8, 32
    S = [0.3 * rng.standard_normal((d, m)), 0.1 * rng.standard_normal(m),
         0.3 * rng.standard_normal((m, d)), 0.1 * rng.standard_normal(d)]
    k, v = rng.standard_normal(d), rng.standard_normal(d)
    gamma, beta = 1 + 0.2 * rng.standard_normal(d), 0.2 * rng.standard_normal(d)
    loss, g = oracle.mlp_loss_grad(*S, k, v, gamma, beta)
    St = [_t(s) for s in S]
    gt = _grad_torch(St, _t(k), _t(v), _t(gamma), _t(beta))
    lt = ((_f_torch(_t(k), St, _t(gamma), _t(beta)) - _t(v)) ** 2).sum().item()
    assert abs(loss - lt) <= 1e-13 * abs(lt)
    for a, b in zip(g, gt):
        assert _close(a, b.numpy(), 1e-12)


@pytest.mark.parametrize("b", [1, 4, 20])
def test_mlp_scan_matches_autograd_scan(b):
    """b = 1 is online GD, b = T (20) batch GD, b = 4 the mini-batch rule."""
    rng = np.random.default_rng(63)
    q, k, v, eta, w1, b1, w2, b2, gamma, beta = _problem(rng, T=20)
    z, S = oracle.mlp(q, k, v, eta, w1, b1, w2, b2, gamma, beta, mini_batch=b)
    zt, St = _scan_torch(_t(q[0, 0]), _t(k[0, 0]), _t(v[0, 0]), _t(eta[0, 0]),
                         [_t(w1[0]), _t(b1[0]), _t(w2[0]), _t(b2[0])], _t(gamma[0]),
                         _t(beta[0]), b)
    assert _close(z[0, 0], zt.numpy(), 1e-12)
    for a, s in zip(S, St):
        assert _close(a[0, 0], s.numpy(), 1e-12)


def test_mlp_eta_zero_closed_form():
    rng = np.random.default_rng(64)
    q, k, v, eta, w1, b1, w2, b2, gamma, beta = _problem(rng, B=2, H=2, T=12)
    eta[:] = 0
    z, S = oracle.mlp(q, k, v, eta, w1, b1, w2, b2, gamma, beta, mini_batch=4)
    for bb in range(2):
        for h in range(2):
            zt = _f_torch(_t(q[bb, h]), [_t(w1[h]), _t(b1[h]), _t(w2[h]), _t(b2[h])],
                          _t(gamma[h]), _t(beta[h]))
            assert _close(z[bb, h], zt.numpy(), 1e-13)
            np.testing.assert_array_equal(S[0][bb, h], w1[h].astype(np.float64))
            np.testing.assert_array_equal(S[3][bb, h], b2[h].astype(np.float64))


def test_mlp_gamma_zero_freezes_state():
    """gamma = 0 makes LN(o) = beta for every input, so the loss has no
    gradient with respect to the state: the state stays S0 and z = q + beta
    (closed form, LN and residual as in "Key takeaways" item 5)."""
    rng = np.random.default_rng(66)
    q, k, v, eta, w1, b1, w2, b2, gamma, beta = _problem(rng, B=1, H=2, T=20)
    gamma[:] = 0
    z, S = oracle.mlp(q, k, v, eta, w1, b1, w2, b2, gamma, beta, mini_batch=4)
    for h in range(2):
        for got, s0 in zip(S, (w1, b1, w2, b2)):
            np.testing.assert_array_equal(got[0, h], s0[h].astype(np.float64))
        np.testing.assert_allclose(z[0, h], q[0, h].astype(np.float64) + beta[h][None].astype(np.float64),
                                   rtol=0, atol=1e-15)


def test_mlp_segment_split_and_permutation():
    rng = np.random.default_rng(65)
    q, k, v, eta, w1, b1, w2, b2, gamma, beta = _problem(rng, B=2, H=2, T=16)
    z, S = oracle.mlp(q, k, v, eta, w1, b1, w2, b2, gamma, beta, mini_batch=4)
    z1, S1 = oracle.mlp(q[:, :, :8], k[:, :, :8], v[:, :, :8], eta[:, :, :8], w1, b1, w2,
                        b2, gamma, beta, mini_batch=4)
    np.testing.assert_array_equal(z1, z[:, :, :8])
    z2, S2 = oracle.mlp(q[:, :, 8:], k[:, :, 8:], v[:, :, 8:], eta[:, :, 8:],
                        *[s.astype(np.float32) for s in S1], gamma, beta, mini_batch=4,
                        state0_per_batch=True)
    assert _close(z2, z[:, :, 8:], 1e-5)
    p = [1, 0]
    zp, _ = oracle.mlp(q[:, p], k[:, p], v[:, p], eta[:, p], w1[p], b1[p], w2[p], b2[p],
                       gamma[p], beta[p], mini_batch=4)
    np.testing.assert_array_equal(zp, z[:, p])


def test_mlp_ragged_tail_equals_zero_eta_padding():
    rng = np.random.default_rng(66)
    q, k, v, eta, w1, b1, w2, b2, gamma, beta = _problem(rng, T=13)
    z, S = oracle.mlp(q, k, v, eta, w1, b1, w2, b2, gamma, beta, mini_batch=4)
    pad = lambda x, val: np.concatenate(
        [x, np.full(x.shape[:2] + (3,) + x.shape[3:], val, x.dtype)], axis=2)
    rz, rS = oracle.mlp(pad(q, 0.5), pad(k, 0.25), pad(v, -1.0), pad(eta, 0.0), w1, b1, w2,
                        b2, gamma, beta, mini_batch=4)
    np.testing.assert_array_equal(z, rz[:, :, :13])
    for a, b in zip(S, rS):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("b,ln,res", [(16, True, True), (4, True, True), (1, False, True),
                                      (5, True, False)])
def test_mlp_decode_step_loop_is_the_scan(b, ln, res):
    """The streaming step looped over a sequence (pos = t mod b) reproduces
    the oracle's scan: z of every token and the final state."""
    rng = np.random.default_rng(70 + b)
    H, T, d, m = 2, 23, 8, 32
    q, k, v = (rng.standard_normal((1, H, T, d)).astype(np.float32) for _ in range(3))
    eta = (0.1 * rng.random((1, H, T))).astype(np.float32)
    w1 = (0.3 * rng.standard_normal((H, d, m))).astype(np.float32)
    b1 = (0.1 * rng.standard_normal((H, m))).astype(np.float32)
    w2 = (0.3 * rng.standard_normal((H, m, d))).astype(np.float32)
    b2 = (0.1 * rng.standard_normal((H, d))).astype(np.float32)
    gamma = (1 + 0.2 * rng.standard_normal((H, d))).astype(np.float32)
    beta = (0.2 * rng.standard_normal((H, d))).astype(np.float32)
    kw = dict(layer_norm=ln, residual=res, eps=1e-6)
    zr, (w1r, b1r, w2r, b2r) = oracle.mlp(q, k, v, eta, w1, b1, w2, b2, gamma, beta,
                                          mini_batch=b, **kw)
    for h in range(H):
        S, Sb = (w1[h], b1[h], w2[h], b2[h]), None
        for t in range(T):
            z, S, Sb = oracle.mlp_decode_step(S, Sb, q[0, h, t], k[0, h, t], v[0, h, t],
                                              eta[0, h, t], gamma[h], beta[h], pos=t % b, **kw)
            np.testing.assert_allclose(z, zr[0, h, t], rtol=1e-12, atol=1e-12)
        for got, want in zip(S, (w1r[0, h], b1r[0, h], w2r[0, h], b2r[0, h])):
            np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
