"""The chunked matrix form the HIP kernels evaluate, written in fp64 numpy
and checked against the oracle's token-by-token walk.

Within a mini-batch every gradient is taken at the state held when it began
(dmarx.github.io record LIT-801, "Key takeaways" item 5: mini-batch inner
GD), and z_t sees the updates of the tokens s <= t (item 1: z_t uses W_t).
For a 16-token tile with rows k_s, q_t and per-token gradient factors g_s
this gives, exactly:

  TTT-Linear  (grad at token s is k_s^T g_s)
    x W_t = x W_base - sum_{s<=t} eta_s (x . k_s) g_s
    H_q   = Q W_base - tril(Q K^T) (eta * G)
    W    <- W_base - K^T (eta * G)
  TTT-MLP  (grads  W1: k^T g_p,  b1: g_p,  W2: a^T g_o,  b2: g_o)
    P_q = Q W1 + b1 - tril(Q K^T + 1) (eta * G_p)
    O_q = A_q W2 + b2 - tril(A_q A_k^T + 1) (eta * G_o)

and, for mini-batches of b = 16 n tokens, the gradient point W_base is kept
for n tiles while the output uses the state after each tile.
These identities are what the kernels rely on; this test pins them.
"""
import numpy as np
import pytest
from scipy.special import erf

import oracle


def _ln(h, gamma, beta, eps):
    mu = h.mean(-1, keepdims=True)
    var = ((h - mu) ** 2).mean(-1, keepdims=True)
    sig = np.sqrt(var + eps)
    xh = (h - mu) / sig
    return xh * gamma + beta, xh, sig


def _ln_bwd(gy, xh, sig, gamma):
    a = gy * gamma
    return (a - a.mean(-1, keepdims=True) - xh * (a * xh).mean(-1, keepdims=True)) / sig


def _gelu(x):
    return 0.5 * x * (1 + erf(x / np.sqrt(2)))


def _gelu_grad(x):
    return 0.5 * (1 + erf(x / np.sqrt(2))) + x * np.exp(-0.5 * x * x) / np.sqrt(2 * np.pi)


def chunk_linear(q, k, v, eta, W0, gamma, beta, b, eps, tile=16, ln=True, res=True):
    T, d = q.shape
    W = W0.copy()
    z = np.zeros_like(q)
    for m0 in range(0, T, b):
        Wb = W.copy()                                  # gradient point
        for t0 in range(m0, min(m0 + b, T), tile):
            sl = slice(t0, min(t0 + tile, T))
            Q, K, V, E = q[sl], k[sl], v[sl], eta[sl]
            Hk = K @ Wb
            if ln:
                y, xh, sig = _ln(Hk, gamma, beta, eps)
                G = _ln_bwd(2 * ((K if res else 0) + y - V), xh, sig, gamma)
            else:
                G = 2 * ((K if res else 0) + Hk - V)
            EG = E[:, None] * G
            Hq = Q @ W - np.tril(Q @ K.T) @ EG         # W: state before tile
            z[sl] = (Q if res else 0) + (_ln(Hq, gamma, beta, eps)[0] if ln else Hq)
            W = W - K.T @ EG
    return z, W


def chunk_mlp(q, k, v, eta, S0, gamma, beta, b, eps):
    W1, b1, W2, b2 = (s.copy() for s in S0)
    T, d = q.shape
    z = np.zeros_like(q)
    assert b == 16 or b >= T
    for t0 in range(0, T, b):
        sl = slice(t0, min(t0 + b, T))
        Q, K, V, E = q[sl], k[sl], v[sl], eta[sl]
        Pk = K @ W1 + b1
        Ak = _gelu(Pk)
        Ok = Ak @ W2 + b2
        y, xh, sig = _ln(Ok, gamma, beta, eps)
        Go = _ln_bwd(2 * (K + y - V), xh, sig, gamma)
        Gp = (Go @ W2.T) * _gelu_grad(Pk)
        EGp, EGo = E[:, None] * Gp, E[:, None] * Go
        Pq = Q @ W1 + b1 - np.tril(Q @ K.T + 1) @ EGp
        Aq = _gelu(Pq)
        Oq = Aq @ W2 + b2 - np.tril(Aq @ Ak.T + 1) @ EGo
        z[sl] = Q + _ln(Oq, gamma, beta, eps)[0]
        W1 = W1 - K.T @ EGp
        b1 = b1 - EGp.sum(0)
        W2 = W2 - Ak.T @ EGo
        b2 = b2 - EGo.sum(0)
    return z, (W1, b1, W2, b2)


def _inputs(rng, T, d, scale):
    q, k, v = (rng.standard_normal((1, 1, T, d)).astype(np.float32) * scale for _ in range(3))
    eta = (1 / (1 + np.exp(-rng.standard_normal((1, 1, T)))) / d).astype(np.float32)
    return q.astype(np.float32), k.astype(np.float32), v.astype(np.float32), eta


@pytest.mark.parametrize("T,b", [(100, 16), (96, 32), (70, 64), (64, 64)])
def test_linear_chunk_form_matches_oracle(T, b):
    rng = np.random.default_rng(71)
    d = 32
    q, k, v, eta = _inputs(rng, T, d, 1.0)
    w0 = (0.02 * rng.standard_normal((1, d, d))).astype(np.float32)
    gamma = (1 + 0.1 * rng.standard_normal((1, d))).astype(np.float32)
    beta = (0.1 * rng.standard_normal((1, d))).astype(np.float32)
    z, w = oracle.linear(q, k, v, eta, w0, gamma, beta, mini_batch=b)
    f = lambda a: a.astype(np.float64)
    zc, wc = chunk_linear(f(q[0, 0]), f(k[0, 0]), f(v[0, 0]), f(eta[0, 0]), f(w0[0]),
                          f(gamma[0]), f(beta[0]), b, 1e-6)
    assert np.abs(zc - z[0, 0]).max() <= 1e-12 * np.abs(z).max()
    assert np.abs(wc - w[0, 0]).max() <= 1e-12 * np.abs(w).max()


def test_linear_chunk_form_theorem1_mode():
    rng = np.random.default_rng(72)
    T, d = 64, 16
    q, k, v, _ = _inputs(rng, T, d, 1.0)
    eta = np.full((1, 1, T), 0.5, np.float32)
    w0 = np.zeros((1, d, d), np.float32)
    z, w = oracle.linear(q, k, v, eta, w0, mini_batch=T, layer_norm=False, residual=False)
    f = lambda a: a.astype(np.float64)
    zc, wc = chunk_linear(f(q[0, 0]), f(k[0, 0]), f(v[0, 0]), f(eta[0, 0]), f(w0[0]), None,
                          None, T, 1e-6, ln=False, res=False)
    assert np.abs(zc - z[0, 0]).max() <= 1e-12 * np.abs(z).max()
    assert np.abs(wc - w[0, 0]).max() <= 1e-12 * np.abs(w).max()


def test_linear_output_split_identity():
    """Q W_base - tril(QK^T)(eta G) == Q W_next + striu(QK^T)(eta G), the
    form that lets the output read the already-updated state."""
    rng = np.random.default_rng(73)
    Q, K, G, Wb = (rng.standard_normal(s) for s in ((16, 8), (16, 8), (16, 8), (8, 8)))
    E = rng.random(16)
    EG = E[:, None] * G
    Wn = Wb - K.T @ EG
    lhs = Q @ Wb - np.tril(Q @ K.T) @ EG
    rhs = Q @ Wn + np.triu(Q @ K.T, 1) @ EG
    assert np.abs(lhs - rhs).max() <= 1e-12 * np.abs(lhs).max()


def test_linear_lookahead_identity():
    """K_t W_t == K_t W_{t-1} - (K_t K_{t-1}^T)(eta G)_{t-1}: the product for
    the next tile can be formed before the current tile's gradient is known
    and corrected afterwards with a 16x16 score tile."""
    rng = np.random.default_rng(75)
    Kp, Kt, G, W = (rng.standard_normal(s) for s in ((16, 8), (16, 8), (16, 8), (8, 8)))
    E = rng.random(16)
    EG = E[:, None] * G
    Wn = W - Kp.T @ EG
    lhs = Kt @ Wn
    rhs = Kt @ W - (Kt @ Kp.T) @ EG
    assert np.abs(lhs - rhs).max() <= 1e-12 * np.abs(lhs).max()


@pytest.mark.parametrize("T", [48, 45])
def test_mlp_chunk_form_matches_oracle(T):
    rng = np.random.default_rng(74)
    d, m = 16, 64
    q, k, v, eta = _inputs(rng, T, d, 0.5)
    S0 = [(0.1 * rng.standard_normal(s)).astype(np.float32)
          for s in ((1, d, m), (1, m), (1, m, d), (1, d))]
    gamma = (1 + 0.1 * rng.standard_normal((1, d))).astype(np.float32)
    beta = (0.1 * rng.standard_normal((1, d))).astype(np.float32)
    z, S = oracle.mlp(q, k, v, eta, *S0, gamma, beta, mini_batch=16)
    f = lambda a: a.astype(np.float64)
    zc, Sc = chunk_mlp(f(q[0, 0]), f(k[0, 0]), f(v[0, 0]), f(eta[0, 0]),
                       [f(s[0]) for s in S0], f(gamma[0]), f(beta[0]), 16, 1e-6)
    assert np.abs(zc - z[0, 0]).max() <= 1e-12 * np.abs(z).max()
    for a, c in zip(S, Sc):
        assert np.abs(a[0, 0] - c).max() <= 1e-12 * max(np.abs(a).max(), 1e-30)


def compact_mlp_stream(q, k, v, eta, S0, gamma, beta, b, eps):
    """The TTT-MLP streaming step with a compact pending state, one token at a
    time in fp64, as the compact kernel keeps its books: the stream carries
    the base and one row (k, u1, a, u2) per token of the current mini-batch;
    at position 0 the rows fold into the base (zero rows at the start); the
    output adds the rank-1 terms of the rows s <= j to the base's products.
    Returns z, the base and the rows still pending."""
    W1, b1, W2, b2 = (s.copy() for s in S0)
    T, d = q.shape
    m = W1.shape[1]
    rows = np.zeros((b, 2 * d + 2 * m))
    z = np.zeros_like(q)
    for t in range(T):
        j = t % b
        if j == 0:
            K, U1 = rows[:, :d], rows[:, d:d + m]
            A, U2 = rows[:, d + m:d + 2 * m], rows[:, d + 2 * m:]
            W1, b1 = W1 + K.T @ U1, b1 + U1.sum(0)
            W2, b2 = W2 + A.T @ U2, b2 + U2.sum(0)
        p = k[t] @ W1 + b1
        a = _gelu(p)
        y, xh, sig = _ln(a @ W2 + b2, gamma, beta, eps)
        go = _ln_bwd(2 * (k[t] + y - v[t]), xh, sig, gamma)
        u1 = -eta[t] * (W2 @ go) * _gelu_grad(p)
        u2 = -eta[t] * go
        rows[j] = np.concatenate([k[t], u1, a, u2])
        R = rows[:j + 1]
        pq = q[t] @ W1 + b1 + (R[:, :d] @ q[t] + 1) @ R[:, d:d + m]
        aq = _gelu(pq)
        oq = aq @ W2 + b2 + (R[:, d + m:d + 2 * m] @ aq + 1) @ R[:, d + 2 * m:]
        z[t] = q[t] + _ln(oq, gamma, beta, eps)[0]
    return z, (W1, b1, W2, b2), rows[:(T - 1) % b + 1]


@pytest.mark.parametrize("T,b", [(45, 16), (48, 16), (23, 5), (9, 1)])
def test_mlp_compact_stream_matches_oracle(T, b):
    """The compact stream's bookkeeping (the fold at position 0, zero rows at
    the start, the pending rows at the end) reproduces the oracle's scan: z of
    every token, and the final state rebuilt from the base and pending rows."""
    rng = np.random.default_rng(75 + b)
    d, m = 16, 64
    q, k, v, eta = _inputs(rng, T, d, 0.5)
    S0 = [(0.1 * rng.standard_normal(s)).astype(np.float32)
          for s in ((1, d, m), (1, m), (1, m, d), (1, d))]
    gamma = (1 + 0.1 * rng.standard_normal((1, d))).astype(np.float32)
    beta = (0.1 * rng.standard_normal((1, d))).astype(np.float32)
    z, S = oracle.mlp(q, k, v, eta, *S0, gamma, beta, mini_batch=b)
    f = lambda a: a.astype(np.float64)
    zc, base, rows = compact_mlp_stream(f(q[0, 0]), f(k[0, 0]), f(v[0, 0]), f(eta[0, 0]),
                                        [f(s[0]) for s in S0], f(gamma[0]), f(beta[0]), b,
                                        1e-6)
    assert np.abs(zc - z[0, 0]).max() <= 1e-12 * np.abs(z).max()
    K, U1 = rows[:, :d], rows[:, d:d + m]
    A, U2 = rows[:, d + m:d + 2 * m], rows[:, d + 2 * m:]
    rebuilt = (base[0] + K.T @ U1, base[1] + U1.sum(0), base[2] + A.T @ U2,
               base[3] + U2.sum(0))
    for a, c in zip(S, rebuilt):
        assert np.abs(a[0, 0] - c).max() <= 1e-12 * max(np.abs(a).max(), 1e-30)
