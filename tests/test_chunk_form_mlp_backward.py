"""The chunked adjoint equations of the TTT-MLP scan that the HIP backward
kernel evaluates, written in fp64 numpy and checked against the backward
oracle (autograd through the token-by-token scan).

Forward, per mini-batch with base (W1, b1, W2, b2) and rows k_s, v_s, q_i,
eta_s (the dmarx.github.io record LIT-801, "Key takeaways" items 1, 2 and 5;
the inner model x + LN(GELU(x W1 + b1) W2 + b2)):

    P = K W1 + b1,  A = GELU(P),  O = A W2 + b2,   x = LN-normalised O (rho),
    t = V - beta - res K,  a = 2 gamma (gamma x - t),
    G_o = rho (a - mean(a) - x mean(a x))        (no LN: G_o = 2 (O - t0), t0 = V - res K)
    U = G_o W2^T,  G_p = U * GELU'(P)
    PQ = Q W1 + b1 - (tril(Q K^T + 1) * eta) G_p,   AQ = GELU(PQ)
    OQ = AQ W2 + b2 - (tril(AQ A^T + 1) * eta) G_o,  z = res Q + LN(OQ)
    next base: W1 - K^T (eta G_p), b1 - sum eta G_p, W2 - A^T (eta G_o), b2 - sum eta G_o

Backward with (A1, a1, A2, a2) the adjoint of the next base:

    DOq = LN backward of dz at OQ (dgamma += dz xq, dbeta += dz)
    dAQ = DOq W2^T - (tril(DOq G_o^T) * eta) A,   dPQ = dAQ * GELU'(PQ)
    dQ  = res dz + dPQ W1^T - (tril(dPQ G_p^T) * eta) K
    KA  = K A1 + a1 + triu(K Q^T + 1) dPQ          AA  = A A2 + a2 + triu(A AQ^T + 1) DOq
    GA1 = G_p A1^T + triu(G_p dPQ^T) Q             GA2 = G_o A2^T + triu(G_o DOq^T) AQ
    deta_s = -KA_s . g_p,s - AA_s . g_o,s
    dG_p = -eta KA;   dU = dG_p * GELU'(P);   dG_o = -eta AA + dU W2
    LN-gradient backward of G_o for dG_o (as for TTT-Linear) -> dO, dt, dgamma
    dV = dt,  dbeta -= dt,  dA = -eta GA2 + dO W2^T
    dP = dA * GELU'(P) + dG_p * U * GELU''(P),   GELU''(x) = phi(x) (2 - x^2)
    dK = dP W1^T - eta GA1 - res dt
    A1 <- A1 + Q^T dPQ + K^T dP,          a1 <- a1 + sum dPQ + sum dP
    A2 <- A2 + AQ^T DOq + A^T dO + dU^T G_o,   a2 <- a2 + sum DOq + sum dO
    initial-state adjoint = (A1, a1, A2, a2) after the first mini-batch.
"""
import math

import numpy as np
import pytest

from oracle.backward import mlp_backward

_erf = np.vectorize(math.erf)


def _gelu_parts(P):
    Phi = 0.5 * (1 + _erf(P / math.sqrt(2)))
    phi = np.exp(-0.5 * P * P) / math.sqrt(2 * math.pi)
    return P * Phi, Phi + P * phi, phi * (2 - P * P)      # GELU, GELU', GELU''


def _ln(O, eps):
    mu = O.mean(-1, keepdims=True)
    rho = 1 / np.sqrt(((O - mu) ** 2).mean(-1, keepdims=True) + eps)
    return (O - mu) * rho, rho


def chunk_forward_tile(S, Q, K, V, eta, gamma, beta, ln, res, eps):
    W1, b1, W2, b2 = S
    n = K.shape[0]
    P = K @ W1 + b1
    A, dA_, d2A = _gelu_parts(P)
    O = A @ W2 + b2
    if ln:
        x, rho = _ln(O, eps)
        t = V - beta - (K if res else 0)
        a = 2 * gamma * (gamma * x - t)
        ma, mx = a.mean(-1, keepdims=True), (a * x).mean(-1, keepdims=True)
        Go = rho * (a - ma - x * mx)
        lnk = (x, rho, t, a, ma, mx)
    else:
        t = V - (K if res else 0)
        Go = 2 * (O - t)
        lnk = None
    U = Go @ W2.T
    Gp = U * dA_
    e = eta[None, :]                                      # [., s]
    M1 = np.tril(Q @ K.T + 1)
    PQ = Q @ W1 + b1 - (M1 * e) @ Gp
    AQ, dAQ_, _ = _gelu_parts(PQ)
    M2 = np.tril(AQ @ A.T + 1)
    OQ = AQ @ W2 + b2 - (M2 * e) @ Go
    if ln:
        xq, rq = _ln(OQ, eps)
        Z = (Q if res else 0) + gamma * xq + beta
    else:
        xq = rq = None
        Z = (Q if res else 0) + OQ
    nxt = (W1 - K.T @ (eta[:, None] * Gp), b1 - (eta[:, None] * Gp).sum(0),
           W2 - A.T @ (eta[:, None] * Go), b2 - (eta[:, None] * Go).sum(0))
    ctx = dict(P=P, A=A, dA=dA_, d2A=d2A, O=O, lnk=lnk, Go=Go, U=U, Gp=Gp, PQ=PQ, AQ=AQ,
               dAQ=dAQ_, xq=xq, rq=rq, t=t)
    return Z, nxt, ctx


def chunk_backward(q, k, v, eta, S0, gamma, beta, dz, dST, b, ln, res, eps):
    T, d = q.shape
    bases, S = [], tuple(x.copy() for x in S0)
    for c0 in range(0, T, b):
        bases.append(S)
        sl = slice(c0, min(c0 + b, T))
        _, S, _ = chunk_forward_tile(S, q[sl], k[sl], v[sl], eta[sl], gamma, beta, ln, res, eps)
    A1, a1, A2, a2 = (np.zeros_like(x) for x in S0) if dST is None else (x.copy() for x in dST)
    dq, dk, dv = (np.zeros((T, d)) for _ in range(3))
    deta = np.zeros(T)
    dgam, dbet = np.zeros(d), np.zeros(d)
    for ci in reversed(range(len(bases))):
        c0 = ci * b
        sl = slice(c0, min(c0 + b, T))
        Q, K, V, e, DZ = q[sl], k[sl], v[sl], eta[sl], dz[sl]
        W1, b1, W2, b2 = bases[ci]
        _, _, c = chunk_forward_tile(bases[ci], Q, K, V, e, gamma, beta, ln, res, eps)
        Gp, Go, A, AQ = c["Gp"], c["Go"], c["A"], c["AQ"]
        ec = e[:, None]
        if ln:
            gdz = gamma * DZ
            dgam += (DZ * c["xq"]).sum(0)
            dbet += DZ.sum(0)
            DOq = c["rq"] * (gdz - gdz.mean(-1, keepdims=True)
                             - c["xq"] * (gdz * c["xq"]).mean(-1, keepdims=True))
        else:
            DOq = DZ.copy()
        dAQ = DOq @ W2.T - (np.tril(DOq @ Go.T) * e[None, :]) @ A
        dPQ = dAQ * c["dAQ"]
        dq[sl] = (DZ if res else 0) + dPQ @ W1.T - (np.tril(dPQ @ Gp.T) * e[None, :]) @ K
        KA = K @ A1 + a1 + np.triu(K @ Q.T + 1) @ dPQ
        AA = A @ A2 + a2 + np.triu(A @ AQ.T + 1) @ DOq
        GA1 = Gp @ A1.T + np.triu(Gp @ dPQ.T) @ Q
        GA2 = Go @ A2.T + np.triu(Go @ DOq.T) @ AQ
        deta[sl] = -(KA * Gp).sum(-1) - (AA * Go).sum(-1)
        dGp = -ec * KA
        dU = dGp * c["dA"]
        dGo = -ec * AA + dU @ W2
        if ln:
            x, rho, t, a, ma, mx = c["lnk"]
            u = dGo
            drho = (u * (a - ma - x * mx)).sum(-1, keepdims=True)
            da = rho * (u - u.mean(-1, keepdims=True) - x * (u * x).mean(-1, keepdims=True))
            dx = -rho * (mx * u + a * (u * x).mean(-1, keepdims=True)) + 2 * gamma ** 2 * da
            dt = -2 * gamma * da
            dgam += (2 * (2 * gamma * x - t) * da).sum(0)
            dO = rho * (dx - dx.mean(-1, keepdims=True) - x * (dx * x).mean(-1, keepdims=True)) \
                - drho * rho ** 2 * x / d
            dbet -= dt.sum(0)
        else:
            dO = 2 * dGo
            dt = -2 * dGo
        dv[sl] = dt
        dAk = -ec * GA2 + dO @ W2.T
        dP = dAk * c["dA"] + dGp * c["U"] * c["d2A"]
        dk[sl] = dP @ W1.T - ec * GA1 - (dt if res else 0)
        A1 = A1 + Q.T @ dPQ + K.T @ dP
        a1 = a1 + dPQ.sum(0) + dP.sum(0)
        A2 = A2 + AQ.T @ DOq + A.T @ dO + dU.T @ Go
        a2 = a2 + DOq.sum(0) + dO.sum(0)
    return dict(dq=dq, dk=dk, dv=dv, deta=deta, dw1=A1, db1=a1, dw2=A2, db2=a2, dgamma=dgam,
                dbeta=dbet)


@pytest.mark.parametrize("ln,res", [(True, True), (True, False), (False, True),
                                    (False, False)])
@pytest.mark.parametrize("b,T,final", [(4, 13, True), (16, 16, False), (5, 5, True)])
def test_chunked_adjoint_equals_oracle(ln, res, b, T, final):
    rng = np.random.default_rng(300 + b + T + 2 * ln + res)
    d, m = 6, 12
    q, k, v, dz = (rng.standard_normal((T, d)) / np.sqrt(d) for _ in range(4))
    eta = rng.random(T) * 0.5
    S0 = (rng.standard_normal((d, m)) * 0.4, rng.standard_normal(m) * 0.2,
          rng.standard_normal((m, d)) * 0.4, rng.standard_normal(d) * 0.2)
    gamma, beta = 1 + 0.3 * rng.standard_normal(d), 0.3 * rng.standard_normal(d)
    dST = tuple(rng.standard_normal(x.shape) for x in S0) if final else None
    eps = 1e-5
    got = chunk_backward(q, k, v, eta, S0, gamma, beta, dz, dST, b, ln, res, eps)
    want = mlp_backward(q[None, None], k[None, None], v[None, None], eta[None, None],
                        *(x[None] for x in S0), gamma[None], beta[None], dz[None, None],
                        None if dST is None else tuple(x[None, None] for x in dST),
                        mini_batch=b, layer_norm=ln, residual=res, eps=eps)
    for name, g in got.items():
        w = want[name]
        w = w[0, 0] if name in ("dq", "dk", "dv", "deta") else w[0]
        np.testing.assert_allclose(g, w, rtol=1e-9, atol=1e-11 * max(1.0, np.abs(w).max()),
                                   err_msg=name)
