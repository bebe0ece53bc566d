"""The chunked adjoint equations the HIP backward kernel evaluates, written in
fp64 numpy and checked against the backward oracle (autograd through the
token-by-token scan).

Forward, per mini-batch with base W and rows k_s, v_s, q_i, eta_s (the
dmarx.github.io record LIT-801, "Key takeaways" items 1, 2 and 5):

    h_s = k_s W,  x_s = LN-normalised h_s (1/sigma_s = rho_s),
    t_s = v_s - beta - res k_s,   a_s = 2 gamma (gamma x_s - t_s),
    g_s = rho_s (a_s - mean(a_s) - x_s mean(a_s x_s))        (dl/dh at the base)
    W_i = W - sum_{s<=i} eta_s k_s^T g_s,   o_i = q_i W_i
        = Q W - (tril(Q K^T) * eta) G                         (row i)
    z_i = res q_i + gamma LN(o_i) + beta;   next base = W_b.

Backward with A = the adjoint of the next base (dW_T for the last one):

    DO    = LN backward of dz (dgamma += dz x_o, dbeta += dz)
    dQ    = res dZ + DO W^T - (tril(DO G^T) * eta) K
    KA_s  = k_s A + sum_{i>=s} (q_i . k_s) do_i        (= k_s A_s)
    GA_s  = g_s A^T + sum_{i>=s} (do_i . g_s) q_i      (= g_s A_s^T)
            where A_s = A + sum_{i>=s} q_i^T do_i is the adjoint of the
            update term eta_s k_s^T g_s (with a minus sign)
    deta_s = -KA_s . g_s,   dg_s = -eta_s KA_s
    g backward (u = dg_s):
      drho = u . (a - mean a - x mean(a x))
      da   = rho (u - mean u - x mean(u x))
      dx   = -rho (mean(a x) u + a mean(u x)) + 2 gamma^2 da
      dt   = -2 gamma da,   dgamma += 2 (2 gamma x - t) da
      dh   = rho (dx - mean dx - x mean(dx x)) - drho rho^2 x / d
      (no LN: g = 2 (h - t), dh = 2u, dt = -2u)
    dv_s = dt_s,  dbeta -= dt_s,  dK = DH W^T - eta GA - res dT
    A    <- A + Q^T DO + K^T DH       (the adjoint of this mini-batch's base)
    dW0  = A after the first mini-batch.

Mini-batches of several 16-token tiles (item 3's batch GD when b >= T) are
walked tile by tile (chunk_backward_tiles): each tile's gradients are taken
at the mini-batch's base W_b, its outputs at the state W_c of the tile's
start, so h = K W_b, o = Q W_c - M1 G, dQ uses W_c^T and dK W_b^T; the
adjoint splits into A (of the running state: A <- A + Q^T DO) and B (of the
base: B <- B + K^T DH), and A <- A + B, B <- 0 at the mini-batch's first
tile.
"""
import numpy as np
import pytest

from oracle.backward import linear_backward


def _grad_rows(W, K, V, gamma, beta, ln, res, eps):
    d = W.shape[0]
    H = K @ W
    if not ln:
        t = V - (K if res else 0)
        return 2 * (H - t), None
    mu = H.mean(-1, keepdims=True)
    rho = 1 / np.sqrt(((H - mu) ** 2).mean(-1, keepdims=True) + eps)
    x = (H - mu) * rho
    t = V - beta - (K if res else 0)
    a = 2 * gamma * (gamma * x - t)
    ma, mx = a.mean(-1, keepdims=True), (a * x).mean(-1, keepdims=True)
    g = rho * (a - ma - x * mx)
    return g, (x, rho, t, a, ma, mx)


def chunk_backward(q, k, v, eta, W0, gamma, beta, dz, dWT, b, ln, res, eps):
    T, d = q.shape
    bases, W = [], W0.copy()
    for c0 in range(0, T, b):
        bases.append(W.copy())
        sl = slice(c0, min(T, c0 + b))
        G, _ = _grad_rows(W, k[sl], v[sl], gamma, beta, ln, res, eps)
        W = W - k[sl].T @ (eta[sl, None] * G)
    A = np.zeros((d, d)) if dWT is None else dWT.copy()
    dq, dk, dv = (np.zeros((T, d)) for _ in range(3))
    deta = np.zeros(T)
    dgam, dbet = np.zeros(d), np.zeros(d)
    for c, c0 in reversed(list(enumerate(range(0, T, b)))):
        W = bases[c]
        sl = slice(c0, min(T, c0 + b))
        Q, K, V, DZ, E = q[sl], k[sl], v[sl], dz[sl], eta[sl]
        G, st = _grad_rows(W, K, V, gamma, beta, ln, res, eps)
        M1 = np.tril(Q @ K.T) * E[None, :]
        O = Q @ W - M1 @ G
        if ln:
            mu = O.mean(-1, keepdims=True)
            rho_o = 1 / np.sqrt(((O - mu) ** 2).mean(-1, keepdims=True) + eps)
            xo = (O - mu) * rho_o
            dgam += (DZ * xo).sum(0)
            dbet += DZ.sum(0)
            dxo = gamma * DZ
            DO = rho_o * (dxo - dxo.mean(-1, keepdims=True)
                          - xo * (dxo * xo).mean(-1, keepdims=True))
        else:
            DO = DZ
        dq[sl] = (DZ if res else 0) + DO @ W.T - (np.tril(DO @ G.T) * E[None, :]) @ K
        KA = K @ A + np.triu(K @ Q.T) @ DO
        GA = G @ A.T + np.triu(G @ DO.T) @ Q
        deta[sl] = -(KA * G).sum(-1)
        u = -E[:, None] * KA
        if ln:
            x, rho, t, a, ma, mx = st
            drho = (u * (a - ma - x * mx)).sum(-1, keepdims=True)
            mux = (u * x).mean(-1, keepdims=True)
            da = rho * (u - u.mean(-1, keepdims=True) - x * mux)
            dx = -rho * (mx * u + a * mux) + 2 * gamma ** 2 * da
            dt = -2 * gamma * da
            dgam += (2 * (2 * gamma * x - t) * da).sum(0)
            dH = (rho * (dx - dx.mean(-1, keepdims=True) - x * (dx * x).mean(-1, keepdims=True))
                  - drho * rho ** 2 * x / d)
            dbet -= dt.sum(0)
        else:
            dH, dt = 2 * u, -2 * u
        dv[sl] = dt
        dk[sl] = dH @ W.T - E[:, None] * GA - (dt if res else 0)
        A = A + Q.T @ DO + K.T @ dH
    return dict(dq=dq, dk=dk, dv=dv, deta=deta, dw0=A, dgamma=dgam, dbeta=dbet)


@pytest.mark.parametrize("ln,res", [(True, True), (True, False), (False, True),
                                    (False, False)])
@pytest.mark.parametrize("b,T,final", [(16, 50, True), (4, 23, False), (16, 16, True),
                                       (16, 7, False)])
def test_chunk_adjoint_equals_the_oracle(ln, res, b, T, final):
    rng = np.random.default_rng(300 + b + T + 2 * ln + res)
    H, d = 1, 16
    q, k, v = (rng.standard_normal((1, H, T, d)) / np.sqrt(d) for _ in range(3))
    eta = 1 / (1 + np.exp(-rng.standard_normal((1, H, T)))) / d * 4
    w0 = 0.3 * rng.standard_normal((H, d, d))
    gamma = 1 + 0.3 * rng.standard_normal((H, d))
    beta = 0.3 * rng.standard_normal((H, d))
    dz = rng.standard_normal((1, H, T, d))
    dwT = rng.standard_normal((1, H, d, d)) if final else None
    want = linear_backward(q, k, v, eta, w0, gamma, beta, dz, dwT, mini_batch=b,
                           layer_norm=ln, residual=res, eps=1e-6)
    got = chunk_backward(q[0, 0], k[0, 0], v[0, 0], eta[0, 0], w0[0], gamma[0], beta[0],
                         dz[0, 0], None if dwT is None else dwT[0, 0], b, ln, res, 1e-6)
    for name in want:
        w = want[name].reshape(got[name].shape)
        err = np.abs(got[name] - w).max() / max(np.abs(w).max(), 1e-30)
        assert err <= 1e-11 or (not ln and name in ("dgamma", "dbeta")), (name, err)


def ulp_perturbed(x, seed):
    """x (fp32) moved by one fp32 ulp in each entry, up or down by a seeded
    sign: the smallest change of an fp32 input."""
    x = np.asarray(x, np.float32)
    up = np.random.default_rng(seed).random(x.shape) < 0.5
    return np.where(up, np.nextafter(x, np.float32(np.inf)),
                    np.nextafter(x, np.float32(-np.inf))).astype(np.float32)


def chunk_backward_tiles(q, k, v, eta, W0, gamma, beta, dz, dWT, b, ln, res, eps, tile=16):
    """The same adjoint walked in tiles of `tile` tokens inside mini-batches
    of b (a multiple of the tile), as the GPU kernel walks it."""
    T, d = q.shape
    n = b // tile
    runs, bases, W = [], [], W0.copy()
    for c, c0 in enumerate(range(0, T, tile)):
        if c % n == 0:
            Wb = W.copy()
        runs.append(W.copy())
        bases.append(Wb)
        sl = slice(c0, min(T, c0 + tile))
        G, _ = _grad_rows(Wb, k[sl], v[sl], gamma, beta, ln, res, eps)
        W = W - k[sl].T @ (eta[sl, None] * G)
    A = np.zeros((d, d)) if dWT is None else dWT.copy()
    Bm = np.zeros((d, d))
    dq, dk, dv = (np.zeros((T, d)) for _ in range(3))
    deta = np.zeros(T)
    dgam, dbet = np.zeros(d), np.zeros(d)
    for c, c0 in reversed(list(enumerate(range(0, T, tile)))):
        Wc, Wb = runs[c], bases[c]
        sl = slice(c0, min(T, c0 + tile))
        Q, K, V, DZ, E = q[sl], k[sl], v[sl], dz[sl], eta[sl]
        G, st = _grad_rows(Wb, K, V, gamma, beta, ln, res, eps)
        O = Q @ Wc - (np.tril(Q @ K.T) * E[None, :]) @ G
        if ln:
            mu = O.mean(-1, keepdims=True)
            rho_o = 1 / np.sqrt(((O - mu) ** 2).mean(-1, keepdims=True) + eps)
            xo = (O - mu) * rho_o
            dgam += (DZ * xo).sum(0)
            dbet += DZ.sum(0)
            dxo = gamma * DZ
            DO = rho_o * (dxo - dxo.mean(-1, keepdims=True)
                          - xo * (dxo * xo).mean(-1, keepdims=True))
        else:
            DO = DZ
        dq[sl] = (DZ if res else 0) + DO @ Wc.T - (np.tril(DO @ G.T) * E[None, :]) @ K
        KA = K @ A + np.triu(K @ Q.T) @ DO
        GA = G @ A.T + np.triu(G @ DO.T) @ Q
        deta[sl] = -(KA * G).sum(-1)
        u = -E[:, None] * KA
        if ln:
            x, rho, t, a, ma, mx = st
            drho = (u * (a - ma - x * mx)).sum(-1, keepdims=True)
            mux = (u * x).mean(-1, keepdims=True)
            da = rho * (u - u.mean(-1, keepdims=True) - x * mux)
            dx = -rho * (mx * u + a * mux) + 2 * gamma ** 2 * da
            dt = -2 * gamma * da
            dgam += (2 * (2 * gamma * x - t) * da).sum(0)
            dH = (rho * (dx - dx.mean(-1, keepdims=True) - x * (dx * x).mean(-1, keepdims=True))
                  - drho * rho ** 2 * x / d)
            dbet -= dt.sum(0)
        else:
            dH, dt = 2 * u, -2 * u
        dv[sl] = dt
        dk[sl] = dH @ Wb.T - E[:, None] * GA - (dt if res else 0)
        A = A + Q.T @ DO
        Bm = Bm + K.T @ dH
        if c % n == 0:
            A, Bm = A + Bm, np.zeros((d, d))
    return dict(dq=dq, dk=dk, dv=dv, deta=deta, dw0=A, dgamma=dgam, dbeta=dbet)


@pytest.mark.parametrize("ln,res", [(True, True), (False, False), (True, False)])
@pytest.mark.parametrize("b,T,tile", [(8, 23, 4), (12, 30, 4), (32, 32, 4), (64, 50, 16),
                                      (32, 50, 16)])
def test_tiled_adjoint_of_longer_minibatches_equals_the_oracle(ln, res, b, T, tile):
    rng = np.random.default_rng(700 + b + T + tile)
    H, d = 1, 16
    q, k, v = (rng.standard_normal((1, H, T, d)) / 4 for _ in range(3))
    eta = 1 / (1 + np.exp(-rng.standard_normal((1, H, T)))) / d * 4
    w0 = 0.3 * rng.standard_normal((H, d, d))
    gamma = 1 + 0.3 * rng.standard_normal((H, d))
    beta = 0.3 * rng.standard_normal((H, d))
    dz = rng.standard_normal((1, H, T, d))
    dwT = rng.standard_normal((1, H, d, d))
    want = linear_backward(q, k, v, eta, w0, gamma, beta, dz, dwT, mini_batch=b,
                           layer_norm=ln, residual=res, eps=1e-6)
    got = chunk_backward_tiles(q[0, 0], k[0, 0], v[0, 0], eta[0, 0], w0[0], gamma[0], beta[0],
                               dz[0, 0], dwT[0, 0], b, ln, res, 1e-6, tile)
    for name in want:
        w = want[name].reshape(got[name].shape)
        err = np.abs(got[name] - w).max() / max(np.abs(w).max(), 1e-30)
        assert err <= 1e-11 or (not ln and name in ("dgamma", "dbeta")), (name, err)


def test_backward_of_an_ill_conditioned_unit_moves_with_one_ulp_of_eta():
    """On unit (0,14) of the 1.3B-layer workload (B4 H32 T8192) -- the
    forward's worst-conditioned unit -- the exact (fp64) backward itself
    moves by more than 3e-4 of its scale in dk when eta moves by one fp32
    ulp (relative 6e-8), while on unit (0,0) it moves by less than 1e-6: a
    sensitivity of the method on that unit, over 300 times that of a
    well-conditioned one, which fp32 rounding anywhere in the scan excites
    as much as the ulp of eta does."""
    from linear_rnn_ttt_amd.inputs import WORKLOADS, make_inputs
    inp = make_inputs(WORKLOADS["linear_1p3b_b4h32_t8k"])
    B, H, T, d = inp["q"].shape
    rng = np.random.default_rng(42)
    dz = rng.standard_normal((B, H, T, d))
    dwT = 0.1 * rng.standard_normal((B, H, d, d))
    shift = {}
    for h in (0, 14):
        f = lambda eta: chunk_backward(
            *(np.asarray(a, np.float64) for a in (inp["q"][0, h], inp["k"][0, h],
                                                   inp["v"][0, h], eta, inp["w0"][h],
                                                   inp["gamma"][h], inp["beta"][h])),
            dz[0, h], dwT[0, h], 16, True, True, 1e-6)["dk"]
        a, b = f(inp["eta"][0, h]), f(ulp_perturbed(inp["eta"][0, h], 1))
        shift[h] = np.abs(a - b).max() / np.abs(a).max()
    assert shift[14] > 3e-4 and shift[0] < 1e-6, shift
