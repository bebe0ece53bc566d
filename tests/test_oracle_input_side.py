"""Pins of the input-side oracle (oracle/input_side.py): the projections
that make q, k, v from the layer input and the learning-rate gate.

The oracle is a matrix product and a logistic function; it is pinned to
values that do not come from it: a hand-worked example, selection weights
whose products are slices of x, the logistic function's special values and
symmetry, and, so that a plausible slip in the layout is caught, a set of
planted mistakes that must each fail one of these pins."""
import json
import math
import os

import numpy as np
import pytest

from oracle.input_side import input_side

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "input_side_d2.json")


def _golden():
    with open(GOLDEN) as f:
        g = json.load(f)
    x = np.array(g["x"], np.float64)[None]
    return g, x


def pin_golden(fn):
    g, x = _golden()
    q, k, v, eta = fn(x, np.array(g["w_in"]), np.array(g["b_eta"]), g["H"], g["d"],
                      g["eta_base"])
    for name, got in (("q", q), ("k", k), ("v", v)):
        np.testing.assert_allclose(got[0, 0], np.array(g[name]), rtol=0, atol=1e-15,
                                   err_msg=name)
    want = [g["eta_base"] / (1.0 + math.exp(-p)) for p in g["eta_pre"]]
    np.testing.assert_allclose(eta[0, 0], want, rtol=1e-15, atol=0)


def pin_selection(fn):
    """Rows of w_in that are unit vectors pick features of x: with H = 2,
    d = 3, D = 20, row r of the q/k/v block selects feature (7 r + 3) mod 20,
    so q[b, h, t, f] = x[b, t, (7 (h d + f) + 3) mod 20] exactly."""
    rng = np.random.default_rng(11)
    B, T, D, H, d = 2, 5, 20, 2, 3
    x = rng.standard_normal((B, T, D))
    w = np.zeros((3 * H * d + H, D))
    for r in range(3 * H * d):
        w[r, (7 * r + 3) % D] = 1.0
    q, k, v, _ = fn(x, w, np.zeros(H), H, d, 1.0)
    for i, out in enumerate((q, k, v)):
        for h in range(H):
            for f in range(d):
                r = i * H * d + h * d + f
                np.testing.assert_array_equal(out[:, h, :, f], x[:, :, (7 * r + 3) % D])


def pin_gate(fn):
    """eta = eta_base / 2 exactly where the pre-activation is 0; the gate of
    the negated weights and bias is eta_base minus the gate; eta tends to
    eta_base for a large positive bias and to 0 for a large negative one;
    per head, head h's own row and bias only."""
    rng = np.random.default_rng(12)
    B, T, D, H, d = 2, 7, 16, 3, 2
    x = rng.standard_normal((B, T, D))
    w = rng.standard_normal((3 * H * d + H, D))
    b = rng.standard_normal(H)
    w0 = w.copy()
    w0[3 * H * d:] = 0.0
    eta = fn(x, w0, np.zeros(H), H, d, 0.3)[3]
    np.testing.assert_array_equal(eta, np.full((B, H, T), 0.15))
    e1 = fn(x, w, b, H, d, 0.3)[3]
    wn = w.copy()
    wn[3 * H * d:] *= -1
    e2 = fn(x, wn, -b, H, d, 0.3)[3]
    np.testing.assert_allclose(e1 + e2, 0.3, rtol=0, atol=1e-15)
    big = fn(x, w0, np.array([40.0, -40.0, 0.0]), H, d, 0.3)[3]
    assert np.all(np.abs(big[:, 0] - 0.3) < 1e-15) and np.all(big[:, 1] < 1e-17)
    # head h's gate from row 3Hd + h and b[h] only: one head's row changed
    w3 = w.copy()
    w3[3 * H * d + 1] += 1.0
    e3 = fn(x, w3, b, H, d, 0.3)[3]
    np.testing.assert_array_equal(e3[:, [0, 2]], e1[:, [0, 2]])
    assert not np.allclose(e3[:, 1], e1[:, 1])


PINS = (pin_golden, pin_selection, pin_gate)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_meets_pin(pin):
    pin(input_side)


# ---- planted mistakes: each must fail at least one pin --------------------------

def _heads_mistake(order):
    def fn(x, w_in, b_eta, H, d, eta_base):
        x = np.asarray(x, np.float64)
        W = np.asarray(w_in, np.float64)
        B, T, D = x.shape
        Y = x @ W.T
        blocks = [Y[..., i * H * d:(i + 1) * H * d] for i in range(3)]
        if order == "feature-major":        # columns read as [d, H] instead of [H, d]
            hs = [b.reshape(B, T, d, H).transpose(0, 3, 1, 2) for b in blocks]
        else:
            hs = [b.reshape(B, T, H, d).transpose(0, 2, 1, 3) for b in blocks]
        if order == "q-k swapped":
            hs = [hs[1], hs[0], hs[2]]
        pre = Y[..., 3 * H * d:] + np.asarray(b_eta)
        if order == "no bias":
            pre = Y[..., 3 * H * d:]
        eta = eta_base / (1 + np.exp(-pre))
        if order == "no base rate":
            eta = 1 / (1 + np.exp(-pre))
        if order == "softplus gate":
            eta = eta_base * np.log1p(np.exp(pre))
        if order == "gate rows off by one":   # pre-activation from rows 3Hd - 1 + h
            pre = Y[..., 3 * H * d - 1:3 * H * d - 1 + H] + np.asarray(b_eta)
            eta = eta_base / (1 + np.exp(-pre))
        return hs[0], hs[1], hs[2], eta.transpose(0, 2, 1)
    return fn


@pytest.mark.parametrize("mistake", ["feature-major", "q-k swapped", "no bias", "no base rate",
                                     "softplus gate", "gate rows off by one"])
def test_pins_catch_planted_mistakes(mistake):
    fn = _heads_mistake(mistake)
    caught = []
    for pin in PINS:
        try:
            pin(fn)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, mistake


def test_scan_consumes_the_projected_inputs():
    """Composition: the scan oracle run on the projected q, k, v, eta equals
    the scan oracle run on the same arrays built by explicit per-token,
    per-head dot products (the layout seen from the scan's side)."""
    import oracle
    rng = np.random.default_rng(13)
    B, T, D, H, d = 1, 20, 8, 2, 64
    x = rng.standard_normal((B, T, D))
    w = rng.standard_normal((3 * H * d + H, D)) / 8
    b = rng.standard_normal(H)
    q, k, v, eta = input_side(x, w, b, H, d, 1.0 / d)
    qq = np.empty((B, H, T, d))
    ee = np.empty((B, H, T))
    for h in range(H):
        for t in range(T):
            for f in range(d):
                qq[0, h, t, f] = sum(x[0, t, j] * w[h * d + f, j] for j in range(D))
            s = sum(x[0, t, j] * w[3 * H * d + h, j] for j in range(D)) + b[h]
            ee[0, h, t] = (1.0 / d) / (1.0 + math.exp(-s))
    np.testing.assert_allclose(q, qq, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(eta, ee, rtol=1e-12, atol=0)
    w0 = 0.02 * rng.standard_normal((H, d, d))
    gamma, beta = np.ones((H, d)), np.zeros((H, d))
    z1, _ = oracle.linear(q, k, v, eta, w0, gamma, beta)
    z2, _ = oracle.linear(qq, k, v, ee, w0, gamma, beta)
    np.testing.assert_allclose(z1, z2, rtol=1e-10, atol=1e-12)
