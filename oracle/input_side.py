"""fp64 CPU oracle of the input side of a TTT layer: the projections that
make q, k and v from the layer input, and the token-dependent learning rate.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this module.  It shares no
code with the GPU path (``linear_rnn_ttt_amd``) and never imports it.

What it computes.  The outer loop trains the projections theta_K, theta_V,
theta_Q that turn the layer input into the inner loop's keys, values and
queries, and the learning rate eta is learned and depends on the token
(dmarx.github.io record LIT-801, "Key takeaways" item 2; the nowfound.app
launch page, "In the maker's words", names the QKV projection matrices).
Per token x_t [D] and head h:

    q_t^h = x_t theta_Q^h,  k_t^h = x_t theta_K^h,  v_t^h = x_t theta_V^h   (d each)
    eta_t^h = eta_base * sigmoid(x_t . theta_eta^h + b_eta^h)

Readings where the pages are silent: the projections are linear maps with
no bias (the pages name matrices); the gate is a per-head sigmoid of a
linear function of x_t scaled by a base rate, so eta stays in (0, eta_base)
-- the pages give no formula for it, and this is the plainest form that is
learned, token dependent and positive.  Stacked weight layout (the GPU
entry point takes the same): w_in [3 H d + H, D], rows h d .. h d + d - 1 =
theta_Q^h transposed, then theta_K, theta_V in the same order, then row
3 H d + h = theta_eta^h.

The definition is a matrix product and a logistic function; the oracle is
that definition in fp64 numpy.  Pinned in tests/test_oracle_input_side.py
by a hand-worked example (tests/golden/input_side_d2.json), selection
weights that reproduce slices of x exactly, the logistic function's special
values and symmetry, and the composition with the scan oracle.
"""
from __future__ import annotations

import numpy as np


def input_side(x, w_in, b_eta, H, d, eta_base):
    """x [B,T,D], w_in [3Hd+H, D], b_eta [H] -> q, k, v [B,H,T,d] and
    eta [B,H,T], all fp64."""
    x = np.asarray(x, np.float64)
    W = np.asarray(w_in, np.float64)
    B, T, D = x.shape
    if W.shape != (3 * H * d + H, D):
        raise ValueError("w_in must be [3 H d + H, D]")
    Y = x @ W.T                                             # [B, T, 3Hd + H]

    def heads(i):
        return np.ascontiguousarray(
            Y[..., i * H * d:(i + 1) * H * d].reshape(B, T, H, d).transpose(0, 2, 1, 3))

    pre = Y[..., 3 * H * d:] + np.asarray(b_eta, np.float64)   # [B, T, H]
    eta = float(eta_base) / (1.0 + np.exp(-pre))
    return heads(0), heads(1), heads(2), np.ascontiguousarray(eta.transpose(0, 2, 1))
