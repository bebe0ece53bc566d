"""Seeded synthetic inputs for the TTT-layer forward scan.

This module holds no arithmetic of the method: it only draws random arrays
with the shapes and value distributions of the workloads and rounds them to
the I/O precision.  Both the GPU path's callers (tests, benchmark) and the
oracle's callers (tests) take their inputs from here.

The pages (arXiv 2407.04620 abstract on codewithpapers.app; "Key
takeaways" item 6 of the dmarx.github.io record LIT-801) evaluate language
models of 125M to 1.3B parameters at 2k to 32k context and name no dataset;
these draws stand in for the layer's projected activations:
  * head dim d = 64, heads x d = model width (12 x 64 = 768 for 125M,
    32 x 64 = 2048 for 1.3B);
  * q, k, v ~ N(0, 1) (fp32 workload) or N(0, 1) / sqrt(d) rounded to bf16;
  * eta_t = sigmoid(N(0, 1)) / d, one per token;
  * W0 (or W1, W2) ~ N(0, 0.02^2) per head, MLP biases 0;
  * LN gamma ~ 1 + N(0, 0.1^2), beta ~ N(0, 0.1^2) per head (gamma = 1,
    beta = 0 for the fp32 workload).

Generator: ``numpy.random.default_rng(seed)`` (PCG64); standard normals
drawn in fp64 in the order q, k, v, eta-logits, state (W0 | W1 then W2),
gamma-noise, beta; each cast to fp32; bf16 tensors rounded from fp32 with
round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_inputs", "bf16_round", "bf16_bits",
           "unit_slice", "InputWorkload", "INPUT_WORKLOADS", "make_input_side"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "linear" | "mlp"
    B: int
    H: int
    T: int
    d: int
    mini_batch: int
    io: str              # "f32" | "bf16"
    seed: int
    theorem1: bool = False   # no LN, no residual, eta = 1/2, W0 = 0
    hidden: int = 256        # MLP hidden width (4d)
    eps: float = 1e-6

    @property
    def tokens(self) -> int:
        return self.B * self.T

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The workloads: a small fp32 one the oracle finishes in seconds (plus its
# Theorem-1 variant), 125M- and 1.3B-shaped layers, the 125M-shaped MLP
# layer, and the long-context shape for both inner models.
WORKLOADS: Dict[str, Workload] = {
    "linear_b1h1_t256_f32": Workload("linear_b1h1_t256_f32", "linear", 1, 1, 256, 64,
                                     16, "f32", 1),
    "theorem1_b1h1_t256_f32": Workload("theorem1_b1h1_t256_f32", "linear", 1, 1, 256,
                                       64, 256, "f32", 101, theorem1=True),
    "linear_125m_b8h12_t2k": Workload("linear_125m_b8h12_t2k", "linear", 8, 12, 2048,
                                      64, 16, "bf16", 2),
    "linear_1p3b_b4h32_t8k": Workload("linear_1p3b_b4h32_t8k", "linear", 4, 32, 8192,
                                      64, 16, "bf16", 3),
    "mlp_125m_b8h12_t2k": Workload("mlp_125m_b8h12_t2k", "mlp", 8, 12, 2048, 64, 16,
                                   "bf16", 4),
    "linear_long_b1h32_t32k": Workload("linear_long_b1h32_t32k", "linear", 1, 32,
                                       32768, 64, 16, "bf16", 5),
    "mlp_long_b1h32_t32k": Workload("mlp_long_b1h32_t32k", "mlp", 1, 32, 32768, 64, 16,
                                    "bf16", 105),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((u >> 16) & 1)
    r = ((u + bias) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16, returned as fp32."""
    return (bf16_bits(x).astype(np.uint32) << 16).view(np.float32)


def _normal(rng, shape, scale=1.0, shift=0.0):
    return (shift + scale * rng.standard_normal(shape)).astype(np.float32)


def make_inputs(w: Workload, *, T: Optional[int] = None, B: Optional[int] = None,
                H: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw the inputs of workload ``w`` (shape overrides allowed for tests).

    Returns fp32 numpy arrays holding exactly the values the scan consumes
    (bf16 workloads: already rounded).  Keys: q, k, v, eta, gamma, beta and
    w0 (linear) or w1, b1, w2, b2 (mlp)."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    T = w.T if T is None else T
    d = w.d
    rng = np.random.default_rng(w.seed)
    shape = (B, H, T, d)
    qkv_scale = 1.0 if w.io == "f32" else 1.0 / np.sqrt(d)
    out: Dict[str, np.ndarray] = {}
    for name in ("q", "k", "v"):
        x = _normal(rng, shape, qkv_scale)
        out[name] = bf16_round(x) if w.io == "bf16" else x
    if w.theorem1:
        out["eta"] = np.full((B, H, T), 0.5, np.float32)
        out["w0"] = np.zeros((H, d, d), np.float32)
        out["gamma"] = np.ones((H, d), np.float32)
        out["beta"] = np.zeros((H, d), np.float32)
        return out
    logits = rng.standard_normal((B, H, T))
    out["eta"] = (1.0 / (1.0 + np.exp(-logits)) / d).astype(np.float32)
    if w.kind == "linear":
        out["w0"] = _normal(rng, (H, d, d), 0.02)
    else:
        m = w.hidden
        out["w1"] = _normal(rng, (H, d, m), 0.02)
        out["w2"] = _normal(rng, (H, m, d), 0.02)
        out["b1"] = np.zeros((H, m), np.float32)
        out["b2"] = np.zeros((H, d), np.float32)
    if w.io == "f32":
        out["gamma"] = np.ones((H, d), np.float32)
        out["beta"] = np.zeros((H, d), np.float32)
    else:
        out["gamma"] = _normal(rng, (H, d), 0.1, 1.0)
        out["beta"] = _normal(rng, (H, d), 0.1)
    return out


def unit_slice(inp: Dict[str, np.ndarray], units, H: int) -> Dict[str, np.ndarray]:
    """Inputs of a subset of (batch, head) units as a [1, n] problem with a
    per-unit initial state (state0_per_batch layout [1, n, ...]).

    ``units`` is a list of (b, h).  Units are independent, so the outputs of
    the sliced problem equal the same units' outputs of the full one."""
    bs = [b for b, _ in units]
    hs = [h for _, h in units]
    out = {}
    for key in ("q", "k", "v", "eta"):
        out[key] = np.ascontiguousarray(inp[key][bs, hs][None])
    for key in ("w0", "w1", "b1", "w2", "b2"):
        if key in inp:
            out[key] = np.ascontiguousarray(inp[key][hs][None])
    for key in ("gamma", "beta"):
        out[key] = np.ascontiguousarray(inp[key][hs])
    return out


# ---- the input side: the layer input x and the projections that make q, k,
# v and the learning-rate gate from it ----------------------------------------
#
# Stand-ins for a trained layer's weights, scaled so that the projections
# have the statistics of the scan workloads above: x ~ N(0, 1) per feature
# (the layer input after a normalisation), rows of theta_Q, theta_K, theta_V
# ~ N(0, 1 / (D d)) so that q, k, v ~ N(0, 1/d), rows of theta_eta
# ~ N(0, 1/D) and b_eta ~ N(0, 0.1^2) so that the gate's pre-activation is
# about N(0, 1), and eta_base = 1/d (so eta = sigmoid(.) / d as above).
# Draw order: x, the q/k/v rows, the eta rows, b_eta; x and the weights are
# rounded to bf16.


@dataclasses.dataclass(frozen=True)
class InputWorkload:
    name: str
    B: int
    T: int
    D: int       # model width (the layer input's features)
    H: int
    d: int
    seed: int

    @property
    def tokens(self) -> int:
        return self.B * self.T

    @property
    def n_out(self) -> int:
        """Rows of the stacked weight: q, k, v of every head, then one eta row per head."""
        return 3 * self.H * self.d + self.H

    def with_(self, **kw) -> "InputWorkload":
        return dataclasses.replace(self, **kw)


INPUT_WORKLOADS: Dict[str, InputWorkload] = {
    "input_125m_b8_t2k": InputWorkload("input_125m_b8_t2k", 8, 2048, 768, 12, 64, 6),
    "input_1p3b_b4_t8k": InputWorkload("input_1p3b_b4_t8k", 4, 8192, 2048, 32, 64, 7),
}


def make_input_side(w: InputWorkload, *, B: Optional[int] = None, T: Optional[int] = None,
                    D: Optional[int] = None, H: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw x [B,T,D], w_in [3 H d + H, D] (rows: theta_Q of heads 0..H-1,
    d rows each, then theta_K, theta_V, then the eta row of each head),
    b_eta [H] and eta_base (a 0-d array).  x and w_in hold bf16 values (as
    fp32 arrays)."""
    B = w.B if B is None else B
    T = w.T if T is None else T
    D = w.D if D is None else D
    H = w.H if H is None else H
    d = w.d
    rng = np.random.default_rng(w.seed)
    x = bf16_round(_normal(rng, (B, T, D)))
    wq = _normal(rng, (3 * H * d, D), 1.0 / np.sqrt(D * d))
    we = _normal(rng, (H, D), 1.0 / np.sqrt(D))
    w_in = bf16_round(np.concatenate([wq, we], 0))
    b_eta = _normal(rng, (H,), 0.1)
    return {"x": x, "w_in": w_in, "b_eta": b_eta, "eta_base": np.float32(1.0 / d)}
