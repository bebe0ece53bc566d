"""Helpers shared by the GPU parity tests: device upload of the seeded
inputs, and the error metrics the tolerances are stated in.

Metrics (the tolerance is on the maximum relative error):
  * z: for every token row, max_j |z - z_ref| / max_j |z_ref|, maxed over
    rows (row-normalised, so entries near zero do not blow it up);
  * state: per unit max |S - S_ref| / max |S_ref|, maxed over units.
Tolerances: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs (fp32 state)."""
import numpy as np
import torch

TOL = {"f32": 1e-4, "bf16": 2e-2}


def to_dev(x, io=None):
    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    if io == "bf16":
        t = t.to(torch.bfloat16)
    return t


def from_dev(t):
    return t.float().cpu().numpy().astype(np.float64)


def z_err(z, zref):
    z = np.asarray(z, np.float64)
    zref = np.asarray(zref, np.float64)
    num = np.abs(z - zref).max(-1)
    den = np.maximum(np.abs(zref).max(-1), 1e-30)
    return float((num / den).max())


def state_err(s, sref):
    s = np.asarray(s, np.float64)
    sref = np.asarray(sref, np.float64)
    lead = s.shape[:2]
    d = np.abs(s - sref).reshape(lead + (-1,)).max(-1)
    m = np.maximum(np.abs(sref).reshape(lead + (-1,)).max(-1), 1e-30)
    return float((d / m).max())
