"""Helpers shared by the GPU parity tests: device upload of the seeded
inputs, and the error metrics the tolerances are stated in.

Metrics (the tolerance is on the maximum relative error):
  * z: for every token row, max_j |z - z_ref| / max_j |z_ref|, maxed over
    rows (row-normalised, so entries near zero do not blow it up);
  * state: per unit max |S - S_ref| / max |S_ref|, maxed over units.
Tolerances: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs (fp32 state).

Conditioning.  For a few (batch, head) units of the long-context workload
the scan itself amplifies rounding along the sequence so strongly that a
plain fp32 evaluation of it (the oracle's own algorithm compiled with fp32
arithmetic, tests/_oracle_f32.py) misses the tolerance against the fp64
oracle.  Only such units may be exempted from the tolerance, and only in the
tests that allow it (strict=False); an exempted unit is still held to
FP32_MULT times the fp32 evaluation's error on that unit.  Every other unit
is held to the tolerance itself."""
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


FP32_MULT = 8.0


def per_unit(err_fn, a, b):
    """err_fn over each (batch, head) unit: [B, H] array."""
    B, H = a.shape[:2]
    return np.array([[err_fn(a[i:i + 1, j:j + 1], b[i:i + 1, j:j + 1]) for j in range(H)]
                     for i in range(B)])


def check_units(name, z, zref, z32, s, sref, s32, tol, strict=True):
    """z, s: GPU output and list of state tensors; zref, sref: the fp64
    oracle's; z32, s32: the fp32 evaluation's (z32 already rounded to the I/O
    type).  Asserts every unit's z and state error is within tol, except,
    with strict=False, on units where the fp32 evaluation itself misses tol:
    there within FP32_MULT times the fp32 evaluation's error."""
    ez = per_unit(z_err, z, zref)
    es = np.max([per_unit(state_err, a, b) for a, b in zip(s, sref)], axis=0)
    fz = per_unit(z_err, z32, zref)
    fs = np.max([per_unit(state_err, a, b) for a, b in zip(s32, sref)], axis=0)
    exempt = np.zeros(ez.shape, bool) if strict else (fz > tol) | (fs > tol)
    bz = np.where(exempt, np.maximum(tol, FP32_MULT * fz), tol)
    bs = np.where(exempt, np.maximum(tol, FP32_MULT * fs), tol)
    held = ~exempt
    print("%s: %d units, %d exempt (fp32 evaluation misses %.0e); z err max %.3e (held units "
          "%.3e, median %.3e); state err max %.3e; fp32 evaluation z err max %.3e; worst "
          "error/bound %.2f" % (
              name, ez.size, exempt.sum(), tol, ez.max(), ez[held].max() if held.any() else 0.0,
              np.median(ez), es.max(), fz.max(), max((ez / bz).max(), (es / bs).max())),
          flush=True)
    worst = np.argsort(ez.ravel())[::-1][:4]
    for u in sorted(set(worst.tolist()) | set(np.flatnonzero(exempt).tolist())):
        i, j = divmod(u, ez.shape[1])
        print("   unit (%d,%d)%s: error z %.2e state %.2e; fp32 evaluation z %.2e state %.2e"
              % (i, j, " exempt" if exempt[i, j] else "", ez[i, j], es[i, j], fz[i, j],
                 fs[i, j]), flush=True)
    assert (ez <= bz).all() and (es <= bs).all()
