"""GPU parity of the TTT-MLP backward pass (ttt_mlp_backward) against the
fp64 backward oracle (oracle.backward.mlp_backward: autograd through the
token-by-token scan, pinned by central differences of the C oracle).

Metric: per unit (per head for the batch-summed state and LN gradients),
max |got - oracle| / max |oracle| over the unit's entries, maxed over
units.  The kernel computes in fp32; bound 1e-4 for fp32 inputs and 2e-2
for bf16 inputs (whose dq, dk, dv are rounded to bf16), as for the forward.

At the full 125M-shaped workload (B8 H12 T2048) every unit is checked
against the chunked adjoint in fp64 (tests/test_chunk_form_mlp_backward.py,
itself held to the oracle at 1e-9), and two whole heads (all batch entries)
against the oracle itself."""
import numpy as np
import pytest
import torch

from linear_rnn_ttt_amd import ttt_mlp_backward
from linear_rnn_ttt_amd.inputs import WORKLOADS, make_inputs
from oracle.backward import mlp_backward

from _parity import TOL, from_dev, to_dev
from test_chunk_form_mlp_backward import chunk_backward

pytestmark = pytest.mark.gpu

MLP = WORKLOADS["mlp_125m_b8h12_t2k"]
STATE = ("w1", "b1", "w2", "b2")
NAMES = ("dq", "dk", "dv", "deta", "dw1", "db1", "dw2", "db2", "dgamma", "dbeta")
PER_TOKEN = ("dq", "dk", "dv", "deta")


def unit_err(got, want, lead):
    got = np.asarray(got, np.float64).reshape(lead + (-1,))
    want = np.asarray(want, np.float64).reshape(lead + (-1,))
    num = np.abs(got - want).max(-1)
    den = np.maximum(np.abs(want).max(-1), 1e-30)
    return num / den


def cotangents(inp, io, seed, final=True):
    B, H, T, d = inp["q"].shape
    rng = np.random.default_rng(seed)
    dz = rng.standard_normal((B, H, T, d)).astype(np.float32)
    if io == "bf16":
        dz = from_dev(to_dev(dz, "bf16"))      # the values the kernel sees
    fin = tuple((0.1 * rng.standard_normal((B, H) + inp[n].shape[-(2 if n[0] == "w" else 1):])
                 ).astype(np.float32) for n in STATE) if final else None
    return dz, fin


def gpu(inp, io, dz, fin, ln=True, res=True, eps=1e-6, per_batch=False):
    dev = {x: to_dev(inp[x], io if x in "qkv" else None) for x in
           ("q", "k", "v", "eta", "gamma", "beta") + STATE}
    out = ttt_mlp_backward(dev["q"], dev["k"], dev["v"], dev["eta"],
                           *(dev[n] for n in STATE), dev["gamma"], dev["beta"], to_dev(dz, io),
                           None if fin is None else tuple(to_dev(x) for x in fin), eps=eps,
                           layer_norm=ln, residual=res, state0_per_batch=per_batch)
    torch.cuda.synchronize()
    return dict(zip(NAMES, (from_dev(t) for t in out)))


def errors(got, want, B, H, per_batch=False):
    e = {}
    for n in NAMES:
        lead = (B, H) if n in PER_TOKEN or (n in ("dw1", "db1", "dw2", "db2") and per_batch) \
            else (H,)
        e[n] = float(unit_err(got[n], want[n], lead).max())
    return e


@pytest.mark.parametrize("case", [
    ("f32 T=50", "f32", 50, {}),
    ("f32 T=16", "f32", 16, {}),
    ("f32 T=1", "f32", 1, {}),
    ("f32 T=15", "f32", 15, {}),
    ("f32 T=17", "f32", 17, {}),
    ("f32 T=40 no LN", "f32", 40, dict(ln=False)),
    ("f32 T=40 no residual", "f32", 40, dict(res=False)),
    ("f32 T=40 no LN, no residual", "f32", 40, dict(ln=False, res=False)),
    ("f32 T=33 per-batch state", "f32", 33, dict(per_batch=True)),
    ("f32 T=33 no final cotangent", "f32", 33, dict(final=False)),
    ("bf16 T=70", "bf16", 70, {}),
    ("bf16 T=48 eps=1e-5", "bf16", 48, dict(eps=1e-5)),
    ("bf16 T=33 no LN", "bf16", 33, dict(ln=False)),
], ids=lambda c: c[0])
def test_mlp_backward_matches_the_oracle(case):
    name, io, T, kw = case
    kw = dict(kw)
    final = kw.pop("final", True)
    per_batch = kw.get("per_batch", False)
    B, H = 2, 3
    inp = make_inputs(MLP.with_(io=io), B=B, H=H, T=T)
    if per_batch:
        rng = np.random.default_rng(9)
        for n in STATE:
            inp[n] = (0.02 * rng.standard_normal((B,) + inp[n].shape)).astype(np.float32)
    dz, fin = cotangents(inp, io, seed=T, final=final)
    got = gpu(inp, io, dz, fin, **kw)
    want = mlp_backward(*(inp[x] for x in ("q", "k", "v", "eta") + STATE + ("gamma", "beta")),
                        dz, fin, mini_batch=16, layer_norm=kw.get("ln", True),
                        residual=kw.get("res", True), eps=kw.get("eps", 1e-6),
                        state0_per_batch=per_batch)
    e = errors(got, want, B, H, per_batch)
    print("%s: %s" % (name, " ".join("%s %.1e" % kv for kv in e.items())), flush=True)
    for n, v in e.items():
        if n in ("dgamma", "dbeta") and not kw.get("ln", True):
            assert not got[n].any(), n
            continue
        assert v <= TOL[io], (n, v)


def test_mlp_backward_full_size_every_unit():
    """B8 H12 T2048, bf16 data: every unit against the fp64 chunked adjoint,
    heads 0 and 7 (every batch entry) against the autograd oracle."""
    w = MLP
    inp = make_inputs(w)
    B, H, T, d = inp["q"].shape
    dz, _ = cotangents(inp, "bf16", seed=2048, final=False)
    got = gpu(inp, "bf16", dz, None)
    assert all(np.isfinite(got[n]).all() for n in NAMES)
    f64 = lambda x: np.asarray(x, np.float64)
    ref = {n: np.zeros_like(got[n]) for n in NAMES}
    for h in range(H):
        S0 = tuple(f64(inp[n][h]) for n in STATE)
        for b in range(B):
            r = chunk_backward(f64(inp["q"][b, h]), f64(inp["k"][b, h]), f64(inp["v"][b, h]),
                               f64(inp["eta"][b, h]), S0, f64(inp["gamma"][h]),
                               f64(inp["beta"][h]), f64(dz[b, h]), None, 16, True, True, 1e-6)
            for n in PER_TOKEN:
                ref[n][b, h] = r[n]
            for n in ("dw1", "db1", "dw2", "db2", "dgamma", "dbeta"):
                ref[n][h] += r[n]
        print("head %d: chunked adjoint done" % h, flush=True)
    e = errors(got, ref, B, H)
    print("full size vs chunked adjoint: %s" % " ".join("%s %.1e" % kv for kv in e.items()),
          flush=True)
    for n, v in e.items():
        assert v <= TOL["bf16"], (n, v)
    for h in (0, 7):
        sub = {x: np.ascontiguousarray(inp[x][:, h:h + 1]) for x in ("q", "k", "v", "eta")}
        for x in STATE + ("gamma", "beta"):
            sub[x] = np.ascontiguousarray(inp[x][h:h + 1])
        want = mlp_backward(*(sub[x] for x in ("q", "k", "v", "eta") + STATE + ("gamma", "beta")),
                            dz[:, h:h + 1])
        gh = {n: got[n][:, h:h + 1] if n in PER_TOKEN else got[n][h:h + 1] for n in NAMES}
        eh = errors(gh, want, B, 1)
        print("head %d vs oracle: %s" % (h, " ".join("%s %.1e" % kv for kv in eh.items())),
              flush=True)
        for n, v in eh.items():
            assert v <= TOL["bf16"], (h, n, v)


def test_mlp_backward_deterministic_and_workspace_reuse():
    inp = make_inputs(MLP, B=2, H=2, T=40)
    dz, fin = cotangents(inp, "bf16", seed=5)
    a = gpu(inp, "bf16", dz, fin)
    for _ in range(9):   # ten runs in all
        b = gpu(inp, "bf16", dz, fin)
        for n in NAMES:
            assert np.array_equal(a[n], b[n]), n


def test_mlp_backward_more_units_than_compute_units():
    """B*H = 320 units (more workgroups than the GPU holds at once), bf16,
    with final-state cotangents, against the oracle."""
    B, H, T = 5, 64, 17
    inp = make_inputs(MLP, B=B, H=H, T=T)
    dz, fin = cotangents(inp, "bf16", seed=321)
    got = gpu(inp, "bf16", dz, fin)
    want = mlp_backward(*(inp[x] for x in ("q", "k", "v", "eta") + STATE + ("gamma", "beta")),
                        dz, fin)
    e = errors(got, want, B, H)
    print("B5 H64 T17: %s" % " ".join("%s %.1e" % kv for kv in e.items()), flush=True)
    for n, v in e.items():
        assert v <= TOL["bf16"], (n, v)
