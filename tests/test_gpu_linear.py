"""GPU parity of the TTT-Linear scan (gfx950 kernels through the C ABI)
against the fp64 oracle on the same seeded inputs.

Small cases compare every output; the full-size workloads (125M- and
1.3B-shaped layers, 32k context) run in the configuration the benchmark
times and compare every (batch, head) unit.  Tolerances: 1e-4 max relative
error for fp32 inputs, 2e-2 for bf16 inputs."""
import numpy as np
import pytest
import torch

import oracle
from linear_rnn_ttt_amd import ttt_linear_forward
from linear_rnn_ttt_amd.inputs import WORKLOADS, bf16_round, make_inputs

import _oracle_f32
from _parity import TOL, check_units, from_dev, state_err, to_dev, z_err

pytestmark = pytest.mark.gpu


def _gpu(inp, io, **kw):
    z, w = ttt_linear_forward(to_dev(inp["q"], io), to_dev(inp["k"], io), to_dev(inp["v"], io),
                              to_dev(inp["eta"]), to_dev(inp["w0"]), to_dev(inp["gamma"]),
                              to_dev(inp["beta"]), **kw)
    torch.cuda.synchronize()
    return from_dev(z), from_dev(w)


def _oracle(inp, **kw):
    return oracle.linear(inp["q"], inp["k"], inp["v"], inp["eta"], inp["w0"], inp["gamma"],
                         inp["beta"], **kw)


def _check(name, inp, io, tol=None, **kw):
    tol = TOL[io] if tol is None else tol
    z, w = _gpu(inp, io, **kw)
    okw = {k: v for k, v in kw.items() if k in ("mini_batch", "layer_norm", "residual", "eps",
                                                 "state0_per_batch")}
    zr, wr = _oracle(inp, **okw)
    ez, ew = z_err(z, zr), state_err(w, wr)
    print("%s: z err %.3e, state err %.3e (tol %.0e)" % (name, ez, ew, tol), flush=True)
    assert ez <= tol and ew <= tol, (ez, ew)
    return z, w


def test_fp32_small_workload():
    w = WORKLOADS["linear_b1h1_t256_f32"]
    _check(w.name, make_inputs(w), "f32")


def test_theorem1_mode_is_linear_attention():
    w = WORKLOADS["theorem1_b1h1_t256_f32"]
    inp = make_inputs(w)
    z, wf = _check(w.name, inp, "f32", mini_batch=256, layer_norm=False, residual=False)
    Q, K, V = (inp[x][0, 0].astype(np.float64) for x in "qkv")
    zb = np.tril(Q @ K.T) @ V                    # z_t = sum_{s<=t} (q_t . k_s) v_s
    assert z_err(z[0, 0], zb) <= 1e-4
    assert state_err(wf, (K.T @ V)[None, None]) <= 1e-4


@pytest.mark.parametrize("T", [1, 15, 16, 17, 47, 300])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_ragged_lengths(T, io):
    base = WORKLOADS["linear_b1h1_t256_f32" if io == "f32" else "linear_125m_b8h12_t2k"]
    inp = make_inputs(base, B=2, H=3, T=T)
    _check("ragged T=%d %s" % (T, io), inp, io)


@pytest.mark.parametrize("case", ["eta0", "gamma0"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_special_cases(case, io):
    """eta = 0: every token sees W0, z = q + LN(q W0); gamma = 0: every
    gradient is exactly zero, so the state stays W0 bit for bit and
    z = q + beta."""
    base = WORKLOADS["linear_b1h1_t256_f32" if io == "f32" else "linear_125m_b8h12_t2k"]
    inp = make_inputs(base, B=1, H=2, T=70)
    inp["eta" if case == "eta0" else "gamma"][:] = 0
    z, w = _check("%s %s" % (case, io), inp, io)
    if case == "gamma0":
        np.testing.assert_array_equal(w[0], inp["w0"])


def test_more_units_than_compute_units():
    """B*H = 320 units, more workgroups than the GPU holds at once."""
    inp = make_inputs(WORKLOADS["linear_125m_b8h12_t2k"], B=10, H=32, T=80)
    _check("B10 H32 T80 bf16", inp, "bf16")


@pytest.mark.parametrize("b", [32, 64, 256])
def test_larger_minibatches(b):
    inp = make_inputs(WORKLOADS["linear_b1h1_t256_f32"], B=1, H=2, T=200)
    _check("mini_batch=%d" % b, inp, "f32", mini_batch=b)


@pytest.mark.parametrize("ln,res", [(False, True), (True, False), (False, False)])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_flags(ln, res, io):
    base = WORKLOADS["linear_b1h1_t256_f32" if io == "f32" else "linear_125m_b8h12_t2k"]
    inp = make_inputs(base, B=1, H=2, T=100)
    _check("ln=%d res=%d %s" % (ln, res, io), inp, io, layer_norm=ln, residual=res)


def test_eps_and_per_batch_state():
    w = WORKLOADS["linear_125m_b8h12_t2k"]
    inp = make_inputs(w, B=2, H=2, T=64)
    inp["w0"] = np.ascontiguousarray(
        np.stack([inp["w0"], 1.5 * inp["w0"][::-1]])).astype(np.float32)
    _check("eps=1e-5 per-batch W0", inp, "bf16", eps=1e-5, state0_per_batch=True)


def test_resume_and_in_place():
    """forward(0:T) vs forward(T1:T) started from forward(0:T1)'s final
    state: equal up to rounding (the LN shift is recomputed from the carried
    state's row sums), and the in-place form (w_out is w0) gives exactly the
    out-of-place result."""
    w = WORKLOADS["linear_125m_b8h12_t2k"]
    inp = make_inputs(w, B=2, H=3, T=256)
    dev = {k: to_dev(v, "bf16" if k in "qkv" else None) for k, v in inp.items()}
    z, wf = ttt_linear_forward(dev["q"], dev["k"], dev["v"], dev["eta"], dev["w0"],
                               dev["gamma"], dev["beta"])
    T1 = 128
    part = lambda x, a, b: x[:, :, a:b].contiguous()
    z1, w1 = ttt_linear_forward(*(part(dev[x], 0, T1) for x in "qkv"),
                                part(dev["eta"], 0, T1), dev["w0"], dev["gamma"], dev["beta"])
    tail = [part(dev[x], T1, 256) for x in "qkv"] + [part(dev["eta"], T1, 256)]
    z2, w2 = ttt_linear_forward(*tail, w1, dev["gamma"], dev["beta"], state0_per_batch=True)
    w1c = w1.clone()
    z3, w3 = ttt_linear_forward(*tail, w1c, dev["gamma"], dev["beta"], state0_per_batch=True,
                                w_out=w1c)
    torch.cuda.synchronize()
    assert torch.equal(z1, z[:, :, :T1])
    assert torch.equal(z3, z2) and torch.equal(w3, w2) and w3.data_ptr() == w1c.data_ptr()
    zc = from_dev(torch.cat([z1, z2], dim=2))
    assert z_err(zc, from_dev(z)) <= 2 ** -7          # a bf16 rounding flip at most
    assert state_err(from_dev(w2), from_dev(wf)) <= 1e-5


@pytest.mark.parametrize("split", [False, True])
def test_deterministic(split):
    """Ten runs of the same launch give the same bits (the two-workgroup
    launch too, whose output side follows a cross-CU hand-off)."""
    w = WORKLOADS["linear_125m_b8h12_t2k"]
    inp = make_inputs(w, B=2, T=512)
    a = _gpu(inp, "bf16", split=split)
    for _ in range(9):
        b = _gpu(inp, "bf16", split=split)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("name,strict", [("linear_125m_b8h12_t2k", True),
                                         ("linear_1p3b_b4h32_t8k", True),
                                         ("linear_long_b1h32_t32k", False)])
def test_full_size_all_units(name, strict):
    """The full workload as the benchmark runs it, every (batch, head) unit
    against the oracle.  The 125M- and 1.3B-shaped layers: every unit within
    the tolerance.  The 32k-token layer: every unit within the tolerance
    except where a plain fp32 evaluation of the scan itself misses it (two
    units whose scan amplifies rounding to O(1)); those are held to a small
    multiple of the fp32 evaluation's error (check_units)."""
    w = WORKLOADS[name]
    inp = make_inputs(w)
    z, wf = _gpu(inp, w.io)
    assert np.isfinite(z).all()
    args = [inp[x] for x in ("q", "k", "v", "eta", "w0", "gamma", "beta")]
    zr, wr = oracle.linear(*args)
    z32, w32 = _oracle_f32.linear(*args)
    if w.io == "bf16":
        z32 = bf16_round(z32)
    check_units(name, z, zr, z32.astype(np.float64), [wf], [wr], [w32.astype(np.float64)],
                TOL[w.io], strict=strict)
