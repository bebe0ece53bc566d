"""GPU parity of the TTT-MLP scan (gfx950 kernel through the C ABI) against
the fp64 oracle on the same seeded inputs.  Tolerances: 1e-4 max relative
error for fp32 inputs, 2e-2 for bf16 inputs (fp32 state)."""
import numpy as np
import pytest
import torch

import oracle
from linear_rnn_ttt_amd import ttt_mlp_forward
from linear_rnn_ttt_amd.inputs import WORKLOADS, bf16_round, make_inputs

import _oracle_f32
from _parity import TOL, check_units, from_dev, state_err, to_dev, z_err

pytestmark = pytest.mark.gpu

STATE = ("w1", "b1", "w2", "b2")


def _gpu(inp, io, **kw):
    z, S = ttt_mlp_forward(to_dev(inp["q"], io), to_dev(inp["k"], io), to_dev(inp["v"], io),
                           to_dev(inp["eta"]), *(to_dev(inp[s]) for s in STATE),
                           to_dev(inp["gamma"]), to_dev(inp["beta"]), **kw)
    torch.cuda.synchronize()
    return from_dev(z), [from_dev(s) for s in S]


def _oracle(inp, **kw):
    return oracle.mlp(inp["q"], inp["k"], inp["v"], inp["eta"], *(inp[s] for s in STATE),
                      inp["gamma"], inp["beta"], **kw)


def _check(name, inp, io, **kw):
    tol = TOL[io]
    z, S = _gpu(inp, io, **kw)
    okw = {k: v for k, v in kw.items() if k in ("layer_norm", "residual", "eps",
                                                 "state0_per_batch")}
    zr, Sr = _oracle(inp, **okw)
    ez = z_err(z, zr)
    es = [state_err(a.reshape(a.shape[:2] + (-1,)), b.reshape(b.shape[:2] + (-1,)))
          for a, b in zip(S, Sr)]
    print("%s: z err %.3e, state errs %s (tol %.0e)" % (
        name, ez, " ".join("%.2e" % e for e in es), tol), flush=True)
    assert ez <= tol and max(es) <= tol, (ez, es)
    return z, S


MLP = WORKLOADS["mlp_125m_b8h12_t2k"]
MLP32 = MLP.with_(io="f32")


def test_bf16_small():
    _check("mlp bf16 B2 H3 T96", make_inputs(MLP, B=2, H=3, T=96), "bf16")


def test_fp32_small():
    _check("mlp f32 B1 H2 T64", make_inputs(MLP32, B=1, H=2, T=64), "f32")


@pytest.mark.parametrize("T", [1, 15, 17, 50])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_ragged_lengths(T, io):
    _check("mlp ragged T=%d %s" % (T, io), make_inputs(MLP if io == "bf16" else MLP32, B=1,
                                                        H=2, T=T), io)


@pytest.mark.parametrize("ln,res", [(False, True), (True, False), (False, False)])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_flags(ln, res, io):
    inp = make_inputs(MLP if io == "bf16" else MLP32, B=1, H=2, T=48)
    _check("mlp ln=%d res=%d %s" % (ln, res, io), inp, io, layer_norm=ln, residual=res)


@pytest.mark.parametrize("case", ["eta0", "gamma0"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_special_cases(case, io):
    """eta = 0: every token sees the initial state (the inner model's plain
    forward, GELU included); gamma = 0: every gradient is exactly zero, so the
    state stays put bit for bit and z = q + beta."""
    inp = make_inputs(MLP if io == "bf16" else MLP32, B=1, H=2, T=40)
    inp["eta" if case == "eta0" else "gamma"][:] = 0
    z, S = _check("mlp %s %s" % (case, io), inp, io)
    if case == "gamma0":
        for a, s in zip(S, STATE):
            np.testing.assert_array_equal(a[0], inp[s])


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_large_hidden_preactivations(io):
    """W1 and b1 scaled so that the hidden pre-activations spread over about
    +-20: GELU and GELU' are then taken far into both tails (GELU(x) -> x and
    0, GELU'(x) -> 1 and 0), beyond the range of the bf16 kernel's Phi table
    (+-6) and into the saturated part of its per-value formula."""
    inp = make_inputs(MLP if io == "bf16" else MLP32, B=1, H=2, T=64)
    rng = np.random.default_rng(11)
    inp["w1"] = (inp["w1"] * 400.0).astype(np.float32)
    inp["b1"] = rng.standard_normal(inp["b1"].shape).astype(np.float32) * 4.0
    # the spread the test relies on (k rows have norm about 1)
    p = np.einsum("btd,hdm->bhtm", inp["k"][:, 0], inp["w1"][:1])
    assert np.abs(p).max() > 12.0
    _check("mlp large pre-activations %s" % io, inp, io)


def test_more_units_than_compute_units():
    """B*H = 320 units, more workgroups than the GPU holds at once."""
    _check("mlp B10 H32 T40 bf16", make_inputs(MLP, B=10, H=32, T=40), "bf16")


def test_per_batch_state_and_eps():
    inp = make_inputs(MLP, B=2, H=2, T=64)
    rng = np.random.default_rng(7)
    for s in STATE:
        x = inp[s]
        inp[s] = np.ascontiguousarray(np.stack([x, x + 0.01 * rng.standard_normal(x.shape)
                                                .astype(np.float32)]))
    _check("mlp per-batch state eps=1e-5", inp, "bf16", state0_per_batch=True, eps=1e-5)


def test_resume_and_in_place():
    inp = make_inputs(MLP, B=1, H=2, T=128)
    dev = {k: to_dev(v, "bf16" if k in "qkv" else None) for k, v in inp.items()}
    args = lambda a, b: [dev[x][:, :, a:b].contiguous() for x in "qkv"] + \
        [dev["eta"][:, :, a:b].contiguous()]
    z, S = ttt_mlp_forward(*args(0, 128), *(dev[s] for s in STATE), dev["gamma"], dev["beta"])
    z1, S1 = ttt_mlp_forward(*args(0, 64), *(dev[s] for s in STATE), dev["gamma"], dev["beta"])
    z2, S2 = ttt_mlp_forward(*args(64, 128), *S1, dev["gamma"], dev["beta"],
                             state0_per_batch=True)
    S1c = [s.clone() for s in S1]
    z3, S3 = ttt_mlp_forward(*args(64, 128), *S1c, dev["gamma"], dev["beta"],
                             state0_per_batch=True, state_out=S1c)
    torch.cuda.synchronize()
    assert torch.equal(z1, z[:, :, :64])
    assert torch.equal(torch.cat([z1, z2], dim=2), z)
    for a, b in zip(S2, S):
        assert torch.equal(a, b)
    assert torch.equal(z3, z2)
    for a, b in zip(S3, S2):
        assert torch.equal(a, b)


def test_deterministic():
    """Ten runs give the same bits."""
    inp = make_inputs(MLP, B=2, H=4, T=256)
    a = _gpu(inp, "bf16")
    for _ in range(9):
        b = _gpu(inp, "bf16")
        assert np.array_equal(a[0], b[0])
        for x, y in zip(a[1], b[1]):
            assert np.array_equal(x, y)


@pytest.mark.parametrize("name", ["mlp_125m_b8h12_t2k", "mlp_long_b1h32_t32k"])
def test_full_size_all_units(name):
    """The full workload as the benchmark runs it, every (batch, head) unit
    against the oracle, each within the tolerance (no exemptions; the fp32
    evaluation's errors are printed beside)."""
    w = WORKLOADS[name]
    inp = make_inputs(w)
    z, S = _gpu(inp, w.io)
    assert np.isfinite(z).all()
    args = [inp[x] for x in ("q", "k", "v", "eta")] + [inp[s] for s in STATE] + [
        inp["gamma"], inp["beta"]]
    zr, Sr = oracle.mlp(*args)
    z32, S32 = _oracle_f32.mlp(*args)
    z32 = bf16_round(z32) if w.io == "bf16" else z32
    flat = lambda X: [np.asarray(x, np.float64).reshape(x.shape[:2] + (-1,)) for x in X]
    check_units(name, z, zr, z32.astype(np.float64), flat(S), flat(Sr), flat(S32), TOL[w.io],
                strict=True)
