"""GPU parity of the TTT-Linear streaming step (ttt_linear_decode_step):
stepping every (batch, head) unit through a sequence one token at a time,
with pos = t mod mini_batch, against the fp64 oracle's scan of the same
sequence (z of every token, final state), and against the GPU scan kernel.
The step computes in fp32 (matrix-vector products, no matrix unit), so its
bound is the scan's: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs (whose z is
rounded to bf16)."""
import numpy as np
import pytest
import torch

import oracle
from linear_rnn_ttt_amd import _lib, ttt_linear_decode_step, ttt_linear_forward
from linear_rnn_ttt_amd.inputs import WORKLOADS, make_inputs

from _parity import TOL, from_dev, state_err, to_dev, z_err

pytestmark = pytest.mark.gpu

BF = WORKLOADS["linear_125m_b8h12_t2k"]
F32 = WORKLOADS["linear_b1h1_t256_f32"]


def _stream(inp, io, b, t0=0, W=None, Wb=None, **kw):
    """Step every unit through inp's tokens; returns (z, W, W_base) on the GPU."""
    dev = {x: to_dev(inp[x], io if x in "qkv" else None) for x in
           ("q", "k", "v", "eta", "gamma", "beta")}
    B, H, T, d = inp["q"].shape
    if W is None:
        W = to_dev(np.broadcast_to(inp["w0"], (B, H, d, d)).copy())
    if Wb is None:
        Wb = torch.zeros_like(W)
    z = torch.empty_like(dev["q"])
    for t in range(T):
        z[:, :, t] = ttt_linear_decode_step(
            dev["q"][:, :, t].contiguous(), dev["k"][:, :, t].contiguous(),
            dev["v"][:, :, t].contiguous(), dev["eta"][:, :, t].contiguous(), W, Wb,
            dev["gamma"], dev["beta"], pos=(t0 + t) % b, mini_batch=b, **kw)
    torch.cuda.synchronize()
    return z, W, Wb


@pytest.mark.parametrize("case", [
    ("bf16 b=16", BF, "bf16", 16, {}),
    ("bf16 b=64", BF, "bf16", 64, {}),
    ("f32 b=16", F32, "f32", 16, {}),
    ("f32 b=5", F32, "f32", 5, {}),
    ("f32 no LN", F32, "f32", 16, dict(layer_norm=False)),
    ("f32 no residual", F32, "f32", 16, dict(residual=False)),
    ("bf16 eps=1e-5", BF, "bf16", 16, dict(eps=1e-5)),
], ids=lambda c: c[0])
def test_decode_loop_matches_the_oracle_scan(case):
    name, wl, io, b, kw = case
    inp = make_inputs(wl, B=2, H=3, T=150)
    z, W, _ = _stream(inp, io, b, **kw)
    okw = {"layer_norm": kw.get("layer_norm", True), "residual": kw.get("residual", True),
           "eps": kw.get("eps", 1e-6)}
    zr, wr = oracle.linear(inp["q"], inp["k"], inp["v"], inp["eta"], inp["w0"], inp["gamma"],
                           inp["beta"], mini_batch=b, **okw)
    ez, ew = z_err(from_dev(z), zr), state_err(from_dev(W), wr)
    print("%s: z err %.3e, state err %.3e (tol %.0e)" % (name, ez, ew, TOL[io]), flush=True)
    assert ez <= TOL[io] and ew <= TOL[io]


def test_decode_continues_a_scan_and_a_cut_stream():
    """The scan's final state (after a whole number of mini-batches) starts a
    stream; a stream cut inside a mini-batch continues from its (W, W_base).
    Both agree with the scan of the whole sequence."""
    inp = make_inputs(BF, B=2, H=2, T=200)
    dev = {x: to_dev(inp[x], "bf16" if x in "qkv" else None) for x in inp}
    z_all, w_all = ttt_linear_forward(dev["q"], dev["k"], dev["v"], dev["eta"], dev["w0"],
                                      dev["gamma"], dev["beta"], split=False)
    T1 = 96
    cut = lambda a, b: {x: (v[:, :, a:b] if x in ("q", "k", "v", "eta") else v)
                        for x, v in inp.items()}
    _, w1 = ttt_linear_forward(*(dev[x][:, :, :T1].contiguous() for x in "qkv"),
                               dev["eta"][:, :, :T1].contiguous(), dev["w0"], dev["gamma"],
                               dev["beta"], split=False)
    z2, W2, Wb2 = _stream(cut(T1, 150), "bf16", 16, t0=T1, W=w1.clone())
    z3, W3, _ = _stream(cut(150, 200), "bf16", 16, t0=150, W=W2, Wb=Wb2)
    torch.cuda.synchronize()
    z = torch.cat([z2, z3], dim=2)
    ez = z_err(from_dev(z), from_dev(z_all[:, :, T1:]))
    ew = state_err(from_dev(W3), from_dev(w_all))
    print("continued stream vs scan: z err %.3e, state err %.3e" % (ez, ew), flush=True)
    assert ez <= 2e-2 and ew <= 1e-3


def test_decode_pos0_records_the_base_and_pos_checked():
    inp = make_inputs(BF, B=1, H=2, T=1)
    dev = {x: to_dev(inp[x], "bf16" if x in "qkv" else None) for x in inp}
    W = to_dev(np.broadcast_to(inp["w0"], (1, 2, 64, 64)).copy())
    W_in = W.clone()
    Wb = torch.full_like(W, float("nan"))      # not read at pos 0
    z = ttt_linear_decode_step(dev["q"][:, :, 0].contiguous(), dev["k"][:, :, 0].contiguous(),
                               dev["v"][:, :, 0].contiguous(), dev["eta"][:, :, 0].contiguous(),
                               W, Wb, dev["gamma"], dev["beta"], pos=0)
    torch.cuda.synchronize()
    assert torch.equal(Wb, W_in) and torch.isfinite(z.float()).all()
    with pytest.raises(_lib.TTTArgumentError) as e:
        ttt_linear_decode_step(dev["q"][:, :, 0].contiguous(), dev["k"][:, :, 0].contiguous(),
                               dev["v"][:, :, 0].contiguous(),
                               dev["eta"][:, :, 0].contiguous(), W, Wb, dev["gamma"],
                               dev["beta"], pos=16, mini_batch=16)
    assert e.value.code == _lib.TTT_ERR_ARG
