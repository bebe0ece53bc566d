"""Launch-level properties of the library on a GPU: its launches can be
captured in a HIP graph and replayed (the split launch clears its counters
with a fill kernel, not a memset), and calls on two streams at once give
the results of the same calls made one after the other (the library keeps
no shared state; each call has its own workspace)."""
import pytest
import torch

import numpy as np

from linear_rnn_ttt_amd import (ttt_input_projection, ttt_linear_backward, ttt_linear_forward,
                                ttt_mlp_backward, ttt_mlp_forward)
from linear_rnn_ttt_amd.inputs import INPUT_WORKLOADS, WORKLOADS, make_input_side, make_inputs

from _parity import to_dev

pytestmark = pytest.mark.gpu

LIN = WORKLOADS["linear_125m_b8h12_t2k"]
MLP = WORKLOADS["mlp_125m_b8h12_t2k"]


def _lin_args(B=2, H=3, T=300, seed_shift=0):
    inp = make_inputs(LIN, B=B, H=H, T=T)
    if seed_shift:
        for x in "qkv":
            inp[x] = inp[x][:, :, ::-1].copy()      # other data, same distribution
    return [to_dev(inp[x], "bf16") for x in "qkv"] + [to_dev(inp[x]) for x in
                                                      ("eta", "w0", "gamma", "beta")]


def _mlp_args(B=1, H=2, T=100):
    inp = make_inputs(MLP, B=B, H=H, T=T)
    return [to_dev(inp[x], "bf16") for x in "qkv"] + [to_dev(inp[x]) for x in
                                                      ("eta", "w1", "b1", "w2", "b2",
                                                       "gamma", "beta")]


def _flat(out):
    """The tensors of an op's result (nested tuples flattened, None dropped)."""
    if isinstance(out, torch.Tensor):
        return [out]
    return [t for x in out if x is not None for t in _flat(x)]


@pytest.mark.parametrize("kind", ["linear backward", "mlp backward", "input side"])
def test_graph_capture_and_replay_of_backward_and_input(kind):
    """The backward passes and the input side captured in a graph: four
    replays, with eager work between them, each bit-identical to the eager
    call (their workspaces are allocated in the graph's pool)."""
    if kind == "linear backward":
        args = _lin_args(T=90)
        dz = to_dev(np.random.default_rng(0).standard_normal((2, 3, 90, 64)).astype(np.float32),
                    "bf16")
        run = lambda: ttt_linear_backward(*args, dz)
    elif kind == "mlp backward":
        args = _mlp_args(T=40)
        dz = to_dev(np.random.default_rng(1).standard_normal((1, 2, 40, 64)).astype(np.float32),
                    "bf16")
        run = lambda: ttt_mlp_backward(*args, dz)
    else:
        inp = make_input_side(INPUT_WORKLOADS["input_125m_b8_t2k"], B=2, T=130, D=192, H=3)
        x, w_in, b_eta = (to_dev(inp["x"], "bf16"), to_dev(inp["w_in"], "bf16"),
                          to_dev(inp["b_eta"]))
        run = lambda: ttt_input_projection(x, w_in, b_eta, heads=3,
                                           eta_base=float(inp["eta_base"]))
    ref = [t.clone() for t in _flat(run())]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = _flat(run())
    for rep in range(4):
        for t in out:
            t.zero_()                              # eager work between the replays
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(out, ref):
            assert torch.equal(got, want), (kind, rep)


@pytest.mark.parametrize("kind", ["linear", "linear split", "mlp"])
def test_graph_capture_and_replay(kind):
    args = _lin_args() if kind != "mlp" else _mlp_args()
    if kind == "mlp":
        run = lambda: ttt_mlp_forward(*args)
    else:
        run = lambda: ttt_linear_forward(*args, split=(kind == "linear split"))
    z_ref, s_ref = run()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                     # warm-up on the capture stream
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        z, st = run()
    for rep in range(4):
        z.zero_()                                  # eager work between the replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(z, z_ref), (kind, rep)
        if kind == "mlp":
            assert all(torch.equal(a, b) for a, b in zip(st, s_ref)), (kind, rep)
        else:
            assert torch.equal(st, s_ref), (kind, rep)


def test_two_streams_at_once():
    a, b = _lin_args(T=700), _lin_args(T=700, seed_shift=1)
    za, wa = ttt_linear_forward(*a, split=True)
    zb, wb = ttt_linear_forward(*b, split=False)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        with torch.cuda.stream(s1):
            z1, w1 = ttt_linear_forward(*a, split=True)
        with torch.cuda.stream(s2):
            z2, w2 = ttt_linear_forward(*b, split=False)
        torch.cuda.synchronize()
        assert torch.equal(z1, za) and torch.equal(w1, wa)
        assert torch.equal(z2, zb) and torch.equal(w2, wb)
