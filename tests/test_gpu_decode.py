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
from linear_rnn_ttt_amd import (_lib, ttt_linear_decode_step, ttt_linear_decode_step_compact,
                               ttt_linear_forward)
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


def _tokens(dev, T):
    return [[dev[x][:, :, t].contiguous() for x in ("q", "k", "v", "eta")] for t in range(T)]


def test_decode_graph_replays_match_eager():
    """Two mini-batches of steps captured into one HIP graph, replayed three
    times from the same starting state (reset by eager copies between the
    replays): every replay equals the eager steps bit for bit."""
    inp = make_inputs(BF, B=2, H=3, T=40)
    dev = {x: to_dev(inp[x], "bf16" if x in "qkv" else None) for x in inp}
    toks = _tokens(dev, 40)
    W0 = to_dev(np.broadcast_to(inp["w0"], (2, 3, 64, 64)).copy())
    W, Wb = W0.clone(), torch.zeros_like(W0)
    zs = torch.empty((40, 2, 3, 64), dtype=torch.bfloat16, device="cuda")

    def steps():
        for t in range(40):
            ttt_linear_decode_step(*toks[t][:4], W, Wb, dev["gamma"], dev["beta"], pos=t % 16,
                                   z=zs[t])

    steps()
    torch.cuda.synchronize()
    z_ref, W_ref, Wb_ref = zs.clone(), W.clone(), Wb.clone()
    W.copy_(W0)
    Wb.zero_()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps()
    torch.cuda.synchronize()
    for r in range(3):
        W.copy_(W0)
        Wb.zero_()
        zs.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(zs, z_ref) and torch.equal(W, W_ref) and torch.equal(Wb, Wb_ref), r


@pytest.mark.parametrize("streams", [4, 256])
def test_decode_bench_shape_sampled_units(streams):
    """The streaming step at the 1.3B layer shape (H = 32) with 4 and 256
    streams, 20 tokens (a mini-batch and a ragged tail), launched from a
    graph as the benchmark does: sampled units against the oracle's step."""
    wl = WORKLOADS["linear_1p3b_b4h32_t8k"].with_(B=streams)
    T = 20
    inp = make_inputs(wl, T=T)
    dev = {x: to_dev(inp[x], "bf16" if x in "qkv" else None) for x in inp}
    toks = _tokens(dev, T)
    W = to_dev(np.broadcast_to(inp["w0"], (streams, 32, 64, 64)).copy())
    Wb = torch.zeros_like(W)
    zs = torch.empty((T, streams, 32, 64), dtype=torch.bfloat16, device="cuda")
    ttt_linear_decode_step(*toks[0], W, Wb, dev["gamma"], dev["beta"], pos=0, z=zs[0])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t in range(1, T):
            ttt_linear_decode_step(*toks[t], W, Wb, dev["gamma"], dev["beta"], pos=t % 16,
                                   z=zs[t])
    graph.replay()
    torch.cuda.synchronize()
    z = from_dev(zs)
    Wg = from_dev(W)
    rng = np.random.default_rng(7)
    units = [(0, 0), (streams - 1, 31)] + [tuple(u) for u in
                                          zip(rng.integers(0, streams, 6), rng.integers(0, 32, 6))]
    worst = 0.0
    for b, h in units:
        Wr, Wbr = inp["w0"][h].astype(np.float64), None
        zr = np.empty((T, 64))
        for t in range(T):
            zr[t], Wr, Wbr = oracle.linear_decode_step(
                Wr, Wbr, inp["q"][b, h, t], inp["k"][b, h, t], inp["v"][b, h, t],
                inp["eta"][b, h, t], inp["gamma"][h], inp["beta"][h], pos=t % 16, eps=wl.eps)
        ez = z_err(z[:, b, h][None, None], zr[None, None])
        ew = state_err(Wg[b, h][None, None], Wr[None, None])
        worst = max(worst, ez, ew)
        assert ez <= TOL["bf16"] and ew <= TOL["bf16"], (b, h, ez, ew)
    print("streams=%d: %d sampled units, worst err %.3e" % (streams, len(units), worst),
          flush=True)


# ---- the compact pending state (ttt_linear_decode_step_compact) -------------

def _stream_compact(inp, io, b, t0=0, Wb=None, Hh=None, **kw):
    """Step every unit through inp's tokens with the compact state; returns
    (z, w_base, hist) on the GPU."""
    dev = {x: to_dev(inp[x], io if x in "qkv" else None) for x in
           ("q", "k", "v", "eta", "gamma", "beta")}
    B, H, T, d = inp["q"].shape
    if Wb is None:
        Wb = to_dev(np.broadcast_to(inp["w0"], (B, H, d, d)).copy())
    if Hh is None:
        Hh = torch.zeros((B, H, b, 2, d), dtype=torch.float32, device="cuda")
    z = torch.empty_like(dev["q"])
    for t in range(T):
        z[:, :, t] = ttt_linear_decode_step_compact(
            dev["q"][:, :, t].contiguous(), dev["k"][:, :, t].contiguous(),
            dev["v"][:, :, t].contiguous(), dev["eta"][:, :, t].contiguous(), Wb, Hh,
            dev["gamma"], dev["beta"], pos=(t0 + t) % b, mini_batch=b, **kw)
    torch.cuda.synchronize()
    return z, Wb, Hh


def compact_state(Wb, Hh, n_used):
    """W = w_base + sum over the first n_used history slots of k_s^T u_s."""
    Wb, Hh = from_dev(Wb), from_dev(Hh)
    return Wb + np.einsum("bhsi,bhsj->bhij", Hh[:, :, :n_used, 0], Hh[:, :, :n_used, 1])


@pytest.mark.parametrize("case", [
    ("bf16 b=16", BF, "bf16", 16, {}),
    ("bf16 b=64", BF, "bf16", 64, {}),
    ("f32 b=16", F32, "f32", 16, {}),
    ("f32 b=5", F32, "f32", 5, {}),
    ("f32 no LN", F32, "f32", 16, dict(layer_norm=False)),
    ("f32 no residual", F32, "f32", 16, dict(residual=False)),
    ("bf16 eps=1e-5", BF, "bf16", 16, dict(eps=1e-5)),
], ids=lambda c: c[0])
def test_compact_loop_matches_the_oracle_scan(case):
    name, wl, io, b, kw = case
    T = 150
    inp = make_inputs(wl, B=2, H=3, T=T)
    z, Wb, Hh = _stream_compact(inp, io, b, **kw)
    okw = {"layer_norm": kw.get("layer_norm", True), "residual": kw.get("residual", True),
           "eps": kw.get("eps", 1e-6)}
    zr, wr = oracle.linear(inp["q"], inp["k"], inp["v"], inp["eta"], inp["w0"], inp["gamma"],
                           inp["beta"], mini_batch=b, **okw)
    W = compact_state(Wb, Hh, b if T % b == 0 else T % b)
    ez, ew = z_err(from_dev(z), zr), state_err(W, wr)
    print("compact %s: z err %.3e, state err %.3e (tol %.0e)" % (name, ez, ew, TOL[io]),
          flush=True)
    assert ez <= TOL[io] and ew <= TOL[io]


def test_compact_continues_a_scan():
    """The scan's final state after whole mini-batches starts a compact stream
    (zero history); the stream's z equals the scan of the whole sequence."""
    inp = make_inputs(BF, B=2, H=2, T=200)
    dev = {x: to_dev(inp[x], "bf16" if x in "qkv" else None) for x in inp}
    z_all, w_all = ttt_linear_forward(dev["q"], dev["k"], dev["v"], dev["eta"], dev["w0"],
                                      dev["gamma"], dev["beta"], split=False)
    T1 = 96
    _, w1 = ttt_linear_forward(*(dev[x][:, :, :T1].contiguous() for x in "qkv"),
                               dev["eta"][:, :, :T1].contiguous(), dev["w0"], dev["gamma"],
                               dev["beta"], split=False)
    cut = {x: (v[:, :, T1:] if x in ("q", "k", "v", "eta") else v) for x, v in inp.items()}
    z2, Wb, Hh = _stream_compact(cut, "bf16", 16, t0=T1, Wb=w1.clone())
    ez = z_err(from_dev(z2), from_dev(z_all[:, :, T1:]))
    ew = state_err(compact_state(Wb, Hh, (200 - T1) % 16 or 16), from_dev(w_all))
    print("compact stream after a scan: z err %.3e, state err %.3e" % (ez, ew), flush=True)
    assert ez <= 2e-2 and ew <= 1e-3


def test_compact_bench_shape_sampled_units():
    """256 streams x 32 heads, 20 tokens (a mini-batch and a ragged tail),
    graph-launched as the benchmark does; sampled units against the
    oracle's step."""
    streams, T = 256, 20
    wl = WORKLOADS["linear_1p3b_b4h32_t8k"].with_(B=streams)
    inp = make_inputs(wl, T=T)
    dev = {x: to_dev(inp[x], "bf16" if x in "qkv" else None) for x in inp}
    toks = _tokens(dev, T)
    Wb = to_dev(np.broadcast_to(inp["w0"], (streams, 32, 64, 64)).copy())
    Hh = torch.zeros((streams, 32, 16, 2, 64), dtype=torch.float32, device="cuda")
    zs = torch.empty((T, streams, 32, 64), dtype=torch.bfloat16, device="cuda")
    ttt_linear_decode_step_compact(*toks[0], Wb, Hh, dev["gamma"], dev["beta"], pos=0, z=zs[0])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t in range(1, T):
            ttt_linear_decode_step_compact(*toks[t], Wb, Hh, dev["gamma"], dev["beta"],
                                           pos=t % 16, z=zs[t])
    graph.replay()
    torch.cuda.synchronize()
    z = from_dev(zs)
    W = compact_state(Wb, Hh, T % 16)
    rng = np.random.default_rng(8)
    units = [(0, 0), (streams - 1, 31)] + [tuple(u) for u in
                                          zip(rng.integers(0, streams, 6), rng.integers(0, 32, 6))]
    worst = 0.0
    for b, h in units:
        Wr, Wbr = inp["w0"][h].astype(np.float64), None
        zr = np.empty((T, 64))
        for t in range(T):
            zr[t], Wr, Wbr = oracle.linear_decode_step(
                Wr, Wbr, inp["q"][b, h, t], inp["k"][b, h, t], inp["v"][b, h, t],
                inp["eta"][b, h, t], inp["gamma"][h], inp["beta"][h], pos=t % 16, eps=wl.eps)
        ez = z_err(z[:, b, h][None, None], zr[None, None])
        ew = state_err(W[b, h][None, None], Wr[None, None])
        worst = max(worst, ez, ew)
        assert ez <= TOL["bf16"] and ew <= TOL["bf16"], (b, h, ez, ew)
    print("compact, %d streams: %d sampled units, worst err %.3e" % (streams, len(units), worst),
          flush=True)
