"""GPU parity of the TTT-MLP streaming step (ttt_mlp_decode_step and its
compact-state form ttt_mlp_decode_step_compact): stepping
every (batch, head) unit through a sequence one token at a time, with
pos = t mod mini_batch, against the fp64 oracle's scan of the same sequence
(z of every token, the final state (W1, b1, W2, b2)).  The step computes in
fp32 (matrix-vector products), so its bound is the MLP scan's: 1e-4 for fp32
inputs, 2e-2 for bf16 inputs (whose z is rounded to bf16)."""
import numpy as np
import pytest
import torch

import oracle
from linear_rnn_ttt_amd import ttt_mlp_decode_step, ttt_mlp_decode_step_compact, ttt_mlp_forward
from linear_rnn_ttt_amd.inputs import WORKLOADS, make_inputs

from _parity import TOL, from_dev, state_err, to_dev, z_err

pytestmark = pytest.mark.gpu

STATE = ("w1", "b1", "w2", "b2")
MLP = WORKLOADS["mlp_125m_b8h12_t2k"]
MLP32 = MLP.with_(io="f32")
LONG = WORKLOADS["mlp_long_b1h32_t32k"]


def _initial(inp, B, H):
    """The shared initial state broadcast to every unit, on the GPU."""
    return [to_dev(np.broadcast_to(inp[s], (B, H) + inp[s].shape[1:]).copy()) for s in STATE]


def _stream(inp, io, b, t0=0, S=None, base=None, **kw):
    """Step every unit through inp's tokens; returns (z, S, base) on the GPU."""
    dev = {x: to_dev(inp[x], io if x in "qkv" else None) for x in
           ("q", "k", "v", "eta", "gamma", "beta")}
    B, H, T, d = inp["q"].shape
    if S is None:
        S = _initial(inp, B, H)
    if base is None:
        base = [torch.zeros_like(s) for s in S]
    z = torch.empty_like(dev["q"])
    for t in range(T):
        z[:, :, t] = ttt_mlp_decode_step(
            dev["q"][:, :, t].contiguous(), dev["k"][:, :, t].contiguous(),
            dev["v"][:, :, t].contiguous(), dev["eta"][:, :, t].contiguous(), S, base,
            dev["gamma"], dev["beta"], pos=(t0 + t) % b, mini_batch=b, **kw)
    torch.cuda.synchronize()
    return z, S, base


def _errs(z, S, zr, Sr):
    flat = lambda x: x.reshape(x.shape[:2] + (-1,))
    return z_err(from_dev(z), zr), [state_err(flat(from_dev(a)), flat(b)) for a, b in zip(S, Sr)]


def _okw(kw):
    return {"layer_norm": kw.get("layer_norm", True), "residual": kw.get("residual", True),
            "eps": kw.get("eps", 1e-6)}


@pytest.mark.parametrize("case", [
    ("bf16 b=16", MLP, "bf16", 16, {}),
    ("f32 b=16", MLP32, "f32", 16, {}),
    ("f32 b=5", MLP32, "f32", 5, {}),
    ("f32 b=1", MLP32, "f32", 1, {}),
    ("f32 no LN", MLP32, "f32", 16, dict(layer_norm=False)),
    ("f32 no residual", MLP32, "f32", 16, dict(residual=False)),
    ("bf16 eps=1e-5", MLP, "bf16", 16, dict(eps=1e-5)),
], ids=lambda c: c[0])
def test_mlp_decode_loop_matches_the_oracle_scan(case):
    name, wl, io, b, kw = case
    inp = make_inputs(wl, B=2, H=3, T=45)
    z, S, _ = _stream(inp, io, b, **kw)
    zr, Sr = oracle.mlp(inp["q"], inp["k"], inp["v"], inp["eta"], *(inp[s] for s in STATE),
                        inp["gamma"], inp["beta"], mini_batch=b, **_okw(kw))
    ez, es = _errs(z, S, zr, Sr)
    print("%s: z err %.3e, state errs %s (tol %.0e)" % (
        name, ez, " ".join("%.2e" % e for e in es), TOL[io]), flush=True)
    assert ez <= TOL[io] and max(es) <= TOL[io], (ez, es)


def test_mlp_decode_carries_the_base_within_a_mini_batch():
    """A stream cut inside a mini-batch and continued from its (S, S_base)
    agrees with the oracle's step-by-step recurrence, position by position;
    the carried base is the state at the mini-batch's start."""
    inp = make_inputs(MLP32, B=1, H=2, T=21)
    z, S, base = _stream(inp, "f32", 16)
    for h in range(2):
        Sh, Sb = tuple(inp[s][h] for s in STATE), None
        for t in range(21):
            zt, Sh, Sb = oracle.mlp_decode_step(Sh, Sb, inp["q"][0, h, t], inp["k"][0, h, t],
                                                inp["v"][0, h, t], inp["eta"][0, h, t],
                                                inp["gamma"][h], inp["beta"][h], pos=t % 16)
            assert z_err(from_dev(z)[0, h, t], zt) <= 1e-4
        for got, want in zip(base, Sb):
            assert state_err(from_dev(got)[0, h].reshape(1, 1, -1),
                             want.reshape(1, 1, -1)) <= 1e-4


def test_mlp_decode_continues_the_gpu_scan():
    """The MLP scan's final state after a whole number of mini-batches starts
    a stream, and the stream continues the sequence as the oracle's scan of
    the whole of it does."""
    T1, T = 32, 61
    inp = make_inputs(MLP, B=2, H=2, T=T)
    dev = {x: to_dev(inp[x], "bf16" if x in "qkv" else None) for x in inp}
    _, S1 = ttt_mlp_forward(*(dev[x][:, :, :T1].contiguous() for x in "qkv"),
                            dev["eta"][:, :, :T1].contiguous(), *(dev[s] for s in STATE),
                            dev["gamma"], dev["beta"])
    rest = {x: (v[:, :, T1:] if x in ("q", "k", "v", "eta") else v) for x, v in inp.items()}
    z2, S2, _ = _stream(rest, "bf16", 16, t0=T1, S=[s.clone() for s in S1])
    zr, Sr = oracle.mlp(inp["q"], inp["k"], inp["v"], inp["eta"], *(inp[s] for s in STATE),
                        inp["gamma"], inp["beta"], mini_batch=16)
    ez, es = _errs(z2, S2, zr[:, :, T1:], Sr)
    print("continued stream: z err %.3e, state errs %s" % (ez, es), flush=True)
    assert ez <= TOL["bf16"] and max(es) <= TOL["bf16"]


@pytest.mark.parametrize("streams", [4, 256])
def test_mlp_decode_bench_shape(streams):
    """The benchmark's shapes (streams x 32 heads): every unit through 18
    tokens (one mini-batch boundary), against the oracle's scan."""
    inp = make_inputs(LONG, B=streams, H=32, T=18)
    z, S, _ = _stream(inp, "bf16", 16)
    zr, Sr = oracle.mlp(inp["q"], inp["k"], inp["v"], inp["eta"], *(inp[s] for s in STATE),
                        inp["gamma"], inp["beta"], mini_batch=16)
    ez, es = _errs(z, S, zr, Sr)
    print("%d streams: z err %.3e, state errs %s" % (streams, ez, es), flush=True)
    assert ez <= TOL["bf16"] and max(es) <= TOL["bf16"]


@pytest.mark.parametrize("compact", [False, True], ids=["S_base", "compact"])
def test_mlp_decode_graph_replay(compact):
    """Steps captured into a HIP graph and replayed give the eager steps'
    results bit for bit (the replay is how a generation loop runs them)."""
    inp = make_inputs(MLP, B=2, H=3, T=20)
    dev = {x: to_dev(inp[x], "bf16" if x in "qkv" else None) for x in inp}
    toks = [[dev[x][:, :, t].contiguous() for x in ("q", "k", "v", "eta")] for t in range(20)]
    S0 = _initial(inp, 2, 3)

    def run(S, aux, z, t_from, t_to):
        for t in range(t_from, t_to):
            if compact:
                ttt_mlp_decode_step_compact(*toks[t], S, aux[0], dev["gamma"], dev["beta"],
                                            pos=t % 16, z=z[t])
            else:
                ttt_mlp_decode_step(*toks[t], S, aux, dev["gamma"], dev["beta"], pos=t % 16,
                                    z=z[t])

    def fresh():
        aux = ([torch.zeros((2, 3, 16, 640), dtype=torch.float32, device="cuda")] if compact
               else [torch.zeros_like(s) for s in S0])
        return ([s.clone() for s in S0], aux,
                torch.empty((20,) + toks[0][0].shape, dtype=torch.bfloat16, device="cuda"))

    Se, be, ze = fresh()
    run(Se, be, ze, 0, 20)
    Sg, bg, zg = fresh()
    run(Sg, bg, zg, 0, 4)
    torch.cuda.synchronize()
    snap = [s.clone() for s in Sg + bg]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(Sg, bg, zg, 4, 20)
    for rep in range(3):
        for dst, src in zip(Sg + bg, snap):
            dst.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(zg, ze), rep
        for a, b in zip(Sg + bg, Se + be):
            assert torch.equal(a, b), rep


def _stream_compact(inp, io, b, t0=0, base=None, hist=None, **kw):
    """The compact step over inp's tokens; returns (z, base, hist) on the GPU."""
    dev = {x: to_dev(inp[x], io if x in "qkv" else None) for x in
           ("q", "k", "v", "eta", "gamma", "beta")}
    B, H, T, d = inp["q"].shape
    m = inp["w1"].shape[-1]
    if base is None:
        base = _initial(inp, B, H)
    if hist is None:
        hist = torch.zeros((B, H, b, 2 * d + 2 * m), dtype=torch.float32, device="cuda")
    z = torch.empty_like(dev["q"])
    for t in range(T):
        z[:, :, t] = ttt_mlp_decode_step_compact(
            dev["q"][:, :, t].contiguous(), dev["k"][:, :, t].contiguous(),
            dev["v"][:, :, t].contiguous(), dev["eta"][:, :, t].contiguous(), base, hist,
            dev["gamma"], dev["beta"], pos=(t0 + t) % b, mini_batch=b, **kw)
    torch.cuda.synchronize()
    return z, base, hist


def _rebuild(base, hist, n_pending, d):
    """The state from the base and the first n_pending history rows (fp64):
    W1 += k^T u1, b1 += u1, W2 += a^T u2, b2 += u2 per row."""
    w1, b1, w2, b2 = (from_dev(x) for x in base)
    h = from_dev(hist)[:, :, :n_pending]
    m = w1.shape[-1]
    k, u1, a, u2 = h[..., :d], h[..., d:d + m], h[..., d + m:d + 2 * m], h[..., d + 2 * m:]
    return (w1 + np.einsum("bhsf,bhsn->bhfn", k, u1), b1 + u1.sum(2),
            w2 + np.einsum("bhsn,bhsf->bhnf", a, u2), b2 + u2.sum(2))


@pytest.mark.parametrize("case", [
    ("bf16 b=16", MLP, "bf16", 16, {}),
    ("f32 b=16", MLP32, "f32", 16, {}),
    ("f32 b=5", MLP32, "f32", 5, {}),
    ("f32 b=1", MLP32, "f32", 1, {}),
    ("f32 no LN", MLP32, "f32", 16, dict(layer_norm=False)),
    ("f32 no residual", MLP32, "f32", 16, dict(residual=False)),
    ("bf16 eps=1e-5", MLP, "bf16", 16, dict(eps=1e-5)),
], ids=lambda c: c[0])
def test_mlp_compact_loop_matches_the_oracle_scan(case):
    """The compact step looped over a sequence: z of every token, and the
    state rebuilt from the base and the pending mini-batch's rows, against
    the oracle's scan."""
    name, wl, io, b, kw = case
    T = 45
    inp = make_inputs(wl, B=2, H=3, T=T)
    z, base, hist = _stream_compact(inp, io, b, **kw)
    zr, Sr = oracle.mlp(inp["q"], inp["k"], inp["v"], inp["eta"], *(inp[s] for s in STATE),
                        inp["gamma"], inp["beta"], mini_batch=b, **_okw(kw))
    S = _rebuild(base, hist, (T - 1) % b + 1, inp["q"].shape[-1])
    flat = lambda x: x.reshape(x.shape[:2] + (-1,))
    ez = z_err(from_dev(z), zr)
    es = [state_err(flat(a), flat(r)) for a, r in zip(S, Sr)]
    print("compact %s: z err %.3e, state errs %s (tol %.0e)" % (
        name, ez, " ".join("%.2e" % e for e in es), TOL[io]), flush=True)
    assert ez <= TOL[io] and max(es) <= TOL[io], (ez, es)


def test_mlp_compact_continues_the_gpu_scan():
    """The MLP scan's final state after a whole number of mini-batches is the
    base of a compact stream with a zero history."""
    T1, T = 32, 61
    inp = make_inputs(MLP, B=2, H=2, T=T)
    dev = {x: to_dev(inp[x], "bf16" if x in "qkv" else None) for x in inp}
    _, S1 = ttt_mlp_forward(*(dev[x][:, :, :T1].contiguous() for x in "qkv"),
                            dev["eta"][:, :, :T1].contiguous(), *(dev[s] for s in STATE),
                            dev["gamma"], dev["beta"])
    rest = {x: (v[:, :, T1:] if x in ("q", "k", "v", "eta") else v) for x, v in inp.items()}
    z2, _, _ = _stream_compact(rest, "bf16", 16, t0=T1, base=[s.clone() for s in S1])
    zr, _ = oracle.mlp(inp["q"], inp["k"], inp["v"], inp["eta"], *(inp[s] for s in STATE),
                       inp["gamma"], inp["beta"], mini_batch=16)
    ez = z_err(from_dev(z2), zr[:, :, T1:])
    print("compact continued stream: z err %.3e" % ez, flush=True)
    assert ez <= TOL["bf16"]


@pytest.mark.parametrize("streams", [4, 256])
def test_mlp_compact_bench_shape(streams):
    """The benchmark's shapes: every unit through 18 tokens (one fold), z
    and the rebuilt state against the oracle's scan."""
    inp = make_inputs(LONG, B=streams, H=32, T=18)
    z, base, hist = _stream_compact(inp, "bf16", 16)
    zr, Sr = oracle.mlp(inp["q"], inp["k"], inp["v"], inp["eta"], *(inp[s] for s in STATE),
                        inp["gamma"], inp["beta"], mini_batch=16)
    S = _rebuild(base, hist, 2, 64)
    flat = lambda x: x.reshape(x.shape[:2] + (-1,))
    ez = z_err(from_dev(z), zr)
    es = [state_err(flat(a), flat(r)) for a, r in zip(S, Sr)]
    print("compact %d streams: z err %.3e, state errs %s" % (streams, ez, es), flush=True)
    assert ez <= TOL["bf16"] and max(es) <= TOL["bf16"]
