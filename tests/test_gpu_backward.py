"""GPU parity of the TTT-Linear backward pass (ttt_linear_backward) against
the fp64 backward oracle (oracle/backward.py: autograd through the
token-by-token scan, pinned by central differences of the C oracle).

Metric: per unit (per head for the batch-summed dW0, dgamma, dbeta),
max |got - oracle| / max |oracle| over the unit's entries, maxed over units.
The kernel computes in fp32; bound 1e-4 for fp32 inputs and 2e-2 for bf16
inputs (whose dq, dk, dv are rounded to bf16), as for the forward."""
import numpy as np
import pytest
import torch

import oracle
from linear_rnn_ttt_amd import _lib, ttt_linear_backward, ttt_linear_forward
from linear_rnn_ttt_amd.inputs import WORKLOADS, make_inputs
from oracle.backward import linear_backward

from _parity import TOL, from_dev, to_dev

pytestmark = pytest.mark.gpu

BF = WORKLOADS["linear_125m_b8h12_t2k"]
F32 = WORKLOADS["linear_b1h1_t256_f32"]
NAMES = ("dq", "dk", "dv", "deta", "dw0", "dgamma", "dbeta")


def unit_err(got, want, lead):
    got = np.asarray(got, np.float64).reshape(lead + (-1,))
    want = np.asarray(want, np.float64).reshape(lead + (-1,))
    num = np.abs(got - want).max(-1)
    den = np.maximum(np.abs(want).max(-1), 1e-30)
    return float((num / den).max())


def cotangents(inp, io, seed, final=True):
    B, H, T, d = inp["q"].shape
    rng = np.random.default_rng(seed)
    dz = rng.standard_normal((B, H, T, d)).astype(np.float32)
    if io == "bf16":
        dz = from_dev(to_dev(dz, "bf16"))      # the values the kernel sees
    dwT = (0.1 * rng.standard_normal((B, H, d, d))).astype(np.float32) if final else None
    return dz, dwT


def run_both(inp, io, dz, dwT, ln=True, res=True, eps=1e-6, per_batch=False):
    dev = {x: to_dev(inp[x], io if x in "qkv" else None) for x in
           ("q", "k", "v", "eta", "w0", "gamma", "beta")}
    out = ttt_linear_backward(dev["q"], dev["k"], dev["v"], dev["eta"], dev["w0"],
                              dev["gamma"], dev["beta"], to_dev(dz, io),
                              None if dwT is None else to_dev(dwT), eps=eps, layer_norm=ln,
                              residual=res, state0_per_batch=per_batch)
    torch.cuda.synchronize()
    got = dict(zip(NAMES, (from_dev(t) for t in out)))
    want = linear_backward(inp["q"], inp["k"], inp["v"], inp["eta"], inp["w0"], inp["gamma"],
                           inp["beta"], dz, dwT, mini_batch=16, layer_norm=ln, residual=res,
                           eps=eps, state0_per_batch=per_batch)
    return got, want


def errors(got, want, B, H, per_batch=False):
    e = {}
    for n in NAMES:
        lead = (B, H) if n in ("dq", "dk", "dv", "deta") or (n == "dw0" and per_batch) else (H,)
        e[n] = unit_err(got[n], want[n], lead)
    return e


@pytest.mark.parametrize("case", [
    ("f32 T=50", F32, "f32", 50, {}),
    ("f32 T=16", F32, "f32", 16, {}),
    ("f32 T=1", F32, "f32", 1, {}),
    ("f32 T=15", F32, "f32", 15, {}),
    ("f32 T=17", F32, "f32", 17, {}),
    ("f32 T=100 no LN", F32, "f32", 100, dict(ln=False)),
    ("f32 T=100 no residual", F32, "f32", 100, dict(res=False)),
    ("f32 T=100 Theorem-1 flags", F32, "f32", 100, dict(ln=False, res=False)),
    ("f32 T=47 per-batch W0", F32, "f32", 47, dict(per_batch=True)),
    ("f32 T=47 no dW_T", F32, "f32", 47, dict(final=False)),
    ("bf16 T=130", BF, "bf16", 130, {}),
    ("bf16 T=64 eps=1e-5", BF, "bf16", 64, dict(eps=1e-5)),
    ("bf16 T=33 no LN", BF, "bf16", 33, dict(ln=False)),
], ids=lambda c: c[0])
def test_backward_matches_the_oracle(case):
    name, wl, io, T, kw = case
    kw = dict(kw)
    final = kw.pop("final", True)
    per_batch = kw.get("per_batch", False)
    B, H = 2, 3
    inp = make_inputs(wl, B=B, H=H, T=T)
    if per_batch:
        rng = np.random.default_rng(9)
        inp["w0"] = (0.02 * rng.standard_normal((B, H, 64, 64))).astype(np.float32)
    dz, dwT = cotangents(inp, io, seed=T, final=final)
    got, want = run_both(inp, io, dz, dwT, **kw)
    e = errors(got, want, B, H, per_batch)
    print("%s: %s" % (name, " ".join("%s %.1e" % kv for kv in e.items())), flush=True)
    for n, v in e.items():
        if n in ("dgamma", "dbeta") and not kw.get("ln", True):
            assert not got[n].any(), n
            continue
        assert v <= TOL[io], (n, v)


def test_backward_is_deterministic_and_reuses_a_workspace():
    inp = make_inputs(BF, B=2, H=2, T=70)
    dz, dwT = cotangents(inp, "bf16", seed=1)
    dev = {x: to_dev(inp[x], "bf16" if x in "qkv" else None) for x in inp}
    args = (dev["q"], dev["k"], dev["v"], dev["eta"], dev["w0"], dev["gamma"], dev["beta"],
            to_dev(dz, "bf16"), to_dev(dwT))
    ws = torch.full((1 << 24,), 255, dtype=torch.uint8, device="cuda")
    a = ttt_linear_backward(*args, workspace=ws)
    b = ttt_linear_backward(*args, workspace=ws)
    c = ttt_linear_backward(*args)
    torch.cuda.synchronize()
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y) and torch.equal(x, z)
    with pytest.raises(_lib.TTTArgumentError) as e:
        ttt_linear_backward(*args, workspace=ws[:1000])
    assert e.value.code == _lib.TTT_ERR_SHAPE
    with pytest.raises(_lib.TTTArgumentError) as e:
        ttt_linear_backward(*args, mini_batch=32)
    assert e.value.code == _lib.TTT_ERR_UNSUPPORTED


def test_backward_full_size_sampled_heads():
    """The 1.3B-layer workload (B4 H32 T8192, bf16), one launch over every
    unit as the benchmark times it; two heads (all four batch entries each,
    so dW0, dgamma and dbeta are complete) against the oracle."""
    wl = WORKLOADS["linear_1p3b_b4h32_t8k"]
    inp = make_inputs(wl)
    dz, dwT = cotangents(inp, "bf16", seed=42)
    dev = {x: to_dev(inp[x], "bf16" if x in "qkv" else None) for x in inp}
    out = ttt_linear_backward(dev["q"], dev["k"], dev["v"], dev["eta"], dev["w0"],
                              dev["gamma"], dev["beta"], to_dev(dz, "bf16"), to_dev(dwT))
    torch.cuda.synchronize()
    got = dict(zip(NAMES, (from_dev(t) for t in out)))
    for n in ("dq", "dk", "dv", "deta"):
        assert np.isfinite(got[n]).all(), n
    for h in (0, 21):
        sl = slice(h, h + 1)
        sub = {x: (inp[x][:, sl] if x in ("q", "k", "v", "eta") else inp[x][sl])
               for x in ("q", "k", "v", "eta", "w0", "gamma", "beta")}
        want = linear_backward(sub["q"], sub["k"], sub["v"], sub["eta"], sub["w0"],
                               sub["gamma"], sub["beta"], dz[:, sl], dwT[:, sl])
        part = {n: (got[n][:, sl] if n in ("dq", "dk", "dv", "deta") else got[n][sl])
                for n in NAMES}
        e = errors(part, want, 4, 1)
        print("head %d: %s" % (h, " ".join("%s %.1e" % kv for kv in e.items())), flush=True)
        for n, v in e.items():
            assert v <= TOL["bf16"], (h, n, v)


@pytest.mark.parametrize("io,T", [("bf16", 77), ("f32", 50), ("bf16", 16)])
def test_forward_save_is_the_forward_and_stores_the_bases(io, T):
    """ttt_linear_forward_save: z and the final state bit for bit those of
    the one-workgroup forward; the stored base of mini-batch c equals the
    oracle's state after the first 16 c tokens."""
    wl = BF if io == "bf16" else F32
    B, H = 2, 2
    inp = make_inputs(wl, B=B, H=H, T=T)
    dev = {x: to_dev(inp[x], io if x in "qkv" else None) for x in inp}
    args = (dev["q"], dev["k"], dev["v"], dev["eta"], dev["w0"], dev["gamma"], dev["beta"])
    p = _lib.TTTParams(B, H, T, 64, 16, _lib.TTT_BF16 if io == "bf16" else _lib.TTT_F32, 0,
                       1e-6, 0)
    import ctypes
    need = int(_lib.lib().ttt_linear_backward_workspace_bytes(ctypes.byref(p)))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    z0, w0 = ttt_linear_forward(*args, split=False)
    z1, w1 = ttt_linear_forward(*args, save_for_backward=ws)
    torch.cuda.synchronize()
    assert torch.equal(z0, z1) and torch.equal(w0, w1)
    tiles = (T + 15) // 16
    bases = from_dev(ws[:B * H * tiles * 4096 * 4].view(torch.float32)).reshape(
        B, H, tiles, 64, 64)
    worst = 0.0
    for c in range(tiles):
        if c == 0:
            ref = np.broadcast_to(inp["w0"].astype(np.float64), (B, H, 64, 64))
        else:
            cut = {x: inp[x][:, :, :16 * c] for x in ("q", "k", "v", "eta")}
            _, ref = oracle.linear(cut["q"], cut["k"], cut["v"], cut["eta"], inp["w0"],
                                   inp["gamma"], inp["beta"])
        worst = max(worst, unit_err(bases[:, :, c], ref, (B, H)))
    print("%s T=%d: bases err %.2e" % (io, T, worst), flush=True)
    assert worst <= 1e-4


@pytest.mark.parametrize("case", [("f32", F32, 50, {}), ("bf16", BF, 70, {}),
                                  ("f32 no LN", F32, 33, dict(ln=False))],
                         ids=lambda c: c[0])
def test_backward_from_saved_bases_matches_the_oracle(case):
    name, wl, T, kw = case
    io = "bf16" if wl is BF else "f32"
    ln = kw.get("ln", True)
    B, H = 2, 3
    inp = make_inputs(wl, B=B, H=H, T=T)
    dz, dwT = cotangents(inp, io, seed=T + 5)
    dev = {x: to_dev(inp[x], io if x in "qkv" else None) for x in inp}
    args = (dev["q"], dev["k"], dev["v"], dev["eta"], dev["w0"], dev["gamma"], dev["beta"])
    ws = torch.full((1 << 22,), 255, dtype=torch.uint8, device="cuda")
    ttt_linear_forward(*args, layer_norm=ln, save_for_backward=ws)
    out = ttt_linear_backward(*args, to_dev(dz, io), to_dev(dwT), layer_norm=ln, workspace=ws,
                              bases_saved=True)
    torch.cuda.synchronize()
    got = dict(zip(NAMES, (from_dev(t) for t in out)))
    want = linear_backward(inp["q"], inp["k"], inp["v"], inp["eta"], inp["w0"], inp["gamma"],
                           inp["beta"], dz, dwT, layer_norm=ln)
    e = errors(got, want, B, H)
    print("%s: %s" % (name, " ".join("%s %.1e" % kv for kv in e.items())), flush=True)
    for n, v in e.items():
        if n in ("dgamma", "dbeta") and not ln:
            continue
        assert v <= TOL[io], (n, v)


def test_backward_from_saved_bases_full_size_one_head():
    """Forward with saved bases, then the backward without the replay, at
    the 1.3B-layer workload; head 5 (all four batch entries) vs the oracle."""
    wl = WORKLOADS["linear_1p3b_b4h32_t8k"]
    inp = make_inputs(wl)
    dz, _ = cotangents(inp, "bf16", seed=43, final=False)
    dev = {x: to_dev(inp[x], "bf16" if x in "qkv" else None) for x in inp}
    args = (dev["q"], dev["k"], dev["v"], dev["eta"], dev["w0"], dev["gamma"], dev["beta"])
    import ctypes
    p = _lib.TTTParams(4, 32, 8192, 64, 16, _lib.TTT_BF16, 0, 1e-6, 0)
    ws = torch.empty(int(_lib.lib().ttt_linear_backward_workspace_bytes(ctypes.byref(p))),
                     dtype=torch.uint8, device="cuda")
    ttt_linear_forward(*args, save_for_backward=ws)
    out = ttt_linear_backward(*args, to_dev(dz, "bf16"), workspace=ws, bases_saved=True)
    torch.cuda.synchronize()
    got = dict(zip(NAMES, (from_dev(t) for t in out)))
    h, sl = 5, slice(5, 6)
    want = linear_backward(inp["q"][:, sl], inp["k"][:, sl], inp["v"][:, sl], inp["eta"][:, sl],
                           inp["w0"][sl], inp["gamma"][sl], inp["beta"][sl], dz[:, sl])
    part = {n: (got[n][:, sl] if n in ("dq", "dk", "dv", "deta") else got[n][sl])
            for n in NAMES}
    e = errors(part, want, 4, 1)
    print("head %d from saved bases: %s" % (h, " ".join("%s %.1e" % kv for kv in e.items())),
          flush=True)
    for n, v in e.items():
        assert v <= TOL["bf16"], (n, v)
