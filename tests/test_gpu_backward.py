"""GPU parity of the TTT-Linear backward pass (ttt_linear_backward) against
the fp64 backward oracle (oracle/backward.py: autograd through the
token-by-token scan, pinned by central differences of the C oracle).

Metric: per unit (per head for the batch-summed dW0, dgamma, dbeta),
max |got - oracle| / max |oracle| over the unit's entries, maxed over units.
The kernel computes in fp32; bound 1e-4 for fp32 inputs and 2e-2 for bf16
inputs (whose dq, dk, dv are rounded to bf16), as for the forward.

At the full 1.3B-layer workload every unit is held to the fp64 chunked
adjoint (tests/test_chunk_form_backward.py, itself held to the oracle at
1e-11), except where plain fp32 evaluations of that same adjoint miss the
tolerance too.  The backward of an ill-conditioned unit is so sensitive that
one fp32 evaluation is not a measure of what fp32 can reach: on unit (0,14)
the fp32 evaluation's dk error ranges from 3e-4 to 3e-2 when eta is moved
by one fp32 ulp, and the fp64 result itself by 6e-3
(tests/test_chunk_form_backward.py pins this).  So the fp32 envelope of a
unit is the largest error of ENVELOPE_SAMPLES fp32 evaluations (eta as
given, then moved by one ulp with seeded signs) against the fp64 result for
eta as given; a unit over the tolerance is exempt only where its envelope is
over the tolerance too, and is then held to FP32_MULT times the envelope."""
import numpy as np
import pytest
import torch

import oracle
from linear_rnn_ttt_amd import _lib, ttt_linear_backward, ttt_linear_forward
from linear_rnn_ttt_amd.inputs import WORKLOADS, make_inputs
from oracle.backward import linear_backward

from _parity import FP32_MULT, TOL, from_dev, to_dev
from test_chunk_form_backward import chunk_backward, ulp_perturbed

pytestmark = pytest.mark.gpu

BF = WORKLOADS["linear_125m_b8h12_t2k"]
F32 = WORKLOADS["linear_b1h1_t256_f32"]
NAMES = ("dq", "dk", "dv", "deta", "dw0", "dgamma", "dbeta")
ENVELOPE_SAMPLES = 8


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


def run_both(inp, io, dz, dwT, ln=True, res=True, eps=1e-6, per_batch=False, mb=16):
    dev = {x: to_dev(inp[x], io if x in "qkv" else None) for x in
           ("q", "k", "v", "eta", "w0", "gamma", "beta")}
    out = ttt_linear_backward(dev["q"], dev["k"], dev["v"], dev["eta"], dev["w0"],
                              dev["gamma"], dev["beta"], to_dev(dz, io),
                              None if dwT is None else to_dev(dwT), mini_batch=mb, eps=eps,
                              layer_norm=ln, residual=res, state0_per_batch=per_batch)
    torch.cuda.synchronize()
    got = dict(zip(NAMES, (from_dev(t) for t in out)))
    want = linear_backward(inp["q"], inp["k"], inp["v"], inp["eta"], inp["w0"], inp["gamma"],
                           inp["beta"], dz, dwT, mini_batch=mb, layer_norm=ln, residual=res,
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
    # mini-batches of several tiles (gradients at the mini-batch's base)
    ("f32 T=50 b=32", F32, "f32", 50, dict(mb=32)),
    ("f32 T=70 b=48 no residual", F32, "f32", 70, dict(mb=48, res=False)),
    ("f32 T=33 b=32 per-batch W0", F32, "f32", 33, dict(mb=32, per_batch=True)),
    ("f32 T=100 b=128 (batch GD over the sequence)", F32, "f32", 100, dict(mb=128)),
    ("f32 T=100 b=112 no LN, no dW_T", F32, "f32", 100, dict(mb=112, ln=False, final=False)),
    ("bf16 T=130 b=64", BF, "bf16", 130, dict(mb=64)),
    ("bf16 T=47 b=32 eps=1e-5", BF, "bf16", 47, dict(mb=32, eps=1e-5)),
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
    runs = [ttt_linear_backward(*args, workspace=ws) for _ in range(8)]   # ten runs in all
    runs.append(ttt_linear_backward(*args))
    torch.cuda.synchronize()
    for r in runs:
        for x, y in zip(a, r):
            assert torch.equal(x, y)
    with pytest.raises(_lib.TTTArgumentError) as e:
        ttt_linear_backward(*args, workspace=ws[:1000])
    assert e.value.code == _lib.TTT_ERR_SHAPE
    with pytest.raises(_lib.TTTArgumentError) as e:
        ttt_linear_backward(*args, mini_batch=24)
    assert e.value.code == _lib.TTT_ERR_UNSUPPORTED
    with pytest.raises(_lib.TTTArgumentError) as e:     # saved bases: 16-token mini-batches
        ttt_linear_backward(*args, mini_batch=32, workspace=ws, bases_saved=True)
    assert e.value.code == _lib.TTT_ERR_UNSUPPORTED


def test_theorem1_mode_backward():
    """Theorem-1 mode (no LN, no residual, b = T: batch GD from W0 over the
    causal prefix) on its own workload against the oracle, and dv against
    the closed form of that mode.  With eta = 1/2 and W0 = 0,
    z_i = sum_{s<=i} (q_i . k_s) v_s, so dv_s = sum_{i>=s} (q_i . k_s) dz_i."""
    wl = WORKLOADS["theorem1_b1h1_t256_f32"]
    inp = make_inputs(wl, B=1, H=2)
    dz, dwT = cotangents(inp, "f32", seed=256, final=False)
    got, want = run_both(inp, "f32", dz, dwT, ln=False, res=False, mb=wl.mini_batch)
    e = errors(got, want, 1, 2)
    print("Theorem-1 mode: %s" % " ".join("%s %.1e" % kv for kv in e.items()), flush=True)
    for n, v in e.items():
        if n in ("dgamma", "dbeta"):
            assert not got[n].any(), n
            continue
        assert v <= TOL["f32"], (n, v)
    q, k = inp["q"].astype(np.float64), inp["k"].astype(np.float64)
    S = np.triu(k @ np.swapaxes(q, -1, -2))              # [.., s, i] = k_s . q_i, i >= s
    dv = S @ dz.astype(np.float64)
    assert unit_err(got["dv"], dv, (1, 2)) <= TOL["f32"]


def _unit_ref(inp, dz, dwT, b, h, dtype, eta=None):
    """The chunked adjoint of unit (b, h) evaluated in `dtype` (eta: the
    unit's eta row to use instead of the input's)."""
    x = lambda a: np.asarray(a, dtype)
    return chunk_backward(x(inp["q"][b, h]), x(inp["k"][b, h]), x(inp["v"][b, h]),
                          x(inp["eta"][b, h] if eta is None else eta), x(inp["w0"][h]),
                          x(inp["gamma"][h]), x(inp["beta"][h]), x(dz[b, h]), x(dwT[b, h]),
                          16, True, True, 1e-6)


def _rel(got, ref):
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def test_backward_full_size_every_unit():
    """The 1.3B-layer workload (B4 H32 T8192, bf16), one launch over every
    unit as the benchmark times it; every unit (every head for dW0, dgamma,
    dbeta) against the fp64 chunked adjoint, with the fp32-envelope
    exemption described above; head 14 (the forward's worst-conditioned
    one) also against the autograd oracle itself."""
    wl = WORKLOADS["linear_1p3b_b4h32_t8k"]
    inp = make_inputs(wl)
    B, H, T, d = inp["q"].shape
    dz, dwT = cotangents(inp, "bf16", seed=42)
    dev = {x: to_dev(inp[x], "bf16" if x in "qkv" else None) for x in inp}
    out = ttt_linear_backward(dev["q"], dev["k"], dev["v"], dev["eta"], dev["w0"],
                              dev["gamma"], dev["beta"], to_dev(dz, "bf16"), to_dev(dwT))
    torch.cuda.synchronize()
    got = dict(zip(NAMES, (from_dev(t) for t in out)))
    for n in NAMES:
        assert np.isfinite(got[n]).all(), n
    per_tok = ("dq", "dk", "dv", "deta")
    per_head = ("dw0", "dgamma", "dbeta")
    ref = {n: np.zeros((B, H, T, d)) for n in ("dq", "dk", "dv")}
    ref["deta"] = np.zeros((B, H, T))
    ref.update(dw0=np.zeros((H, d, d)), dgamma=np.zeros((H, d)), dbeta=np.zeros((H, d)))
    for b in range(B):
        for h in range(H):
            r = _unit_ref(inp, dz, dwT, b, h, np.float64)
            for n in per_tok:
                ref[n][b, h] = r[n]
            for n in per_head:
                ref[n][h] += r[n]
    err = {n: np.array([[_rel(got[n][b, h], ref[n][b, h]) for h in range(H)] for b in range(B)])
           for n in per_tok}
    err.update({n: np.array([_rel(got[n][h], ref[n][h]) for h in range(H)]) for n in per_head})
    worst = {n: float(v.max()) for n, v in err.items()}
    print("every unit vs the chunked adjoint (worst): %s" % " ".join(
        "%s %.1e" % kv for kv in worst.items()), flush=True)
    tol = TOL["bf16"]
    bad_heads = sorted({h for n in per_tok for h in np.nonzero((err[n] > tol).any(0))[0]} |
                       {h for n in per_head for h in np.nonzero(err[n] > tol)[0]})
    for h in bad_heads:
        env = {n: np.zeros(B) for n in per_tok}
        env.update({n: 0.0 for n in per_head})
        for smp in range(ENVELOPE_SAMPLES):
            head_sum = {n: 0.0 for n in per_head}
            for b in range(B):
                eta = inp["eta"][b, h] if smp == 0 else ulp_perturbed(inp["eta"][b, h], smp)
                r = _unit_ref(inp, dz, dwT, b, h, np.float32, eta=eta)
                for n in per_tok:
                    env[n][b] = max(env[n][b], _rel(r[n], ref[n][b, h]))
                for n in per_head:
                    head_sum[n] = head_sum[n] + r[n].astype(np.float64)
            for n in per_head:
                env[n] = max(env[n], _rel(head_sum[n], ref[n][h]))
        for n in NAMES:
            cases = ([(b, err[n][b, h], env[n][b]) for b in range(B)] if n in per_tok
                     else [(None, err[n][h], env[n])])
            for b, e_gpu, e_env in cases:
                if e_gpu <= tol:
                    continue
                print("head %d unit %s %s: %.2e (fp32 envelope %.2e)" % (h, b, n, e_gpu, e_env),
                      flush=True)
                assert e_env > tol, (h, b, n, e_gpu, e_env)
                assert e_gpu <= FP32_MULT * e_env, (h, b, n, e_gpu, e_env)
    h, sl = 14, slice(14, 15)
    want = linear_backward(inp["q"][:, sl], inp["k"][:, sl], inp["v"][:, sl], inp["eta"][:, sl],
                           inp["w0"][sl], inp["gamma"][sl], inp["beta"][sl], dz[:, sl],
                           dwT[:, sl])
    mine = {n: (ref[n][:, sl] if n in per_tok else ref[n][sl]) for n in NAMES}
    part = {n: (got[n][:, sl] if n in per_tok else got[n][sl]) for n in NAMES}
    print("head %d vs the oracle: %s" % (h, " ".join(
        "%s %.1e" % kv for kv in errors(part, want, B, 1).items())), flush=True)
    assert max(errors(mine, want, B, 1).values()) <= 1e-9   # the chunked adjoint is the oracle


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


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_backward_without_saved_bases_is_the_training_path(io):
    """With 16-token mini-batches the backward takes its bases from the
    forward kernel itself, so a call without saved bases gives the same bits
    as ttt_linear_forward(save_for_backward=...) followed by the backward
    from those bases (ragged T, per-batch W0 too)."""
    wl = BF if io == "bf16" else F32
    for T, per_batch in ((70, False), (33, True)):
        inp = make_inputs(wl, B=2, H=3, T=T)
        if per_batch:
            inp["w0"] = np.stack([inp["w0"], 0.5 * inp["w0"]])
        dz, dwT = cotangents(inp, io, seed=T + 11)
        dev = {x: to_dev(inp[x], io if x in "qkv" else None) for x in inp}
        args = (dev["q"], dev["k"], dev["v"], dev["eta"], dev["w0"], dev["gamma"], dev["beta"])
        kw = dict(state0_per_batch=per_batch)
        a = ttt_linear_backward(*args, to_dev(dz, io), to_dev(dwT), **kw)
        ws = torch.full((1 << 22,), 255, dtype=torch.uint8, device="cuda")
        ttt_linear_forward(*args, save_for_backward=ws, **kw)
        b = ttt_linear_backward(*args, to_dev(dz, io), to_dev(dwT), workspace=ws,
                                bases_saved=True, **kw)
        torch.cuda.synchronize()
        for n, x, y in zip(NAMES, a, b):
            assert torch.equal(x, y), (T, n)


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


def test_backward_more_units_than_compute_units():
    """B*H = 320 units (more workgroups than the GPU holds at once), bf16,
    with a final-state cotangent, against the oracle."""
    B, H, T = 10, 32, 20
    inp = make_inputs(BF, B=B, H=H, T=T)
    dz, dwT = cotangents(inp, "bf16", seed=320)
    got, want = run_both(inp, "bf16", dz, dwT)
    e = errors(got, want, B, H)
    print("B10 H32 T20: %s" % " ".join("%s %.1e" % kv for kv in e.items()), flush=True)
    for n, v in e.items():
        assert v <= TOL["bf16"], (n, v)
