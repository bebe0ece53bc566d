"""The two-workgroup TTT-Linear launch (ttt_linear_forward_split) against
the one-workgroup launch (ttt_linear_forward).  The output workgroup replays
the state updates from the gradient stream with the same products, in the
same order, as the update waves of the one-workgroup kernel, so z and the
final state must agree bit for bit; the one-workgroup launch is itself
checked against the oracle in test_gpu_linear.py.  Also: workspace reuse and
the unit-count limit on a GPU."""
import numpy as np
import pytest
import torch

from linear_rnn_ttt_amd import _lib, ttt_linear_forward
from linear_rnn_ttt_amd.inputs import WORKLOADS, make_inputs

from _parity import to_dev

pytestmark = pytest.mark.gpu

BASE = WORKLOADS["linear_125m_b8h12_t2k"]
F32 = WORKLOADS["linear_b1h1_t256_f32"]


def _dev(inp, io):
    return [to_dev(inp[x], io) for x in "qkv"] + [to_dev(inp[x]) for x in
                                                  ("eta", "w0", "gamma", "beta")]


def _both(args, **kw):
    zf, wf = ttt_linear_forward(*args, split=False, **kw)
    zs, ws = ttt_linear_forward(*args, split=True, **kw)
    torch.cuda.synchronize()
    return zf, wf, zs, ws


def _assert_same(name, zf, wf, zs, ws):
    dz = (zf.float() - zs.float()).abs().max().item()
    dw = (wf - ws).abs().max().item()
    print("%s: split vs one-workgroup max |dz| %.3e, |dW| %.3e" % (name, dz, dw), flush=True)
    assert torch.isfinite(zs.float()).all()
    assert torch.equal(zf, zs) and torch.equal(wf, ws)


@pytest.mark.parametrize("case", [
    ("bf16 ragged", BASE, dict(B=2, H=3, T=597), {}),
    ("bf16 one block", BASE, dict(B=1, H=2, T=40), {}),
    ("bf16 one tile", BASE, dict(B=1, H=1, T=16), {}),
    ("bf16 one token", BASE, dict(B=1, H=1, T=1), {}),
    ("f32 ragged", F32, dict(B=2, H=2, T=300), {}),
    ("bf16 b=64", BASE, dict(B=2, H=2, T=500), dict(mini_batch=64)),
    ("f32 b=T", F32, dict(B=1, H=2, T=200), dict(mini_batch=208)),
    ("bf16 no LN", BASE, dict(B=1, H=2, T=333), dict(layer_norm=False)),
    ("bf16 no residual", BASE, dict(B=1, H=2, T=333), dict(residual=False)),
    ("f32 linear model", F32, dict(B=1, H=2, T=150), dict(layer_norm=False, residual=False)),
], ids=lambda c: c[0])
def test_split_equals_one_workgroup(case):
    name, w, shape, kw = case
    inp = make_inputs(w, **shape)
    _assert_same(name, *_both(_dev(inp, w.io), **kw))


def test_split_per_batch_state_and_eps():
    inp = make_inputs(BASE, B=2, H=2, T=300)
    inp["w0"] = np.ascontiguousarray(
        np.stack([inp["w0"], 1.5 * inp["w0"][::-1]])).astype(np.float32)
    _assert_same("per-batch W0 eps=1e-5",
                 *_both(_dev(inp, "bf16"), eps=1e-5, state0_per_batch=True))


@pytest.mark.parametrize("name", ["linear_125m_b8h12_t2k", "linear_1p3b_b4h32_t8k",
                                  "linear_long_b1h32_t32k"])
def test_split_equals_one_workgroup_full_size(name):
    w = WORKLOADS[name]
    _assert_same(name, *_both(_dev(make_inputs(w), w.io)))


def test_split_reuses_a_workspace():
    """One workspace for consecutive calls: the counters are cleared by each
    launch and the stream is rewritten before it is read, so a second call
    (other inputs, shorter sequence) sees nothing of the first."""
    a = make_inputs(BASE, B=2, H=2, T=700)
    b = make_inputs(WORKLOADS["linear_1p3b_b4h32_t8k"], B=2, H=2, T=450)
    p = _lib.TTTParams(2, 2, 700, 64, 16, _lib.TTT_BF16, 0, 1e-6, 0)
    import ctypes
    need = int(_lib.lib().ttt_linear_split_workspace_bytes(ctypes.byref(p)))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for label, inp in (("first", a), ("second", b), ("first again", a)):
        args = _dev(inp, "bf16")
        zf, wf = ttt_linear_forward(*args, split=False)
        zs, wss = ttt_linear_forward(*args, split=True, workspace=ws)
        torch.cuda.synchronize()
        _assert_same("reused workspace, " + label, zf, wf, zs, wss)
        units = 4
        assert ws[units * 256: units * 256 + 128].view(torch.int32).eq(0).all()  # error words


def test_split_rejects_more_units_than_half_the_compute_units():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    H = cus // 2 + 1
    inp = make_inputs(BASE, B=1, H=H, T=32)
    with pytest.raises(_lib.TTTArgumentError) as e:
        ttt_linear_forward(*_dev(inp, "bf16"), split=True)
    assert e.value.code == _lib.TTT_ERR_UNSUPPORTED


def test_split_refuses_in_place_resume_and_auto_falls_back():
    inp = make_inputs(BASE, B=1, H=2, T=4096)
    inp["w0"] = np.ascontiguousarray(np.stack([inp["w0"]])).astype(np.float32)
    args = _dev(inp, "bf16")
    w0 = args[4]
    with pytest.raises(_lib.TTTArgumentError) as e:
        ttt_linear_forward(*args, split=True, state0_per_batch=True, w_out=w0)
    assert e.value.code == _lib.TTT_ERR_ALIAS
    ref_z, ref_w = ttt_linear_forward(*args, split=False, state0_per_batch=True)
    z, wf = ttt_linear_forward(*args, state0_per_batch=True, w_out=w0)   # auto: one workgroup
    torch.cuda.synchronize()
    assert torch.equal(z, ref_z) and torch.equal(wf, ref_w) and wf.data_ptr() == w0.data_ptr()
