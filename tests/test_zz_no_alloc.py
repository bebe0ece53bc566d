"""GPU check of ttt_linear_forward_split_noalloc (the two-workgroup TTT-Linear
scan with its scratch in the library's fixed per-device array) against
ttt_linear_forward_split (the same launch with a caller workspace): two
calls in a row, the second on a smaller problem, each bit-identical to the
workspace launch (same kernels) and within the bf16 tolerance of the
oracle."""
import numpy as np
import pytest
import torch

import oracle
from linear_rnn_ttt_amd import ttt_linear_forward, ttt_linear_forward_split_noalloc
from linear_rnn_ttt_amd.inputs import WORKLOADS, make_inputs

from _parity import TOL, from_dev, state_err, to_dev, z_err

pytestmark = pytest.mark.gpu


def _run(inp):
    dev = {k: to_dev(v, "bf16" if k in "qkv" else None) for k, v in inp.items()}
    args = [dev[x] for x in ("q", "k", "v", "eta", "w0", "gamma", "beta")]
    z_ref, w_ref = ttt_linear_forward(*args, split=True)
    z = torch.empty_like(dev["q"])
    w = torch.empty_like(w_ref)
    ttt_linear_forward_split_noalloc(*args, z=z, w_out=w)
    torch.cuda.synchronize()
    return z, w, z_ref, w_ref


def test_noalloc_matches_workspace_launch_twice():
    base = WORKLOADS["linear_1p3b_b4h32_t8k"]
    for B, H, T in ((2, 16, 3000), (1, 8, 700)):   # second call smaller
        print("noalloc split B%d H%d T%d" % (B, H, T), flush=True)
        inp = make_inputs(base, B=B, H=H, T=T)
        z, w, z_ref, w_ref = _run(inp)
        assert torch.equal(z, z_ref) and torch.equal(w, w_ref)
        zr, wr = oracle.linear(*(inp[x] for x in ("q", "k", "v", "eta", "w0", "gamma", "beta")))
        ez, ew = z_err(from_dev(z), zr), state_err(from_dev(w), wr)
        print("   bit-identical to the workspace launch; z err %.3e, state err %.3e"
              % (ez, ew), flush=True)
        assert ez <= TOL["bf16"] and ew <= TOL["bf16"]
