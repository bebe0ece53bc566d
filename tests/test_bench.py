"""Host logic of bench.py (no GPU): the algorithmic byte and flop counts every
roofline fraction divides by, recounted here by hand from what each launch
must read and write, and the one-GPU contract of the command line."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from linear_rnn_ttt_amd.inputs import INPUT_WORKLOADS, WORKLOADS  # noqa: E402


def test_scan_counts_of_the_headline_workload():
    """B4 H32 T8192, d = 64, bf16 I/O: q, k, v read and z written (2 bytes
    each), eta read (4 bytes) per token and head; W0 read per head and the
    final state written per unit (fp32); 6 d^2 flops per token and head."""
    w = WORKLOADS["linear_1p3b_b4h32_t8k"]
    token_heads = 4 * 32 * 8192
    by_hand = token_heads * (4 * 64 * 2 + 4) + 32 * 64 * 64 * 4 + 4 * 32 * 64 * 64 * 4
    alg = bench.algorithmic(w)
    assert alg["bytes"] == by_hand == 543_686_656
    assert alg["flops"] == token_heads * 6 * 64 * 64


def test_scan_counts_of_the_mlp_workload():
    """B8 H12 T2048, hidden 256: the state is W1, b1, W2, b2 in fp32, and
    the method's seven d x 4d products per token cost 14 d 4d flops."""
    w = WORKLOADS["mlp_125m_b8h12_t2k"]
    token_heads = 8 * 12 * 2048
    state = (64 * 256 + 256 + 256 * 64 + 64) * 4
    alg = bench.algorithmic(w)
    assert alg["bytes"] == token_heads * 516 + 12 * state + 96 * state == 115_743_744
    assert alg["flops"] == token_heads * 14 * 64 * 256 == 45_097_156_608


def test_streaming_step_counts():
    """One token per unit: W and W_base move (read W, write W, read or write
    W_base: 3 d^2 fp32), plus q, k, v, z and eta; the compact form reads the
    base and the rows before position j and writes row j (2 d fp32 per row),
    and at j = 0 folds the 16 rows into the base (read them, write the base)."""
    w = WORKLOADS["linear_1p3b_b4h32_t8k"].with_(B=256)
    units = 256 * 32
    io = 4 * 64 * 2 + 4
    assert bench.decode_bytes(w) == units * (3 * 64 * 64 * 4 + io)
    base, row = 64 * 64 * 4, 2 * 64 * 4
    positions = [base + (base + 16 * row if j == 0 else j * row) + row for j in range(16)]
    per_unit = sum(positions) // 16 + io
    assert per_unit == 22_788
    assert bench.decode_compact_bytes(w) == units * per_unit


def test_backward_counts():
    """Backward per token and head: q, k, v, dz read and dq, dk, dv written,
    eta read and deta written; 20 d^2 flops (the replay's two products and the
    adjoint's eight d x d matrix-vector products)."""
    w = WORKLOADS["linear_1p3b_b4h32_t8k"]
    alg = bench.backward_alg(w)
    assert alg["bytes_per_token_head"] == 7 * 64 * 2 + 8
    assert alg["flops"] == 4 * 32 * 8192 * 20 * 64 * 64
    m = bench.mlp_backward_alg(WORKLOADS["mlp_125m_b8h12_t2k"])
    assert m["flops"] == 8 * 12 * 2048 * 44 * 64 * 256


def test_input_side_counts():
    """x [B T, D] times the stacked weights [3 H d + H, D]: 2 M D N flops;
    bytes x and the weights (bf16), b_eta, q, k, v (bf16) and eta (fp32)."""
    w = INPUT_WORKLOADS["input_1p3b_b4_t8k"]
    M, D, H, d = 4 * 8192, 2048, 32, 64
    N = 3 * H * d + H
    alg = bench.input_alg(w)
    assert alg["flops"] == 2 * M * D * N
    assert alg["bytes"] == M * D * 2 + N * D * 2 + H * 4 + 3 * M * H * d * 2 + M * H * 4


def test_kernel_hashes_cover_existing_sources():
    for kind, files in bench.KERNEL_SOURCES.items():
        for f in files:
            assert os.path.exists(os.path.join(ROOT, "linear_rnn_ttt_amd", "csrc", f)), (kind, f)
        assert len(bench.kernel_hash(kind)) == 16


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n, capsys):
    assert bench.main(["--gpus", str(n)]) == 2
    assert "exactly one GPU" in capsys.readouterr().err
