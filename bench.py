#!/usr/bin/env python3
"""Benchmark of the TTT-layer forward scan on one MI355X.

A step is one forward scan over the whole workload (every (batch, head)
unit, every token): one call of the Python op ttt_linear_forward (or
ttt_mlp_forward) as a user makes it, on inputs already resident in HBM.  For
TTT-Linear the op picks the one- or the two-workgroup launch by the unit
count and length (linear_uses_split); the JSON line names the one used.

Default workload: TTT-Linear at the 1.3B-model layer shape, B = 4, H = 32,
d = 64, T = 8192, mini-batch 16, bf16 q/k/v/z, fp32 state and eta (seeded
synthetic inputs, see linear_rnn_ttt_amd/inputs.py).

Output: one JSON line with the throughput (tokens/s = B*T per second), the
roofline of the scan kernel (algorithmic bytes or flops per launch over the
launch time measured with HIP events on the launch stream) and the fp64 CPU
oracle timed on the host cores.

Other timed modes: --backward (the scan's backward pass, --train with the
forward that saves the bases), --decode [--compact] (the streaming step),
--input (the input side: q, k, v projections and the learning-rate gate).

Summary modes (turn rocprofv3 output into the short summaries kept under
profiles/):
  --summarize-trace DIR                 a `rocprofv3 --kernel-trace --stats`
      run of this benchmark: per-kernel average durations;
  --summarize-pmc FETCH_DIR WRITE_DIR   two `rocprofv3 --pmc` runs (FETCH_SIZE,
      then WRITE_SIZE) of `bench.py --copy-calibration`: HBM traffic per
      launch, scaled by the same counters read on a plain 1 GiB copy.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TTT layer forward tokens/s at 1.3B shape T=8k; % MFMA/HBM roofline"
DEFAULT_WORKLOAD = "linear_1p3b_b4h32_t8k"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFS = 2500.0    # MI355X dense bf16 matrix
COPY_BYTES = 1 << 30           # calibration copy: 1 GiB read + 1 GiB written
KERNEL_SOURCES = {
    "linear": ["ttt_linear.hip", "ttt_tile.hpp", "ttt_device.hpp", "ttt_kernels.hpp",
               "ttt_args.hpp"],
    "mlp": ["ttt_mlp.hip", "ttt_tile.hpp", "ttt_device.hpp", "ttt_kernels.hpp", "ttt_args.hpp"],
    "decode": ["ttt_decode.hip", "ttt_device.hpp", "ttt_kernels.hpp", "ttt_args.hpp"],
    "backward": ["ttt_backward.hip", "ttt_backward.hpp", "ttt_device.hpp", "ttt_args.hpp",
                 "ttt_linear.hip", "ttt_tile.hpp", "ttt_kernels.hpp"],
    "decode_compact": ["ttt_decode_compact.hip", "ttt_stream.hpp", "ttt_device.hpp",
                       "ttt_args.hpp"],
    "mlp_decode": ["ttt_mlp_decode.hip", "ttt_stream.hpp", "ttt_device.hpp", "ttt_args.hpp"],
    "mlp_decode_compact": ["ttt_mlp_decode_compact.hip", "ttt_mlp_compact.hpp",
                           "ttt_device.hpp", "ttt_args.hpp"],
    "mlp_backward": ["ttt_mlp_backward.hip", "ttt_mlp_backward.hpp", "ttt_args.hpp",
                     "ttt_device.hpp"],
    "input": ["ttt_input.hip", "ttt_input.hpp", "ttt_args.hpp", "ttt_device.hpp"],
}
# Other kernels a call launches whose time and traffic belong to it (the
# TTT-Linear backward takes its 16-token mini-batch bases from the forward
# kernel).
CALL_EXTRA = {"backward": ["ttt_linear_fwd"]}
KERNEL_NAME = {"linear": "ttt_linear_fwd", "mlp": "ttt_mlp_fwd", "decode": "ttt_linear_decode_k",
               "backward": "ttt_linear_bwd_k", "decode_compact": "ttt_linear_decode_compact_k",
               "mlp_decode": "ttt_mlp_decode_k",
               "mlp_decode_compact": "ttt_mlp_decode_compact_k",
               "mlp_backward": "ttt_mlp_bwd_k", "input": "ttt_input_k"}
BACKWARD_METRIC = "TTT-Linear backward tokens/s at 1.3B shape T=8k; % fp32 MFMA roofline"
TRAIN_METRIC = ("TTT-Linear training step (forward saving the bases + backward) tokens/s at "
                "1.3B shape T=8k; % fp32 MFMA roofline of the backward")
MLP_BACKWARD_METRIC = "TTT-MLP backward tokens/s at 125M shape T=2k; % fp32 MFMA roofline"
INPUT_METRIC = ("TTT input side (q, k, v projections and the eta gate) tokens/s; "
                "% bf16 MFMA roofline")
DEFAULT_INPUT_WORKLOAD = "input_1p3b_b4_t8k"
# MI355X dense fp32 matrix (MFMA) rate: the roof of fp32-precision
# contractions; both backward kernels run their products on it.
FP32_MFMA_PEAK_TFS = 157.3
DECODE_METRIC = ("TTT-Linear streaming step tokens/s (one token per (batch, head) unit per "
                 "launch); % HBM roofline")
MLP_DECODE_METRIC = ("TTT-MLP streaming step tokens/s (one token per (batch, head) unit per "
                     "launch); % HBM roofline")


def kernel_hash(kind: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "linear_rnn_ttt_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def pmc_summary_path(kind: str, workload: str) -> str:
    return os.path.join(ROOT, "profiles", "%s_%s_hbm_traffic.md" % (KERNEL_NAME[kind], workload))


def algorithmic(w) -> dict:
    """What the method itself must move and compute per launch.

    Bytes: per token-head read q, k, v (3 d elements) and eta (4 B), write z
    (d elements); per head read the initial state once; per unit write the
    final state.  Flops: the three d x d (Linear) or seven d x 4d (MLP)
    products per token-head that the method defines (x W for the gradient
    point, its backward/update, and the output), 2 flops per multiply-add."""
    es = 2 if w.io == "bf16" else 4
    th = w.B * w.H * w.T
    d = w.d
    per_th = 4 * d * es + 4
    if w.kind == "linear":
        state = d * d * 4
        flops_th = 6 * d * d
    else:
        m = w.hidden
        state = (2 * d * m + m + d) * 4
        flops_th = 14 * d * m
    return {"bytes": th * per_th + w.H * state + w.B * w.H * state,
            "bytes_per_token_head": per_th, "state_bytes_per_unit": state,
            "flops": th * flops_th, "flops_per_token_head": flops_th}


def read_traffic(kind: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel source changed since."""
    path = pmc_summary_path(kind, workload)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256") != kernel_hash(kind):
        return None
    try:
        return int(float(vals["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def upload(inp, io):
    import torch

    dev = {}
    for k, v in inp.items():
        t = torch.from_numpy(v).cuda()
        dev[k] = t.to(torch.bfloat16) if (io == "bf16" and k in ("q", "k", "v")) else t
    return dev


def make_step(w, dev):
    from linear_rnn_ttt_amd import ttt_linear_forward, ttt_mlp_forward

    if w.kind == "linear":
        z, wo = ttt_linear_forward(dev["q"], dev["k"], dev["v"], dev["eta"], dev["w0"],
                                   dev["gamma"], dev["beta"], mini_batch=w.mini_batch,
                                   eps=w.eps)

        def step():
            ttt_linear_forward(dev["q"], dev["k"], dev["v"], dev["eta"], dev["w0"],
                               dev["gamma"], dev["beta"], mini_batch=w.mini_batch, eps=w.eps,
                               z=z, w_out=wo)
        return step, z
    z, so = ttt_mlp_forward(dev["q"], dev["k"], dev["v"], dev["eta"], dev["w1"], dev["b1"],
                            dev["w2"], dev["b2"], dev["gamma"], dev["beta"], eps=w.eps)

    def step():
        ttt_mlp_forward(dev["q"], dev["k"], dev["v"], dev["eta"], dev["w1"], dev["b1"],
                        dev["w2"], dev["b2"], dev["gamma"], dev["beta"], eps=w.eps, z=z,
                        state_out=so)
    return step, z


def launch_desc(w) -> str:
    if w.kind == "linear":
        from linear_rnn_ttt_amd.ops import linear_uses_split
        import torch
        if linear_uses_split(w.B, w.H, w.T,
                             dtype=torch.bfloat16 if w.io == "bf16" else torch.float32):
            return "ttt_linear_forward_split: two workgroups per (batch, head) unit"
        return "ttt_linear_forward: one workgroup per (batch, head) unit"
    return "ttt_mlp_forward: one workgroup per (batch, head) unit"


def cpu_baseline(w, inp, budget_s: float):
    """The fp64 oracle as it stands, on the host cores (at most 16 threads,
    the host share of one GPU).  The whole workload when it fits the
    budget, else a prefix of every unit's sequence; scaled to tokens/s."""
    import oracle

    cores = min(os.cpu_count() or 1, 16)
    # probe: every unit over its first 256 tokens, to size the sample
    units = w.B * w.H
    T_probe = min(w.T, 256)
    sub = lambda x, T: x[..., :T, :] if x.ndim == 4 else x[..., :T]
    args = lambda T: [sub(inp[k], T) for k in ("q", "k", "v", "eta")]
    t0 = time.perf_counter()
    if w.kind == "linear":
        oracle.linear(*args(T_probe), inp["w0"], inp["gamma"], inp["beta"],
                      mini_batch=w.mini_batch, eps=w.eps, n_threads=cores)
    else:
        oracle.mlp(*args(T_probe), inp["w1"], inp["b1"], inp["w2"], inp["b2"], inp["gamma"],
                   inp["beta"], mini_batch=w.mini_batch, eps=w.eps, n_threads=cores)
    probe = time.perf_counter() - t0
    est_full = probe * w.T / T_probe
    T_s = w.T if est_full <= budget_s else max(16, int(w.T * budget_s / est_full) // 16 * 16)
    # a short sample is repeated until about min(5 s, budget) of wall time;
    # the median run is reported
    times = []
    while not times or (sum(times) < min(5.0, budget_s) and len(times) < 50):
        t0 = time.perf_counter()
        if w.kind == "linear":
            oracle.linear(*args(T_s), inp["w0"], inp["gamma"], inp["beta"],
                          mini_batch=w.mini_batch, eps=w.eps, n_threads=cores)
        else:
            oracle.mlp(*args(T_s), inp["w1"], inp["b1"], inp["w2"], inp["b2"], inp["gamma"],
                       inp["beta"], mini_batch=w.mini_batch, eps=w.eps, n_threads=cores)
        times.append(time.perf_counter() - t0)
    dt = sorted(times)[len(times) // 2]
    sample = ("whole workload" if T_s == w.T else
              "all %d units, first %d of %d tokens each" % (units, T_s, w.T))
    return {"value": round(w.B * T_s / dt, 1), "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "sample": sample + ", median of %d runs of %.2f s wall, fp64"
            % (len(times), dt), **host_info()}


def copy_calibration():
    """A plain copy of known size, outside the timed region, for scaling the
    rocprofv3 FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def host_info() -> dict:
    """The host the CPU baseline ran on: logical CPUs and the CPU model."""
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


def side_measurements(step, stream, n: int = 5) -> dict:
    """Measurements beside the timed steps (not part of `value`):
    - cold launches: a 512 MB buffer is written before each launch (outside
      the launch's events), so the 256 MB MALL holds none of the inputs;
    - the achievable HBM bandwidth of a plain 1 GiB device-to-device copy,
      a second denominator beside the 8 TB/s peak."""
    import torch

    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold = []
    for _ in range(n):
        flush.fill_(1)
        s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_.record(stream)
        step()
        e_.record(stream)
        torch.cuda.synchronize()
        cold.append(s_.elapsed_time(e_))
    del flush
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s_.record(stream)
    for _ in range(n):
        dst.copy_(src)
    e_.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * COPY_BYTES * n / (s_.elapsed_time(e_) / 1e3) / 1e9   # read + write
    del src, dst
    cold.sort()
    return {"cold_median_launch_ms": round(cold[len(cold) // 2], 4),
            "hbm_copy_gbs": round(copy_gbs, 1)}


def run(args) -> dict:
    import torch

    from linear_rnn_ttt_amd.inputs import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    inp = make_inputs(w)
    dev = upload(inp, w.io)
    step, z = make_step(w, dev)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    if args.copy_calibration:
        copy_calibration()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        step()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [s.elapsed_time(e) for s, e in ev]
    avg_launch_s = sum(launch_ms) / len(launch_ms) / 1e3
    median_launch_ms = sorted(launch_ms)[len(launch_ms) // 2]
    side = side_measurements(step, stream)
    ms_per_step = wall / args.steps * 1e3
    ok = bool(torch.isfinite(z.float()).all().item())

    alg = algorithmic(w)
    if w.kind == "linear":
        achieved = alg["bytes"] / avg_launch_s / 1e9
        traffic = read_traffic(w.kind, w.name)
        cold_gbs = alg["bytes"] / (side["cold_median_launch_ms"] / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 5), "traffic": traffic,
                "kernel": KERNEL_NAME[w.kind], "avg_launch_ms": round(avg_launch_s * 1e3, 4),
                "median_launch_ms": round(median_launch_ms, 4),
                "algorithmic_bytes_per_launch": alg["bytes"],
                "cold_median_launch_ms": side["cold_median_launch_ms"],
                "cold_frac": round(cold_gbs / HBM_PEAK_GBS, 5),
                "hbm_copy_gbs": side["hbm_copy_gbs"],
                "frac_of_copy": round(achieved / side["hbm_copy_gbs"], 5)}
    else:
        achieved = alg["flops"] / avg_launch_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": BF16_MFMA_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_MFMA_PEAK_TFS, 5),
                "traffic": read_traffic(w.kind, w.name), "kernel": KERNEL_NAME[w.kind],
                "avg_launch_ms": round(avg_launch_s * 1e3, 4),
                "median_launch_ms": round(median_launch_ms, 4),
                "algorithmic_flops_per_launch": alg["flops"],
                "cold_median_launch_ms": side["cold_median_launch_ms"],
                "hbm_copy_gbs": side["hbm_copy_gbs"]}

    out = {
        "metric": METRIC,
        "value": round(w.B * w.T / (ms_per_step / 1e3), 1),
        "unit": "tokens/s",
        "token_heads_per_s": round(w.B * w.H * w.T / (ms_per_step / 1e3), 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.io == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "inner_model": "TTT-" + ("Linear" if w.kind == "linear"
                                                                 else "MLP"),
                   "B": w.B, "H": w.H, "T": w.T, "d": w.d, "mini_batch": w.mini_batch,
                   "io": w.io, "state": "fp32", "ln_eps": w.eps, "global_batch": w.B,
                   "seq_len": w.T, "parallelism": "none (1 GPU)", "launch": launch_desc(w)},
        "roofline": roof,
        "outputs_finite": ok,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_budget)
    return out


def decode_workload(args):
    """The streaming step's shape: the named workload's heads and head size
    with --batch streams (default: the workload's own batch)."""
    from linear_rnn_ttt_amd.inputs import WORKLOADS

    w = WORKLOADS[args.workload]
    if args.batch:
        w = w.with_(B=args.batch)
    return w


def decode_tag(w, compact=False) -> str:
    """Profile name of a streaming-step shape: streams, heads, I/O type."""
    return "streaming_%sb%dh%d_%s%s" % ("mlp_" if w.kind == "mlp" else "", w.B, w.H, w.io,
                                         "_compact" if compact else "")


def decode_compact_bytes(w) -> int:
    """Algorithmic bytes of one compact streaming step over all units,
    averaged over the b positions of a mini-batch: the base read (d^2 fp32
    for TTT-Linear, 2 d m + m + d for TTT-MLP), the history rows s < j read
    and row j written (2 d fp32 each for TTT-Linear, 2 d + 2 m for TTT-MLP),
    at j = 0 the fold (all b rows read, the base written), q, k, v read and z
    written (4 d io elements), eta (4 B)."""
    es = 2 if w.io == "bf16" else 4
    b, d = w.mini_batch, w.d
    if w.kind == "linear":
        base, row = d * d * 4, 2 * d * 4
    else:
        base, row = (2 * d * w.hidden + w.hidden + d) * 4, (2 * d + 2 * w.hidden) * 4
    per_pos = [base + (base + b * row if j == 0 else j * row) + row for j in range(b)]
    return w.B * w.H * (sum(per_pos) // b + 4 * d * es + 4)


def decode_bytes(w) -> int:
    """Algorithmic bytes of one streaming step over all units: the state read
    and written, the mini-batch base read or written (3 x the state: d^2
    fp32 for TTT-Linear, 2 d m + m + d fp32 for TTT-MLP), q, k, v read and z
    written (4 d io elements), eta (4 B)."""
    es = 2 if w.io == "bf16" else 4
    state = w.d * w.d if w.kind == "linear" else 2 * w.d * w.hidden + w.hidden + w.d
    return w.B * w.H * (3 * state * 4 + 4 * w.d * es + 4)


def decode_flops(w) -> int:
    """Multiply-adds x 2 of one streaming step over all units: TTT-Linear
    3 d^2 (k W, the update, q W); TTT-MLP 7 d m (k W1 and q W1, a W2 at the
    base and a_q W2 after the update, g W2^T, the two rank-1 updates)."""
    per = 3 * w.d * w.d if w.kind == "linear" else 7 * w.d * w.hidden
    return 2 * per * w.B * w.H


def run_decode(args) -> dict:
    """Streaming steps: B streams of H heads each take `steps` consecutive
    tokens, one ttt_linear_decode_step launch per token (pos = t mod the
    mini-batch size), with inputs and state resident in HBM.  The warm-up
    tokens run eagerly; the timed tokens are captured once into a HIP graph
    and replayed, as a generation loop launches them, so that the host's
    per-call argument checks stay out of the per-step time.  The launch time
    is the replay's event time over the steps (it includes the graph's
    launch gaps, so the bandwidth it gives is a lower bound)."""
    import torch

    from linear_rnn_ttt_amd import (ttt_linear_decode_step, ttt_linear_decode_step_compact,
                                    ttt_mlp_decode_step, ttt_mlp_decode_step_compact)
    from linear_rnn_ttt_amd.inputs import make_inputs

    w = decode_workload(args)
    compact = bool(getattr(args, "compact", False))
    n_tok = args.warmup + args.steps
    inp = make_inputs(w, T=max(w.mini_batch, n_tok))
    dev = upload(inp, w.io)
    B, H, d = w.B, w.H, w.d
    toks = [[dev[x][:, :, t].contiguous() for x in ("q", "k", "v", "eta")]
            for t in range(n_tok)]
    mlp = w.kind == "mlp"
    if mlp:
        S = [dev[x].expand((B, H) + dev[x].shape[1:]).contiguous()
             for x in ("w1", "b1", "w2", "b2")]
        Sb = [torch.zeros_like(x) for x in S]
        hist = torch.zeros((B, H, w.mini_batch, 2 * d + 2 * w.hidden), dtype=torch.float32,
                           device="cuda")
    else:
        W = dev["w0"].expand(B, H, d, d).contiguous()
        Wb = torch.zeros_like(W)
        hist = torch.zeros((B, H, w.mini_batch, 2, d), dtype=torch.float32, device="cuda")
    z = torch.empty((B, H, d), dtype=dev["q"].dtype, device="cuda")

    def step(t):
        q, k, v, eta = toks[t]
        if mlp and compact:   # S holds the base, hist the mini-batch's rows
            ttt_mlp_decode_step_compact(q, k, v, eta, S, hist, dev["gamma"], dev["beta"],
                                        pos=t % w.mini_batch, mini_batch=w.mini_batch, eps=w.eps,
                                        z=z)
        elif mlp:
            ttt_mlp_decode_step(q, k, v, eta, S, Sb, dev["gamma"], dev["beta"],
                                pos=t % w.mini_batch, mini_batch=w.mini_batch, eps=w.eps, z=z)
        elif compact:   # W holds the base, hist the mini-batch's rows
            ttt_linear_decode_step_compact(q, k, v, eta, W, hist, dev["gamma"], dev["beta"],
                                           pos=t % w.mini_batch, mini_batch=w.mini_batch,
                                           eps=w.eps, z=z)
        else:
            ttt_linear_decode_step(q, k, v, eta, W, Wb, dev["gamma"], dev["beta"],
                                   pos=t % w.mini_batch, mini_batch=w.mini_batch, eps=w.eps,
                                   z=z)

    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()
    if args.copy_calibration:
        copy_calibration()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t in range(args.warmup, n_tok):
            step(t)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    graph.replay()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_launch_s = start.elapsed_time(end) / args.steps / 1e3
    ms_per_step = wall / args.steps * 1e3
    byts = decode_compact_bytes(w) if compact else decode_bytes(w)
    kind = ("mlp_" if mlp else "") + ("decode_compact" if compact else "decode")
    achieved = byts / avg_launch_s / 1e9
    if mlp:
        launch = (("ttt_mlp_decode_step_compact" if compact else "ttt_mlp_decode_step") +
                  ": one 1024-thread workgroup per (stream, head) unit, steps replayed from one "
                  "HIP graph")
        pending = ("compact: base + the mini-batch's (k, u1, a, u2) rows" if compact
                   else "S and S_base")
    else:
        launch = (("ttt_linear_decode_step_compact" if compact else "ttt_linear_decode_step") +
                  ": one 256-thread workgroup per (stream, head) unit, steps replayed from one "
                  "HIP graph")
        pending = ("compact: base + the mini-batch's (k, u) rows" if compact else "W and W_base")
    out = {
        "metric": MLP_DECODE_METRIC if mlp else DECODE_METRIC,
        "value": round(B / (ms_per_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.io == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": decode_tag(w, compact),
                   "inner_model": "TTT-MLP" if mlp else "TTT-Linear", "streams": B,
                   "H": H, "d": d, "mini_batch": w.mini_batch, "io": w.io, "state": "fp32",
                   "parallelism": "none (1 GPU)", "pending_state": pending, "launch": launch},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 5),
                     "traffic": read_traffic(kind, decode_tag(w, compact)),
                     "kernel": KERNEL_NAME[kind],
                     "avg_launch_ms": round(avg_launch_s * 1e3, 5),
                     "algorithmic_bytes_per_launch": byts},
        "outputs_finite": bool(torch.isfinite(z.float()).all().item()),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_decode(w, inp, args.cpu_budget)
    return out


def cpu_baseline_decode(w, inp, budget_s: float):
    """The oracle's fp64 streaming step (one unit at a time, one core) over
    every unit for consecutive tokens, until the budget is spent (the drawn
    tokens are reused in turn once the stream runs past them)."""
    import numpy as np

    import oracle

    B, H, d = w.B, w.H, w.d
    if w.kind == "mlp":
        S = [[tuple(inp[x][h].astype(np.float64) for x in ("w1", "b1", "w2", "b2"))
              for h in range(H)] for _ in range(B)]
        Sb = [[None] * H for _ in range(B)]
    else:
        W = np.broadcast_to(inp["w0"].astype(np.float64), (B, H, d, d)).copy()
        Wb = np.zeros_like(W)
    t, t0 = 0, time.perf_counter()
    n_drawn = inp["q"].shape[2]
    while time.perf_counter() - t0 < budget_s:
        i = t % n_drawn
        for b in range(B):
            for h in range(H):
                tok = (inp["q"][b, h, i], inp["k"][b, h, i], inp["v"][b, h, i],
                       inp["eta"][b, h, i], inp["gamma"][h], inp["beta"][h])
                if w.kind == "mlp":
                    _, S[b][h], Sb[b][h] = oracle.mlp_decode_step(
                        S[b][h], Sb[b][h], *tok, pos=t % w.mini_batch, eps=w.eps)
                else:
                    _, W[b, h], Wb[b, h] = oracle.linear_decode_step(
                        W[b, h], Wb[b, h], *tok, pos=t % w.mini_batch, eps=w.eps)
        t += 1
    dt = time.perf_counter() - t0
    return {"value": round(B * t / dt, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "%d consecutive tokens of all %d units, %.2f s wall, fp64" % (
                t, B * H, dt)}


def backward_alg(w) -> dict:
    """What the backward itself must move and compute per launch.

    Bytes per token-head: q, k, v and dz read and dq, dk, dv written (7 d io
    elements), eta read and deta written (8 B); per head W0, gamma, beta read
    and their gradients written.  The mini-batch bases the kernel stores and
    reloads (2 x 16 KB per 16 tokens and unit) are its own choice and are not
    counted.  Flops per token-head: 10 d x d matrix-vector products, 2 flops
    per multiply-add -- the forward replay of the bases (k W and the update)
    and the eight products of the chunked adjoint (k W, q W, dO W^T, k A,
    g A^T, dh W^T, and the rank-1 updates q^T dO and k^T dh of A)."""
    es = 2 if w.io == "bf16" else 4
    th = w.B * w.H * w.T
    d = w.d
    per_th = 7 * d * es + 8
    per_head = 2 * (d * d + 2 * d) * 4
    return {"bytes": th * per_th + w.H * per_head, "bytes_per_token_head": per_th,
            "flops": th * 20 * d * d, "flops_per_token_head": 20 * d * d,
            "bases_bytes": 2 * w.B * w.H * ((w.T + 15) // 16) * d * d * 4}


def run_backward(args) -> dict:
    """One call of ttt_linear_backward over the whole workload per step
    (cotangent dz seeded N(0, 1) in the io dtype, no cotangent on the final
    state, as in a language model), inputs and a preallocated workspace
    resident in HBM.  The launch time is the event time of the call on its
    stream (the scan kernel and the small batch-sum kernel).

    With --train a step is the training step instead: the forward that
    stores the mini-batch bases (ttt_linear_forward_save, z and W_T written)
    and the backward from those bases (TTT_BASES_SAVED); the roofline is the
    backward call's, timed with events around it inside the step."""
    import numpy as np
    import torch

    from linear_rnn_ttt_amd import _lib, ttt_linear_backward
    from linear_rnn_ttt_amd.inputs import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    if w.kind == "mlp":
        return run_mlp_backward(args, w)
    inp = make_inputs(w)
    dev = upload(inp, w.io)
    dz = np.random.default_rng(w.seed + 1000).standard_normal(inp["q"].shape).astype(np.float32)
    dz_dev = torch.from_numpy(dz).cuda().to(dev["q"].dtype)
    p = _lib.TTTParams(w.B, w.H, w.T, w.d, w.mini_batch,
                       _lib.TTT_BF16 if w.io == "bf16" else _lib.TTT_F32, 0, w.eps, 0)
    import ctypes
    ws = torch.empty(int(_lib.lib().ttt_linear_backward_workspace_bytes(ctypes.byref(p))),
                     dtype=torch.uint8, device="cuda")
    args_ = (dev["q"], dev["k"], dev["v"], dev["eta"], dev["w0"], dev["gamma"], dev["beta"],
             dz_dev)

    train = bool(getattr(args, "train", False))
    from linear_rnn_ttt_amd import ttt_linear_forward
    z = torch.empty_like(dev["q"])
    w_T = torch.empty((w.B, w.H, w.d, w.d), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(s_=None, e_=None):
        if train:
            ttt_linear_forward(*args_[:7], mini_batch=w.mini_batch, eps=w.eps, z=z, w_out=w_T,
                               save_for_backward=ws)
        if s_ is not None:
            s_.record(stream)
        out = ttt_linear_backward(*args_, mini_batch=w.mini_batch, eps=w.eps, workspace=ws,
                                  bases_saved=train)
        if e_ is not None:
            e_.record(stream)
        return out

    for _ in range(args.warmup):
        out = step()
    torch.cuda.synchronize()
    if args.copy_calibration:
        copy_calibration()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_, e_ in ev:
        out = step(s_, e_)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_launch_s = sum(s_.elapsed_time(e_) for s_, e_ in ev) / len(ev) / 1e3
    ms_per_step = wall / args.steps * 1e3
    alg = backward_alg(w)
    tflops = alg["flops"] / avg_launch_s / 1e12
    res = {
        "metric": TRAIN_METRIC if train else BACKWARD_METRIC,
        "value": round(w.tokens / (ms_per_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",   # fp32 matrix-unit products, fp32 accumulation (bf16 io)
        "data": "synthetic",
        "config": {"workload": w.name + ("_train_step" if train else "_backward"),
                   "inner_model": "TTT-Linear", "B": w.B,
                   "H": w.H, "T": w.T, "d": w.d, "mini_batch": w.mini_batch, "io": w.io,
                   "parallelism": "none (1 GPU)",
                   "launch": ("ttt_linear_forward_save (one 768-thread workgroup per unit) + "
                              if train else "") +
                             ("ttt_linear_backward: " +
                              ("" if train else "the bases from the forward kernel (one "
                               "768-thread workgroup per unit), ") +
                              "front half of every 16-token tile (one 512-thread workgroup "
                              "per unit and tile), reverse walk (one 512-thread workgroup "
                              "per unit); fp32 matrix-unit products, bases and front "
                              "records in a workspace" +
                              (", bases stored by the forward" if train else "")
                              if w.mini_batch == 16 else
                              "ttt_linear_backward: one 512-thread workgroup per (batch, "
                              "head) unit, fp32 matrix-unit products, bases in a "
                              "workspace")},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3),
                     "peak": FP32_MFMA_PEAK_TFS, "unit": "TFLOP/s",
                     "frac": round(tflops / FP32_MFMA_PEAK_TFS, 5),
                     "traffic": read_traffic("backward", w.name + ("_train" if train else "")),
                     "kernel": KERNEL_NAME["backward"],
                     "avg_launch_ms": round(avg_launch_s * 1e3, 4),
                     "algorithmic_flops_per_launch": alg["flops"],
                     "algorithmic_bytes_per_launch": alg["bytes"],
                     "hbm_gbs_algorithmic": round(alg["bytes"] / avg_launch_s / 1e9, 1)},
        "outputs_finite": bool(all(torch.isfinite(t.float()).all().item() for t in out[:4])),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_backward(w, inp, dz, args.cpu_budget)
    return res


def mlp_backward_alg(w) -> dict:
    """What the TTT-MLP backward itself must move and compute per launch.

    Bytes per token-head: q, k, v and dz read and dq, dk, dv written (7 d io
    elements), eta read and deta written (8 B); per head the initial state
    (W1, b1, W2, b2) and gamma, beta read and their gradients written.  The
    mini-batch bases and intermediates the kernel keeps in its workspace are
    its own choice and are not counted.  Flops per token-head: 22 products of
    a row with a d x m (or m x d) matrix, 2 flops per multiply-add -- the
    forward (k W1, a W2, g_o W2^T, q W1, a_q W2 and the two state updates)
    and the fifteen of the chunked adjoint (dO_q W2^T, dp_q W1^T, k A1,
    a A2, g_p A1^T, g_o A2^T, du W2, do W2^T, dp W1^T and the five rank-1
    updates of the adjoint state)."""
    es = 2 if w.io == "bf16" else 4
    th = w.B * w.H * w.T
    d, m = w.d, w.hidden
    per_th = 7 * d * es + 8
    per_head = 2 * (2 * d * m + m + d + 2 * d) * 4
    return {"bytes": th * per_th + w.H * per_head, "bytes_per_token_head": per_th,
            "flops": th * 44 * d * m, "flops_per_token_head": 44 * d * m}


def run_mlp_backward(args, w) -> dict:
    import ctypes

    import numpy as np
    import torch

    from linear_rnn_ttt_amd import _lib, ttt_mlp_backward

    from linear_rnn_ttt_amd.inputs import make_inputs

    inp = make_inputs(w)
    dev = upload(inp, w.io)
    dz = np.random.default_rng(w.seed + 1000).standard_normal(inp["q"].shape).astype(np.float32)
    dz_dev = torch.from_numpy(dz).cuda().to(dev["q"].dtype)
    p = _lib.TTTParams(w.B, w.H, w.T, w.d, w.mini_batch,
                       _lib.TTT_BF16 if w.io == "bf16" else _lib.TTT_F32, 0, w.eps, 0)
    ws = torch.empty(int(_lib.lib().ttt_mlp_backward_workspace_bytes(ctypes.byref(p), w.hidden)),
                     dtype=torch.uint8, device="cuda")
    args_ = (dev["q"], dev["k"], dev["v"], dev["eta"], dev["w1"], dev["b1"], dev["w2"],
             dev["b2"], dev["gamma"], dev["beta"], dz_dev)
    stream = torch.cuda.current_stream()

    def step(s_=None, e_=None):
        if s_ is not None:
            s_.record(stream)
        out = ttt_mlp_backward(*args_, eps=w.eps, workspace=ws)
        if e_ is not None:
            e_.record(stream)
        return out

    for _ in range(args.warmup):
        out = step()
    torch.cuda.synchronize()
    if args.copy_calibration:
        copy_calibration()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_, e_ in ev:
        out = step(s_, e_)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_launch_s = sum(s_.elapsed_time(e_) for s_, e_ in ev) / len(ev) / 1e3
    ms_per_step = wall / args.steps * 1e3
    alg = mlp_backward_alg(w)
    tflops = alg["flops"] / avg_launch_s / 1e12
    res = {
        "metric": MLP_BACKWARD_METRIC,
        "value": round(w.tokens / (ms_per_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",   # fp32 matrix-unit products, fp32 accumulation
        "data": "synthetic",
        "config": {"workload": w.name + "_backward", "inner_model": "TTT-MLP", "B": w.B,
                   "H": w.H, "T": w.T, "d": w.d, "hidden": w.hidden,
                   "mini_batch": w.mini_batch, "io": w.io, "parallelism": "none (1 GPU)",
                   "launch": "ttt_mlp_backward: one 512-thread workgroup per (batch, head) "
                             "unit, forward replay then the reverse walk, fp32 matrix-unit "
                             "products over a per-unit workspace"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3),
                     "peak": FP32_MFMA_PEAK_TFS, "unit": "TFLOP/s",
                     "frac": round(tflops / FP32_MFMA_PEAK_TFS, 5),
                     "traffic": read_traffic("mlp_backward", w.name),
                     "kernel": KERNEL_NAME["mlp_backward"],
                     "avg_launch_ms": round(avg_launch_s * 1e3, 4),
                     "algorithmic_flops_per_launch": alg["flops"],
                     "algorithmic_bytes_per_launch": alg["bytes"],
                     "hbm_gbs_algorithmic": round(alg["bytes"] / avg_launch_s / 1e9, 1)},
        "outputs_finite": bool(all(torch.isfinite(t.float()).all().item() for t in out[:4])),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_mlp_backward(w, inp, dz, args.cpu_budget)
    return res


def input_workload(args):
    from linear_rnn_ttt_amd.inputs import INPUT_WORKLOADS

    name = args.workload if args.workload in INPUT_WORKLOADS else DEFAULT_INPUT_WORKLOAD
    return INPUT_WORKLOADS[name]


def input_alg(w) -> dict:
    """Algorithmic work of one input-side launch: flops 2 M D N (M = B T
    tokens, N = 3 H d + H output columns); bytes: x and the stacked weights
    read once (bf16), b_eta, q, k, v written (bf16) and eta (fp32)."""
    M, N = w.B * w.T, w.n_out
    flops = 2 * M * w.D * N
    bytes_ = M * w.D * 2 + N * w.D * 2 + w.H * 4 + 3 * M * w.H * w.d * 2 + M * w.H * 4
    return {"flops": flops, "bytes": bytes_, "flops_per_token": 2 * w.D * N}


def run_input(args) -> dict:
    import numpy as np
    import torch

    from linear_rnn_ttt_amd import ttt_input_projection
    from linear_rnn_ttt_amd.inputs import make_input_side

    w = input_workload(args)
    inp = make_input_side(w)
    x = torch.from_numpy(inp["x"]).cuda().to(torch.bfloat16)
    wi = torch.from_numpy(inp["w_in"]).cuda().to(torch.bfloat16)
    be = torch.from_numpy(inp["b_eta"]).cuda()
    eb = float(inp["eta_base"])
    out = ttt_input_projection(x, wi, be, heads=w.H, eta_base=eb, head_dim=w.d)
    stream = torch.cuda.current_stream()

    def step(s_=None, e_=None):
        if s_ is not None:
            s_.record(stream)
        ttt_input_projection(x, wi, be, heads=w.H, eta_base=eb, head_dim=w.d, out=out)
        if e_ is not None:
            e_.record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.copy_calibration:
        copy_calibration()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_, e_ in ev:
        step(s_, e_)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_launch_s = sum(s_.elapsed_time(e_) for s_, e_ in ev) / len(ev) / 1e3
    ms_per_step = wall / args.steps * 1e3
    alg = input_alg(w)
    tflops = alg["flops"] / avg_launch_s / 1e12
    res = {
        "metric": INPUT_METRIC,
        "value": round(w.tokens / (ms_per_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",   # bf16 matrix-unit products, fp32 accumulation
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "d_model": w.D, "H": w.H,
                   "d": w.d, "n_out": w.n_out, "parallelism": "none (1 GPU)",
                   "launch": "ttt_input_projection: one 512-thread workgroup per 256 x 128 "
                             "output tile, bf16 16x16x32 matrix-unit products"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3),
                     "peak": BF16_MFMA_PEAK_TFS, "unit": "TFLOP/s",
                     "frac": round(tflops / BF16_MFMA_PEAK_TFS, 5),
                     "traffic": read_traffic("input", w.name),
                     "kernel": KERNEL_NAME["input"],
                     "avg_launch_ms": round(avg_launch_s * 1e3, 4),
                     "algorithmic_flops_per_launch": alg["flops"],
                     "algorithmic_bytes_per_launch": alg["bytes"],
                     "hbm_gbs_algorithmic": round(alg["bytes"] / avg_launch_s / 1e9, 1)},
        "outputs_finite": bool(all(torch.isfinite(t.float()).all().item() for t in out)),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_input(w, inp, args.cpu_budget)
    return res


def cpu_baseline_input(w, inp, budget_s: float):
    """The fp64 input-side oracle on the first n tokens of batch entry 0, n
    doubled from 64 until a run takes a quarter of the budget; tokens/s."""
    from oracle.input_side import input_side

    n, dt = 32, 0.0
    while dt < budget_s / 4 and n < w.T:
        n *= 2
        t0 = time.perf_counter()
        input_side(inp["x"][:1, :n], inp["w_in"], inp["b_eta"], w.H, w.d, inp["eta_base"])
        dt = time.perf_counter() - t0
    return {"value": round(n / dt, 1), "unit": "tokens/s", "cores": _blas_threads(),
            "kind": "oracle",
            "sample": "batch entry 0, first %d tokens, %.2f s wall, fp64 numpy" % (n, dt)}


def _blas_threads() -> int:
    """Threads the fp64 matrix products may use (the BLAS pool; numpy does
    not report it, so the OpenMP / BLAS environment or the core count)."""
    for var in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS", "MKL_NUM_THREADS"):
        if os.environ.get(var, "").isdigit():
            return int(os.environ[var])
    return os.cpu_count() or 1


def cpu_baseline_mlp_backward(w, inp, dz, budget_s: float):
    """The fp64 TTT-MLP backward oracle on one unit (batch 0, head 0) for the
    first T_s tokens, T_s doubled from 64 until a run takes a quarter of the
    budget; scaled to the metric's unit (one unit is 1/H of a token)."""
    from oracle.backward import mlp_backward

    T_s, dt = 32, 0.0
    while dt < budget_s / 4 and T_s < w.T:
        T_s *= 2
        sl = (slice(0, 1), slice(0, 1), slice(0, T_s))
        t0 = time.perf_counter()
        mlp_backward(inp["q"][sl], inp["k"][sl], inp["v"][sl], inp["eta"][sl], inp["w1"][:1],
                     inp["b1"][:1], inp["w2"][:1], inp["b2"][:1], inp["gamma"][:1],
                     inp["beta"][:1], dz[sl], mini_batch=w.mini_batch, eps=w.eps)
        dt = time.perf_counter() - t0
    import torch
    return {"value": round(T_s / w.H / dt, 2), "unit": "tokens/s",
            "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": "unit (0, 0), first %d tokens, %.2f s wall, fp64 torch autograd" % (
                T_s, dt)}


def cpu_baseline_backward(w, inp, dz, budget_s: float):
    """The fp64 backward oracle on one unit (batch 0, head 0) for the first
    T_s tokens, T_s doubled from 256 until a run takes a quarter of the
    budget; scaled to the metric's unit (one unit is 1/H of a token)."""
    from oracle.backward import linear_backward

    T_s, dt = 128, 0.0
    while dt < budget_s / 4 and T_s < w.T:
        T_s *= 2
        sl = (slice(0, 1), slice(0, 1), slice(0, T_s))
        t0 = time.perf_counter()
        linear_backward(inp["q"][sl], inp["k"][sl], inp["v"][sl], inp["eta"][sl],
                        inp["w0"][:1], inp["gamma"][:1], inp["beta"][:1], dz[sl],
                        mini_batch=w.mini_batch, eps=w.eps)
        dt = time.perf_counter() - t0
    import torch
    return {"value": round(T_s / w.H / dt, 2), "unit": "tokens/s",
            "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": "unit (0, 0), first %d tokens, %.2f s wall, fp64 torch autograd" % (
                T_s, dt)}


# ---------------------------------------------------------------------------
# rocprofv3 summaries (rocprofv3 writes an SQLite database, run_results.db)

def _db(d: str):
    import sqlite3

    files = glob.glob(os.path.join(d, "**", "*results.db"), recursive=True)
    if not files:
        raise SystemExit("no rocprofv3 results database under %s" % d)
    return sqlite3.connect(sorted(files)[-1])


def _counter_per_dispatch(d, counter, reduce="sum"):
    """[(kernel name, dispatch id, value)] for one counter (summed, or the
    maximum, over the counter's instances within a dispatch)."""
    con = _db(d)
    return con.execute(
        "select kernel_name, dispatch_id, %s(value) from counters_collection "
        "where counter_name = ? group by dispatch_id order by dispatch_id" % reduce,
        (counter,)).fetchall()


PIPE_COUNTERS = ["SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_LDS",
                 "SQ_LDS_BANK_CONFLICT", "SQ_BUSY_CU_CYCLES", "SQ_WAVE_CYCLES", "SQ_INSTS_VALU",
                 "SQ_INSTS_MFMA", "GRBM_GUI_ACTIVE"]


def _per_call(rows):
    """Mean per call of a per-dispatch counter over [(kernel name, value)]:
    the mean over the dispatches of each kernel instance, summed over the
    instances (a call launches each instance once: the TTT-Linear backward's
    replay, front and reverse-walk roles; every other kernel has one)."""
    by = {}
    for n, v in rows:
        by.setdefault(n, []).append(v)
    return sum(sum(v) / len(v) for v in by.values())


def summarize_pipes(d, args, cmd, workgroups: int):
    """Pipe utilisation of the profiled kernel from one `rocprofv3 --pmc`
    pass of PIPE_COUNTERS.  The busy fractions are per busy CU: the active
    cycles of a pipe over SQ_BUSY_CU_CYCLES (the sum over the CUs of the
    cycles they hold work, about workgroups x kernel cycles here).
    GRBM_GUI_ACTIVE reads about 8x the kernel's cycles on this device (one
    count per XCD), so rocprofv3's derived VALUBusy / MfmaUtil formulas,
    which divide by it, read low by that factor; it is shown for the check."""
    kind, name, _, _ = _profiled(args)
    kname = KERNEL_NAME[kind]
    vals = {}
    for ctr in PIPE_COUNTERS:
        names = [kname] + CALL_EXTRA.get(kind, [])
        rows = [(n, v) for n, _, v in _counter_per_dispatch(
            d, ctr, "max" if ctr.startswith("GRBM") else "sum") if any(k in n for k in names)]
        vals[ctr] = _per_call(rows)
    busy = vals["SQ_BUSY_CU_CYCLES"]
    per_cu = busy / workgroups
    lines = [
        "# Pipe utilisation of `%s` on %s (rocprofv3 --pmc)" % (kname, name), "",
        "One counter pass of the benchmark:", "", "    " + cmd, "",
        "- kernel_source_sha256: `%s`" % kernel_hash(kind),
        "- counters (mean per dispatch): " + ", ".join(
            "%s %.4g" % (k, v) for k, v in vals.items()),
        "- workgroups per launch: %d" % workgroups,
        "- busy CU cycles per workgroup: %.4g (SQ_BUSY_CU_CYCLES / workgroups); "
        "GRBM_GUI_ACTIVE / 8 XCDs: %.4g" % (per_cu, vals["GRBM_GUI_ACTIVE"] / 8), "",
        "| pipe, per busy CU | fraction of cycles |", "|---|---|",
        "| VALU issuing (SQ_ACTIVE_INST_VALU) | %.1f %% |" % (
            100 * vals["SQ_ACTIVE_INST_VALU"] / busy),
        "| matrix unit busy, per SIMD (SQ_VALU_MFMA_BUSY_CYCLES / 4 SIMDs) | %.1f %% |" % (
            100 * vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (4 * busy)),
        "| LDS instructions active (SQ_ACTIVE_INST_LDS) | %.1f %% |" % (
            100 * vals["SQ_ACTIVE_INST_LDS"] / busy),
        "| LDS stalled on bank conflicts (SQ_LDS_BANK_CONFLICT) | %.1f %% |" % (
            100 * vals["SQ_LDS_BANK_CONFLICT"] / busy),
        "", "Instructions per workgroup and launch: VALU %.0f, MFMA %.0f." % (
            vals["SQ_INSTS_VALU"] / workgroups, vals["SQ_INSTS_MFMA"] / workgroups),
    ]
    return "\n".join(lines) + "\n"


def _profiled(args):
    """(kind, profile name, algorithmic bytes, algorithmic flops) per launch
    of the profiled kernel."""
    from linear_rnn_ttt_amd.inputs import WORKLOADS

    if args.decode:
        w = decode_workload(args)
        if args.compact:
            return (("mlp_" if w.kind == "mlp" else "") + "decode_compact", decode_tag(w, True),
                    decode_compact_bytes(w), decode_flops(w))
        return ("mlp_decode" if w.kind == "mlp" else "decode", decode_tag(w), decode_bytes(w),
                decode_flops(w))
    if args.input:
        w = input_workload(args)
        alg = input_alg(w)
        return "input", w.name, alg["bytes"], alg["flops"]
    if args.backward:
        w = WORKLOADS[args.workload]
        if w.kind == "mlp":
            alg = mlp_backward_alg(w)
            return "mlp_backward", w.name, alg["bytes"], alg["flops"]
        alg = backward_alg(w)
        return "backward", w.name + ("_train" if args.train else ""), alg["bytes"], alg["flops"]
    w = WORKLOADS[args.workload]
    alg = algorithmic(w)
    return w.kind, w.name, alg["bytes"], alg["flops"]


def summarize_trace(d, args, cmd):
    kind, name, alg_bytes, alg_flops = _profiled(args)
    con = _db(d)
    rows = con.execute("select name, total_calls, total_duration, average, percentage from "
                       "top_kernels order by total_duration desc limit 8").fetchall()
    lines = ["# Kernel trace: %s on %s (rocprofv3 --kernel-trace --stats)" % (
        KERNEL_NAME[kind], name), "", "Command:", "", "    " + cmd, "",
        "- kernel_source_sha256: `%s`" % kernel_hash(kind), "",
        "| kernel | calls | total (us) | average (us) | % of GPU time |", "|---|---|---|---|---|"]
    for name, calls, tot, avg, pct in rows:
        short = name if len(name) < 70 else name[:67] + "..."
        lines.append("| `%s` | %d | %.1f | %.2f | %.1f |" % (short, calls, tot, avg, pct))
    per_name = []
    for kn in [KERNEL_NAME[kind]] + CALL_EXTRA.get(kind, []):
        per_name += con.execute("select name, count(*), avg(duration) from kernels where name "
                                "like ? group by name order by name", ("%" + kn + "%",)
                                ).fetchall()
    k = con.execute("select count(*), avg(duration), min(duration), max(duration) from kernels "
                    "where name like ?", ("%" + KERNEL_NAME[kind] + "%",)).fetchone()
    if len(per_name) > 1:
        # one launch of each instance per call (the backward's replay, front
        # and reverse-walk roles): the call's time is the sum of their averages
        lines += ["", "Kernels of one call (one launch of each): %s" % ", ".join(
            [KERNEL_NAME[kind]] + CALL_EXTRA.get(kind, [])), ""]
        lines += ["- `%s`: %d launches, average %.2f us" % (n if len(n) < 90 else n[:87] + "...",
                                                             cnt, avg / 1e3)
                  for n, cnt, avg in per_name]
        avg_us = sum(avg for _, _, avg in per_name) / 1e3
        lines += ["", "Average %.2f us per call (sum over the instances); %d algorithmic bytes "
                  "per call -> %.1f GB/s (%.2f%% of 8 TB/s); %.3e algorithmic flops -> "
                  "%.2f TFLOP/s." % (avg_us, alg_bytes, alg_bytes / avg_us / 1e3,
                                     100 * alg_bytes / avg_us / 1e3 / HBM_PEAK_GBS, alg_flops,
                                     alg_flops / avg_us / 1e6)]
    elif k and k[0]:
        avg_us = k[1] / 1e3
        lines += ["", "Kernel %s: %d launches, average %.2f us (min %.2f, max %.2f)." % (
            KERNEL_NAME[kind], k[0], avg_us, k[2] / 1e3, k[3] / 1e3)]
        lines += ["", "Average %.2f us per launch; %d algorithmic bytes per launch "
                  "-> %.1f GB/s (%.2f%% of 8 TB/s); %.3e algorithmic flops -> %.2f TFLOP/s." % (
                      avg_us, alg_bytes, alg_bytes / avg_us / 1e3,
                      100 * alg_bytes / avg_us / 1e3 / HBM_PEAK_GBS, alg_flops,
                      alg_flops / avg_us / 1e6)]
    return "\n".join(lines) + "\n"


def summarize_pmc(fetch_dir, write_dir, args, cmd_fetch, cmd_write):
    kind, name, alg, _ = _profiled(args)
    kname = KERNEL_NAME[kind]
    fetch = _counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _counter_per_dispatch(write_dir, "WRITE_SIZE")
    names = [kname] + CALL_EXTRA.get(kind, [])
    kf = [(n, v) for n, _, v in fetch if any(k in n for k in names)]
    kw = [(n, v) for n, _, v in write if any(k in n for k in names)]
    # the 1 GiB device-to-device copy: the largest copyBuffer dispatch
    cf = max(v for n, _, v in fetch if "copyBuffer" in n)
    cw = max(v for n, _, v in write if "copyBuffer" in n)
    f_fetch = (COPY_BYTES / 1024.0) / cf
    f_write = (COPY_BYTES / 1024.0) / cw
    fetch_kib = _per_call(kf)
    write_kib = _per_call(kw)
    traffic = fetch_kib * 1024 * f_fetch + write_kib * 1024 * f_write
    lines = [
        "# HBM traffic of `%s` on %s (rocprofv3 --pmc)" % (kname, name),
        "",
        "Two counter runs of the benchmark (kernel launches plus one plain 1 GiB",
        "device-to-device copy whose counters scale the kernel's):",
        "",
        "    " + cmd_fetch,
        "    " + cmd_write,
        "",
        "- kernel_source_sha256: `%s`" % kernel_hash(kind),
        "- dispatches_measured: %d (FETCH_SIZE), %d (WRITE_SIZE)" % (len(kf), len(kw)),
        "- fetch_kib_per_dispatch: %.1f" % fetch_kib,
        "- write_kib_per_dispatch: %.1f" % write_kib,
        "- copy_fetch_kib (1 GiB copy): %.1f -> factor %.4f" % (cf, f_fetch),
        "- copy_write_kib (1 GiB copy): %.1f -> factor %.4f" % (cw, f_write),
        "- traffic_bytes_per_launch: %d" % int(traffic),
        "- algorithmic_bytes_per_launch: %d" % alg,
        "- traffic / algorithmic: %.3f" % (traffic / alg),
    ]
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0,
                    help="seconds of oracle wall time for the CPU baseline sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB copy before the timed region (counter scaling)")
    ap.add_argument("--decode", action="store_true",
                    help="time the TTT-Linear streaming step instead of the scan")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (of the workload's inner model) instead of "
                         "the forward scan")
    ap.add_argument("--compact", action="store_true",
                    help="with --decode: the compact pending state (base + mini-batch rows)")
    ap.add_argument("--train", action="store_true",
                    help="with --backward: time forward (saving the bases) + backward")
    ap.add_argument("--input", action="store_true",
                    help="time the input side (ttt_input_projection) on --workload "
                         "input_1p3b_b4_t8k (default) or input_125m_b8_t2k")
    ap.add_argument("--batch", type=int, default=0,
                    help="streams for --decode (default: the workload's batch)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--pmc-commands", nargs=2, default=["", ""])
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR")
    ap.add_argument("--summarize-pipes", nargs=2, metavar=("PMC_DIR", "WORKGROUPS"))
    ap.add_argument("--trace-command", default="")
    args = ap.parse_args(argv)

    if args.summarize_trace:
        sys.stdout.write(summarize_trace(args.summarize_trace, args, args.trace_command))
        return 0
    if args.summarize_pipes:
        sys.stdout.write(summarize_pipes(args.summarize_pipes[0], args, args.trace_command,
                                         int(args.summarize_pipes[1])))
        return 0
    if args.summarize_pmc:
        sys.stdout.write(summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1],
                                       args, *args.pmc_commands))
        return 0
    if args.gpus != 1:
        print("bench.py: the benchmark runs on exactly one GPU (the scan shards over "
              "independent (batch, head) units with no exchange; multi-GPU runs are not "
              "provided). Use --gpus 1.", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("bench.py: --steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2
    out = (run_decode(args) if args.decode else
           run_backward(args) if args.backward else
           run_input(args) if args.input else run(args))
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
