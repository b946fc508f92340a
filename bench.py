#!/usr/bin/env python3
"""Throughput of the chunkwise causal linear-attention path on one MI355X.

A step is one call of the hot path over one batch of synthetic input that is
already resident in HBM:
  - chunk workloads: one la_chunk_fwd (C = 64, the final state written; o in
    bf16 where bf16 output meets the bf16 tolerance at full size, the decay and
    delta-rule workloads, else fp32);
  - decode workload: 100 back-to-back la_decode_step calls (one "step" = 100
    tokens per sequence-head, as the workload is quoted).
  - short-convolution workload: one la_short_conv over q, k and v;
  - backward workload: one la_chunk_bwd (gradients of q, k, v and the gates).
The headline workload (the JSON line's value) is the largest single-GPU
workload, gated linear attention with data-dependent scalar decay at B=4, H=32,
L=8192, d=128; by default the other workloads are timed too and reported under
"workloads". Every workload is timed with HIP
events on the stream the kernels run on, over K timed steps after W warm-up steps.
Working sets below twice the 256 MB Infinity Cache are rotated over several
input copies so that the timed steps read HBM, not the cache.

Roofline: the algorithmic bytes and flops of one step (q, k, v, the gates read
once and o written once in bf16: the non-materialized lower bound; flop counts of
the chunkwise method, no credit for masking) divided by the measured time,
against 8 TB/s HBM and 2.517 PFLOP/s dense fp16/bf16 MFMA. The bytes the launch
actually moves (fp32 o where the workload keeps it, and the final state) are
reported beside them as "bytes_as_launched".
`traffic` is filled from profiles/traffic.json when its recorded kernel-source
hash matches the current sources, else null.

The CPU baseline times the fp64 oracle (tests' reference implementation) over the
whole headline workload on every core of the process's CPU affinity set.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       [--only] [--no-cpu-baseline] [--copy-calibration BYTES]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

HEADLINE = "decay_bf16_b4h32_l8192_d128"
METRIC = "tokens/sec + % bf16 MFMA peak (chunk fwd); decode state GB/s % of HBM peak"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2517.0     # 256 CU x 4096 flop/clk x 2.4 GHz, dense fp16/bf16
CACHE_BYTES = 256 * 2 ** 20   # Infinity Cache (MALL)
CSRC = os.path.join(ROOT, "chunkwise_linear_rnn_causal_amd", "csrc")


def kernel_source_hash() -> str:
    """Hash of the library sources (csrc/) with comments and blank lines removed, so
    that a counter record stays valid across comment-only edits and no longer."""
    import re
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        h.update("\n".join(l.rstrip() for l in src.splitlines() if l.strip()).encode())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# algorithmic work per step (chunkwise method: flops of the chunk products,
# bytes of every input read once and every output written once)
# ---------------------------------------------------------------------------
def o_dtype(c: dict) -> str:
    """Output dtype the workload is benchmarked (and tested at full size) with."""
    return c.get("o_dtype", "f32")


def chunk_work(c: dict) -> tuple[float, float, float]:
    """(flop, algorithmic bytes, bytes as launched) of one chunk forward.

    Algorithmic bytes: q, k, v and the gates read once, o written once in the
    input dtype (the non-materialized lower bound). As launched: o in the dtype
    the launch writes (fp32 where bf16 output would break the tolerance) plus
    the fp32 final state."""
    B, H, L, dk, dv, C = c["B"], c["H"], c["L"], c["dk"], c["dv"], c["C"]
    BH = B * H
    esz = 2 if c["dtype"] == "bf16" else 4
    if c["variant"] in ("gated_delta", "kda"):
        per_tok = (2 * C * C * (3 * dk + 2 * dv) + 6 * C * dk * dv + C ** 3 / 3) / C
    else:
        per_tok = 2 * C * (dk + dv) + 4 * dk * dv
    flop = per_tok * BH * L
    nbytes = BH * L * (2 * dk + dv) * esz                        # q, k, v in
    if c["variant"] in ("decay", "gated_delta"):
        nbytes += BH * L * 4                                     # log-gates
    if c["variant"] in ("vector_decay", "kda"):
        nbytes += BH * L * dk * 4                                # one log-gate per key channel
    if c["variant"] in ("gated_delta", "kda"):
        nbytes += BH * L * 4                                     # beta
    algo = nbytes + BH * L * dv * esz                            # o out in the input dtype
    launched = nbytes + BH * L * dv * (2 if o_dtype(c) == "bf16" else 4) + BH * dk * dv * 4
    return flop, algo, launched


def conv_work(c: dict) -> tuple[float, float]:
    """(flop, bytes) of one short convolution over q, k and v: each element read
    once and written once, K multiply-adds per output element; taps once."""
    BH, L, K = c["B"] * c["H"], c["L"], c["K"]
    esz = 2 if c["dtype"] == "bf16" else 4
    elems = BH * L * (2 * c["dk"] + c["dv"])
    flop = 2.0 * K * elems
    nbytes = 2 * elems * esz + c["H"] * (2 * c["dk"] + c["dv"]) * K * 4
    return flop, nbytes


def bwd_work(c: dict) -> tuple[float, float]:
    """(flop, bytes) of one backward pass: q, k, v, dO and the gates read once;
    dq, dk, dv and the gate gradient written once in fp32. Each forward product
    has two gradient products, so the flop count is twice the forward's."""
    B, H, L, dk, dv, C = c["B"], c["H"], c["L"], c["dk"], c["dv"], c["C"]
    BH = B * H
    esz = 2 if c["dtype"] == "bf16" else 4
    if c["variant"] == "gated_delta":
        fwd = (2 * C * C * (3 * dk + 2 * dv) + 6 * C * dk * dv + C ** 3 / 3) / C
    else:
        fwd = 2 * C * (dk + dv) + 4 * dk * dv
    flop = 2.0 * fwd * BH * L
    nbytes = BH * L * ((2 * dk + 2 * dv) * esz + (2 * dk + dv) * 4)
    if c["variant"] in ("decay", "gated_delta"):
        nbytes += 2 * BH * L * 4                                 # gates in, gate gradient out
    if c["variant"] == "vector_decay":
        nbytes += 2 * BH * L * dk * 4                            # per-channel gates in, their gradient out
    if c["variant"] == "gated_delta":
        nbytes += 2 * BH * L * 4                                 # beta in, its gradient out
    return flop, nbytes


def decode_work(c: dict) -> tuple[float, float]:
    """(flop, bytes) of ONE decode step over all sequence-heads: the fp32 state read
    and written, q, k, v in bf16, the fp32 log-gate, o out in bf16."""
    NH, dk, dv = c["N"] * c["H"], c["dk"], c["dv"]
    flop = 5.0 * dk * dv * NH                                    # gamma*S + k v^T, then S^T q
    nbytes = NH * (2 * dk * dv * 4 + (2 * dk + dv) * 2 + 4 + dv * 2)
    return flop, nbytes


# ---------------------------------------------------------------------------
def to_dev(x, device):
    import torch
    if x is None:
        return None
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def time_steps(fn, steps: int, warmup: int, stream):
    """Run fn(i) warmup times untimed, then exactly `steps` times inside one timed
    region bracketed by device synchronisation and a pair of HIP events recorded on
    `stream` (the stream every kernel of the step is launched on). Returns
    (event ms per step, wall ms per step)."""
    import torch
    for i in range(warmup):
        fn(i)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        fn(warmup + i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall * 1e3 / steps


def bench_chunk(name: str, steps: int, warmup: int, device) -> dict:
    import torch
    import chunkwise_linear_rnn_causal_amd as la
    c = W.CONFIGS[name]
    inp = W.config_chunk_inputs(name, seed=0)
    flop, nbytes, launched = chunk_work(c)
    copies = max(1, min(4, math.ceil(2 * CACHE_BYTES / launched)))
    odt = torch.bfloat16 if o_dtype(c) == "bf16" else torch.float32
    sets = []
    for _ in range(copies):
        s = dict(q=to_dev(inp.q, device), k=to_dev(inp.k, device), v=to_dev(inp.v, device),
                 lg=to_dev(inp.log_gate, device), beta=to_dev(inp.beta, device))
        s["o"] = torch.empty((c["B"], c["H"], c["L"], c["dv"]), dtype=odt, device=device)
        s["S"] = torch.empty((c["B"], c["H"], c["dk"], c["dv"]), dtype=torch.float32, device=device)
        dt = 1 if c["dtype"] == "bf16" else 0
        wsb = la.la_chunk_fwd_workspace_size(c["variant"], dt, c["B"], c["H"], c["L"], c["dk"], c["dv"], c["C"])
        s["ws"] = torch.empty(max(wsb, 1), dtype=torch.uint8, device=device) if wsb else None
        sets.append(s)
    stream = torch.cuda.current_stream(device)

    def step(i):
        s = sets[i % copies]
        la.la_chunk_fwd(c["variant"], s["q"], s["k"], s["v"], s["lg"], s["beta"], C=c["C"],
                        o=s["o"], state_out=s["S"], workspace=s["ws"], stream=stream)

    ms, wall_ms = time_steps(step, steps, warmup, stream)
    t = ms / 1e3
    toks = c["B"] * c["L"]
    return dict(workload=name, variant=c["variant"], tokens_per_s=toks / t, ms_per_step=t * 1e3,
                wall_ms_per_step=wall_ms, flop=flop, bytes=nbytes, bytes_as_launched=launched,
                output_dtype=o_dtype(c),
                achieved_gbs=nbytes / t / 1e9, achieved_tflops=flop / t / 1e12,
                launched_gbs=launched / t / 1e9,
                hbm_frac=nbytes / t / 1e9 / HBM_PEAK_GBS, mfma_frac=flop / t / 1e12 / MFMA_PEAK_TFLOPS,
                roofline_frac=max(nbytes / (HBM_PEAK_GBS * 1e9), flop / (MFMA_PEAK_TFLOPS * 1e12)) / t,
                input_copies=copies, B=c["B"], H=c["H"], L=c["L"], d_k=c["dk"], d_v=c["dv"], C=c["C"])


def bench_decode(name: str, steps: int, warmup: int, device, variant: str = "decay") -> dict:
    import torch
    import chunkwise_linear_rnn_causal_amd as la
    c = W.CONFIGS[name]
    N, H, dk, dv, nsteps = c["N"], c["H"], c["dk"], c["dv"], c["steps"]
    delta = variant == "gated_delta"
    S = to_dev(W.make_decode_state(N, H, dk, dv, seed=0), device)
    with ThreadPoolExecutor(min(16, len(os.sched_getaffinity(0)))) as ex:
        host = list(ex.map(lambda i: W.make_decode_step(N, H, dk, dv, step=i, seed=0, with_beta=delta),
                           range(nsteps)))
    ins = [(to_dev(h.q, device), to_dev(h.k, device), to_dev(h.v, device), to_dev(h.log_gate, device),
            to_dev(h.beta, device)) for h in host]
    # o in bf16 for the decay step (the workload's layout); the delta rule writes
    # fp32 o, because bf16 rounding of its output alone reaches the bf16 tolerance
    o = torch.empty((N, H, dv), dtype=torch.float32 if delta else torch.bfloat16, device=device)
    flop1, bytes1 = decode_work(c)
    if delta:  # + retrieval S^T k (2 d_k d_v flop), beta (4 bytes) and fp32 o per head
        flop1 += 2.0 * dk * dv * N * H
        bytes1 += 4 * N * H + 2 * dv * N * H
    stream = torch.cuda.current_stream(device)

    def step(_):
        for (q, k, v, lg, be) in ins:
            la.la_decode_step(variant, q, k, v, lg, S, o=o, beta=be, stream=stream)

    ms, wall_ms = time_steps(step, steps, warmup, stream)
    t = ms / 1e3                            # one step = nsteps decode launches
    t1 = t / nsteps
    # tokens: one new token per sequence per decode launch (all H heads of it)
    return dict(workload=name if not delta else name.replace("decode_decay", "decode_gated_delta"),
                variant=variant + "_decode", tokens_per_s=N * nsteps / t,
                ms_per_step=t * 1e3, ms_per_decode_launch=t1 * 1e3,
                wall_ms_per_step=wall_ms, flop=flop1 * nsteps, bytes=bytes1 * nsteps,
                achieved_gbs=bytes1 / t1 / 1e9, achieved_tflops=flop1 / t1 / 1e12,
                hbm_frac=bytes1 / t1 / 1e9 / HBM_PEAK_GBS, mfma_frac=None,
                roofline_frac=bytes1 / (HBM_PEAK_GBS * 1e9) / t1,
                N=N, H=H, d_k=dk, d_v=dv, decode_launches_per_step=nsteps)


def bench_convfwd(name: str, steps: int, warmup: int, device) -> dict:
    """The delta rule with the short convolution fused into its preparation
    (la_chunk_fwd_conv), and, for comparison on the same inputs, the unfused
    sequence la_short_conv then la_chunk_fwd (reported as unfused_ms_per_step)."""
    import torch
    import chunkwise_linear_rnn_causal_amd as la
    c = W.CONFIGS[name]
    B, H, L, dk, dv, K = c["B"], c["H"], c["L"], c["dk"], c["dv"], c["K"]
    inp = W.make_chunk_inputs(c["variant"], c["dtype"], B, H, L, dk, dv, seed=0, recipe=c["recipe"])
    taps = [to_dev(t, device) for t in W.make_conv_inputs(c["dtype"], 1, H, 1, dk, dv, K, seed=0).taps]
    gc = dict(c, kind="chunk")
    flop, nbytes, launched = chunk_work(gc)
    flop += 2.0 * K * (2 * dk + dv) * B * H * L
    copies = max(1, min(4, math.ceil(2 * CACHE_BYTES / launched)))
    sets = []
    for _ in range(copies):
        st = dict(q=to_dev(inp.q, device), k=to_dev(inp.k, device), v=to_dev(inp.v, device),
                  lg=to_dev(inp.log_gate, device), beta=to_dev(inp.beta, device))
        st["o"] = torch.empty((B, H, L, dv), dtype=torch.float32, device=device)
        st["S"] = torch.empty((B, H, dk, dv), dtype=torch.float32, device=device)
        sets.append(st)
    ws = torch.empty(la.la_chunk_fwd_conv_workspace_size(c["variant"], 1, B, H, L, dk, dv, c["C"], K),
                     dtype=torch.uint8, device=device)
    stream = torch.cuda.current_stream(device)

    def step(i):
        st = sets[i % copies]
        la.la_chunk_fwd_conv(c["variant"], st["q"], st["k"], st["v"], *taps, st["lg"], st["beta"], C=c["C"],
                             o=st["o"], state_out=st["S"], workspace=ws, stream=stream)

    ms, wall_ms = time_steps(step, steps, warmup, stream)
    # unfused: the standalone convolution into bf16 buffers, then the forward
    ys = [torch.empty_like(sets[0][x]) for x in ("q", "k", "v")]
    wsf = torch.empty(la.la_chunk_fwd_workspace_size(c["variant"], 1, B, H, L, dk, dv, c["C"]),
                      dtype=torch.uint8, device=device)

    def step_unfused(i):
        st = sets[i % copies]
        la.la_short_conv(st["q"], st["k"], st["v"], *taps, q_out=ys[0], k_out=ys[1], v_out=ys[2], stream=stream)
        la.la_chunk_fwd(c["variant"], ys[0], ys[1], ys[2], st["lg"], st["beta"], C=c["C"], o=st["o"],
                        state_out=st["S"], workspace=wsf, stream=stream)

    ms_u, _ = time_steps(step_unfused, steps, warmup, stream)
    t = ms / 1e3
    toks = B * L
    return dict(workload=name, variant="conv_" + c["variant"], tokens_per_s=toks / t, ms_per_step=t * 1e3,
                wall_ms_per_step=wall_ms, unfused_ms_per_step=ms_u, flop=flop, bytes=nbytes,
                bytes_as_launched=launched, output_dtype="f32",
                achieved_gbs=nbytes / t / 1e9, achieved_tflops=flop / t / 1e12,
                hbm_frac=nbytes / t / 1e9 / HBM_PEAK_GBS, mfma_frac=flop / t / 1e12 / MFMA_PEAK_TFLOPS,
                roofline_frac=max(nbytes / (HBM_PEAK_GBS * 1e9), flop / (MFMA_PEAK_TFLOPS * 1e12)) / t,
                input_copies=copies, B=B, H=H, L=L, d_k=dk, d_v=dv, C=c["C"], K=K)


def bench_conv(name: str, steps: int, warmup: int, device) -> dict:
    import torch
    import chunkwise_linear_rnn_causal_amd as la
    c = W.CONFIGS[name]
    ci = W.config_conv_inputs(name, seed=0)
    flop, nbytes = conv_work(c)
    copies = max(1, min(4, math.ceil(2 * CACHE_BYTES / nbytes)))
    taps = [to_dev(t, device) for t in ci.taps]
    sets = []
    for _ in range(copies):
        xs = [to_dev(x, device) for x in ci.x]
        ys = [torch.empty_like(x) for x in xs]
        sets.append((xs, ys))
    stream = torch.cuda.current_stream(device)

    def step(i):
        xs, ys = sets[i % copies]
        la.la_short_conv(*xs, *taps, q_out=ys[0], k_out=ys[1], v_out=ys[2], stream=stream)

    ms, wall_ms = time_steps(step, steps, warmup, stream)
    t = ms / 1e3
    toks = c["B"] * c["L"]
    return dict(workload=name, variant="short_conv_qkv", tokens_per_s=toks / t, ms_per_step=t * 1e3,
                wall_ms_per_step=wall_ms, flop=flop, bytes=nbytes,
                achieved_gbs=nbytes / t / 1e9, achieved_tflops=flop / t / 1e12,
                hbm_frac=nbytes / t / 1e9 / HBM_PEAK_GBS, mfma_frac=None,
                roofline_frac=nbytes / (HBM_PEAK_GBS * 1e9) / t, input_copies=copies,
                B=c["B"], H=c["H"], L=c["L"], d_k=c["dk"], d_v=c["dv"], K=c["K"])


def bench_bwd(name: str, steps: int, warmup: int, device) -> dict:
    import torch
    import chunkwise_linear_rnn_causal_amd as la
    c = W.CONFIGS[name]
    inp = W.make_chunk_inputs(c["variant"], c["dtype"], c["B"], c["H"], c["L"], c["dk"], c["dv"],
                              seed=0, recipe=c["recipe"])
    do = W.make_backward_dout(c["dtype"], c["B"], c["H"], c["L"], c["dv"], seed=0)
    flop, nbytes = bwd_work(c)
    q, k, v, lg, be, dO = (to_dev(x, device) for x in (inp.q, inp.k, inp.v, inp.log_gate, inp.beta, do))
    dt = 1 if c["dtype"] == "bf16" else 0
    ws = torch.empty(la.la_chunk_bwd_workspace_size(c["variant"], dt, c["B"], c["H"], c["L"], c["dk"],
                                                    c["dv"], c["C"]), dtype=torch.uint8, device=device)
    stream = torch.cuda.current_stream(device)

    def step(_):
        la.la_chunk_bwd(c["variant"], q, k, v, dO, lg, beta=be, workspace=ws, stream=stream)

    ms, wall_ms = time_steps(step, steps, warmup, stream)
    t = ms / 1e3
    toks = c["B"] * c["L"]
    return dict(workload=name, variant=c["variant"] + "_backward", tokens_per_s=toks / t,
                ms_per_step=t * 1e3, wall_ms_per_step=wall_ms, flop=flop, bytes=nbytes,
                achieved_gbs=nbytes / t / 1e9, achieved_tflops=flop / t / 1e12,
                hbm_frac=nbytes / t / 1e9 / HBM_PEAK_GBS, mfma_frac=flop / t / 1e12 / MFMA_PEAK_TFLOPS,
                roofline_frac=max(nbytes / (HBM_PEAK_GBS * 1e9), flop / (MFMA_PEAK_TFLOPS * 1e12)) / t,
                workspace_bytes=ws.numel(), B=c["B"], H=c["H"], L=c["L"], d_k=c["dk"], d_v=c["dv"],
                C=c["C"])


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(name: str, min_seconds: float = 10.0) -> dict:
    """Time the fp64 oracle over the whole workload on every core of the affinity set."""
    import oracle
    c = W.CONFIGS[name]
    inp = W.config_chunk_inputs(name, seed=0)
    args = [inp.f64(x) for x in ("q", "k", "v")]
    kw = dict(log_gate=inp.f64("log_gate"), beta=inp.f64("beta"))
    cores = len(os.sched_getaffinity(0))
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(c["variant"], *args, threads=cores, **kw)
        passes += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    toks = c["B"] * c["L"] * passes
    return dict(value=toks / el, unit="tokens/s", cores=cores, cpu_model=cpu_model(), kind="oracle",
                sample=f"whole workload ({c['B'] * c['H']} batch-heads x {c['L']} tokens), "
                       f"{passes} passes, {el:.1f} s wall, fp64 per-token recurrence, "
                       f"OpenMP over batch-heads on {cores} threads")


def traffic_for(workload: str):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("workloads", {}).get(workload, {}).get("hbm_bytes_per_launch")


def copy_calibration(nbytes: int) -> None:
    """A plain device-to-device copy of known size, for scaling the FETCH_SIZE /
    WRITE_SIZE counters (run under rocprofv3 --pmc)."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "launches": 3}))


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(W.CONFIGS))
    ap.add_argument("--only", action="store_true", help="time only --workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(independent batch-heads would shard across GPUs with no exchange).",
              file=sys.stderr)
        return 2
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return 0

    import torch
    import chunkwise_linear_rnn_causal_amd as la
    la.load_library()
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)

    names = [args.workload] if args.only else [args.workload] + [n for n in W.CONFIGS if n != args.workload]
    results = {}
    for name in names:
        kind = W.CONFIGS[name]["kind"]
        print(f"[bench] {name}", file=sys.stderr, flush=True)
        steps = args.steps if kind != "decode" else max(1, min(args.steps, 5))
        warm = args.warmup if kind != "decode" else max(1, min(args.warmup, 2))
        fn = {"chunk": bench_chunk, "decode": bench_decode, "conv": bench_conv, "bwd": bench_bwd,
              "convfwd": bench_convfwd}[kind]
        results[name] = fn(name, steps, warm, device)
        r = results[name]
        print(f"[bench] {name}: {r['ms_per_step']:.4f} ms/step, {r['achieved_gbs']:.0f} GB/s, "
              f"{r['achieved_tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        if kind == "decode" and not args.only:
            # the delta-rule decode step at the same shape (not one of the quoted workloads)
            r = bench_decode(name, steps, warm, device, variant="gated_delta")
            results[r["workload"]] = r
            print(f"[bench] {r['workload']}: {r['ms_per_step']:.4f} ms/step, {r['achieved_gbs']:.0f} GB/s",
                  file=sys.stderr, flush=True)
            torch.cuda.empty_cache()

    head = results[args.workload]
    c = W.CONFIGS[args.workload]
    bound = "hbm" if head["bytes"] / HBM_PEAK_GBS >= head["flop"] / 1e3 / MFMA_PEAK_TFLOPS else "mfma"
    if bound == "hbm":
        roof = dict(bound="hbm", achieved=head["achieved_gbs"], peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=head["achieved_gbs"] / HBM_PEAK_GBS)
    else:
        roof = dict(bound="mfma", achieved=head["achieved_tflops"], peak=MFMA_PEAK_TFLOPS,
                    unit="TFLOP/s", frac=head["achieved_tflops"] / MFMA_PEAK_TFLOPS)
    roof["traffic"] = traffic_for(args.workload)
    if "bytes_as_launched" in head:
        roof["algorithmic_bytes_per_launch"] = head["bytes"]
        roof["bytes_as_launched"] = head["bytes_as_launched"]
        roof["bytes_as_launched_note"] = ("o written in " + head["output_dtype"] +
                                          " plus the fp32 final state; frac uses the algorithmic bytes")

    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": args.workload, "variant": c.get("variant"), "B": c.get("B"),
                   "H": c.get("H"), "L": c.get("L"), "d_k": c["dk"], "d_v": c["dv"], "C": c.get("C"),
                   "inputs": c["dtype"], "mfma_operands": "f16" if c["dtype"] == "bf16" else "f32",
                   "accumulate": "f32", "output": o_dtype(c), "parallelism": "single-gpu"},
        "roofline": roof,
        "mfma": {"achieved": head["achieved_tflops"], "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": head["mfma_frac"]},
        "kernel_source_hash": kernel_source_hash(),
        "workloads": {n: {k: (round(v, 6) if isinstance(v, float) else v) for k, v in r.items()}
                      for n, r in results.items() if n != args.workload},
    }
    if not args.no_cpu_baseline and c["kind"] == "chunk":
        print("[bench] cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
