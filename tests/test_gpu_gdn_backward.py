"""GPU parity of the delta rule's backward pass (la_chunk_bwd, "gated_delta", bf16
inputs) against the fp64 oracle's reverse mode of the per-token recurrence:
every head-size pair over several chunks and a ragged tail, with and without the
gate (DeltaNet), edge lengths, with and without initial state and final-state
gradient, and every head of the delta-rule workload at full size. Every
gradient (q, k, v, log-gate, beta, initial state) is held to max|err| <= 2e-2
RMS of the oracle's, the bf16 rule."""
import numpy as np
import pytest
import torch

import chunkwise_linear_rnn_causal_amd as la
import oracle
import workloads as W
from gpu_util import TOL, assert_close, dev, host64

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dlog_gate", "dstate_in", "dbeta")


def _inputs(B, H, L, dk, dv, seed, with_state=True, gate=True):
    inp = W.make_chunk_inputs("gated_delta", "bf16", B, H, L, dk, dv, seed=seed, with_state=with_state)
    r = np.random.default_rng(seed + 2000)
    do = W.f32_to_bf16_bits(r.standard_normal((B, H, L, dv)).astype(np.float32))
    dso = r.normal(0.0, 0.1, size=(B, H, dk, dv)).astype(np.float32) if with_state else None
    lg = inp.log_gate if gate else None
    return inp, lg, do, dso


def _check(B, H, L, dk, dv, seed, with_state=True, gate=True, tag=""):
    print(f"[gdn-bwd] {tag} B{B} H{H} L{L} dk{dk} dv{dv} state={with_state} gate={gate}", flush=True)
    inp, lg, do, dso = _inputs(B, H, L, dk, dv, seed, with_state, gate)
    g = la.la_chunk_bwd("gated_delta", dev(inp.q), dev(inp.k), dev(inp.v), dev(do), dev(lg),
                        dev(inp.state_in), dev(dso), beta=dev(inp.beta), want_d_state_in=True)
    torch.cuda.synchronize()
    g = [host64(x) for x in g]
    ref = oracle.backward("gated_delta", inp.f64("q"), inp.f64("k"), inp.f64("v"), W.to_f64(do),
                          log_gate=None if lg is None else lg.astype(np.float64),
                          state_in=inp.f64("state_in"),
                          d_state_out=None if dso is None else dso.astype(np.float64),
                          beta=inp.f64("beta"))
    errs = {}
    for name, got, want in zip(NAMES, g, ref):
        if want is None or got is None or got.size == 0:
            continue
        errs[name] = assert_close(got, want, TOL["bf16"], name)
    return errs


@pytest.mark.parametrize("dk,dv", [(32, 32), (32, 64), (32, 128), (64, 32), (64, 64), (64, 128),
                                   (128, 32), (128, 64), (128, 128)])
def test_gdn_backward_matches_oracle(dk, dv):
    _check(2, 3, 3 * 64 + 17, dk, dv, seed=51)


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128)])
def test_gdn_backward_without_gate(dk, dv):
    """DeltaNet: no log-gate (alpha = 1), no gate gradient."""
    _check(2, 2, 150, dk, dv, seed=52, gate=False)


@pytest.mark.parametrize("L", [0, 1, 17, 63, 64, 65, 130])
def test_gdn_backward_edge_lengths(L):
    _check(1, 2, L, 64, 64, seed=53, tag="edge")


def test_gdn_backward_without_states():
    """No initial state and no final-state gradient."""
    _check(2, 2, 150, 128, 64, seed=54, with_state=False)


def test_gdn_backward_deterministic():
    inp, lg, do, dso = _inputs(2, 2, 200, 64, 128, seed=55)
    runs = []
    for _ in range(2):
        g = la.la_chunk_bwd("gated_delta", dev(inp.q), dev(inp.k), dev(inp.v), dev(do), dev(lg),
                            dev(inp.state_in), dev(dso), beta=dev(inp.beta), want_d_state_in=True)
        torch.cuda.synchronize()
        runs.append([host64(x) for x in g])
    for x, y in zip(*runs):
        assert np.array_equal(x, y)


def test_gdn_backward_full_size_all_heads():
    """The delta-rule workload (B2 H16 L8192 d128), every head against the oracle."""
    name = "gated_delta_bf16_b2h16_l8192_d128"
    c = W.CONFIGS[name]
    B, H, L, dk, dv = c["B"], c["H"], c["L"], c["dk"], c["dv"]
    print("[gdn-bwd] full size", flush=True)
    inp = W.config_chunk_inputs(name, seed=0)
    do = W.make_backward_dout("bf16", B, H, L, dv, seed=0)
    g = la.la_chunk_bwd("gated_delta", dev(inp.q), dev(inp.k), dev(inp.v), dev(do), dev(inp.log_gate),
                        beta=dev(inp.beta))
    torch.cuda.synchronize()
    ref = oracle.backward("gated_delta", inp.f64("q"), inp.f64("k"), inp.f64("v"), W.to_f64(do),
                          log_gate=inp.f64("log_gate"), beta=inp.f64("beta"), threads=8)
    for i, nm in enumerate(NAMES):
        if g[i] is None or ref[i] is None:
            continue
        e = assert_close(host64(g[i]), ref[i], TOL["bf16"], nm)
        print(f"[gdn-bwd] full size {nm} max|err|/RMS = {e:.2e}", flush=True)
