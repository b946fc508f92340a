"""GPU parity of the per-key-channel decay's backward pass (la_chunk_bwd,
"vector_decay", bf16 inputs) against the fp64 oracle's reverse mode of the
per-token recurrence: every head-size pair over several chunks and a ragged tail,
GLA-style and strong gates (the strong ones take the bf16 operand path), gates
below the clamp, edge lengths, with and without states, determinism, and every
head of the per-channel decay workload at full size. Every gradient (q, k, v,
the per-channel log-gates, the initial state) is held to max|err| <= 2e-2 RMS of
the oracle's, the bf16 rule."""
import numpy as np
import pytest
import torch

import chunkwise_linear_rnn_causal_amd as la
import oracle
import workloads as W
from gpu_util import TOL, assert_close, dev, host64

pytestmark = pytest.mark.gpu

VD = "vector_decay"
NAMES = ("dq", "dk", "dv", "dlog_gate", "dstate_in")


def _inputs(B, H, L, dk, dv, seed, with_state=True, recipe="gla"):
    inp = W.make_chunk_inputs(VD, "bf16", B, H, L, dk, dv, seed=seed, with_state=with_state, recipe=recipe)
    r = np.random.default_rng(seed + 3000)
    do = W.f32_to_bf16_bits(r.standard_normal((B, H, L, dv)).astype(np.float32))
    dso = r.normal(0.0, 0.1, size=(B, H, dk, dv)).astype(np.float32) if with_state else None
    return inp, do, dso


def _run(inp, do, dso, lg=None):
    lg = inp.log_gate if lg is None else lg
    g = la.la_chunk_bwd(VD, dev(inp.q), dev(inp.k), dev(inp.v), dev(do), dev(lg), dev(inp.state_in), dev(dso),
                        want_d_state_in=True)
    torch.cuda.synchronize()
    return [host64(x) for x in g]


def _ref(inp, do, dso, lg=None, threads=0):
    lg = inp.log_gate if lg is None else lg
    return oracle.backward(VD, inp.f64("q"), inp.f64("k"), inp.f64("v"), W.to_f64(do),
                           log_gate=lg.astype(np.float64), state_in=inp.f64("state_in"),
                           d_state_out=None if dso is None else dso.astype(np.float64), threads=threads)


def _check(B, H, L, dk, dv, seed, with_state=True, recipe="gla", tag=""):
    print(f"[vd-bwd] {tag} B{B} H{H} L{L} dk{dk} dv{dv} state={with_state} recipe={recipe}", flush=True)
    inp, do, dso = _inputs(B, H, L, dk, dv, seed, with_state, recipe)
    got = _run(inp, do, dso)
    ref = _ref(inp, do, dso)
    errs = {}
    for name, x, y in zip(NAMES, got, ref):
        if x is None or y is None or x.size == 0:
            continue
        errs[name] = assert_close(x, y, TOL["bf16"], name)
    return errs


@pytest.mark.parametrize("dk,dv", [(32, 32), (32, 64), (32, 128), (64, 32), (64, 64), (64, 128),
                                   (128, 32), (128, 64), (128, 128)])
@pytest.mark.parametrize("recipe", ["gla", "gla_strong"])
def test_vector_decay_backward_matches_oracle(dk, dv, recipe):
    """B=2, H=3, L = 3*64 + 17 with an initial state and a final-state gradient;
    GLA gates (log sigmoid(x)/16) and strong gates spread over [-10, 0]."""
    _check(2, 3, 3 * 64 + 17, dk, dv, seed=61, recipe=recipe)


@pytest.mark.parametrize("L", [0, 1, 17, 63, 64, 65, 130])
def test_vector_decay_backward_edge_lengths(L):
    _check(1, 2, L, 64, 64, seed=62, tag="edge")


def test_vector_decay_backward_without_states():
    """No initial state and no final-state gradient."""
    _check(2, 2, 150, 128, 64, seed=63, with_state=False)


def test_vector_decay_backward_gates_below_the_clamp():
    """Gates far below -10 are taken as -10 (as in the forward); the gradients
    stay within the bf16 tolerance of the oracle, which uses them as given."""
    inp, do, dso = _inputs(2, 2, 3 * 64 + 29, 128, 64, seed=64, recipe="gla_strong")
    lg = inp.log_gate.copy()
    lg[..., ::8] = -30.0
    lg[:, :, 70:75, :] = -60.0
    got = _run(inp, do, dso, lg)
    ref = _ref(inp, do, dso, lg)
    for name, x, y in zip(NAMES, got, ref):
        assert_close(x, y, TOL["bf16"], name)


def test_vector_decay_backward_uniform_gate_is_scalar_decay():
    """The same gate on every key channel is the scalar decay: the per-channel
    gate gradient summed over the channels is the scalar one, and dq, dk, dv agree
    with the scalar backward."""
    inp = W.make_chunk_inputs("decay", "bf16", 2, 2, 200, 64, 64, seed=65, with_state=True)
    r = np.random.default_rng(65)
    do = W.f32_to_bf16_bits(r.standard_normal((2, 2, 200, 64)).astype(np.float32))
    lg_vec = np.repeat(inp.log_gate[..., None], 64, axis=-1)
    args = (dev(inp.q), dev(inp.k), dev(inp.v), dev(do))
    gv = la.la_chunk_bwd(VD, *args, dev(lg_vec), dev(inp.state_in), want_d_state_in=True)
    gs = la.la_chunk_bwd("decay", *args, dev(inp.log_gate), dev(inp.state_in), want_d_state_in=True)
    torch.cuda.synchronize()
    gv, gs = [host64(x) for x in gv], [host64(x) for x in gs]
    for i, nm in enumerate(("dq", "dk", "dv")):
        assert_close(gv[i], gs[i], TOL["bf16"], nm)
    assert_close(gv[3].sum(-1), gs[3], TOL["bf16"], "summed gate gradient")
    assert_close(gv[4], gs[4], TOL["bf16"], "dstate_in")


def test_vector_decay_backward_deterministic():
    inp, do, dso = _inputs(2, 2, 200, 64, 128, seed=66)
    a = _run(inp, do, dso)
    b = _run(inp, do, dso)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_vector_decay_backward_full_size_all_heads():
    """The per-channel decay workload (B4 H32 L8192 d128), every head against the
    oracle, with the output gradient the backward workload uses."""
    name = "vector_decay_bf16_b4h32_l8192_d128"
    c = W.CONFIGS[name]
    B, H, L, dk, dv = c["B"], c["H"], c["L"], c["dk"], c["dv"]
    print("[vd-bwd] full size", flush=True)
    inp = W.config_chunk_inputs(name, seed=0)
    do = W.make_backward_dout("bf16", B, H, L, dv, seed=0)
    g = la.la_chunk_bwd(VD, dev(inp.q), dev(inp.k), dev(inp.v), dev(do), dev(inp.log_gate))
    torch.cuda.synchronize()
    g = [host64(x) if x is not None else None for x in g]
    print("[vd-bwd] full size: oracle", flush=True)
    ref = oracle.backward(VD, inp.f64("q"), inp.f64("k"), inp.f64("v"), W.to_f64(do),
                          log_gate=inp.f64("log_gate"), threads=16)
    for i, nm in enumerate(NAMES[:4]):
        e = assert_close(g[i], ref[i], TOL["bf16"], nm)
        print(f"[vd-bwd] full size {nm} max|err|/RMS = {e:.2e}", flush=True)
