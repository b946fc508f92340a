"""GPU parity of the backward pass (la_chunk_bwd) against the fp64 oracle's
reverse-mode gradients: several chunks and a ragged tail at every head size,
edge lengths, with and without initial state and final-state gradient, and
sampled heads of the decay workload at full size. Every gradient is compared
with the normwise rule of its input dtype (bf16 2e-2, fp32 1e-4 of RMS)."""
import numpy as np
import pytest
import torch

import chunkwise_linear_rnn_causal_amd as la
import oracle
import workloads as W
from gpu_util import TOL, assert_close, dev, host64

pytestmark = pytest.mark.gpu


def _grad_inputs(var, dt, B, H, L, dk, dv, seed, with_state=True):
    inp = W.make_chunk_inputs(var, dt, B, H, L, dk, dv, seed=seed, with_state=with_state)
    r = np.random.default_rng(seed + 1000)
    do32 = r.standard_normal((B, H, L, dv)).astype(np.float32)
    do = W.f32_to_bf16_bits(do32) if dt == "bf16" else do32
    dso = r.normal(0.0, 0.1, size=(B, H, dk, dv)).astype(np.float32) if with_state else None
    return inp, do, dso


def _run(inp, do, dso, var, want_dsi=True):
    outs = la.la_chunk_bwd(var, dev(inp.q), dev(inp.k), dev(inp.v), dev(do), dev(inp.log_gate),
                           dev(inp.state_in), dev(dso), want_d_state_in=want_dsi)
    torch.cuda.synchronize()
    return [host64(x) for x in outs]


def _oracle(inp, do, dso, var):
    return oracle.backward(var, inp.f64("q"), inp.f64("k"), inp.f64("v"), W.to_f64(do),
                           log_gate=inp.f64("log_gate"), state_in=inp.f64("state_in"),
                           d_state_out=None if dso is None else dso.astype(np.float64))


def _cases():
    out = []
    for var in ("plain", "decay"):
        for dt in ("bf16", "f32"):
            for dk, dv in [(32, 32), (64, 64), (128, 128), (64, 128), (128, 32), (32, 128)]:
                if dt == "f32" and not (dk * dv <= 4096 or dk + dv == 160):
                    continue
                out.append((var, dt, dk, dv))
    return out


@pytest.mark.parametrize("var,dt,dk,dv", _cases(), ids=lambda x: str(x))
def test_backward_matches_oracle(var, dt, dk, dv):
    inp, do, dso = _grad_inputs(var, dt, 2, 3, 3 * 64 + 17, dk, dv, seed=41)
    g = _run(inp, do, dso, var)
    ref = _oracle(inp, do, dso, var)
    for name, got, want in zip(("dq", "dk", "dv", "dlog_gate", "dstate_in"), g, ref):
        if want is None or got is None:
            continue
        assert_close(got, want, TOL[dt], name)


@pytest.mark.parametrize("var", ["plain", "decay"])
@pytest.mark.parametrize("L", [0, 1, 17, 63, 64, 65, 130])
def test_backward_edge_lengths(var, L):
    inp, do, dso = _grad_inputs(var, "f32", 1, 2, L, 64, 64, seed=42)
    g = _run(inp, do, dso, var)
    ref = _oracle(inp, do, dso, var)
    for name, got, want in zip(("dq", "dk", "dv", "dlog_gate", "dstate_in"), g, ref):
        if want is None or got is None or got.size == 0:
            continue
        assert_close(got, want, TOL["f32"], name)


@pytest.mark.parametrize("var", ["plain", "decay"])
def test_backward_without_states(var):
    """No initial state and no final-state gradient."""
    inp, do, _ = _grad_inputs(var, "bf16", 2, 2, 150, 128, 64, seed=43, with_state=False)
    g = _run(inp, do, None, var, want_dsi=False)
    ref = _oracle(inp, do, None, var)
    for name, got, want in zip(("dq", "dk", "dv", "dlog_gate"), g[:4], ref[:4]):
        if want is None or got is None:
            continue
        assert_close(got, want, TOL["bf16"], name)


def test_backward_deterministic():
    inp, do, dso = _grad_inputs("decay", "bf16", 2, 2, 200, 64, 128, seed=44)
    a = _run(inp, do, dso, "decay")
    b = _run(inp, do, dso, "decay")
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_backward_full_size_decay_sampled_heads():
    """The decay workload (B4 H32 L8192 d128) in the launch the benchmark times;
    three sampled batch-heads against the oracle."""
    c = W.CONFIGS["decay_bf16_b4h32_l8192_d128"]
    B, H, L, dk, dv = c["B"], c["H"], c["L"], c["dk"], c["dv"]
    print("[bwd] full size", flush=True)
    inp = W.config_chunk_inputs("decay_bf16_b4h32_l8192_d128", seed=0)
    do = W.make_backward_dout("bf16", B, H, L, dv, seed=0)
    g = la.la_chunk_bwd("decay", dev(inp.q), dev(inp.k), dev(inp.v), dev(do), dev(inp.log_gate))
    torch.cuda.synchronize()
    heads = [(0, 0), (B - 1, H - 1), (1, 7)]
    ref_in = W.config_chunk_inputs("decay_bf16_b4h32_l8192_d128", seed=0, heads=heads)
    do_h = np.stack([do[b, h] for b, h in heads])[None]
    ref = oracle.backward("decay", ref_in.f64("q"), ref_in.f64("k"), ref_in.f64("v"), W.to_f64(do_h),
                          log_gate=ref_in.f64("log_gate"))
    for i, name in enumerate(("dq", "dk", "dv", "dlog_gate")):
        got = np.stack([host64(g[i][b, h]) for b, h in heads])[None]
        e = assert_close(got, ref[i], TOL["bf16"], name)
        print(f"[bwd] {name} err={e:.2e}", flush=True)


# ---- normalized variant: the plain backward of do / den plus the normalizer term

def _norm_run(inp, do, dso, dzo, want=True):
    g = la.la_chunk_bwd("normalized", dev(inp.q), dev(inp.k), dev(inp.v), dev(do), None, dev(inp.state_in),
                        dev(dso), z_in=dev(inp.z_in), d_z_out=dev(dzo), want_d_state_in=want, want_d_z_in=want)
    torch.cuda.synchronize()
    return [host64(x) for x in g]


def _norm_ref(inp, do, dso, dzo):
    return oracle.backward("normalized", inp.f64("q"), inp.f64("k"), inp.f64("v"), W.to_f64(do),
                           state_in=inp.f64("state_in"), z_in=inp.f64("z_in"),
                           d_state_out=None if dso is None else dso.astype(np.float64),
                           d_z_out=None if dzo is None else dzo.astype(np.float64))


def _norm_case(dt, B, H, L, dk, dv, seed, with_state=True):
    inp = W.make_chunk_inputs("normalized", dt, B, H, L, dk, dv, seed=seed, with_state=with_state,
                              with_z=with_state)
    r = np.random.default_rng(seed + 1000)
    do32 = r.standard_normal((B, H, L, dv)).astype(np.float32)
    do = W.f32_to_bf16_bits(do32) if dt == "bf16" else do32
    dso = r.normal(0.0, 0.1, size=(B, H, dk, dv)).astype(np.float32) if with_state else None
    dzo = r.normal(0.0, 0.1, size=(B, H, dk)).astype(np.float32) if with_state else None
    return inp, do, dso, dzo


NORM_NAMES = ("dq", "dk", "dv", "-", "dstate_in", "dz_in")


def test_normalized_backward_refuses_large_states():
    """fp32 operand tiles: d_k * d_v above 4096 (other than 32 x 128) is refused."""
    inp, do, dso, dzo = _norm_case("bf16", 1, 1, 64, 128, 128, seed=48)
    with pytest.raises(la.LinAttnError):
        _norm_run(inp, do, dso, dzo)


@pytest.mark.parametrize("dt,dk,dv", [(dt, dk, dv) for dt in ("bf16", "f32")
                                      for dk, dv in [(32, 32), (64, 64), (32, 64), (64, 32), (128, 32), (32, 128)]])
def test_normalized_backward_matches_oracle(dt, dk, dv):
    print(f"[bwd] normalized {dt} dk{dk} dv{dv}", flush=True)
    inp, do, dso, dzo = _norm_case(dt, 2, 3, 3 * 64 + 17, dk, dv, seed=45)
    g = _norm_run(inp, do, dso, dzo)
    ref = _norm_ref(inp, do, dso, dzo)
    for name, got, want in zip(NORM_NAMES, g, ref):
        if want is None or got is None:
            continue
        assert_close(got, want, TOL[dt], name)


@pytest.mark.parametrize("L", [0, 1, 17, 63, 64, 65, 130])
def test_normalized_backward_edge_lengths(L):
    inp, do, dso, dzo = _norm_case("f32", 1, 2, L, 64, 64, seed=46)
    g = _norm_run(inp, do, dso, dzo)
    ref = _norm_ref(inp, do, dso, dzo)
    for name, got, want in zip(NORM_NAMES, g, ref):
        if want is None or got is None or got.size == 0:
            continue
        assert_close(got, want, TOL["f32"], name)


def test_normalized_backward_without_states():
    inp, do, _, _ = _norm_case("bf16", 2, 2, 150, 64, 64, seed=47, with_state=False)
    g = _norm_run(inp, do, None, None, want=False)
    ref = _norm_ref(inp, do, None, None)
    for name, got, want in zip(NORM_NAMES[:3], g[:3], ref[:3]):
        assert_close(got, want, TOL["bf16"], name)


def test_normalized_backward_full_size_all_heads():
    """The normalized workload (B8 H16 L2048 d64), every head against the oracle."""
    name = "normalized_bf16_b8h16_l2048_d64"
    c = W.CONFIGS[name]
    B, H, L, dk, dv = c["B"], c["H"], c["L"], c["dk"], c["dv"]
    print("[bwd] normalized full size", flush=True)
    inp = W.config_chunk_inputs(name, seed=0)
    do = W.make_backward_dout("bf16", B, H, L, dv, seed=0)
    g = la.la_chunk_bwd("normalized", dev(inp.q), dev(inp.k), dev(inp.v), dev(do))
    torch.cuda.synchronize()
    ref = oracle.backward("normalized", inp.f64("q"), inp.f64("k"), inp.f64("v"), W.to_f64(do), threads=16)
    for i, nm in enumerate(("dq", "dk", "dv")):
        e = assert_close(host64(g[i]), ref[i], TOL["bf16"], nm)
        print(f"[bwd] normalized full size {nm} max|err|/RMS = {e:.2e}", flush=True)
