"""GPU parity at the full sizes of the workloads, in the launch configuration
the benchmark times (la_chunk_fwd with C = 64 and a final-state output; 100
back-to-back la_decode_step calls, decay and delta rule; one la_short_conv). The oracle checks sampled
batch-heads, which the seeded generator regenerates on their own (every (tensor,
b, h) slice has its own random stream), the whole first decode step, and every
element of the short convolution."""
import numpy as np
import pytest
import torch

import chunkwise_linear_rnn_causal_amd as la
import oracle
import workloads as W
from gpu_util import TOL, assert_close, dev, host64

pytestmark = pytest.mark.gpu


def _sample_heads(B, H):
    heads = {(0, 0), (B - 1, H - 1), (B // 2, H // 3)}
    return sorted(heads)


@pytest.mark.parametrize("name", [n for n, c in W.CONFIGS.items() if c["kind"] == "chunk"])
def test_full_size_chunk_config(name):
    c = W.CONFIGS[name]
    print(f"[config] {name}", flush=True)
    inp = W.config_chunk_inputs(name, seed=0)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    lg, be = dev(inp.log_gate), dev(inp.beta)
    o, S, _ = la.la_chunk_fwd(c["variant"], q, k, v, lg, be, C=c["C"], want_state=True)
    torch.cuda.synchronize()
    heads = _sample_heads(c["B"], c["H"])
    ref_in = W.config_chunk_inputs(name, seed=0, heads=heads)
    ro, rs, _ = oracle.forward(c["variant"], ref_in.f64("q"), ref_in.f64("k"), ref_in.f64("v"),
                               log_gate=ref_in.f64("log_gate"), beta=ref_in.f64("beta"))
    got_o = np.stack([host64(o[b, h]) for b, h in heads])[None]
    got_s = np.stack([host64(S[b, h]) for b, h in heads])[None]
    e_o = assert_close(got_o, ro, TOL[c["dtype"]], f"{name} o")
    e_s = assert_close(got_s, rs, TOL[c["dtype"]], f"{name} state")
    print(f"[config] {name} heads={heads} err_o={e_o:.2e} err_state={e_s:.2e}", flush=True)
    # every output finite
    assert bool(torch.isfinite(o.float()).all())


@pytest.mark.parametrize("variant", ["decay", "gated_delta"])
def test_full_size_decode_config(variant):
    """100 decode steps at the decode workload's shape, bf16 output; the delta rule
    runs at the same shape with beta = sigmoid(N(0,1)) per sequence-head, as the
    benchmark times it."""
    c = W.CONFIGS["decode_decay_bf16_n512h32_d128"]
    N, H, dk, dv, steps = c["N"], c["H"], c["dk"], c["dv"], c["steps"]
    delta = variant == "gated_delta"
    print(f"[config] decode full size, {variant}", flush=True)
    S0 = W.make_decode_state(N, H, dk, dv, seed=0)
    S = dev(S0)
    heads = [(0, 0), (N - 1, H - 1), (N // 2, H // 3), (17, 5)]
    hs = {name: [] for name in ("q", "k", "v", "lg", "beta")}
    o_last = None
    for step in range(steps):
        st = W.make_decode_step(N, H, dk, dv, step=step, seed=0, with_beta=delta)
        o = la.la_decode_step(variant, dev(st.q), dev(st.k), dev(st.v), dev(st.log_gate), S,
                              beta=dev(st.beta) if delta else None, out_dtype=torch.bfloat16)
        for name, x in (("q", st.q), ("k", st.k), ("v", st.v), ("lg", st.log_gate), ("beta", st.beta)):
            if x is not None:
                hs[name].append(np.stack([x[n, h] for n, h in heads]))
        if step == 0:
            torch.cuda.synchronize()
            ro, rS = oracle.decode_step(variant, W.to_f64(st.q), W.to_f64(st.k), W.to_f64(st.v),
                                        st.log_gate.astype(np.float64), S0,
                                        beta=st.beta.astype(np.float64) if delta else None)
            assert_close(host64(o), ro, TOL["bf16"], "step 1 o (all heads)")
            assert_close(host64(S), rS, 1e-4, "step 1 state (all heads)")
            del rS
        o_last = o
    torch.cuda.synchronize()
    Sref = np.stack([S0[n, h] for n, h in heads]).astype(np.float64)
    for step in range(steps):
        ro, Sref = oracle.decode_step(variant, W.to_f64(hs["q"][step]), W.to_f64(hs["k"][step]),
                                      W.to_f64(hs["v"][step]), hs["lg"][step].astype(np.float64), Sref,
                                      beta=hs["beta"][step].astype(np.float64) if delta else None)
    got_o = np.stack([host64(o_last[n, h]) for n, h in heads])
    got_S = np.stack([host64(S[n, h]) for n, h in heads])
    e_o = assert_close(got_o, ro, TOL["bf16"], "step 100 o")
    e_s = assert_close(got_S, Sref, 1e-4, "step 100 state")
    print(f"[config] decode {variant} step100 err_o={e_o:.2e} err_state={e_s:.2e}", flush=True)


def test_full_size_short_conv_config():
    """The short convolution at the benchmark's size (q, k, v of the delta-rule
    workload, K = 4), one launch as timed; every element against the oracle
    within the per-element fp32-sum + bf16-rounding bound."""
    name = "short_conv_qkv_bf16_b2h16_l8192_d128_k4"
    print(f"[config] {name}", flush=True)
    ci = W.config_conv_inputs(name, seed=0)
    xs = [dev(x) for x in ci.x]
    ws = [dev(t) for t in ci.taps]
    outs = la.la_short_conv(*xs, *ws, want_state=True)
    torch.cuda.synchronize()
    for i, tname in enumerate("qkv"):
        x = ci.f64("x", i)
        ry, rs = oracle.short_conv(x, ci.taps[i], None)
        got = host64(outs[i])
        bound_src, _ = oracle.short_conv(np.abs(x), np.abs(ci.taps[i]), None)
        lim = 1e-6 * bound_src + 2.0 ** -8 * np.abs(ry)
        assert bool(np.all(np.abs(got - ry) <= lim)), f"{tname}: out of bound"
        assert np.array_equal(host64(outs[3 + i]), rs), f"{tname} window"
        print(f"[config] {name} {tname} max|err|={float(np.abs(got - ry).max()):.2e}", flush=True)
