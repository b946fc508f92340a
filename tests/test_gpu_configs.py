"""GPU parity at the full sizes of the workloads, in the launch configuration
the benchmark times (la_chunk_fwd with C = 64 and a final-state output, in the
workload's output dtype; 100 back-to-back la_decode_step calls, decay and delta
rule; one la_short_conv). Every element of every output is compared with the
fp64 oracle: the whole tensors, not sampled heads."""
import numpy as np
import pytest
import torch

import chunkwise_linear_rnn_causal_amd as la
import oracle
import workloads as W
from gpu_util import TOL, assert_close, dev, host64, rel_err

pytestmark = pytest.mark.gpu

CHUNK = [n for n, c in W.CONFIGS.items() if c["kind"] == "chunk"]


def _o_dtypes():
    """(workload, output dtype) pairs: fp32 output for every workload, and bf16
    output where the workload's benchmarked output is bf16."""
    out = [(n, "f32") for n in CHUNK]
    out += [(n, "bf16") for n in CHUNK if W.CONFIGS[n].get("o_dtype") == "bf16"]
    return out


@pytest.mark.parametrize("name,o_dt", _o_dtypes(), ids=lambda x: str(x))
def test_full_size_chunk_config(name, o_dt):
    c = W.CONFIGS[name]
    print(f"[config] {name} o={o_dt}", flush=True)
    inp = W.config_chunk_inputs(name, seed=0)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    lg, be = dev(inp.log_gate), dev(inp.beta)
    o, S, _ = la.la_chunk_fwd(c["variant"], q, k, v, lg, be, C=c["C"], want_state=True,
                              out_dtype=torch.bfloat16 if o_dt == "bf16" else None)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all())
    del q, k, v, lg, be
    ro, rs, _ = oracle.forward(c["variant"], inp.f64("q"), inp.f64("k"), inp.f64("v"),
                               log_gate=inp.f64("log_gate"), beta=inp.f64("beta"))
    got_o, got_s = host64(o), host64(S)
    del o, S
    e_o = assert_close(got_o, ro, TOL[c["dtype"]], f"{name} o")
    e_s = assert_close(got_s, rs, TOL[c["dtype"]], f"{name} state")
    print(f"[config] {name} o={o_dt} all heads: max|err|/RMS o={e_o:.3e} state={e_s:.3e}", flush=True)


@pytest.mark.parametrize("variant", ["decay", "gated_delta"])
def test_full_size_decode_config(variant):
    """100 decode steps at the decode workload's shape with bf16 output; the delta
    rule runs at the same shape with beta = sigmoid(N(0,1)) per sequence-head and
    fp32 output (bf16 rounding of its output alone reaches the bf16 tolerance), as
    the benchmark times both. Every head is compared after step 1 and step 100."""
    c = W.CONFIGS["decode_decay_bf16_n512h32_d128"]
    N, H, dk, dv, steps = c["N"], c["H"], c["dk"], c["dv"], c["steps"]
    delta = variant == "gated_delta"
    print(f"[config] decode full size, {variant}", flush=True)
    S0 = W.make_decode_state(N, H, dk, dv, seed=0)
    S = dev(S0)
    Sref = S0.astype(np.float64)
    del S0
    for step in range(steps):
        st = W.make_decode_step(N, H, dk, dv, step=step, seed=0, with_beta=delta)
        o = la.la_decode_step(variant, dev(st.q), dev(st.k), dev(st.v), dev(st.log_gate), S,
                              beta=dev(st.beta) if delta else None,
                              out_dtype=torch.float32 if delta else torch.bfloat16)
        ro, Sref = oracle.decode_step(variant, W.to_f64(st.q), W.to_f64(st.k), W.to_f64(st.v),
                                      st.log_gate.astype(np.float64), Sref,
                                      beta=st.beta.astype(np.float64) if delta else None, copy=False)
        if step in (0, steps - 1):
            torch.cuda.synchronize()
            e_o = assert_close(host64(o), ro, TOL["bf16"], f"step {step + 1} o (all heads)")
            e_s = assert_close(host64(S), Sref, 1e-4, f"step {step + 1} state (all heads)")
            print(f"[config] decode {variant} step {step + 1} all heads: max|err|/RMS o={e_o:.3e} "
                  f"state={e_s:.3e}", flush=True)


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
        print(f"[config] {name} {tname} max|err|={float(np.abs(got - ry).max()):.2e} "
              f"max|err|/RMS={rel_err(got, ry):.2e}", flush=True)
