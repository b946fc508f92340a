"""GPU parity of Kimi Delta Attention (la_chunk_fwd and la_decode_step, "kda",
bf16 inputs): the delta rule with one gate per key channel, against the fp64
oracle's per-token recurrence. Every head-size pair over several chunks and a
ragged tail with an initial state; the delta rule's gate distribution per
channel, GLA-style gates and strong gates spread over [-10, 0]; gates below the
-10 floor; edge lengths; C = 128 against C = 64; the scalar-gate special case
against the delta rule's own path; bf16 output; the decode step alone and after
a prefill. The full-size workload is in test_gpu_configs.py."""
import numpy as np
import pytest
import torch

import chunkwise_linear_rnn_causal_amd as la
import oracle
import workloads as W
from gpu_util import TOL, assert_close, dev, gpu_chunk, host64, oracle_chunk

pytestmark = pytest.mark.gpu

KDA = "kda"


@pytest.mark.parametrize("dk,dv", [(32, 32), (32, 64), (32, 128), (64, 32), (64, 64), (64, 128),
                                   (128, 32), (128, 64), (128, 128)])
@pytest.mark.parametrize("recipe", ["kda", "kda_gla", "kda_strong"])
def test_kda_matches_oracle(dk, dv, recipe):
    print(f"[kda] B2 H3 L209 dk{dk} dv{dv} {recipe}", flush=True)
    inp = W.make_chunk_inputs(KDA, "bf16", 2, 3, 3 * 64 + 17, dk, dv, seed=71, recipe=recipe, with_state=True)
    o, s, _ = gpu_chunk(inp, 64)
    ro, rs, _ = oracle_chunk(inp)
    assert_close(o, ro, TOL["bf16"], "o")
    assert_close(s, rs, TOL["bf16"], "state")


@pytest.mark.parametrize("L", [0, 1, 17, 63, 64, 65, 130])
def test_kda_edge_lengths(L):
    print(f"[kda] edge L{L}", flush=True)
    inp = W.make_chunk_inputs(KDA, "bf16", 1, 2, L, 64, 64, seed=72, with_state=True)
    o, s, _ = gpu_chunk(inp, 64)
    ro, rs, _ = oracle_chunk(inp)
    if L > 0:
        assert_close(o, ro, TOL["bf16"], "o")
    assert_close(s, rs, TOL["bf16"] if L else 1e-7, "state")


def test_kda_chunk_128_is_two_64_token_chunks():
    inp = W.make_chunk_inputs(KDA, "bf16", 2, 2, 300, 128, 64, seed=73, with_state=True)
    o64, s64, _ = gpu_chunk(inp, 64)
    o128, s128, _ = gpu_chunk(inp, 128)
    assert np.array_equal(o64, o128) and np.array_equal(s64, s128)


def test_kda_gates_below_the_floor():
    """Per-channel log-gates far below -10 are taken as -10 (a gate of e^-10
    already damps the channel's history to 4.5e-5 per token): within the bf16
    tolerance of the oracle, which uses them as given."""
    inp = W.make_chunk_inputs(KDA, "bf16", 2, 2, 3 * 64 + 29, 128, 64, seed=74, with_state=True,
                              recipe="kda_strong")
    lg = inp.log_gate.copy()
    lg[..., ::8] = -30.0
    lg[:, :, 70:75, :] = -60.0
    inp.log_gate = lg
    o, s, _ = gpu_chunk(inp, 64)
    ro, rs, _ = oracle_chunk(inp)
    assert_close(o, ro, TOL["bf16"], "o")
    assert_close(s, rs, TOL["bf16"], "state")


def test_kda_uniform_gate_is_the_delta_rule():
    """The same gate on every key channel is the scalar-gate delta rule: KDA's
    path and the delta rule's own path agree to their rounding."""
    inp = W.make_chunk_inputs("gated_delta", "bf16", 2, 3, 250, 128, 128, seed=75, with_state=True)
    lg_vec = np.repeat(inp.log_gate[..., None], 128, axis=-1)
    args = (dev(inp.q), dev(inp.k), dev(inp.v))
    ok, sk, _ = la.la_chunk_fwd(KDA, *args, dev(lg_vec), dev(inp.beta), dev(inp.state_in), want_state=True)
    og, sg, _ = la.la_chunk_fwd("gated_delta", *args, dev(inp.log_gate), dev(inp.beta), dev(inp.state_in),
                                want_state=True)
    torch.cuda.synchronize()
    ro, rs, _ = oracle_chunk(inp)
    assert_close(host64(ok), ro, TOL["bf16"], "kda o")
    assert_close(host64(og), ro, TOL["bf16"], "delta rule o")
    assert_close(host64(ok), host64(og), TOL["bf16"], "kda vs delta rule")
    assert_close(host64(sk), rs, TOL["bf16"], "kda state")


def test_kda_bf16_output():
    """bf16 output: the fp32 result rounded to nearest even."""
    inp = W.make_chunk_inputs(KDA, "bf16", 1, 3, 200, 128, 128, seed=76, with_state=True)
    args = (dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.log_gate), dev(inp.beta), dev(inp.state_in))
    o32, _, _ = la.la_chunk_fwd(KDA, *args)
    o16, _, _ = la.la_chunk_fwd(KDA, *args, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16))


@pytest.mark.parametrize("dt,o_dt", [("bf16", "f32"), ("bf16", "bf16"), ("f32", "f32")])
@pytest.mark.parametrize("dk,dv", [(32, 64), (64, 32), (128, 128)])
def test_kda_decode_matches_oracle(dt, o_dt, dk, dv):
    """One decode step on N x H sequence-heads (fp32 state in place)."""
    N, H = 5, 3
    r = np.random.default_rng(77)
    x = lambda *s: r.standard_normal(s).astype(np.float32)
    store = (lambda a: W.f32_to_bf16_bits(a)) if dt == "bf16" else (lambda a: a)
    q = store((x(N, H, dk) / np.sqrt(dk)).astype(np.float32))
    k = store((x(N, H, dk) / np.sqrt(dk)).astype(np.float32))
    v = store(x(N, H, dv))
    lg = np.log(1.0 / (1.0 + np.exp(-r.normal(3.0, 1.0, (N, H, dk))))).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-r.normal(0.0, 1.0, (N, H))))).astype(np.float32)
    S0 = (0.3 * x(N, H, dk, dv)).astype(np.float32)
    S = dev(S0)
    o = la.la_decode_step(KDA, dev(q), dev(k), dev(v), dev(lg), S, beta=dev(beta),
                             out_dtype=torch.bfloat16 if o_dt == "bf16" else None)
    torch.cuda.synchronize()
    f64 = (lambda a: W.to_f64(a)) if dt == "bf16" else (lambda a: a.astype(np.float64))
    ro, rs = oracle.decode_step(KDA, f64(q), f64(k), f64(v), lg.astype(np.float64), S0.astype(np.float64),
                                beta=beta.astype(np.float64))
    assert_close(host64(S), rs, 1e-4, "state")  # the step is fp32 end to end
    assert_close(host64(o), ro, TOL["bf16"] if o_dt == "bf16" else 1e-4, "o")


def test_kda_prefill_then_decode():
    """la_chunk_fwd over 150 tokens with state_out, then 3 decode steps on that
    state: equal to the oracle's recurrence over 153 tokens."""
    B, H, L, dk, dv, extra = 2, 2, 150, 64, 64, 3
    inp = W.make_chunk_inputs(KDA, "bf16", B, H, L + extra, dk, dv, seed=78, with_state=True)
    part = lambda a, s: None if a is None else np.ascontiguousarray(a[:, :, s])
    _, S, _ = la.la_chunk_fwd(KDA, dev(part(inp.q, slice(0, L))), dev(part(inp.k, slice(0, L))),
                              dev(part(inp.v, slice(0, L))), dev(part(inp.log_gate, slice(0, L))),
                              dev(part(inp.beta, slice(0, L))), dev(inp.state_in), want_state=True)
    outs = []
    for t in range(L, L + extra):
        o = la.la_decode_step(KDA, dev(part(inp.q, t)), dev(part(inp.k, t)), dev(part(inp.v, t)),
                                 dev(part(inp.log_gate, t)), S, beta=dev(part(inp.beta, t)))
        outs.append(host64(o))
    torch.cuda.synchronize()
    ro, rs, _ = oracle_chunk(inp)
    for i, t in enumerate(range(L, L + extra)):
        assert_close(outs[i], ro[:, :, t], TOL["bf16"], f"o at {t}")
    assert_close(host64(S), rs, TOL["bf16"], "state")
