"""GPU parity of the per-key-channel decay (LA_VECTOR_DECAY, the GLA vector gate)
against the fp64 oracle: several chunks and a ragged tail at every head size,
GLA-style and strong gates up to the supported bound, edge lengths, state carry
in place, bf16 output, the scalar-gate special case, and the decode step."""
import numpy as np
import pytest
import torch

import chunkwise_linear_rnn_causal_amd as la
import oracle
import workloads as W
from gpu_util import TOL, assert_close, dev, gpu_chunk, host64, oracle_chunk

pytestmark = pytest.mark.gpu

VD = "vector_decay"


def _cases():
    out = []
    for dt in ("bf16", "f32"):
        for dk, dv in [(32, 32), (64, 64), (128, 128), (64, 128), (128, 96), (32, 64)]:
            if dt == "f32" and dk == 128:
                continue
            out.append((dt, dk, dv))
    return out


@pytest.mark.parametrize("dt,dk,dv", _cases(), ids=lambda x: str(x))
@pytest.mark.parametrize("recipe", ["gla", "gla_strong"])
def test_vector_decay_matches_oracle(dt, dk, dv, recipe):
    """B=2, H=3, L = 3*64 + 17 with an initial state; GLA gates (log sigmoid(x)/16)
    and strong gates spread over [-10, 0]."""
    inp = W.make_chunk_inputs(VD, dt, 2, 3, 3 * 64 + 17, dk, dv, seed=31, recipe=recipe,
                              with_state=True)
    o, s, _ = gpu_chunk(inp, 64)
    ro, rs, _ = oracle_chunk(inp)
    assert_close(o, ro, TOL[dt], "o")
    assert_close(s, rs, TOL[dt], "state")


@pytest.mark.parametrize("L", [0, 1, 5, 15, 16, 17, 63, 64, 65, 130])
def test_vector_decay_edge_lengths(L):
    inp = W.make_chunk_inputs(VD, "bf16", 1, 2, L, 64, 64, seed=32, with_state=True)
    o, s, _ = gpu_chunk(inp, 64)
    ro, rs, _ = oracle_chunk(inp)
    if L > 0:
        assert_close(o, ro, TOL["bf16"], "o")
    assert_close(s, rs, TOL["bf16"] if L else 1e-7, "state")


def test_vector_decay_uniform_gate_is_scalar_decay():
    """The same gate on every key channel is the scalar decay: the two kernels
    agree (to their rounding) and both match the oracle."""
    inp = W.make_chunk_inputs("decay", "f32", 2, 2, 200, 64, 64, seed=33, with_state=True)
    lg_vec = np.repeat(inp.log_gate[..., None], 64, axis=-1)
    q, k, v, s0 = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.state_in)
    ov, sv, _ = la.la_chunk_fwd(VD, q, k, v, dev(lg_vec), state_in=s0, want_state=True)
    od, sd, _ = la.la_chunk_fwd("decay", q, k, v, dev(inp.log_gate), state_in=s0, want_state=True)
    torch.cuda.synchronize()
    ro, rs, _ = oracle_chunk(inp)
    assert_close(host64(ov), ro, TOL["f32"], "vector o")
    assert_close(host64(od), ro, TOL["f32"], "scalar o")
    assert_close(host64(sv), rs, TOL["f32"], "vector state")


def test_vector_decay_resume_in_place():
    """Carry the state across a split with state_out == state_in; equals one pass."""
    L1, L2 = 100, 77
    inp = W.make_chunk_inputs(VD, "f32", 1, 2, L1 + L2, 64, 64, seed=34)
    q, k, v, lg = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.log_gate)
    S = torch.zeros((1, 2, 64, 64), dtype=torch.float32, device="cuda")
    part = lambda x, a, b: x[:, :, a:b].contiguous()
    o1, _, _ = la.la_chunk_fwd(VD, part(q, 0, L1), part(k, 0, L1), part(v, 0, L1), part(lg, 0, L1),
                               state_in=S, state_out=S)
    o2, _, _ = la.la_chunk_fwd(VD, part(q, L1, L1 + L2), part(k, L1, L1 + L2), part(v, L1, L1 + L2),
                               part(lg, L1, L1 + L2), state_in=S, state_out=S)
    torch.cuda.synchronize()
    ro, rs, _ = oracle_chunk(inp, state_in=False)
    assert_close(np.concatenate([host64(o1), host64(o2)], axis=2), ro, TOL["f32"], "o")
    assert_close(host64(S), rs, TOL["f32"], "state")


def test_vector_decay_bf16_output_and_determinism():
    inp = W.make_chunk_inputs(VD, "bf16", 2, 2, 2 * 64 + 9, 128, 64, seed=35)
    q, k, v, lg = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.log_gate)
    o, _, _ = la.la_chunk_fwd(VD, q, k, v, lg, out_dtype=torch.bfloat16)
    o32, _, _ = la.la_chunk_fwd(VD, q, k, v, lg)
    o32b, _, _ = la.la_chunk_fwd(VD, q, k, v, lg)
    torch.cuda.synchronize()
    assert torch.equal(o32, o32b)
    assert torch.equal(o, o32.to(torch.bfloat16))
    ro, _, _ = oracle_chunk(inp, state_in=False)
    rms = float(np.sqrt(np.mean(ro ** 2)))
    assert np.all(np.abs(host64(o) - ro) <= TOL["bf16"] * rms + 2.0 ** -8 * np.abs(ro))


def test_vector_decay_wide_grid():
    """Many heads (the benchmark's slicing: 32-column workgroups), ragged tail."""
    inp = W.make_chunk_inputs(VD, "bf16", 2, 64, 150, 128, 128, seed=36, with_state=True)
    o, s, _ = gpu_chunk(inp, 64)
    ro, rs, _ = oracle_chunk(inp)
    assert_close(o, ro, TOL["bf16"], "o")
    assert_close(s, rs, TOL["bf16"], "state")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(dk, dv) for dk in (32, 64, 128) for dv in (32, 64, 128)])
def test_vector_decay_decode(dt, dk, dv):
    """Three one-token steps in place with per-channel gates, against the oracle;
    with bf16 inputs the middle step writes o in bf16."""
    N, H = 5, 3
    S0 = W.make_decode_state(N, H, dk, dv, seed=37)
    S = dev(S0)
    Sref = S0.astype(np.float64)
    rng = np.random.default_rng(37)
    for step in range(3):
        st = W.make_decode_step(N, H, dk, dv, step=step, seed=37, dtype=dt)
        lg = (np.log(1.0 / (1.0 + np.exp(-rng.normal(0.0, 1.0, size=(N, H, dk))))) / 16.0).astype(np.float32)
        o_bf16 = dt == "bf16" and step == 1
        o = la.la_decode_step(VD, dev(st.q), dev(st.k), dev(st.v), dev(lg), S,
                              out_dtype=torch.bfloat16 if o_bf16 else None)
        assert o.dtype == (torch.bfloat16 if o_bf16 else torch.float32)
        torch.cuda.synchronize()
        ro, Sref = oracle.decode_step(VD, W.to_f64(st.q), W.to_f64(st.k), W.to_f64(st.v),
                                      lg.astype(np.float64), Sref)
        assert_close(host64(o), ro, TOL[dt], f"o step {step}")
        assert_close(host64(S), Sref, 1e-4, f"state step {step}")


def test_vector_decay_prefill_then_decode():
    B, H, L, d = 2, 3, 190, 128
    inp = W.make_chunk_inputs(VD, "bf16", B, H, L + 1, d, d, seed=38)
    q, k, v, lg = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.log_gate)
    pre = lambda x: x[:, :, :L].contiguous()
    _, S, _ = la.la_chunk_fwd(VD, pre(q), pre(k), pre(v), pre(lg), want_state=True)
    last = lambda x: x[:, :, L].contiguous()
    o = la.la_decode_step(VD, last(q), last(k), last(v), last(lg), S)
    torch.cuda.synchronize()
    ro, rs, _ = oracle_chunk(inp, state_in=False)
    assert_close(host64(o), ro[:, :, L], TOL["bf16"], "o")
    assert_close(host64(S), rs, TOL["bf16"], "state")


@pytest.mark.parametrize("C", [64, 128])
def test_vector_decay_gates_below_the_rebasing_range(C):
    """Per-channel log-gates far below -10 (every eighth gate at -30, some whole
    tokens at -60): the kernel takes them as -10, which damps the history to
    4.5e-5 per token instead of less; the result stays within the bf16
    tolerance of the oracle, which uses the gates as given."""
    inp = W.make_chunk_inputs(VD, "bf16", 2, 2, 3 * 64 + 29, 128, 64, seed=41, with_state=True,
                              recipe="gla_strong")
    lg = inp.log_gate.copy()
    lg[..., ::8] = -30.0
    lg[:, :, 70:75, :] = -60.0
    inp.log_gate = lg
    o, s, _ = gpu_chunk(inp, C)
    ro, rs, _ = oracle_chunk(inp)
    assert_close(o, ro, TOL["bf16"], "o")
    assert_close(s, rs, TOL["bf16"], "state")
