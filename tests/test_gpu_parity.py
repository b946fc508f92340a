"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, element by
element on the same seeded inputs. Sizes span several chunks and a ragged tail;
edge cases cover empty and tiny sequences, state carry, determinism and head
isolation. The full-size workloads are in test_gpu_configs.py."""
import numpy as np
import pytest
import torch

import chunkwise_linear_rnn_causal_amd as la
import oracle
import workloads as W
from gpu_util import TOL, assert_close, dev, gpu_chunk, host64, oracle_chunk

pytestmark = pytest.mark.gpu

SHAPES = [(32, 32), (64, 64), (128, 128), (64, 128), (128, 96)]


def _cases():
    out = []
    for var in ("plain", "normalized", "decay", "gated_delta"):
        for dt in ("bf16", "f32"):
            for C in (64, 128):
                for dk, dv in SHAPES:
                    out.append((var, dt, C, dk, dv))
    return out


@pytest.mark.parametrize("var,dt,C,dk,dv", _cases(), ids=lambda x: str(x))
def test_chunk_matches_oracle(var, dt, C, dk, dv):
    """B=2, H=3, L = 3C + 17 (three full chunks and a ragged one), with a random
    initial state (and normalizer), against the oracle."""
    L = 3 * C + 17
    inp = W.make_chunk_inputs(var, dt, 2, 3, L, dk, dv, seed=11, with_state=True,
                              with_z=(var == "normalized"))
    o, s, z = gpu_chunk(inp, C)
    ro, rs, rz = oracle_chunk(inp)
    assert_close(o, ro, TOL[dt], "o")
    assert_close(s, rs, TOL[dt], "state")
    if var == "normalized":
        assert_close(z, rz, 1e-5, "z")


@pytest.mark.parametrize("var", ["plain", "normalized", "decay", "gated_delta"])
@pytest.mark.parametrize("L", [0, 1, 5, 63, 64, 65])
def test_edge_lengths(var, L):
    """Empty, single-token, shorter-than-a-chunk and chunk-boundary sequences."""
    inp = W.make_chunk_inputs(var, "bf16", 1, 2, L, 64, 64, seed=3, with_state=True,
                              with_z=(var == "normalized"))
    o, s, z = gpu_chunk(inp, 64)
    ro, rs, rz = oracle_chunk(inp)
    if L > 0:
        assert_close(o, ro, TOL["bf16"], "o")
    assert_close(s, rs, TOL["bf16"] if L else 1e-7, "state")
    if var == "normalized":
        assert_close(z, rz, 1e-5, "z")


@pytest.mark.parametrize("var", ["plain", "decay", "gated_delta"])
def test_no_initial_state(var):
    inp = W.make_chunk_inputs(var, "bf16", 1, 2, 200, 128, 128, seed=4)
    o, s, _ = gpu_chunk(inp, 64, state_in=False)
    ro, rs, _ = oracle_chunk(inp, state_in=False)
    assert_close(o, ro, TOL["bf16"], "o")
    assert_close(s, rs, TOL["bf16"], "state")


@pytest.mark.parametrize("var", ["plain", "normalized", "decay", "gated_delta"])
def test_resume_in_place_equals_one_pass(var):
    """Carry (S, z) across a split with state_out == state_in (in-place), and
    compare with a single pass and with the oracle."""
    L1, L2 = 130, 77
    inp = W.make_chunk_inputs(var, "f32", 1, 2, L1 + L2, 64, 64, seed=5)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    lg, be = dev(inp.log_gate), dev(inp.beta)
    norm = var == "normalized"
    o_full, s_full, z_full = la.la_chunk_fwd(var, q, k, v, lg, be, want_state=True, want_z=norm)
    sl = lambda x, a, b: None if x is None else x[:, :, a:b].contiguous()
    S = torch.zeros((1, 2, 64, 64), dtype=torch.float32, device="cuda")
    Z = torch.zeros((1, 2, 64), dtype=torch.float32, device="cuda") if norm else None
    Z2 = torch.zeros_like(Z) if norm else None
    o1, _, _ = la.la_chunk_fwd(var, sl(q, 0, L1), sl(k, 0, L1), sl(v, 0, L1), sl(lg, 0, L1),
                               sl(be, 0, L1), S, Z, state_out=S, z_out=Z2)
    o2, _, _ = la.la_chunk_fwd(var, sl(q, L1, None), sl(k, L1, None), sl(v, L1, None),
                               sl(lg, L1, None), sl(be, L1, None), S, Z2, state_out=S, z_out=Z)
    torch.cuda.synchronize()
    o_split = np.concatenate([host64(o1), host64(o2)], axis=2)
    assert_close(o_split, host64(o_full), 1e-5, "split vs one pass")
    assert_close(host64(S), host64(s_full), 1e-5, "state")
    ro, rs, rz = oracle_chunk(inp, state_in=False, z_in=False)
    assert_close(o_split, ro, TOL["f32"], "o vs oracle")
    assert_close(host64(S), rs, TOL["f32"], "state vs oracle")
    if norm:
        assert_close(host64(Z), rz, 1e-6, "z vs oracle")


@pytest.mark.parametrize("var", ["decay", "gated_delta", "normalized"])
def test_deterministic(var):
    inp = W.make_chunk_inputs(var, "bf16", 2, 4, 300, 128, 128, seed=6)
    a = gpu_chunk(inp, 64)
    b = gpu_chunk(inp, 64)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("var", ["plain", "decay", "gated_delta"])
def test_chunk_sizes_agree(var):
    """C = 64 and C = 128 compute the same result (tensorplay section 3.3: the
    chunk size changes the schedule, not the value)."""
    inp = W.make_chunk_inputs(var, "bf16", 1, 2, 500, 64, 64, seed=7)
    o64, s64, _ = gpu_chunk(inp, 64, state_in=False)
    o128, s128, _ = gpu_chunk(inp, 128, state_in=False)
    ro, rs, _ = oracle_chunk(inp, state_in=False)
    assert_close(o64, ro, TOL["bf16"], "C=64")
    assert_close(o128, ro, TOL["bf16"], "C=128")


@pytest.mark.parametrize("var,dt,dk", [("gated_delta", "bf16", 128), ("gated_delta", "f32", 64),
                                       ("vector_decay", "bf16", 128), ("decay", "f32", 128)])
def test_c128_sub_chunk_schedule(var, dt, dk):
    """Where a 128-token chunk runs as two 64-token sub-chunks (the delta rule:
    block forward substitution of the 128 x 128 UT system; the per-channel gate;
    fp32 tiles at d_k = 128), C = 128 gives the bits of C = 64, and both match
    the oracle."""
    inp = W.make_chunk_inputs(var, dt, 2, 2, 3 * 128 + 37, dk, 64, seed=14, with_state=True)
    o64, s64, _ = gpu_chunk(inp, 64)
    o128, s128, _ = gpu_chunk(inp, 128)
    assert np.array_equal(o64, o128) and np.array_equal(s64, s128)
    ro, rs, _ = oracle_chunk(inp)
    assert_close(o128, ro, TOL[dt], "o")
    assert_close(s128, rs, TOL[dt], "state")


@pytest.mark.parametrize("var", ["plain", "normalized", "decay", "gated_delta"])
def test_nan_head_does_not_leak(var):
    """Heads are independent: a NaN in one head's query stays in that head."""
    inp = W.make_chunk_inputs(var, "bf16", 2, 2, 150, 64, 64, seed=8)
    clean = gpu_chunk(inp, 64, state_in=False)[0]
    inp.q = inp.q.copy()
    inp.q[1, 0, 70, 5] = 0x7FC0  # bf16 quiet NaN
    dirty = gpu_chunk(inp, 64, state_in=False)[0]
    others = [(0, 0), (0, 1), (1, 1)]
    for b, h in others:
        assert np.array_equal(clean[b, h], dirty[b, h]), (b, h)
    assert np.isnan(dirty[1, 0, 70]).any()


def test_associative_recall_on_gpu():
    """One-hot keys, beta = 1, alpha = 1 (tensorplay section 6 example, extended
    with a rebinding): the delta rule returns the last value bound to each key,
    plain linear attention the sum of the values bound to it."""
    d = 32
    writes = [(0, 4.0), (1, 3.0), (2, 6.0), (0, 9.0)]
    queries = [0, 2, 1]
    T = len(writes) + len(queries)
    q = np.zeros((1, 1, T, d), np.float32); k = np.zeros_like(q); v = np.zeros((1, 1, T, d), np.float32)
    for t, (key, val) in enumerate(writes):
        k[0, 0, t, key] = 1.0
        v[0, 0, t, 0] = val
    for i, key in enumerate(queries):
        q[0, 0, len(writes) + i, key] = 1.0
    beta = np.ones((1, 1, T), np.float32)
    o, _, _ = la.la_chunk_fwd("gated_delta", dev(q), dev(k), dev(v), None, dev(beta))
    o2, _, _ = la.la_chunk_fwd("plain", dev(q), dev(k), dev(v))
    torch.cuda.synchronize()
    got = host64(o)[0, 0, len(writes):, 0]
    got2 = host64(o2)[0, 0, len(writes):, 0]
    assert np.allclose(got, [9.0, 6.0, 3.0], atol=1e-5), got
    assert np.allclose(got2, [13.0, 6.0, 3.0], atol=1e-5), got2


# ---------------------------------------------------------------------------
# decode step
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(dk, dv) for dk in (32, 64, 128) for dv in (32, 64, 128)])
@pytest.mark.parametrize("var", ["plain", "decay", "gated_delta", "deltanet"])
def test_decode_matches_oracle(var, dt, dk, dv):
    """One-token steps, three in a row on the same state; "deltanet" is the delta
    rule without a log-gate (alpha = 1). With bf16 inputs the middle step writes
    o in bf16."""
    N, H = 5, 3
    S0 = W.make_decode_state(N, H, dk, dv, seed=2)
    S = dev(S0)
    Sref = S0.astype(np.float64)
    delta = var in ("gated_delta", "deltanet")
    kind = "gated_delta" if delta else var
    for step in range(3):
        st = W.make_decode_step(N, H, dk, dv, step=step, seed=2, dtype=dt, with_beta=delta)
        lg = st.log_gate if var in ("decay", "gated_delta") else None
        o_bf16 = dt == "bf16" and step == 1
        o = la.la_decode_step(kind, dev(st.q), dev(st.k), dev(st.v), dev(lg), S, beta=dev(st.beta),
                              out_dtype=torch.bfloat16 if o_bf16 else None)
        assert o.dtype == (torch.bfloat16 if o_bf16 else torch.float32)
        torch.cuda.synchronize()
        ro, Sref = oracle.decode_step(kind, W.to_f64(st.q), W.to_f64(st.k), W.to_f64(st.v),
                                      None if lg is None else lg.astype(np.float64), Sref,
                                      beta=None if st.beta is None else st.beta.astype(np.float64))
        assert_close(host64(o), ro, TOL[dt], f"o step {step}")
        assert_close(host64(S), Sref, 1e-4, f"state step {step}")


def test_prefill_then_decode():
    """Prefill L tokens with the chunk kernel, then decode token L+1 from its
    final state: equals the oracle over L+1 tokens (tensorplay section 2.2)."""
    B, H, L, d = 2, 3, 190, 128
    inp = W.make_chunk_inputs("decay", "bf16", B, H, L + 1, d, d, seed=9)
    q, k, v, lg = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.log_gate)
    pre = lambda x: x[:, :, :L].contiguous()
    _, S, _ = la.la_chunk_fwd("decay", pre(q), pre(k), pre(v), pre(lg), want_state=True)
    last = lambda x: x[:, :, L].contiguous()
    o = la.la_decode_step("decay", last(q), last(k), last(v), last(lg), S)
    torch.cuda.synchronize()
    ro, rs, _ = oracle_chunk(inp, state_in=False)
    assert_close(host64(o), ro[:, :, L], TOL["bf16"], "o")
    assert_close(host64(S), rs, TOL["bf16"], "state")


def test_prefill_then_decode_gated_delta():
    """Delta rule: prefill L tokens with the chunk kernel, then decode token L+1
    from its final state; equals the oracle over L+1 tokens."""
    B, H, L, d = 2, 3, 150, 128
    inp = W.make_chunk_inputs("gated_delta", "bf16", B, H, L + 1, d, d, seed=12)
    q, k, v, lg, be = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.log_gate), dev(inp.beta)
    pre = lambda x: x[:, :, :L].contiguous()
    _, S, _ = la.la_chunk_fwd("gated_delta", pre(q), pre(k), pre(v), pre(lg), pre(be), want_state=True)
    last = lambda x: x[:, :, L].contiguous()
    o = la.la_decode_step("gated_delta", last(q), last(k), last(v), last(lg), S, beta=last(be))
    torch.cuda.synchronize()
    ro, rs, _ = oracle_chunk(inp, state_in=False)
    assert_close(host64(o), ro[:, :, L], TOL["bf16"], "o")
    assert_close(host64(S), rs, TOL["bf16"], "state")


@pytest.mark.parametrize("var", ["plain", "normalized", "decay", "gated_delta"])
@pytest.mark.parametrize("C", [64, 128])
def test_bf16_output(var, C):
    """o_dt = bf16: the same kernels, with the output rounded to nearest even.
    Bound: the fp32-output tolerance plus bf16's rounding of each value
    (|err| <= 2e-2 RMS + 2^-8 |o|)."""
    inp = W.make_chunk_inputs(var, "bf16", 2, 2, 2 * C + 9, 128, 64, seed=12)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    o, _, _ = la.la_chunk_fwd(var, q, k, v, dev(inp.log_gate), dev(inp.beta), C=C,
                              out_dtype=torch.bfloat16)
    o32, _, _ = la.la_chunk_fwd(var, q, k, v, dev(inp.log_gate), dev(inp.beta), C=C)
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    ro, _, _ = oracle_chunk(inp, state_in=False)
    got = host64(o)
    rms = float(np.sqrt(np.mean(ro ** 2)))
    assert np.all(np.abs(got - ro) <= TOL["bf16"] * rms + 2.0 ** -8 * np.abs(ro))
    # bf16 output is the RNE rounding of the fp32 output of the same kernel
    assert torch.equal(o, o32.to(torch.bfloat16))


@pytest.mark.parametrize("var,B,H,dk,dv", [
    ("plain", 4, 64, 64, 64),          # 256 heads x 64 columns: 64-column, 8-wave workgroups
    ("normalized", 2, 128, 32, 128),
    ("decay", 2, 64, 128, 128),
    ("gated_delta", 2, 32, 64, 128),   # 64 heads x 4 slices: 32-column, 8-wave delta rule
])
def test_wide_grid_geometry(var, B, H, dk, dv):
    """Workload shapes with enough heads to select the wider workgroup
    geometries; a ragged tail included."""
    inp = W.make_chunk_inputs(var, "bf16", B, H, 150, dk, dv, seed=13, with_state=True,
                              with_z=(var == "normalized"))
    o, s, z = gpu_chunk(inp, 64)
    ro, rs, rz = oracle_chunk(inp)
    assert_close(o, ro, TOL["bf16"], "o")
    assert_close(s, rs, TOL["bf16"], "state")
    if var == "normalized":
        assert_close(z, rz, 1e-5, "z")

# Lengths that run the steady-state loop of the split-role kernels (prefetch two
# or three chunks ahead, unrolled by the prefetch depth) and leave it at every
# remainder, with and without a ragged last chunk.
SCHEDULE_LENGTHS = [4 * 64 + 23, 5 * 64, 5 * 64 + 1, 6 * 64 + 40, 7 * 64 + 63, 8 * 64, 9 * 64 + 7]


@pytest.mark.parametrize("L", SCHEDULE_LENGTHS)
@pytest.mark.parametrize("var,dk,dv", [
    ("plain", 64, 64),          # 32-column split roles, three prefetch sets
    ("normalized", 64, 64),
    ("decay", 64, 64),
    ("gated_delta", 64, 64),    # 16-column split roles, three prefetch sets
    ("decay", 128, 128),        # queries loaded straight into registers
    ("gated_delta", 128, 128),  # one prefetch set
])
def test_split_role_schedules(var, dk, dv, L):
    """Split-role chunk kernels through their steady-state loop and every exit
    remainder, against the oracle (B=1, H=2, random initial state)."""
    inp = W.make_chunk_inputs(var, "bf16", 1, 2, L, dk, dv, seed=17, with_state=True,
                              with_z=(var == "normalized"))
    o, s, z = gpu_chunk(inp, 64)
    ro, rs, rz = oracle_chunk(inp)
    assert_close(o, ro, TOL["bf16"], "o")
    assert_close(s, rs, TOL["bf16"], "state")
    if var == "normalized":
        assert_close(z, rz, 1e-5, "z")


def test_split_role_schedule_two_sets():
    """Decay, d = 128, 128 heads: 64-column split roles with two prefetch sets
    and direct queries, through the steady-state loop and a ragged tail."""
    inp = W.make_chunk_inputs("decay", "bf16", 2, 64, 5 * 64 + 9, 128, 128, seed=19, with_state=True)
    o, s, _ = gpu_chunk(inp, 64)
    ro, rs, _ = oracle_chunk(inp)
    assert_close(o, ro, TOL["bf16"], "o")
    assert_close(s, rs, TOL["bf16"], "state")
