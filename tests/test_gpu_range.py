"""GPU parity where the carried quantities leave fp16's range.

With bf16 inputs the tensor-core operands are fp16 (largest finite value 65504).
The state S and the normalizer z are unbounded running sums: z grows about
linearly with the sequence (proig-chaa notes "线性注意力", sections 13-14), S too
when the values have a mean, and a caller may hand in any initial state
(tensorplay "Talk Linear Attention", section 2.2: the state carries the whole
history). These tests drive S, z and the delta rule's pseudo-values U past 65504
and compare every output with the fp64 oracle at the bf16 tolerance."""
import numpy as np
import pytest

import workloads as W
from gpu_util import TOL, assert_close, gpu_chunk, oracle_chunk

pytestmark = pytest.mark.gpu

FP16_MAX = 65504.0


def _scaled_start(inp, s_scale, z_scale=None):
    inp.state_in = (inp.state_in.astype(np.float64) * s_scale).astype(np.float32)
    if z_scale is not None and inp.z_in is not None:
        inp.z_in = (inp.z_in.astype(np.float64) * z_scale).astype(np.float32)
    return inp


@pytest.mark.parametrize("C", [64, 128])
def test_normalized_long_sequence(C):
    """Normalized linear attention over 131,089 tokens with the elu+1 features of
    the normalized workload: z passes 65504 after about 51k tokens."""
    L = 131072 + 17
    print(f"[range] normalized L={L} C={C}", flush=True)
    inp = W.make_chunk_inputs("normalized", "bf16", 1, 2, L, 64, 64, seed=21)
    o, s, z = gpu_chunk(inp, C, state_in=False, z_in=False)
    ro, rs, rz = oracle_chunk(inp, state_in=False, z_in=False)
    assert rz.max() > 2 * FP16_MAX
    assert_close(o, ro, TOL["bf16"], "o")
    assert_close(s, rs, TOL["bf16"], "state")
    assert_close(z, rz, 1e-5, "z")


@pytest.mark.parametrize("var", ["plain", "normalized"])
@pytest.mark.parametrize("C,dk,dv", [(64, 64, 64), (64, 128, 128), (128, 64, 64), (128, 128, 128)])
def test_state_grows_past_fp16(var, C, dk, dv):
    """Values with mean 50 make S grow by about 4000 per chunk: S passes 65504 in
    the 17th chunk and reaches 10^5 and beyond."""
    L = 40 * C + 9
    print(f"[range] growing state {var} C={C} dk={dk} dv={dv}", flush=True)
    inp = W.make_chunk_inputs(var, "bf16", 1, 2, L, dk, dv, seed=22, recipe="elu1")
    inp.v = W.f32_to_bf16_bits(W.bf16_bits_to_f32(inp.v) + 50.0)
    o, s, z = gpu_chunk(inp, C, state_in=False, z_in=False)
    ro, rs, rz = oracle_chunk(inp, state_in=False, z_in=False)
    assert np.abs(rs).max() > 2 * FP16_MAX
    assert_close(o, ro, TOL["bf16"], "o")
    assert_close(s, rs, TOL["bf16"], "state")


def _large_start_cases():
    out = []
    for var in ("plain", "normalized", "decay", "gated_delta"):
        for C in (64, 128):
            if var == "gated_delta" and C != 64:
                continue
            for dk, dv in ((64, 64), (128, 128), (32, 128)):
                out.append((var, C, dk, dv))
    return out


@pytest.mark.parametrize("var,C,dk,dv", _large_start_cases(), ids=lambda x: str(x))
@pytest.mark.parametrize("scale", [1e6, 1e7])
def test_large_initial_state(var, C, dk, dv, scale):
    """state_in entries of order 10^5-10^6 (N(0, 0.1^2) times 10^6 or 10^7), z_in
    of order 10^5 for the normalized variant: outputs, final state and
    normalizer against the oracle."""
    L = 3 * C + 17
    print(f"[range] large state_in {var} C={C} dk={dk} dv={dv} scale={scale:g}", flush=True)
    inp = W.make_chunk_inputs(var, "bf16", 2, 3, L, dk, dv, seed=23, with_state=True,
                              with_z=(var == "normalized"))
    inp = _scaled_start(inp, scale, 1e5)
    assert np.abs(inp.state_in).max() > 4 * FP16_MAX
    o, s, z = gpu_chunk(inp, C)
    ro, rs, rz = oracle_chunk(inp)
    assert_close(o, ro, TOL["bf16"], "o")
    assert_close(s, rs, TOL["bf16"], "state")
    if var == "normalized":
        assert_close(z, rz, 1e-5, "z")


@pytest.mark.parametrize("L", [5 * 64 + 23, 9 * 64 + 7])
def test_large_state_split_role_schedules(L):
    """Decay and the delta rule at d = 128 with 128 heads (64- and 32-column
    split-role workgroups) through the steady-state loop, from a state of order 10^6."""
    for var, H in (("decay", 64), ("gated_delta", 64)):
        print(f"[range] large state_in split roles {var} L={L}", flush=True)
        inp = W.make_chunk_inputs(var, "bf16", 2, H, L, 128, 128, seed=24, with_state=True)
        inp = _scaled_start(inp, 1e7)
        o, s, _ = gpu_chunk(inp, 64)
        ro, rs, _ = oracle_chunk(inp)
        assert_close(o, ro, TOL["bf16"], f"{var} o")
        assert_close(s, rs, TOL["bf16"], f"{var} state")
