"""The seeded input generator: storage rounding, determinism, distributions."""
import numpy as np
import torch

import workloads as W


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100_000).astype(np.float32) * 7
    x[:4] = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -0.0, 65504.0]   # ties to even
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = W.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_slices_regenerate_identically():
    full = W.make_chunk_inputs("gated_delta", "bf16", 2, 3, 40, 8, 8, seed=5)
    part = W.make_chunk_inputs("gated_delta", "bf16", 2, 3, 40, 8, 8, seed=5, heads=[(1, 2), (0, 1)])
    assert np.array_equal(part.q[0, 0], full.q[1, 2]) and np.array_equal(part.v[0, 1], full.v[0, 1])
    assert np.array_equal(part.log_gate[0, 0], full.log_gate[1, 2])
    assert np.array_equal(part.beta[0, 1], full.beta[0, 1])


def test_recipes():
    n = W.make_chunk_inputs("normalized", "bf16", 1, 2, 512, 16, 16, seed=0)
    assert np.all(n.f64("q") > 0) and np.all(n.f64("k") > 0)          # elu(x)+1 > 0
    g = W.make_chunk_inputs("gated_delta", "bf16", 1, 2, 512, 32, 32, seed=0)
    norms = np.linalg.norm(g.f64("k"), axis=-1)
    assert np.allclose(norms, 1.0, atol=2e-2)                           # L2-normalised, then bf16
    gam = np.exp(g.f64("log_gate"))
    assert 0.95 < gam.mean() < 0.99 and np.all(gam < 1)                # sigmoid(N(4,1))
    assert 0.3 < g.beta.mean() < 0.7 and np.all((g.beta > 0) & (g.beta < 1))
    p = W.make_chunk_inputs("plain", "f32", 1, 1, 4096, 32, 32, seed=0)
    assert p.q.dtype == np.float32 and abs(p.q.std() * np.sqrt(32) - 1) < 0.02


def test_decode_inputs():
    S = W.make_decode_state(4, 2, 16, 16, seed=0)
    assert S.dtype == np.float32 and abs(S.std() - 0.1) < 0.01
    st = W.make_decode_step(4, 2, 16, 16, step=3, seed=0)
    st2 = W.make_decode_step(4, 2, 16, 16, step=3, seed=0)
    assert np.array_equal(st.q, st2.q) and st.q.shape == (4, 2, 16) and st.log_gate.shape == (4, 2)
