"""GPU parity of the causal depthwise short convolution (la_short_conv) against the
fp64 oracle, element by element: several token tiles and ragged tails, every tap
count, with and without an incoming window, skipped tensors, pieces carried
through the window (including in place), the one-token decode use, and the
convolution feeding the chunkwise forward."""
import numpy as np
import pytest
import torch

import chunkwise_linear_rnn_causal_amd as la
import oracle
import workloads as W
from gpu_util import TOL, assert_close, dev, gpu_chunk, host64, oracle_chunk

pytestmark = pytest.mark.gpu


def conv_bound(x, w, win, dtype):
    """Per-element bound on |gpu - oracle|: the fp32 sum of K products is within
    K * 2^-24 * sum|w x| of the exact value (1e-6 * sum|w x| covers K <= 4 with
    margin), and a bf16 result adds at most half an ulp, 2^-8 |y| relative."""
    s, _ = oracle.short_conv(np.abs(x), np.abs(w), None if win is None else np.abs(win))
    return s * 1e-6, (2.0 ** -8 if dtype == "bf16" else 0.0)


def check_conv(got, ref, x, w, win, dtype, what):
    abs_b, rel_b = conv_bound(x, w, win, dtype)
    err = np.abs(got - ref)
    lim = abs_b + rel_b * np.abs(ref) + 1e-30
    bad = err > lim
    assert not bad.any(), f"{what}: {int(bad.sum())} elements out of bound, worst excess {float((err - lim).max()):.3e}"


def run_gpu(ci, use=(True, True, True), window=True, want_state=True):
    xs = [dev(ci.x[i]) if use[i] else None for i in range(3)]
    ws = [dev(ci.taps[i]) if use[i] else None for i in range(3)]
    wins = [dev(ci.window[i]) if (use[i] and window and ci.window[i] is not None) else None
            for i in range(3)]
    outs = la.la_short_conv(*xs, *ws, q_state_in=wins[0], k_state_in=wins[1], v_state_in=wins[2],
                            want_state=want_state)
    torch.cuda.synchronize()
    return [host64(o) for o in outs[:3]], [host64(s) for s in outs[3:]]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("L", [0, 1, 2, 3, 17, 100, 257])
def test_short_conv_matches_oracle(dt, K, L):
    ci = W.make_conv_inputs(dt, 2, 3, L, 64, 32, K, seed=21 + L, with_window=K > 1)
    ys, ss = run_gpu(ci)
    for i, name in enumerate("qkv"):
        x, win = ci.f64("x", i), ci.f64("window", i)
        ry, rs = oracle.short_conv(x, ci.taps[i], win)
        if L > 0:
            check_conv(ys[i], ry, x, ci.taps[i], win, dt, f"{name} y")
        assert np.array_equal(ss[i], rs), f"{name} window"     # raw copies: bit-exact


@pytest.mark.parametrize("dk,dv", [(32, 128), (128, 64), (96, 96), (8, 16)])
def test_short_conv_shapes_and_zero_window(dk, dv):
    ci = W.make_conv_inputs("bf16", 1, 4, 300, dk, dv, 4, seed=5)
    ys, ss = run_gpu(ci, window=False)
    for i in range(3):
        x = ci.f64("x", i)
        ry, rs = oracle.short_conv(x, ci.taps[i], None)
        check_conv(ys[i], ry, x, ci.taps[i], None, "bf16", "y")
        assert np.array_equal(ss[i], rs)


def test_short_conv_skips_tensors():
    ci = W.make_conv_inputs("bf16", 2, 2, 70, 64, 64, 4, seed=6, with_window=True)
    ys, ss = run_gpu(ci, use=(True, False, True))
    assert ys[1] is None and ss[1] is None
    for i in (0, 2):
        x, win = ci.f64("x", i), ci.f64("window", i)
        ry, rs = oracle.short_conv(x, ci.taps[i], win)
        check_conv(ys[i], ry, x, ci.taps[i], win, "bf16", "y")
        assert np.array_equal(ss[i], rs)


@pytest.mark.parametrize("cuts", [(1, 2, 3), (5, 40), (17,), (2, 3, 4, 5, 6, 7)])
def test_short_conv_pieces_in_place_equal_one_pass(cuts):
    """Convolve in pieces with the window updated in place (state_out is
    state_in); the pieces reproduce one pass bit for bit, and the window ends as
    the last K-1 inputs."""
    L, K = 64, 4
    ci = W.make_conv_inputs("bf16", 2, 3, L, 64, 32, K, seed=7, with_window=True)
    x = [dev(ci.x[i]) for i in range(3)]
    w = [dev(ci.taps[i]) for i in range(3)]
    one = la.la_short_conv(*x, *w, q_state_in=dev(ci.window[0]), k_state_in=dev(ci.window[1]),
                           v_state_in=dev(ci.window[2]), want_state=True)
    win = [dev(ci.window[i]).clone() for i in range(3)]
    parts, t0 = [[], [], []], 0
    for t1 in list(cuts) + [L]:
        xp = [xi[:, :, t0:t1].contiguous() for xi in x]
        outs = la.la_short_conv(*xp, *w, q_state_in=win[0], k_state_in=win[1], v_state_in=win[2],
                                q_state_out=win[0], k_state_out=win[1], v_state_out=win[2])
        for i in range(3):
            parts[i].append(outs[i])
        t0 = t1
    torch.cuda.synchronize()
    for i in range(3):
        assert torch.equal(torch.cat(parts[i], dim=2), one[i]), i
        assert torch.equal(win[i], one[3 + i]), i


def test_short_conv_decode_steps():
    """The decode use: one token per call with the window carried in place equals
    convolving the tokens in one pass (and the oracle)."""
    T, K = 6, 4
    ci = W.make_conv_inputs("f32", 3, 2, T, 128, 128, K, seed=8, with_window=True)
    x = [dev(ci.x[i]) for i in range(3)]
    w = [dev(ci.taps[i]) for i in range(3)]
    win = [dev(ci.window[i]).clone() for i in range(3)]
    steps = []
    for t in range(T):
        xt = [xi[:, :, t:t + 1].contiguous() for xi in x]
        steps.append(la.la_short_conv(*xt, *w, q_state_in=win[0], k_state_in=win[1], v_state_in=win[2],
                                      q_state_out=win[0], k_state_out=win[1], v_state_out=win[2])[:3])
    torch.cuda.synchronize()
    for i in range(3):
        got = host64(torch.cat([s[i] for s in steps], dim=2))
        xi, wi = ci.f64("x", i), ci.f64("window", i)
        ry, rs = oracle.short_conv(xi, ci.taps[i], wi)
        check_conv(got, ry, xi, ci.taps[i], wi, "f32", "decode y")
        assert np.array_equal(host64(win[i]), rs)


def test_short_conv_deterministic():
    ci = W.make_conv_inputs("bf16", 2, 4, 333, 64, 64, 4, seed=9, with_window=True)
    a, _ = run_gpu(ci)
    b, _ = run_gpu(ci)
    for i in range(3):
        assert np.array_equal(a[i], b[i])


@pytest.mark.parametrize("variant", ["decay", "plain"])
def test_short_conv_then_chunk_forward(variant):
    """The convolution as the prologue of the chunkwise forward: conv on the GPU,
    then la_chunk_fwd on its outputs, against the oracle's convolution followed
    by the oracle's recurrence. q, k, v are scaled by 1/sqrt(d) so the state
    stays well conditioned."""
    B, H, L, d, K = 2, 2, 200, 64, 4
    ci = W.make_conv_inputs("f32", B, H, L, d, d, K, seed=10)
    for i in range(3):
        ci.x[i] = (ci.x[i] / np.float32(np.sqrt(d))).astype(np.float32)
    xs = [dev(ci.x[i]) for i in range(3)]
    ws = [dev(ci.taps[i]) for i in range(3)]
    qc, kc, vc = la.la_short_conv(*xs, *ws)[:3]
    lg_np = W.make_chunk_inputs("decay", "f32", B, H, L, d, d, seed=10).log_gate
    lg = dev(lg_np) if variant == "decay" else None
    o, s, _ = la.la_chunk_fwd(variant, qc, kc, vc, lg, C=64, want_state=True)
    torch.cuda.synchronize()
    rq, rk, rv = (oracle.short_conv(ci.f64("x", i), ci.taps[i])[0] for i in range(3))
    ro, rs, _ = oracle.forward(variant, rq, rk, rv,
                               log_gate=None if lg_np is None or variant != "decay" else lg_np.astype(np.float64))
    assert_close(host64(o), ro, TOL["f32"], "o")
    assert_close(host64(s), rs, TOL["f32"], "state")
