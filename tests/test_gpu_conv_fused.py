"""GPU parity of la_chunk_fwd_conv, the gated delta rule with the short causal
convolution of q, k, v fused into its preparation, against the fp64 oracle's
short convolution followed by its delta-rule recurrence: head sizes, tap counts,
edge lengths (shorter than the window too), incoming windows, in-place window
updates, a sequence run in two pieces chained through the windows and the state,
C = 128, and every head of the delta-rule workload at full size. o and the final
state are held to the bf16 rule (max|err| <= 2e-2 RMS); the outgoing windows are
raw copies and must match bit for bit."""
import numpy as np
import pytest
import torch

import chunkwise_linear_rnn_causal_amd as la
import oracle
import workloads as W
from gpu_util import TOL, assert_close, dev, host64

pytestmark = pytest.mark.gpu


def _unit_rows(r, shape):
    x = r.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _case(B, H, L, dk, dv, K, seed, windows=True, gate=True, state=True):
    inp = W.make_chunk_inputs("gated_delta", "bf16", B, H, L, dk, dv, seed=seed, with_state=state)
    ci = W.make_conv_inputs("bf16", 1, H, 1, dk, dv, K, seed=seed)
    r = np.random.default_rng(seed + 3000)
    wins = [None, None, None]
    if windows and K > 1:
        wins = [W.f32_to_bf16_bits(_unit_rows(r, (B, H, K - 1, dk)).astype(np.float32)),
                W.f32_to_bf16_bits(_unit_rows(r, (B, H, K - 1, dk)).astype(np.float32)),
                W.f32_to_bf16_bits(r.standard_normal((B, H, K - 1, dv)).astype(np.float32))]
    lg = inp.log_gate if gate else None
    return inp, ci.taps, wins, lg


def _oracle(inp, taps, wins, lg, state=True):
    xs = []
    for i, name in enumerate(("q", "k", "v")):
        y, _ = oracle.short_conv(inp.f64(name), taps[i].astype(np.float64),
                                 None if wins[i] is None else W.to_f64(wins[i]))
        xs.append(y)
    o, s, _ = oracle.forward("gated_delta", xs[0], xs[1], xs[2],
                             log_gate=None if lg is None else lg.astype(np.float64), beta=inp.f64("beta"),
                             state_in=inp.f64("state_in") if state else None)
    return o, s


def _expected_windows(inp, wins, K):
    out = []
    for i, name in enumerate(("q", "k", "v")):
        x = getattr(inp, name)
        B, H, L, d = x.shape
        prev = wins[i] if wins[i] is not None else np.zeros((B, H, K - 1, d), np.uint16)
        out.append(np.concatenate([prev, x], axis=2)[:, :, L:L + K - 1] if K > 1 else prev)
    return out


def _run(inp, taps, wins, lg, K, state=True, want_windows=True, C=64, win_out=None):
    kw = {}
    if win_out is not None:
        kw = dict(q_win_out=win_out[0], k_win_out=win_out[1], v_win_out=win_out[2])
    o, s, w = la.la_chunk_fwd_conv("gated_delta", dev(inp.q), dev(inp.k), dev(inp.v),
                                   *[dev(t) for t in taps], dev(lg), dev(inp.beta),
                                   dev(inp.state_in) if state else None,
                                   q_win_in=dev(wins[0]), k_win_in=dev(wins[1]), v_win_in=dev(wins[2]),
                                   want_windows=want_windows, want_state=True, C=C, **kw)
    torch.cuda.synchronize()
    return o, s, w


def _check(B, H, L, dk, dv, K, seed, tag="", **kw):
    print(f"[conv-fused] {tag} B{B} H{H} L{L} dk{dk} dv{dv} K{K} {kw}", flush=True)
    state = kw.pop("state", True)
    windows = kw.pop("windows", True)
    gate = kw.pop("gate", True)
    C = kw.pop("C", 64)
    inp, taps, wins, lg = _case(B, H, L, dk, dv, K, seed, windows=windows, gate=gate, state=state)
    o, s, w = _run(inp, taps, wins, lg, K, state=state, C=C)
    ro, rs = _oracle(inp, taps, wins, lg, state=state)
    if L > 0:
        assert_close(host64(o), ro, TOL["bf16"], "o")
    assert_close(host64(s), rs, TOL["bf16"] if L > 0 else 0.0, "state")
    if K > 1:
        for got, want in zip(w, _expected_windows(inp, wins, K)):
            assert np.array_equal(got.cpu().view(torch.int16).numpy().view(np.uint16), want)


@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 64), (128, 128), (64, 128), (128, 64), (32, 128)])
def test_conv_fused_matches_oracle(dk, dv):
    _check(2, 3, 3 * 64 + 17, dk, dv, 4, seed=61)


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_conv_fused_tap_counts(K):
    _check(1, 2, 150, 64, 64, K, seed=62)


@pytest.mark.parametrize("L", [0, 1, 2, 3, 5, 63, 64, 65, 130])
def test_conv_fused_edge_lengths(L):
    _check(1, 2, L, 64, 64, 4, seed=63, tag="edge")


def test_conv_fused_without_gate_windows_or_state():
    _check(2, 2, 200, 128, 128, 4, seed=64, gate=False, windows=False, state=False)


def test_conv_fused_chunk_128():
    _check(1, 2, 300, 128, 128, 4, seed=65, C=128)


def test_conv_fused_in_place_windows_and_pieces():
    """A sequence run as two calls: the first call's windows (updated in place) and
    final state feed the second; the outputs equal one pass of the oracle."""
    B, H, L1, L2, dk, dv, K = 1, 2, 100, 77, 64, 64, 4
    inp, taps, wins, lg = _case(B, H, L1 + L2, dk, dv, K, seed=66, state=True)
    ro, rs = _oracle(inp, taps, wins, lg)
    sl = lambda x, a, b: None if x is None else np.ascontiguousarray(x[:, :, a:b])
    wdev = [dev(x) for x in wins]
    outs = []
    state = dev(inp.state_in)
    for a, b in ((0, L1), (L1, L1 + L2)):
        o, s, _ = la.la_chunk_fwd_conv("gated_delta", dev(sl(inp.q, a, b)), dev(sl(inp.k, a, b)),
                                       dev(sl(inp.v, a, b)), *[dev(t) for t in taps], dev(sl(lg, a, b)),
                                       dev(sl(inp.beta, a, b)), state, q_win_in=wdev[0], k_win_in=wdev[1],
                                       v_win_in=wdev[2], q_win_out=wdev[0], k_win_out=wdev[1],
                                       v_win_out=wdev[2], want_windows=True, want_state=True)
        torch.cuda.synchronize()
        outs.append(host64(o))
        state = s
    assert_close(np.concatenate(outs, axis=2), ro, TOL["bf16"], "o")
    assert_close(host64(state), rs, TOL["bf16"], "state")


def test_conv_fused_full_size_all_heads():
    """The delta-rule workload (B2 H16 L8192 d128) with a K = 4 convolution in
    front, every head against the oracle."""
    c = W.CONFIGS["gated_delta_bf16_b2h16_l8192_d128"]
    B, H, L, dk, dv = c["B"], c["H"], c["L"], c["dk"], c["dv"]
    print("[conv-fused] full size", flush=True)
    inp = W.config_chunk_inputs("gated_delta_bf16_b2h16_l8192_d128", seed=0)
    taps = W.make_conv_inputs("bf16", 1, H, 1, dk, dv, 4, seed=0).taps
    o, s, _ = la.la_chunk_fwd_conv("gated_delta", dev(inp.q), dev(inp.k), dev(inp.v), *[dev(t) for t in taps],
                                   dev(inp.log_gate), dev(inp.beta), want_state=True)
    torch.cuda.synchronize()
    xs = [oracle.short_conv(inp.f64(nm), taps[i].astype(np.float64), threads=16)[0]
          for i, nm in enumerate(("q", "k", "v"))]
    ro, rs, _ = oracle.forward("gated_delta", xs[0], xs[1], xs[2], log_gate=inp.f64("log_gate"),
                               beta=inp.f64("beta"), threads=16)
    e_o = assert_close(host64(o), ro, TOL["bf16"], "o")
    e_s = assert_close(host64(s), rs, TOL["bf16"], "state")
    print(f"[conv-fused] full size max|err|/RMS o {e_o:.2e} state {e_s:.2e}", flush=True)
