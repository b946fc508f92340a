"""Guard bands around every buffer the library writes.

Each output (and the caller's workspace) is a view into a larger buffer whose
leading and trailing bands hold a fixed bit pattern; after the call both bands must
be bit-identical, so no kernel wrote before or past its buffer. Ragged lengths put
the last chunk's rows right next to the trailing band, where an unchecked row index
or a store of a padded tile would land. The guarded call must also produce the same
bits as a call with ordinary buffers (the kernels are deterministic)."""
import ctypes
import math

import numpy as np
import pytest
import torch

import chunkwise_linear_rnn_causal_amd as la
import workloads as W
from gpu_util import dev

pytestmark = pytest.mark.gpu

GUARD = 4096  # elements (bytes for the workspace) in each band
# fill patterns: a NaN payload for fp32, a NaN for bf16, a byte pattern for the workspace
PATTERN = {torch.float32: (torch.int32, 0x7FC0BEEF), torch.bfloat16: (torch.int16, 0x7FBE),
           torch.uint8: (torch.uint8, 0xA5)}


class Guarded:
    """A contiguous view of `shape` between two bands of the fill pattern."""

    def __init__(self, shape, dtype):
        self.n = math.prod(shape)
        self.buf = torch.empty(self.n + 2 * GUARD, dtype=dtype, device="cuda")
        raw, bits = PATTERN[dtype]
        self.buf.view(raw).fill_(bits)
        self.view = self.buf[GUARD:GUARD + self.n].view(shape)

    def check(self, what):
        raw, bits = PATTERN[self.buf.dtype]
        r = self.buf.view(raw)
        lead, tail = r[:GUARD], r[GUARD + self.n:]
        assert bool((lead == bits).all()), f"{what}: write before the buffer"
        assert bool((tail == bits).all()), f"{what}: write past the end of the buffer"


FWD_CASES = [(var, L, dk, odt) for var in ("plain", "normalized", "decay", "gated_delta", "vector_decay", "kda")
             for L in (17, 65, 147) for dk in (64, 128) for odt in (torch.float32, torch.bfloat16)]


@pytest.mark.parametrize("var,L,dk,odt", FWD_CASES, ids=lambda x: str(x).replace("torch.", ""))
def test_chunk_forward_writes_stay_in_bounds(var, L, dk, odt):
    B, H, dv = 1, 3, dk
    print(f"[guard] fwd {var} L{L} d{dk} o={odt}", flush=True)
    inp = W.make_chunk_inputs(var, "bf16", B, H, L, dk, dv, seed=71, with_state=True,
                              with_z=(var == "normalized"))
    args = [dev(x) for x in (inp.q, inp.k, inp.v, inp.log_gate, inp.beta, inp.state_in)]
    z_in = dev(inp.z_in) if var == "normalized" else None
    o = Guarded((B, H, L, dv), odt)
    s = Guarded((B, H, dk, dv), torch.float32)
    z = Guarded((B, H, dk), torch.float32) if var == "normalized" else None
    ws_bytes = la.la_chunk_fwd_workspace_size(var, 1, B, H, L, dk, dv, 64)
    ws = Guarded((ws_bytes,), torch.uint8) if ws_bytes else None
    la.la_chunk_fwd(var, *args, z_in, C=64, o=o.view, state_out=s.view, z_out=z.view if z else None,
                    workspace=ws.view if ws else None)
    ref_o, ref_s, ref_z = la.la_chunk_fwd(var, *args, z_in, C=64, out_dtype=odt, want_state=True,
                                          want_z=z is not None)
    torch.cuda.synchronize()
    for g, what in ((o, "o"), (s, "state_out"), (z, "z_out"), (ws, "workspace")):
        if g is not None:
            g.check(f"{var} {what}")
    assert torch.equal(o.view, ref_o) and torch.equal(s.view, ref_s)
    if z is not None:
        assert torch.equal(z.view, ref_z)


@pytest.mark.parametrize("var", ["plain", "decay", "gated_delta", "vector_decay", "kda"])
@pytest.mark.parametrize("odt", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_decode_writes_stay_in_bounds(var, odt):
    N, H, dk, dv = 3, 5, 128, 128
    print(f"[guard] decode {var} o={odt}", flush=True)
    S0 = W.make_decode_state(N, H, dk, dv, seed=72)
    st = W.make_decode_step(N, H, dk, dv, step=0, seed=72, with_beta=True)
    r = np.random.default_rng(72)
    if var in ("vector_decay", "kda"):
        lg = np.log(1.0 / (1.0 + np.exp(-r.normal(4.0, 1.0, (N, H, dk))))).astype(np.float32)
    else:
        lg = st.log_gate
    beta = st.beta if var in ("gated_delta", "kda") else None
    S = Guarded((N, H, dk, dv), torch.float32)
    S.view.copy_(dev(S0))
    o = Guarded((N, H, dv), odt)
    la.la_decode_step(var, dev(st.q), dev(st.k), dev(st.v), dev(lg) if var != "plain" else None, S.view,
                      o=o.view, beta=dev(beta))
    S_ref = dev(S0)
    o_ref = la.la_decode_step(var, dev(st.q), dev(st.k), dev(st.v), dev(lg) if var != "plain" else None, S_ref,
                              out_dtype=odt, beta=dev(beta))
    torch.cuda.synchronize()
    S.check(f"{var} state")
    o.check(f"{var} o")
    assert torch.equal(S.view, S_ref) and torch.equal(o.view, o_ref)


BWD_CASES = [("plain", "bf16", 64), ("decay", "bf16", 128), ("gated_delta", "bf16", 128),
             ("vector_decay", "bf16", 128), ("normalized", "f32", 64), ("decay", "f32", 64)]


@pytest.mark.parametrize("var,dt,d", BWD_CASES)
@pytest.mark.parametrize("L", [17, 65, 147])
def test_backward_writes_stay_in_bounds(var, dt, d, L):
    """The C entry point called with guarded gradient buffers and workspace."""
    B, H = 1, 3
    print(f"[guard] bwd {var} {dt} d{d} L{L}", flush=True)
    norm, gdn = var == "normalized", var == "gated_delta"
    inp = W.make_chunk_inputs(var, dt, B, H, L, d, d, seed=73, with_state=True, with_z=norm)
    do = W.make_backward_dout(dt, B, H, L, d, seed=73)
    r = np.random.default_rng(73)
    dso = r.normal(0.0, 0.1, (B, H, d, d)).astype(np.float32)
    dzo = r.normal(0.0, 0.1, (B, H, d)).astype(np.float32) if norm else None
    q, k, v, lg, be, si, dO = (dev(x) for x in (inp.q, inp.k, inp.v, inp.log_gate, inp.beta, inp.state_in, do))
    zi = dev(inp.z_in) if norm else None
    dso_t, dzo_t = dev(dso), dev(dzo)
    gshape = (B, H, L, d) if var == "vector_decay" else (B, H, L)
    outs = {"dq": Guarded((B, H, L, d), torch.float32), "dk": Guarded((B, H, L, d), torch.float32),
            "dv": Guarded((B, H, L, d), torch.float32),
            "dlg": Guarded(gshape, torch.float32) if lg is not None else None,
            "dbe": Guarded((B, H, L), torch.float32) if gdn else None,
            "dsi": Guarded((B, H, d, d), torch.float32),
            "dzi": Guarded((B, H, d), torch.float32) if norm else None}
    code = 1 if dt == "bf16" else 0
    ws_bytes = la.la_chunk_bwd_workspace_size(var, code, B, H, L, d, d, 64)
    ws = Guarded((max(ws_bytes, 256),), torch.uint8)
    lib = la.load_library()

    def p(x):
        return None if x is None else ctypes.c_void_p(x.view.data_ptr() if isinstance(x, Guarded) else x.data_ptr())

    st = lib.la_chunk_bwd(la.VARIANTS[var], code, p(q), p(k), p(v), p(lg), p(be), p(si), p(zi), p(dO),
                          p(dso_t), p(dzo_t), p(outs["dq"]), p(outs["dk"]), p(outs["dv"]), p(outs["dlg"]),
                          p(outs["dbe"]), p(outs["dsi"]), p(outs["dzi"]), B, H, L, d, d, 64, p(ws),
                          ws.n, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, la.la_status_str(st)
    ref = la.la_chunk_bwd(var, q, k, v, dO, lg, si, dso_t, beta=be, z_in=zi, d_z_out=dzo_t,
                          want_d_state_in=True, want_d_z_in=norm)
    torch.cuda.synchronize()
    for name, g in outs.items():
        if g is not None:
            g.check(f"{var} {name}")
    ws.check(f"{var} workspace")
    pairs = [("dq", ref[0]), ("dk", ref[1]), ("dv", ref[2]), ("dsi", ref[4])]
    if lg is not None:
        pairs.append(("dlg", ref[3]))
    if gdn:
        pairs.append(("dbe", ref[5]))
    if norm:
        pairs.append(("dzi", ref[5]))
    for name, want in pairs:
        assert torch.equal(outs[name].view, want), name


@pytest.mark.parametrize("L", [1, 17, 70])
def test_short_conv_writes_stay_in_bounds(L):
    B, H, d, K = 2, 3, 64, 4
    print(f"[guard] short conv L{L}", flush=True)
    ci = W.make_conv_inputs("bf16", B, H, L, d, d, K, seed=74, with_window=True)
    xs = [dev(x) for x in ci.x]
    taps = [dev(t) for t in ci.taps]
    wins = [dev(w) for w in ci.window]
    outs = [Guarded((B, H, L, d), torch.bfloat16) for _ in range(3)]
    wouts = [Guarded((B, H, K - 1, d), torch.bfloat16) for _ in range(3)]
    la.la_short_conv(*xs, *taps, q_state_in=wins[0], k_state_in=wins[1], v_state_in=wins[2],
                     q_out=outs[0].view, k_out=outs[1].view, v_out=outs[2].view,
                     q_state_out=wouts[0].view, k_state_out=wouts[1].view, v_state_out=wouts[2].view)
    ref = la.la_short_conv(*xs, *taps, q_state_in=wins[0], k_state_in=wins[1], v_state_in=wins[2],
                           want_state=True)
    torch.cuda.synchronize()
    for i in range(3):
        outs[i].check(f"conv out {i}")
        wouts[i].check(f"conv window {i}")
        assert torch.equal(outs[i].view, ref[i]) and torch.equal(wouts[i].view, ref[3 + i])


@pytest.mark.parametrize("L", [17, 65, 147])
@pytest.mark.parametrize("odt", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_conv_fused_forward_writes_stay_in_bounds(L, odt):
    """The delta rule with the short convolution fused: o, the state, the three
    carried windows and the workspace, each between guard bands."""
    from test_gpu_conv_fused import _case
    B, H, d, K = 1, 3, 128, 4
    print(f"[guard] conv-fused L{L} o={odt}", flush=True)
    inp, taps, wins, lg = _case(B, H, L, d, d, K, 75, windows=True, gate=True, state=True)
    args = [dev(x) for x in (inp.q, inp.k, inp.v)] + [dev(t) for t in taps] + [dev(lg), dev(inp.beta),
                                                                             dev(inp.state_in)]
    win_in = dict(q_win_in=dev(wins[0]), k_win_in=dev(wins[1]), v_win_in=dev(wins[2]))
    o = Guarded((B, H, L, d), odt)
    s = Guarded((B, H, d, d), torch.float32)
    wo = [Guarded((B, H, K - 1, d), torch.bfloat16) for _ in range(3)]
    ws_bytes = la.la_chunk_fwd_conv_workspace_size("gated_delta", 1, B, H, L, d, d, 64, K)
    ws = Guarded((ws_bytes,), torch.uint8) if ws_bytes else None
    la.la_chunk_fwd_conv("gated_delta", *args, **win_in, o=o.view, state_out=s.view,
                         q_win_out=wo[0].view, k_win_out=wo[1].view, v_win_out=wo[2].view,
                         workspace=ws.view if ws else None)
    ref_o, ref_s, ref_w = la.la_chunk_fwd_conv("gated_delta", *args, **win_in, out_dtype=odt, want_state=True,
                                               want_windows=True)
    torch.cuda.synchronize()
    for g, what in [(o, "o"), (s, "state_out"), (ws, "workspace")] + [(w, f"window {i}") for i, w in enumerate(wo)]:
        if g is not None:
            g.check(f"conv-fused {what}")
    assert torch.equal(o.view, ref_o) and torch.equal(s.view, ref_s)
    for i in range(3):
        assert torch.equal(wo[i].view, ref_w[i])


@pytest.mark.parametrize("var", ["decay", "gated_delta", "normalized"])
@pytest.mark.parametrize("L", [17, 147])
def test_noalloc_forward_writes_stay_in_bounds(var, L):
    """The allocation-free forward: its outputs between guard bands, the same bits
    as the forward with a caller workspace."""
    B, H, d = 1, 3, 128 if var != "normalized" else 64
    print(f"[guard] noalloc {var} L{L}", flush=True)
    inp = W.make_chunk_inputs(var, "bf16", B, H, L, d, d, seed=76, with_state=True, with_z=(var == "normalized"))
    args = [dev(x) for x in (inp.q, inp.k, inp.v, inp.log_gate, inp.beta, inp.state_in)]
    z_in = dev(inp.z_in) if var == "normalized" else None
    o = Guarded((B, H, L, d), torch.float32)
    s = Guarded((B, H, d, d), torch.float32)
    z = Guarded((B, H, d), torch.float32) if var == "normalized" else None
    la.la_chunk_fwd_noalloc(var, *args, z_in, o=o.view, state_out=s.view, z_out=z.view if z else None)
    ref_o, ref_s, ref_z = la.la_chunk_fwd(var, *args, z_in, out_dtype=torch.float32, want_state=True,
                                          want_z=z is not None)
    torch.cuda.synchronize()
    for g, what in ((o, "o"), (s, "state_out"), (z, "z_out")):
        if g is not None:
            g.check(f"noalloc {var} {what}")
    assert torch.equal(o.view, ref_o) and torch.equal(s.view, ref_s)
    if z is not None:
        assert torch.equal(z.view, ref_z)
