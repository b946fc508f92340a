"""HIP graph capture of the entry points, and independent calls on two streams.

The entry points allocate nothing and issue no memset, copy or synchronisation on
the stream, so a sequence of calls can be captured once and replayed. Each graph
test replays its graph several times, with eager work and synchronisations
between the replays, and checks every replay against the eager result bit for bit
(the kernels are deterministic). Calls with their own buffers and workspaces may
run on two streams at once."""
import pytest
import torch

import chunkwise_linear_rnn_causal_amd as la
import workloads as W
from gpu_util import dev

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _eager_noise():
    # unrelated eager work between replays
    a = torch.randn(512, 512, device="cuda")
    (a @ a).sum().item()


def test_decode_steps_in_a_graph():
    """Ten decode steps on one state, alternating the delta rule and decay."""
    N, H, dk, dv, steps = 64, 8, 128, 128, 10
    print(f"[graph] decode N{N} H{H} d{dk} steps={steps}", flush=True)
    S0 = dev(W.make_decode_state(N, H, dk, dv, seed=5))
    ins = []
    for i in range(steps):
        st = W.make_decode_step(N, H, dk, dv, step=i, seed=5, with_beta=True)
        ins.append((dev(st.q), dev(st.k), dev(st.v), dev(st.log_gate), dev(st.beta)))
    outs = [torch.empty((N, H, dv), dtype=torch.bfloat16, device="cuda") for _ in range(steps)]

    def run(S):
        for i, (q, k, v, lg, be) in enumerate(ins):
            delta = i % 2 == 0
            la.la_decode_step("gated_delta" if delta else "decay", q, k, v, lg, S, o=outs[i],
                              beta=be if delta else None)

    S = S0.clone()
    run(S)
    torch.cuda.synchronize()
    ref_S, ref_o = S.clone(), [o.clone() for o in outs]

    Sg = S0.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(Sg)
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        Sg.copy_(S0)
        for o in outs:
            o.fill_(0)
        _eager_noise()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Sg, ref_S), f"replay {rep}: state"
        for i, (o, r) in enumerate(zip(outs, ref_o)):
            assert torch.equal(o, r), f"replay {rep}: o of step {i}"


@pytest.mark.parametrize("var", ["normalized", "decay", "gated_delta"])
def test_chunk_forward_in_a_graph(var):
    """One chunk forward (ragged length, initial state; the delta rule with its
    workspace) captured and replayed."""
    B, H, L, dk, dv, C = 2, 4, 3 * 64 + 29, 128 if var != "normalized" else 64, 64, 64
    print(f"[graph] chunk {var} B{B} H{H} L{L} d{dk}x{dv}", flush=True)
    inp = W.make_chunk_inputs(var, "bf16", B, H, L, dk, dv, seed=21, with_state=True,
                              with_z=(var == "normalized"))
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    lg, be = dev(inp.log_gate), dev(inp.beta)
    s_in, z_in = dev(inp.state_in), dev(inp.z_in)
    o = torch.empty((B, H, L, dv), dtype=torch.float32, device="cuda")
    S = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
    z = torch.empty((B, H, dk), dtype=torch.float32, device="cuda") if var == "normalized" else None
    ws_bytes = la.la_chunk_fwd_workspace_size(var, 1, B, H, L, dk, dv, C)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda") if ws_bytes else None

    def run():
        la.la_chunk_fwd(var, q, k, v, lg, be, C=C, state_in=s_in, z_in=z_in, o=o, state_out=S,
                        z_out=z, workspace=ws)

    run()
    torch.cuda.synchronize()
    ref = [o.clone(), S.clone()] + ([z.clone()] if z is not None else [])

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        got = [o, S] + ([z] if z is not None else [])
        for t in got:
            t.fill_(0)
        _eager_noise()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("o", "state", "z"), got, ref):
            assert torch.equal(t, r), f"replay {rep}: {name}"


def test_independent_calls_on_two_streams():
    """Two delta-rule forwards and two decode steps, each with its own buffers and
    workspace, issued on two streams at once: the same bits as one after the other."""
    print("[streams] two delta-rule forwards and two decode steps", flush=True)
    B, H, L, dk, dv, C = 2, 4, 5 * 64 + 7, 128, 128, 64
    calls = []
    for seed in (31, 32):
        inp = W.make_chunk_inputs("gated_delta", "bf16", B, H, L, dk, dv, seed=seed, with_state=True)
        args = [dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.log_gate), dev(inp.beta), dev(inp.state_in)]
        o = torch.empty((B, H, L, dv), dtype=torch.float32, device="cuda")
        S = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
        ws = torch.empty(la.la_chunk_fwd_workspace_size("gated_delta", 1, B, H, L, dk, dv, C),
                         dtype=torch.uint8, device="cuda")
        calls.append((args, o, S, ws))
    N, Hd = 32, 8
    dec = []
    for seed in (41, 42):
        S0 = dev(W.make_decode_state(N, Hd, dk, dv, seed=seed))
        st = W.make_decode_step(N, Hd, dk, dv, step=0, seed=seed, with_beta=True)
        dec.append((S0, S0.clone(), [dev(st.q), dev(st.k), dev(st.v), dev(st.log_gate), dev(st.beta)],
                    torch.empty((N, Hd, dv), dtype=torch.float32, device="cuda")))

    def run(i, stream):
        (q, k, v, lg, be, s_in), o, S, ws = calls[i]
        la.la_chunk_fwd("gated_delta", q, k, v, lg, be, state_in=s_in, C=C, o=o, state_out=S,
                        workspace=ws, stream=stream)
        _, Sd, (dq, dk_, dv_, dlg, dbe), do = dec[i]
        la.la_decode_step("gated_delta", dq, dk_, dv_, dlg, Sd, o=do, beta=dbe, stream=stream)

    cur = torch.cuda.current_stream()
    for i in range(2):
        run(i, cur)
    torch.cuda.synchronize()
    ref = [(c[1].clone(), c[2].clone(), d[1].clone(), d[3].clone()) for c, d in zip(calls, dec)]
    for c, d in zip(calls, dec):
        c[1].fill_(0)
        c[2].fill_(0)
        d[1].copy_(d[0])
        d[3].fill_(0)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for i in range(2):
        run(i, streams[i])
    torch.cuda.synchronize()
    for i, (c, d) in enumerate(zip(calls, dec)):
        for name, got, r in zip(("o", "state", "decode state", "decode o"), (c[1], c[2], d[1], d[3]), ref[i]):
            assert torch.equal(got, r), f"call {i}: {name}"
