"""la_chunk_fwd_noalloc (through the C ABI) against la_chunk_fwd with a caller
workspace: the same results, to the bf16 tolerance when the sequence runs in
pieces chained through the state, bit for bit when it runs in one piece. Calls
follow one another on the same static scratch, larger ones first, so a stale
scratch would show."""
import numpy as np
import pytest
import torch

import chunkwise_linear_rnn_causal_amd as la
import workloads as W
from gpu_util import TOL, assert_close, dev, host64, oracle_chunk

pytestmark = pytest.mark.gpu


def _both(inp, C=64, state_out=True, state_in=True):
    args = [dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.log_gate), dev(inp.beta),
            dev(inp.state_in) if state_in else None]
    o_ref, s_ref, _ = la.la_chunk_fwd(inp.variant, *args, C=C, want_state=True)
    B, H, L, dv, dk = inp.B, inp.H, inp.L, inp.dv, inp.dk
    o = torch.full((B, H, L, dv), float("nan"), dtype=torch.float32, device="cuda")
    s = torch.full((B, H, dk, dv), float("nan"), dtype=torch.float32, device="cuda") if state_out else None
    la.la_chunk_fwd_noalloc(inp.variant, *args, C=C, o=o, state_out=s)
    torch.cuda.synchronize()
    return o, s, o_ref, s_ref


def test_noalloc_matches_the_workspace_entry_point():
    # 1) the delta-rule workload's full size: 268 MB of per-chunk products, run
    #    in pieces through the 64 MiB scratch, the state carried in state_out
    print("[noalloc] gated_delta B2 H16 L8192 d128 (pieces, state_out)", flush=True)
    inp = W.make_chunk_inputs("gated_delta", "bf16", 2, 16, 8192, 128, 128, seed=31, with_state=True)
    o, s, o_ref, s_ref = _both(inp)
    eo = assert_close(host64(o), host64(o_ref), TOL["bf16"], "o, pieces vs one pass")
    es = assert_close(host64(s), host64(s_ref), TOL["bf16"], "state, pieces vs one pass")
    print(f"[noalloc] pieces vs one pass: max|diff|/RMS o={eo:.2e} state={es:.2e}", flush=True)

    # 2) smaller, pieces again, no state_out (the state is carried in the scratch)
    print("[noalloc] gated_delta B4 H32 L1100 d128 (pieces, no state_out)", flush=True)
    inp = W.make_chunk_inputs("gated_delta", "bf16", 4, 32, 1100, 128, 128, seed=32, with_state=True)
    o, _, o_ref, _ = _both(inp, state_out=False)
    assert_close(host64(o), host64(o_ref), TOL["bf16"], "o, pieces vs one pass")
    ro, _, _ = oracle_chunk(inp)
    eo = assert_close(host64(o), ro, TOL["bf16"], "o, pieces vs oracle")
    print(f"[noalloc] pieces without state_out vs oracle: max|err|/RMS o={eo:.2e}", flush=True)

    # 3) smaller again: one piece, bit for bit
    print("[noalloc] gated_delta B1 H3 L300 d64 (one piece)", flush=True)
    inp = W.make_chunk_inputs("gated_delta", "bf16", 1, 3, 300, 64, 64, seed=33, with_state=True)
    o, s, o_ref, s_ref = _both(inp)
    assert torch.equal(o, o_ref) and torch.equal(s, s_ref)


@pytest.mark.parametrize("var,dt", [("gated_delta", "f32"), ("decay", "bf16"), ("normalized", "bf16"),
                                    ("kda", "bf16")])
def test_noalloc_one_piece_is_bit_exact(var, dt):
    print(f"[noalloc] {var} {dt} one piece", flush=True)
    inp = W.make_chunk_inputs(var, dt, 2, 3, 201, 64, 64, seed=34, with_state=True)
    o, s, o_ref, s_ref = _both(inp)
    assert torch.equal(o, o_ref) and torch.equal(s, s_ref)


def test_noalloc_in_place_carry_over_pieces():
    """state_out == state_in, several pieces (96 heads of d = 128: 21 chunks per
    piece), ragged last chunk; against the oracle."""
    print("[noalloc] gated_delta B3 H32 L2000 d128, state_out = state_in", flush=True)
    inp = W.make_chunk_inputs("gated_delta", "bf16", 3, 32, 2000, 128, 128, seed=35, with_state=True)
    q, k, v, lg, be = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.log_gate), dev(inp.beta)
    S = dev(inp.state_in)
    o, _, _ = la.la_chunk_fwd_noalloc("gated_delta", q, k, v, lg, be, S, state_out=S)
    torch.cuda.synchronize()
    ro, rs, _ = oracle_chunk(inp)
    assert_close(host64(o), ro, TOL["bf16"], "o")
    assert_close(host64(S), rs, TOL["bf16"], "state")
