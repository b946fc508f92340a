"""The Python binding refuses mismatched tensors before any library call: wrong
shapes, dtypes or devices would otherwise reach the kernels as raw pointers and
read or write out of bounds. Runs on the CPU (no kernel is launched)."""
from __future__ import annotations

import pytest
import torch

import chunkwise_linear_rnn_causal_amd as la

bf, f32 = torch.bfloat16, torch.float32
B, H, L, DK, DV = 2, 3, 70, 64, 32


def t(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def fwd_args(variant="decay"):
    gate = t(B, H, L, DK, dtype=f32) if variant == "vector_decay" else t(B, H, L, dtype=f32)
    return dict(q=t(B, H, L, DK), k=t(B, H, L, DK), v=t(B, H, L, DV),
                log_gate=None if variant in ("plain", "normalized") else gate,
                beta=t(B, H, L, dtype=f32) if variant == "gated_delta" else None)


@pytest.mark.parametrize("change, msg", [
    (dict(k=t(B, H, L, DK, dtype=f32)), "k has dtype"),
    (dict(k=t(B, H, L + 1, DK)), "k has shape"),
    (dict(v=t(B, H + 1, L, DV)), "v has shape"),
    (dict(log_gate=t(B, H, L, dtype=torch.float64)), "log_gate has dtype"),
    (dict(log_gate=t(B, H, L - 1, dtype=f32)), "log_gate has shape"),
    (dict(state_in=t(B, H, DV, DK, dtype=f32)), "state_in has shape"),
    (dict(state_in=t(B, H, DK, DV)), "state_in has dtype"),
    (dict(o=t(B, H, L, DK, dtype=f32)), "o has shape"),
    (dict(state_out=t(B, 1, DK, DV, dtype=f32)), "state_out has shape"),
])
def test_chunk_fwd_rejects_mismatched_tensors(change, msg):
    a = fwd_args()
    a.update(change)
    with pytest.raises(ValueError, match=msg):
        la.la_chunk_fwd("decay", **a)


def test_chunk_fwd_vector_decay_needs_a_gate_per_key_channel():
    a = fwd_args("vector_decay")
    a["log_gate"] = t(B, H, L, dtype=f32)  # the scalar-gate shape
    with pytest.raises(ValueError, match=r"log_gate has shape"):
        la.la_chunk_fwd("vector_decay", **a)


def test_chunk_fwd_rejects_normalizer_and_beta_shapes():
    a = fwd_args("normalized")
    with pytest.raises(ValueError, match="z_in has shape"):
        la.la_chunk_fwd("normalized", **a, z_in=t(B, H, DV, dtype=f32))
    a = fwd_args("gated_delta")
    a["beta"] = t(B, H, L, 1, dtype=f32)
    with pytest.raises(ValueError, match="beta has shape"):
        la.la_chunk_fwd("gated_delta", **a)


@pytest.mark.parametrize("variant", ["plain", "normalized", "decay", "gated_delta", "vector_decay"])
def test_chunk_fwd_well_formed_cpu_tensors_are_refused_for_the_device(variant):
    with pytest.raises(ValueError, match="GPU device"):
        la.la_chunk_fwd(variant, **fwd_args(variant))


def test_chunk_fwd_rejects_unknown_variant():
    with pytest.raises(ValueError, match="unknown variant"):
        la.la_chunk_fwd("softmax", **fwd_args())


N = 5


def dec_args(variant="decay"):
    return dict(q=t(N, H, DK), k=t(N, H, DK), v=t(N, H, DV),
                log_gate=t(N, H, DK, dtype=f32) if variant == "vector_decay" else t(N, H, dtype=f32),
                state=t(N, H, DK, DV, dtype=f32))


@pytest.mark.parametrize("change, msg", [
    (dict(state=t(N, H - 1, DK, DV, dtype=f32)), "state has shape"),
    (dict(state=t(N, H, DK, DV)), "state has dtype"),
    (dict(k=t(N, H, DK, dtype=f32)), "k has dtype"),
    (dict(v=t(N + 1, H, DV)), "v has shape"),
    (dict(log_gate=t(N, H, 1, dtype=f32)), "log_gate has shape"),
    (dict(o=t(N, H, DK, dtype=f32)), "o has shape"),
])
def test_decode_step_rejects_mismatched_tensors(change, msg):
    a = dec_args()
    a.update(change)
    with pytest.raises(ValueError, match=msg):
        la.la_decode_step("decay", a.pop("q"), a.pop("k"), a.pop("v"), a.pop("log_gate"), a.pop("state"), **a)


def test_decode_step_vector_gate_shape_and_device():
    a = dec_args("vector_decay")
    with pytest.raises(ValueError, match="GPU device"):
        la.la_decode_step("vector_decay", a["q"], a["k"], a["v"], a["log_gate"], a["state"])
    with pytest.raises(ValueError, match="log_gate has shape"):
        la.la_decode_step("vector_decay", a["q"], a["k"], a["v"], t(N, H, dtype=f32), a["state"])


@pytest.mark.parametrize("change, msg", [
    (dict(d_o=t(B, H, L, DV, dtype=f32)), "d_o has dtype"),
    (dict(d_o=t(B, H, L, DK)), "d_o has shape"),
    (dict(log_gate=t(B, H, L, DK, dtype=f32)), "log_gate has shape"),
    (dict(d_state_out=t(B, H, DV, DK, dtype=f32)), "d_state_out has shape"),
])
def test_chunk_bwd_rejects_mismatched_tensors(change, msg):
    a = dict(q=t(B, H, L, DK), k=t(B, H, L, DK), v=t(B, H, L, DV), d_o=t(B, H, L, DV),
             log_gate=t(B, H, L, dtype=f32))
    a.update(change)
    with pytest.raises(ValueError, match=msg):
        la.la_chunk_bwd("decay", **a)


def test_short_conv_rejects_mismatched_tensors():
    x, w = t(B, H, L, DK), t(H, DK, 4, dtype=f32)
    with pytest.raises(ValueError, match="w_q has shape"):
        la.la_short_conv(q=x, w_q=t(H + 1, DK, 4, dtype=f32))
    with pytest.raises(ValueError, match="q_state_in has shape"):
        la.la_short_conv(q=x, w_q=w, q_state_in=t(B, H, 4, DK))
    with pytest.raises(ValueError, match="k has shape"):
        la.la_short_conv(q=x, k=t(B, H, L - 1, DK), w_q=w, w_k=w)
    with pytest.raises(ValueError, match="GPU device"):
        la.la_short_conv(q=x, w_q=w)
